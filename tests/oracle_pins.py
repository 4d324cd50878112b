"""Pins of the fp64 oracle to things other than itself.

Every pin takes an oracle object (oracle.Oracle) so that the same checks run
against the real oracle (test_oracle_pins.py) and against deliberately broken
copies of it (test_oracle_mutants.py, which requires every planted mistake to
fail at least one pin).

What each pin rests on:
  - hand-derived worked examples (tests/golden/worked_examples.json);
  - closed forms: zero router -> all logits tie at 0; zero gate or zero up
    projection -> output exactly 0; identical experts -> output independent of
    the routing; a +100 bias forces a choice;
  - exact integer arithmetic: small-integer inputs make every logit an exact
    integer, so the selection is fixed by integer comparisons done in Python;
  - brute force: on tiny inputs the top-k set is the k-subset with the largest
    logit sum (ties: lexicographically smallest), found by enumeration;
  - independent dense formulations in numpy: k = E is dense softmax gating
    (yunthe page, section 1.1), and any k is a masked sum over all experts;
  - library primitives: numpy's stable argsort / bincount / cumsum for the
    permutation, numpy matmul for the logits;
  - invariants the pages fix: renormalised weights sum to one; every token
    appears exactly k times; unselected experts do no work (Baidu page,
    section 四), so changing their weights changes nothing.
"""
import itertools
import json
import math
import os

import numpy as np

import moe_synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden",
                      "worked_examples.json")


# ----------------------------------------------------------- test helpers

def wide(a):
    """Exact fp64 view of a float32 / bf16-bits array (format helper)."""
    if a.dtype == np.uint16:
        return moe_synth.bf16_bits_to_f32(a).astype(np.float64)
    return np.asarray(a, np.float64)


def np_silu(z):
    return z / (1.0 + np.exp(-z))


def np_dense_layer(x, Wr, Wgu, Wd, k, S=0, bias=None):
    """Independent numpy formulation: every expert evaluated densely on every
    token, then masked by the selection.  Selection by np.lexsort on
    (expert index, -logit); weights = softmax over the selected logits."""
    x, Wr, Wgu, Wd = wide(x), wide(Wr), wide(Wgu), wide(Wd)
    T = x.shape[0]
    E = Wr.shape[0]
    f = Wgu.shape[1] // 2
    L = x @ Wr.T
    if bias is not None:
        L = L + np.asarray(bias, np.float64)[None, :]
    outs = []
    for e in range(E + S):
        g = x @ Wgu[e, :f, :].T
        u = x @ Wgu[e, f:, :].T
        outs.append((np_silu(g) * u) @ Wd[e].T)
    outs = np.stack(outs)                       # [E+S, T, d]
    y = np.zeros((T, x.shape[1]))
    idx = np.zeros((T, k), np.int32)
    w = np.zeros((T, k))
    for t in range(T):
        order = np.lexsort((np.arange(E), -L[t]))
        sel = order[:k]
        ls = L[t, sel]
        ws = np.exp(ls - ls.max())
        ws /= ws.sum()
        idx[t] = sel
        w[t] = ws
        for j in range(k):
            y[t] += ws[j] * outs[sel[j], t]
        for s in range(S):
            y[t] += outs[E + s, t]
    return y, idx, w, L


def rand_layer(key, T, d, f, E, k, S=0, dtype="f32", wstd=0.3):
    seed = key
    x = moe_synth.normal((seed, 5, 0), (T, d), 1.0, dtype)
    Wr = moe_synth.normal((seed, 5, 1), (E, d), wstd, dtype)
    Wgu = moe_synth.normal((seed, 5, 2), (E + S, 2 * f, d), wstd, dtype)
    Wd = moe_synth.normal((seed, 5, 3), (E + S, d, f), wstd, dtype)
    return x, Wr, Wgu, Wd


def rel_err(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b)) / max(1e-300, np.max(np.abs(b))))


# ------------------------------------------------------------------ pins

def pin_golden_route(orc):
    g = json.load(open(GOLDEN))
    for name in ("route_topk_renorm", "route_ties_lower_index"):
        c = g[name]
        x = np.array(c["x"], np.float32)
        Wr = np.array(c["W_router"], np.float32)
        L, idx, w = orc.route(x, Wr, c["k"])
        assert np.array_equal(L, np.array(c["logits"])), name
        assert np.array_equal(idx, np.array(c["idx"])), name
        assert np.allclose(w, np.array(c["w"]), rtol=0, atol=1e-15), name


def pin_golden_layer(orc):
    g = json.load(open(GOLDEN))
    c = g["swiglu_expert"]
    x = np.array(c["x"], np.float32)
    Wgu = np.array(c["W_gate_up"], np.float32)
    Wd = np.array(c["W_down"], np.float32)
    Wr = np.zeros((1, 1), np.float32)
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, 1)
    assert abs(y[0, 0] - c["y"][0][0]) <= 1e-14, (y, c["y"])
    assert abs(y[0, 0] - c["y_if_gate_up_swapped"][0][0]) > 0.5

    c = g["two_expert_layer"]
    x = np.array(c["x"], np.float32)
    Wr = np.array(c["W_router"], np.float32)
    E = Wr.shape[0]
    Wgu = np.zeros((E, 2, 2), np.float32)
    Wd = np.zeros((E, 2, 1), np.float32)
    for e in range(E):
        Wgu[e, 0, 0] = e + 1
        Wgu[e, 1, 0] = 1
        Wd[e, 0, 0] = e + 1
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, c["k"])
    assert np.array_equal(idx, np.array(c["idx"]))
    assert np.allclose(y, np.array(c["y"]), rtol=0, atol=1e-14), y


def pin_zero_router_ties(orc):
    for E, k in ((8, 2), (8, 4), (6, 1), (16, 8)):
        T, d = 16, 32
        x = moe_synth.normal((11, 5, 0), (T, d), 1.0, "f32")
        Wr = np.zeros((E, d), np.float32)
        L, idx, w = orc.route(x, Wr, k)
        assert np.all(L == 0.0)
        assert np.array_equal(idx, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
        assert np.all(w == 1.0 / k)          # k a power of two: exact
        counts, offsets, ss, sp = orc.permute(idx, E)
        assert list(counts[:k]) == [T] * k and not counts[k:].any()
        # group of expert j lists the tokens in order
        for j in range(k):
            grp = ss[offsets[j]:offsets[j + 1]]
            assert np.array_equal(grp, np.arange(T) * k + j)


def pin_duplicate_rows_tie(orc):
    T, d, E = 32, 24, 8
    x = moe_synth.normal((12, 5, 0), (T, d), 1.0, "f32")
    Wr = moe_synth.normal((12, 5, 1), (E, d), 0.1, "f32")
    Wr[5] = Wr[2]
    bias = np.zeros(E, np.float32)
    bias[2] = bias[5] = 50.0
    for k in (1, 2, 3):
        L, idx, w = orc.route(x, Wr, k, bias=bias)
        assert np.all(idx[:, 0] == 2)
        if k >= 2:
            assert np.all(idx[:, 1] == 5)
            assert np.all(w[:, 0] == w[:, 1])


def pin_integer_exact_routing(orc):
    T, d, E = 96, 16, 7
    xi = moe_synth.small_ints((13, 5, 0), (T, d), -3, 3)
    Wi = moe_synth.small_ints((13, 5, 1), (E, d), -3, 3)
    for k in (1, 2, 3, 7):
        L, idx, w = orc.route(xi, Wi, k)
        for t in range(T):
            li = [sum(int(xi[t, i]) * int(Wi[e, i]) for i in range(d)) for e in range(E)]
            assert list(L[t]) == [float(v) for v in li]
            ranked = sorted(range(E), key=lambda e: (-li[e], e))[:k]
            assert list(idx[t]) == ranked, (t, li, idx[t], ranked)
            m = max(li[e] for e in ranked)
            ex = [math.exp(li[e] - m) for e in ranked]
            ref = [v / sum(ex) for v in ex]
            assert max(abs(a - b) for a, b in zip(w[t], ref)) <= 1e-15


def pin_bruteforce_subsets(orc):
    for dtype, seed in (("f32", 14), ("bf16", 15)):
        T, d, E = 8, 10, 6
        x = moe_synth.normal((seed, 5, 0), (T, d), 1.0, dtype)
        Wr = moe_synth.normal((seed, 5, 1), (E, d), 0.5, dtype)
        Lnp = wide(x) @ wide(Wr).T
        for k in range(1, E + 1):
            L, idx, w = orc.route(x, Wr, k)
            assert np.allclose(L, Lnp, rtol=1e-13, atol=1e-13)
            for t in range(T):
                best = max(itertools.combinations(range(E), k),
                           key=lambda c: (sum(L[t, e] for e in c), [-e for e in c]))
                assert sorted(idx[t]) == list(best)
                # slot order is rank order
                assert all(L[t, idx[t, j]] >= L[t, idx[t, j + 1]] for j in range(k - 1))


def pin_weights_renormalised(orc):
    T, d, E = 64, 40, 12
    x = moe_synth.normal((16, 5, 0), (T, d), 1.0, "bf16")
    Wr = moe_synth.normal((16, 5, 1), (E, d), 0.2, "bf16")
    for k in (1, 3, 5, 12):
        L, idx, w = orc.route(x, Wr, k)
        assert np.all(np.abs(w.sum(1) - 1.0) <= 1e-15)
        assert np.all(np.diff(w, axis=1) <= 0)
        # top-k then softmax over the k picked scores (Baidu page, section 四)
        sel = np.take_along_axis(L, idx.astype(np.int64), 1)
        ref = np.exp(sel - sel.max(1, keepdims=True))
        ref /= ref.sum(1, keepdims=True)
        assert np.max(np.abs(w - ref)) <= 1e-15


def pin_dense_gating_k_equals_E(orc):
    T, d, f, E = 5, 6, 4, 4
    x, Wr, Wgu, Wd = rand_layer(17, T, d, f, E, E)
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, E)
    # dense soft gating over all experts (yunthe page, section 1.1)
    xd, Wrd, Wgud, Wdd = wide(x), wide(Wr), wide(Wgu), wide(Wd)
    L = xd @ Wrd.T
    p = np.exp(L - L.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    yd = np.zeros((T, d))
    for e in range(E):
        h = np_silu(xd @ Wgud[e, :f].T) * (xd @ Wgud[e, f:].T)
        yd += p[:, e:e + 1] * (h @ Wdd[e].T)
    assert rel_err(y, yd) <= 1e-12


def pin_dense_masked_bruteforce(orc):
    for (T, d, f, E, k, S, dt, seed) in ((7, 8, 6, 5, 2, 0, "f32", 18),
                                         (9, 8, 8, 6, 3, 1, "bf16", 19),
                                         (6, 5, 7, 4, 1, 2, "f32", 20)):
        x, Wr, Wgu, Wd = rand_layer(seed, T, d, f, E, k, S, dt)
        bias = np.linspace(0.3, -0.4, E).astype(np.float32)
        y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        yd, idxd, wd, _ = np_dense_layer(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        assert np.array_equal(idx, idxd)
        assert np.max(np.abs(w - wd)) <= 1e-14
        assert rel_err(y, yd) <= 1e-12, rel_err(y, yd)


def pin_identical_experts(orc):
    T, d, f, E, k = 12, 10, 6, 5, 3
    x, Wr, Wgu, Wd = rand_layer(21, T, d, f, E, k)
    Wgu[:] = Wgu[0]
    Wd[:] = Wd[0]
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k)
    xd = wide(x)
    h = np_silu(xd @ wide(Wgu[0, :f]).T) * (xd @ wide(Wgu[0, f:]).T)
    assert rel_err(y, h @ wide(Wd[0]).T) <= 1e-13


def pin_zero_gate_or_up(orc):
    T, d, f, E, k = 10, 12, 8, 4, 2
    for half in (0, 1):
        x, Wr, Wgu, Wd = rand_layer(22 + half, T, d, f, E, k, S=1)
        Wgu[:, half * f:(half + 1) * f, :] = 0
        y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k, S=1)
        assert np.all(y == 0.0)


def pin_onehot_bias(orc):
    T, d, E = 40, 16, 9
    x = moe_synth.normal((24, 5, 0), (T, d), 1.0, "f32")
    Wr = moe_synth.normal((24, 5, 1), (E, d), 0.3, "f32")
    for e_star in (0, 4, 8):
        bias = np.zeros(E, np.float32)
        bias[e_star] = 100.0
        L, idx, w = orc.route(x, Wr, 3, bias=bias)
        assert np.all(idx[:, 0] == e_star)
        assert np.all(w[:, 0] > 0.999)


def pin_permutation(orc):
    rng = np.random.default_rng([25, 5, 0])
    for (T, k, E, S) in ((50, 3, 7, 0), (64, 8, 16, 1), (1, 1, 1, 0), (33, 2, 40, 2),
                         (0, 2, 4, 0)):
        idx = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32) \
            if T else np.zeros((0, k), np.int32)
        counts, offsets, ss, sp = orc.permute(idx, E, S)
        flat = idx.ravel()
        assert np.array_equal(counts[:E], np.bincount(flat, minlength=E))
        assert np.all(counts[E:] == T)
        assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
        assert offsets[E] == T * k and offsets[E + S] == T * k + S * T
        assert np.array_equal(ss, np.argsort(flat, kind="stable"))
        assert np.array_equal(sp[ss], np.arange(T * k))
        assert np.array_equal(np.sort(ss), np.arange(T * k))
        tok_counts = np.bincount(ss // k, minlength=T) if T else np.zeros(0)
        assert np.all(tok_counts == k)


def pin_unselected_do_nothing(orc):
    T, d, f, E, k = 20, 12, 8, 8, 2
    x, Wr, Wgu, Wd = rand_layer(26, T, d, f, E, k)
    bias = np.zeros(E, np.float32)
    bias[5:] = -100.0
    y0, idx, w0 = orc.layer_forward(x, Wr, Wgu, Wd, k, bias=bias)
    assert np.all(idx < 5)
    Wgu2, Wd2 = Wgu.copy(), Wd.copy()
    Wgu2[5:] *= -3.0
    Wd2[5:] += 1.0
    y1, _, _ = orc.layer_forward(x, Wr, Wgu2, Wd2, k, bias=bias)
    assert np.array_equal(y0, y1)


def pin_bf16_widening(orc):
    T, d, f, E, k = 9, 16, 8, 5, 2
    x, Wr, Wgu, Wd = rand_layer(27, T, d, f, E, k, S=1, dtype="bf16")
    as32 = [moe_synth.bf16_bits_to_f32(a) for a in (x, Wr, Wgu, Wd)]
    yb, ib, wb = orc.layer_forward(x, Wr, Wgu, Wd, k, S=1)
    yf, i_f, wf = orc.layer_forward(*as32, k, S=1)
    assert np.array_equal(ib, i_f) and np.array_equal(wb, wf) and np.array_equal(yb, yf)
    # and bf16 patterns really are the upper half of binary32
    one = np.array([[0x3F80]], np.uint16)   # 1.0
    half = np.array([[0xBF00]], np.uint16)  # -0.5
    L, _, _ = orc.route(one, half, 1)
    assert L[0, 0] == -0.5


def pin_decomposed_path(orc):
    """route -> permute -> gate_up -> down -> combine equals the whole layer;
    combine on rows of known values equals its closed form."""
    T, d, f, E, k, S = 11, 8, 6, 5, 2, 1
    x, Wr, Wgu, Wd = rand_layer(28, T, d, f, E, k, S)
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S)
    L, idx2, w2 = orc.route(x, Wr, k)
    assert np.array_equal(idx, idx2) and np.array_equal(w, w2)
    counts, offsets, ss, sp = orc.permute(idx2, E, S)
    R = T * k + S * T
    tok = np.concatenate([ss // k, np.tile(np.arange(T), S)]).astype(np.int64)
    ex = np.concatenate([idx2.ravel()[ss],
                         np.repeat(np.arange(E, E + S), T)]).astype(np.int32)
    act = orc.gate_up_rows(x, Wgu, tok, ex)
    O = orc.down_rows(act.astype(np.float32), Wd, ex)
    y2 = orc.combine(O.astype(np.float32), sp, w2, T, k, S)
    assert rel_err(y2, y) <= 1e-5
    # closed form of the combine: O rows filled with their row number
    Orow = np.repeat(np.arange(R, dtype=np.float32)[:, None], d, 1)
    yc = orc.combine(Orow, sp, w2, T, k, S)
    exp = (w2 * sp.reshape(T, k)).sum(1) + sum(T * k + s * T + np.arange(T) for s in range(S))
    assert np.max(np.abs(yc - exp[:, None])) <= 1e-12


def pin_sharding_identity(orc):
    """Experts split into disjoint ranges: the partial outputs sum to the full
    output (aitoday page, section 'Expert Parallelism': each device computes
    with its own experts, partial outputs are all-reduced)."""
    T, d, f, E, k = 16, 8, 6, 8, 3
    x, Wr, Wgu, Wd = rand_layer(29, T, d, f, E, k)
    y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k)
    counts, offsets, ss, sp = orc.permute(idx, E)
    tok = (ss // k).astype(np.int64)
    ex = idx.ravel()[ss]
    O = orc.down_rows(orc.gate_up_rows(x, Wgu, tok, ex).astype(np.float32), Wd, ex)
    total = np.zeros((T, d))
    for lo, hi in ((0, 3), (3, 5), (5, 8)):
        part = np.zeros_like(O, dtype=np.float32)
        rows = slice(offsets[lo], offsets[hi])
        part[rows] = O[rows]
        total += orc.combine(part, sp, w, T, k)
    full = orc.combine(O.astype(np.float32), sp, w, T, k)
    assert rel_err(total, full) <= 1e-12
    assert rel_err(full, y) <= 1e-5


def pin_forced_natural_selection(orc):
    """Forcing the selection the oracle makes by itself changes nothing: the
    same experts in the same slot order give bitwise the same y and weights."""
    for (T, d, f, E, k, S, dt, seed) in ((9, 8, 6, 6, 2, 0, "f32", 30),
                                         (7, 8, 8, 5, 3, 1, "bf16", 31)):
        x, Wr, Wgu, Wd = rand_layer(seed, T, d, f, E, k, S, dt)
        bias = np.linspace(0.2, -0.1, E).astype(np.float32)
        y0, idx0, w0 = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        y1, idx1, w1 = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias,
                                         forced_idx=idx0)
        assert np.array_equal(idx1, idx0)
        assert np.array_equal(w1, w0) and np.array_equal(y1, y0)


def pin_forced_other_selection(orc):
    """A forced k-set that is not the natural top-k: the output is the dense
    per-expert outputs (numpy, independent of the oracle) masked to the
    forced experts, with weights = softmax over the forced experts' logits
    (Baidu page, section 四: softmax over the picked scores), slot j holding
    the weight of forced expert j."""
    for (T, d, f, E, k, S, dt, seed) in ((8, 8, 6, 6, 2, 0, "f32", 32),
                                         (6, 8, 8, 7, 3, 1, "bf16", 33)):
        x, Wr, Wgu, Wd = rand_layer(seed, T, d, f, E, k, S, dt)
        bias = np.linspace(-0.3, 0.3, E).astype(np.float32)
        _, idx_nat, _, L = np_dense_layer(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        # the k lowest-ranked experts, in ascending expert order: disjoint from
        # the natural selection whenever 2k <= E
        forced = np.stack([np.sort(np.lexsort((np.arange(E), L[t]))[:k])
                           for t in range(T)]).astype(np.int32)
        assert not np.any([set(forced[t]) & set(idx_nat[t]) for t in range(T)])
        y, idx, w = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias, forced_idx=forced)
        assert np.array_equal(idx, forced)
        xd, Wgud, Wdd = wide(x), wide(Wgu), wide(Wd)
        outs = np.stack([(np_silu(xd @ Wgud[e, :f].T) * (xd @ Wgud[e, f:].T)) @ Wdd[e].T
                         for e in range(E + S)])
        y_ref = np.zeros((T, d))
        for t in range(T):
            ls = L[t, forced[t]]
            ws = np.exp(ls - ls.max())
            ws /= ws.sum()
            assert np.max(np.abs(w[t] - ws)) <= 1e-14
            y_ref[t] = sum(ws[j] * outs[forced[t, j], t] for j in range(k))
            y_ref[t] += sum(outs[E + s, t] for s in range(S))
        assert rel_err(y, y_ref) <= 1e-12, rel_err(y, y_ref)


# ------------------------------------------- router auxiliaries (capacity, balance)

def brute_capacity(idx, E, S, C):
    """Independent construction of the capacity permutation by sorting: a
    copy is kept when fewer than C earlier copies (smaller slot) chose its
    expert; dropped copies first (by expert, then slot), then the kept ones
    (by expert, then slot)."""
    flat = [int(v) for v in np.asarray(idx).ravel()]
    n = len(flat)
    T = np.asarray(idx).shape[0]
    kept = [sum(1 for q in range(s) if flat[q] == flat[s]) < C for s in range(n)]
    dropped = sorted((flat[s], s) for s in range(n) if not kept[s])
    keep_list = sorted((flat[s], s) for s in range(n) if kept[s])
    order = [s for _, s in dropped] + [s for _, s in keep_list]
    counts = [sum(1 for (e, _) in keep_list if e == g) for g in range(E)] + [T] * S
    offsets = [len(dropped)]
    for c in counts:
        offsets.append(offsets[-1] + c)
    slot_pos = [-1] * n
    for r, s in enumerate(order):
        if kept[s]:
            slot_pos[s] = r
    return (np.array(counts, np.int32), np.array(offsets, np.int32),
            np.array(order, np.int32), np.array(slot_pos, np.int32),
            np.array(kept, bool).reshape(np.asarray(idx).shape))


def pin_capacity_permutation(orc):
    """Expert capacity (yunthe page, section 3.1): brute-force construction
    on small inputs, the no-limit and zero-capacity special cases."""
    rng = np.random.default_rng([40, 5, 0])
    for (T, k, E, S) in ((30, 3, 5, 0), (17, 2, 9, 1), (1, 1, 1, 0), (24, 4, 4, 2),
                         (0, 2, 3, 1)):
        if T:
            # skewed choice: low experts far more popular
            idx = np.stack([rng.choice(E, k, replace=False, p=np.arange(E, 0, -1) / (E * (E + 1) / 2))
                            for _ in range(T)]).astype(np.int32)
        else:
            idx = np.zeros((0, k), np.int32)
        free = orc.permute(idx, E, S)
        for C in (0, 1, 2, 5, T, T * k + 3):
            got = orc.permute(idx, E, S, capacity=C)
            ref = brute_capacity(idx, E, S, C)
            for a, b, name in zip(got, ref[:4], ("counts", "offsets", "sorted_slot", "slot_pos")):
                assert np.array_equal(a, b), (T, k, E, S, C, name)
            assert got[1][E] == T * k and got[1][E + S] == T * k + S * T
            assert np.all(got[0][:E] <= C)
            if C >= T:
                for a, b in zip(got, free):
                    assert np.array_equal(a, b)
            if C == 0:
                assert np.all(got[3] == -1) and np.all(got[0][:E] == 0)


def pin_expert_capacity(orc):
    """Capacity from a factor: ceil(factor * T*k / E) (yunthe page, sections
    4.1 and 5.2: the factor scales an expert's even share of the tokens)."""
    assert orc.expert_capacity(4096, 8, 128, 1.25) == 320
    assert orc.expert_capacity(10, 2, 3, 1.0) == 7
    assert orc.expert_capacity(4096, 8, 256, 1.0) == 128
    assert orc.expert_capacity(7, 1, 4, 0.0) == 0
    assert orc.expert_capacity(8192, 2, 8, 2.0) == 4096


def pin_capacity_layer(orc):
    """The layer with a capacity equals the dense numpy formulation with the
    dropped copies' terms removed and the kept weights unchanged; a capacity
    of at least T changes nothing; capacity 0 leaves the shared experts."""
    for (T, d, f, E, k, S, dt, seed) in ((24, 8, 6, 4, 2, 0, "f32", 41),
                                         (20, 8, 8, 5, 3, 1, "bf16", 42)):
        x, Wr, Wgu, Wd = rand_layer(seed, T, d, f, E, k, S, dt)
        bias = np.linspace(0.8, -0.8, E).astype(np.float32)  # skewed load
        _, idx, w, _ = np_dense_layer(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        xd, Wgud, Wdd = wide(x), wide(Wgu), wide(Wd)
        outs = np.stack([(np_silu(xd @ Wgud[e, :f].T) * (xd @ Wgud[e, f:].T)) @ Wdd[e].T
                         for e in range(E + S)])
        y_free, _, _ = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias)
        for C in (0, 3, 7, T):
            keep = brute_capacity(idx, E, S, C)[4]
            y_ref = np.zeros((T, d))
            for t in range(T):
                for j in range(k):
                    if keep[t, j]:
                        y_ref[t] += w[t, j] * outs[idx[t, j], t]
                y_ref[t] += sum(outs[E + s, t] for s in range(S))
            y, idx_o, w_o = orc.layer_forward(x, Wr, Wgu, Wd, k, S=S, bias=bias, capacity=C)
            assert np.array_equal(idx_o, idx)
            assert rel_err(y, y_ref) <= 1e-12, (C, rel_err(y, y_ref))
            if C >= T:
                assert np.array_equal(y, y_free)
            if C == 0:
                shared = sum((outs[E + s] for s in range(S)), np.zeros((T, d)))
                assert rel_err(y, shared) <= 1e-12 if S else np.all(y == 0.0)


def pin_balance_closed_forms(orc):
    """Balance loss (yunthe page, section 3.1): a zero router gives every
    expert probability 1/E, so importance = 1/E and the loss is
    -(1/E) log1p(E * 1e-8); a +1000 bias on one expert gives importance =
    that expert's unit vector and the loss in closed form; no tokens: NaN."""
    for (T, d, E, dt) in ((13, 8, 6, "f32"), (5, 16, 32, "bf16")):
        x = moe_synth.normal((43, 5, T), (T, d), 1.0, dt)
        Wr = np.zeros((E, d), np.float32 if dt == "f32" else np.uint16)
        imp, loss = orc.balance(x, Wr)
        assert np.max(np.abs(imp - 1.0 / E)) <= 1e-16
        # the oracle's log(u) - log(u + 1e-8) cancels: a few ulps of log(u)
        assert abs(loss - (-math.log1p(E * 1e-8) / E)) <= 4e-16 * abs(math.log(1.0 / E))
        bias = np.zeros(E, np.float32)
        bias[2] = 1000.0
        Wr2 = moe_synth.normal((43, 6, T), (E, d), 0.3, dt)
        imp, loss = orc.balance(x, Wr2, bias=bias)
        assert imp[2] == 1.0 and np.all(np.delete(imp, 2) == 0.0)
        u = 1.0 / E
        ref = (u * (math.log(u) - math.log(1.0 + 1e-8))
               + (E - 1) * u * (math.log(u) - math.log(1e-8))) / E
        assert abs(loss - ref) <= 1e-13 * abs(ref)
    imp, loss = orc.balance(np.zeros((0, 8), np.float32), np.ones((3, 8), np.float32))
    assert np.all(np.isnan(imp)) and math.isnan(loss)


def pin_balance_library(orc):
    """Balance statistics against library routines on a random router:
    importance = mean of scipy's softmax of numpy-matmul logits (bias added),
    loss = torch.nn.functional.kl_div(log(importance + 1e-8), uniform,
    reduction='batchmean'), the form the yunthe page's section 3.1 example
    writes.  The importance sums to one."""
    import scipy.special
    import torch
    for (T, d, E, dt, seed) in ((40, 16, 8, "f32", 44), (33, 24, 20, "bf16", 45)):
        x = moe_synth.normal((seed, 5, 0), (T, d), 1.0, dt)
        Wr = moe_synth.normal((seed, 5, 1), (E, d), 0.4, dt)
        bias = np.linspace(0.5, -1.0, E).astype(np.float32)
        imp, loss, probs = orc.balance(x, Wr, bias=bias, want_probs=True)
        L = wide(x) @ wide(Wr).T + bias.astype(np.float64)[None, :]
        p_ref = scipy.special.softmax(L, axis=1)
        assert rel_err(probs, p_ref) <= 1e-13
        assert rel_err(imp, p_ref.mean(0)) <= 1e-13
        assert abs(imp.sum() - 1.0) <= 1e-13
        ref = torch.nn.functional.kl_div(torch.log(torch.tensor(imp) + 1e-8),
                                         torch.full((E,), 1.0 / E, dtype=torch.float64),
                                         reduction="batchmean").item()
        assert abs(loss - ref) <= 1e-12 * abs(ref), (loss, ref)
        # the loss is KL(u || imp) / E up to the 1e-8 guard: zero only at uniform
        assert loss > 0


# --------------------------------------------------------- MXFP4 weights

# FP4 E2M1 magnitudes of codes 0..7 as the OCP Microscaling specification
# tabulates them (code | 8 is the negative)
E2M1_TABLE = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def np_dequant_mxfp4(q, sc):
    """Table lookup: codes from the nibbles (even element low), magnitudes
    from the specification's table, times 2^(X - 127) per 32-element block."""
    q = np.asarray(q, np.uint8)
    codes = np.stack([q & 15, q >> 4], axis=-1).reshape(q.shape[:-1] + (q.shape[-1] * 2,))
    mag = E2M1_TABLE[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    scale = np.where(sc == 255, np.nan, np.ldexp(1.0, sc.astype(np.int64) - 127))
    return val * np.repeat(scale, 32, axis=-1)


def pin_mxfp4_codes_and_scales(orc):
    """Every byte value in both nibble positions against the table; every
    E8M0 exponent (255 is NaN); one scale per 32-element block."""
    q = np.arange(256, dtype=np.uint8).reshape(8, 32)        # K = 64 per row
    sc = np.array([[127, 127]] * 8, np.uint8)
    got = orc.dequant_mxfp4(q, sc)
    assert np.array_equal(got, np_dequant_mxfp4(q, sc))
    assert got[0, 2] == 0.5 and got[0, 3] == 0.0                # byte 0x01
    assert got[0, 34] == 0.5 and got[0, 35] == 0.5              # byte 0x11
    assert got[1, 30] == -6.0 and got[1, 31] == 1.0             # byte 0x2f
    b = q.reshape(-1)
    lo = np.where(b & 8, -E2M1_TABLE[b & 7], E2M1_TABLE[b & 7])
    hi = np.where((b >> 4) & 8, -E2M1_TABLE[(b >> 4) & 7], E2M1_TABLE[(b >> 4) & 7])
    flat = got.reshape(-1)
    assert np.array_equal(flat[0::2], lo) and np.array_equal(flat[1::2], hi)
    # scales: code 2 (1.0) everywhere, exponent X in every block
    X = np.arange(256, dtype=np.uint8).reshape(4, 64)
    q1 = np.full((4, 64 * 16), 0x22, np.uint8)                  # K = 2048 per row
    v = orc.dequant_mxfp4(q1, X)
    want = np.repeat(np.where(X == 255, np.nan, 2.0 ** (X.astype(np.float64) - 127)), 32, axis=1)
    assert np.array_equal(np.isnan(v), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(v[ok], want[ok])
    # blocks are 32 elements of one row: changing one scale byte moves
    # exactly that block
    q2 = np.full((2, 32), 0x44, np.uint8)                       # 2.0 everywhere, K = 64
    s2 = np.array([[127, 127], [127, 127]], np.uint8)
    base = orc.dequant_mxfp4(q2, s2)
    s2[1, 0] = 128
    moved = orc.dequant_mxfp4(q2, s2)
    diff = moved != base
    assert diff[1, :32].all() and not diff[1, 32:].any() and not diff[0].any()


def pin_mxfp4_layer(orc):
    """A layer with MXFP4 expert weights is the bf16 layer on the dequantised
    weights; the dequantised values of the synthetic scale range are exact in
    float32, and the numpy table lookup agrees with the oracle everywhere."""
    cfg = moe_synth.tiny_config(T=9, d=64, f=32, E=5, k=2, S=1, dtype="bf16")
    inp = moe_synth.make_layer_inputs(cfg, 46, experts=False)
    mx = moe_synth.make_mxfp4_experts(cfg, 46)
    wgu = orc.dequant_mxfp4(mx["Wq_gate_up"], mx["Ws_gate_up"])
    wd = orc.dequant_mxfp4(mx["Wq_down"], mx["Ws_down"])
    assert np.array_equal(wgu, np_dequant_mxfp4(mx["Wq_gate_up"], mx["Ws_gate_up"]))
    assert np.array_equal(wd, np_dequant_mxfp4(mx["Wq_down"], mx["Ws_down"]))
    assert np.array_equal(wgu.astype(np.float32).astype(np.float64), wgu)
    x32 = moe_synth.bf16_bits_to_f32(inp["x"])
    wr32 = moe_synth.bf16_bits_to_f32(inp["W_router"])
    y, idx, w = orc.layer_forward(x32, wr32, wgu.astype(np.float32), wd.astype(np.float32),
                                  cfg.k, S=cfg.S)
    y_ref, idx_ref, w_ref, _ = np_dense_layer(x32, wr32, wgu.astype(np.float32),
                                              wd.astype(np.float32), cfg.k, S=cfg.S)
    assert np.array_equal(idx, idx_ref)
    assert rel_err(y, y_ref) <= 1e-12


# ------------------------------------------------------------- backward

def torch_dense_grads(x, Wr, Wgu, Wd, dy, k, S=0, bias=None):
    """Independent gradients: the layer written densely in torch (fp64 on
    the CPU, every expert evaluated on every token, the top-k taken by
    torch.topk on detached logits, softmax over the selected logits) and
    differentiated by autograd."""
    import torch
    t = lambda a: torch.tensor(wide(a), dtype=torch.float64, requires_grad=True)
    X, WR, WGU, WD = t(x), t(Wr), t(Wgu), t(Wd)
    B = torch.tensor(np.asarray(bias, np.float64) if bias is not None
                     else np.zeros(Wr.shape[0]), dtype=torch.float64, requires_grad=True)
    DY = torch.tensor(wide(dy), dtype=torch.float64)
    E = Wr.shape[0]
    f = Wgu.shape[1] // 2
    L = X @ WR.T + B
    sel = torch.topk(L.detach(), k, dim=1).indices
    w = torch.softmax(torch.gather(L, 1, sel), dim=1)
    outs = []
    for e in range(E + S):
        g = X @ WGU[e, :f].T
        u = X @ WGU[e, f:].T
        outs.append((torch.nn.functional.silu(g) * u) @ WD[e].T)
    outs = torch.stack(outs, 1)                                   # [T, E+S, d]
    y = (w.unsqueeze(2) * torch.gather(outs[:, :E], 1,
                                       sel.unsqueeze(2).expand(-1, -1, outs.shape[2]))).sum(1)
    if S:
        y = y + outs[:, E:].sum(1)
    w.retain_grad()
    (y * DY).sum().backward()
    return dict(dx=X.grad.numpy(), dW_gate_up=WGU.grad.numpy(), dW_down=WD.grad.numpy(),
                dW_router=WR.grad.numpy(), db=B.grad.numpy(), dw=w.grad.numpy(),
                sel=sel.numpy())


def pin_backward_autograd(orc):
    """Every gradient against torch autograd on a dense formulation, fp32
    and bf16 inputs, with a shared expert and a router bias."""
    for (T, d, f, E, k, S, dt, seed) in ((10, 8, 6, 5, 2, 0, "f32", 50),
                                         (7, 16, 8, 6, 3, 1, "bf16", 51)):
        x, Wr, Wgu, Wd = rand_layer(seed, T, d, f, E, k, S, dt)
        dy = moe_synth.normal((seed, 6, 0), (T, d), 1.0, dt)
        bias = np.linspace(0.3, -0.2, E).astype(np.float32)
        ref = torch_dense_grads(x, Wr, Wgu, Wd, dy, k, S, bias)
        got = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, S=S, bias=bias,
                                 experts=np.arange(E + S))
        _, idx, _ = orc.route(x, Wr, k, bias=bias)
        assert np.array_equal(np.sort(idx, 1), np.sort(ref["sel"], 1))
        for name in ("dx", "dW_gate_up", "dW_down", "dW_router", "db"):
            assert rel_err(got[name], ref[name]) <= 1e-12, (name, rel_err(got[name], ref[name]))
        # dw: slot order of the oracle (rank order) vs torch.topk's order
        for t in range(T):
            order = [list(ref["sel"][t]).index(e) for e in idx[t]]
            assert np.max(np.abs(got["dw"][t] - ref["dw"][t, order])) <= 1e-12


def pin_backward_finite_differences(orc):
    """Central differences of L = sum(y * dy) through the oracle's own
    forward: perturbations by 2^-12, exact in float32, that move no expert
    in or out of any token's top-k."""
    T, d, f, E, k, S = 6, 8, 6, 4, 2, 1
    x, Wr, Wgu, Wd = rand_layer(52, T, d, f, E, k, S, "f32")
    Wr = Wr * 3.0                       # clear logit gaps: the selection holds
    dy = moe_synth.normal((52, 6, 0), (T, d), 1.0, "f32")
    bias = np.linspace(0.2, -0.1, E).astype(np.float32)
    got = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, S=S, bias=bias, experts=np.arange(E + S))
    _, idx0, _ = orc.route(x, Wr, k, bias=bias)
    h = 2.0 ** -12

    def loss(x_, Wr_, Wgu_, Wd_, b_):
        _, idx, _ = orc.route(x_, Wr_, k, bias=b_)
        assert np.array_equal(idx, idx0), "perturbation changed the selection"
        y, _, _ = orc.layer_forward(x_, Wr_, Wgu_, Wd_, k, S=S, bias=b_)
        return float((y * wide(dy)).sum())

    rng = np.random.default_rng([52, 9])
    args = dict(x=x, Wr=Wr, Wgu=Wgu, Wd=Wd, b=bias)
    grads = dict(x=got["dx"], Wr=got["dW_router"], Wgu=got["dW_gate_up"], Wd=got["dW_down"],
                 b=got["db"])
    for name in ("x", "Wr", "Wgu", "Wd", "b"):
        for _ in range(4):
            pos = tuple(int(rng.integers(0, n)) for n in args[name].shape)
            plus = {kk: v.copy() for kk, v in args.items()}
            minus = {kk: v.copy() for kk, v in args.items()}
            plus[name][pos] += np.float32(h)
            minus[name][pos] -= np.float32(h)
            fd = (loss(plus["x"], plus["Wr"], plus["Wgu"], plus["Wd"], plus["b"])
                  - loss(minus["x"], minus["Wr"], minus["Wgu"], minus["Wd"], minus["b"])) / (2 * h)
            g = grads[name][pos]
            assert abs(fd - g) <= 1e-5 * (1.0 + abs(g)), (name, pos, fd, g)


def pin_backward_structure(orc):
    """Experts that no token selects get zero weight gradients; the router
    bias gradient sums to zero over the experts (each token's softmax
    gradient over its k selected logits sums to zero); listing tokens or
    experts changes nothing."""
    T, d, f, E, k = 12, 8, 6, 6, 2
    x, Wr, Wgu, Wd = rand_layer(53, T, d, f, E, k)
    dy = moe_synth.normal((53, 6, 0), (T, d), 1.0, "f32")
    bias = np.zeros(E, np.float32)
    bias[4:] = -100.0                   # experts 4, 5 never selected
    full = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, bias=bias, experts=np.arange(E))
    assert np.all(full["dW_gate_up"][4:] == 0) and np.all(full["dW_down"][4:] == 0)
    assert np.all(full["dW_router"][4:] == 0) and np.all(full["db"][4:] == 0)
    assert abs(full["db"].sum()) <= 1e-12 * np.abs(full["db"]).sum()
    part = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, bias=bias, tokens=[7, 2],
                              experts=[3, 0], router=False)
    assert np.array_equal(part["dx"], full["dx"][[7, 2]])
    assert np.array_equal(part["dW_gate_up"], full["dW_gate_up"][[3, 0]])
    assert np.array_equal(part["dW_down"], full["dW_down"][[3, 0]])



def pin_backward_capacity(orc):
    """With an expert capacity: a capacity no expert reaches changes nothing
    (bitwise); dropped copies get dw = 0; and central differences through
    the capacity forward (the same keep set at every perturbation, since the
    selection holds) match every gradient."""
    T, d, f, E, k = 8, 8, 6, 3, 2
    x, Wr, Wgu, Wd = rand_layer(54, T, d, f, E, k, 0, "f32")
    Wr = Wr * 3.0
    dy = moe_synth.normal((54, 6, 0), (T, d), 1.0, "f32")
    bias = np.linspace(0.2, -0.1, E).astype(np.float32)
    free = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, bias=bias, experts=np.arange(E))
    wide_cap = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, bias=bias, experts=np.arange(E),
                                  capacity=T * k)
    for name in free:
        assert np.array_equal(free[name], wide_cap[name]), name
    C = 3
    got = orc.layer_backward(x, Wr, Wgu, Wd, dy, k, bias=bias, experts=np.arange(E),
                             capacity=C)
    _, idx0, _ = orc.route(x, Wr, k, bias=bias)
    _, _, _, slot_pos = orc.permute(idx0, E, capacity=C)
    dropped = slot_pos.reshape(T, k) < 0
    assert dropped.any() and not dropped.all()
    assert np.all(got["dw"][dropped] == 0)
    assert np.all(got["dw"][~dropped] != 0)
    h = 2.0 ** -12

    def loss(x_, Wr_, Wgu_, Wd_, b_):
        _, idx, _ = orc.route(x_, Wr_, k, bias=b_)
        assert np.array_equal(idx, idx0), "perturbation changed the selection"
        y, _, _ = orc.layer_forward(x_, Wr_, Wgu_, Wd_, k, bias=b_, capacity=C)
        return float((y * wide(dy)).sum())

    rng = np.random.default_rng([54, 9])
    args = dict(x=x, Wr=Wr, Wgu=Wgu, Wd=Wd, b=bias)
    grads = dict(x=got["dx"], Wr=got["dW_router"], Wgu=got["dW_gate_up"], Wd=got["dW_down"],
                 b=got["db"])
    for name in ("x", "Wr", "Wgu", "Wd", "b"):
        for _ in range(5):
            pos = tuple(int(rng.integers(0, n)) for n in args[name].shape)
            plus = {kk: v.copy() for kk, v in args.items()}
            minus = {kk: v.copy() for kk, v in args.items()}
            plus[name][pos] += np.float32(h)
            minus[name][pos] -= np.float32(h)
            fd = (loss(plus["x"], plus["Wr"], plus["Wgu"], plus["Wd"], plus["b"])
                  - loss(minus["x"], minus["Wr"], minus["Wgu"], minus["Wd"], minus["b"])) / (2 * h)
            g = grads[name][pos]
            assert abs(fd - g) <= 1e-5 * (1.0 + abs(g)), (name, pos, fd, g)
    # a dropped copy's expert sees no gradient from that token: the tokens
    # whose every copy of expert e was dropped leave dW of e as if absent
    for e in range(E):
        kept_tok = [t for t in range(T) for j in range(k) if idx0[t, j] == e and not dropped[t, j]]
        if not kept_tok:
            assert np.all(got["dW_gate_up"][e] == 0) and np.all(got["dW_down"][e] == 0)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
