"""Parity of each step of the layer (HIP path through the C ABI) with the
fp64 oracle, on seeded inputs that span several tiles, ragged tails, empty
experts and the size limits."""
import numpy as np
import pytest

import moe_synth
import oracle
import mixture_experts_sparse_router_amd as moe
from gpu_util import (abs_scores, assert_rows_close, check_routing, dev, dt_code, empty,
                      host)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _sync():
    torch.cuda.synchronize()


# ------------------------------------------------------------------ route

def _route_case(name):
    n = moe_synth.normal
    if name == "tiny_fp32":
        inp = moe_synth.make_layer_inputs(moe_synth.CONFIGS[1], 1, experts=False)
        return inp["x"], inp["W_router"], None, 2
    if name == "gpt_oss_20b_decode":
        inp = moe_synth.make_layer_inputs(moe_synth.CONFIGS[2], 2, experts=False)
        return inp["x"], inp["W_router"], None, 4
    if name == "fine_grained_zipf_full":
        inp = moe_synth.make_layer_inputs(moe_synth.CONFIGS[4], 4, experts=False)
        return inp["x"], inp["W_router"], inp["bias"], 8
    if name == "deepseek_v3_full":
        inp = moe_synth.make_layer_inputs(moe_synth.CONFIGS[5], 5, experts=False)
        return inp["x"], inp["W_router"], None, 8
    if name == "zero_router_ties":
        return n((40, 5, 0), (40, 64), 1.0, "bf16"), np.zeros((16, 64), np.uint16), None, 4
    if name == "duplicate_rows":
        x = n((41, 5, 0), (33, 96), 1.0, "bf16")
        W = n((41, 5, 1), (12, 96), 0.05, "bf16")
        W[7] = W[3]
        b = np.zeros(12, np.float32)
        b[3] = b[7] = 30.0
        return x, W, b, 3
    if name == "integer_exact_f32":
        return (moe_synth.small_ints((42, 5, 0), (70, 24), -3, 3),
                moe_synth.small_ints((42, 5, 1), (7, 24), -3, 3), None, 3)
    if name == "integer_exact_bf16":
        return (moe_synth.to_bf16_bits(moe_synth.small_ints((43, 5, 0), (70, 24), -3, 3)),
                moe_synth.to_bf16_bits(moe_synth.small_ints((43, 5, 1), (9, 24), -2, 2)),
                None, 4)
    if name == "ragged_E100_d136":
        return n((44, 5, 0), (37, 136), 1.0, "bf16"), n((44, 5, 1), (100, 136), 0.1, "bf16"), \
            np.linspace(0.5, -0.5, 100).astype(np.float32), 5
    if name == "max_E1024":
        return n((45, 5, 0), (50, 64), 1.0, "bf16"), n((45, 5, 1), (1024, 64), 0.1, "bf16"), \
            None, 8
    if name == "screen_E1024":
        return n((47, 5, 0), (100, 64), 1.0, "bf16"), n((47, 5, 1), (1024, 64), 0.1, "bf16"), \
            None, 8
    if name == "screen_E300_ragged":
        return n((48, 5, 0), (77, 136), 1.0, "bf16"), n((48, 5, 1), (300, 136), 0.1, "bf16"), \
            np.linspace(0.2, -0.3, 300).astype(np.float32), 6
    if name == "screen_E8_long_d":
        return n((49, 5, 0), (130, 4104), 1.0, "bf16"), n((49, 5, 1), (8, 4104), 0.02, "bf16"), \
            None, 2
    if name == "screen_zero_router":
        return n((50, 5, 0), (90, 96), 1.0, "bf16"), np.zeros((40, 96), np.uint16), None, 5
    if name == "screen_zero_router_E100":
        # every expert stays a candidate (more than 64): ranked in rounds
        return n((52, 5, 0), (90, 96), 1.0, "bf16"), np.zeros((100, 96), np.uint16), None, 5
    if name == "screen_duplicate_rows":
        x = n((51, 5, 0), (97, 256), 1.0, "bf16")
        W = n((51, 5, 1), (64, 256), 0.05, "bf16")
        W[40] = W[9]
        b = np.zeros(64, np.float32)
        b[9] = b[40] = 30.0
        return x, W, b, 4
    if name == "k_equals_E":
        return n((46, 5, 0), (19, 40), 1.0, "f32"), n((46, 5, 1), (6, 40), 0.2, "f32"), None, 6
    raise KeyError(name)


ROUTE_CASES = ["tiny_fp32", "gpt_oss_20b_decode", "zero_router_ties", "duplicate_rows",
               "integer_exact_f32", "integer_exact_bf16", "ragged_E100_d136", "max_E1024",
               "k_equals_E", "screen_E1024", "screen_E300_ragged", "screen_E8_long_d",
               "screen_zero_router", "screen_zero_router_E100", "screen_duplicate_rows",
               "fine_grained_zipf_full", "deepseek_v3_full"]


@pytest.mark.parametrize("name", ROUTE_CASES)
def test_route(name):
    x, W, bias, k = _route_case(name)
    dtype = "bf16" if x.dtype == np.uint16 else "f32"
    T, d = x.shape
    E = W.shape[0]
    print(f"route {name}: T={T} d={d} E={E} k={k} {dtype}", flush=True)
    s = moe.shape(T, d, 8, E, k, 0, dt_code(dtype))
    idx_d, w_d = empty((T, k), "i32"), empty((T, k), "f32")
    moe.moe_route(s, dev(x), dev(W), dev(bias), idx_d, w_d)
    _sync()
    L, idx_ref, w_ref = oracle.route(x, W, k, bias=bias)
    amb = check_routing(host(idx_d), host(w_d), L, abs_scores(x, W), idx_ref, w_ref)
    assert len(amb) <= max(1, T // 1000), f"{len(amb)} near-tie tokens"
    if name in ("zero_router_ties", "duplicate_rows", "screen_zero_router",
                "screen_zero_router_E100", "screen_duplicate_rows") or name.startswith("integer"):
        assert not amb and np.array_equal(host(idx_d), idx_ref)


# The layer's router at bf16, T > 64, E <= 256 with E <= 64 or a router
# matrix of at least 2 MB keeps K-split partial sums in the workspace (two
# kernels: screen partials, then selection; every tile shape: E <= 16, 32,
# 64, 128, 256); the same checks through moe_layer_forward, with f chosen so
# that the workspace holds the partials of at least one split.  The Zipf
# workload (E = 128, 0.5 MB) routes with the one-kernel screen.
SPLIT_ROUTE_CASES = ["screen_E8_long_d", "screen_zero_router", "split_zero_router_E100",
                     "screen_duplicate_rows", "split_E24_ragged", "split_E200_d5200",
                     "split_E16_T1000", "split_integer_exact", "fine_grained_zipf_full",
                     "deepseek_v3_full"]


def _split_case(name):
    n = moe_synth.normal
    if name == "split_E24_ragged":
        return n((60, 5, 0), (333, 264), 1.0, "bf16"), n((60, 5, 1), (24, 264), 0.05, "bf16"), \
            np.linspace(0.1, -0.1, 24).astype(np.float32), 3
    if name == "split_E200_d5200":
        # ragged last K step (5200 = 81 * 64 + 16)
        return n((61, 5, 0), (700, 5200), 1.0, "bf16"), n((61, 5, 1), (200, 5200), 0.02, "bf16"), \
            None, 6
    if name == "split_zero_router_E100":
        # every expert stays a candidate (more than 64): ranked in rounds
        return n((64, 5, 0), (90, 10496), 1.0, "bf16"), np.zeros((100, 10496), np.uint16), None, 5
    if name == "split_E16_T1000":
        return n((62, 5, 0), (1000, 512), 1.0, "bf16"), n((62, 5, 1), (16, 512), 0.05, "bf16"), \
            None, 2
    if name == "split_integer_exact":
        # exact logits and exact ties everywhere: ties go to the lower index
        return (moe_synth.to_bf16_bits(moe_synth.small_ints((63, 5, 0), (200, 136), -2, 2)),
                moe_synth.to_bf16_bits(moe_synth.small_ints((63, 5, 1), (48, 136), -1, 1)),
                None, 5)
    return _route_case(name)


@pytest.mark.parametrize("name", SPLIT_ROUTE_CASES)
def test_route_split(name):
    x, W, bias, k = _split_case(name)
    T, d = x.shape
    E = W.shape[0]
    assert x.dtype == np.uint16 and T > 64 and E <= 256
    # act + expert_out hold the partials of one split at least
    f = 8
    while T * k * (f + d) * 2 < T * E * 8 + (T + E) * 8 + 1024:
        f += 8
    print(f"route (layer workspace) {name}: T={T} d={d} E={E} k={k} f={f}", flush=True)
    s = moe.shape(T, d, f, E, k, 0, moe.MOE_DT_BF16)
    Wgu = torch.zeros(E, 2 * f, d, dtype=torch.bfloat16, device="cuda")
    Wd = torch.zeros(E, d, f, dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(s, dev(x), dev(W), dev(bias), Wgu, Wd, y, ws)
    _sync()
    views = moe.workspace_views(s, ws)
    idx, w = host(views["topk_idx"]), host(views["topk_w"])
    L, idx_ref, w_ref = oracle.route(x, W, k, bias=bias)
    amb = check_routing(idx, w, L, abs_scores(x, W), idx_ref, w_ref)
    assert len(amb) <= max(1, T // 1000), f"{len(amb)} near-tie tokens"
    if "zero_router" in name or "duplicate" in name or "integer" in name:
        assert not amb and np.array_equal(idx, idx_ref)
    # the standalone routers agree exactly: moe_route (one fused kernel) and
    # moe_route_ws (the layer's path, in a workspace of its own)
    idx_d, w_d = empty((T, k), "i32"), empty((T, k), "f32")
    moe.moe_route(s, dev(x), dev(W), dev(bias), idx_d, w_d)
    _sync()
    assert np.array_equal(host(idx_d), idx)
    assert np.array_equal(host(w_d), w)
    need = moe.route_workspace_size(s)
    rws = torch.empty(need, dtype=torch.uint8, device="cuda") if need else None
    idx_d.fill_(-1)
    w_d.fill_(0.0)
    moe.moe_route_ws(s, dev(x), dev(W), dev(bias), idx_d, w_d, rws)
    _sync()
    assert np.array_equal(host(idx_d), idx)
    assert np.array_equal(host(w_d), w)
    del ws
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- permute

PERMUTE_CASES = [
    # (T, E, k, S, zipf).  T*k >= 8192 copies with E <= 1023 take the
    # multi-workgroup kernels (2048 copies per workgroup), the rest one
    # workgroup: ragged last chunks (8196, 10500), the largest key count
    # (E = 1023), just below the switch (8190) and E = 1024 above it
    (16, 32, 4, 0, None), (37, 8, 2, 0, None), (1, 1, 1, 0, None), (0, 4, 2, 1, None),
    (4096, 128, 8, 0, 1.2), (4096, 256, 8, 1, None), (8192, 8, 2, 0, None),
    (300, 1000, 7, 24, None), (513, 1023, 64, 1, None), (2000, 64, 3, 2, 2.0),
    (2049, 1023, 4, 1, None), (1500, 60, 7, 2, 2.0), (1170, 7, 7, 0, None),
    (200, 1024, 64, 0, None),
]


@pytest.mark.parametrize("case", PERMUTE_CASES, ids=str)
def test_permute(case):
    T, E, k, S, zipf = case
    print(f"permute T={T} E={E} k={k} S={S} zipf={zipf}", flush=True)
    idx = moe_synth.random_routing((50, T, E), T, E, k, zipf) if T else \
        np.zeros((0, k), np.int32)
    s = moe.shape(T, 8, 8, E, k, S, moe.MOE_DT_BF16)
    G = E + S
    counts, offsets = empty((G,), "i32"), empty((G + 1,), "i32")
    ss, sp = empty((T * k,), "i32"), empty((T * k,), "i32")
    moe.moe_permute(s, dev(idx) if T else empty((0,), "i32"), counts, offsets, ss, sp)
    _sync()
    c_ref, o_ref, ss_ref, sp_ref = oracle.permute(idx, E, S)
    assert np.array_equal(host(counts), c_ref)
    assert np.array_equal(host(offsets), o_ref)
    assert np.array_equal(host(ss), ss_ref)
    assert np.array_equal(host(sp), sp_ref)


def _expect_with_invalid(idx, E, S, T, cap):
    """The documented layout when some ids lie outside [0, E): those copies
    first (slot order), then the copies over capacity (by expert, slot
    order), then each expert's kept copies; dropped copies get slot_pos -1."""
    flat = idx.ravel().astype(np.int64)
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    per = [np.flatnonzero(flat == e) for e in range(E)]
    rows = [np.flatnonzero(~valid)]
    rows += [p[cap:] for p in per]
    n_drop = sum(len(r) for r in rows)
    rows += [p[:cap] for p in per]
    ss = np.concatenate(rows).astype(np.int64)
    counts = np.array([min(len(p), cap) for p in per] + [T] * S, np.int64)
    offsets = np.concatenate([[n_drop], n_drop + np.cumsum(counts)])
    sp = np.full(n, -1, np.int64)
    sp[ss[n_drop:]] = np.arange(n_drop, n)
    return counts, offsets, ss, sp


@pytest.mark.parametrize("case", [(37, 8, 2, 0), (4096, 128, 8, 1), (1500, 60, 7, 2)], ids=str)
def test_permute_invalid_ids(case):
    """Ids outside [0, E) select no expert: their copies take the first rows,
    in slot order, with slot_pos -1 (one-workgroup and multi-workgroup
    forms, with and without a capacity)."""
    T, E, k, S = case
    idx = moe_synth.random_routing((51, T, E), T, E, k, None)
    rng = np.random.default_rng([51, T])
    flat = idx.ravel().copy()
    m = rng.random(flat.size) < 0.05
    flat[m] = rng.choice(np.array([-1, E, E + 7, -(1 << 30)], np.int32), int(m.sum()))
    idx = flat.reshape(idx.shape).astype(np.int32)
    s = moe.shape(T, 8, 8, E, k, S, moe.MOE_DT_BF16)
    G = E + S
    for cap in (None, max(1, T * k // E // 2)):
        print(f"permute invalid ids T={T} E={E} k={k} S={S} capacity={cap}", flush=True)
        counts, offsets = empty((G,), "i32"), empty((G + 1,), "i32")
        ss, sp = empty((T * k,), "i32"), empty((T * k,), "i32")
        if cap is None:
            moe.moe_permute(s, dev(idx), counts, offsets, ss, sp)
        else:
            moe.moe_permute_capacity(s, dev(idx), cap, counts, offsets, ss, sp)
        _sync()
        want = _expect_with_invalid(idx, E, S, T, T * k if cap is None else cap)
        for got, w, what in zip((counts, offsets, ss, sp), want,
                                ("counts", "offsets", "sorted_slot", "slot_pos")):
            assert np.array_equal(host(got), w), f"{what} differs (capacity {cap})"


# ----------------------------------------------------------- expert GEMMs

def _rows_of(idx, ss, T, k, E, S):
    """(token, expert) of every permuted row, from an oracle permutation."""
    tok = np.concatenate([ss // k, np.tile(np.arange(T), S)]).astype(np.int64)
    ex = np.concatenate([idx.ravel()[ss], np.repeat(np.arange(E, E + S), T)]).astype(np.int32)
    return tok, ex


GEMM_CASES = [
    # (name, T, d, f, E, k, S, dtype, zipf)
    ("decode_gpt_oss_shape", 16, 2880, 2880, 32, 4, 0, "bf16", None),
    ("decode_T1_k1", 1, 512, 264, 4, 1, 0, "bf16", None),
    ("decode_T50_shared", 50, 320, 200, 12, 3, 1, "bf16", None),
    ("tiled_ragged_shared", 300, 256, 200, 6, 2, 1, "bf16", None),
    ("tiled_zipf_empty_experts", 700, 520, 136, 24, 4, 0, "bf16", 1.5),
    ("tiled_one_big_group", 400, 192, 384, 3, 1, 0, "bf16", 3.0),
    ("tiled_T65", 65, 128, 64, 2, 2, 0, "bf16", None),
    # >= 512 rows per group on average: the 256-row tiles; K % 32 = 8 in both GEMMs
    ("tiled_bm256_ragged_k", 1100, 264, 136, 2, 1, 0, "bf16", None),
    # routed groups of 112-168 rows on average: the 192-row tiles (ragged K,
    # a shared expert, several bands of n-tiles)
    ("tiled_bm192_ragged_k", 700, 264, 200, 10, 2, 0, "bf16", None),
    ("tiled_bm192_shared", 520, 520, 136, 4, 1, 1, "bf16", None),
    ("tiled_bm192_bands", 300, 1280, 1216, 4, 2, 0, "bf16", None),
    # K shorter than one K tile (40 and 24): one partly zero-filled tile
    ("tiled_k_below_tile", 100, 40, 24, 4, 2, 0, "bf16", None),
    # the most expert groups the library takes (E + S = 1024)
    ("tiled_1024_groups", 128, 64, 32, 1000, 2, 24, "bf16", None),
    ("f32_tiny_shape", 128, 256, 512, 8, 2, 0, "f32", None),
    ("f32_ragged_shared", 90, 72, 40, 5, 2, 2, "f32", 1.0),
    # many n-tiles: gate_up has ceil(1160/128) = 10 (bands of 4: 4, 4, 2), down
    # ceil(1288/256) = 6 (4, 2), so the tile order runs over several bands
    # and a partial last band; 128-row tiles (200 rows per group on average)
    ("tiled_bands_bm128", 600, 1288, 1160, 6, 2, 0, "bf16", None),
    # the same n-tiling on the 256-row tiles (600 rows per group on average)
    ("tiled_bands_bm256", 1200, 1288, 1160, 2, 1, 0, "bf16", None),
    # 140 routed rows per group on average, Zipf-skewed (328, 123, 59 and 50 rows
    # with this seed): the weight-panel kernel with each of its row-block counts
    # (12 and 10 for the two m-tiles of the largest group, then 8 and 6)
    ("panel_row_blocks", 560, 264, 136, 4, 1, 0, "bf16", 1.5),
]


def _gemm_inputs(case):
    name, T, d, f, E, k, S, dtype, zipf = case
    seed = 60 + GEMM_CASES.index(case)
    x = moe_synth.normal((seed, 5, 0), (T, d), 1.0, dtype)
    Wgu = moe_synth.normal((seed, 5, 2), (E + S, 2 * f, d), 0.05, dtype)
    Wd = moe_synth.normal((seed, 5, 3), (E + S, d, f), 0.05, dtype)
    idx = moe_synth.random_routing((seed, 5, 4), T, E, k, zipf)
    counts, offsets, ss, sp = oracle.permute(idx, E, S)
    return x, Wgu, Wd, idx, counts, offsets, ss, sp


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: c[0])
def test_gate_up(case):
    name, T, d, f, E, k, S, dtype, zipf = case
    print(f"gate_up {case}", flush=True)
    x, Wgu, Wd, idx, counts, offsets, ss, sp = _gemm_inputs(case)
    R = T * k + S * T
    s = moe.shape(T, d, f, E, k, S, dt_code(dtype))
    act = empty((R, f), dtype)
    act.fill_(float("nan"))
    moe.moe_grouped_gemm_gate_up(s, dev(x), dev(ss), dev(offsets), dev(Wgu), act)
    _sync()
    tok, ex = _rows_of(idx, ss, T, k, E, S)
    ref = oracle.gate_up_rows(x, Wgu, tok, ex)
    assert_rows_close(host(act), ref, dtype, f"gate_up {name}")


@pytest.mark.parametrize("case", GEMM_CASES, ids=lambda c: c[0])
def test_down(case):
    name, T, d, f, E, k, S, dtype, zipf = case
    print(f"down {case}", flush=True)
    x, Wgu, Wd, idx, counts, offsets, ss, sp = _gemm_inputs(case)
    R = T * k + S * T
    act = moe_synth.normal((70, 5, 0), (R, f), 0.5, dtype)
    s = moe.shape(T, d, f, E, k, S, dt_code(dtype))
    out = empty((R, d), dtype)
    out.fill_(float("nan"))
    moe.moe_grouped_gemm_down(s, dev(act), dev(offsets), dev(Wd), out)
    _sync()
    tok, ex = _rows_of(idx, ss, T, k, E, S)
    ref = oracle.down_rows(act, Wd, ex)
    assert_rows_close(host(out), ref, dtype, f"down {name}")


@pytest.mark.parametrize("case", GEMM_CASES[:4], ids=lambda c: c[0])
def test_grouped_gemm_both(case):
    """moe_grouped_gemm = gate_up then down on the same buffers."""
    name, T, d, f, E, k, S, dtype, zipf = case
    x, Wgu, Wd, idx, counts, offsets, ss, sp = _gemm_inputs(case)
    R = T * k + S * T
    s = moe.shape(T, d, f, E, k, S, dt_code(dtype))
    act, out = empty((R, f), dtype), empty((R, d), dtype)
    moe.moe_grouped_gemm(s, dev(x), dev(ss), dev(offsets), dev(Wgu), dev(Wd), act, out)
    _sync()
    tok, ex = _rows_of(idx, ss, T, k, E, S)
    ref_act = oracle.gate_up_rows(x, Wgu, tok, ex)
    assert_rows_close(host(act), ref_act, dtype, f"act {name}")
    # the down projection of the oracle's activation
    ref_out = oracle.down_rows(ref_act.astype(np.float32), moe_synth.bf16_bits_to_f32(Wd)
                               if dtype == "bf16" else Wd, ex)
    assert_rows_close(host(out), ref_out, dtype, f"out {name}")


# ---------------------------------------------------------------- combine

COMBINE_CASES = [(16, 2880, 32, 4, 0, "bf16"), (128, 256, 8, 2, 0, "f32"),
                 (77, 264, 10, 3, 2, "bf16"), (1, 8, 1, 1, 1, "f32"),
                 (4096, 7168, 256, 8, 1, "bf16")]


@pytest.mark.parametrize("case", COMBINE_CASES, ids=str)
def test_combine(case):
    T, d, E, k, S, dtype = case
    print(f"combine {case}", flush=True)
    idx = moe_synth.random_routing((80, T, E), T, E, k)
    counts, offsets, ss, sp = oracle.permute(idx, E, S)
    R = T * k + S * T
    O = moe_synth.normal((80, 5, 1), (R, d), 1.0, dtype)
    w = moe_synth.random_unit((80, 5, 2), (T, k))
    s = moe.shape(T, d, 8, E, k, S, dt_code(dtype))
    y = empty((T, d), dtype)
    moe.moe_combine(s, dev(O), dev(sp), dev(w), y)
    _sync()
    ref = oracle.combine(O, sp, w.astype(np.float64), T, k, S)
    assert_rows_close(host(y), ref, dtype, "combine")
