"""Router auxiliaries on the GPU against the fp64 oracle: the load-balance
statistics and loss (moe_route_balance) and the expert-capacity variant
(moe_permute_capacity, moe_layer_forward_capacity).

Rules: routing and permutations bit-exact (as everywhere); importance within
2e-2 relative per expert (the bf16 tolerance, which the screen's proven logit
bound also guarantees: at most 2^-14 ||x|| ||w|| <= 0.01 on these inputs,
so exp moves by under 2%); the loss within 2e-2 relative plus what the
measured importance errors can move it by, (1/E) max_e |log ratio|."""
import math

import numpy as np
import pytest

import moe_synth
import oracle
import mixture_experts_sparse_router_amd as moe
from gpu_util import (abs_scores, assert_rows_close, check_routing, dev, dt_code, empty,
                      host, layer_inputs_to_device)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _router_case(name):
    n = moe_synth.normal
    C = moe_synth.CONFIGS
    if name in ("tiny_fp32", "gpt_oss_20b_decode", "mixtral_prefill", "fine_grained_zipf_full",
                "deepseek_v3_full"):
        cid = {"tiny_fp32": 1, "gpt_oss_20b_decode": 2, "mixtral_prefill": 3,
               "fine_grained_zipf_full": 4, "deepseek_v3_full": 5}[name]
        inp = moe_synth.make_layer_inputs(C[cid], cid, experts=False)
        return inp["x"], inp["W_router"], inp["bias"], C[cid].k
    if name == "screen_E300_ragged":
        return n((48, 5, 0), (77, 136), 1.0, "bf16"), n((48, 5, 1), (300, 136), 0.1, "bf16"), \
            np.linspace(0.2, -0.3, 300).astype(np.float32), 6
    if name == "small_E1024":
        return n((45, 5, 0), (50, 64), 1.0, "bf16"), n((45, 5, 1), (1024, 64), 0.1, "bf16"), \
            None, 8
    if name == "screen_zero_router_E100":
        return n((52, 5, 0), (90, 96), 1.0, "bf16"), np.zeros((100, 96), np.uint16), None, 5
    if name == "tiled_f32_E600":
        return n((53, 5, 0), (70, 40), 1.0, "f32"), n((53, 5, 1), (600, 40), 0.3, "f32"), \
            np.linspace(-0.4, 0.4, 600).astype(np.float32), 3
    raise KeyError(name)


BALANCE_CASES = ["tiny_fp32", "gpt_oss_20b_decode", "screen_E300_ragged", "small_E1024",
                 "screen_zero_router_E100", "tiled_f32_E600", "mixtral_prefill",
                 "fine_grained_zipf_full", "deepseek_v3_full"]


def _route_balance(s, x, W, bias):
    ws = torch.empty(moe.route_balance_workspace_size(s), dtype=torch.uint8, device="cuda")
    idx, w = empty((s.T, s.k), "i32"), empty((s.T, s.k), "f32")
    imp = torch.empty(s.E, dtype=torch.float64, device="cuda")
    loss = torch.empty(1, dtype=torch.float64, device="cuda")
    moe.moe_route_balance(s, x, W, bias, idx, w, imp, loss, ws)
    torch.cuda.synchronize()
    return host(idx), host(w), host(imp), float(host(loss)[0])


@pytest.mark.parametrize("name", BALANCE_CASES)
def test_route_balance(name):
    x, W, bias, k = _router_case(name)
    dtype = "bf16" if x.dtype == np.uint16 else "f32"
    T, d = x.shape
    E = W.shape[0]
    print(f"route_balance {name}: T={T} d={d} E={E} k={k} {dtype}", flush=True)
    s = moe.shape(T, d, 8, E, k, 0, dt_code(dtype))
    xd, Wd, bd = dev(x), dev(W), dev(bias)
    idx, w, imp, loss = _route_balance(s, xd, Wd, bd)
    # the routing is moe_route's, bit for bit
    idx_r, w_r = empty((T, k), "i32"), empty((T, k), "f32")
    moe.moe_route(s, xd, Wd, bd, idx_r, w_r)
    torch.cuda.synchronize()
    assert np.array_equal(idx, host(idx_r)) and np.array_equal(w, host(w_r))
    L, idx_ref, w_ref = oracle.route(x, W, k, bias=bias)
    amb = check_routing(idx, w, L, abs_scores(x, W), idx_ref, w_ref)
    assert len(amb) <= max(1, T // 1000)
    # statistics
    imp_ref, loss_ref = oracle.balance(x, W, bias=bias)
    rel = np.abs(imp - imp_ref) / np.maximum(imp_ref, 1e-300)
    assert np.all((rel <= 2e-2) | (np.abs(imp - imp_ref) <= 1e-12)), \
        f"importance: worst rel err {rel.max():.3e} at expert {int(rel.argmax())}"
    assert abs(imp.sum() - 1.0) <= 1e-6
    moved = np.max(np.abs(np.log((imp + 1e-8) / (imp_ref + 1e-8)))) / E
    assert abs(loss - loss_ref) <= 2e-2 * abs(loss_ref) + moved + 1e-15, (loss, loss_ref)
    print(f"  importance worst rel err {rel.max():.3e}, loss {loss:.9e} vs {loss_ref:.9e} "
          f"(rel {abs(loss - loss_ref) / abs(loss_ref):.2e})", flush=True)
    # repeated calls are bitwise identical
    _, _, imp2, loss2 = _route_balance(s, xd, Wd, bd)
    assert np.array_equal(imp, imp2) and loss == loss2


def test_route_balance_empty_batch():
    """No tokens: the mean over no tokens is NaN, and so is the loss."""
    s = moe.shape(0, 64, 8, 6, 2, 0, moe.MOE_DT_BF16)
    W = dev(moe_synth.normal((54, 5, 1), (6, 64), 0.1, "bf16"))
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    idx, w = empty((0, 2), "i32"), empty((0, 2), "f32")
    imp = torch.zeros(6, dtype=torch.float64, device="cuda")
    loss = torch.zeros(1, dtype=torch.float64, device="cuda")
    ws = torch.empty(max(1, moe.route_balance_workspace_size(s)), dtype=torch.uint8,
                     device="cuda")
    moe.moe_route_balance(s, x, W, None, idx, w, imp, loss, ws)
    torch.cuda.synchronize()
    assert np.all(np.isnan(host(imp))) and math.isnan(float(host(loss)[0]))


# ------------------------------------------------------------ capacity

CAPACITY_CASES = [
    # (T, E, k, S, zipf, capacities)
    (16, 32, 4, 0, None, (0, 1, 2)),
    (37, 8, 2, 0, None, (3, 9, 37)),
    (4096, 128, 8, 0, 1.2, (0, 1, 256, 320, 512)),
    (4096, 256, 8, 1, None, (128, 160)),
    (8192, 8, 2, 0, None, (1024, 2048, 2200)),
    (513, 1023, 64, 1, None, (10, 40)),
    (0, 4, 2, 1, None, (0, 5)),
]


@pytest.mark.parametrize("case", CAPACITY_CASES, ids=str)
def test_permute_capacity(case):
    T, E, k, S, zipf, caps = case
    idx = moe_synth.random_routing((55, T, E), T, E, k, zipf) if T else np.zeros((0, k), np.int32)
    s = moe.shape(T, 8, 8, E, k, S, moe.MOE_DT_BF16)
    G = E + S
    di = dev(idx)
    for C in caps:
        print(f"permute_capacity T={T} E={E} k={k} S={S} zipf={zipf} capacity={C}", flush=True)
        counts, offsets = empty((G,), "i32"), empty((G + 1,), "i32")
        ss, sp = empty((T * k,), "i32"), empty((T * k,), "i32")
        moe.moe_permute_capacity(s, di, C, counts, offsets, ss, sp)
        torch.cuda.synchronize()
        ref = oracle.permute(idx, E, S, capacity=C)
        for got, want, what in zip((counts, offsets, ss, sp), ref,
                                   ("counts", "offsets", "sorted_slot", "slot_pos")):
            assert np.array_equal(host(got), want), f"{what} differs at capacity {C}"


def _run_capacity_layer(cfg, dinp, C):
    s = moe.shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.S, dt_code(cfg.dtype))
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = empty((cfg.T, cfg.d), cfg.dtype)
    moe.moe_layer_forward_capacity(s, dinp["x"], dinp["W_router"], dinp["bias"],
                                   dinp["W_gate_up"], dinp["W_down"], C, y, ws)
    torch.cuda.synchronize()
    return host(y), moe.workspace_views(s, ws)


def _sample(T, n=24):
    if T <= n:
        return np.arange(T)
    return np.unique(np.linspace(0, T - 1, n).astype(np.int64))


@pytest.mark.parametrize("cid,factors", [(1, (0.5, 1.0)), (2, (0.0, 1.0)), (4, (1.25,))])
def test_layer_capacity(cid, factors):
    """The layer with a capacity from a capacity factor (1.0 to 2.0 on the
    yunthe page, section 5.2; smaller ones force drops on uniform loads)
    against the oracle; the permutation is the oracle's; tokens that keep
    every copy get bitwise the output of the layer without a capacity."""
    cfg = moe_synth.CONFIGS[cid]
    inp = moe_synth.make_layer_inputs(cfg, cid)
    dinp = layer_inputs_to_device(inp)
    s = moe.shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.S, dt_code(cfg.dtype))
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y_free = empty((cfg.T, cfg.d), cfg.dtype)
    moe.moe_layer_forward(s, dinp["x"], dinp["W_router"], dinp["bias"], dinp["W_gate_up"],
                          dinp["W_down"], y_free, ws)
    torch.cuda.synchronize()
    y_free = host(y_free)
    for factor in factors:
        C = moe.expert_capacity(cfg.T, cfg.k, cfg.E, factor)
        assert C == oracle.expert_capacity(cfg.T, cfg.k, cfg.E, factor)
        print(f"layer_capacity {cfg.name}: factor {factor} -> capacity {C}", flush=True)
        y, views = _run_capacity_layer(cfg, dinp, C)
        idx = host(views["topk_idx"])
        ref = oracle.permute(idx, cfg.E, cfg.S, capacity=C)
        for what, want in zip(("counts", "offsets", "sorted_slot", "slot_pos"), ref):
            assert np.array_equal(host(views[what]), want), what
        kept = (ref[3] >= 0).reshape(cfg.T, cfg.k)
        toks = np.arange(cfg.T) if cfg.T <= 128 else _sample(cfg.T)
        y_ref, idx_ref, _ = oracle.layer_forward(inp["x"], inp["W_router"], inp["W_gate_up"],
                                                 inp["W_down"], cfg.k, S=cfg.S,
                                                 bias=inp["bias"], tokens=toks, capacity=C)
        assert np.array_equal(idx[toks], idx_ref)
        worst = assert_rows_close(y[toks], y_ref, cfg.dtype, f"{cfg.name} capacity {C}")
        full = kept.all(1)
        assert np.array_equal(y[full], y_free[full])
        print(f"  dropped {int((~kept).sum())} of {kept.size} copies, worst row rel err "
              f"{worst:.3e}", flush=True)
    torch.cuda.empty_cache()
