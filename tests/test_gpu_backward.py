"""Backward pass on the GPU (moe_layer_backward after moe_layer_forward)
against the oracle's gradients (oracle.layer_backward, pinned to torch
autograd and central differences).

Comparison: gradients are fp32 on the GPU from bf16 operands, with dO and
dH rounded to bf16, so the rule is the bf16 one, per row of every gradient
(a token's dx, a weight-gradient row): ||got - ref|| <= 2e-2 ||ref|| plus
1e-3 of the largest row norm of that tensor (rows of an expert with one or
two tokens can nearly cancel).  Repeated calls are bitwise identical."""
import numpy as np
import pytest

import moe_synth
import oracle
import mixture_experts_sparse_router_amd as moe
from gpu_util import dev, host, layer_inputs_to_device

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def assert_grad_rows(got, ref, what, tol=2e-2, floor=1e-3):
    ref = np.asarray(ref, np.float64)
    ref = ref.reshape(-1, ref.shape[-1]) if ref.ndim > 1 else ref.reshape(1, -1)
    got = np.asarray(got, np.float64).reshape(ref.shape)
    num = np.linalg.norm(got - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    lim = tol * den + floor * max(den.max(), 1e-300)
    bad = num > lim
    assert not bad.any(), (f"{what}: {int(bad.sum())} rows off, worst ratio "
                           f"{float((num / np.maximum(den, 1e-300)).max()):.3e}")
    return float((num / np.maximum(den, 1e-30)).max())


def run_fwd_bwd(cfg, dinp, dy):
    s = moe.shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.S, moe.MOE_DT_BF16)
    fws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward(s, dinp["x"], dinp["W_router"], dinp["bias"], dinp["W_gate_up"],
                          dinp["W_down"], y, fws)
    G = cfg.E + cfg.S
    out = {"dx": torch.empty(cfg.T, cfg.d, device="cuda"),
           "dW_router": torch.empty(cfg.E, cfg.d, device="cuda"),
           "db": torch.empty(cfg.E, device="cuda"),
           "dW_gate_up": torch.empty(G, 2 * cfg.f, cfg.d, device="cuda"),
           "dW_down": torch.empty(G, cfg.d, cfg.f, device="cuda"),
           "dw": torch.empty(cfg.T, cfg.k, device="cuda")}
    bws = torch.empty(moe.backward_workspace_size(s), dtype=torch.uint8, device="cuda")
    moe.moe_layer_backward(s, dinp["x"], dinp["W_router"], dinp["W_gate_up"], dinp["W_down"],
                           dy, fws, out["dx"], out["dW_router"], out["db"], out["dW_gate_up"],
                           out["dW_down"], out["dw"], bws)
    torch.cuda.synchronize()
    return s, fws, bws, out


BWD_CASES = [
    # (T, d, f, E, k, S, zipf, seed): decode and prefill sizes, several
    # 128-tiles in every dimension with ragged tails, empty experts, shared
    (16, 136, 200, 6, 2, 0, None, 1),
    (70, 264, 136, 5, 2, 1, None, 2),
    (300, 128, 256, 12, 3, 0, 1.2, 3),
    (9, 64, 40, 8, 4, 2, 1.2, 4),
    # the recomputed H through the forward's 192-row tiles (routed groups of
    # 140 rows on average) and 256-row tiles (groups of 600 rows)
    (140, 136, 200, 4, 4, 0, None, 5),
    (600, 128, 136, 2, 2, 1, None, 6),
    # groups of at least 512 rows on average: the expert-gradient GEMMs in
    # 256 x 256 tiles, several of them in every dimension with ragged tails
    (1100, 520, 264, 2, 1, 0, None, 7),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=str)
def test_backward_small(case):
    T, d, f, E, k, S, zipf, seed = case
    print(f"backward T={T} d={d} f={f} E={E} k={k} S={S} zipf={zipf}", flush=True)
    cfg = moe_synth.tiny_config(T=T, d=d, f=f, E=E, k=k, S=S, dtype="bf16", zipf_s=zipf)
    cfg = cfg.scaled(w_std=0.08)
    inp = moe_synth.make_layer_inputs(cfg, 70 + seed)
    dyh = moe_synth.normal((70 + seed, 8, 0), (T, d), 1.0, "bf16")
    dinp = layer_inputs_to_device(inp)
    s, fws, bws, out = run_fwd_bwd(cfg, dinp, dev(dyh))
    ref = oracle.layer_backward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"], dyh,
                                k, S=S, bias=inp["bias"], experts=np.arange(E + S))
    idx = host(moe.workspace_views(s, fws)["topk_idx"])
    _, idx_ref, _ = oracle.route(inp["x"], inp["W_router"], k, bias=inp["bias"])
    assert np.array_equal(idx, idx_ref)
    worst = {}
    for name in ("dx", "dW_router", "dW_gate_up", "dW_down"):
        worst[name] = assert_grad_rows(host(out[name]), ref[name], name)
    db, db_ref = host(out["db"]), ref["db"]
    assert np.all(np.abs(db - db_ref) <= 2e-2 * np.abs(db_ref) + 1e-3 * np.abs(db_ref).max())
    # dw_tj = dy_t . O_tj with O rounded to bf16 by the forward: the error of
    # a dot product of rounded operands is bounded relative to sum |dy_i O_i|
    views = moe.workspace_views(s, fws)
    O = moe_synth.bf16_bits_to_f32(host(views["expert_out"])).astype(np.float64)
    sp = host(views["slot_pos"]).reshape(T, k)
    dyw = moe_synth.bf16_bits_to_f32(dyh).astype(np.float64)
    cond = np.einsum("tjd,td->tj", np.abs(O[sp]), np.abs(dyw))
    dw, dw_ref = host(out["dw"]), ref["dw"]
    assert np.all(np.abs(dw - dw_ref) <= 2e-2 * cond), float((np.abs(dw - dw_ref) / cond).max())
    # experts without tokens: exactly zero gradients
    counts = host(moe.workspace_views(s, fws)["counts"])
    empty_e = np.nonzero(counts[:E] == 0)[0]
    assert np.all(host(out["dW_gate_up"])[empty_e] == 0)
    assert np.all(host(out["dW_down"])[empty_e] == 0)
    assert np.all(host(out["dW_router"])[empty_e] == 0)
    # repeated calls are bitwise identical
    again = {k2: torch.empty_like(v) for k2, v in out.items()}
    moe.moe_layer_backward(s, dinp["x"], dinp["W_router"], dinp["W_gate_up"], dinp["W_down"],
                           dev(dyh), fws, again["dx"], again["dW_router"], again["db"],
                           again["dW_gate_up"], again["dW_down"], again["dw"], bws)
    torch.cuda.synchronize()
    for name in out:
        assert torch.equal(out[name], again[name]), name
    print("  worst row rel err " + ", ".join(f"{k2} {v:.2e}" for k2, v in worst.items()),
          flush=True)


CAP_CASES = [
    # (T, d, f, E, k, S, zipf, capacity factor, seed): skewed routing so that
    # the popular experts drop copies; capacity 0 drops every routed copy;
    # the last case runs the multi-workgroup permutation (T*k >= 8192)
    (64, 136, 200, 6, 2, 1, 1.2, 1.0, 11),
    (33, 64, 72, 5, 3, 0, 1.5, 0.6, 12),
    (20, 64, 40, 4, 2, 1, None, 0.0, 13),
    (4200, 64, 64, 8, 2, 0, 1.1, 1.25, 14),
]


@pytest.mark.parametrize("case", CAP_CASES, ids=str)
def test_backward_capacity(case):
    """moe_layer_backward after moe_layer_forward_capacity against the
    oracle's gradients of the capacity forward (pinned by central
    differences): dropped copies add no expert gradient, get dw = 0, and
    their logits keep dl."""
    T, d, f, E, k, S, zipf, factor, seed = case
    print(f"backward capacity T={T} d={d} f={f} E={E} k={k} S={S} factor={factor}", flush=True)
    cfg = moe_synth.tiny_config(T=T, d=d, f=f, E=E, k=k, S=S, dtype="bf16", zipf_s=zipf)
    cfg = cfg.scaled(w_std=0.08)
    inp = moe_synth.make_layer_inputs(cfg, 90 + seed)
    dyh = moe_synth.normal((90 + seed, 8, 0), (T, d), 1.0, "bf16")
    dinp = layer_inputs_to_device(inp)
    C = oracle.expert_capacity(T, k, E, factor)
    s = moe.shape(T, d, f, E, k, S, moe.MOE_DT_BF16)
    fws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    y = torch.empty(T, d, dtype=torch.bfloat16, device="cuda")
    moe.moe_layer_forward_capacity(s, dinp["x"], dinp["W_router"], dinp["bias"],
                                   dinp["W_gate_up"], dinp["W_down"], C, y, fws)
    G = E + S
    out = {"dx": torch.empty(T, d, device="cuda"),
           "dW_router": torch.empty(E, d, device="cuda"),
           "db": torch.empty(E, device="cuda"),
           "dW_gate_up": torch.empty(G, 2 * f, d, device="cuda"),
           "dW_down": torch.empty(G, d, f, device="cuda"),
           "dw": torch.empty(T, k, device="cuda")}
    bws = torch.empty(moe.backward_workspace_size(s), dtype=torch.uint8, device="cuda")
    moe.moe_layer_backward(s, dinp["x"], dinp["W_router"], dinp["W_gate_up"], dinp["W_down"],
                           dev(dyh), fws, out["dx"], out["dW_router"], out["db"],
                           out["dW_gate_up"], out["dW_down"], out["dw"], bws)
    torch.cuda.synchronize()
    views = moe.workspace_views(s, fws)
    sp = host(views["slot_pos"]).reshape(T, k)
    dropped = sp < 0
    _, idx_ref, _ = oracle.route(inp["x"], inp["W_router"], k, bias=inp["bias"])
    _, _, _, sp_ref = oracle.permute(idx_ref, E, S, capacity=C)
    assert np.array_equal(sp, sp_ref.reshape(T, k))
    assert dropped.any()
    ref = oracle.layer_backward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"], dyh,
                                k, S=S, bias=inp["bias"], experts=np.arange(G), capacity=C)
    worst = {}
    for name in ("dx", "dW_router", "dW_gate_up", "dW_down"):
        worst[name] = assert_grad_rows(host(out[name]), ref[name], name)
    db, db_ref = host(out["db"]), ref["db"]
    assert np.all(np.abs(db - db_ref) <= 2e-2 * np.abs(db_ref) + 1e-3 * np.abs(db_ref).max())
    dw = host(out["dw"])
    assert np.all(dw[dropped] == 0)
    # expert_out rows of dropped copies are never written: read kept rows only
    kept = ~dropped
    tk, jk = np.nonzero(kept)
    O = moe_synth.bf16_bits_to_f32(host(views["expert_out"])[sp[kept]]).astype(np.float64)
    dyw = moe_synth.bf16_bits_to_f32(dyh).astype(np.float64)
    cond = np.einsum("cd,cd->c", np.abs(O), np.abs(dyw[tk]))
    assert np.all(np.abs(dw[tk, jk] - ref["dw"][tk, jk]) <= 2e-2 * cond)
    # experts whose every copy was dropped (or that none selected): zero
    # expert gradients; their router rows still move (the dropped logits)
    counts = host(views["counts"])[:E]
    empty_e = np.nonzero(counts == 0)[0]
    assert np.all(host(out["dW_gate_up"])[empty_e] == 0)
    assert np.all(host(out["dW_down"])[empty_e] == 0)
    print(f"  capacity {C}, {int(dropped.sum())} of {T * k} copies dropped; worst row rel err "
          + ", ".join(f"{k2} {v:.2e}" for k2, v in worst.items()), flush=True)


def test_backward_decode_full():
    """The gpt-oss-20b-shaped decode layer (T=16, d=f=2880, E=32, top-4):
    every gradient."""
    cfg = moe_synth.CONFIGS[2]
    inp = moe_synth.make_layer_inputs(cfg, 2)
    dyh = moe_synth.normal((2, 8, 0), (cfg.T, cfg.d), 1.0, "bf16")
    dinp = layer_inputs_to_device(inp)
    s, fws, bws, out = run_fwd_bwd(cfg, dinp, dev(dyh))
    ref = oracle.layer_backward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"], dyh,
                                cfg.k, S=cfg.S, bias=inp["bias"],
                                experts=np.arange(cfg.E + cfg.S))
    for name in ("dx", "dW_router", "dW_gate_up", "dW_down"):
        w = assert_grad_rows(host(out[name]), ref[name], name)
        print(f"  {name}: worst row rel err {w:.2e}", flush=True)


def test_backward_fine_grained_zipf_sampled():
    """The Zipf-skewed workload at full size (T=4096, E=128, top-8): dx of
    sampled tokens and the weight gradients of sampled experts (one of the
    largest groups and two small ones), against the oracle."""
    cfg = moe_synth.CONFIGS[4]
    inp = moe_synth.make_layer_inputs(cfg, 4)
    dyh = moe_synth.normal((4, 8, 0), (cfg.T, cfg.d), 1.0, "bf16")
    dinp = layer_inputs_to_device(inp)
    s, fws, bws, out = run_fwd_bwd(cfg, dinp, dev(dyh))
    counts = host(moe.workspace_views(s, fws)["counts"])[:cfg.E]
    order = np.argsort(counts)
    small = [int(e) for e in order if counts[e] > 0][:2]
    mid = int(np.argmin(np.abs(counts - 300)))       # a few hundred rows: several m-tiles
    experts = [mid] + [e for e in small if e != mid]
    toks = np.unique(np.linspace(0, cfg.T - 1, 12).astype(np.int64))
    ref = oracle.layer_backward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"], dyh,
                                cfg.k, S=cfg.S, bias=inp["bias"], tokens=toks,
                                experts=experts, router=False)
    assert_grad_rows(host(out["dx"])[toks], ref["dx"], "dx")
    assert_grad_rows(host(out["dW_gate_up"])[experts], ref["dW_gate_up"], "dW_gate_up")
    assert_grad_rows(host(out["dW_down"])[experts], ref["dW_down"], "dW_down")
    print(f"  experts {experts} with {counts[experts].tolist()} rows", flush=True)
    torch.cuda.empty_cache()
