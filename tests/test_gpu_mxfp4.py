"""MXFP4 expert weights on the GPU against the fp64 oracle.

The oracle dequantises the MXFP4 tensors (oracle.dequant_mxfp4, pinned to
the specification's value table) into exact float32 weights and evaluates
the layer on them; the HIP path reads the packed codes and scales itself.
  - dequantisation is checked bit for bit: a down GEMM whose activation rows
    are one-hot returns single weights, which bf16 holds exactly;
  - the GEMMs and the layer within the bf16 tolerance (2e-2 per row);
  - routing and the permutation the layer's gate_up kernel writes
    bit-exact (they do not depend on the expert weights)."""
import numpy as np
import pytest

import moe_synth
import oracle
import mixture_experts_sparse_router_amd as moe
from gpu_util import assert_rows_close, dev, empty, host

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _bf16_bits(v64):
    """Exact bf16 bit patterns of values that are bf16 numbers."""
    bits = moe_synth.to_bf16_bits(np.asarray(v64, np.float32))
    assert np.array_equal(moe_synth.bf16_bits_to_f32(bits).astype(np.float64),
                          np.asarray(v64, np.float64)), "not a bf16 number"
    return bits


def _groups(counts, S=0, T=0):
    counts = list(counts) + [T] * S
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return np.array(counts, np.int32), offsets


@pytest.mark.parametrize("scale_range", [(100, 140), (10, 245)], ids=["mid", "wide"])
def test_mxfp4_dequant_bit_exact(scale_range):
    """out[r, i] = W[e_r, i, n_r] exactly when act row r is one-hot at n_r."""
    T, d, f, E = 40, 96, 160, 3
    counts, offsets = _groups([17, 0, 23])
    R = int(offsets[-1])
    s = moe.shape(T, d, f, E, 1, 0, moe.MOE_DT_BF16)
    q, sc = moe_synth.mxfp4((60, 1, scale_range[0]), E * d, f, scale_range)
    q, sc = q.reshape(E, d, f // 2), sc.reshape(E, d, f // 32)
    rng = np.random.default_rng([60, 2])
    n_r = rng.integers(0, f, size=R)
    act = np.zeros((R, f), np.float32)
    act[np.arange(R), n_r] = 1.0
    out = empty((R, d), "bf16")
    moe.moe_grouped_gemm_down_mxfp4(s, dev(moe_synth.to_bf16_bits(act)), dev(offsets),
                                    dev(q), dev(sc), out)
    torch.cuda.synchronize()
    W = oracle.dequant_mxfp4(q, sc)                   # [E, d, f]
    e_r = np.repeat(np.arange(E), counts)
    want = W[e_r, :, n_r]                             # [R, d]
    got = moe_synth.bf16_bits_to_f32(host(out)).astype(np.float64)
    _bf16_bits(want)  # every weight is a bf16 number
    # equal as numbers (a -0 weight comes back as +0: 0 + (-0) * 1 = +0)
    assert np.array_equal(got, want), \
        f"{int((got != want).sum())} of {got.size} weights differ"


GEMM_CASES = [
    # (T, d, f, E, k, S, seed): decode shapes, ragged row counts, empty
    # experts, 1..4 row blocks of 16, a shared expert, K steps past the row
    (16, 2880, 2880, 32, 4, 0, 1),
    (1, 64, 32, 4, 1, 0, 2),
    (64, 160, 96, 8, 2, 1, 3),
    (37, 96, 224, 5, 3, 0, 4),
    (20, 288, 64, 7, 2, 0, 5),
    (48, 544, 352, 12, 1, 2, 6),
]


def _gemm_case(T, d, f, E, k, S, seed):
    cfg = moe_synth.tiny_config(T=T, d=d, f=f, E=E, k=k, S=S, dtype="bf16")
    x = moe_synth.normal((61, seed, 0), (T, d), 1.0, "bf16")
    idx = moe_synth.random_routing((61, seed, 1), T, E, k, 1.5 if E > 4 else None)
    mx = moe_synth.make_mxfp4_experts(cfg, 61 * 100 + seed)
    return cfg, x, idx, mx


@pytest.mark.parametrize("case", GEMM_CASES, ids=str)
def test_mxfp4_gemms(case):
    T, d, f, E, k, S, seed = case
    print(f"mxfp4 gemms T={T} d={d} f={f} E={E} k={k} S={S}", flush=True)
    cfg, x, idx, mx = _gemm_case(*case)
    s = moe.shape(T, d, f, E, k, S, moe.MOE_DT_BF16)
    counts, offsets, ss, sp = oracle.permute(idx, E, S)
    R = s.R
    act = empty((R, f), "bf16")
    out = empty((R, d), "bf16")
    d_off, d_ss = dev(offsets), dev(ss)
    moe.moe_grouped_gemm_gate_up_mxfp4(s, dev(x), d_ss, d_off, dev(mx["Wq_gate_up"]),
                                       dev(mx["Ws_gate_up"]), act)
    moe.moe_grouped_gemm_down_mxfp4(s, act, d_off, dev(mx["Wq_down"]), dev(mx["Ws_down"]), out)
    torch.cuda.synchronize()
    tok = np.concatenate([ss // k, np.tile(np.arange(T), S)]).astype(np.int64)
    ex = np.concatenate([idx.ravel()[ss], np.repeat(np.arange(E, E + S), T)]).astype(np.int32)
    wgu = oracle.dequant_mxfp4(mx["Wq_gate_up"], mx["Ws_gate_up"]).astype(np.float32)
    wd = oracle.dequant_mxfp4(mx["Wq_down"], mx["Ws_down"]).astype(np.float32)
    x32 = moe_synth.bf16_bits_to_f32(x)
    act_ref = oracle.gate_up_rows(x32, wgu, tok, ex)
    a = host(act)
    assert_rows_close(a, act_ref, "bf16", "gate_up mxfp4")
    # down on the GPU's own activations (rounded to bf16, as the layer does)
    out_ref = oracle.down_rows(moe_synth.bf16_bits_to_f32(a), wd, ex)
    assert_rows_close(host(out), out_ref, "bf16", "down mxfp4")


@pytest.mark.parametrize("seed", [2, 12])
def test_mxfp4_layer_decode(seed):
    """The gpt-oss-20b-shaped decode layer with MXFP4 expert weights, every
    token, against the oracle on the dequantised weights; two calls are
    bitwise identical."""
    cfg = moe_synth.CONFIGS[2]
    print(f"mxfp4 layer {cfg.name} seed={seed}", flush=True)
    inp = moe_synth.make_layer_inputs(cfg, seed, experts=False)
    mx = moe_synth.make_mxfp4_experts(cfg, seed)
    s = moe.shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.S, moe.MOE_DT_BF16)
    ws = torch.empty(moe.workspace_size(s), dtype=torch.uint8, device="cuda")
    dm = {k: dev(v) for k, v in mx.items()}
    ys = []
    for _ in range(2):
        y = empty((cfg.T, cfg.d), "bf16")
        moe.moe_layer_forward_mxfp4(s, dev(inp["x"]), dev(inp["W_router"]), dev(inp["bias"]),
                                    dm["Wq_gate_up"], dm["Ws_gate_up"], dm["Wq_down"],
                                    dm["Ws_down"], y, ws)
        torch.cuda.synchronize()
        ys.append(host(y))
    assert np.array_equal(ys[0], ys[1])
    views = moe.workspace_views(s, ws)
    wgu = oracle.dequant_mxfp4(mx["Wq_gate_up"], mx["Ws_gate_up"]).astype(np.float32)
    wd = oracle.dequant_mxfp4(mx["Wq_down"], mx["Ws_down"]).astype(np.float32)
    x32 = moe_synth.bf16_bits_to_f32(inp["x"])
    wr32 = moe_synth.bf16_bits_to_f32(inp["W_router"])
    y_ref, idx_ref, w_ref = oracle.layer_forward(x32, wr32, wgu, wd, cfg.k, S=cfg.S,
                                                 bias=inp["bias"])
    assert np.array_equal(host(views["topk_idx"]), idx_ref)
    assert np.max(np.abs(host(views["topk_w"]) - w_ref)) <= 1e-6
    # the permutation, written by the gate_up kernel itself
    for got, want, what in zip((views["counts"], views["offsets"], views["sorted_slot"],
                                views["slot_pos"]), oracle.permute(idx_ref, cfg.E, cfg.S),
                               ("counts", "offsets", "sorted_slot", "slot_pos")):
        assert np.array_equal(host(got), want), what
    worst = assert_rows_close(ys[0], y_ref, "bf16", "mxfp4 layer")
    print(f"  worst row rel err {worst:.3e}", flush=True)
