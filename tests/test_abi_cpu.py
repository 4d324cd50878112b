"""C ABI of libmoe on a host without a GPU: the library loads, exports every
entry point include/moe.h declares, and rejects bad arguments before any HIP
call (none of these calls launches work)."""
import ctypes
import os
import re

import pytest

import mixture_experts_sparse_router_amd as moe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z0-9_]+)\s*\(", src)))


def exported_functions():
    out = os.popen(f"nm -D --defined-only {moe.LIB_PATH}").read()
    return sorted(set(re.findall(r" T (moe_[a-z0-9_]+)$", out, flags=re.M)))


def test_header_and_library_agree():
    decl = declared_functions()
    assert decl, "no declarations parsed"
    assert decl == exported_functions()
    assert sorted(moe.ENTRY_POINTS) == decl
    for name in decl:
        assert hasattr(moe.lib(), name)


def test_status_strings_and_version():
    assert moe.status_string(0) == "MOE_OK"
    assert moe.status_string(1) == "MOE_ERR_INVALID_ARG"
    assert moe.status_string(3) == "MOE_ERR_WORKSPACE"
    assert moe.status_string(99) == "MOE_ERR_UNKNOWN"
    assert moe.version().startswith("moe-gfx950")


def _ws_expected(s):
    es = 2 if s.dt == moe.MOE_DT_BF16 else 4
    Tk, R, G = s.T * s.k, s.R, s.G
    sizes = [Tk * 4, Tk * 4, G * 4, (G + 1) * 4, Tk * 4, Tk * 4, R * s.f * es, R * s.d * es]
    off, at = [], 0
    for v in sizes:
        off.append(at)
        at += (v + 255) // 256 * 256
    return off, at


@pytest.mark.parametrize("dims", [(16, 2880, 2880, 32, 4, 0, 1), (128, 256, 512, 8, 2, 0, 0),
                                  (4096, 7168, 2048, 256, 8, 1, 1), (0, 64, 64, 4, 1, 0, 1)])
def test_workspace_layout(dims):
    s = moe.shape(*dims)
    off, total = _ws_expected(s)
    assert moe.workspace_size(s) == total
    got = moe.workspace_offsets(s)
    assert [got[n] for n in moe.WS_NAMES] == off
    assert all(v % 256 == 0 for v in off)


BAD_SHAPES = [
    dict(T=-1), dict(d=0), dict(d=12), dict(f=20), dict(E=0), dict(k=0), dict(k=9),
    dict(n_shared=-1), dict(dt=7),
]


def _shape(**kw):
    base = dict(T=16, d=64, f=64, E=8, k=2, n_shared=0, dt=moe.MOE_DT_BF16)
    base.update(kw)
    return moe.shape(**base)


@pytest.mark.parametrize("kw", BAD_SHAPES, ids=lambda k: ",".join(f"{a}={b}" for a, b in k.items()))
def test_bad_shape_rejected(kw):
    s = _shape(**kw)
    L = moe.lib()
    p = ctypes.c_void_p(4096)  # never dereferenced: the shape check comes first
    assert moe.workspace_size(s) == 0
    assert L.moe_route(ctypes.byref(s), p, p, None, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(s), p, p, p, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_combine(ctypes.byref(s), p, p, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(ctypes.byref(s), p, p, None, p, p, p, p, 1 << 40,
                               None) == moe.MOE_ERR_INVALID_ARG


def test_unsupported_shapes():
    L = moe.lib()
    p = ctypes.c_void_p(4096)
    for s in (_shape(E=1024, n_shared=1), _shape(E=128, k=65),
              _shape(T=1 << 30, k=4),
              # bf16 past decode size: x or one expert's weights of 2 GiB or more
              _shape(T=1 << 17, d=1 << 13, k=2, dt=moe.MOE_DT_BF16),
              _shape(T=128, d=1 << 15, f=1 << 14, dt=moe.MOE_DT_BF16)):
        assert L.moe_route(ctypes.byref(s), p, p, None, p, p, None) == moe.MOE_ERR_UNSUPPORTED
    # just inside those limits, and any size at decode batch or in fp32
    for s in (_shape(T=(1 << 17) - 8, d=1 << 13, k=2, dt=moe.MOE_DT_BF16),
              _shape(T=64, d=1 << 15, f=1 << 14, dt=moe.MOE_DT_BF16),
              _shape(T=128, d=1 << 15, f=1 << 14, dt=moe.MOE_DT_F32)):
        assert L.moe_workspace_size(ctypes.byref(s)) > 0


def test_null_and_misaligned_pointers():
    L = moe.lib()
    s = _shape()
    good = ctypes.c_void_p(4096)
    odd = ctypes.c_void_p(4096 + 2)
    assert L.moe_route(None, good, good, None, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(s), None, good, None, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(s), odd, good, None, good, good, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route(ctypes.byref(s), good, good, ctypes.c_void_p(4097), good, good,
                       None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_gemm_gate_up(ctypes.byref(s), good, good, good, None, good,
                                      None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_gemm_down(ctypes.byref(s), good, good, good, odd,
                                   None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_gemm(ctypes.byref(s), good, good, good, good, good, good, None,
                              None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute(ctypes.byref(s), good, good, None, good, good,
                         None) == moe.MOE_ERR_INVALID_ARG
    out = (ctypes.c_size_t * 8)()
    assert L.moe_workspace_offsets(ctypes.byref(s), None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_workspace_offsets(ctypes.byref(_shape(k=0)), out) == moe.MOE_ERR_INVALID_ARG


def test_workspace_checks():
    L = moe.lib()
    s = _shape()
    good = ctypes.c_void_p(4096)
    need = moe.workspace_size(s)
    assert need > 0
    assert L.moe_layer_forward(ctypes.byref(s), good, good, None, good, good, good, good,
                               need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward(ctypes.byref(s), good, good, None, good, good, good,
                               ctypes.c_void_p(4096 + 16), need, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward(ctypes.byref(s), good, good, None, good, good, good, None,
                               need, None) == moe.MOE_ERR_INVALID_ARG


def test_empty_layer_enqueues_nothing():
    """T = 0: every buffer is empty, the call succeeds without touching HIP."""
    L = moe.lib()
    s = _shape(T=0)
    good = ctypes.c_void_p(4096)
    assert L.moe_layer_forward(ctypes.byref(s), None, good, None, good, good, None, good,
                               moe.workspace_size(s), None) == moe.MOE_OK


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    s = _shape()
    x = torch.zeros(16, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        moe.moe_route(s, x, x, None, x, x)


def test_static_entry_checks_before_any_hip_call():
    """moe_layer_forward_static rejects bad arguments and shapes whose
    intermediates exceed its static array before touching HIP."""
    L = moe.lib()
    src = open(HEADER).read()
    assert f"#define MOE_STATIC_SCRATCH_BYTES (32u << 20)" in src
    assert moe.STATIC_SCRATCH_BYTES == 32 << 20
    p = ctypes.c_void_p(4096)
    big = moe.shape(4096, 2048, 768, 128, 8, 0, moe.MOE_DT_BF16)  # ~184 MB of intermediates
    assert moe.workspace_size(big) > moe.STATIC_SCRATCH_BYTES
    assert L.moe_layer_forward_static(ctypes.byref(big), p, p, None, p, p, p,
                                      None) == moe.MOE_ERR_WORKSPACE
    s = _shape()
    assert moe.workspace_size(s) <= moe.STATIC_SCRATCH_BYTES
    assert L.moe_layer_forward_static(None, p, p, None, p, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_static(ctypes.byref(_shape(k=0)), p, p, None, p, p, p,
                                      None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_static(ctypes.byref(s), None, p, None, p, p, p,
                                      None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_static(ctypes.byref(s), p, p, ctypes.c_void_p(4097), p, p, p,
                                      None) == moe.MOE_ERR_INVALID_ARG
    # an empty batch needs no intermediates and enqueues nothing
    assert L.moe_layer_forward_static(ctypes.byref(_shape(T=0)), None, p, None, p, p, None,
                                      None) == moe.MOE_OK


def test_expert_capacity_matches_oracle():
    import oracle
    for (T, k, E, f) in ((4096, 8, 128, 1.25), (4096, 8, 256, 1.0), (10, 2, 3, 1.0),
                         (7, 1, 4, 0.0), (8192, 2, 8, 2.0), (0, 3, 5, 1.5), (1, 1, 1, 1e-9)):
        assert moe.expert_capacity(T, k, E, f) == oracle.expert_capacity(T, k, E, f)
    for bad in ((-1, 1, 1, 1.0), (1, 0, 1, 1.0), (1, 1, 0, 1.0), (1, 1, 1, -0.5),
                (1, 1, 1, float("nan")), (1, 1, 1, 1e10)):
        assert moe.expert_capacity(*bad) == -1


def test_route_balance_workspace_and_checks():
    L = moe.lib()
    for dims in ((4096, 7168, 2048, 256, 8, 1, 1), (100, 64, 64, 7, 2, 0, 0), (0, 64, 64, 4, 1, 0, 1)):
        s = moe.shape(*dims)
        nb = (s.T + 15) // 16
        expect = (s.T * s.E * 4 + 255) // 256 * 256 + (nb * s.E * 8 + 255) // 256 * 256
        assert moe.route_balance_workspace_size(s) == expect
    assert moe.route_balance_workspace_size(_shape(k=0)) == 0
    s = _shape()
    p = ctypes.c_void_p(4096)
    need = moe.route_balance_workspace_size(s)
    args = lambda imp, ws, nbytes: (ctypes.byref(s), p, p, None, p, p, imp, p, ws, nbytes, None)
    assert L.moe_route_balance(*args(p, p, need - 1)) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route_balance(*args(None, p, need)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_balance(*args(p, ctypes.c_void_p(4096 + 64), need)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_balance(*args(p, None, need)) == moe.MOE_ERR_INVALID_ARG
    bad = _shape(E=0)
    assert L.moe_route_balance(ctypes.byref(bad), p, p, None, p, p, p, p, p, 1 << 30,
                               None) == moe.MOE_ERR_INVALID_ARG


def test_route_workspace_and_checks():
    L = moe.lib()
    bf16, f32 = moe.MOE_DT_BF16, moe.MOE_DT_F32
    # large bf16 batches with few experts or a large router matrix: at least
    # one split's fp64 partials, [T, E]
    for dims in ((8192, 4096, 14336, 8, 2, 0, bf16), (4096, 7168, 2048, 256, 8, 1, bf16),
                 (100, 64, 64, 7, 2, 0, bf16)):
        s = moe.shape(*dims)
        assert moe.route_workspace_size(s) >= s.T * s.E * 8
    # decode batches, fp32, and E = 128 with a 0.5 MB router: no workspace
    for dims in ((16, 2880, 2880, 32, 4, 0, bf16), (4096, 2048, 768, 128, 8, 0, bf16),
                 (4096, 4096, 64, 8, 2, 0, f32), (0, 64, 64, 4, 1, 0, bf16)):
        assert moe.route_workspace_size(moe.shape(*dims)) == 0
    assert moe.route_workspace_size(_shape(k=0)) == 0
    s = moe.shape(8192, 4096, 14336, 8, 2, 0, bf16)
    p = ctypes.c_void_p(4096)
    need = moe.route_workspace_size(s)
    args = lambda ws, nbytes: (ctypes.byref(s), p, p, None, p, p, ws, nbytes, None)
    assert L.moe_route_ws(*args(p, need - 1)) == moe.MOE_ERR_WORKSPACE
    assert L.moe_route_ws(*args(None, need)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_ws(*args(ctypes.c_void_p(4096 + 64), need)) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_route_ws(ctypes.byref(s), None, p, None, p, p, p, need,
                          None) == moe.MOE_ERR_INVALID_ARG
    bad = _shape(E=0)
    assert L.moe_route_ws(ctypes.byref(bad), p, p, None, p, p, p, 1 << 30,
                          None) == moe.MOE_ERR_INVALID_ARG


def test_capacity_entry_points_check_arguments():
    L = moe.lib()
    s = _shape()
    p = ctypes.c_void_p(4096)
    assert L.moe_permute_capacity(ctypes.byref(s), p, -1, p, p, p, p, None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute_capacity(ctypes.byref(_shape(k=0)), p, 4, p, p, p, p,
                                  None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_permute_capacity(ctypes.byref(s), p, 4, p, None, p, p,
                                  None) == moe.MOE_ERR_INVALID_ARG
    need = moe.workspace_size(s)
    assert L.moe_layer_forward_capacity(ctypes.byref(s), p, p, None, p, p, -1, p, p, need,
                                        None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_capacity(ctypes.byref(s), p, p, None, p, p, 3, p, p, need - 1,
                                        None) == moe.MOE_ERR_WORKSPACE
    # an empty batch needs no work at all
    assert L.moe_layer_forward_capacity(ctypes.byref(_shape(T=0)), None, p, None, p, p, 0, None,
                                        p, moe.workspace_size(_shape(T=0)), None) == moe.MOE_OK


def test_mxfp4_entry_points_check_shapes_and_pointers():
    L = moe.lib()
    p = ctypes.c_void_p(4096)
    good = moe.shape(16, 64, 96, 8, 2, 0, moe.MOE_DT_BF16)
    need = moe.workspace_size(good)
    for bad in (moe.shape(16, 64, 96, 8, 2, 0, moe.MOE_DT_F32),   # fp32 activations
                moe.shape(65, 64, 96, 8, 2, 0, moe.MOE_DT_BF16),  # past decode size
                moe.shape(16, 48, 96, 8, 2, 0, moe.MOE_DT_BF16),  # d not a multiple of 32
                moe.shape(16, 64, 104, 8, 2, 0, moe.MOE_DT_BF16)):  # f not a multiple of 32
        assert L.moe_grouped_gemm_gate_up_mxfp4(ctypes.byref(bad), p, p, p, p, p, p,
                                                None) == moe.MOE_ERR_UNSUPPORTED
        assert L.moe_grouped_gemm_down_mxfp4(ctypes.byref(bad), p, p, p, p, p,
                                             None) == moe.MOE_ERR_UNSUPPORTED
        assert L.moe_layer_forward_mxfp4(ctypes.byref(bad), p, p, None, p, p, p, p, p, p,
                                         1 << 40, None) == moe.MOE_ERR_UNSUPPORTED
    odd = ctypes.c_void_p(4096 + 8)
    assert L.moe_grouped_gemm_gate_up_mxfp4(ctypes.byref(good), p, p, p, odd, p, p,
                                            None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_grouped_gemm_down_mxfp4(ctypes.byref(good), p, p, p, None, p,
                                         None) == moe.MOE_ERR_INVALID_ARG
    assert L.moe_layer_forward_mxfp4(ctypes.byref(good), p, p, None, p, p, p, p, p, p,
                                     need - 1, None) == moe.MOE_ERR_WORKSPACE
    assert L.moe_layer_forward_mxfp4(ctypes.byref(_shape(k=0)), p, p, None, p, p, p, p, p, p,
                                     need, None) == moe.MOE_ERR_INVALID_ARG


def test_backward_checks_before_any_hip_call():
    L = moe.lib()
    p = ctypes.c_void_p(4096)
    s = _shape()
    fneed, bneed = moe.workspace_size(s), moe.backward_workspace_size(s)
    assert bneed > 0
    assert moe.backward_workspace_size(_shape(dt=moe.MOE_DT_F32)) == 0

    def call(shape, fbytes=fneed, bbytes=bneed, dx=p, fw=p, ws=p, dw=None):
        return L.moe_layer_backward(ctypes.byref(shape), p, p, p, p, p, fw, fbytes, dx, p, p, p,
                                    p, dw, ws, bbytes, None)
    assert call(_shape(dt=moe.MOE_DT_F32)) == moe.MOE_ERR_UNSUPPORTED
    assert call(_shape(k=0)) == moe.MOE_ERR_INVALID_ARG
    assert call(s, fbytes=fneed - 1) == moe.MOE_ERR_WORKSPACE
    assert call(s, bbytes=bneed - 1) == moe.MOE_ERR_WORKSPACE
    assert call(s, dx=None) == moe.MOE_ERR_INVALID_ARG
    assert call(s, fw=ctypes.c_void_p(4096 + 16)) == moe.MOE_ERR_INVALID_ARG
    assert call(s, ws=None) == moe.MOE_ERR_INVALID_ARG
    assert call(s, dw=ctypes.c_void_p(4096 + 4)) == moe.MOE_ERR_INVALID_ARG
