"""ctypes front end of the fp64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
benchmark's CPU-baseline leg may import this package; the product path
(the HIP library and its binding) never does, and this package imports
nothing from it.

Arrays go in as numpy arrays: float32 for fp32 data, uint16 (raw bfloat16
bit patterns) for bf16 data.  Results come back as fp64 / int32 numpy arrays.

`Oracle(path)` binds one compiled oracle library; the module-level functions
use the default build (oracle/liboracle.so, compiled on first use).  The
mutation tests bind deliberately broken copies through the same class to
show that the pins catch them.
"""
import ctypes
import os

import numpy as np

from . import build as _build

F32 = 0
BF16 = 1

_i64 = ctypes.c_int64
_i32p = ctypes.POINTER(ctypes.c_int32)
_i64p = ctypes.POINTER(ctypes.c_int64)
_f64p = ctypes.POINTER(ctypes.c_double)
_f32p = ctypes.POINTER(ctypes.c_float)
_vp = ctypes.c_void_p
_int = ctypes.c_int

_SIGNATURES = {
    "oracle_route": [_i64, _i64, _i64, _i64, _int, _vp, _vp, _f32p, _f64p, _i32p,
                     _f64p],
    "oracle_permute": [_i64, _i64, _i64, _i64, _i32p, _i32p, _i32p, _i32p, _i32p],
    "oracle_permute_capacity": [_i64, _i64, _i64, _i64, _i64, _i32p, _i32p, _i32p,
                                _i32p, _i32p],
    "oracle_expert_capacity": [_i64, _i64, _i64, ctypes.c_double],
    "oracle_balance": [_i64, _i64, _i64, _int, _vp, _vp, _f32p, _f64p, _f64p, _f64p],
    "oracle_dequant_mxfp4": [_i64, _i64, _vp, _vp, _f64p],
    "oracle_layer_backward": [_i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp, _f32p, _vp,
                              _vp, _vp, _i64, _i64, _i64p, _f64p, _i64, _i32p, _f64p,
                              _f64p, _f64p, _f64p, _f64p],
    "oracle_gate_up_rows": [_i64, _i64p, _i32p, _i64, _i64, _int, _vp, _vp, _f64p],
    "oracle_down_rows": [_i64, _i32p, _i64, _i64, _int, _vp, _vp, _f64p],
    "oracle_combine": [_i64, _i64, _i64, _i64, _int, _vp, _i32p, _f64p, _f64p],
    "oracle_layer_forward": [_i64, _i64, _i64, _i64, _i64, _i64, _int, _vp, _vp,
                             _f32p, _vp, _vp, _i64, _i64p, _i32p, _i64, _i32p,
                             _f64p, _f64p],
    "oracle_num_threads": [],
    "oracle_set_num_threads": [_int],
}


def _dt(a: np.ndarray) -> int:
    if a.dtype == np.float32:
        return F32
    if a.dtype == np.uint16:
        return BF16
    raise TypeError(f"oracle takes float32 or uint16 (bf16 bits), got {a.dtype}")


def _c(a, dtype=None):
    return np.ascontiguousarray(a if dtype is None else np.asarray(a, dtype=dtype))


def _p(a, typ=None):
    if a is None:
        return None
    return a.ctypes.data_as(_vp if typ is None else typ)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (rc={rc})")


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        L = ctypes.CDLL(path)
        for name, argtypes in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int64 if name == "oracle_expert_capacity" else ctypes.c_int
        self.path = path
        self.L = L

    def num_threads(self) -> int:
        return self.L.oracle_num_threads()

    def set_num_threads(self, n: int) -> None:
        self.L.oracle_set_num_threads(int(n))

    def route(self, x, W_router, k, bias=None):
        """Return (logits[T,E] f64, idx[T,k] i32, w[T,k] f64)."""
        x = _c(x)
        W_router = _c(W_router)
        dt = _dt(x)
        assert _dt(W_router) == dt
        T, d = x.shape
        E = W_router.shape[0]
        b = None if bias is None else _c(bias, np.float32)
        logits = np.empty((T, E), np.float64)
        idx = np.empty((T, k), np.int32)
        w = np.empty((T, k), np.float64)
        rc = self.L.oracle_route(T, d, E, k, dt, _p(x), _p(W_router), _p(b, _f32p),
                                 _p(logits, _f64p), _p(idx, _i32p), _p(w, _f64p))
        _check(rc, "oracle_route")
        return logits, idx, w

    def permute(self, idx, E, S=0, capacity=None):
        """Return (counts[E+S], offsets[E+S+1], sorted_slot[T*k], slot_pos[T*k]).
        capacity: None (no limit) or the most copies one expert keeps."""
        idx = _c(idx, np.int32)
        T, k = idx.shape
        counts = np.empty(E + S, np.int32)
        offsets = np.empty(E + S + 1, np.int32)
        sorted_slot = np.empty(T * k, np.int32)
        slot_pos = np.empty(T * k, np.int32)
        args = (_p(idx, _i32p), _p(counts, _i32p), _p(offsets, _i32p),
                _p(sorted_slot, _i32p), _p(slot_pos, _i32p))
        if capacity is None:
            rc = self.L.oracle_permute(T, k, E, S, *args)
        else:
            assert capacity >= 0
            rc = self.L.oracle_permute_capacity(T, k, E, S, int(capacity), *args)
        _check(rc, "oracle_permute")
        return counts, offsets, sorted_slot, slot_pos

    def layer_backward(self, x, W_router, W_gate_up, W_down, dy, k, S=0, bias=None,
                       tokens=None, experts=(), router=True, capacity=None):
        """Gradients of sum(y * dy).  Returns a dict: dx [n_tok, d] for the
        listed tokens (all when tokens is None), dW_gate_up [n, 2f, d] and
        dW_down [n, d, f] for the listed experts, and with router=True dW_router
        [E, d], db [E], dw [T, k]; all fp64.  capacity: the forward with that
        expert capacity (layer_forward's); dropped copies get no gradient
        through their expert and dw 0."""
        x, W_router, W_gate_up, W_down, dy = (_c(a) for a in (x, W_router, W_gate_up,
                                                               W_down, dy))
        dt = _dt(x)
        for a in (W_router, W_gate_up, W_down, dy):
            assert _dt(a) == dt
        T, d = x.shape
        E = W_router.shape[0]
        f = W_gate_up.shape[1] // 2
        assert W_gate_up.shape == (E + S, 2 * f, d) and W_down.shape == (E + S, d, f)
        assert dy.shape == (T, d)
        b = None if bias is None else _c(bias, np.float32)
        tl = None if tokens is None else _c(tokens, np.int64)
        n_tok = T if tl is None else tl.shape[0]
        el = _c(np.asarray(experts, np.int32).reshape(-1), np.int32)
        n_exp = el.shape[0]
        out = {"dx": np.empty((n_tok, d), np.float64),
               "dW_gate_up": np.empty((n_exp, 2 * f, d), np.float64),
               "dW_down": np.empty((n_exp, d, f), np.float64)}
        if router:
            out.update(dW_router=np.empty((E, d), np.float64), db=np.empty(E, np.float64),
                       dw=np.empty((T, k), np.float64))
        rc = self.L.oracle_layer_backward(
            T, d, f, E, k, S, dt, _p(x), _p(W_router), _p(b, _f32p), _p(W_gate_up),
            _p(W_down), _p(dy), -1 if capacity is None else int(capacity), n_tok,
            _p(tl, _i64p), _p(out["dx"], _f64p), n_exp,
            _p(el, _i32p) if n_exp else None,
            _p(out["dW_gate_up"], _f64p) if n_exp else None,
            _p(out["dW_down"], _f64p) if n_exp else None,
            _p(out.get("dW_router"), _f64p), _p(out.get("db"), _f64p),
            _p(out.get("dw"), _f64p))
        _check(rc, "oracle_layer_backward")
        return out

    def dequant_mxfp4(self, q, scales):
        """fp64 values [..., K] of MXFP4 weights: q [..., K/2] uint8 (two FP4
        elements per byte, even element in the low nibble), scales [..., K/32]
        uint8 (E8M0)."""
        q = _c(q, np.uint8)
        scales = _c(scales, np.uint8)
        K = q.shape[-1] * 2
        assert scales.shape[:-1] == q.shape[:-1] and scales.shape[-1] * 32 == K
        rows = int(np.prod(q.shape[:-1]))
        out = np.empty(q.shape[:-1] + (K,), np.float64)
        rc = self.L.oracle_dequant_mxfp4(rows, K, _p(q), _p(scales), _p(out, _f64p))
        _check(rc, "oracle_dequant_mxfp4")
        return out

    def expert_capacity(self, T, k, E, factor):
        """ceil(factor * T*k / E)."""
        c = self.L.oracle_expert_capacity(T, k, E, float(factor))
        _check(0 if c >= 0 else -1, "oracle_expert_capacity")
        return int(c)

    def balance(self, x, W_router, bias=None, want_probs=False):
        """Return (importance[E] f64, loss f64) or, with want_probs, also the
        dense softmax probs[T,E]."""
        x = _c(x)
        W_router = _c(W_router)
        dt = _dt(x)
        assert _dt(W_router) == dt
        T, d = x.shape
        E = W_router.shape[0]
        b = None if bias is None else _c(bias, np.float32)
        probs = np.empty((T, E), np.float64) if want_probs else None
        imp = np.empty(E, np.float64)
        loss = np.empty(1, np.float64)
        rc = self.L.oracle_balance(T, d, E, dt, _p(x), _p(W_router), _p(b, _f32p),
                                   _p(probs, _f64p), _p(imp, _f64p), _p(loss, _f64p))
        _check(rc, "oracle_balance")
        if want_probs:
            return imp, float(loss[0]), probs
        return imp, float(loss[0])

    def gate_up_rows(self, x, W_gate_up, tok, expert):
        """SwiGLU activations [n, f] (fp64) of (token, expert) pairs."""
        x = _c(x)
        W_gate_up = _c(W_gate_up)
        dt = _dt(x)
        assert _dt(W_gate_up) == dt
        d = x.shape[1]
        f = W_gate_up.shape[1] // 2
        tok = _c(tok, np.int64)
        expert = _c(expert, np.int32)
        n = tok.shape[0]
        act = np.empty((n, f), np.float64)
        rc = self.L.oracle_gate_up_rows(n, _p(tok, _i64p), _p(expert, _i32p), d, f,
                                        dt, _p(x), _p(W_gate_up), _p(act, _f64p))
        _check(rc, "oracle_gate_up_rows")
        return act

    def down_rows(self, act, W_down, expert):
        """Down projections [n, d] (fp64) of activation rows act[n, f]."""
        act = _c(act)
        W_down = _c(W_down)
        dt = _dt(act)
        assert _dt(W_down) == dt
        n, f = act.shape
        d = W_down.shape[1]
        expert = _c(expert, np.int32)
        out = np.empty((n, d), np.float64)
        rc = self.L.oracle_down_rows(n, _p(expert, _i32p), d, f, dt, _p(act),
                                     _p(W_down), _p(out, _f64p))
        _check(rc, "oracle_down_rows")
        return out

    def combine(self, O, slot_pos, w, T, k, S=0):
        """y[T, d] (fp64) from permuted expert outputs O[T*k + S*T, d]."""
        O = _c(O)
        dt = _dt(O)
        d = O.shape[1]
        slot_pos = _c(slot_pos, np.int32)
        w = _c(w, np.float64)
        y = np.empty((T, d), np.float64)
        rc = self.L.oracle_combine(T, k, S, d, dt, _p(O), _p(slot_pos, _i32p),
                                   _p(w, _f64p), _p(y, _f64p))
        _check(rc, "oracle_combine")
        return y

    def layer_forward(self, x, W_router, W_gate_up, W_down, k, S=0, bias=None,
                      tokens=None, forced_idx=None, capacity=None):
        """Whole layer.  Returns (y[n,d] f64, idx[n,k] i32, w[n,k] f64) for the
        listed tokens (all tokens when tokens is None).  capacity: None or the
        most copies one expert keeps."""
        x = _c(x)
        W_router = _c(W_router)
        W_gate_up = _c(W_gate_up)
        W_down = _c(W_down)
        dt = _dt(x)
        for a in (W_router, W_gate_up, W_down):
            assert _dt(a) == dt
        T, d = x.shape
        E = W_router.shape[0]
        f = W_gate_up.shape[1] // 2
        assert W_gate_up.shape == (E + S, 2 * f, d), W_gate_up.shape
        assert W_down.shape == (E + S, d, f), W_down.shape
        b = None if bias is None else _c(bias, np.float32)
        tl = None if tokens is None else _c(tokens, np.int64)
        n = T if tl is None else tl.shape[0]
        fi = None if forced_idx is None else _c(forced_idx, np.int32)
        if fi is not None:
            assert fi.shape == (n, k)
        y = np.empty((n, d), np.float64)
        idx = np.empty((n, k), np.int32)
        w = np.empty((n, k), np.float64)
        rc = self.L.oracle_layer_forward(T, d, f, E, k, S, dt, _p(x), _p(W_router),
                                         _p(b, _f32p), _p(W_gate_up), _p(W_down), n,
                                         _p(tl, _i64p), _p(fi, _i32p),
                                         -1 if capacity is None else int(capacity),
                                         _p(idx, _i32p), _p(w, _f64p), _p(y, _f64p))
        _check(rc, "oracle_layer_forward")
        return y, idx, w


_default = None


def default() -> Oracle:
    """The oracle built from oracle.c, compiling it first if it is missing."""
    global _default
    if _default is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        _default = Oracle(_build.LIB)
    return _default


def num_threads():
    return default().num_threads()


def set_num_threads(n):
    default().set_num_threads(n)


def route(*a, **kw):
    return default().route(*a, **kw)


def permute(*a, **kw):
    return default().permute(*a, **kw)


def gate_up_rows(*a, **kw):
    return default().gate_up_rows(*a, **kw)


def down_rows(*a, **kw):
    return default().down_rows(*a, **kw)


def combine(*a, **kw):
    return default().combine(*a, **kw)


def layer_forward(*a, **kw):
    return default().layer_forward(*a, **kw)


def expert_capacity(*a, **kw):
    return default().expert_capacity(*a, **kw)


def balance(*a, **kw):
    return default().balance(*a, **kw)


def dequant_mxfp4(*a, **kw):
    return default().dequant_mxfp4(*a, **kw)


def layer_backward(*a, **kw):
    return default().layer_backward(*a, **kw)
