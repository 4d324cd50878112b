"""Seeded synthetic inputs for the MoE layer: the only module that both the
HIP path's tests/benchmark and the fp64 oracle take data from.

It holds no arithmetic of the method (no routing, no expert function, no
combine): only shapes, random draws and the bfloat16 encoding of the draws.

Recipe (the same for every workload):
  - numpy PCG64; every tensor piece has its own stream
    default_rng([seed, tensor_id, part]) so pieces can be drawn in parallel and
    any piece can be regenerated alone;
      tensor_id 0: x, part = block of 256 token rows
      tensor_id 1: W_router, part 0
      tensor_id 2: W_gate_up, part = expert index (routed 0..E-1, shared E..)
      tensor_id 3: W_down,    part = expert index
      tensor_id 5..: free-standing test tensors
  - x ~ N(0, 1); router and expert weights ~ N(0, 0.02) (0.02 a standard
    deviation); draws in float32, then rounded to nearest-even bfloat16 for
    bf16 workloads (stored as raw uint16 bit patterns);
  - optional Zipf(s) router prior: bias_e = -s * ln(e + 1) in float32, i.e.
    the prior routing probability of expert e is proportional to (e+1)^-s;
  - MXFP4 expert weights (the quantised decode variant): tensor_id 6
    (gate_up) and 7 (down), part = expert index; uniformly random bytes of
    packed FP4 codes and E8M0 block scales drawn uniformly from
    MXFP4_SCALE_RANGE, which puts the values at the size of N(0, 0.02)
    weights (|value| mostly 2^-8 .. 2^-4).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

X_ROWS_PER_STREAM = 256


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int          # tokens
    d: int          # model dim
    f: int          # expert FFN dim
    E: int          # routed experts
    k: int          # experts per token
    S: int          # shared (always-on) experts
    dtype: str      # "f32" or "bf16"
    zipf_s: float | None = None   # Zipf router prior exponent, or None
    x_std: float = 1.0
    w_std: float = 0.02

    @property
    def R(self) -> int:
        """Rows of the permuted expert buffers: routed copies + shared rows."""
        return self.T * self.k + self.S * self.T

    def scaled(self, **kw) -> "LayerConfig":
        d = dict(self.__dict__)
        d.update(kw)
        return LayerConfig(**d)


# The five workloads.  Shapes follow the named models; weights are random.
CONFIGS = {
    1: LayerConfig("tiny_fp32", T=128, d=256, f=512, E=8, k=2, S=0, dtype="f32"),
    2: LayerConfig("gpt_oss_20b_decode", T=16, d=2880, f=2880, E=32, k=4, S=0,
                   dtype="bf16"),
    3: LayerConfig("mixtral_8x7b_prefill", T=8192, d=4096, f=14336, E=8, k=2, S=0,
                   dtype="bf16"),
    4: LayerConfig("fine_grained_zipf", T=4096, d=2048, f=768, E=128, k=8, S=0,
                   dtype="bf16", zipf_s=1.2),
    5: LayerConfig("deepseek_v3", T=4096, d=7168, f=2048, E=256, k=8, S=1,
                   dtype="bf16"),
}


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return uint16 patterns.
    (Inputs are finite draws; NaN/Inf never occur.)"""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (b >> np.uint32(16)) & np.uint32(1)
    return ((b + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 patterns to float32 (bit shift)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return a if dtype == "f32" else to_bf16_bits(a)


def normal(key, shape, std: float, dtype: str) -> np.ndarray:
    """One seeded N(0, std) tensor; key = [seed, tensor_id, part]."""
    rng = np.random.default_rng(list(key))
    a = rng.standard_normal(int(np.prod(shape)), dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return _encode(a, dtype).reshape(shape)


def _workers(threads):
    if threads:
        return threads
    return max(1, min(16, os.cpu_count() or 1))


def zipf_bias(E: int, s: float) -> np.ndarray:
    return (-s * np.log(np.arange(1, E + 1, dtype=np.float64))).astype(np.float32)


def make_x(cfg: LayerConfig, seed: int, threads=None) -> np.ndarray:
    npdt = np.float32 if cfg.dtype == "f32" else np.uint16
    x = np.empty((cfg.T, cfg.d), npdt)
    nblk = (cfg.T + X_ROWS_PER_STREAM - 1) // X_ROWS_PER_STREAM

    def blk(b):
        r0 = b * X_ROWS_PER_STREAM
        r1 = min(cfg.T, r0 + X_ROWS_PER_STREAM)
        x[r0:r1] = normal((seed, 0, b), (r1 - r0, cfg.d), cfg.x_std, cfg.dtype)

    with ThreadPoolExecutor(_workers(threads)) as ex:
        list(ex.map(blk, range(nblk)))
    return x


def make_layer_inputs(cfg: LayerConfig, seed: int, threads=None,
                      experts: bool = True) -> dict:
    """All inputs of one layer as host numpy arrays:
    x[T,d], W_router[E,d], bias[E] (float32) or None,
    W_gate_up[E+S, 2f, d], W_down[E+S, d, f]."""
    npdt = np.float32 if cfg.dtype == "f32" else np.uint16
    out = {
        "x": make_x(cfg, seed, threads),
        "W_router": normal((seed, 1, 0), (cfg.E, cfg.d), cfg.w_std, cfg.dtype),
        "bias": zipf_bias(cfg.E, cfg.zipf_s) if cfg.zipf_s else None,
    }
    if experts:
        n = cfg.E + cfg.S
        wgu = np.empty((n, 2 * cfg.f, cfg.d), npdt)
        wd = np.empty((n, cfg.d, cfg.f), npdt)

        def one(e):
            wgu[e] = normal((seed, 2, e), (2 * cfg.f, cfg.d), cfg.w_std, cfg.dtype)
            wd[e] = normal((seed, 3, e), (cfg.d, cfg.f), cfg.w_std, cfg.dtype)

        with ThreadPoolExecutor(_workers(threads)) as ex:
            list(ex.map(one, range(n)))
        out["W_gate_up"] = wgu
        out["W_down"] = wd
    return out


MXFP4_SCALE_RANGE = (119, 121)   # E8M0 exponents 2^-8 .. 2^-6


def mxfp4(key, rows: int, K: int, scale_range=MXFP4_SCALE_RANGE):
    """Seeded MXFP4 matrix [rows, K]: (packed codes uint8 [rows, K/2],
    E8M0 scales uint8 [rows, K/32]).  Raw bytes only: the decoding is the
    oracle's and the kernels' business."""
    assert K % 32 == 0
    rng = np.random.default_rng(list(key))
    q = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sc = rng.integers(scale_range[0], scale_range[1] + 1, size=(rows, K // 32), dtype=np.uint8)
    return q, sc


def make_mxfp4_experts(cfg: LayerConfig, seed: int, threads=None) -> dict:
    """MXFP4 expert weights of a layer: Wq_gate_up [E+S, 2f, d/2],
    Ws_gate_up [E+S, 2f, d/32], Wq_down [E+S, d, f/2], Ws_down [E+S, d, f/32]."""
    n = cfg.E + cfg.S
    out = {"Wq_gate_up": np.empty((n, 2 * cfg.f, cfg.d // 2), np.uint8),
           "Ws_gate_up": np.empty((n, 2 * cfg.f, cfg.d // 32), np.uint8),
           "Wq_down": np.empty((n, cfg.d, cfg.f // 2), np.uint8),
           "Ws_down": np.empty((n, cfg.d, cfg.f // 32), np.uint8)}

    def one(e):
        out["Wq_gate_up"][e], out["Ws_gate_up"][e] = mxfp4((seed, 6, e), 2 * cfg.f, cfg.d)
        out["Wq_down"][e], out["Ws_down"][e] = mxfp4((seed, 7, e), cfg.d, cfg.f)

    with ThreadPoolExecutor(_workers(threads)) as ex:
        list(ex.map(one, range(n)))
    return out


def tiny_config(T=8, d=16, f=8, E=6, k=2, S=0, dtype="f32", zipf_s=None) -> LayerConfig:
    return LayerConfig(f"tiny_T{T}_d{d}_f{f}_E{E}_k{k}_S{S}_{dtype}", T=T, d=d, f=f,
                       E=E, k=k, S=S, dtype=dtype, zipf_s=zipf_s)


def small_ints(key, shape, lo: int, hi: int) -> np.ndarray:
    """Seeded integers in [lo, hi] as float32 (exact in every format used)."""
    rng = np.random.default_rng(list(key))
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def random_routing(key, T: int, E: int, k: int, zipf_s: float | None = None) -> np.ndarray:
    """Seeded expert ids [T, k] (int32), distinct within a row; with zipf_s
    the ids are drawn without replacement with probability ~ (e+1)^-zipf_s,
    which leaves some experts with many copies and some with none."""
    rng = np.random.default_rng(list(key))
    idx = np.empty((T, k), np.int32)
    if zipf_s is None:
        for t in range(T):
            idx[t] = rng.permutation(E)[:k]
    else:
        p = np.arange(1, E + 1, dtype=np.float64) ** -zipf_s
        p /= p.sum()
        for t in range(T):
            idx[t] = rng.choice(E, size=k, replace=False, p=p)
    return idx


def random_unit(key, shape) -> np.ndarray:
    """Seeded float32 values in (0, 1]."""
    rng = np.random.default_rng(list(key))
    return (1.0 - rng.random(size=shape)).astype(np.float32)
