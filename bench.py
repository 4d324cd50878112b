"""Benchmark of one MoE FFN layer forward (router -> top-k -> permutation ->
grouped SwiGLU GEMMs -> combine) through libmoe's C ABI on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N] [--no-cpu]
                    [--no-prefill]

A step is one moe_layer_forward over one batch of seeded synthetic inputs
already resident in HBM.  Before the W warmup steps, untimed steps run for
--spinup-ms (default 200 ms) so that the GPU clocks have ramped up from idle
(short runs otherwise time part of the ramp).  Default workload: the gpt-oss-20b-shaped decode
layer (T=16, d=2880, f=2880, E=32, top-4, bf16).  Prints ONE JSON line:
tokens/s of the whole layer (wall clock around exactly K steps, with the
same interval also measured by HIP events on the stream the kernels run
on), the roofline of the dominant kernel (the gate_up grouped GEMM), the
fp64 CPU oracle's rate on the host cores, and, under "prefill", the same
layer measurement for the Mixtral-8x7B-shaped prefill workload against the
bf16 MFMA peak; for decode workloads, under "mxfp4", the same layer with
MXFP4 expert weights.  Each workload also reports, under layer.aux, the router
auxiliaries: routing with the balance statistics against routing alone, and
the layer with an expert capacity of 1.25 times the even share; and, under
layer.backward, the backward pass (all gradients) after one forward.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
FP32_PEAK_TFLOPS = 157.3
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
# the decode GEMM kernel's sources: stored counters hold while these are unchanged
GEMM_SRCS = tuple(os.path.join(ROOT, "mixture_experts_sparse_router_amd", "csrc", f)
                  for f in ("gemm_stream.hip", "decode_rows.h", "moe_common.h"))
PREFILL_CONFIG = 3             # Mixtral-8x7B-shaped prefill


def parse(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--config", type=int, default=2,
                   help="workload 1..5 (2 = gpt-oss-20b-shaped decode, the headline)")
    p.add_argument("--seed", type=int, default=None)
    p.add_argument("--spinup-ms", type=float, default=200.0,
                   help="untimed layer steps for this long before the warmup steps, so that "
                        "the GPU clocks have left their idle state (reported as spinup_ms)")
    p.add_argument("--no-cpu", action="store_true", help="skip the oracle CPU baseline")
    p.add_argument("--cpu-seconds", type=float, default=10.0)
    p.add_argument("--no-prefill", action="store_true",
                   help="skip the Mixtral-shaped prefill measurement")
    p.add_argument("--prefill-steps", type=int, default=20)
    p.add_argument("--no-aux", action="store_true",
                   help="skip the router-auxiliary timings (balance loss, capacity)")
    p.add_argument("--no-mxfp4", action="store_true",
                   help="skip the MXFP4-weight decode measurement")
    p.add_argument("--rotate", type=int, default=1,
                   help="use N device copies of the expert weights in turn, so that no step "
                        "finds the previous step's weights in a cache (default 1)")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="only run a plain 1 GiB device copy (torch copy_) 10 times: the "
                        "reference kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE")
    return p.parse_args(argv)


def alg_counts(cfg, counts):
    """Algorithmic bytes / flops of the layer and of each GEMM, from the
    actual routing: active experts' weights read once, router weights, x in,
    y out; GEMM flops over the routed + shared rows."""
    b = 4 if cfg.dtype == "f32" else 2
    G = cfg.E + cfg.S
    active = int(sum(1 for g in range(G) if counts[g] > 0))
    R = cfg.T * cfg.k + cfg.S * cfg.T
    w_gu = active * 2 * cfg.f * cfg.d * b
    w_d = active * cfg.d * cfg.f * b
    layer_bytes = w_gu + w_d + cfg.E * cfg.d * b + 2 * cfg.T * cfg.d * b
    gate_up_bytes = w_gu + cfg.T * cfg.d * b + R * cfg.f * b
    down_bytes = w_d + R * cfg.f * b + R * cfg.d * b
    layer_flops = 2 * cfg.T * cfg.d * cfg.E + 6 * cfg.d * cfg.f * R
    return dict(active=active, R=R, layer_bytes=layer_bytes, gate_up_bytes=gate_up_bytes,
                down_bytes=down_bytes, layer_flops=layer_flops,
                gate_up_flops=4 * cfg.d * cfg.f * R, down_flops=2 * cfg.d * cfg.f * R)


def binding_roof(flops, nbytes, fp32=False):
    """The roof that bounds a kernel of these algorithmic flops and bytes: the
    one whose time at peak is longer (flop/byte below the ridge -> HBM)."""
    peak_tf = FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS
    t_mfma = flops / (peak_tf * 1e12)
    t_hbm = nbytes / (HBM_PEAK_GBS * 1e9)
    return ("mfma", peak_tf) if t_mfma > t_hbm else ("hbm", HBM_PEAK_GBS)


def time_calls(torch, fn, n):
    """Average GPU time of fn() over n back-to-back calls, HIP events recorded
    on the current stream (the stream every call enqueues on)."""
    st = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for _ in range(3):  # warm: first calls pay for code and cache misses
        fn()
    e0.record(st)
    for _ in range(n):
        fn()
    e1.record(st)
    e1.synchronize()
    return e0.elapsed_time(e1) / n * 1e-3  # seconds


def gemm_src_hash():
    """sha256 (first 16 hex digits) of the decode GEMM kernel's sources."""
    h = hashlib.sha256()
    for path in GEMM_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(key):
    """HBM traffic of the dominant kernel from committed rocprofv3 --pmc
    counters, valid only while the kernel source is unchanged."""
    try:
        data = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    ent = data.get(key)
    if not ent:
        return None
    if ent.get("gemm_src_sha256_16") != gemm_src_hash():
        return None
    return ent.get("bytes_per_launch")


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, inp, seconds):
    """The fp64 oracle, as it stands, on a bounded sample of the workload's
    tokens (calls of at most 16 tokens, cycling through the batch, until
    `seconds` of wall time have passed)."""
    import numpy as np
    import oracle
    T = cfg.T
    toks = np.arange(T)
    per_call = min(T, 16)
    n_done = 0
    t0 = time.perf_counter()
    calls = 0
    while True:
        sel = toks[(calls * per_call) % T:][:per_call]
        oracle.layer_forward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"],
                             cfg.k, S=cfg.S, bias=inp["bias"], tokens=sel)
        n_done += len(sel)
        calls += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    out = dict(value=n_done / el, unit="tokens/s", cores=oracle.num_threads(),
               kind="oracle", cpu_model=cpu_model(),
               sample=f"{n_done} tokens of the same workload in {calls} oracle calls of "
                      f"<= {per_call} tokens, {el:.1f} s wall")
    if T <= 128:
        # small workloads: the same sample on one core as well
        threads = oracle.num_threads()
        oracle.set_num_threads(1)
        try:
            n1, c1, t1 = 0, 0, time.perf_counter()
            while True:
                sel = toks[(c1 * per_call) % T:][:per_call]
                oracle.layer_forward(inp["x"], inp["W_router"], inp["W_gate_up"], inp["W_down"],
                                     cfg.k, S=cfg.S, bias=inp["bias"], tokens=sel)
                n1 += len(sel)
                c1 += 1
                e1 = time.perf_counter() - t1
                if e1 >= seconds / 3:
                    break
        finally:
            oracle.set_num_threads(threads)
        out["single_core"] = dict(value=n1 / e1, unit="tokens/s", cores=1,
                                  sample=f"{n1} tokens in {c1} calls, {e1:.1f} s wall")
    return out


class Layer:
    """Device buffers and the step function of one workload."""

    def __init__(self, torch, moe, cfg, seed, rotate=1):
        import numpy as np
        import moe_synth
        self.cfg, self.seed = cfg, seed
        self.inp = moe_synth.make_layer_inputs(cfg, seed)

        def dev(a):
            if a is None:
                return None
            if a.dtype == np.uint16:
                return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
            return torch.from_numpy(a).cuda()

        self.d = {k: dev(v) for k, v in self.inp.items()}
        self.rot = max(1, rotate)
        self.w_gu = [self.d["W_gate_up"]] + [self.d["W_gate_up"].clone()
                                             for _ in range(self.rot - 1)]
        self.w_dn = [self.d["W_down"]] + [self.d["W_down"].clone()
                                          for _ in range(self.rot - 1)]
        self.dt = moe.MOE_DT_BF16 if cfg.dtype == "bf16" else moe.MOE_DT_F32
        self.s = moe.shape(cfg.T, cfg.d, cfg.f, cfg.E, cfg.k, cfg.S, self.dt)
        self.ws = torch.empty(moe.workspace_size(self.s), dtype=torch.uint8, device="cuda")
        self.y = torch.empty(cfg.T, cfg.d, dtype=torch.bfloat16 if self.dt else torch.float32,
                             device="cuda")
        self.views = moe.workspace_views(self.s, self.ws)
        # the layer's router keeps partial sums in its workspace; timed alone
        # through moe_route_ws with a workspace of its own
        nr = moe.route_workspace_size(self.s)
        self.rws = torch.empty(nr, dtype=torch.uint8, device="cuda") if nr else None
        self.moe = moe

    def step(self, i=0):
        d = self.d
        self.moe.moe_layer_forward(self.s, d["x"], d["W_router"], d["bias"],
                                   self.w_gu[i % self.rot], self.w_dn[i % self.rot], self.y,
                                   self.ws)

    def kernel_times(self, torch, n):
        """Average time of each step's entry point called alone, back to back,
        on the buffers of the last layer call."""
        moe, s, d, v = self.moe, self.s, self.d, self.views
        return {
            "route": time_calls(torch, lambda: moe.moe_route_ws(
                s, d["x"], d["W_router"], d["bias"], v["topk_idx"], v["topk_w"], self.rws), n),
            "permute": time_calls(torch, lambda: moe.moe_permute(
                s, v["topk_idx"], v["counts"], v["offsets"], v["sorted_slot"],
                v["slot_pos"]), n),
            "gate_up": time_calls(torch, lambda: moe.moe_grouped_gemm_gate_up(
                s, d["x"], v["sorted_slot"], v["offsets"], d["W_gate_up"], v["act"]), n),
            "down": time_calls(torch, lambda: moe.moe_grouped_gemm_down(
                s, v["act"], v["offsets"], d["W_down"], v["expert_out"]), n),
            "combine": time_calls(torch, lambda: moe.moe_combine(
                s, v["expert_out"], v["slot_pos"], v["topk_w"], self.y), n),
        }

    def aux_times(self, torch, n, factor=1.25):
        """The router auxiliaries on this workload: moe_route_balance (routing
        plus importance and balance loss) against moe_route (both the
        one-kernel router, without a workspace for partial sums), and the
        layer with an expert capacity of `factor` times the even share."""
        moe, s, d, v, cfg = self.moe, self.s, self.d, self.views, self.cfg
        ws_b = torch.empty(max(1, moe.route_balance_workspace_size(s)), dtype=torch.uint8,
                           device="cuda")
        imp = torch.empty(cfg.E, dtype=torch.float64, device="cuda")
        loss = torch.empty(1, dtype=torch.float64, device="cuda")
        cap = moe.expert_capacity(cfg.T, cfg.k, cfg.E, factor)
        ws_c = torch.empty_like(self.ws)
        y_c = torch.empty_like(self.y)
        t_route = time_calls(torch, lambda: moe.moe_route(
            s, d["x"], d["W_router"], d["bias"], v["topk_idx"], v["topk_w"]), n)
        t_bal = time_calls(torch, lambda: moe.moe_route_balance(
            s, d["x"], d["W_router"], d["bias"], v["topk_idx"], v["topk_w"], imp, loss, ws_b),
            n)
        t_cap = time_calls(torch, lambda: moe.moe_layer_forward_capacity(
            s, d["x"], d["W_router"], d["bias"], self.w_gu[0], self.w_dn[0], cap, y_c, ws_c),
            n)
        kept = int(moe.workspace_views(s, ws_c)["counts"][:cfg.E].sum().item())
        return {"route_us": round(t_route * 1e6, 2),
                "route_balance_us": round(t_bal * 1e6, 2),
                "balance_loss": float(loss.item()),
                "capacity_factor": factor, "capacity": cap,
                "copies_kept": kept, "copies": cfg.T * cfg.k,
                "layer_capacity_ms": round(t_cap * 1e3, 4)}

    def backward_time(self, torch, n):
        """moe_layer_backward after one forward call: average time over n
        calls (HIP events), and its MFMA fraction on the expert GEMMs'
        16 * R * d * f flops (H recomputed 4, dA 2, dX 4, dW_down 2,
        dW_gate_up 4)."""
        moe, s, d, cfg = self.moe, self.s, self.d, self.cfg
        if s.dt != moe.MOE_DT_BF16:
            return None
        self.step(0)
        G = cfg.E + cfg.S
        f32 = dict(dtype=torch.float32, device="cuda")
        g = {"dx": torch.empty(cfg.T, cfg.d, **f32), "dWr": torch.empty(cfg.E, cfg.d, **f32),
             "db": torch.empty(cfg.E, **f32),
             "dWgu": torch.empty(G, 2 * cfg.f, cfg.d, **f32),
             "dWd": torch.empty(G, cfg.d, cfg.f, **f32), "dw": torch.empty(cfg.T, cfg.k, **f32)}
        dy = torch.randn(cfg.T, cfg.d, device="cuda").to(torch.bfloat16)
        bws = torch.empty(moe.backward_workspace_size(s), dtype=torch.uint8, device="cuda")

        def bwd():
            moe.moe_layer_backward(s, d["x"], d["W_router"], self.w_gu[0], self.w_dn[0], dy,
                                   self.ws, g["dx"], g["dWr"], g["db"], g["dWgu"], g["dWd"],
                                   g["dw"], bws)
        bwd()
        torch.cuda.synchronize()
        t = time_calls(torch, bwd, n)
        R = cfg.T * cfg.k + cfg.S * cfg.T
        flops = 16 * R * cfg.d * cfg.f
        out = {"ms": round(t * 1e3, 4), "expert_gemm_flops": flops,
               "mfma_frac": round(flops / t / 1e12 / BF16_PEAK_TFLOPS, 4)}
        del g, bws
        torch.cuda.empty_cache()
        return out

    def timed_steps(self, torch, steps):
        """Exactly `steps` layer calls between two synchronisations: wall
        clock, and HIP events recorded on the stream the calls enqueue on."""
        st = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(st)
        for i in range(steps):
            self.step(i)
        e1.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        return wall, e0.elapsed_time(e1) * 1e-3

    def summary(self, torch, kt, layer_s):
        cfg = self.cfg
        counts = self.views["counts"].cpu().numpy()
        ac = alg_counts(cfg, counts)
        fp32 = self.dt == self.moe.MOE_DT_F32
        bound, peak = binding_roof(ac["gate_up_flops"], ac["gate_up_bytes"], fp32)
        if bound == "hbm":
            achieved, unit = ac["gate_up_bytes"] / kt["gate_up"] / 1e9, "GB/s"
        else:
            achieved, unit = ac["gate_up_flops"] / kt["gate_up"] / 1e12, "TFLOP/s"
        roof = dict(bound=bound, kernel="grouped_gemm_gate_up", achieved=round(achieved, 2),
                    peak=peak, unit=unit, frac=round(achieved / peak, 4),
                    traffic=load_traffic(cfg.name),
                    alg_bytes_per_launch=ac["gate_up_bytes"],
                    alg_flops_per_launch=ac["gate_up_flops"],
                    avg_launch_us=round(kt["gate_up"] * 1e6, 2))
        mfma_peak = FP32_PEAK_TFLOPS if fp32 else BF16_PEAK_TFLOPS
        layer = {"alg_bytes": ac["layer_bytes"], "alg_flops": ac["layer_flops"],
                 "hbm_frac": round(ac["layer_bytes"] / layer_s / 1e9 / HBM_PEAK_GBS, 4),
                 "mfma_frac": round(ac["layer_flops"] / layer_s / 1e12 / mfma_peak, 4),
                 "kernel_us": {k: round(v * 1e6, 2) for k, v in kt.items()},
                 "gemm_frac": {
                     "gate_up_hbm": round(ac["gate_up_bytes"] / kt["gate_up"] / 1e9
                                          / HBM_PEAK_GBS, 4),
                     "gate_up_mfma": round(ac["gate_up_flops"] / kt["gate_up"] / 1e12
                                           / mfma_peak, 4),
                     "down_hbm": round(ac["down_bytes"] / kt["down"] / 1e9 / HBM_PEAK_GBS, 4),
                     "down_mfma": round(ac["down_flops"] / kt["down"] / 1e12 / mfma_peak, 4)}}
        return ac, roof, layer


def mxfp4_extra(torch, moe, L, steps):
    """The same decode layer with MXFP4 expert weights (FP4 E2M1 codes, one
    E8M0 scale per 32 weights, 0.53125 bytes per weight): layer time over
    `steps` calls (HIP events), each GEMM alone, and the gate_up GEMM's
    fraction of HBM peak on its algorithmic bytes."""
    import moe_synth
    cfg, s, d, v = L.cfg, L.s, L.d, L.views
    mx = moe_synth.make_mxfp4_experts(cfg, L.seed)
    dm0 = {k: torch.from_numpy(a).cuda() for k, a in mx.items()}
    # the MXFP4 weights (0.38 GB at the gpt-oss-20b shape; 0.13 GB for the down
    # projection) would fit the GPU's 256 MB last-level cache when one copy is
    # read over and over: calls cycle through enough copies that each GEMM's
    # weights read between two uses of the same copy exceed 1 GiB
    wbytes = min(dm0["Wq_down"].numel() + dm0["Ws_down"].numel(),
                 dm0["Wq_gate_up"].numel() + dm0["Ws_gate_up"].numel())
    ncopy = max(1, -(-(1 << 30) // max(1, wbytes)))
    dms = [dm0] + [{k: t.clone() for k, t in dm0.items()} for _ in range(ncopy - 1)]
    ws = torch.empty_like(L.ws)
    y = torch.empty_like(L.y)
    views = moe.workspace_views(s, ws)
    it = [0]

    def nxt():
        it[0] += 1
        return dms[it[0] % ncopy]

    def step():
        dm = nxt()
        moe.moe_layer_forward_mxfp4(s, d["x"], d["W_router"], d["bias"], dm["Wq_gate_up"],
                                    dm["Ws_gate_up"], dm["Wq_down"], dm["Ws_down"], y, ws)

    def gate_up():
        dm = nxt()
        moe.moe_grouped_gemm_gate_up_mxfp4(s, d["x"], views["sorted_slot"], views["offsets"],
                                           dm["Wq_gate_up"], dm["Ws_gate_up"], views["act"])

    def down():
        dm = nxt()
        moe.moe_grouped_gemm_down_mxfp4(s, views["act"], views["offsets"], dm["Wq_down"],
                                        dm["Ws_down"], views["expert_out"])
    for _ in range(5):
        step()
    torch.cuda.synchronize()
    t_layer = time_calls(torch, step, max(steps, 100))
    n = 100
    t_gu = time_calls(torch, gate_up, n)
    t_dn = time_calls(torch, down, n)
    counts = views["counts"].cpu().numpy()
    G = cfg.E + cfg.S
    active = int(sum(1 for g in range(G) if counts[g] > 0))
    R = cfg.T * cfg.k + cfg.S * cfg.T
    per_w = 0.5 + 1.0 / 32.0
    gu_bytes = int(active * 2 * cfg.f * cfg.d * per_w) + cfg.T * cfg.d * 2 + R * cfg.f * 2
    dn_bytes = int(active * cfg.d * cfg.f * per_w) + R * cfg.f * 2 + R * cfg.d * 2
    layer_bytes = (int(active * 3 * cfg.f * cfg.d * per_w) + cfg.E * cfg.d * 2
                   + 2 * cfg.T * cfg.d * 2)
    return {"weights": "MXFP4 (FP4 E2M1, E8M0 scale per 32)", "active_experts": active,
            "weight_copies": ncopy,
            "ms_per_step_hip_events": round(t_layer * 1e3, 4),
            "tokens_per_s": round(cfg.T / t_layer, 1),
            "layer_alg_bytes": layer_bytes,
            "layer_hbm_frac": round(layer_bytes / t_layer / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_us": {"gate_up": round(t_gu * 1e6, 2), "down": round(t_dn * 1e6, 2)},
            "gate_up_alg_bytes": gu_bytes,
            "gate_up_hbm_frac": round(gu_bytes / t_gu / 1e9 / HBM_PEAK_GBS, 4),
            "down_hbm_frac": round(dn_bytes / t_dn / 1e9 / HBM_PEAK_GBS, 4)}


def config_dict(cfg, seed, ac, rot):
    return {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "f": cfg.f, "E": cfg.E,
            "k": cfg.k, "shared": cfg.S, "zipf_s": cfg.zipf_s, "seed": seed,
            "active_experts": ac["active"], "weight_copies": rot,
            "parallelism": "single GPU"}


def prefill_extra(torch, moe, steps, no_cpu, no_aux=False):
    """The Mixtral-8x7B-shaped prefill layer (T=8192, d=4096, f=14336, E=8,
    top-2): layer tokens/s and its fraction of the bf16 MFMA peak."""
    import moe_synth
    cfg = moe_synth.CONFIGS[PREFILL_CONFIG]
    L = Layer(torch, moe, cfg, PREFILL_CONFIG)
    for i in range(3):
        L.step(i)
    kt = L.kernel_times(torch, 5)
    wall, ev = L.timed_steps(torch, steps)
    ac, roof, layer = L.summary(torch, kt, ev / steps)
    if not no_aux:
        layer["aux"] = L.aux_times(torch, 5)
        layer["backward"] = L.backward_time(torch, 3)
    out = {"workload": cfg.name, "steps": steps,
           "ms_per_step": round(wall / steps * 1e3, 4),
           "ms_per_step_hip_events": round(ev / steps * 1e3, 4),
           "tokens_per_s": round(cfg.T * steps / wall, 1),
           "config": config_dict(cfg, PREFILL_CONFIG, ac, 1),
           "roofline": roof, "layer": layer}
    if not no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, L.inp, 5.0)
    del L
    torch.cuda.empty_cache()
    return out


def main(argv=None):
    args = parse(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the layer runs on a single MI355X)", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "launches": 10}), flush=True)
        return

    import moe_synth
    import mixture_experts_sparse_router_amd as moe

    cfg = moe_synth.CONFIGS[args.config]
    seed = args.seed if args.seed is not None else args.config
    torch.cuda.set_device(0)
    L = Layer(torch, moe, cfg, seed, args.rotate)

    # clock spin-up (untimed), then the warmup steps
    t_spin = time.perf_counter()
    while (time.perf_counter() - t_spin) * 1e3 < args.spinup_ms:
        for i in range(10):
            L.step(i)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        L.step(i)
    torch.cuda.synchronize()
    # per-step kernel times (each entry point timed alone on the same buffers)
    kt = L.kernel_times(torch, max(20, min(args.steps, 200)))
    wall, ev = L.timed_steps(torch, args.steps)
    ms_per_step = wall / args.steps * 1e3
    tok_s = cfg.T * args.steps / wall
    ac, roof, layer = L.summary(torch, kt, wall / args.steps)
    layer["ms_per_step_hip_events"] = round(ev / args.steps * 1e3, 4)
    layer["hbm_frac_hip_events"] = round(ac["layer_bytes"] / (ev / args.steps) / 1e9
                                         / HBM_PEAK_GBS, 4)
    if not args.no_aux:
        layer["aux"] = L.aux_times(torch, max(20, min(args.steps, 100)))
        layer["backward"] = L.backward_time(torch, 10 if cfg.T > 64 else 50)
    mx = None
    if not args.no_mxfp4 and cfg.T <= 64 and cfg.dtype == "bf16" and cfg.d % 32 == 0 \
            and cfg.f % 32 == 0:
        mx = mxfp4_extra(torch, moe, L, args.steps)

    out = {
        "metric": "MoE layer tokens/s",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "spinup_ms": args.spinup_ms,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) tokens, N(0,0.02) weights)",
        "config": config_dict(cfg, seed, ac, L.rot),
        "roofline": roof,
        "layer": layer,
        "cpu_baseline": None,
    }
    if mx is not None:
        out["mxfp4"] = mx
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(cfg, L.inp, args.cpu_seconds)
        out["cpu_baseline"]["gpu_over_cpu"] = round(tok_s / out["cpu_baseline"]["value"], 1)
    if not args.no_prefill and args.config != PREFILL_CONFIG:
        del L
        torch.cuda.empty_cache()
        out["prefill"] = prefill_extra(torch, moe, args.prefill_steps, args.no_cpu,
                                       args.no_aux)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
