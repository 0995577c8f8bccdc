"""Benchmark of the NVFP4 x Q8_0 hot path on one MI355X.

Headline (``value``): decode weight-streaming throughput, GB/s of NVFP4 weight
bytes, for one transformer layer at hidden 5120 / ffn 17408 with M = 1 token:
one step = Q8_0 quantization of the four GEMV inputs + the QKV [7168x5120],
O [5120x5120], gate+up [34816x5120] and down [5120x17408] GEMVs.  The layer's
185.8 MB of weights are replicated ``--copies`` times in HBM and step s uses copy
s % copies, so consecutive steps never find their weights in the 256 MB
Infinity Cache.  Inputs are resident in HBM before the timed region.

Also measured in the same run (reported as sub-objects of the JSON line): the
prefill GEMM TFLOP/s at M = 2048 (and 256), N = 17408, K = 5120; the small
GEMV (N = 4864, K = 896) and the Q4_1 GEMV / GEMM (N = K = 4096); the oracle's
CPU throughput on the same layer.  ``--stack`` instead measures the 64-layer
stack (M = 1 or 8) of the same layer shapes.

Roofline: per-kernel durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream).  Peaks: HBM 8000 GB/s, dense
fp16 MFMA 2500 TFLOP/s (the GEMM computes in fp16 x fp16 -> fp32).

Every timed region starts at the GPU's steady clock: the W warm-up steps of the
layer (default 2000, about 0.1 s, before K = 2000 timed steps) and, for every other
measurement, about 0.25 s of untimed repeats of the same work run right before it.  An idle MI355X needs tens of
milliseconds to raise its engine clock; a GEMM timed during that ramp reads ~20 %
slow, an HBM-bound GEMV about 1 %.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
METRIC = "NVFP4×Q8_0 GEMV weight GB/s (M=1) and GEMM TOPS (M=2048), % of roofline"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=2000)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--copies", type=int, default=8, help="distinct HBM copies of the layer weights")
    p.add_argument("--spin-up", type=float, default=0.25,
                   help="seconds of untimed repeats before each timed measurement other than the layer step "
                        "(shorter values keep profiler traces small)")
    p.add_argument("--eager", action="store_true",
                   help="launch every kernel from Python instead of replaying a captured HIP graph")
    p.add_argument("--no-gemm", action="store_true")
    p.add_argument("--no-extras", action="store_true")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--stack", action="store_true", help="64-layer stack instead of one layer")
    p.add_argument("--tokens", type=int, default=1, help="tokens for --stack (1 or 8)")
    p.add_argument("--only-gemm", action="store_true", help="time only the prefill GEMM (profiling)")
    p.add_argument("--only-moe", action="store_true", help="time only the expert-routed decode step (profiling)")
    p.add_argument("--only-q4-1", action="store_true", help="time only the Q4_1 GEMV and GEMM (profiling)")
    p.add_argument("--traffic-probe", action="store_true",
                   help="for rocprofv3 --pmc runs: one 256 MiB device copy (calibration) and 4 gate+up "
                        "GEMV launches over distinct weight copies, then exit")
    return p.parse_args()


# ---------------------------------------------------------------------------
# helpers
# ---------------------------------------------------------------------------

def dev_tensor(a):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def nvfp4_bytes(N, K):
    return N * K * 9 // 16


def gemv_alg_bytes(M, N, K):
    """Bytes the product must move: packed weights + Q8_0 activations (codes +
    binary16 scale per 32) + float32 outputs."""
    return nvfp4_bytes(N, K) + M * K * 17 // 16 + 4 * M * N


class Layer:
    """Device-resident decode layer: packed weights (``copies`` replicas), activations."""

    def __init__(self, M, copies, seed_base=0, share_from=None):
        import torch

        import gemm_q8_act_amd as nvq
        from gemm_q8_act_amd import synth

        self.M = M
        self.mats = []
        for i, (name, N, K) in enumerate(synth.LAYER):
            if share_from is None:
                codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name, seed_base), "uniform")
                packed = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
            else:
                packed, ws = share_from.mats[i]["w"][0], share_from.mats[i]["ws"]
            if share_from is None:
                ws_list = [packed] + [packed.clone() for _ in range(copies - 1)]
            else:
                ws_list = [packed.clone() for _ in range(copies)]
            x = dev_tensor(synth.activations(M, K, synth.seed_for("layer", "x_" + name, seed_base)))
            self.mats.append(dict(
                name=name, N=N, K=K, w=ws_list, ws=float(ws), x=x,
                q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                d=torch.empty((M, K // 32), dtype=torch.int16, device="cuda"),
                y=torch.empty((M, N), dtype=torch.float32, device="cuda")))

    def weight_bytes(self):
        return sum(nvfp4_bytes(m["N"], m["K"]) for m in self.mats)

    def step(self, copy):
        import gemm_q8_act_amd as nvq

        for m in self.mats:
            nvq.nvq_quantize_act_q8_0(m["x"], m["q"], m["d"])
            nvq.nvq_gemv_nvfp4(m["w"][copy], m["ws"], m["q"], m["d"], m["y"])


def kernel_src_hash():
    h = hashlib.sha256()
    for f in sorted(os.listdir(os.path.join(ROOT, "gemm_q8_act_amd", "csrc"))):
        with open(os.path.join(ROOT, "gemm_q8_act_amd", "csrc", f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(kernel_key):
    """HBM traffic per launch measured with rocprofv3 --pmc (FETCH_SIZE, WRITE_SIZE),
    recorded under profiles/ with the hash of the kernel sources it was taken on;
    None once the kernels have changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    e = t.get(kernel_key)
    if not e or e.get("src_hash") != kernel_src_hash():
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------

def time_layer(args):
    import torch

    M = 1
    layer = Layer(M, args.copies)
    torch.cuda.synchronize()
    for c in range(args.copies):  # one eager pass over every weight copy before capture
        layer.step(c)
    torch.cuda.synchronize()

    graph = None
    if not args.eager:
        # one graph holds `copies` consecutive steps (one per weight copy)
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s_cap):
                for c in range(args.copies):
                    layer.step(c)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()

    # the W untimed warm-up steps run right before the timed region: an idle GPU takes
    # tens of milliseconds to raise its engine clock
    if graph is not None:
        for _ in range(max(1, -(-args.warmup // args.copies))):
            graph.replay()
    else:
        for s in range(args.warmup):
            layer.step(s % args.copies)
    steps = args.steps
    if graph is not None:
        reps = max(1, steps // args.copies)
        steps = reps * args.copies
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if graph is not None:
        for _ in range(reps):
            graph.replay()
    else:
        for s in range(steps):
            layer.step(s % args.copies)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0

    # per-kernel durations: HIP events on the launch stream around batches of
    # back-to-back launches of one GEMV over >= 1 GB of weight copies
    per = {}
    for m in layer.mats:
        per[m["name"]] = gemv_batch_time(layer, m)
        per[m["name"]]["dot4_us"] = gemv_batch_time(layer, m, dot4=True)["us_avg"]
    return layer, steps, elapsed, per


def gemv_batch_time(layer, m, dot4=False, min_bytes=1 << 30, reps=6):
    """Average launch duration of one GEMV: HIP events (on the launch stream) around a
    batch of back-to-back launches that rotate through at least ``min_bytes`` of
    distinct weight copies, so no launch finds its weights in the 256 MB Infinity
    Cache.  A backlog queued before each batch (see ``backlog``) lets the host enqueue
    the whole batch before the GPU reaches it, so the batch runs at the GPU's pace."""
    import torch

    import gemm_q8_act_amd as nvq

    fn = nvq.nvq_gemv_nvfp4_dot4 if dot4 else nvq.nvq_gemv_nvfp4
    wbytes = nvfp4_bytes(m["N"], m["K"])
    extra = max(0, -(-min_bytes // wbytes) - len(m["w"]))
    ws = list(m["w"]) + [m["w"][i % len(m["w"])].clone() for i in range(extra)]
    it = iter(range(10 ** 9))
    host_s, call_s = spin_up(lambda: fn(ws[next(it) % len(ws)], m["ws"], m["q"], m["d"], m["y"]))
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        backlog(host_s, call_s, len(ws))
        e0.record()
        for w in ws:
            fn(w, m["ws"], m["q"], m["d"], m["y"])
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / len(ws))
    nlaunch = len(ws)
    del ws
    us = 1e3 * float(np.mean(ms))
    ab = gemv_alg_bytes(layer.M, m["N"], m["K"])
    return dict(N=m["N"], K=m["K"], us_avg=us, us_p50=1e3 * float(np.median(ms)), alg_bytes=ab,
                GBps=ab / (us * 1e-6) / 1e9, launches_per_batch=nlaunch)


_SLEEP_RATE = []
SPIN_UP_S = 0.25


def spin_up(fn, seconds=None):
    """Untimed repeats of ``fn`` for about ``seconds`` (default ``--spin-up``) of wall
    time before a timed region: an idle MI355X takes tens of milliseconds to bring its
    engine clock up, and a matrix-core-bound kernel timed during that ramp reads up to
    ~20 % slow."""
    import torch

    seconds = SPIN_UP_S if seconds is None else seconds
    t0 = time.perf_counter()
    while True:
        a = time.perf_counter()
        for _ in range(8):
            fn()
        b = time.perf_counter()
        torch.cuda.synchronize()
        c = time.perf_counter()
        if c - t0 >= seconds:
            return (b - a) / 8, (c - a) / 8  # host enqueue time per call, wall time per call


def backlog(host_s, call_s, n):
    """Queue work ahead of a timed batch of ``n`` calls so that the GPU never waits for
    the host: nothing when a call keeps the GPU busy for at least four times the host's
    enqueue time (the host stays well ahead by itself), else a sleep kernel that lasts
    about as long as the host needs to enqueue the batch.  The sleep is kept that short
    because the engine clock sinks while it runs: a 5 ms sleep before a prefill GEMM
    costs it ~12 %.  With only a 2x margin, back-to-back 17 us GEMV launches read ~4 %
    slow against their traced durations: the queue stays one launch deep."""
    import torch

    if call_s >= 4.0 * host_s:
        return
    torch.cuda._sleep(int(sleep_cycles_per_ms() * (1e3 * 1.5 * n * host_s + 0.2)))


def sleep_cycles_per_ms():
    """Rate of torch.cuda._sleep (its spin counter ticks per ms), measured once."""
    import torch

    if not _SLEEP_RATE:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(1000000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_RATE.append(1e6 / max(e0.elapsed_time(e1), 1e-3))
    return _SLEEP_RATE[0]


def torch_reference_rates():
    """Context, not ceilings: torch's own device-to-device copy of 1 GiB (read + write
    bytes) and float32 sum over 1 GiB (read bytes).  A tuned streaming read reaches
    more than either on this chip (about 7 TB/s with 16-byte non-temporal loads)."""
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    v = a.view(torch.float32)
    for _ in range(2):
        b.copy_(a)
        v.sum()
    torch.cuda.synchronize()
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    for _ in range(5):
        v.sum()
    e2.record()
    torch.cuda.synchronize()
    copy_s = e0.elapsed_time(e1) / 5 * 1e-3
    read_s = e1.elapsed_time(e2) / 5 * 1e-3
    return dict(copy_GBps=2 * n / copy_s / 1e9, sum_read_GBps=n / read_s / 1e9,
                note="torch kernels on 1 GiB: device copy (read+write bytes), float32 sum (read bytes); "
                     "not a ceiling")


def torch_fp16_gemm_rate(M=2048, N=17408, K=5120, reps=20):
    """Context, not a ceiling of this kernel: torch.matmul (the vendor library's plain
    fp16 GEMM, no quantization) of the prefill shape, y[M][N] = x[M][K] . W[N][K]^T,
    timed like the GEMM below, on random N(0, 1) operands and on constant ones.  The
    gap between the two is the chip's power limit: random operands toggle more bits,
    and the engine clock drops to stay within the board power."""
    import torch

    out = dict(M=M, N=N, K=K)
    for kind in ("random", "constant"):
        if kind == "random":
            g = torch.Generator(device="cuda")
            g.manual_seed(1)
            a = torch.randn((M, K), dtype=torch.float16, device="cuda", generator=g)
            b = torch.randn((N, K), dtype=torch.float16, device="cuda", generator=g)
        else:
            a = torch.ones((M, K), dtype=torch.float16, device="cuda")
            b = torch.ones((N, K), dtype=torch.float16, device="cuda")
        bt = b.t()
        spin_up(lambda: torch.matmul(a, bt))
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            torch.matmul(a, bt)
        e1.record()
        torch.cuda.synchronize()
        us = 1e3 * e0.elapsed_time(e1) / reps
        tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
        out[kind] = dict(us_avg=us, TFLOPs=tf, frac=tf / FP16_PEAK_TFLOPS)
        del a, b, bt
    out["note"] = "torch.matmul fp16 x fp16 -> fp16 (vendor GEMM), context only"
    return out


def time_gemm(M, N=17408, K=5120, reps=20):
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("prefill", "w") + M)
    w = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
    x = dev_tensor(synth.activations(M, K, synth.seed_for("prefill", "x") + M, outliers=True))
    q = torch.empty((M, K), dtype=torch.int8, device="cuda")
    d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
    b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
    y = torch.empty((M, N), dtype=torch.float32, device="cuda")
    nvq.nvq_quantize_act_q8_0(x, q, d, b)
    need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_NVFP4, M, N, K)
    wsp = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    spin_up(lambda: nvq.nvq_gemm_nvfp4(w, ws, q, d, y, workspace=wsp))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for e0, e1 in ev:
        e0.record()
        nvq.nvq_gemm_nvfp4(w, ws, q, d, y, workspace=wsp)
        e1.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    us = 1e3 * float(np.mean(ms))
    tflops = 2.0 * M * N * K / (us * 1e-6) / 1e12
    return dict(M=M, N=N, K=K, us_avg=us, us_p50=1e3 * float(np.median(ms)), TFLOPs=tflops,
                frac=tflops / FP16_PEAK_TFLOPS)


def time_extras():
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    out = {}
    # small decode GEMV N=4864 K=896 (L2-resident, launch-bound)
    N, K = 4864, 896
    codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("gemv_small", "w"))
    w = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
    x = dev_tensor(synth.activations(1, K, synth.seed_for("gemv_small", "x")))
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    d = torch.empty((1, K // 32), dtype=torch.int16, device="cuda")
    b = torch.empty((1, K // 16), dtype=torch.int16, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    nvq.nvq_quantize_act_q8_0(x, q, d, b)
    us = _event_time(lambda: nvq.nvq_gemv_nvfp4(w, ws, q, d, y), 200)
    out["gemv_small_N4864_K896"] = dict(us_avg=us, GBps=gemv_alg_bytes(1, N, K) / (us * 1e-6) / 1e9)
    out.update(time_act_quant())
    out.update(time_q4_1())
    out["moe_routed_gemv"] = time_moe()
    return out


def time_act_quant():
    """Q8_0 activation quantization with bsum16: the prefill input (M = 2048, K = 5120,
    0.1 % outliers) against HBM, and one decode row (M = 1), which is launch-bound."""
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    out = {}
    for M, K in ((2048, 5120), (1, 5120)):
        x = dev_tensor(synth.activations(M, K, synth.seed_for("prefill", "x") + M, outliers=True))
        q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
        b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
        us = _event_time(lambda: nvq.nvq_quantize_act_q8_0(x, q, d, b), 100)
        byts = M * K * 4 + M * K + M * (K // 32) * 2 + M * (K // 16) * 2  # x in; q, d16, bsum16 out
        gbps = byts / (us * 1e-6) / 1e9
        out[f"act_quant_M{M}_K{K}"] = dict(us_avg=us, GBps=gbps, frac=gbps / HBM_PEAK_GBS, bytes=byts)
    return out


def time_q4_1():
    """Q4_1 N = K = 4096: the GEMV at M = 1 and the GEMM at M = 512."""
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    out = {}
    N = K = 4096
    qw, dw, mw = synth.q4_1_weights(N, K, synth.seed_for("q4_1", "w"))
    w = dev_tensor(nvq.nvq_pack_q4_1(qw, dw, mw))
    for M in (1, 512):
        x = dev_tensor(synth.activations(M, K, synth.seed_for("q4_1", "x") + M))
        q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
        b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        nvq.nvq_quantize_act_q8_0(x, q, d, b)
        if M == 1:
            us = _event_time(lambda: nvq.nvq_gemv_q4_1(w, q, d, b, y), 200)
            byts = N * K * 5 // 8 + K * 17 // 16 + K // 8 + 4 * N
            out["q4_1_gemv_N4096_K4096"] = dict(us_avg=us, GBps=byts / (us * 1e-6) / 1e9,
                                                note="10.5 MB of weights: Infinity-Cache resident across repeats")
        else:
            need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q4_1, M, N, K)
            wsq = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            us = _event_time(lambda: nvq.nvq_gemm_q4_1(w, q, d, b, y, workspace=wsq), 20)
            tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
            out["q4_1_gemm_M512_N4096_K4096"] = dict(
                us_avg=us, TFLOPs=tf, frac=tf / FP16_PEAK_TFLOPS,
                note="fp16 MFMA, three passes per product (weight and activation each split in two terms)")
    return out


def time_moe(steps=400):
    """Expert-routed decode step: 256 NVFP4 experts of N = K = 2048 (604 MB, more than
    the 256 MB Infinity Cache), one token, 6 distinct experts per step drawn afresh
    for every step (ids resident on the device before timing).  16 distinct experts
    are generated and copied into the 256 expert slots (distinct HBM buffers)."""
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    wl = synth.WORKLOADS["moe"]
    E, A, N, K = wl["experts"], wl["active"], wl["N"], wl["K"]
    eb = nvfp4_bytes(N, K)
    w = torch.empty(E * eb, dtype=torch.uint8, device="cuda")
    wsc = np.empty(E, np.float32)
    for e in range(16):
        codes, scales, s = synth.nvfp4_weights(N, K, synth.seed_for("moe", "w", e), "uniform")
        w[e * eb:(e + 1) * eb].copy_(dev_tensor(nvq.nvq_pack_nvfp4(codes, scales)))
        wsc[e] = s
    for e in range(16, E):
        w[e * eb:(e + 1) * eb].copy_(w[(e % 16) * eb:(e % 16 + 1) * eb])
        wsc[e] = wsc[e % 16]
    wsc_d = torch.from_numpy(wsc).cuda()
    ids = torch.from_numpy(synth.expert_ids(steps, A, E, synth.seed_for("moe", "ids"))).cuda()
    x = dev_tensor(synth.activations(1, K, synth.seed_for("moe", "x")))
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    d = torch.empty((1, K // 32), dtype=torch.int16, device="cuda")
    y = torch.empty((1, A, N), dtype=torch.float32, device="cuda")
    nvq.nvq_quantize_act_q8_0(x, q, d)
    it = iter(range(10 ** 9))

    def step():
        s = next(it) % steps
        nvq.nvq_gemv_nvfp4_routed(w, wsc_d, ids[s:s + 1], q, d, y)

    us = _event_time(step, steps)
    byts = A * eb + K * 17 // 16 + A * N * 4
    return dict(us_avg=us, GBps=byts / (us * 1e-6) / 1e9, frac=byts / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                experts=E, active=A, N=N, K=K, weight_bytes_per_step=A * eb,
                note="one launch per step (grid 128 tiles x 6 experts); each step's 6 experts drawn afresh")


def _event_time(fn, reps):
    import torch

    host_s, call_s = spin_up(fn)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    backlog(host_s, call_s, reps)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def cpu_baseline():
    """The oracle (plain scalar C, untouched) on the same decode layer: Q8_0
    quantization of the four inputs + all output rows of the four GEMVs, split over
    host threads by output rows."""
    import oracle
    from gemm_q8_act_amd import synth

    o = oracle.load()
    threads = min(16, os.cpu_count() or 1)
    mats = []
    for name, N, K in synth.LAYER:
        codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name, 0), "uniform")
        x = synth.activations(1, K, synth.seed_for("layer", "x_" + name, 0))
        mats.append((N, K, codes, scales, ws, x))
    t0 = time.perf_counter()
    wbytes = 0
    passes = 0
    while True:  # whole-layer passes until about 10 s of wall time have gone by
        for N, K, codes, scales, ws, x in mats:
            q, d, _ = o.quantize_q8_0(x)
            o.matmul_threads("nvfp4", (codes, scales, ws), q, d, np.arange(N), threads)
            wbytes += nvfp4_bytes(N, K)
        passes += 1
        el = time.perf_counter() - t0
        if el >= 10.0:
            break
    return dict(value=wbytes / el / 1e9, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{passes} passes over the full decode layer (Q8_0 of the 4 inputs + all 52224 output "
                       f"rows of the QKV/O/gate+up/down GEMVs), M=1; {el:.2f} s wall on {threads} host threads")


def run_stack(args):
    """64-layer stack of the layer shapes, one token step = 256 GEMVs (+ their
    input quantization) back to back on one stream."""
    import torch

    M = args.tokens
    # layer 0's packed weights are cloned into 63 more distinct HBM buffers
    # (11.9 GB in all); activations differ per layer
    layers = [Layer(M, 1)]
    layers += [Layer(M, 1, seed_base=i, share_from=layers[0]) for i in range(1, 64)]
    torch.cuda.synchronize()
    wbytes = sum(l.weight_bytes() for l in layers)
    for _ in range(2):
        for l in layers:
            l.step(0)
    torch.cuda.synchronize()
    graph = None
    if not args.eager:  # one stack step (256 quantizations + 256 GEMVs) per graph replay
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s_cap):
                for l in layers:
                    l.step(0)
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()
    # untimed warm-up steps for about SPIN_UP_S seconds right before the timed region
    # (the engine clock of an idle GPU takes tens of milliseconds to come up)
    warm = 0
    t0 = time.perf_counter()
    while warm < 2 or time.perf_counter() - t0 < SPIN_UP_S:
        if graph is not None:
            graph.replay()
        else:
            for l in layers:
                l.step(0)
        torch.cuda.synchronize()
        warm += 1
    steps = max(2, args.steps // 20)
    t0 = time.perf_counter()
    for _ in range(steps):
        if graph is not None:
            graph.replay()
        else:
            for l in layers:
                l.step(0)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gbps = wbytes * steps / el / 1e9
    line = dict(metric=METRIC, value=gbps, unit="GB/s", n_gpus=1, steps=steps, warmup=warm,
                ms_per_step=1e3 * el / steps, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="int8/fp32", data="synthetic",
                config=dict(workload=f"64-layer decode stack, M={M}, hidden 5120, ffn 17408",
                            weight_bytes=wbytes, graph=not args.eager),
                roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=gbps / HBM_PEAK_GBS, traffic=None))
    print(json.dumps(line), flush=True)


def traffic_probe():
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    n = 256 << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    torch.cuda.synchronize()
    b.copy_(a)  # calibration: n bytes read, n bytes written
    torch.cuda.synchronize()
    name, N, K = [t for t in synth.LAYER if t[0] == "gate_up"][0]
    codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name, 0), "uniform")
    w0 = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
    wl = [w0] + [w0.clone() for _ in range(3)]
    x = dev_tensor(synth.activations(1, K, synth.seed_for("layer", "x_" + name, 0)))
    q = torch.empty((1, K), dtype=torch.int8, device="cuda")
    d = torch.empty((1, K // 32), dtype=torch.int16, device="cuda")
    y = torch.empty((1, N), dtype=torch.float32, device="cuda")
    nvq.nvq_quantize_act_q8_0(x, q, d, None)
    torch.cuda.synchronize()
    for w in wl:
        nvq.nvq_gemv_nvfp4(w, float(ws), q, d, y)
    torch.cuda.synchronize()
    log(f"traffic probe: copy {n} B; 4 x gate+up GEMV N={N} K={K}, {nvfp4_bytes(N, K)} weight bytes each")


def summarize_pmc(fetch_csv, write_csv):
    """HBM bytes per dispatch from two rocprofv3 --pmc runs of --traffic-probe
    (FETCH_SIZE, then WRITE_SIZE, KiB per dispatch), each scaled by the factor that
    maps the counter to the known bytes of the 256 MiB calibration copy."""
    import collections
    import csv

    def dispatches(path, counter):  # [(kernel name, grid, value summed over instances)]
        acc = collections.defaultdict(float)
        names = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                acc[r["Dispatch_Id"]] += float(r["Counter_Value"])
                names[r["Dispatch_Id"]] = (r["Kernel_Name"].split("(")[0], r.get("Grid_Size", ""))
        return [(names[i][0], names[i][1], v) for i, v in acc.items()]

    f = dispatches(fetch_csv, "FETCH_SIZE")
    wr = dispatches(write_csv, "WRITE_SIZE")
    n = 256 << 20
    # the calibration copy is the largest copyBuffer dispatch of each run
    cf = max(v for k, g, v in f if "copyBuffer" in k)
    cw = max(v for k, g, v in wr if "copyBuffer" in k)
    ff, fw = (n / 1024) / cf, (n / 1024) / cw
    res = dict(calibration=dict(copy_bytes=n, fetch_kib=cf, write_kib=cw, fetch_factor=ff, write_factor=fw))
    gf = [(k, g, v) for k, g, v in f if "gemv_nvfp4_kernel" in k]
    gw = [v for k, g, v in wr if "gemv_nvfp4_kernel" in k]
    if gf:
        vf, vw = float(np.mean([v for _, _, v in gf])), float(np.mean(gw)) if gw else 0.0
        res["gemv_nvfp4_gate_up"] = dict(
            kernel=gf[0][0], grid=gf[0][1], dispatches=len(gf), fetch_kib=vf, write_kib=vw,
            bytes_per_launch=(vf * ff + vw * fw) * 1024, alg_bytes_per_launch=gemv_alg_bytes(1, 34816, 5120),
            src_hash=kernel_src_hash())
    print(json.dumps(res, indent=1))


def summarize_trace(path):
    """Per-(kernel, grid) summary of a rocprofv3 kernel_trace.csv."""
    import collections
    import csv

    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    for r in rows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
        agg[(r["Kernel_Name"].split("(")[0], grid)].append(dur)
    out = []
    for (name, grid), d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d, np.float64) / 1e3
        out.append(f"{name[:60]:60s} grid={grid:>16s} n={len(d):5d} avg_us={d.mean():9.2f} "
                   f"p50_us={np.median(d):9.2f} min_us={d.min():9.2f} total_us={d.sum():11.1f}")
    print("\n".join(out))


def summarize_clock(run_dir):
    """Engine clock per (kernel, grid) from a ``rocprofv3 --pmc GRBM_COUNT`` run:
    GRBM_COUNT (GPU clocks, summed over the XCDs) / XCD count / dispatch time.  The
    counting window is a few microseconds longer than the dispatch, so kernels shorter
    than ~0.2 ms read high; long ones read the clock they ran at."""
    import collections
    import csv

    xcc = next(int(r["Num_Xcc"]) for r in csv.DictReader(open(os.path.join(run_dir, "run_agent_info.csv")))
               if r.get("Name", "").startswith("gfx"))
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(os.path.join(run_dir, "run_counter_collection.csv"))):
        if r["Counter_Name"] != "GRBM_COUNT":
            continue
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        agg[(r["Kernel_Name"].split("(")[0], r["Grid_Size"])].append((us, float(r["Counter_Value"]) / xcc / us))
    for (name, grid), v in sorted(agg.items(), key=lambda kv: -sum(u for u, _ in kv[1])):
        us = np.array([u for u, _ in v])
        mhz = np.array([f for _, f in v])
        print(f"{name[:60]:60s} grid={grid:>9s} n={len(v):5d} avg_us={us.mean():9.2f} "
              f"clock_MHz p50={np.median(mhz):6.0f} min={mhz.min():6.0f} max={mhz.max():6.0f}")


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-trace":
        summarize_trace(sys.argv[2])
        return
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-clock":
        summarize_clock(sys.argv[2])
        return
    if len(sys.argv) == 4 and sys.argv[1] == "--summarize-pmc":
        summarize_pmc(sys.argv[2], sys.argv[3])
        return
    args = parse()
    global SPIN_UP_S
    SPIN_UP_S = args.spin_up
    ws = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or ws != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}, WORLD_SIZE {ws}).", file=sys.stderr, flush=True)
        sys.exit(2)
    import torch

    import gemm_q8_act_amd as nvq

    nvq.lib()  # fails loudly if libnvq.so is missing
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)

    if args.traffic_probe:
        traffic_probe()
        return
    if args.stack:
        run_stack(args)
        return
    if args.only_gemm:
        for M in (2048, 256):
            log(json.dumps(time_gemm(M)))
        return
    if args.only_moe:
        log(json.dumps(time_moe()))
        return
    if args.only_q4_1:
        log(json.dumps(time_q4_1()))
        return

    log("decode layer ...")
    layer, steps, elapsed, per = time_layer(args)
    wbytes = layer.weight_bytes()
    gbps = wbytes * steps / elapsed / 1e9
    # dominant kernel: the gate+up GEMV (54 % of the step's weight bytes)
    gu = per["gate_up"]
    roofline = dict(bound="hbm", achieved=gu["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=gu["GBps"] / HBM_PEAK_GBS, traffic=load_traffic("gemv_nvfp4_gate_up"),
                    kernel="gemv_nvfp4_kernel<0,false,4,5> (matrix-core decode GEMV), gate+up N=34816 K=5120",
                    us_per_launch=gu["us_avg"], alg_bytes_per_launch=gu["alg_bytes"])
    line = dict(metric=METRIC, value=gbps, unit="GB/s", n_gpus=1, steps=steps, warmup=args.warmup,
                ms_per_step=1e3 * elapsed / steps, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="int8/fp32", data="synthetic",
                config=dict(workload="decode layer hidden=5120 ffn=17408, M=1: Q8_0 + QKV/O/gate_up/down GEMVs",
                            weight_bytes_per_step=wbytes, weight_copies=args.copies,
                            graph=not args.eager),
                roofline=roofline, per_kernel=per)
    if not args.no_extras:
        line["torch_reference_rates"] = torch_reference_rates()
    if not args.no_gemm:
        log("prefill gemm ...")
        g = {f"M{M}": time_gemm(M) for M in (2048, 256)}
        g2 = g["M2048"]
        line["gemm"] = dict(metric="NVFP4xQ8_0 prefill GEMM TFLOP/s (M=2048, N=17408, K=5120)",
                            value=g2["TFLOPs"], unit="TFLOP/s",
                            roofline=dict(bound="mfma", achieved=g2["TFLOPs"], peak=FP16_PEAK_TFLOPS,
                                          unit="TFLOP/s", frac=g2["frac"], traffic=None,
                                          kernel="gemm_nvfp4_kernel<NvCfg<1,8,8,1>> + ksplit_reduce_kernel (fp16 "
                                                 "MFMA 32x32x16 on the exact hi/lo activation split)",
                                          mfma_issued_frac=2.0 * g2["frac"],
                                          note="algorithmic flops 2*M*N*K; the hi/lo split issues twice "
                                               "that on the matrix cores"),
                            runs=g, vendor_fp16_gemm=torch_fp16_gemm_rate())
    if not args.no_extras:
        log("extras ...")
        line["extras"] = time_extras()
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
