"""Benchmark of the NVFP4 x Q8_0 hot path on one MI355X.

Headline (``value``): decode weight-streaming throughput, GB/s of NVFP4 weight
bytes, for one transformer layer at hidden 5120 / ffn 17408 with M = 1 token:
one step = Q8_0 quantization of the four GEMV inputs + the QKV [7168x5120],
O [5120x5120], gate+up [34816x5120] and down [5120x17408] GEMVs, run as the library
runs a single token: four nvq_gemv_nvfp4_fused launches (the quantization inside
each GEMV).  The same step as eight launches (nvq_quantize_act_q8_0 +
nvq_gemv_nvfp4 per matrix) is timed beside it (``layer_two_launch``).  The layer's
185.8 MB of weights are replicated ``--copies`` times in HBM and step s uses copy
s % copies, so consecutive steps never find their weights in the 256 MB
Infinity Cache.  Inputs are resident in HBM before the timed region.

Also measured in the same run (reported as sub-objects of the JSON line): the
64-layer stack of the same layer shapes at M = 1 and M = 8 (11.9 GB of weights per
step); the prefill GEMM TFLOP/s at M = 2048 (and 256), N = 17408, K = 5120; the
small GEMV (N = 4864, K = 896), the Q4_1, Q4_K and IQ4_XS GEMVs (HBM-cold, rotating
over >= 1 GB of weight copies) and GEMMs (N = K = 4096); the oracle's CPU throughput on
the same layer.
``--stack`` measures only the stack (M = ``--tokens``).

Roofline: per-kernel durations come from HIP events recorded on the stream the
kernels are launched on (torch's current stream).  Peaks: HBM 8000 GB/s, dense
fp16 MFMA 2500 TFLOP/s (the GEMM computes in fp16 x fp16 -> fp32).

Every timed region starts at the GPU's steady clock: the layer runs its W warm-up
steps and then at least ``--spin-up`` seconds (default 0.25) of further untimed steps
right before the K timed ones, and every other measurement is preceded by the same
spin-up of its own work.  An idle MI355X needs tens of milliseconds to raise its
engine clock; a GEMM timed during that ramp reads ~20 % slow, an HBM-bound GEMV
about 1 %.  Exactly K layer steps are timed: captured HIP graphs of one to
``--copies`` consecutive steps (one per weight copy) are replayed so that step s uses
copy s % copies.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
# The integer-MFMA Q4-family GEMM is bound by its vector work: per output and 32-block a
# float conversion, a scale multiply and one fma (3 wave64 instructions per 64 lanes, 4
# cycles each), against 64 useful flops.  1024 SIMDs x 2.4 GHz / 4 x 64 / 3 x 64 flops:
I8_GEMM_VALU_CEILING_TFLOPS = 1024 * 2.4e9 / 4 * 64 / 3 * 64 / 1e12
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
    p.add_argument("--no-stack", action="store_true", help="skip the 64-layer stack sub-objects")
    p.add_argument("--stack", action="store_true", help="64-layer stack instead of one layer")
    p.add_argument("--tokens", type=int, default=1, help="tokens for --stack (1 or 8)")
    p.add_argument("--only-gemm", action="store_true", help="time only the prefill GEMM (profiling)")
    p.add_argument("--only-moe", action="store_true", help="time only the expert-routed decode step (profiling)")
    p.add_argument("--only-q4-1", action="store_true",
                   help="time only the Q4_1, Q4_K, Q5_K, Q6_K and IQ4_XS GEMVs and GEMMs (profiling)")
    p.add_argument("--floors", action="store_true",
                   help="loads-only floors of the decode GEMV launch shapes on the layer set, and the measured "
                        "ceilings, as one JSON line")
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


def fused_alg_bytes(N, K):
    """Bytes the fused quantization + GEMV of one token must move: packed weights +
    the float32 activation row + float32 outputs."""
    return nvfp4_bytes(N, K) + 4 * K + 4 * N


class Layer:
    """Device-resident decode layer: packed weights (``copies`` replicas), activations.
    ``share_from``: take that layer's packed weights (cloned into ``copies`` new
    buffers, or used as they are with ``clone=False``) instead of generating them."""

    def __init__(self, M, copies, seed_base=0, share_from=None, clone=True):
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
            elif clone:
                ws_list = [packed.clone() for _ in range(copies)]
            else:
                ws_list = list(share_from.mats[i]["w"])
            x = dev_tensor(synth.activations(M, K, synth.seed_for("layer", "x_" + name, seed_base)))
            self.mats.append(dict(
                name=name, N=N, K=K, w=ws_list, ws=float(ws), x=x,
                q=torch.empty((M, K), dtype=torch.int8, device="cuda"),
                d=torch.empty((M, K // 32), dtype=torch.int16, device="cuda"),
                y=torch.empty((M, N), dtype=torch.float32, device="cuda")))

    def weight_bytes(self):
        return sum(nvfp4_bytes(m["N"], m["K"]) for m in self.mats)

    def step(self, copy):
        """Quantization launch + GEMV launch per matrix."""
        import gemm_q8_act_amd as nvq

        for m in self.mats:
            nvq.nvq_quantize_act_q8_0(m["x"], m["q"], m["d"])
            nvq.nvq_gemv_nvfp4(m["w"][copy], m["ws"], m["q"], m["d"], m["y"])

    def step_fused(self, copy):
        """One launch per matrix: the quantization fused into the GEMV (M = 1 only)."""
        import gemm_q8_act_amd as nvq

        for m in self.mats:
            nvq.nvq_gemv_nvfp4_fused(m["w"][copy], m["ws"], m["x"], m["y"])


# the sources each measured kernel is built from (its traffic record is valid while
# they are unchanged)
KERNEL_SOURCES = {
    "gemv_nvfp4_gate_up": ("gemv_nvfp4.hip", "nvq_device.h"),
    "gemv_nvfp4_fused_gate_up": ("gemv_nvfp4.hip", "nvq_device.h"),
    "gemm_nvfp4_m2048": ("gemm_nvfp4.hip", "ksplit.h", "nvq_device.h"),
    "gemm_q4_1_m512": ("q4_1.hip", "ksplit.h", "nvq_device.h"),
}


def gemm_alg_bytes(fmt, M, N, K):
    """Algorithmic bytes of one GEMM call: packed weights + Q8_0 codes and scales + fp32 y."""
    wb = N * K * 9 // 16 if fmt == "nvfp4" else N * K * 5 // 8
    return wb + M * K + M * (K // 32) * 2 + 4 * M * N


def _code_only(text):
    """Source text without comments and with whitespace collapsed: a comment edit does
    not change the kernel a traffic record was taken on."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_src_hash(kernel_key):
    """Hash of the kernel's sources (comments stripped) and of the per-file compiler
    options they are built with: a record is stale once either changes."""
    from gemm_q8_act_amd import build as nvq_build

    h = hashlib.sha256()
    for f in sorted(KERNEL_SOURCES[kernel_key]):
        with open(os.path.join(ROOT, "gemm_q8_act_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
        if nvq_build.FILE_FLAGS.get(f):
            h.update(" ".join(nvq_build.FILE_FLAGS[f]).encode())
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
    if not e or e.get("src_hash") != kernel_src_hash(kernel_key):
        return None
    return e.get("bytes_per_launch")


# ---------------------------------------------------------------------------
# measurements
# ---------------------------------------------------------------------------

def time_layer(args, fused=True, layer=None):
    """Exactly --steps layer steps (after --warmup steps and the spin-up), fused
    (one launch per matrix) or as quantization + GEMV launches."""
    import torch

    M = 1
    if layer is None:
        layer = Layer(M, args.copies)
    step = layer.step_fused if fused else layer.step
    torch.cuda.synchronize()
    for c in range(args.copies):  # one eager pass over every weight copy before capture
        step(c)
    torch.cuda.synchronize()

    graphs = {}
    if not args.eager:
        # graphs[r] holds r consecutive layer steps over weight copies 0 .. r-1: a run of
        # n steps replays graphs[copies] n // copies times, then graphs[n % copies], so
        # step s always uses copy s % copies and any number of steps is exact.  (One
        # replay per step would add the graph launch's own ~6 us to every 47 us step.)
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            for r in range(1, args.copies + 1):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=s_cap):
                    for c in range(r):
                        step(c)
                graphs[r] = g
        torch.cuda.current_stream().wait_stream(s_cap)
        torch.cuda.synchronize()

    def run_steps(n):
        if graphs:
            for _ in range(n // args.copies):
                graphs[args.copies].replay()
            if n % args.copies:
                graphs[n % args.copies].replay()
        else:
            for s in range(n):
                step(s % args.copies)

    # the W untimed warm-up steps, then untimed steps for at least --spin-up seconds,
    # right before the timed region: an idle GPU takes tens of milliseconds to raise
    # its engine clock, and a few warm-up steps do not span that
    run_steps(args.warmup)
    spin = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < SPIN_UP_S:
        run_steps(64)
        spin += 64
        torch.cuda.synchronize()
    steps = args.steps
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    run_steps(steps)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    del graphs
    return layer, steps, elapsed, spin


def layer_kernel_times(layer):
    """Per-kernel durations: HIP events on the launch stream around batches of
    back-to-back launches of one GEMV over >= 1 GB of weight copies; the plain GEMV
    (its Q8_0 input already made), the fused one (from the float32 row), the v_dot4
    variant, and one quantization launch."""
    per = {}
    for m in layer.mats:
        per[m["name"]] = gemv_batch_time(layer, m)
        f = gemv_batch_time(layer, m, fused=True)
        per[m["name"]].update(fused_us=f["us_avg"], fused_us_p50=f["us_p50"], fused_GBps=f["GBps"],
                              fused_alg_bytes=f["alg_bytes"])
        per[m["name"]]["dot4_us"] = gemv_batch_time(layer, m, dot4=True)["us_avg"]
        per[m["name"]]["quant_us"] = _event_time(lambda: __import__("gemm_q8_act_amd").nvq_quantize_act_q8_0(
            m["x"], m["q"], m["d"]), 200)
    return per


def gemv_batch_time(layer, m, dot4=False, fused=False, min_bytes=1 << 30, reps=6):
    """Average launch duration of one GEMV: HIP events (on the launch stream) around a
    batch of back-to-back launches that rotate through at least ``min_bytes`` of
    distinct weight copies, so no launch finds its weights in the 256 MB Infinity
    Cache.  A backlog queued before each batch (see ``backlog``) lets the host enqueue
    the whole batch before the GPU reaches it, so the batch runs at the GPU's pace."""
    import torch

    import gemm_q8_act_amd as nvq

    if fused:
        def fn(w):
            nvq.nvq_gemv_nvfp4_fused(w, m["ws"], m["x"], m["y"])
    else:
        g = nvq.nvq_gemv_nvfp4_dot4 if dot4 else nvq.nvq_gemv_nvfp4

        def fn(w):
            g(w, m["ws"], m["q"], m["d"], m["y"])
    wbytes = nvfp4_bytes(m["N"], m["K"])
    extra = max(0, -(-min_bytes // wbytes) - len(m["w"]))
    ws = list(m["w"]) + [m["w"][i % len(m["w"])].clone() for i in range(extra)]
    it = iter(range(10 ** 9))
    host_s, call_s = spin_up(lambda: fn(ws[next(it) % len(ws)]))
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        backlog(host_s, call_s, len(ws))
        e0.record()
        for w in ws:
            fn(w)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / len(ws))
    nlaunch = len(ws)
    del ws
    us = 1e3 * float(np.mean(ms))
    ab = fused_alg_bytes(m["N"], m["K"]) if fused else gemv_alg_bytes(layer.M, m["N"], m["K"])
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


def measured_ceilings():
    """Ceilings measured with the library's own probes (include/nvq_probe.h): the
    streaming-read rate over 4 GiB (16-byte non-temporal loads, best of four grid
    sizes) and the rate of back-to-back fp16 MFMAs (v_mfma_f32_32x32x16_f16, two
    wavefronts per SIMD) on constant and on hashed operands -- the board lowers its
    clock when the operands toggle many bits, so the second is what a GEMM on real
    data can at most issue."""
    import torch

    import gemm_q8_act_amd as nvq

    n = 4 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(3)
    read = {}
    for blocks in (2048, 4096, 8192, 16384):
        sink = torch.empty(4 * blocks, dtype=torch.int32, device="cuda")
        us = _event_time(lambda: nvq.nvq_probe_read(src, blocks, sink), 5)
        read[blocks] = n / (us * 1e-6) / 1e9
    del src
    torch.cuda.empty_cache()
    blocks, iters = 512, 4000
    out = torch.empty(256 * blocks, dtype=torch.float32, device="cuda")
    flops = blocks * 4 * 12 * iters * 32768
    mfma = {}
    for kind, rnd in (("constant", False), ("random", True)):
        us = _event_time(lambda: nvq.nvq_probe_mfma(blocks, iters, rnd, out), 20)
        mfma[kind] = flops / (us * 1e-6) / 1e12
    best = max(read, key=read.get)
    return dict(read_GBps=read[best], read_bytes=n, read_blocks=best,
                read_GBps_by_blocks={str(k): v for k, v in read.items()},
                mfma_fp16_constant_TFLOPs=mfma["constant"], mfma_fp16_random_TFLOPs=mfma["random"],
                note="nvq_probe_read (4 GiB, 256-thread blocks, 8 loads in flight per thread) and nvq_probe_mfma "
                     "(512 blocks x 256 threads, 12 MFMAs per iteration, constant / hashed fp16 operands)")


def time_floors():
    """Loads-only floors of the single-token decode GEMV on the layer set: for every
    matrix, nvq_probe_gemv_loads (the GEMV's weight loads and nothing else) with the
    plain and fused GEMVs' own launch shapes and over a sweep of K splits (blocks per
    tile) and launch shapes, each HBM-cold (launches rotating over >= 1 GB of weight
    copies), next to the GEMVs themselves timed the same way."""
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    # the launch shapes nvq_gemv_nvfp4 (M = 1) and nvq_gemv_nvfp4_fused pick for a shape
    def plain_shape(N, K):
        ntiles, nch = (N + 15) // 16, (K + 127) // 128
        if nch >= 64 and ntiles <= 1024:
            return (8, 3)
        return (8, 5) if ntiles >= 1024 else (4, 5)

    def fused_shape(N, K):
        ntiles, nch = (N + 15) // 16, (K + 127) // 128
        if nch <= 12:
            return (4, 3)
        if ntiles < 1024:
            return (16, 3) if nch >= 64 else (8, 3)
        return (8, 5)

    out = {}
    for name, N, K in synth.LAYER:
        codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name, 0), "uniform")
        w = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
        wbytes = nvfp4_bytes(N, K)
        copies = [w] + [w.clone() for _ in range(-(-(1 << 30) // wbytes) - 1)]
        x = dev_tensor(synth.activations(1, K, synth.seed_for("layer", "x_" + name, 0)))
        q = torch.empty((1, K), dtype=torch.int8, device="cuda")
        d = torch.empty((1, K // 32), dtype=torch.int16, device="cuda")
        y = torch.empty((1, N), dtype=torch.float32, device="cuda")
        nvq.nvq_quantize_act_q8_0(x, q, d)
        ntiles, nch = (N + 15) // 16, (K + 127) // 128
        sink = torch.empty(16 * ntiles * 8, dtype=torch.int32, device="cuda")

        def floor(S, W, P):
            return rotated_time(lambda wi: nvq.nvq_probe_gemv_loads(wi, N, K, S, W, P, sink), copies)

        gemv_us = rotated_time(lambda wi: nvq.nvq_gemv_nvfp4(wi, ws, q, d, y), copies)
        fused_us = rotated_time(lambda wi: nvq.nvq_gemv_nvfp4_fused(wi, ws, x, y), copies)
        pw, pp = plain_shape(N, K)
        fw, fp = fused_shape(N, K)
        sweep = {}
        for S in (1, 2, 4, 8):
            if S > nch:
                continue
            for W, P in ((4, 5), (8, 3), (8, 5), (16, 3)):
                sweep[f"S{S}_W{W}_P{P}"] = floor(S, W, P)
        best = min(sweep, key=sweep.get)
        fl_plain = sweep[f"S1_W{pw}_P{pp}"]
        fl_fused = sweep.get(f"S1_W{fw}_P{fp}") or floor(1, fw, fp)
        gb = lambda us: wbytes / (us * 1e-6) / 1e9
        out[name] = dict(N=N, K=K, weight_bytes=wbytes, copies=len(copies),
                         gemv_us=gemv_us, gemv_GBps=gb(gemv_us), fused_us=fused_us, fused_GBps=gb(fused_us),
                         floor_plain_shape=dict(shape=f"S1_W{pw}_P{pp}", us=fl_plain, GBps=gb(fl_plain)),
                         floor_fused_shape=dict(shape=f"S1_W{fw}_P{fp}", us=fl_fused, GBps=gb(fl_fused)),
                         floor_best=dict(shape=best, us=sweep[best], GBps=gb(sweep[best])),
                         gemv_vs_floor=fl_plain / gemv_us, fused_vs_floor=fl_fused / fused_us,
                         sweep_us=sweep)
        del copies
        torch.cuda.empty_cache()
    return out


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

    def two():
        nvq.nvq_quantize_act_q8_0(x, q, d)
        nvq.nvq_gemv_nvfp4(w, ws, q, d, y)

    us2 = _event_time(two, 200)
    usf = _event_time(lambda: nvq.nvq_gemv_nvfp4_fused(w, ws, x, y), 200)
    out["gemv_small_N4864_K896"] = dict(us_avg=us, GBps=gemv_alg_bytes(1, N, K) / (us * 1e-6) / 1e9,
                                        quant_plus_gemv_us=us2, fused_us=usf,
                                        note="L2-resident; us_avg is the GEMV on ready Q8_0 input, fused_us the one "
                                             "launch from float32 input, quant_plus_gemv_us the two launches")
    out.update(time_act_quant())
    out.update(time_q4_1())
    out.update(time_q4x("q4_k"))
    out.update(time_q4x("q5_k"))
    out.update(time_q4x("q6_k"))
    out.update(time_q4x("iq4_xs"))
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
            byts = N * K * 5 // 8 + K * 17 // 16 + K // 8 + 4 * N
            us_hot = _event_time(lambda: nvq.nvq_gemv_q4_1(w, q, d, b, y), 200)
            # HBM-cold: back-to-back launches rotating over >= 1 GB of distinct copies
            copies = [w] + [w.clone() for _ in range(-(-(1 << 30) // (N * K * 5 // 8)) - 1)]
            us = rotated_time(lambda wi: nvq.nvq_gemv_q4_1(wi, q, d, b, y), copies)
            gbps = byts / (us * 1e-6) / 1e9
            out["q4_1_gemv_N4096_K4096"] = dict(
                us_avg=us, GBps=gbps, alg_bytes=byts, copies=len(copies),
                roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbps / HBM_PEAK_GBS,
                              traffic=None, kernel="gemv_q4_1_m1_kernel (v_dot4 on unsigned codes)"),
                us_cache_resident=us_hot,
                note=f"HBM-cold: back-to-back launches over {len(copies)} distinct weight copies (>= 1 GB); "
                     f"us_cache_resident repeats one 10.5 MB copy (Infinity-Cache resident)")
            del copies
        else:
            need = nvq.nvq_gemm_workspace_bytes(nvq.NVQ_FMT_Q4_1, M, N, K)
            wsq = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            us = _event_time(lambda: nvq.nvq_gemm_q4_1(w, q, d, b, y, workspace=wsq), 20)
            tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
            out["q4_1_gemm_M512_N4096_K4096"] = dict(
                us_avg=us, TFLOPs=tf, frac=tf / INT8_PEAK_TOPS,
                frac_of_valu_ceiling=tf / I8_GEMM_VALU_CEILING_TFLOPS,
                traffic=load_traffic("gemm_q4_1_m512"), alg_bytes_per_launch=gemm_alg_bytes("q4_1", M, N, K),
                note="int8 MFMA (one exact code x activation sum per 32-block), block scales applied in fp32 "
                     "on the vector unit; frac against the int8 dense peak, frac_of_valu_ceiling against the "
                     f"{I8_GEMM_VALU_CEILING_TFLOPS:.0f} TFLOP/s the scaling's 3 vector instructions per output "
                     "and 32-block allow")
    return out


def time_q4x(fmt):
    """Q4_K, Q5_K, Q6_K or IQ4_XS (``fmt``) at N = K = 4096 (the Q4_1 workload's shape):
    the GEMV at M = 1 (HBM-cold) and the GEMM at M = 512."""
    import torch

    import gemm_q8_act_amd as nvq
    from gemm_q8_act_amd import synth

    out = {}
    N = K = 4096
    if fmt == "q4_k":
        w = dev_tensor(nvq.nvq_pack_q4_k(*synth.q4_k_weights(N, K, synth.seed_for("q4_k", "w"))))
        wbytes, abytes = nvq.nvq_q4_k_weight_bytes(N, K), K * 17 // 16 + K // 8
        gemv = lambda wi, q, d, b, y: nvq.nvq_gemv_q4_k(wi, q, d, b, y)
        gemm = lambda q, d, b, y, ws: nvq.nvq_gemm_q4_k(w, q, d, b, y, workspace=ws)
        ffmt, kname, blk = nvq.NVQ_FMT_Q4_K, "gemv_q4_1_m1_kernel<Q4_K> (v_dot4 on unsigned codes)", "144"
    elif fmt == "q5_k":
        w = dev_tensor(nvq.nvq_pack_q5_k(*synth.q5_k_weights(N, K, synth.seed_for("q5_k", "w"))))
        wbytes, abytes = nvq.nvq_q5_k_weight_bytes(N, K), K * 17 // 16 + K // 8
        gemv = lambda wi, q, d, b, y: nvq.nvq_gemv_q5_k(wi, q, d, b, y)
        gemm = lambda q, d, b, y, ws: nvq.nvq_gemm_q5_k(w, q, d, b, y, workspace=ws)
        ffmt, kname, blk = nvq.NVQ_FMT_Q5_K, "gemv_q4_1_m1_kernel<Q5_K> (fifth bits spliced, v_dot4)", "176"
    elif fmt == "q6_k":
        w = dev_tensor(nvq.nvq_pack_q6_k(*synth.q6_k_weights(N, K, synth.seed_for("q6_k", "w"))))
        wbytes, abytes = nvq.nvq_q6_k_weight_bytes(N, K), K * 17 // 16
        gemv = lambda wi, q, d, b, y: nvq.nvq_gemv_q6_k(wi, q, d, y)
        gemm = lambda q, d, b, y, ws: nvq.nvq_gemm_q6_k(w, q, d, y, workspace=ws)
        ffmt, kname, blk = nvq.NVQ_FMT_Q6_K, "gemv_q4_1_m1_kernel<Q6_K> (6-bit codes, per-16 scales, v_dot4)", "210"
    else:
        qw, ls, dd, table = synth.iq4_xs_weights(N, K, synth.seed_for("iq4_xs", "w"))
        w = dev_tensor(nvq.nvq_pack_iq4_xs(qw, ls, dd))
        wbytes, abytes = nvq.nvq_iq4_xs_weight_bytes(N, K), K * 17 // 16
        gemv = lambda wi, q, d, b, y: nvq.nvq_gemv_iq4_xs(wi, table, q, d, y)
        gemm = lambda q, d, b, y, ws: nvq.nvq_gemm_iq4_xs(w, table, q, d, y, workspace=ws)
        ffmt, kname, blk = nvq.NVQ_FMT_IQ4_XS, "gemv_q4_1_m1_kernel<IQ4_XS> (table lookups + v_dot4)", "136"
    for M in (1, 512):
        x = dev_tensor(synth.activations(M, K, synth.seed_for(fmt, "x") + M))
        q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
        b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        nvq.nvq_quantize_act_q8_0(x, q, d, b)
        if M == 1:
            byts = wbytes + abytes + 4 * N
            us_hot = _event_time(lambda: gemv(w, q, d, b, y), 200)
            copies = [w] + [w.clone() for _ in range(-(-(1 << 30) // wbytes) - 1)]
            us = rotated_time(lambda wi: gemv(wi, q, d, b, y), copies)
            gbps = byts / (us * 1e-6) / 1e9
            out[f"{fmt}_gemv_N4096_K4096"] = dict(
                us_avg=us, GBps=gbps, alg_bytes=byts, copies=len(copies),
                roofline=dict(bound="hbm", achieved=gbps, peak=HBM_PEAK_GBS, unit="GB/s", frac=gbps / HBM_PEAK_GBS,
                              traffic=None, kernel=kname),
                us_cache_resident=us_hot,
                note=f"HBM-cold over {len(copies)} distinct weight copies (>= 1 GB); {blk} bytes per 256 weights")
            del copies
        else:
            need = nvq.nvq_gemm_workspace_bytes(ffmt, M, N, K)
            wsq = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
            us = _event_time(lambda: gemm(q, d, b, y, wsq), 20)
            tf = 2.0 * M * N * K / (us * 1e-6) / 1e12
            if fmt == "q6_k":
                out[f"{fmt}_gemm_M512_N4096_K4096"] = dict(
                    us_avg=us, TFLOPs=tf, frac=tf / FP16_PEAK_TFLOPS,
                    note="the two-term fp16 kernel (one scale per 16 weights; three fp16 MFMA passes per product)")
            else:
                out[f"{fmt}_gemm_M512_N4096_K4096"] = dict(
                    us_avg=us, TFLOPs=tf, frac=tf / INT8_PEAK_TOPS,
                    frac_of_valu_ceiling=tf / I8_GEMM_VALU_CEILING_TFLOPS,
                    note="the Q4_1 integer-MFMA kernel with this format's block scales (frac against the int8 "
                         "dense peak)")
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


def rotated_time(fn, copies, reps=6):
    """Average duration of ``fn(copy)`` over back-to-back launches that rotate through
    ``copies`` (distinct HBM buffers, >= 1 GB in all, so no launch finds its weights in
    the 256 MB Infinity Cache): HIP events on the launch stream around each batch."""
    import torch

    it = iter(range(10 ** 9))
    host_s, call_s = spin_up(lambda: fn(copies[next(it) % len(copies)]))
    ms = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        backlog(host_s, call_s, len(copies))
        e0.record()
        for c in copies:
            fn(c)
        e1.record()
        torch.cuda.synchronize()
        ms.append(e0.elapsed_time(e1) / len(copies))
    return 1e3 * float(np.mean(ms))


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


def host_cpu():
    """Host CPU description: model name, logical CPUs, CPUs this process may run on."""
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    try:
        allowed = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        allowed = os.cpu_count() or 1
    return dict(cpu_model=model, logical_cpus=os.cpu_count(), cpus_allowed=allowed)


def cpu_baseline():
    """The oracle (plain scalar C, untouched) on the same decode layer: Q8_0
    quantization of the four inputs + all output rows of the four GEMVs, split over
    host threads by output rows (about 10 s), then one pass on a single thread."""
    import oracle
    from gemm_q8_act_amd import synth

    o = oracle.load()
    hc = host_cpu()
    threads = max(1, min(16, hc["cpus_allowed"]))
    mats = []
    for name, N, K in synth.LAYER:
        codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("layer", name, 0), "uniform")
        x = synth.activations(1, K, synth.seed_for("layer", "x_" + name, 0))
        mats.append((N, K, codes, scales, ws, x))

    def passes(nthreads, seconds):
        t0 = time.perf_counter()
        wbytes = n = 0
        while True:  # whole-layer passes until `seconds` of wall time have gone by
            for N, K, codes, scales, ws, x in mats:
                q, d, _ = o.quantize_q8_0(x)
                o.matmul_threads("nvfp4", (codes, scales, ws), q, d, np.arange(N), nthreads)
                wbytes += nvfp4_bytes(N, K)
            n += 1
            el = time.perf_counter() - t0
            if el >= seconds:
                return wbytes / el / 1e9, n, el

    gbps, n, el = passes(threads, 10.0)
    gbps1, n1, el1 = passes(1, 0.0)  # one pass
    return dict(value=gbps, unit="GB/s", cores=threads, kind="oracle",
                sample=f"{n} passes over the full decode layer (Q8_0 of the 4 inputs + all 52224 output rows of "
                       f"the QKV/O/gate+up/down GEMVs, 185.8 MB of NVFP4 weights), M=1; {el:.2f} s wall on "
                       f"{threads} host threads; then {n1} pass on 1 thread in {el1:.2f} s",
                single_thread_GBps=gbps1, host=hc)


def stack_layers(M, weights_from=None):
    """64 device-resident layers: layer 0's packed weights cloned into 63 more distinct
    HBM buffers (11.9 GB in all), or the weights of ``weights_from`` (another stack)
    used as they are; activations differ per layer."""
    if weights_from is None:
        layers = [Layer(M, 1)]
        layers += [Layer(M, 1, seed_base=i, share_from=layers[0]) for i in range(1, 64)]
    else:
        layers = [Layer(M, 1, seed_base=i, share_from=weights_from[i], clone=False) for i in range(64)]
    return layers


def time_stack(layers, steps, eager=False, fused=False):
    """One token step over the 64-layer stack = 256 GEMVs (+ their input
    quantization) back to back on one stream, one captured graph per step.
    ``fused`` (M = 1): one launch per matrix, the quantization inside the GEMV;
    otherwise a quantization launch + a GEMV launch per matrix."""
    import torch

    M = layers[0].M
    torch.cuda.synchronize()
    wbytes = sum(l.weight_bytes() for l in layers)
    if fused:
        alg = sum(fused_alg_bytes(m["N"], m["K"]) for l in layers for m in l.mats)
    else:
        alg = sum(gemv_alg_bytes(M, m["N"], m["K"]) for l in layers for m in l.mats)
    step = (lambda l: l.step_fused(0)) if fused else (lambda l: l.step(0))
    for _ in range(2):
        for l in layers:
            step(l)
    torch.cuda.synchronize()
    graph = None
    if not eager:  # one stack step (256 quantizations + 256 GEMVs) per graph replay
        s_cap = torch.cuda.Stream()
        s_cap.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s_cap):
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=s_cap):
                for l in layers:
                    step(l)
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
                step(l)
        torch.cuda.synchronize()
        warm += 1
    t0 = time.perf_counter()
    for _ in range(steps):
        if graph is not None:
            graph.replay()
        else:
            for l in layers:
                step(l)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    gbps = wbytes * steps / el / 1e9
    del graph
    return dict(M=M, steps=steps, warmup_steps=warm, ms_per_step=1e3 * el / steps, weight_GBps=gbps,
                weight_bytes_per_step=wbytes, alg_bytes_per_step=alg,
                roofline=dict(bound="hbm", achieved=alg * steps / el / 1e9, peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=alg * steps / el / 1e9 / HBM_PEAK_GBS, traffic=None,
                              scope=("whole stack step: 256 fused quantization + GEMV launches; algorithmic "
                                     "bytes = weights + fp32 activations + fp32 outputs") if fused else
                                    ("whole stack step: 256 Q8_0 launches + 256 GEMVs; algorithmic bytes = "
                                     "weights + Q8_0 activations + fp32 outputs")),
                graph=not eager)


def run_stack(args):
    """--stack: the 64-layer stack alone at M = --tokens, as the one JSON line."""
    M = args.tokens
    r = time_stack(stack_layers(M), max(2, min(args.steps, 50)), args.eager, fused=M == 1)
    line = dict(metric=METRIC, value=r["weight_GBps"], unit="GB/s", n_gpus=1, steps=r["steps"],
                warmup=r["warmup_steps"], ms_per_step=r["ms_per_step"], higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype="int8/fp32", data="synthetic",
                config=dict(workload=f"64-layer decode stack, M={M}, hidden 5120, ffn 17408"
                                     + (", fused quantization + GEMV launches" if M == 1 else ""),
                            weight_bytes=r["weight_bytes_per_step"], graph=r["graph"]),
                roofline=r["roofline"])
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
    for w in wl:
        nvq.nvq_gemv_nvfp4_fused(w, float(ws), x, y)
    torch.cuda.synchronize()
    log(f"traffic probe: copy {n} B; 4 x gate+up GEMV and 4 x fused gate+up N={N} K={K}, "
        f"{nvfp4_bytes(N, K)} weight bytes each")
    del wl, w0, w
    # the prefill GEMM (M = 2048, N = 17408, K = 5120) and the Q4_1 GEMM (M = 512,
    # N = K = 4096), two calls each on the bench's inputs
    for fmt, (M, N, K) in (("nvfp4", (2048, 17408, 5120)), ("q4_1", (512, 4096, 4096))):
        if fmt == "nvfp4":
            codes, scales, ws = synth.nvfp4_weights(N, K, synth.seed_for("prefill", "w") + M)
            w = dev_tensor(nvq.nvq_pack_nvfp4(codes, scales))
            x = dev_tensor(synth.activations(M, K, synth.seed_for("prefill", "x") + M, outliers=True))
        else:
            qw, dw, mw = synth.q4_1_weights(N, K, synth.seed_for("q4_1", "w"))
            w = dev_tensor(nvq.nvq_pack_q4_1(qw, dw, mw))
            x = dev_tensor(synth.activations(M, K, synth.seed_for("q4_1", "x") + M))
        q = torch.empty((M, K), dtype=torch.int8, device="cuda")
        d = torch.empty((M, K // 32), dtype=torch.int16, device="cuda")
        b = torch.empty((M, K // 16), dtype=torch.int16, device="cuda")
        y = torch.empty((M, N), dtype=torch.float32, device="cuda")
        nvq.nvq_quantize_act_q8_0(x, q, d, b)
        fmt_id = nvq.NVQ_FMT_NVFP4 if fmt == "nvfp4" else nvq.NVQ_FMT_Q4_1
        wsp = torch.empty(max(nvq.nvq_gemm_workspace_bytes(fmt_id, M, N, K), 16), dtype=torch.uint8, device="cuda")
        torch.cuda.synchronize()
        for _ in range(2):
            if fmt == "nvfp4":
                nvq.nvq_gemm_nvfp4(w, ws, q, d, y, workspace=wsp)
            else:
                nvq.nvq_gemm_q4_1(w, q, d, b, y, workspace=wsp)
        torch.cuda.synchronize()
        log(f"traffic probe: 2 x {fmt} GEMM M={M} N={N} K={K}")


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
                names[r["Dispatch_Id"]] = (short_kernel_name(r["Kernel_Name"]), r.get("Grid_Size", ""))
        return [(names[i][0], names[i][1], v) for i, v in acc.items()]

    f = dispatches(fetch_csv, "FETCH_SIZE")
    wr = dispatches(write_csv, "WRITE_SIZE")
    n = 256 << 20
    # the calibration copy is the largest copyBuffer dispatch of each run
    cf = max(v for k, g, v in f if "copyBuffer" in k)
    cw = max(v for k, g, v in wr if "copyBuffer" in k)
    ff, fw = (n / 1024) / cf, (n / 1024) / cw
    res = dict(calibration=dict(copy_bytes=n, fetch_kib=cf, write_kib=cw, fetch_factor=ff, write_factor=fw))
    for key, name, alg in (("gemv_nvfp4_gate_up", "gemv_nvfp4_kernel", gemv_alg_bytes(1, 34816, 5120)),
                           ("gemv_nvfp4_fused_gate_up", "gemv_nvfp4_fused_kernel", fused_alg_bytes(34816, 5120))):
        gf = [(k, g, v) for k, g, v in f if name in k]
        gw = [v for k, g, v in wr if name in k]
        if gf:
            vf, vw = float(np.mean([v for _, _, v in gf])), float(np.mean(gw)) if gw else 0.0
            res[key] = dict(
                kernel=gf[0][0], grid=gf[0][1], dispatches=len(gf), fetch_kib=vf, write_kib=vw,
                bytes_per_launch=(vf * ff + vw * fw) * 1024, alg_bytes_per_launch=alg,
                src_hash=kernel_src_hash(key))
    # GEMM calls: the main kernel and its K-split reduction, summed per call
    for key, main, red, alg in (("gemm_nvfp4_m2048", "gemm_nvfp4_kernel<", "ksplit_reduce_kernel<NvCfg<",
                                 gemm_alg_bytes("nvfp4", 2048, 17408, 5120)),
                                ("gemm_q4_1_m512", "gemm_q4x_i8_kernel<", "ksplit_reduce_kernel<QI8Cfg<",
                                 gemm_alg_bytes("q4_1", 512, 4096, 4096))):
        parts = {}
        for label, name in (("main", main), ("reduce", red)):
            gf = [(k, g, v) for k, g, v in f if k.startswith(name)]
            gw = [v for k, g, v in wr if k.startswith(name)]
            if gf:
                vf, vw = float(np.mean([v for _, _, v in gf])), float(np.mean(gw)) if gw else 0.0
                parts[label] = dict(kernel=gf[0][0], grid=gf[0][1], dispatches=len(gf), fetch_kib=vf, write_kib=vw,
                                    bytes=(vf * ff + vw * fw) * 1024)
        if "main" in parts:
            res[key] = dict(parts=parts, bytes_per_launch=sum(p["bytes"] for p in parts.values()),
                            alg_bytes_per_launch=alg, src_hash=kernel_src_hash(key),
                            note="per call: the main kernel plus its K-split reduction")
    print(json.dumps(res, indent=1))


def short_kernel_name(name):
    """A kernel's name with its template arguments and without its parameter list,
    namespaces and return type: ``gemm_q4_1_f16x2_kernel<Q41Cfg<2, 4, 2, 2>, 1, false>``."""
    name = name.replace("(anonymous namespace)::", "").replace("nvq::", "")
    name = name.split("(")[0]
    return name[5:] if name.startswith("void ") else name


def summarize_trace(path):
    """Per-(kernel, grid) summary of a rocprofv3 kernel_trace.csv."""
    import collections
    import csv

    rows = list(csv.DictReader(open(path)))
    agg = collections.defaultdict(list)
    for r in rows:
        dur = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
        grid = "x".join(r.get(k, "?") for k in ("Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"))
        agg[(short_kernel_name(r["Kernel_Name"]), grid)].append(dur)
    out = []
    for (name, grid), d in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        d = np.array(d, np.float64) / 1e3
        out.append(f"{name[:66]:66s} grid={grid:>16s} n={len(d):5d} avg_us={d.mean():9.2f} "
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


def summarize_counters(run_dir):
    """Per (kernel, grid) average over dispatches of every counter of a rocprofv3 --pmc
    run (``*counter_collection.csv`` in ``run_dir``), with the average dispatch time."""
    import collections
    import csv

    path = next(os.path.join(run_dir, f) for f in os.listdir(run_dir) if f.endswith("counter_collection.csv"))
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    disp = collections.defaultdict(set)
    dur = {}
    for r in csv.DictReader(open(path)):
        k = (short_kernel_name(r["Kernel_Name"])[:80], r.get("Grid_Size", ""))
        acc[k][r["Counter_Name"]] += float(r["Counter_Value"])
        disp[k].add(r["Dispatch_Id"])
        if "Start_Timestamp" in r:
            dur[(k, r["Dispatch_Id"])] = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
    for k, cs in acc.items():
        n = len(disp[k])
        us = [v for (kk, _), v in dur.items() if kk == k]
        print(f"{k[0]} grid={k[1]} dispatches={n} avg_us={sum(us) / max(1, len(us)):.2f}")
        for c, v in sorted(cs.items()):
            print(f"    {c:28s} {v / n:16.1f}")


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-counters":
        summarize_counters(sys.argv[2])
        return
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
        print("bench.py measures one GPU only: the library has no multi-GPU path "
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
    if args.floors:
        log("ceilings ...")
        c = measured_ceilings()
        log("loads-only floors ...")
        f = time_floors()
        print(json.dumps(dict(ceilings=c, floors=f)), flush=True)
        return
    if args.only_q4_1:
        log(json.dumps(time_q4_1()))
        log(json.dumps(time_q4x("q4_k")))
        log(json.dumps(time_q4x("q5_k")))
        log(json.dumps(time_q4x("q6_k")))
        log(json.dumps(time_q4x("iq4_xs")))
        return

    log("decode layer ...")
    layer, steps, elapsed, spin = time_layer(args, fused=True)
    _, steps2, elapsed2, spin2 = time_layer(args, fused=False, layer=layer)
    per = layer_kernel_times(layer)
    wbytes = layer.weight_bytes()
    gbps = wbytes * steps / elapsed / 1e9
    # dominant kernel: the gate+up GEMV (54 % of the step's weight bytes), here fused
    gu = per["gate_up"]
    gf = gu["fused_GBps"]
    roofline = dict(bound="hbm", achieved=gf, peak=HBM_PEAK_GBS, unit="GB/s", frac=gf / HBM_PEAK_GBS,
                    traffic=load_traffic("gemv_nvfp4_fused_gate_up"),
                    kernel="gemv_nvfp4_fused_kernel<8,5,3> (Q8_0 quantization + matrix-core decode GEMV, one "
                           "launch), gate+up N=34816 K=5120",
                    scope="the dominant kernel of the step alone (the fused gate+up GEMV, 54 % of the step's "
                          "weight bytes); `value` is the whole layer step (4 fused launches)",
                    us_per_launch=gu["fused_us"], alg_bytes_per_launch=gu["fused_alg_bytes"])
    roofline_gemv = dict(bound="hbm", achieved=gu["GBps"], peak=HBM_PEAK_GBS, unit="GB/s",
                         frac=gu["GBps"] / HBM_PEAK_GBS, traffic=load_traffic("gemv_nvfp4_gate_up"),
                         kernel="gemv_nvfp4_kernel<0,false,8,5> (matrix-core decode GEMV on Q8_0 input), gate+up",
                         us_per_launch=gu["us_avg"], alg_bytes_per_launch=gu["alg_bytes"])
    line = dict(metric=METRIC, value=gbps, unit="GB/s", n_gpus=1, steps=steps, warmup=args.warmup,
                ms_per_step=1e3 * elapsed / steps, higher_is_better=True, scaling="weak", vs_baseline=None,
                dtype="int8/fp32", data="synthetic",
                config=dict(workload="decode layer hidden=5120 ffn=17408, M=1: Q8_0 quantization + "
                                     "QKV/O/gate_up/down GEMVs, fused (one launch per matrix)",
                            weight_bytes_per_step=wbytes, weight_copies=args.copies,
                            graph=not args.eager, spin_up_steps=spin),
                roofline=roofline, roofline_gemv=roofline_gemv,
                layer_two_launch=dict(value=wbytes * steps2 / elapsed2 / 1e9, unit="GB/s", steps=steps2,
                                      ms_per_step=1e3 * elapsed2 / steps2, spin_up_steps=spin2,
                                      note="the same step as nvq_quantize_act_q8_0 + nvq_gemv_nvfp4 per matrix "
                                           "(8 launches)"),
                per_kernel=per)
    del layer
    if not args.no_stack:
        log("64-layer stack, M = 1 and 8 ...")
        nst = max(5, min(args.steps, 40))
        st1 = stack_layers(1)
        s1 = time_stack(st1, nst, args.eager, fused=True)
        s1b = time_stack(st1, nst, args.eager)
        st8 = stack_layers(8, weights_from=st1)
        s8 = time_stack(st8, nst, args.eager)
        line["stack"] = {"M1": s1, "M1_two_launch": s1b, "M8": s8,
                         "workload": "64 layers of the layer set (QKV/O/gate_up/down), 11.9 GB of NVFP4 weights "
                                     "resident, one graph replay per token step; M1: one fused quantization + "
                                     "GEMV launch per matrix; M1_two_launch: a Q8_0 launch + a GEMV launch per "
                                     "matrix; M8: batched decode (a Q8_0 launch + a batched GEMV per matrix)"}
        del st1, st8
        torch.cuda.empty_cache()
    if not args.no_extras:
        line["torch_reference_rates"] = torch_reference_rates()
        log("measured ceilings ...")
        ceil = measured_ceilings()
        line["ceilings"] = ceil
        for r in (line["roofline"], line["roofline_gemv"]):
            r["frac_of_measured_read"] = r["achieved"] / ceil["read_GBps"]
        if "stack" in line:
            for k in ("M1", "M1_two_launch", "M8"):
                rr = line["stack"][k]["roofline"]
                rr["frac_of_measured_read"] = rr["achieved"] / ceil["read_GBps"]
    if not args.no_gemm:
        log("prefill gemm ...")
        g = {f"M{M}": time_gemm(M) for M in (2048, 256)}
        g2 = g["M2048"]
        line["gemm"] = dict(metric="NVFP4xQ8_0 prefill GEMM TFLOP/s (M=2048, N=17408, K=5120)",
                            value=g2["TFLOPs"], unit="TFLOP/s",
                            roofline=dict(bound="mfma", achieved=g2["TFLOPs"], peak=FP16_PEAK_TFLOPS,
                                          unit="TFLOP/s", frac=g2["frac"], traffic=load_traffic("gemm_nvfp4_m2048"),
                                          alg_bytes_per_launch=gemm_alg_bytes("nvfp4", 2048, 17408, 5120),
                                          kernel="gemm_nvfp4_kernel<NvCfg<1,8,8,1>> + ksplit_reduce_kernel (fp16 "
                                                 "MFMA 32x32x16 on the exact hi/lo activation split)",
                                          mfma_issued_frac=2.0 * g2["frac"],
                                          note="algorithmic flops 2*M*N*K; the hi/lo split issues twice "
                                               "that on the matrix cores"),
                            runs=g, vendor_fp16_gemm=torch_fp16_gemm_rate())
        if "ceilings" in line:
            rg = line["gemm"]["roofline"]
            rg["mfma_issued_TFLOPs"] = 2.0 * g2["TFLOPs"]
            rg["frac_of_measured_mfma_random"] = 2.0 * g2["TFLOPs"] / line["ceilings"]["mfma_fp16_random_TFLOPs"]
    if not args.no_extras:
        log("extras ...")
        line["extras"] = time_extras()
    if not args.no_cpu:
        log("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
