"""Benchmark of the FP8 attention hot path on one MI355X.

One step = one dynamically scaled FP8 attention call on a batch already resident in HBM:
observe the Q/K/V amax, update the 16-slot ring and the scales, quantise Q/K/V to E4M3
(fp8attn_quantize_dynamic: a quantise pass that observes the amax while it quantises with
the ring's other 15 slots, the scales kernel, and a re-quantise pass that exits at once
unless the window maximum moved), then the FP8 flash-attention kernel (fp8attn_attend).
The same kernels with the amax read as a pass of its own (observe, scales, plain quantise)
are timed afterwards for reference, then the BF16 skip-path kernel on the same batch
(same-hardware baseline). Workload: the kernel point (one sequence of 8192 tokens, 16
heads, head_dim 128, bf16 N(0,1) with x20 outlier columns).

Prints ONE JSON line. value = attention FLOPs of the step (4 * S^2 * d * H) / step time,
in TFLOP/s, the step time being the wall time of K back-to-back steps between two device
synchronisations. The timed steps replay a HIP graph of one step (its four kernel launches
captured once), so that the Python side of the launches, which on a slow host can take
longer than the kernels, stays out of the figure; the same K steps launched one by one from
Python are reported beside it (ms_per_step_eager_launches). Before them, an untimed warm-up of at least W steps and at least
--settle-ms of continuous work: after an idle stretch the GPU's clock ramps up over the
first tens of milliseconds of work (at the kernel point a step averages about 450 us over
its first 20 runs and settles near 325 us after about 50 ms), and the benchmark reports the
sustained rate. Kernel durations come from HIP events recorded on the stream the kernels
run on (torch's current stream), in loops of their own after the timed steps: around each
launch of K more steps (mean and median), and, for the two attention kernels, around
back-to-back bursts of K launches (the roofline figure and the FP8/BF16 ratio use those).

The HBM-bound passes are also measured where their inputs cannot sit in the 256 MB
Infinity Cache: on the same batch with a 512 MB read-only sweep (the benchmark's own stream
kernel, csrc/stream_probe.hip) immediately before every timed launch, each pass in a loop of
its own; and on the 3-image 4K batch (3 x 32400 tokens, 16 heads, 1.2 GB of bf16 input),
beside the same stream kernels' read-only, copy and 2:1 read:write rates over the same
sizes (the practical HBM ceiling). The oracle is timed on the host cores over the whole
forward of the benchmark batch (cpu_baseline).

--gpus N > 1 is refused: the benchmark runs on one GPU.
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

FP8_PEAK_TFLOPS = 5000.0      # MI355X dense FP8 MFMA (published)
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense BF16 MFMA (published)
HBM_PEAK_GBS = 8000.0         # MI355X HBM3E (published)
METRIC = "FP8 attn TFLOP/s & % FP8-MFMA peak at S=8192 d=128; quant GB/s"
PMC_FILE = os.path.join(ROOT, "profiles", "attn_fp8_kernel_point_pmc.json")
ATTN_SRC = os.path.join(ROOT, "fp8_dynamic_scaled_amd", "csrc", "attn_fp8.hip")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--settle-ms", type=float, default=200.0,
                    help="the untimed warm-up also lasts at least this long (ms of "
                         "continuous work), past the GPU clock's ramp after idle")
    ap.add_argument("--workload", default="kernel")
    ap.add_argument("--no-cpu-baseline", action="store_true",
                    help="skip the oracle timing on the host cores")
    ap.add_argument("--no-cold-quant", action="store_true",
                    help="skip the quantisation measurements beyond the Infinity Cache")
    ap.add_argument("--no-regime", action="store_true",
                    help="skip the image-resolution sweep and the DiT-forward comparison")
    ap.add_argument("--regime-case", default=None,
                    help="run only the resolution case of this name (for profiling) and print "
                         "its row")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the benchmark, run one plain device copy of this many MiB "
                         "(reference for HBM byte counters)")
    return ap.parse_args()


def source_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def _oracle_head_task(args):
    """One (sequence, head) of the oracle's FP8 attention, single-threaded (pool worker)."""
    q8, k8, v8, scales, sm = args
    from threadpoolctl import threadpool_limits
    import oracle
    with threadpool_limits(1):
        oracle.fp8_attention_head(q8, k8, v8, scales[0], scales[1], scales[2], sm)
    return q8.shape[0]


def cpu_baseline(w, q, k, v, cu):
    """Time the oracle (as it stands) on the host cores: amax, scales and quantisation of all
    of Q, K and V, then the FP8 attention of every query row of every (sequence, head), one
    (sequence, head) per task in a process pool of one single-threaded worker per available
    core (at most 16, the host share of one GPU)."""
    import multiprocessing as mp
    import oracle
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from parity_util import bits
    affinity = len(os.sched_getaffinity(0))
    workers = max(1, min(affinity, 16))
    host = [bits(t) for t in (q, k, v)]
    t0 = time.perf_counter()
    amax = [oracle.amax_bf16(b) for b in host]
    sc = [oracle.scale_pair(a) for a in oracle.AmaxRing().update(amax)]
    codes = [oracle.quantize_bf16(b, s[1]) for b, s in zip(host, sc)]
    t_quant = time.perf_counter() - t0
    sm = float(np.float32(1.0 / math.sqrt(w.head_dim)))
    tasks = []
    for i in range(w.num_seqs):
        lo, hi = w.cu_seqlens[i], w.cu_seqlens[i + 1]
        for h in range(w.num_heads):
            tasks.append((codes[0][lo:hi, h].copy(), codes[1][lo:hi, h].copy(),
                          codes[2][lo:hi, h].copy(), [x[0] for x in sc], sm))
    t1 = time.perf_counter()
    # fresh worker processes (spawned, not forked from this GPU-holding process): they import
    # only numpy and the oracle
    with mp.get_context("spawn").Pool(workers) as pool:
        rows = sum(pool.map(_oracle_head_task, tasks, chunksize=1))
    t_attn = time.perf_counter() - t1
    t_all = t_quant + t_attn
    return {"value": w.flops() / t_all / 1e12, "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": (f"{w.name}: the whole forward, no extrapolation -- amax + scales + "
                       f"quantisation of all of Q/K/V ({t_quant:.1f} s, one process) and the "
                       f"FP8 attention of all {rows} (row, head) pairs over all of their keys "
                       f"({t_attn:.1f} s: {len(tasks)} (sequence, head) tasks on {workers} "
                       f"single-threaded worker processes); value = workload FLOPs / "
                       f"{t_all:.1f} s"),
            "affinity_cpus": affinity, "seconds_measured": round(t_all, 2)}


STREAM_LIB = os.path.join(ROOT, "fp8_dynamic_scaled_amd", "lib", "libfp8attn_stream.so")


class StreamProbe:
    """The benchmark's own HBM stream kernels (csrc/stream_probe.hip)."""

    def __init__(self, dev):
        import ctypes
        import torch
        if not os.path.exists(STREAM_LIB):
            raise RuntimeError(f"{STREAM_LIB} missing: build with python -m fp8_dynamic_scaled_amd.build")
        self.lib = ctypes.CDLL(STREAM_LIB)
        self.lib.stream_probe.restype = ctypes.c_int
        self.lib.stream_probe.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
        self.ctypes = ctypes
        self.torch = torch
        self.sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)

    def run(self, src, dst, rd, wr, unroll=2, blocks=0):
        """rd (wr) 16-byte reads (writes) per unit over all of src; returns bytes moved."""
        units = src.numel() * src.element_size() // (16 * rd)
        c = self.ctypes
        rc = self.lib.stream_probe(c.c_void_p(src.data_ptr()),
                                   c.c_void_p(0 if dst is None else dst.data_ptr()), units,
                                   rd, wr, unroll, blocks, c.c_void_p(self.sink.data_ptr()),
                                   c.c_void_p(self.torch.cuda.current_stream().cuda_stream))
        if rc != 0:
            raise RuntimeError(f"stream_probe failed: {rc}")
        return units * 16 * (rd + wr)

    def best(self, src, dst, rd, wr, reps=10):
        """The best rate (GB/s) over a small sweep of launch shapes (loads in flight per
        thread x blocks), each timed over `reps` back-to-back launches; and that shape."""
        torch = self.torch
        out = (0.0, None)
        for unroll in (2, 4):
            for blocks in (256, 512, 1024, 2048):
                nb = self.run(src, dst, rd, wr, unroll, blocks)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(reps):
                    self.run(src, dst, rd, wr, unroll, blocks)
                e1.record()
                torch.cuda.synchronize()
                gbs = nb / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
                if gbs > out[0]:
                    out = (gbs, {"loads_in_flight_per_thread": unroll, "blocks": blocks})
        return out


def cold_quant(fa, w, q, k, v, cu_d, cu, st, ws, dev, reps=10):
    """The HBM-bound passes where their inputs are not cache-resident.

    (1) The benchmark batch (101 MB of bf16, which the 256 MB Infinity Cache would otherwise
    hold): before every timed launch a 512 MB read-only sweep by the benchmark's own stream
    kernel evicts it (reads leave no dirty lines to write back); each pass is timed in its own
    loop, so that no other pass re-reads the inputs in between.
    (2) The 3-image 4K batch (1.19 GB of bf16 per forward, beyond the cache), back to back.
    (3) The benchmark's own stream kernels on the 4K batch's sizes: read-only, copy, and two
    bytes read per byte written (the quantise pass's pattern): the practical HBM ceiling.
    """
    import torch
    from workloads import WORKLOADS, make_qkv
    sp = StreamProbe(dev)
    out = {}
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush.fill_(1)
    n = w.elements()

    def timed_cold(fn):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps + 2)]
        for e0, e1 in ev:
            sp.run(flush, None, 1, 0)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        return sum(e0.elapsed_time(e1) for e0, e1 in ev[2:]) / reps

    # a dynamic state whose window maximum is steady for these inputs
    for _ in range(3):
        fa.quantize_dynamic(st, q, k, v, cu_d, cu, workspace=ws)
    t_amax = timed_cold(lambda: fa.observe_amax(st, q, k, v))
    fa.scales(st, "dynamic")       # takes the observations and clears them
    t_quant = timed_cold(lambda: fa.quantize(st, q, k, v, cu_d, cu, workspace=ws))
    t_dyn = timed_cold(lambda: fa.quantize_dynamic(st, q, k, v, cu_d, cu, workspace=ws))
    out[w.name + "_cold"] = {
        "amax_ms": round(t_amax, 5), "amax_gbs": round(3 * n * 2 / (t_amax * 1e-3) / 1e9, 1),
        "quantize_ms": round(t_quant, 5),
        "quant_gbs": round(3 * n * 3 / (t_quant * 1e-3) / 1e9, 1),
        "one_pass_dynamic_ms": round(t_dyn, 5),
        "one_pass_dynamic_gbs": round(3 * n * 3 / (t_dyn * 1e-3) / 1e9, 1),
        "note": "each pass in its own loop, a 512 MB read-only sweep (own stream kernel) "
                "before every timed launch; bytes: amax 2 B, quantise and the one-pass "
                "dynamic path 3 B per element of Q, K, V (window maximum steady)"}
    del flush
    w4 = WORKLOADS["4k"]
    q4, k4, v4 = make_qkv(w4, 0, dev)
    cu4 = np.asarray(w4.cu_seqlens, dtype=np.int32)
    cu4_d = torch.tensor(cu4, dtype=torch.int32, device=dev)
    st4 = fa.new_state(dev)
    ws4 = torch.empty(fa.workspace_bytes(w4.total_tokens, w4.num_seqs, w4.num_heads,
                                         w4.head_dim), dtype=torch.uint8, device=dev)
    n4 = w4.elements()
    for _ in range(3):
        fa.quantize_dynamic(st4, q4, k4, v4, cu4_d, cu4, workspace=ws4)

    def timed(fn, r=reps):
        fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(r):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / r

    am = timed(lambda: fa.observe_amax(st4, q4, k4, v4))
    fa.scales(st4, "dynamic")
    qm = timed(lambda: fa.quantize(st4, q4, k4, v4, cu4_d, cu4, workspace=ws4))
    om = timed(lambda: fa.quantize_dynamic(st4, q4, k4, v4, cu4_d, cu4, workspace=ws4))
    # own stream kernels over the same sizes: a 1.19 GB source (Q, K, V in bf16) and a
    # 0.6 GB destination (their E4M3 bytes)
    src = torch.empty(3 * n4 * 2, dtype=torch.uint8, device=dev)
    src.fill_(3)
    dst = torch.empty(3 * n4, dtype=torch.uint8, device=dev)
    half = src[:3 * n4]
    rd_gbs, rd_cfg = sp.best(src, None, 1, 0)
    cp_gbs, cp_cfg = sp.best(half, dst, 1, 1)
    s21_gbs, s21_cfg = sp.best(src, dst, 2, 1)
    q_gbs = 3 * n4 * 3 / (qm * 1e-3) / 1e9
    a_gbs = 3 * n4 * 2 / (am * 1e-3) / 1e9
    out["4k"] = {
        "elements_per_tensor": n4,
        "amax_ms": round(am, 5), "amax_gbs": round(a_gbs, 1),
        "quantize_ms": round(qm, 5), "quant_gbs": round(q_gbs, 1),
        "quant_frac_hbm_peak": round(q_gbs / HBM_PEAK_GBS, 4),
        "one_pass_dynamic_ms": round(om, 5),
        "one_pass_dynamic_gbs": round(3 * n4 * 3 / (om * 1e-3) / 1e9, 1),
        "stream_read_gbs": round(rd_gbs, 1), "stream_copy_gbs": round(cp_gbs, 1),
        "stream_2to1_gbs": round(s21_gbs, 1),
        "stream_launch_shapes": {"read": rd_cfg, "copy": cp_cfg, "2to1": s21_cfg},
        "quant_frac_of_stream_2to1": round(q_gbs / s21_gbs, 3),
        "amax_frac_of_stream_read": round(a_gbs / rd_gbs, 3),
        "note": "3 x 32400 tokens, 16 heads: 1.19 GB bf16 in, 0.6 GB E4M3 out per quantise; "
                "stream_*: the benchmark's own kernels over the same sizes (read-only 1.19 GB; "
                "copy 0.6 GB to 0.6 GB; 2:1 = 1.19 GB read and 0.6 GB written, the quantise "
                "pass's ratio), back to back, the best of 2 x 4 launch shapes"}
    del q4, k4, v4, ws4, src, dst
    torch.cuda.empty_cache()
    return out


# The end-to-end encoder table of the pages' FP8 ViT attention section ("Performance"):
# 3 images per request at HD, FullHD, QHD and 4K. Patches of 16 pixels; the FullHD height
# is taken as 1088 (68 patch rows), the next multiple of 32, so every image splits into
# whole 2x2-merged patch groups. A 448x448 image (28x28 patches) is added below them, and
# two batches of many small images.
RESOLUTIONS = (("448x448", 28, 28, 3), ("HD 720x1280", 45, 80, 3),
               ("FullHD 1080x1920", 68, 120, 3), ("QHD 1440x2560", 90, 160, 3),
               ("4K 2160x3840", 135, 240, 3),
               # many small images in one batch: the short-sequence regime
               ("448x448 x64", 28, 28, 64), ("256x256 x256", 16, 16, 256))


def settle(fns, min_rounds, ms):
    """Untimed warm-up: rounds of `fns` until at least `min_rounds` rounds have run and at
    least `ms` milliseconds of wall time have passed with the GPU kept busy (the host waits
    for the device every ~5 ms of work, so it never runs far ahead of it)."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for f in fns:
        f()
    torch.cuda.synchronize()
    est = max(time.perf_counter() - t0, 1e-6)
    chunk = max(1, int(5e-3 / est))
    rounds = 1
    while rounds < min_rounds or (time.perf_counter() - t0) * 1e3 < ms:
        for _ in range(chunk):
            for f in fns:
                f()
        rounds += chunk
        torch.cuda.synchronize()
    return rounds


def _burst_ms(fn, n):
    """ms per call of `fn` over n back-to-back calls between one HIP event pair."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def _median_burst_ms(fn, burst_ms=25.0, bursts=3):
    """Median over `bursts` bursts of back-to-back calls, each about `burst_ms` long (at
    least 5 calls)."""
    est = _burst_ms(fn, 2)
    n = max(5, min(2000, math.ceil(burst_ms / max(est, 1e-3))))
    t = sorted(_burst_ms(fn, n) for _ in range(bursts))
    return t[len(t) // 2]


def regime(fa, dev, settle_ms=60.0, only=None):
    """FP8 dynamic step (one-pass quantise + FP8 attention) against the BF16 kernel on
    3-image batches per resolution (16 heads, bf16 N(0,1) with x20 outlier columns), and on
    one forward of the DiT video workload (57600 tokens, 40 heads)."""
    import torch
    from workloads import WORKLOADS, Workload, make_qkv
    rows = {}
    cases = [(name, Workload(name, 6, tuple(i * ph * pw for i in range(n + 1)), 16,
                             outliers=True))
             for name, ph, pw, n in RESOLUTIONS]
    # one 4K image and twenty 448x448 images in one request: very unequal sequences
    mixed = [0, 135 * 240]
    for _ in range(20):
        mixed.append(mixed[-1] + 28 * 28)
    cases.append(("4K 2160x3840 + 20 x 448x448", Workload("mixed", 6, tuple(mixed), 16,
                                                           outliers=True)))
    cases.append(("DiT forward 57600 tokens, H=40", WORKLOADS["dit"]))
    # one GPU's share of that forward under head (Ulysses) sharding of degree 4
    cases.append(("DiT forward, one of 4 head shards (H=10)",
                  Workload("dit-shard", 5, (0, 57600), 10, outliers=True)))
    if only is not None:
        cases = [c for c in cases if c[0] == only]
        if not cases:
            raise SystemExit(f"no resolution case named {only!r}")
    for name, w in cases:
        q, k, v = make_qkv(w, 0, dev)
        cu = np.asarray(w.cu_seqlens, dtype=np.int32)
        cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
        H = w.num_heads
        st = fa.new_state(dev)
        ws = torch.empty(fa.workspace_bytes(w.total_tokens, w.num_seqs, H, w.head_dim),
                         dtype=torch.uint8, device=dev)
        out = torch.empty_like(q)

        def quant():
            fa.quantize_dynamic(st, q, k, v, cu_d, cu, workspace=ws)

        def attn():
            fa.attend(st, ws, cu_d, cu, H, out=out)

        def fp8_step():
            quant()
            attn()

        def bf16():
            fa.forward(None, q, k, v, cu_d, cu, skip=True, out=out)

        settle([fp8_step, bf16], 3, settle_ms)
        t_step, t_q, t_a, t_b = (_median_burst_ms(f) for f in (fp8_step, quant, attn, bf16))
        rows[name] = {"tokens_per_image": w.seq_lens[0], "images": w.num_seqs, "heads": H,
                      "tokens_total": w.total_tokens,
                      "fp8_step_ms": round(t_step, 4), "quantize_dynamic_ms": round(t_q, 4),
                      "attn_fp8_ms": round(t_a, 4), "attn_bf16_ms": round(t_b, 4),
                      "fp8_step_speedup": round(t_b / t_step, 3),
                      "attn_only_speedup": round(t_b / t_a, 3),
                      "attn_fp8_tflops": round(w.flops() / (t_a * 1e-3) / 1e12, 1)}
        del q, k, v, ws, out
        torch.cuda.empty_cache()
    return rows


def dit_schedule_time(fa, dev):
    """The DiT workload's whole schedule: 4 denoising steps x 8 layers of one 57 600-token,
    40-head full-attention forward, the step and layer skip selectors (steps 0,1 and layers
    0-2, vLLM-Omni "Quantized KV Cache", "Parameters") routing 22 of the 32 forwards to the
    BF16 kernel and the rest through each layer's dynamic FP8 path; against all 32 in BF16.
    One set of inputs serves every forward (the times do not depend on the values)."""
    import torch
    from workloads import WORKLOADS, dit_schedule, make_qkv
    w = WORKLOADS["dit"]
    q, k, v = make_qkv(w, 0, dev)
    cu = np.asarray(w.cu_seqlens, dtype=np.int32)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    out = torch.empty_like(q)
    layers = [fa.AttentionLayer(dev) for _ in range(w.layers)]
    sched = dit_schedule(w, fa.parse_selector(w.skip_steps), fa.parse_selector(w.skip_layers))

    def run(all_bf16):
        for (_, _, layer, skip) in sched:
            layers[layer](q, k, v, cu_d, cu, skip=skip or all_bf16, out=out)

    settle([lambda: run(False)], 1, 0.0)
    t_mixed = _burst_ms(lambda: run(False), 1)
    t_bf16 = _burst_ms(lambda: run(True), 1)
    n_bf16 = sum(1 for x in sched if x[3])
    res = {"forwards": len(sched), "bf16_forwards": n_bf16, "fp8_forwards": len(sched) - n_bf16,
           "schedule_ms": round(t_mixed, 2), "all_bf16_ms": round(t_bf16, 2),
           "speedup": round(t_bf16 / t_mixed, 3)}
    del q, k, v, out, layers
    torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus_requested": args.gpus}))
        sys.exit(2)

    import torch
    import fp8_dynamic_scaled_amd as fa
    from workloads import WORKLOADS, make_qkv

    if args.regime_case is not None:
        dev = torch.device("cuda", 0)
        torch.cuda.set_device(dev)
        print(json.dumps({"resolution_case": regime(fa, dev, args.settle_ms, args.regime_case)}))
        return

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    q, k, v = make_qkv(w, 0, dev)
    cu = np.asarray(w.cu_seqlens, dtype=np.int32)
    cu_d = torch.tensor(cu, dtype=torch.int32, device=dev)
    B, H, D, T = w.num_seqs, w.num_heads, w.head_dim, w.total_tokens
    st = fa.new_state(dev)
    ws = torch.empty(fa.workspace_bytes(T, B, H, D), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)
    n = w.elements()
    flops = w.flops()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fa.quantize_dynamic(st, q, k, v, cu_d, cu, workspace=ws)
        if ev is not None:
            ev[1].record()
        fa.attend(st, ws, cu_d, cu, H, out=out)
        if ev is not None:
            ev[2].record()

    def separate(ev):
        ev[0].record()
        fa.observe_amax(st, q, k, v)
        ev[1].record()
        fa.scales(st, "dynamic")
        ev[2].record()
        fa.quantize(st, q, k, v, cu_d, cu, workspace=ws)
        ev[3].record()

    warm_rounds = settle([step], args.warmup, args.settle_ms)
    # the same steps launched one by one from Python, for reference: on a slow host the
    # Python side of two binding calls and four launches can take longer than the kernels
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms_step_eager = (time.perf_counter() - t0) * 1e3 / args.steps

    # the timed steps: one step captured in a HIP graph (observe-quantise, scales,
    # re-quantise check, attention; no allocation, copy or memset inside) and replayed K
    # times, so the launches come from the graph and the host's speed stays out of the step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    settle([graph.replay], 1, 50.0)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        graph.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # per-kernel durations: K more steps with events around each launch (not timed above)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    names = ("quantize_dynamic", "attn_fp8")
    samples = {k2: [e[i].elapsed_time(e[i + 1]) for e in evs] for i, k2 in enumerate(names)}

    # reference: the same step with the amax read as a pass of its own
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    for i in range(args.steps):
        separate(sev[i])
        fa.attend(st, ws, cu_d, cu, H, out=out)
    torch.cuda.synchronize()
    for i, k2 in enumerate(("amax", "scales", "quantize")):
        samples[k2] = [e[i].elapsed_time(e[i + 1]) for e in sev]
    per = {k2: sum(v2) / len(v2) for k2, v2 in samples.items()}            # ms per launch (mean)
    per_median = {k2: sorted(v2)[len(v2) // 2] for k2, v2 in samples.items()}

    # both attention kernels as back-to-back bursts between one event pair, so that the
    # per-launch event packets and dispatch fences of the step loop do not enter the
    # kernel time (the roofline and the FP8/BF16 ratio use these)
    fa.quantize_dynamic(st, q, k, v, cu_d, cu, workspace=ws)
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    b0.record()
    for _ in range(args.steps):
        fa.attend(st, ws, cu_d, cu, H, out=out)
    b1.record()
    torch.cuda.synchronize()
    ms_fp8_burst = b0.elapsed_time(b1) / args.steps

    # BF16 skip-path kernel on the same batch, after a warm-up of its own
    settle([lambda: fa.forward(None, q, k, v, cu_d, cu, skip=True, out=out)], args.warmup,
           args.settle_ms)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(args.steps):
        fa.forward(None, q, k, v, cu_d, cu, skip=True, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms_bf16 = e0.elapsed_time(e1) / args.steps

    cold = None if args.no_cold_quant else cold_quant(fa, w, q, k, v, cu_d, cu, st, ws, dev)

    attn_tflops = flops / (ms_fp8_burst * 1e-3) / 1e12
    quant_gbs = (3 * n * 3) / (per["quantize"] * 1e-3) / 1e9
    dyn_gbs = (3 * n * 3) / (per["quantize_dynamic"] * 1e-3) / 1e9
    amax_gbs = (3 * n * 2) / (per["amax"] * 1e-3) / 1e9
    bf16_tflops = flops / (ms_bf16 * 1e-3) / 1e12

    traffic = None
    if os.path.exists(PMC_FILE):
        with open(PMC_FILE) as f:
            pmc = json.load(f)
        if pmc.get("kernel_source_sha256") == source_sha(ATTN_SRC) and pmc.get("workload") == w.name:
            traffic = pmc.get("hbm_bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "warmup_steps_run": warm_rounds,
        "settle_ms": args.settle_ms,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_eager_launches": round(ms_step_eager, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 (fp32 accumulate)",
        "data": f"synthetic (seeded bf16; {w.description.split(';')[0].split(', ', 2)[-1]})",
        "config": {"workload": f"{w.name}: {w.description}", "num_seqs": B, "seq_len": w.seq_lens[0],
                   "num_heads": H, "head_dim": D, "causal": False, "scaling": "dynamic 16-slot ring",
                   "launch": "one step captured in a HIP graph, replayed per timed step"},
        "roofline": {"bound": "mfma", "kernel": "attn_fp8_kernel",
                     "achieved": round(attn_tflops, 2), "peak": FP8_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
                     "traffic": traffic,
                     "algorithmic_per_launch": f"{flops:.4e} FLOP (4*S^2*d*H)"},
        "kernels_ms": {k2: round(v2, 5) for k2, v2 in per.items()},
        "kernels_ms_median": {k2: round(v2, 5) for k2, v2 in per_median.items()},
        "attn_fp8_tflops": round(attn_tflops, 2),
        "attn_fp8_frac_fp8_peak": round(attn_tflops / FP8_PEAK_TFLOPS, 4),
        "attn_bf16_ms": round(ms_bf16, 5),
        "attn_bf16_tflops": round(bf16_tflops, 2),
        "attn_bf16_frac_bf16_peak": round(bf16_tflops / BF16_PEAK_TFLOPS, 4),
        "attn_fp8_ms": round(ms_fp8_burst, 5),
        "fp8_over_bf16_speedup": round(ms_bf16 / ms_fp8_burst, 3),
        "kernel_times_note": "attn_fp8_ms and attn_bf16_ms: K back-to-back launches between "
                             "one HIP event pair (the roofline uses attn_fp8_ms); kernels_ms: "
                             "HIP events around each launch of K further steps, which add the "
                             "event packets and dispatch fences of each launch; all after the "
                             "warm-up",
        "quant_gbs": round(quant_gbs, 1),
        "dynamic_quant_gbs": round(dyn_gbs, 1),
        "dynamic_quant_note": "fp8attn_quantize_dynamic (quantise + observe, scales, "
                              "re-quantise check): 3 B per element of Q, K, V over its time",
        "quant_frac_hbm_peak": round(quant_gbs / HBM_PEAK_GBS, 4),
        "amax_gbs": round(amax_gbs, 1),
        "amax_frac_hbm_peak": round(amax_gbs / HBM_PEAK_GBS, 4),
        "quant_algorithmic_bytes": f"{3 * n * 3:.4e} (2 B read + 1 B write per element, 3 tensors)",
        "amax_algorithmic_bytes": f"{3 * n * 2:.4e} (2 B read per element, 3 tensors)",
    }
    if cold is not None:
        result["quant_beyond_infinity_cache"] = cold
    if not args.no_regime:
        result["resolution_sweep"] = regime(fa, dev)
        result["resolution_sweep_note"] = (
            "per case: 60 ms of alternating FP8 steps and BF16 calls as warm-up, then for "
            "each figure the median of 3 bursts of back-to-back calls of about 25 ms; fp8_step = fp8attn_quantize_dynamic + fp8attn_attend (dynamic "
            "scaling, window maximum steady), attn_bf16 = the skip-path kernel; 3 images "
            "per request unless the name says x N, 16-pixel patches, H=16 (DiT: one "
            "forward, H=40)")
        result["dit_schedule"] = dit_schedule_time(fa, dev)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, cu)
    if args.copy_calibration_mib > 0:
        # one launch of the benchmark's own copy kernel over a known number of bytes: the
        # reference for scaling the HBM byte counters of a profiled run
        nb = args.copy_calibration_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        StreamProbe(dev).run(src, dst, 1, 1)
        torch.cuda.synchronize()
        result["copy_calibration_bytes"] = nb
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
