#!/usr/bin/env python3
"""Benchmark of the AWQ W4A16 hot path on one MI355X.

One step = one pass of the whole hot path over one Llama-2-7B decoder layer's linears
(seeded synthetic fp16 weights ~ N(0, 0.02^2), activations ~ N(0, 1) with 1% of the
channels x20, group 128, 4-bit + zero point):
  1. scale search (statistic, 20-point alpha grid, error, argmin) for the four
     shared-input groups q|k|v [12288x4096], o [4096x4096], gate|up [22016x4096],
     down [4096x11008], calibration X = 512 tokens;
  2. quantize + pack of the four groups with their chosen scales (the seven matrices);
  3. decode GEMV at M = 1 over 32 layer copies (one token through the 32 decoder layers
     of a 7B model: 3.37 GB of packed weights, far above the 256 MB last-level cache, so
     every launch streams from HBM), with q|k|v and gate|up launched as one GEMV each
     (they share their input; the fused-module decode of the pages), gate|up with its
     SiLU(gate) * up epilogue (the fused MLP module); the same sweep with one launch
     per matrix (no epilogue) is timed and reported beside it;
  4. prefill MFMA dequant-GEMM at M = 2048 over the four groups (gate|up fused as in 3);
  5. weight clipping after the scale search: 20 shrink ratios per group (r = 1 .. 0.905
     on the clip_steps = 200 grid) of each group's W diag(s);
  6. the equivalent transform's other half: each group's 1/s folded into the producer
     of its input (norm weights for q|k|v and gate|up, v_proj rows for o, up_proj rows
     for down).
Inputs are resident in HBM before the timed region. Each part is captured once in a
HIP graph (so host launch overhead is not kernel time) and replayed. The K timed steps
run in phases, part by part (K decode sweeps back to back, then K prefill GEMMs, and so
on), so each part is measured in the steady state it has in service; HIP events on the
launch stream bracket each phase. The headline value is the GEMV bandwidth; the GEMM
rate is reported beside it.

Beside the step, the same run measures and reports:
  * the chip's peaks, measured in this process: a read stream at the fused decode
    launch's size, at 1 GiB and at 8 GiB, and an fp16 MFMA loop; every roofline fraction
    is given against the published peak (`frac`) and the measured one;
  * per-replay distributions (median, p10, p90 over --reps replays) of every part, and
    the GPU clocks before and after;
  * the single-linear workload (K = N = 1024: search with T = 256, pack, M = 1 and 16);
  * the Llama-2-70B decode sweep: 80 layers' packed weights resident (35.6 GB), M = 1
    and M = 32;
  * the single-layer "hot" decode (105 MB, resident in the last-level cache; labelled);
  * the crossover table, the format variants, and the CPU oracle on the host cores
    (one thread and all threads) on bounded samples.

Prints ONE JSON line. `python bench.py --gpus N` with N > 1 exits: this build runs
on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
CALIB_T = 512
PREFILL_M = 2048
DECODE_LAYERS = 32
LAYERS_70B = 80
GROUP = 128

MATRICES = [  # name, search group, row offset inside the group, N, K
    ("q_proj", "qkv", 0, 4096, 4096), ("k_proj", "qkv", 4096, 4096, 4096),
    ("v_proj", "qkv", 8192, 4096, 4096), ("o_proj", "o", 0, 4096, 4096),
    ("gate_proj", "gate_up", 0, 11008, 4096), ("up_proj", "gate_up", 11008, 11008, 4096),
    ("down_proj", "down", 0, 4096, 11008),
]
SEARCH_GROUPS = {"qkv": (12288, 4096), "o": (4096, 4096), "gate_up": (22016, 4096), "down": (4096, 11008)}
# Llama-2-70B decoder layer as launched in decode: q|k|v (GQA, 8 kv heads), o, gate|up
# (fused, SiLU epilogue), down
GROUPS_70B = {"qkv": (10240, 8192), "o": (8192, 8192), "gate_up": (57344, 8192), "down": (8192, 28672)}
GATED = {"gate_up"}  # the fused MLP module: SiLU(gate) * up in the launch's epilogue
GEMM_COPIES = 5      # layer copies the prefill GEMM rotates over (5 x 105 MB)


def packed_bytes(N, K, group=GROUP, w_bit=4):
    """Bytes of one packed [N][K] weight: codes, fp16 scales, zeros (3/4-bit: two per byte)."""
    G = K // group
    return N * K * w_bit // 8 + N * G * 2 + N * (G if w_bit == 8 else (G + 1) // 2)


def linear_bytes(M, N, K, gated=False, group=GROUP, w_bit=4):
    """Algorithmic HBM bytes of one W4A16 linear: the packed weight, X and Y as written
    (a gated launch writes Y of N/2 columns: SiLU(gate) * up)."""
    return packed_bytes(N, K, group, w_bit) + 2 * M * K + 2 * M * (N // 2 if gated else N)


def kernel_source_hash(files=("gemv.hip", "common.hpp")):
    """Hash of the sources of the measured decode kernel (HBM counters are reported only
    while these are unchanged)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_bit_02_amd", "csrc")
    for f in files:
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_bit_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


def pct(v, q):
    s = sorted(v)
    if not s:
        return None
    i = min(len(s) - 1, max(0, int(round(q * (len(s) - 1)))))
    return s[i]


def dist(ms_list):
    """median / p10 / p90 / mean of per-replay times (ms)."""
    return {"median_ms": round(pct(ms_list, 0.5), 5), "p10_ms": round(pct(ms_list, 0.1), 5),
            "p90_ms": round(pct(ms_list, 0.9), 5), "mean_ms": round(sum(ms_list) / len(ms_list), 5),
            "n": len(ms_list)}


def gpu_clocks():
    """Current GPU shader and memory clocks as the driver reports them (rocm-smi), or None."""
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True, text=True,
                           timeout=20)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        return {k: v for k, v in card.items() if "sclk" in k or "mclk" in k or "fclk" in k}
    except Exception as e:  # noqa: BLE001 -- clocks are context only
        return {"error": type(e).__name__}


class Timer:
    """Per-replay HIP event pairs on one stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def replays(self, fn, reps):
        ev = [(self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            a.record(self.stream)
            fn()
            b.record(self.stream)
        ev[-1][1].synchronize()
        return [a.elapsed_time(b) for a, b in ev]

    def block(self, fn, reps):
        a, b = self.torch.cuda.Event(enable_timing=True), self.torch.cuda.Event(enable_timing=True)
        a.record(self.stream)
        for _ in range(reps):
            fn()
        b.record(self.stream)
        b.synchronize()
        return a.elapsed_time(b) / reps


class Rotation:
    """Calls one of several equivalent runners per call, in turn (rotating input copies)."""

    def __init__(self, fns):
        self.fns, self.next, self.last = fns, 0, None

    def __call__(self):
        self.last = self.next
        self.fns[self.next]()
        self.next = (self.next + 1) % len(self.fns)


def capture(torch, stream, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        fn()
    return g


# ---------------------------------------------------------------------------- peaks
def measure_peaks(torch, lib, dev, stream, timer, reps, sizes):
    """Read-stream bandwidth at each size and the fp16 MFMA rate, measured on this machine."""
    import ctypes as C
    out = {"read_stream": {}, "method": "awq_peak_read_stream / awq_peak_mfma (include/awq_peaks.h); "
                                        "median over replays, HIP events"}
    for label, nbytes, copies in sizes:
        # `copies` distinct buffers read one after another inside one graph (their sum far
        # beyond the 256 MB last-level cache), so every launch streams from HBM and the
        # graph launch overhead is shared: per-launch time = replay time / copies
        n = nbytes // 16 * 16
        bufs = [torch.full((n,), 7, dtype=torch.uint8, device=dev) for _ in range(copies)]
        sink = torch.empty(4 * (n // 16384 + 1), dtype=torch.int32, device=dev)
        best = None
        for per_thread in (4, 8, 16):
            def run(u=per_thread):
                for b in bufs:
                    lib.awq_peak_read_stream(C.c_void_p(b.data_ptr()), n, C.c_void_p(sink.data_ptr()),
                                             u, C.c_void_p(stream.cuda_stream))
            with torch.cuda.stream(stream):
                run()
                g = capture(torch, stream, run)
                g.replay()
                t = [x / copies for x in timer.replays(g.replay, max(10, reps // 2))]
            med = pct(t, 0.5)
            if best is None or med < best[0]:
                best = (med, per_thread, t)
        med, per_thread, t = best
        out["read_stream"][label] = {"bytes": n, "gbs": round(n / (med * 1e-3) / 1e9, 1),
                                     "gbs_p10": round(n / (pct(t, 0.9) * 1e-3) / 1e9, 1),
                                     "gbs_p90": round(n / (pct(t, 0.1) * 1e-3) / 1e9, 1),
                                     "median_us": round(med * 1e3, 3), "loads_per_thread": per_thread,
                                     "launches_per_graph": copies}
        del bufs, sink
        torch.cuda.empty_cache()
    fs = torch.empty(4 * 8192, dtype=torch.float32, device=dev)
    iters, blocks = 4096, 2048  # 8 waves per CU
    flops = blocks * 4 * iters * 8 * 2 * 32 * 32 * 16

    def mfma():
        lib.awq_peak_mfma(iters, C.c_void_p(fs.data_ptr()), blocks, C.c_void_p(stream.cuda_stream))
    with torch.cuda.stream(stream):
        mfma()
        g = capture(torch, stream, mfma)
        t = timer.replays(g.replay, max(10, reps // 5))
    out["mfma_f16_tflops"] = round(flops / (pct(t, 0.5) * 1e-3) / 1e12, 1)
    out["mfma_loop"] = {"blocks": blocks, "waves_per_block": 4, "iters": iters,
                        "median_ms": round(pct(t, 0.5), 4)}
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------- crossover
def crossover(awq, packed, dev, stream, ms=(1, 2, 4, 8, 16, 32, 64), reps=20):
    """GEMV vs GEMM time (us) over the four 7B groups per M (one launch per group, events
    around `reps` back-to-back sweeps): the data behind the M <= awq_gemv_max_m dispatch."""
    import torch
    out = {"M": list(ms), "gemv_us": [], "skinny_us": [], "gemm_us": [], "gemv_max_m": awq.gemv_max_m()}
    for M in ms:
        X = {K: torch.randn((M, K), device=dev).half() for K in (4096, 11008)}
        for kern, key in (("gemv", "gemv_us"), ("skinny", "skinny_us"), ("gemm", "gemm_us")):
            if (kern == "gemv" and M > 8) or (kern == "skinny" and M > 64):
                out[key].append(None)
                continue
            with torch.cuda.stream(stream):
                def sweep():
                    for g, p in packed.items():
                        awq.linear_w4a16(X[p.K], p, kernel=kern)
                sweep()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(reps):
                    sweep()
                b.record(stream)
            b.synchronize()
            out[key].append(round(a.elapsed_time(b) * 1e3 / reps, 2))
    return out


# ---------------------------------------------------------------------------- variants
# Format variants measured beside the headline (4-bit, asymmetric, 128-channel groups):
# the same parts on the same inputs with one config field changed each.
VARIANTS = {"group64": {"group_size": 64}, "group32": {"group_size": 32},
            "symmetric": {"zero_point": False}, "int8": {"w_bit": 8}, "int3": {"w_bit": 3}}
VARIANT_LAYERS = 16  # decode layer copies per variant: 1.6-3.3 GB, far beyond the on-chip caches


def time_variants(awq, si, dev, stream, Xcal, Wg, s_best, xdec, xpre, steps, warmup, log):
    """Decode sweep, prefill GEMM, quantize+pack, scale search and clip search per format
    variant, each part captured in a graph and timed like the headline parts (warm-up
    replays, then `steps` replays between two events on the launch stream)."""
    import torch
    out = {}
    for vname, kw in VARIANTS.items():
        group, w_bit = kw.get("group_size", GROUP), kw.get("w_bit", 4)
        log(f"bench: variant {vname}: packing {VARIANT_LAYERS} layer copies")
        packed = []
        with torch.cuda.stream(stream):
            for c in range(VARIANT_LAYERS):
                layer = {}
                for i, (g, (N, K)) in enumerate(SEARCH_GROUPS.items()):
                    w = Wg[g] if c == 0 else si.torch_weights(N, K, 1000 + 7 * c + i, dev)
                    layer[g] = awq.quantize_pack(w, s_best[g] if c == 0 else None,
                                                 out=awq.alloc_packed(N, K, dev, group, w_bit), **kw)
                    del w
                packed.append(layer)
        yfus = {g: torch.empty((1, N // 2 if g in GATED else N), dtype=torch.float16, device=dev)
                for g, (N, K) in SEARCH_GROUPS.items()}
        ypre = {g: torch.empty((PREFILL_M, N // 2 if g in GATED else N), dtype=torch.float16, device=dev)
                for g, (N, K) in SEARCH_GROUPS.items()}
        ws = {g: awq.SearchWorkspace(CALIB_T, N, K, dev) for g, (N, K) in SEARCH_GROUPS.items()}
        sres = {g: awq.search_scales(Xcal[g], Wg[g], workspace=ws[g], **kw) for g in SEARCH_GROUPS}

        def gemv():
            for layer in packed:
                for g, (N, K) in SEARCH_GROUPS.items():
                    linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                    linear(xdec[K], layer[g], out=yfus[g])

        def gemm():
            for g, (N, K) in SEARCH_GROUPS.items():
                linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                linear(xpre[K], packed[0][g], out=ypre[g])

        def pack():
            for g in SEARCH_GROUPS:
                awq.quantize_pack(Wg[g], s_best[g], out=packed[0][g], **kw)

        def search():
            for g in SEARCH_GROUPS:
                awq.search_scales(Xcal[g], Wg[g], workspace=ws[g], out=sres[g], **kw)

        def clip():
            for g in SEARCH_GROUPS:
                awq.clip_search(Xcal[g], Wg[g], s_best[g], 200, 20, **kw)

        parts = {"gemv": gemv, "gemm": gemm, "quant_pack": pack, "search": search, "clip": clip}
        ms = {}
        with torch.cuda.stream(stream):
            for fn in parts.values():
                fn()
            torch.cuda.synchronize()
            y_eager = {g: yfus[g].clone() for g in yfus}
            for pname, fn in parts.items():
                graph = capture(torch, stream, fn)
                for _ in range(warmup):
                    graph.replay()
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                a.record(stream)
                for _ in range(steps):
                    graph.replay()
                b.record(stream)
                b.synchronize()
                ms[pname] = a.elapsed_time(b) / steps
                del graph
            for g in yfus:
                assert torch.equal(yfus[g], y_eager[g]), f"graph replay differs ({vname} gemv)"

        dec_bytes = VARIANT_LAYERS * sum(linear_bytes(1, N, K, g in GATED, group, w_bit)
                                         for g, (N, K) in SEARCH_GROUPS.items())
        dec_gbs = dec_bytes / (ms["gemv"] * 1e-3) / 1e9
        gemm_tf = sum(2 * PREFILL_M * N * K for N, K in SEARCH_GROUPS.values()) / (ms["gemm"] * 1e-3) / 1e12
        pack_gbs = sum(N * K * 2 + packed_bytes(N, K, group, w_bit)
                       for N, K in SEARCH_GROUPS.values()) / (ms["quant_pack"] * 1e-3) / 1e9
        search_tf = sum(2 * CALIB_T * N * K * 20 for N, K in SEARCH_GROUPS.values()) / (ms["search"] * 1e-3) / 1e12
        clip_tf = sum(2 * CALIB_T * N * K * 20 for N, K in SEARCH_GROUPS.values()) / (ms["clip"] * 1e-3) / 1e12
        out[vname] = {
            "config": {"group_size": group, "w_bit": w_bit, "zero_point": kw.get("zero_point", True)},
            "decode": {"gbs": round(dec_gbs, 2), "ms": round(ms["gemv"], 4),
                       "frac": round(dec_gbs / HBM_PEAK_GBS, 4), "layers": VARIANT_LAYERS,
                       "launches": VARIANT_LAYERS * len(SEARCH_GROUPS)},
            "gemm": {"tflops": round(gemm_tf, 2), "ms": round(ms["gemm"], 4),
                     "frac": round(gemm_tf / FP16_MFMA_PEAK_TFLOPS, 4)},
            "quant_pack": {"gbs": round(pack_gbs, 2), "ms": round(ms["quant_pack"], 4),
                           "frac": round(pack_gbs / HBM_PEAK_GBS, 4)},
            "search": {"tflops_algorithmic": round(search_tf, 2), "ms": round(ms["search"], 4),
                       "best_alpha_index": {g: int(sres[g].best_idx.item()) for g in SEARCH_GROUPS}},
            "clip_search": {"tflops_algorithmic": round(clip_tf, 2), "ms": round(ms["clip"], 4)},
        }
        log(f"bench: variant {vname}: decode {dec_gbs:.0f} GB/s, gemm {gemm_tf:.0f} TF, "
            f"search {ms['search']:.2f} ms, clip {ms['clip']:.2f} ms")
        del packed, yfus, ypre, ws, sres
        torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------- dense reference
def dense_reference(torch, dev, stream, timer, reps):
    """torch's dense fp16 GEMM (the vendor library, no weight widening) on the four 7B GEMM
    shapes at M = 2048: a measured practical ceiling for the W4A16 GEMM, same box, same run."""
    out = {"library": "torch.mm fp16 (hipBLASLt / rocBLAS), operands contiguous, fp16 output", "shapes": {}}
    tot_ms = tot_fl = 0.0
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    for name, (N, K) in SEARCH_GROUPS.items():
        a = torch.randn((PREFILL_M, K), generator=g, device=dev).half()
        b = torch.randn((K, N), generator=g, device=dev).half()  # W^T, contiguous
        c = torch.empty((PREFILL_M, N), dtype=torch.float16, device=dev)

        def mm(a=a, b=b, c=c):
            torch.mm(a, b, out=c)
        with torch.cuda.stream(stream):
            mm()
            torch.cuda.synchronize()
            gr = capture(torch, stream, mm)
            gr.replay()
            t = pct(timer.replays(gr.replay, reps), 0.5)
        fl = 2 * PREFILL_M * N * K
        out["shapes"][name] = {"N": N, "K": K, "ms": round(t, 4), "tflops": round(fl / (t * 1e-3) / 1e12, 1)}
        tot_ms += t
        tot_fl += fl
        del a, b, c, gr
    out["tflops"] = round(tot_fl / (tot_ms * 1e-3) / 1e12, 1)
    out["ms"] = round(tot_ms, 4)
    torch.cuda.synchronize()
    return out


# ---------------------------------------------------------------------------- single linear
def single_linear(awq, si, dev, stream, timer, reps):
    """The single-linear workload: K = N = 1024, W ~ N(0, 0.02^2), calibration X of 256
    tokens with 10 outlier channels x20; the 20-point search, the pack with the chosen
    scale, and the linear at M = 1 and M = 16."""
    import torch
    N = K = 1024
    W = si.torch_weights(N, K, 7000, dev)
    Xc = si.torch_activations(256, K, 7001, dev, channel_offset=K)
    xs = {M: si.torch_activations(M, K, 7002 + M, dev, channel_offset=K) for M in (1, 16)}
    ws = awq.SearchWorkspace(256, N, K, dev)
    with torch.cuda.stream(stream):
        res = awq.search_scales(Xc, W, workspace=ws)
        p = awq.quantize_pack(W, res.s_best)
        ys = {M: awq.linear_w4a16(xs[M], p) for M in xs}
        parts = {"search": lambda: awq.search_scales(Xc, W, workspace=ws, out=res),
                 "quant_pack": lambda: awq.quantize_pack(W, res.s_best, out=p)}
        for M in xs:
            parts[f"linear_m{M}"] = (lambda M=M: awq.linear_w4a16(xs[M], p, out=ys[M]))
        out = {"workload": "single linear K=N=1024, calibration T=256, 20 alpha, group 128; "
                           "linear at M=1 and M=16"}
        for name, fn in parts.items():
            # 32 calls per graph: one call of this size is a few microseconds
            def many(fn=fn):
                for _ in range(32):
                    fn()
            g = capture(torch, stream, many)
            g.replay()
            t = [x / 32 for x in timer.replays(g.replay, reps)]
            out[name] = {"us_median": round(pct(t, 0.5) * 1e3, 3), "us_p10": round(pct(t, 0.1) * 1e3, 3),
                         "us_p90": round(pct(t, 0.9) * 1e3, 3)}
    out["search"]["tflops_algorithmic"] = round(2 * 256 * N * K * 20 / (out["search"]["us_median"] * 1e-6) / 1e12, 2)
    out["quant_pack"]["gbs"] = round((2 * N * K + packed_bytes(N, K)) / (out["quant_pack"]["us_median"] * 1e-6) / 1e9, 1)
    for M in xs:
        out[f"linear_m{M}"]["gbs"] = round(linear_bytes(M, N, K) / (out[f"linear_m{M}"]["us_median"] * 1e-6) / 1e9, 1)
    out["best_alpha_index"] = int(res.best_idx.item())
    out["note"] = "each figure is one call's time inside a graph of 32 back-to-back calls (L2-resident operands)"
    return out


# ---------------------------------------------------------------------------- 70B sweep
def sweep_70b(awq, si, dev, stream, timer, reps, log):
    """Decode over 80 Llama-2-70B layers whose packed weights (35.6 GB) are all resident:
    per layer q|k|v, o, gate|up (fused, SiLU epilogue) and down, at M = 1 and M = 32."""
    import torch
    log(f"bench: packing {LAYERS_70B} Llama-2-70B layers")
    layers = []
    with torch.cuda.stream(stream):
        for c in range(LAYERS_70B):
            layer = {}
            for i, (g, (N, K)) in enumerate(GROUPS_70B.items()):
                w = si.torch_weights(N, K, 20000 + 7 * c + i, dev)
                layer[g] = awq.quantize_pack(w)
                del w
            layers.append(layer)
        torch.cuda.synchronize()
    resident = sum(p.nbytes() for layer in layers for p in layer.values())
    out = {"workload": "Llama-2-70B decoder layers (q|k|v 10240x8192, o 8192x8192, gate|up 2x28672x8192 "
                       "fused with SiLU epilogue, down 8192x28672), 80 layers resident",
           "resident_packed_bytes": resident, "launches_per_sweep": 4 * LAYERS_70B}
    for M in (1, 32):
        xin = {K: si.torch_activations(M, K, 21000 + K + M, dev, channel_offset=K) for K in (8192, 28672)}
        ys = {g: torch.empty((M, N // 2 if g in GATED else N), dtype=torch.float16, device=dev)
              for g, (N, K) in GROUPS_70B.items()}

        def sweep():
            for layer in layers:
                for g, (N, K) in GROUPS_70B.items():
                    linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                    linear(xin[K], layer[g], out=ys[g])
        with torch.cuda.stream(stream):
            sweep()
            g = capture(torch, stream, sweep)
            for _ in range(2):
                g.replay()
            t = timer.replays(g.replay, max(10, reps // 3))
        nbytes = LAYERS_70B * sum(linear_bytes(M, N, K, gname in GATED) for gname, (N, K) in GROUPS_70B.items())
        flops = LAYERS_70B * sum(2 * M * N * K for N, K in GROUPS_70B.values())
        med = pct(t, 0.5)
        out[f"m{M}"] = {"gbs": round(nbytes / (med * 1e-3) / 1e9, 1), "ms_median": round(med, 4),
                        "ms_p10": round(pct(t, 0.1), 4), "ms_p90": round(pct(t, 0.9), 4),
                        "frac": round(nbytes / (med * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                        "tflops": round(flops / (med * 1e-3) / 1e12, 2), "bytes": nbytes,
                        "kernel": "vector GEMV" if M == 1 else "skinny MFMA GEMV"}
        log(f"bench: 70B decode M={M}: {out[f'm{M}']['gbs']:.0f} GB/s")
        del g
    del layers
    torch.cuda.empty_cache()
    return out


# ---------------------------------------------------------------------------- CPU oracle
def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline():
    """The CPU oracle (plain NumPy, fp64 where the method's arithmetic is exact) timed on
    this machine's host cores on bounded samples of the benchmark's work, with one BLAS thread
    and with all of them. The headline figure is the oracle's W4A16 linear at M = 1 (the
    GPU's headline metric) with all threads."""
    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle
    import synthetic_inputs as si

    def timed(fn):
        t0 = time.perf_counter()
        fn()
        return time.perf_counter() - t0

    # inputs (untimed)
    mats = {}
    for i, (name, _, _, N, K) in enumerate(MATRICES):
        W = si.weights(N, K, offset=500 + i)
        mats[name] = (W, oracle.quantize_pack(W)[:3], si.activations(1, K, offset=600 + i, channel_offset=K))
    W_o, pk_o, _ = mats["o_proj"]
    x16 = si.activations(16, 4096, offset=616, channel_offset=4096)
    x2048 = si.activations(2048, 4096, offset=617, channel_offset=4096)
    rows2048 = 512  # sample: the M = 2048 linear on 512 of o_proj's 4096 rows
    pk_o_rows = tuple(a[:rows2048] for a in pk_o)
    Wc1 = si.weights(1024, 1024, offset=7000)
    Xc1 = si.activations(256, 1024, offset=7001, channel_offset=1024)
    Xc4 = si.activations(CALIB_T, 4096, offset=7100, channel_offset=4096)

    legs = {}
    blas = [p for p in threadpool_info() if p.get("user_api") == "blas"]
    all_threads = max((p.get("num_threads", 1) for p in blas), default=1)
    for label, nthreads in (("threads_1", 1), ("threads_all", all_threads)):
        with threadpool_limits(limits=nthreads, user_api="blas"):
            r = {}
            t = sum(timed(lambda m=m: oracle.linear_reference(m[2], *m[1], m[0].shape[1])) for m in mats.values())
            b = sum(linear_bytes(1, m[0].shape[0], m[0].shape[1]) for m in mats.values())
            r["linear_m1"] = {"gbs": round(b / t / 1e9, 4), "s": round(t, 3),
                              "sample": "7 Llama-2-7B matrices, M=1"}
            t = timed(lambda: oracle.linear_reference(x16, *pk_o, 4096))
            r["linear_m16"] = {"gbs": round(linear_bytes(16, 4096, 4096) / t / 1e9, 4), "s": round(t, 3),
                               "sample": "o_proj 4096x4096, M=16"}
            t = timed(lambda: oracle.linear_reference(x2048, *pk_o_rows, 4096))
            r["linear_m2048"] = {"gflops": round(2 * 2048 * rows2048 * 4096 / t / 1e9, 3), "s": round(t, 3),
                                 "sample": f"o_proj rows 0..{rows2048 - 1} (of 4096), M=2048"}
            pack_names = ("q_proj", "o_proj", "down_proj")
            t = sum(timed(lambda n=n: oracle.quantize_pack(mats[n][0])) for n in pack_names)
            b = sum(2 * mats[n][0].size + packed_bytes(*mats[n][0].shape) for n in pack_names)
            r["quant_pack"] = {"gbs": round(b / t / 1e9, 4), "s": round(t, 3),
                               "sample": "O1-O6 on q_proj, o_proj, down_proj (3 of the 7 matrices)"}
            t = timed(lambda: oracle.search_scales(Xc1, Wc1))
            r["search_single_linear"] = {"gflops": round(2 * 256 * 1024 * 1024 * 20 / t / 1e9, 3), "s": round(t, 3),
                                         "sample": "full 20-point search, K=N=1024, T=256"}
            t = timed(lambda: oracle.search_errors(Xc4, W_o, grid_points=[7]))
            r["search_7b_block"] = {"gflops": round(2 * CALIB_T * 4096 * 4096 / t / 1e9, 3), "s": round(t, 3),
                                    "sample": "one grid point of the o_proj search (T=512); the full 7B "
                                              "block search is 4.145 TFLOP (4 groups x 20 points)",
                                    "est_full_block_s": round(t * 4.145e12 / (2 * CALIB_T * 4096 * 4096), 1)}
            legs[label] = r
    nproc = os.cpu_count()
    return {"value": legs["threads_all"]["linear_m1"]["gbs"], "unit": "GB/s", "cores": all_threads,
            "kind": "oracle",
            "sample": "oracle fp64 W4A16 linear, M=1, on the 7 Llama-2-7B matrices (105.3 MB algorithmic), "
                      f"{all_threads} BLAS threads; other legs below, with 1 and {all_threads} threads",
            "nproc": nproc, "cpu_model": cpu_model(), "blas": blas[0].get("internal_api") if blas else None,
            "legs": legs}


def load_traffic(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json), or None
    when the measured kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("kernel_source_hash") != kernel_source_hash():
        return None
    return d.get("kernels", {}).get(kernel_key)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--reps", type=int, default=50, help="replays per part for the distributions")
    ap.add_argument("--layers", type=int, default=DECODE_LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the format variants (64/32-channel groups, symmetric, 8- and 3-bit)")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the headline step (no peaks, distributions, 70B, single linear, crossover)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    ap.add_argument("--only", default="", metavar="PARTS",
                    help="comma-separated parts (search, clip, quant_pack, fold, gemv, gemv_unfused, "
                         "gemm, mfma_loop, read_stream) run eagerly --steps times each, then exit without timing: "
                         "a short driver for hardware counter passes")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="BYTES",
                    help="first run one plain device copy of BYTES (a known-size kernel for "
                         "calibrating HBM traffic counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py: this build runs on one GPU; --gpus N with N > 1 is not supported "
              "(the multi-GPU sharding is a design note only).", file=sys.stderr)
        sys.exit(2)

    import torch
    import synthetic_inputs as si
    import weight_only_bit_02_amd as awq
    from weight_only_bit_02_amd import _abi

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
    lib = _abi.load()
    if args.copy_probe:
        src = torch.empty(args.copy_probe, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ------------------------------------------------------------------ inputs (untimed)
    # The linears sharing an input are one search group and one packed tensor (q|k|v and
    # gate|up concatenated along N); a single matrix is a row slice of its group's
    # packed tensor (the format is row-major per output channel).
    log("bench: generating inputs")
    Wg = {g: si.torch_weights(N, K, 100 + i, dev) for i, (g, (N, K)) in enumerate(SEARCH_GROUPS.items())}
    Xcal = {g: si.torch_activations(CALIB_T, K, 200 + i, dev, channel_offset=K)
            for i, (g, (N, K)) in enumerate(SEARCH_GROUPS.items())}
    ws = {g: awq.SearchWorkspace(CALIB_T, N, K, dev) for g, (N, K) in SEARCH_GROUPS.items()}
    sres = {g: awq.SearchResult(torch.empty(K, dtype=torch.float16, device=dev),
                                torch.empty(1, dtype=torch.int32, device=dev),
                                torch.empty(20, dtype=torch.float64, device=dev),
                                torch.empty((20, K), dtype=torch.float16, device=dev))
            for g, (N, K) in SEARCH_GROUPS.items()}
    packed = [{g: awq.alloc_packed(N, K, dev) for g, (N, K) in SEARCH_GROUPS.items()} for _ in range(args.layers)]

    def row_slice(p, off, n):
        return awq.PackedLinear(p.qweight[off:off + n], p.scales[off:off + n], p.zeros[off:off + n], n, p.K)

    views = [{name: row_slice(packed[c][g], off, N) for name, g, off, N, K in MATRICES} for c in range(args.layers)]
    log(f"bench: packing {args.layers} layer copies")
    for c in range(1, args.layers):
        for i, (g, (N, K)) in enumerate(SEARCH_GROUPS.items()):
            w = si.torch_weights(N, K, 1000 + 7 * c + i, dev)
            awq.quantize_pack(w, out=packed[c][g])
            del w
    xdec = {4096: si.torch_activations(1, 4096, 300, dev, channel_offset=4096),
            11008: si.torch_activations(1, 11008, 301, dev, channel_offset=11008)}
    ydec = {name: torch.empty((1, N), dtype=torch.float16, device=dev) for name, _, _, N, K in MATRICES}
    yfus = {g: torch.empty((1, N // 2 if g in GATED else N), dtype=torch.float16, device=dev)
            for g, (N, K) in SEARCH_GROUPS.items()}
    xpre = {4096: si.torch_activations(PREFILL_M, 4096, 400, dev, channel_offset=4096),
            11008: si.torch_activations(PREFILL_M, 11008, 401, dev, channel_offset=11008)}
    ypre = {g: torch.empty((PREFILL_M, N // 2 if g in GATED else N), dtype=torch.float16, device=dev)
            for g, (N, K) in SEARCH_GROUPS.items()}
    torch.cuda.synchronize()

    # ------------------------------------------------------------------ the parts
    def part_search():
        for g in SEARCH_GROUPS:
            awq.search_scales(Xcal[g], Wg[g], workspace=ws[g], out=sres[g])

    def part_pack():
        for g in SEARCH_GROUPS:
            awq.quantize_pack(Wg[g], sres[g].s_best, out=packed[0][g])

    def part_gemv():  # decode: q|k|v and gate|up as one launch each (shared input), SiLU * up
        for c in range(args.layers):
            for g, (N, K) in SEARCH_GROUPS.items():
                linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                linear(xdec[K], packed[c][g], out=yfus[g])

    def part_gemv_unfused():  # decode: one launch per matrix
        for c in range(args.layers):
            for name, _, _, N, K in MATRICES:
                awq.linear_w4a16(xdec[K], views[c][name], out=ydec[name])

    def part_gemv_hot():  # the same four launches on ONE layer copy, 32 times (cache-resident)
        for _ in range(args.layers):
            for g, (N, K) in SEARCH_GROUPS.items():
                linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                linear(xdec[K], packed[0][g], out=yfus[g])

    # The equivalent transform's other half: each group's 1/s folded into what produces its
    # input -- the two norm weights (q|k|v, gate|up), the v_proj rows (o), the up_proj rows
    # (down) -- out of place, so the search inputs are untouched.
    norm_w = {g: si.torch_activations(1, 4096, 500 + i, dev) for i, g in enumerate(("qkv", "gate_up"))}
    fold_jobs = [(norm_w["qkv"], "qkv", 1), (norm_w["gate_up"], "gate_up", 1),
                 (Wg["qkv"][8192:12288], "o", 0), (Wg["gate_up"][11008:22016], "down", 0)]
    fold_out = [torch.empty_like(a) for a, _, _ in fold_jobs]
    fold_bytes = sum(4 * a.numel() + 2 * (a.shape[1] if axis == 1 else a.shape[0]) for a, _, axis in fold_jobs)

    # Weight clipping after the scale search: 20 shrink ratios (r = 1 .. 0.905 on the
    # clip_steps = 200 grid) per group of each group's W diag(s).
    CLIP_SHRINK = 20
    clip_ws = {g: torch.empty(lib.awq_clip_search_workspace_size(CALIB_T, N, K, CLIP_SHRINK, None),
                              dtype=torch.uint8, device=dev) for g, (N, K) in SEARCH_GROUPS.items()}
    clip_out = {}

    def part_clip():
        for g in SEARCH_GROUPS:
            clip_out[g] = awq.clip_search(Xcal[g], Wg[g], sres[g].s_best, 200, CLIP_SHRINK,
                                          workspace=clip_ws[g])

    def part_fold():
        for (a, g, axis), o in zip(fold_jobs, fold_out):
            awq.apply_inverse_scale(a, sres[g].s_best, axis, out=o)

    # The prefill GEMM rotates over GEMM_COPIES layer copies (5 x 105 MB of packed weights,
    # beyond the 256 MB last-level cache), one copy per replay, so no replay finds its
    # weights cached by the one before.
    def make_part_gemm(c):
        def part_gemm():
            for g, (N, K) in SEARCH_GROUPS.items():
                linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
                linear(xpre[K], packed[c][g], out=ypre[g])
        return part_gemm
    gemm_copies = min(GEMM_COPIES, args.layers)
    part_gemm = make_part_gemm(0)

    parts = [("search", part_search), ("clip", part_clip), ("quant_pack", part_pack), ("fold", part_fold),
             ("gemv", part_gemv), ("gemv_unfused", part_gemv_unfused), ("gemm", part_gemm)]
    stream = torch.cuda.Stream()
    if args.only:
        fs = torch.empty(4 * 8192, dtype=torch.float32, device=dev)

        def part_mfma_loop():  # the fp16 MFMA loop of the peak measurement (counter calibration)
            import ctypes as C
            lib.awq_peak_mfma(4096, C.c_void_p(fs.data_ptr()), 2048, C.c_void_p(stream.cuda_stream))
        rs_n = sum(linear_bytes(1, N, K, g in GATED) for g, (N, K) in SEARCH_GROUPS.items()) // 4 // 16 * 16
        rs_bufs = [torch.full((rs_n,), 7, dtype=torch.uint8, device=dev) for _ in range(8)] \
            if "read_stream" in args.only else []
        rs_sink = torch.empty(4 * (rs_n // 16384 + 1), dtype=torch.int32, device=dev)

        def part_read_stream():  # plain reads of one average fused decode launch's bytes
            import ctypes as C
            for b in rs_bufs:
                lib.awq_peak_read_stream(C.c_void_p(b.data_ptr()), rs_n, C.c_void_p(rs_sink.data_ptr()),
                                         4, C.c_void_p(stream.cuda_stream))
        known = dict(parts, mfma_loop=part_mfma_loop, read_stream=part_read_stream)
        chosen = [p for p in args.only.split(",") if p]
        unknown = [p for p in chosen if p not in known]
        if unknown:
            print(f"bench.py: unknown part(s) {unknown}; choose from {sorted(known)}", file=sys.stderr)
            sys.exit(2)
        with torch.cuda.stream(stream):
            for pname in chosen:
                log(f"bench: part {pname} x{args.steps} (eager)")
                for _ in range(args.steps):
                    known[pname]()
                torch.cuda.synchronize()
        print(json.dumps({"only": chosen, "steps": args.steps}), flush=True)
        return
    timer = Timer(torch, stream)
    runners = {}
    with torch.cuda.stream(stream):
        for _, fn in parts:  # eager warm-up (also loads the code objects)
            fn()
        torch.cuda.synchronize()
        eager_ref = {"best": {g: sres[g].best_idx.clone() for g in SEARCH_GROUPS},
                     "y": {n: ydec[n].clone() for n in ydec}, "yf": {g: yfus[g].clone() for g in yfus},
                     "fold": [o.clone() for o in fold_out]}
        gemm_eager = []  # the prefill outputs of each layer copy, eager
        for c in range(gemm_copies):
            make_part_gemm(c)()
            torch.cuda.synchronize()
            gemm_eager.append({g: ypre[g].clone() for g in ypre})
        for pname, fn in parts:
            if pname == "gemm":
                fns = [make_part_gemm(c) for c in range(gemm_copies)]
                runners[pname] = Rotation(fns if args.no_graph else
                                          [capture(torch, stream, f).replay for f in fns])
            else:
                runners[pname] = fn if args.no_graph else capture(torch, stream, fn).replay
        torch.cuda.synchronize()

        # Timed in phases: the K steps run part by part (K decode sweeps, then K prefill
        # GEMMs, ...), each part back to back with itself, as it runs in service (a decode
        # loop never follows an 11 ms quantization search, after which the VALU-bound decode
        # kernel runs at a lower clock). Warm-up ends with the decode parts, so the first
        # timed phase follows its own kind of work. One event pair brackets each phase.
        order = ["gemv", "gemv_unfused", "gemm", "fold", "quant_pack", "search", "clip"]
        log(f"bench: warmup {args.warmup} steps")
        for pname in reversed(order):
            for _ in range(args.warmup):
                runners[pname]()
        torch.cuda.synchronize()
        clocks_before = None if args.no_extras else gpu_clocks()
        ev = {pname: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for pname in order}
        log(f"bench: timing {args.steps} steps")
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for pname in order:
            ev[pname][0].record(stream)
            for _ in range(args.steps):
                runners[pname]()
            ev[pname][1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        part_ms = {pname: ev[pname][0].elapsed_time(ev[pname][1]) / args.steps for pname in order}
        clocks_after = None if args.no_extras else gpu_clocks()

        # graph replays must reproduce the eager results bit for bit
        for g in SEARCH_GROUPS:
            assert torch.equal(sres[g].best_idx, eager_ref["best"][g]), "graph replay differs (search)"
            assert torch.equal(yfus[g], eager_ref["yf"][g]), "graph replay differs (gemv)"
            assert torch.equal(ypre[g], gemm_eager[runners["gemm"].last][g]), "graph replay differs (gemm)"
        for n in ydec:
            assert torch.equal(ydec[n], eager_ref["y"][n]), "graph replay differs (gemv, per matrix)"
        for o, e in zip(fold_out, eager_ref["fold"]):
            assert torch.equal(o, e), "graph replay differs (fold)"

        # per-replay distributions (after the timed steps, the same graphs)
        distributions = {}
        if not args.no_extras:
            log(f"bench: distributions over {args.reps} replays per part")
            for pname in order:
                runners[pname]()
                distributions[pname] = dist(timer.replays(runners[pname], args.reps))
            hot = runners["gemv_hot"] = capture(torch, stream, part_gemv_hot).replay
            hot()
            distributions["gemv_hot"] = dist(timer.replays(hot, args.reps))

    # ------------------------------------------------------------------ figures
    n_gemv = args.layers * len(SEARCH_GROUPS)
    gemv_bytes = args.layers * sum(linear_bytes(1, N, K, g in GATED) for g, (N, K) in SEARCH_GROUPS.items())
    gemv_gbs = gemv_bytes / (part_ms["gemv"] * 1e-3) / 1e9
    n_gemv_u = args.layers * len(MATRICES)
    gemv_bytes_u = args.layers * sum(linear_bytes(1, N, K) for _, _, _, N, K in MATRICES)
    gemv_gbs_u = gemv_bytes_u / (part_ms["gemv_unfused"] * 1e-3) / 1e9
    gemm_flops = sum(2 * PREFILL_M * N * K for N, K in SEARCH_GROUPS.values())
    gemm_tflops = gemm_flops / (part_ms["gemm"] * 1e-3) / 1e12
    search_flops = sum(2 * CALIB_T * N * K * 20 for N, K in SEARCH_GROUPS.values())
    search_tflops = search_flops / (part_ms["search"] * 1e-3) / 1e12
    pack_bytes = sum(N * K * 2 + packed_bytes(N, K) for N, K in SEARCH_GROUPS.values())
    pack_gbs = pack_bytes / (part_ms["quant_pack"] * 1e-3) / 1e9
    fold_gbs = fold_bytes / (part_ms["fold"] * 1e-3) / 1e9
    clip_flops = sum(2 * CALIB_T * N * K * CLIP_SHRINK for N, K in SEARCH_GROUPS.values())
    clip_tflops = clip_flops / (part_ms["clip"] * 1e-3) / 1e12
    best = {g: int(sres[g].best_idx.item()) for g in SEARCH_GROUPS}

    traffic = load_traffic("gemv_m1")
    result = {
        "metric": "W4A16 GEMV GB/s @M=1 and dequant-GEMM TFLOP/s @M=2048, 7B shapes",
        "value": round(gemv_gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16 (int4 weights, fp32 accumulate)",
        "data": "synthetic (seeded; W ~ N(0,0.02^2), X ~ N(0,1) with 1% channels x20)",
        "config": {"workload": "Llama-2-7B decoder-layer linears (q,k,v,o 4096x4096; gate,up 11008x4096; "
                               "down 4096x11008): decode GEMV M=1 over "
                               f"{args.layers} layer copies with q|k|v and gate|up (SiLU(gate)*up epilogue) launched together; "
                               f"prefill GEMM M={PREFILL_M}; scale search T={CALIB_T}, 20 alpha, group 128; "
                               "quantize+pack",
                   "gemv_launches_per_step": n_gemv, "group_size": GROUP, "w_bit": 4,
                   "graphs": not args.no_graph, "timing": "phased (each part K times back to back)",
                   "gemm_layer_copies": gemm_copies},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "awq::k_gemv1s (M=1 decode GEMV; q|k|v, o, gate|up gated, down)",
                     "avg_launch_us": round(part_ms["gemv"] * 1e3 / n_gemv, 3),
                     "algorithmic_bytes_per_launch": round(gemv_bytes / n_gemv)},
        "gemm": {"tflops": round(gemm_tflops, 2), "ms": round(part_ms["gemm"], 4),
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                              "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                              "kernel": "awq::k_gemm_wide (256-row tiles: 256 x 128 for q|k|v, o "
                                        "and down, 256 x 256 for gate|up)"}},
        "search": {"tflops_algorithmic": round(search_tflops, 2), "ms": round(part_ms["search"], 4),
                   "best_alpha_index": best,
                   "roofline": {"bound": "mfma", "achieved": round(search_tflops, 2),
                                "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(search_tflops / FP16_MFMA_PEAK_TFLOPS, 4),
                                "kernel": "awq::k_search_err (plus its statistic, scale and reduce kernels)"}},
        "clip_search": {"tflops_algorithmic": round(clip_tflops, 2), "ms": round(part_ms["clip"], 4),
                        "ratios": CLIP_SHRINK, "clip_steps": 200,
                        "roofline": {"bound": "mfma", "achieved": round(clip_tflops, 2),
                                     "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(clip_tflops / FP16_MFMA_PEAK_TFLOPS, 4)}},
        "fold_inverse_scale": {"gbs": round(fold_gbs, 2), "ms": round(part_ms["fold"], 4),
                               "bytes": fold_bytes,
                               "roofline": {"bound": "hbm", "achieved": round(fold_gbs, 2),
                                            "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                            "frac": round(fold_gbs / HBM_PEAK_GBS, 4)}},
        "quant_pack": {"gbs": round(pack_gbs, 2), "ms": round(part_ms["quant_pack"], 4),
                       "roofline": {"bound": "hbm", "achieved": round(pack_gbs, 2), "peak": HBM_PEAK_GBS,
                                    "unit": "GB/s", "frac": round(pack_gbs / HBM_PEAK_GBS, 4)}},
        "gemv_ms": round(part_ms["gemv"], 4),
        "gemv_per_matrix": {"gbs": round(gemv_gbs_u, 2), "ms": round(part_ms["gemv_unfused"], 4),
                            "launches_per_step": n_gemv_u, "frac": round(gemv_gbs_u / HBM_PEAK_GBS, 4),
                            "avg_launch_us": round(part_ms["gemv_unfused"] * 1e3 / n_gemv_u, 3)},
        "source_hash": source_hash(),
    }
    if not args.no_extras:
        result["clocks"] = {"before": clocks_before, "after": clocks_after}
        result["distributions"] = distributions
        dh = distributions["gemv_hot"]
        result["decode_hot"] = {
            "label": "single layer copy replayed (105 MB, resident in the 256 MB last-level cache): "
                     "not an HBM figure",
            "gbs": round(gemv_bytes / (dh["median_ms"] * 1e-3) / 1e9, 1), "median_ms": dh["median_ms"]}
        log("bench: measured peaks")
        peaks = measure_peaks(torch, lib, dev, stream, timer, args.reps,
                              [("fused_decode_launch", round(gemv_bytes / n_gemv), 32),
                               ("1GiB", 2 ** 30, 4), ("8GiB", 2 ** 33, 2)])
        result["peaks"] = peaks
        rs = peaks["read_stream"]
        # the measured peak: the best read stream; beside it the read stream of the decode
        # launch's own size (the same fixed launch cost per 26 MB)
        hbm_meas = max(v["gbs"] for v in rs.values())
        peaks["hbm_measured_gbs"] = hbm_meas
        result["roofline"]["measured_peak"] = hbm_meas
        result["roofline"]["frac_of_measured_peak"] = round(gemv_gbs / hbm_meas, 4)
        result["roofline"]["same_size_read_stream_gbs"] = rs["fused_decode_launch"]["gbs"]
        result["roofline"]["frac_of_same_size_read_stream"] = round(gemv_gbs / rs["fused_decode_launch"]["gbs"], 4)
        for key, tf in (("gemm", gemm_tflops), ("search", search_tflops), ("clip_search", clip_tflops)):
            result[key]["roofline"]["measured_peak"] = peaks["mfma_f16_tflops"]
            result[key]["roofline"]["frac_of_measured_peak"] = round(tf / peaks["mfma_f16_tflops"], 4)
        for key, gbs in (("quant_pack", pack_gbs), ("fold_inverse_scale", fold_gbs)):
            result[key]["roofline"]["measured_peak"] = hbm_meas
            result[key]["roofline"]["frac_of_measured_peak"] = round(gbs / hbm_meas, 4)
        log("bench: single linear")
        result["single_linear"] = single_linear(awq, si, dev, stream, timer, args.reps)
        result["crossover"] = crossover(awq, packed[0], dev, stream)
        log("bench: dense fp16 reference GEMM")
        dref = dense_reference(torch, dev, stream, timer, args.reps)
        dref["w4a16_over_dense"] = round(gemm_tflops / dref["tflops"], 3)
        result["gemm"]["dense_fp16_reference"] = dref
    if not args.no_variants:
        del views
        packed = packed[:1]
        torch.cuda.empty_cache()
        result["variants"] = time_variants(awq, si, dev, stream, Xcal, Wg,
                                           {g: sres[g].s_best for g in SEARCH_GROUPS},
                                           xdec, xpre, args.steps, args.warmup, log)
    if not args.no_extras:
        del packed, runners
        torch.cuda.empty_cache()
        r70 = sweep_70b(awq, si, dev, stream, timer, args.reps, log)
        r70["m1"]["frac_of_measured_peak"] = round(r70["m1"]["gbs"] / result["peaks"]["hbm_measured_gbs"], 4)
        result["llama2_70b_decode"] = r70
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (bounded samples)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
