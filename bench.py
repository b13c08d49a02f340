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

Prints ONE JSON line. `python bench.py --gpus N` with N > 1 exits: this build runs
on one GPU.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, published
CALIB_T = 512
PREFILL_M = 2048
DECODE_LAYERS = 32
GROUP = 128

MATRICES = [  # name, search group, row offset inside the group, N, K
    ("q_proj", "qkv", 0, 4096, 4096), ("k_proj", "qkv", 4096, 4096, 4096),
    ("v_proj", "qkv", 8192, 4096, 4096), ("o_proj", "o", 0, 4096, 4096),
    ("gate_proj", "gate_up", 0, 11008, 4096), ("up_proj", "gate_up", 11008, 11008, 4096),
    ("down_proj", "down", 0, 4096, 11008),
]
SEARCH_GROUPS = {"qkv": (12288, 4096), "o": (4096, 4096), "gate_up": (22016, 4096), "down": (4096, 11008)}


def packed_bytes(N, K, group=GROUP, w_bit=4):
    """Bytes of one packed [N][K] weight: codes, fp16 scales, zeros (3/4-bit: two per byte)."""
    G = K // group
    return N * K * w_bit // 8 + N * G * 2 + N * (G if w_bit == 8 else (G + 1) // 2)


def linear_bytes(M, N, K, gated=False, group=GROUP, w_bit=4):
    """Algorithmic HBM bytes of one W4A16 linear: packed weight + X + Y (gated: Y is N/2 wide)."""
    return packed_bytes(N, K, group, w_bit) + 2 * M * K + 2 * M * (N // 2 if gated else N)


GATED = {"gate_up"}  # the fused MLP module: SiLU(gate) * up in the launch's epilogue


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "weight_only_bit_02_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        h.update(open(os.path.join(csrc, f), "rb").read())
    return h.hexdigest()[:16]


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
                graph = torch.cuda.CUDAGraph()
                with torch.cuda.graph(graph, stream=stream):
                    fn()
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


def cpu_baseline(budget_s: float = 15.0):
    """The CPU oracle's W4A16 linear at M = 1 on the 7B matrices, bounded to ~budget_s."""
    import numpy as np
    import oracle
    import synthetic_inputs as si
    done_bytes, wall, cpu, names = 0, 0.0, 0.0, []
    for i, (name, _, _, N, K) in enumerate(MATRICES):
        W = si.weights(N, K, offset=500 + i)
        qw, sc, zb, _ = oracle.quantize_pack(W)
        x = si.activations(1, K, offset=600 + i)
        t0, c0 = time.perf_counter(), time.process_time()
        oracle.linear_reference(x, qw, sc, zb, K)
        wall += time.perf_counter() - t0
        cpu += time.process_time() - c0
        done_bytes += linear_bytes(1, N, K)
        names.append(name)
        if wall > budget_s:
            break
    return {"value": round(done_bytes / wall / 1e9, 4), "unit": "GB/s",
            "cores": max(1, round(cpu / wall)), "kind": "oracle",
            "sample": f"oracle fp64 W4A16 linear, M=1, on {len(names)} of the 7 Llama-2-7B matrices "
                      f"({', '.join(names)}); {done_bytes / 1e6:.1f} MB algorithmic in {wall:.2f} s"}


def load_traffic(kernel_key):
    """HBM bytes per launch measured with rocprofv3 counters (profiles/traffic.json), or None
    when the kernels changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    d = json.load(open(path))
    if d.get("source_hash") != source_hash():
        return None
    return d.get("kernels", {}).get(kernel_key)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=DECODE_LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the format variants (64/32-channel groups, symmetric, 8- and 3-bit)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
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

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    log = lambda *a: print(*a, file=sys.stderr, flush=True)
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
    clip_ws = {g: torch.empty(awq.load_library().awq_clip_search_workspace_size(CALIB_T, N, K, CLIP_SHRINK, None),
                              dtype=torch.uint8, device=dev) for g, (N, K) in SEARCH_GROUPS.items()}
    clip_out = {}

    def part_clip():
        for g in SEARCH_GROUPS:
            clip_out[g] = awq.clip_search(Xcal[g], Wg[g], sres[g].s_best, 200, CLIP_SHRINK,
                                          workspace=clip_ws[g])

    def part_fold():
        for (a, g, axis), o in zip(fold_jobs, fold_out):
            awq.apply_inverse_scale(a, sres[g].s_best, axis, out=o)

    def part_gemm():
        for g, (N, K) in SEARCH_GROUPS.items():
            linear = awq.linear_w4a16_gated_silu if g in GATED else awq.linear_w4a16
            linear(xpre[K], packed[0][g], out=ypre[g])

    parts = [("search", part_search), ("clip", part_clip), ("quant_pack", part_pack), ("fold", part_fold),
             ("gemv", part_gemv),
             ("gemv_unfused", part_gemv_unfused), ("gemm", part_gemm)]
    stream = torch.cuda.Stream()
    runners = {}
    with torch.cuda.stream(stream):
        for _, fn in parts:  # eager warm-up (also loads the code objects)
            fn()
        torch.cuda.synchronize()
        eager_ref = {"best": {g: sres[g].best_idx.clone() for g in SEARCH_GROUPS},
                     "y": {n: ydec[n].clone() for n in ydec}, "yf": {g: yfus[g].clone() for g in yfus},
                     "Y": {g: ypre[g].clone() for g in ypre}, "fold": [o.clone() for o in fold_out]}
        for pname, fn in parts:
            if args.no_graph:
                runners[pname] = fn
            else:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=stream):
                    fn()
                runners[pname] = g.replay
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

        # graph replays must reproduce the eager results bit for bit
        for g in SEARCH_GROUPS:
            assert torch.equal(sres[g].best_idx, eager_ref["best"][g]), "graph replay differs (search)"
            assert torch.equal(yfus[g], eager_ref["yf"][g]), "graph replay differs (gemv)"
            assert torch.equal(ypre[g], eager_ref["Y"][g]), "graph replay differs (gemm)"
        for n in ydec:
            assert torch.equal(ydec[n], eager_ref["y"][n]), "graph replay differs (gemv, per matrix)"
        for o, e in zip(fold_out, eager_ref["fold"]):
            assert torch.equal(o, e), "graph replay differs (fold)"

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
                   "graphs": not args.no_graph, "timing": "phased (each part K times back to back)"},
        "roofline": {"bound": "hbm", "achieved": round(gemv_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gemv_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "k_gemv1 (M=1)",
                     "avg_launch_us": round(part_ms["gemv"] * 1e3 / n_gemv, 3),
                     "algorithmic_bytes_per_launch": round(gemv_bytes / n_gemv)},
        "gemm": {"tflops": round(gemm_tflops, 2), "ms": round(part_ms["gemm"], 4),
                 "roofline": {"bound": "mfma", "achieved": round(gemm_tflops, 2),
                              "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                              "frac": round(gemm_tflops / FP16_MFMA_PEAK_TFLOPS, 4)}},
        "search": {"tflops_algorithmic": round(search_tflops, 2), "ms": round(part_ms["search"], 4),
                   "best_alpha_index": best,
                   "roofline": {"bound": "mfma", "achieved": round(search_tflops, 2),
                                "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
                                "frac": round(search_tflops / FP16_MFMA_PEAK_TFLOPS, 4)}},
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
    result["crossover"] = crossover(awq, packed[0], dev, stream)
    if not args.no_variants:
        del packed, views
        torch.cuda.empty_cache()
        result["variants"] = time_variants(awq, si, dev, stream, Xcal, Wg,
                                           {g: sres[g].s_best for g in SEARCH_GROUPS},
                                           xdec, xpre, args.steps, args.warmup, log)
    if not args.no_cpu_baseline:
        log("bench: timing the CPU oracle (bounded sample)")
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
