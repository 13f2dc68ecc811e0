#!/usr/bin/env python3
"""Throughput of the rollout-guided FP4 hot path on one MI355X.

Workload: the long-trajectory stream. 20 guided (deepest) MoE layers x 17
chunks of 8,192 tokens x 2,048 hidden, bf16 train/rollout pairs (8K prompt +
128K response = 139,264 tokens per layer), NVFP4 with one FP32 global scale
per chunk. A step is one pass of the whole path over that batch:

  rollout side   encode_guidance(bits=1), one call over the whole stream (its
                 340 chunks are the call's global-scale groups): per-chunk
                 amax -> global scale, E4M3 block scales, RTN codes, the
                 packed mantissa-bit plane
  training side  guided_fake_quant_stats(bits=1), one call per layer:
                 Reconstruct + BracketFP4 + selection + bf16 dequantization
                 -> y_t, and in the same pass the layer's sums of
                 (x_t - x_r)^2 and (y_t - y_r)^2 (y_r the rollout's RTN
                 output, recomputed from x_r)

Inputs are seeded synthetic tensors drawn on the GPU (no model, no dataset);
they are resident in HBM before the timed region starts. Every kernel runs
through the C ABI of libtrace_fp4.so; the binding only passes pointers.

Prints one JSON line. ``roofline`` covers the call with the largest share of
step time, from HIP events recorded on the launch stream around each phase;
``kernels`` also reports plain guided_fake_quant (no statistics) and the
statistics pass with mismatch counts, each timed the same way outside the
step, and the per-layer encode call; ``mismatch`` summarizes those counts
(code distances between the training and rollout sides, per layer);
``copy_ceiling`` times the library's stream references (and torch's copy) on
the same device as the HBM rates the kernels are compared with;
``cpu_baseline`` times the CPU oracle on a bounded sample of the same
workload in a process pool.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, AMD public specification
HIDDEN = 2048
CHUNK = 8192
NV = 0

# Algorithmic bytes per element (one read of every input, one write of every
# output; the per-chunk global scales add 8 bytes per 16.8M elements), NVFP4,
# 1-bit guidance.
BPE = {
    "encode_guidance": 2 + 1 / 8 + 1 / 16,                 # x_r in; mantissa bits, scales out
    "guided_fake_quant_stats": 2 + 2 + 1 / 8 + 1 / 16 + 2,  # x_t, x_r, bits, scales in; y_t out
    "guided_fake_quant": 2 + 1 / 8 + 1 / 16 + 2,           # x_t, bits, scales in; y_t out
    "guided_fake_quant_stats+mismatch": 2 + 2 + 1 / 8 + 1 / 16 + 2,
}
# rocprofv3 kernel names of each call's main kernel (the counter summary of
# the dominant one is profiles/<name>_stream_nvfp4_pmc.txt).
KERNEL_NAME = {
    "encode_guidance": "onepass_encode_kernel",
    "guided_fake_quant_stats": "guided_kernel",
    "guided_fake_quant": "guided_kernel",
    "guided_fake_quant_stats+mismatch": "guided_kernel",
}
KERNEL_SRC = os.path.join(ROOT, "precision_rl_nvfp4_amd", "csrc", "trace_fp4_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")
MX = 1

# The workloads other than the stream, as [layers, rows, cols] train/rollout
# pairs of the 20 guided (deepest) layers. enc_gr: rows per global-scale
# group (one S per layer tensor, or per K / V tensor); the step encodes every
# layer's rollout tensor in one call, then runs the training side layer by
# layer (guided_fake_quant_stats; for per-expert scales the grouped calls and
# discrepancy_stats, since the fused statistics take equal groups only).
CONFIGS = {
    "stream": None,
    "moe": dict(workload="moe_nvfp4_20x65536x2048", fmt=NV, bits=1, rows=65536, cols=HIDDEN, enc_gr=65536),
    "moe_expert": dict(workload="moe_nvfp4_per_expert_20x65536x2048", fmt=NV, bits=1, rows=65536, cols=HIDDEN,
                       enc_gr=0),
    "kv": dict(workload="kv_nvfp4_20x2x65536x256", fmt=NV, bits=4, rows=2 * 65536, cols=256, enc_gr=65536),
    "mxfp4": dict(workload="mxfp4_20x65536x2048", fmt=MX, bits=1, rows=65536, cols=HIDDEN, enc_gr=0),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=20, help="guided layers (deepest first)")
    ap.add_argument("--chunks", type=int, default=17, help="8192-token chunks per layer")
    ap.add_argument("--cpu-workers", type=int, default=0, help="0: usable cores, at most 16")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle wall time")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the plain guided_fake_quant timing")
    ap.add_argument("--no-diag", action="store_true", help="skip the mismatch-diagnostics pass")
    ap.add_argument("--no-record", action="store_true", help="skip the record-path timings")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the record-width and per-token-scale timings")
    ap.add_argument("--encode-batch", type=int, default=-1,
                    help="groups per batch of the two-pass NVFP4 encode (library default if < 0)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain device copy of known size (counter calibration)")
    ap.add_argument("--config", choices=sorted(CONFIGS), default="stream",
                    help="workload: stream (the 136K-token stream, default), moe (routed-expert "
                         "activations, one S per layer), moe_expert (one S per expert), kv (FP4 KV "
                         "cache, full codes), mxfp4 (MXFP4 with midpoint ties)")
    return ap.parse_args()


# ---------------------------------------------------------------- workload

class Workload:
    """All chunks of the stream, resident in HBM, as [layers, chunks*8192, 2048]."""

    def __init__(self, torch, syn, layers, chunks, dev):
        self.layers, self.chunks = layers, chunks
        self.rows = chunks * CHUNK
        self.n = self.rows * HIDDEN                      # elements per layer call
        shape = (layers, self.rows, HIDDEN)
        self.xt = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.xr = torch.empty_like(self.xt)
        for li, layer in enumerate(syn.GUIDED_LAYERS[:layers]):
            sigma = syn.stream_sigma(layer, dev)
            for c in range(chunks):
                xt, xr = syn.stream_pair(layer, c, dev, sigma=sigma)
                self.xt[li, c * CHUNK:(c + 1) * CHUNK].copy_(xt)
                self.xr[li, c * CHUNK:(c + 1) * CHUNK].copy_(xr)
                del xt, xr
        self.guide = torch.empty((layers, self.rows, HIDDEN // 8), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((layers, self.rows, HIDDEN // 16), dtype=torch.uint8, device=dev)
        self.gscale = torch.empty((layers, chunks, 2), dtype=torch.float32, device=dev)
        self.yt = torch.empty_like(self.xt)
        self.acc = torch.zeros((layers, 3), dtype=torch.float64, device=dev)
        self.counts = torch.zeros((layers, 32), dtype=torch.int64, device=dev)

    def bytes_resident(self):
        ts = [self.xt, self.xr, self.guide, self.scales, self.gscale, self.yt, self.acc]
        return sum(t.numel() * t.element_size() for t in ts)


def build_phases(lib, w, stream, qwork, swork):
    """Argument tuples of every ABI call, grouped by phase. The step encodes
    the whole stream (every layer's chunks, one S per chunk) in one call, then
    runs the guided pass with the statistics layer by layer; the per-layer
    encode calls are timed outside the step (and feed the record path)."""
    qb, sb = qwork.numel() * qwork.element_size(), swork.numel() * swork.element_size()
    enc_all = [(NV, 1, w.layers * w.rows, HIDDEN, CHUNK, w.xr.data_ptr(), None, w.guide.data_ptr(),
                w.scales.data_ptr(), w.gscale.data_ptr(), None, qwork.data_ptr(), qb, stream)]
    enc, gst, gfq, dia = [], [], [], []
    for i in range(w.layers):
        p = lambda t: t[i].data_ptr()  # noqa: E731
        enc.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xr), None, p(w.guide), p(w.scales),
                    p(w.gscale), None, qwork.data_ptr(), qb, stream))
        gst.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xt), p(w.xr), p(w.guide), p(w.scales),
                    p(w.gscale), p(w.yt), None, p(w.acc), None, 0, swork.data_ptr(), sb, stream))
        gfq.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xt), p(w.guide), p(w.scales), p(w.gscale),
                    p(w.yt), None, stream))
        dia.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xt), p(w.xr), p(w.guide), p(w.scales),
                    p(w.gscale), p(w.yt), None, p(w.acc), p(w.counts), 0, swork.data_ptr(), sb, stream))
    step = [("encode_guidance", lib.encode_guidance, enc_all),
            ("guided_fake_quant_stats", lib.guided_fake_quant_stats, gst)]
    per_layer = [("encode_guidance", lib.encode_guidance, enc)]
    extra = [("guided_fake_quant", lib.guided_fake_quant, gfq)]
    diag = [("guided_fake_quant_stats+mismatch", lib.guided_fake_quant_stats, dia)]
    return step, per_layer, extra, diag


def variant_phases(lib, w, stream, qwork, torch, dev):
    """Record widths 2, 3 and 4 (chunk scales) and the 1-bit record with one
    global scale per token: (name, bytes/elem of encode, of guided, phases)."""
    qb = qwork.numel() * qwork.element_size()
    guide = torch.empty((w.layers, w.rows, HIDDEN // 2), dtype=torch.uint8, device=dev)
    gtok = torch.empty((w.layers, w.rows, 2), dtype=torch.float32, device=dev)
    out = []
    for name, bits, gr in (("bits2", 2, CHUNK), ("bits3", 3, CHUNK), ("bits4", 4, CHUNK),
                           ("bits1_per_token", 1, 1)):
        gs = w.gscale if gr == CHUNK else gtok
        enc, gfq = [], []
        for i in range(w.layers):
            p = lambda t: t[i].data_ptr()  # noqa: E731
            enc.append((NV, bits, w.rows, HIDDEN, gr, p(w.xr), None, p(guide), p(w.scales), p(gs),
                        None, qwork.data_ptr(), qb, stream))
            gfq.append((NV, bits, w.rows, HIDDEN, gr, p(w.xt), p(guide), p(w.scales), p(gs), p(w.yt),
                        None, stream))
        gbytes = 8 / (gr * HIDDEN)                     # {S, A} per group
        out.append((name, 2 + bits / 8 + 1 / 16 + gbytes, 2 + bits / 8 + 1 / 16 + 4 / (gr * HIDDEN) + 2,
                    [("encode_guidance", lib.encode_guidance, enc),
                     ("guided_fake_quant", lib.guided_fake_quant, gfq)]))
    return out, (guide, gtok)


def rtn_decode_phases(lib, w, stream, qwork, codes, gsq, dwork):
    """The other steps of the path, per layer: vanilla fake quantization of
    X_t (quantize_rtn with codes, scales and y, S from each chunk's amax),
    RTN under the rollout scales (guided_fake_quant bits=0), the 1-bit
    Reconstruct alone (decode_guidance) and the discrepancy sums alone
    (discrepancy_stats over four distinct layer-sized bf16 arrays):
    (name, bytes/elem, phase)."""
    qb = qwork.numel() * qwork.element_size()
    db = dwork.numel() * dwork.element_size()
    q, g0, dec, st, eg = [], [], [], [], []
    for i in range(w.layers):
        p = lambda t: t[i].data_ptr()  # noqa: E731
        q.append((NV, w.rows, HIDDEN, CHUNK, p(w.xt), None, p(codes), p(w.scales), p(gsq), p(w.yt),
                  qwork.data_ptr(), qb, stream))
        g0.append((NV, 0, w.rows, HIDDEN, CHUNK, p(w.xt), None, p(w.scales), p(w.gscale), p(w.yt), None, stream))
        dec.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xt), p(w.guide), p(w.scales), p(w.gscale), p(codes), stream))
        # the rollout encode with each chunk's S supplied (one read, no combine)
        eg.append((NV, 1, w.rows, HIDDEN, CHUNK, p(w.xr), p(w.gscale), p(w.guide), p(w.scales), None, None,
                   None, 0, stream))
        yr = w.xt[(i + 1) % w.layers].data_ptr()     # a fourth array of the layer's size
        st.append((w.n, p(w.xt), p(w.xr), p(w.yt), yr, p(w.acc), 0, dwork.data_ptr(), db, stream))
    return [("quantize_rtn", 2 + 1 / 2 + 1 / 16 + 2, ("quantize_rtn", lib.quantize_rtn, q)),
            ("guided_fake_quant_bits0", 2 + 1 / 16 + 2, ("guided_fake_quant", lib.guided_fake_quant, g0)),
            ("decode_guidance", 2 + 1 / 8 + 1 / 16 + 1 / 2, ("decode_guidance", lib.decode_guidance, dec)),
            ("discrepancy_stats", 8, ("discrepancy_stats", lib.discrepancy_stats, st)),
            ("encode_guidance_S_supplied", 2 + 1 / 8 + 1 / 16, ("encode_guidance", lib.encode_guidance, eg))]


def record_path(torch, w, step, per_layer, stream, dev, layers):
    """Device-to-host transfer of each layer's compact record (mantissa-bit
    plane, scales, chunk scales) through the pinned ring: alone, and pushed
    right after each layer's encode while the step runs. Plus the gather of a
    request's pages of an FP4 KV code plane."""
    from precision_rl_nvfp4_amd.record import RecordRing, gather_pages

    planes = [[w.guide[i], w.scales[i], w.gscale[i]] for i in range(layers)]
    rec_bytes = sum(t.numel() * t.element_size() for t in planes[0])
    depth = 4
    out = {"bytes_per_layer": rec_bytes, "layers": layers, "ring_slots": depth}
    with RecordRing(rec_bytes, depth) as ring:
        def drain(pending, keep):
            while len(pending) > keep:
                s0 = pending.pop(0)
                ring.wait(s0)
                ring.release(s0)

        for rep in range(2):                           # the first pass warms the path
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pending = []
            for i in range(layers):
                drain(pending, depth - 1)
                pending.append(ring.push(planes[i], stream=stream))
            drain(pending, 0)
            alone = time.perf_counter() - t0
        out["d2h_GB_s"] = round(layers * rec_bytes / alone / 1e9, 2)

        enc, gst = per_layer[0][2], step[1][2]
        for rep in range(2):
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            pending = []
            for i in range(layers):
                st = per_layer[0][1](*enc[i])
                if st != 0:
                    raise RuntimeError(f"encode_guidance returned {st}")
                drain(pending, depth - 1)
                pending.append(ring.push(planes[i], stream=stream))
                st = step[1][1](*gst[i])
                if st != 0:
                    raise RuntimeError(f"guided_fake_quant_stats returned {st}")
            torch.cuda.synchronize()
            gpu_done = time.perf_counter() - t0
            drain(pending, 0)
            with_rec = time.perf_counter() - t0
        out["step_ms_with_records"] = round(with_rec * 1e3, 3)
        out["step_kernels_ms_with_records"] = round(gpu_done * 1e3, 3)

    # FP4 KV cache: 4 KiB pages (16 tokens x 2 heads x 256 codes), a request
    # owning 16,384 scattered pages of a 65,536-page pool.
    page_bytes, npool, nreq = 4096, 65536, 16384
    pool = torch.randint(0, 256, (npool * page_bytes,), dtype=torch.uint8, device=dev)
    ids = torch.randperm(npool, device=dev)[:nreq].to(torch.int32)
    outb = torch.empty(nreq * page_bytes, dtype=torch.uint8, device=dev)
    for _ in range(3):
        gather_pages(pool, page_bytes, ids, out=outb)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 20
    e0.record()
    for _ in range(reps):
        gather_pages(pool, page_bytes, ids, out=outb)
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    out["kv_gather"] = {"bytes": nreq * page_bytes, "avg_us": round(us, 2),
                        "GB_s": round(2 * nreq * page_bytes / (us * 1e-6) / 1e9, 1)}
    return out


def moe_per_expert(torch, syn, dev, reps):
    """One MoE layer (65,536 routed rows x 2048, 256 experts) with one global
    scale per expert from the routing offsets: encode (bits=1) and guided
    rounding, each timed per call with events."""
    import precision_rl_nvfp4_amd as tq

    xt, xr, _, offsets = syn.moe_pair(20, device=dev)
    n = xt.numel()
    work = tq.grouped_workspace("nvfp4", xt.shape[0], xt.shape[1], offsets.numel() - 1, device=dev)
    g = tq.encode_guidance_grouped(xr, offsets, "nvfp4", 1, work=work)
    y = torch.empty_like(xt)
    # The layer (256 MiB per side) would partly stay in the 256 MB Infinity
    # Cache between repetitions: an untimed 512 MiB write evicts it first.
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    out = {}
    for name, fn, bpe in (("encode_guidance_grouped", lambda: tq.encode_guidance_grouped(
                               xr, offsets, "nvfp4", 1, guide=g.guide, scales=g.scales,
                               gscale_out=g.gscale, work=work), 2 + 1 / 8 + 1 / 16),
                          ("guided_fake_quant_grouped", lambda: tq.guided_fake_quant(xt, g, y=y, work=work),
                           2 + 1 / 8 + 1 / 16 + 2)):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            flush.fill_(1)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = sum(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3 / reps
        gbs = bpe * n / (us * 1e-6) / 1e9
        out[name] = {"avg_us_per_call": round(us, 2), "elements_per_call": n, "GB_s": round(gbs, 1),
                     "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}
    return out


def other_configs(torch, syn, dev, reps):
    """The MXFP4 and FP4 KV-cache workloads, timed per call with events (the
    Infinity Cache flushed before each call): MXFP4 encode (bits=1) and
    guided rounding on [65536, 2048] pairs with midpoint ties; the KV cache's
    full-code record (bits=4) and guided rounding on the 40 K and V tensors of
    20 layers ([65536, 256] each), as one call over all 40 (one S per tensor)
    and as one call per tensor."""
    import precision_rl_nvfp4_amd as tq

    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def timeit(fn, n, bpe, calls=1):
        fn()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for e0, e1 in ev:
            flush.fill_(1)
            e0.record()
            fn()
            e1.record()
        torch.cuda.synchronize()
        us = sum(e0.elapsed_time(e1) for e0, e1 in ev) * 1e3 / reps / calls
        gbs = bpe * n / (us * 1e-6) / 1e9
        return {"avg_us_per_call": round(us, 2), "calls_per_pass": calls, "elements_per_call": n,
                "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}

    out = {}
    xt, xr = syn.mxfp4_pair(device=dev)
    n = xt.numel()
    g = tq.encode_guidance(xr, "mxfp4", 1)
    y = torch.empty_like(xt)
    out["mxfp4_65536x2048"] = {
        "encode_guidance": timeit(lambda: tq.encode_guidance(xr, "mxfp4", 1, guide=g.guide, scales=g.scales),
                                  n, 2 + 1 / 8 + 1 / 32),
        "guided_fake_quant": timeit(lambda: tq.guided_fake_quant(xt, g, y=y), n, 2 + 1 / 8 + 1 / 32 + 2)}
    del xt, xr, g, y
    layers = 20
    kt = torch.empty((2 * layers, 65536, 256), dtype=torch.bfloat16, device=dev)
    kr = torch.empty_like(kt)
    for li in range(layers):
        for which in (0, 1):
            a, b = syn.kv_pair(20 + li, which, device=dev)
            kt[2 * li + which].copy_(a)
            kr[2 * li + which].copy_(b)
            del a, b
    ft, fr = kt.view(-1, 256), kr.view(-1, 256)
    n_all, n_one = ft.numel(), kt[0].numel()
    work = tq.quant_workspace("nvfp4", ft.shape[0], 256, 65536, device=dev)
    g = tq.encode_guidance(fr, "nvfp4", 4, group_rows=65536, work=work)
    y = torch.empty_like(ft)
    be, bg = 2 + 1 / 2 + 1 / 16, 2 + 1 / 2 + 1 / 16 + 2
    out["kv_40x65536x256"] = {
        "encode_guidance_one_call": timeit(lambda: tq.encode_guidance(
            fr, "nvfp4", 4, group_rows=65536, guide=g.guide, scales=g.scales, gscale_out=g.gscale, work=work),
            n_all, be),
        "guided_fake_quant_one_call": timeit(lambda: tq.guided_fake_quant(ft, g, bits=4, y=y), n_all, bg)}
    w1 = tq.quant_workspace("nvfp4", 65536, 256, 0, device=dev)
    gs = [tq.encode_guidance(kr[i], "nvfp4", 4, work=w1) for i in range(2 * layers)]
    ys = [torch.empty_like(kt[i]) for i in range(2 * layers)]
    out["kv_40x65536x256"]["encode_guidance_per_tensor"] = timeit(
        lambda: [tq.encode_guidance(kr[i], "nvfp4", 4, guide=gs[i].guide, scales=gs[i].scales,
                                    gscale_out=gs[i].gscale, work=w1) for i in range(2 * layers)],
        n_one, be, calls=2 * layers)
    out["kv_40x65536x256"]["guided_fake_quant_per_tensor"] = timeit(
        lambda: [tq.guided_fake_quant(kt[i], gs[i], bits=4, y=ys[i]) for i in range(2 * layers)],
        n_one, bg, calls=2 * layers)
    return out


def mismatch_report(counts):
    """Fig. 6-style summary of the per-layer mismatch counts: how often RTN
    under the rollout scales misses the rollout code, how many of those misses
    are one codeword away, how often the guided code still misses, and how
    often guidance moves the magnitude up or down."""
    def frac(a, b):
        return round(a / b, 6) if b else None
    tot = [sum(c[k] for c in counts) for k in range(32)]
    n = sum(tot[:15])
    rtn_mis, g_mis = n - tot[15], n - tot[0]
    return {"elements": n,
            "rtn_mismatch_rate": frac(rtn_mis, n),
            "rtn_adjacent_fraction": frac(tot[16], rtn_mis),
            "guided_mismatch_rate": frac(g_mis, n),
            "guided_adjacent_fraction": frac(tot[1], g_mis),
            "moved_up_per_layer": [c[30] for c in counts],
            "moved_down_per_layer": [c[31] for c in counts],
            "rtn_mismatch_rate_per_layer": [frac(sum(c[15:30]) - c[15], sum(c[15:30])) for c in counts]}


def run_phases(phases, events=None):
    for j, (name, fn, calls) in enumerate(phases):
        if events is not None:
            events[j].record()
        for a in calls:
            st = fn(*a)
            if st != 0:
                raise RuntimeError(f"{name} returned {st}")
    if events is not None:
        events[len(phases)].record()


def timed(torch, phases, steps):
    """Run `steps` passes with events around each phase; returns (wall s, per-phase ms lists)."""
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(phases) + 1)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps):
        run_phases(phases, evs[k])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [[evs[k][j].elapsed_time(evs[k][j + 1]) for k in range(steps)] for j in range(len(phases))]
    return wall, per


def kernel_entry(name, ms_list, calls, n, bpe=None):
    steps = len(ms_list)
    ms = sum(ms_list)
    per_call_us = ms * 1e3 / (steps * calls)
    algo = (BPE[name] if bpe is None else bpe) * n
    gbs = algo / (per_call_us * 1e-6) / 1e9
    return {"avg_us_per_call": round(per_call_us, 2), "calls_per_pass": calls,
            "elements_per_call": n, "algorithmic_bytes_per_call": int(algo),
            "GB_s": round(gbs, 1), "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4),
            "Gelem_s": round(n / (per_call_us * 1e-6) / 1e9, 1),
            "phase_ms_per_pass": round(ms / steps, 3)}


# ---------------------------------------------------------------- counters

def read_traffic(kernel, workload="stream_nvfp4"):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 --pmc
    summary of that workload, or None when there is none or the kernel source
    changed since the counters were taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    src_hash = hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()
    if fields.get("kernel_source_sha256") != src_hash:
        return None
    try:
        return float(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


# ---------------------------------------------------------------- CPU baseline

def _oracle_unit(args):
    """encode (rollout) -> guided (training) -> discrepancy sums of one slice,
    taken as one tensor: args = (train bits, rollout bits[, fmt, bits])."""
    import numpy as np
    from oracle import fp4 as ofp4
    bt, br = args[:2]
    fmt, bits = (args[2], args[3]) if len(args) > 2 else (ofp4.NVFP4, 1)
    e = ofp4.encode_guidance(fmt, bits, br)
    g = ofp4.guided_fake_quant(fmt, bits, bt, e["guide"], e["scales"], e["gscale"])
    ofp4.discrepancy_stats(bt, br, g["y"], e["y"])
    return int(np.asarray(bt).size)


def single_core_tiny(torch, target_s=2.0):
    """The same oracle chain on the tiny pair (256 tokens x 2048, seed 0) in
    this process, i.e. on one core, repeated for about `target_s` seconds."""
    import synthetic as syn
    xt, xr = syn.tiny_pair("cpu")
    args = (syn.bits_u16(xt).reshape(-1), syn.bits_u16(xr).reshape(-1))
    _oracle_unit(args)                                   # warm
    reps, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < target_s:
        n = _oracle_unit(args)
        reps += 1
    wall = time.perf_counter() - t0
    return {"value": round(reps * n / wall / 1e9, 6), "unit": "Gelem/s", "cores": 1,
            "sample": f"{reps} passes of encode(bits=1) -> guided(bits=1) -> sums over 256 x 2048, {wall:.1f} s"}


def cpu_baseline(torch, w, workers, target_s):
    """The oracle, as it stands, over slices of the workload (1024 rows of
    2048, or as many rows of a narrower tensor; each slice taken as one tensor
    with its own global scale), through the same encode -> guided ->
    discrepancy path, in rounds of one slice per worker process until about
    `target_s` seconds have passed."""
    import multiprocessing as mp

    import numpy as np
    cols = getattr(w, "cols", HIDDEN)
    fmt, bits = getattr(w, "fmt", NV), getattr(w, "bits", 1)
    rows = max(1024, 2 ** 21 // cols)

    def slice_bits(t, layer, r0):
        return t[layer, r0:r0 + rows].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)

    ctx = mp.get_context("spawn")
    elems, rounds, j = 0, 0, 0
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_unit, [(np.zeros(32, np.uint16), np.zeros(32, np.uint16))] * workers)  # warm
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < target_s and rounds < 64:
            jobs = []
            for _ in range(workers):
                layer = j % w.layers
                r0 = ((j * 37) % (w.rows // rows)) * rows
                jobs.append((slice_bits(w.xt, layer, r0), slice_bits(w.xr, layer, r0), fmt, bits))
                j += 1
            elems += sum(pool.map(_oracle_unit, jobs, chunksize=1))
            rounds += 1
        wall = time.perf_counter() - t0
    single = single_core_tiny(torch)
    return {
        "value": round(elems / wall / 1e9, 6),
        "unit": "Gelem/s",
        "cores": workers,
        "host_cpus": os.cpu_count(),
        "single_core_tiny": single,
        "kind": "oracle",
        "sample": (f"{rounds * workers} slices of {rows} rows x {cols} from the "
                   f"{getattr(w, 'workload', 'streamed')} workload ({elems} elements per side), each one "
                   f"{'NVFP4' if fmt == NV else 'MXFP4'} tensor: encode(bits={bits}) -> guided(bits={bits}) -> "
                   f"discrepancy sums; {workers} worker processes, {rounds} rounds, {wall:.1f} s wall"),
    }


# ---------------------------------------------------------------- ceiling

def warn_wait_failures(fails):
    """A single-pass wait that gave up still gives exact results (the waiting
    wave reads what it waited for from the input), but it means the launch
    did not have the device to itself: the timing is then not the kernel's."""
    if fails:
        print(f"bench: WARNING: {fails} single-pass encode waits gave up during the run "
              f"(results exact, timing disturbed: another process or stream held the device)",
              file=sys.stderr, flush=True)


def _timed_rate(torch, fn, moved, reps):
    for _ in range(3):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    gbs = moved / (us * 1e-6) / 1e9
    return {"bytes_read_plus_written": moved, "avg_us": round(us, 2), "GB_s": round(gbs, 1),
            "frac_of_peak": round(gbs / HBM_PEAK_GBS, 4)}


def copy_ceiling(torch, dev, nbytes=1 << 30, reps=10):
    """The HBM rates plain streams reach on this GPU in this run, timed with
    events, reported beside the roofline (whose `peak` stays the published 8
    TB/s): the library's stream references (trace_stream_copy, one stream in
    and one out; trace_stream_mix, two in and one out, the fused guided
    pass's mix), which use the kernels' access policy, and torch's copy."""
    import precision_rl_nvfp4_amd as tq
    a = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    b = torch.empty_like(a)
    out = torch.empty_like(a)
    a.fill_(1)
    b.fill_(2)
    res = {"kernel": "trace_stream_copy (library stream reference: one stream in, one out)"}
    res.update(_timed_rate(torch, lambda: tq.stream_copy(a, out), 2 * nbytes, reps))
    mix = {"kernel": "trace_stream_mix (library stream reference: two in, one out)"}
    mix.update(_timed_rate(torch, lambda: tq.stream_mix(a, b, out), 3 * nbytes, reps))
    tc = {"kernel": "torch copy_ (device to device)"}
    tc.update(_timed_rate(torch, lambda: out.copy_(a), 2 * nbytes, reps))
    res["two_in_one_out"] = mix
    res["torch_copy"] = tc
    del a, b, out
    return res


# ---------------------------------------------------------------- other workloads

class LayeredWorkload:
    """One of the non-stream workloads (CONFIGS): `layers` train/rollout
    pairs of [rows, cols], resident as [layers, rows, cols], plus the record
    and output buffers of the step."""

    def __init__(self, torch, syn, name, spec, layers, dev):
        self.name, self.workload = name, spec["workload"]
        self.fmt, self.bits = spec["fmt"], spec["bits"]
        self.layers, self.rows, self.cols = layers, spec["rows"], spec["cols"]
        self.enc_gr = spec["enc_gr"]
        self.n = self.rows * self.cols
        shape = (layers, self.rows, self.cols)
        self.xt = torch.empty(shape, dtype=torch.bfloat16, device=dev)
        self.xr = torch.empty_like(self.xt)
        self.offsets = []
        for li, layer in enumerate(syn.GUIDED_LAYERS[:layers]):
            if name in ("moe", "moe_expert"):
                a, b, _, offs = syn.moe_pair(layer, device=dev)
                self.offsets.append(offs)
                self.xt[li].copy_(a)
                self.xr[li].copy_(b)
            elif name == "kv":
                for which in (0, 1):
                    a, b = syn.kv_pair(layer, which, device=dev)
                    self.xt[li, which * 65536:(which + 1) * 65536].copy_(a)
                    self.xr[li, which * 65536:(which + 1) * 65536].copy_(b)
            else:
                a, b = syn.mxfp4_pair(self.rows, self.cols, device=dev, layer=layer)
                self.xt[li].copy_(a)
                self.xr[li].copy_(b)
            del a, b
        B = 16 if self.fmt == NV else 32
        self.B = B
        self.guide = torch.empty((layers, self.rows, self.cols * self.bits // 8), dtype=torch.uint8, device=dev)
        self.scales = torch.empty((layers, self.rows, self.cols // B), dtype=torch.uint8, device=dev)
        if name == "moe_expert":
            E = self.offsets[0].numel() - 1
            self.gscale = torch.empty((layers, E, 2), dtype=torch.float32, device=dev)
            self.yr = torch.empty_like(self.xt)
        elif self.fmt == NV:
            self.gscale = torch.empty((layers, self.rows // self.enc_gr, 2), dtype=torch.float32, device=dev)
            self.yr = None
        else:
            self.gscale, self.yr = None, None
        self.yt = torch.empty_like(self.xt)
        self.acc = torch.zeros((layers, 3), dtype=torch.float64, device=dev)

    def bytes_resident(self):
        ts = [self.xt, self.xr, self.guide, self.scales, self.yt, self.acc] + \
            [t for t in (self.gscale, self.yr) if t is not None]
        return sum(t.numel() * t.element_size() for t in ts)


def layered_phases(lib, tq, w, stream):
    """Argument tuples of the step's calls: (phases, bytes per element of
    each phase's calls, workspaces kept alive)."""
    p = lambda t, i: t[i].data_ptr()  # noqa: E731
    L, R, C, b = w.layers, w.rows, w.cols, w.bits
    plane = b / 8 + 1 / w.B
    keep = []
    if w.name == "moe_expert":
        E = w.offsets[0].numel() - 1
        gb = int(lib.trace_grouped_workspace_bytes(NV, R, C, E))
        gwork = [tq._workspace(gb, w.xt.device, None) for _ in range(L)]
        db = int(lib.trace_stats_workspace_bytes(w.n))
        dwork = tq.stats_workspace(w.n, w.xt.device)
        keep += gwork + [dwork]
        enc, gfq, dst = [], [], []
        for i in range(L):
            enc.append((NV, b, R, C, E, w.offsets[i].data_ptr(), p(w.xr, i), p(w.guide, i), p(w.scales, i),
                        p(w.gscale, i), p(w.yr, i), gwork[i].data_ptr(), gb, stream))
            gfq.append((NV, b, R, C, E, w.offsets[i].data_ptr(), p(w.xt, i), p(w.guide, i), p(w.scales, i),
                        p(w.gscale, i), p(w.yt, i), None, gwork[i].data_ptr(), gb, stream))
            dst.append((w.n, p(w.xt, i), p(w.xr, i), p(w.yt, i), p(w.yr, i), p(w.acc, i), 0, dwork.data_ptr(),
                        db, stream))
        phases = [("encode_guidance_grouped", lib.encode_guidance_grouped, enc),
                  ("guided_fake_quant_grouped", lib.guided_fake_quant_grouped, gfq),
                  ("discrepancy_stats", lib.discrepancy_stats, dst)]
        bpe = {"encode_guidance_grouped": 2 + plane + 2 + 8 * E / w.n,
               "guided_fake_quant_grouped": 2 + plane + 4 * E / w.n + 2, "discrepancy_stats": 8}
        return phases, bpe, keep
    qb = int(lib.trace_quant_workspace_bytes(w.fmt, L * R, C, w.enc_gr))
    qwork = tq._workspace(qb, w.xt.device, None)
    sb = int(lib.trace_guided_stats_workspace_bytes(w.fmt, R, C, w.enc_gr))
    swork = tq._workspace(sb, w.xt.device, None)
    keep += [t for t in (qwork, swork) if t is not None]
    gptr = lambda i: None if w.gscale is None else p(w.gscale, i)  # noqa: E731
    enc = [(w.fmt, b, L * R, C, w.enc_gr, w.xr.data_ptr(), None, w.guide.data_ptr(), w.scales.data_ptr(),
            None if w.gscale is None else w.gscale.data_ptr(), None,
            None if qwork is None else qwork.data_ptr(), qb, stream)]
    gst = [(w.fmt, b, R, C, w.enc_gr, p(w.xt, i), p(w.xr, i), p(w.guide, i), p(w.scales, i), gptr(i),
            p(w.yt, i), None, p(w.acc, i), None, 0, None if swork is None else swork.data_ptr(), sb, stream)
           for i in range(L)]
    gs = 8 / (w.enc_gr * C) if (w.fmt == NV and w.enc_gr) else 0.0
    phases = [("encode_guidance", lib.encode_guidance, enc),
              ("guided_fake_quant_stats", lib.guided_fake_quant_stats, gst)]
    bpe = {"encode_guidance": 2 + plane + gs, "guided_fake_quant_stats": 2 + 2 + plane + gs / 2 + 2}
    return phases, bpe, keep


def kv_per_tensor_phases(lib, tq, w, stream):
    """The KV workload's K and V tensors one call each: encode_guidance
    (bits=4, one S per tensor) and guided_fake_quant_stats, 2 x layers calls
    of [65536, 256] per phase."""
    R = w.rows // 2
    C, b = w.cols, w.bits
    qb = int(lib.trace_quant_workspace_bytes(NV, R, C, 0))
    sb = int(lib.trace_guided_stats_workspace_bytes(NV, R, C, 0))
    qwork = tq._workspace(qb, w.xt.device, None)
    swork = tq._workspace(sb, w.xt.device, None)
    enc, gst = [], []
    for i in range(w.layers):
        for k in (0, 1):
            rs = slice(k * R, (k + 1) * R)
            enc.append((NV, b, R, C, 0, w.xr[i, rs].data_ptr(), None, w.guide[i, rs].data_ptr(),
                        w.scales[i, rs].data_ptr(), w.gscale[i, k].data_ptr(), None, qwork.data_ptr(), qb, stream))
            gst.append((NV, b, R, C, 0, w.xt[i, rs].data_ptr(), w.xr[i, rs].data_ptr(), w.guide[i, rs].data_ptr(),
                        w.scales[i, rs].data_ptr(), w.gscale[i, k].data_ptr(), w.yt[i, rs].data_ptr(), None,
                        w.acc[i].data_ptr(), None, k, swork.data_ptr(), sb, stream))
    plane = b / 8 + 1 / 16
    phases = [("encode_guidance_per_tensor", lib.encode_guidance, enc),
              ("guided_fake_quant_stats_per_tensor", lib.guided_fake_quant_stats, gst)]
    bpe = {"encode_guidance_per_tensor": 2 + plane + 8 / (R * C),
           "guided_fake_quant_stats_per_tensor": 2 + 2 + plane + 4 / (R * C) + 2}
    return phases, bpe, [qwork, swork]


LAYERED_KERNEL = {"encode_guidance": "quantize_kernel", "guided_fake_quant_stats": "guided_kernel",
                  "encode_guidance_grouped": "quantize_kernel", "guided_fake_quant_grouped": "guided_kernel",
                  "discrepancy_stats": "stats_partial_kernel"}


def main_layered(args, torch, syn, tq, lib, dev):
    """bench.py --config moe | moe_expert | kv | mxfp4: the step of that
    workload, with the same timing, roofline and CPU-baseline fields as the
    stream's line."""
    spec = CONFIGS[args.config]
    layers = min(args.layers, 20)
    log(f"bench: generating {layers} layers of the {spec['workload']} workload")
    t0 = time.perf_counter()
    w = LayeredWorkload(torch, syn, args.config, spec, layers, dev)
    stream = torch.cuda.current_stream(dev)
    phases, bpe, keep = layered_phases(lib, tq, w, stream.cuda_stream)
    torch.cuda.synchronize()
    log(f"bench: workload ready in {time.perf_counter() - t0:.1f} s, {w.bytes_resident() / 2**30:.1f} GiB resident")
    fails0 = tq.encode_wait_failures()
    for i in range(args.warmup):
        run_phases(phases)
        torch.cuda.synchronize()
        log(f"bench: warmup step {i + 1}/{args.warmup} done")
    wall, per = timed(torch, phases, args.steps)
    log(f"bench: {args.steps} timed steps in {wall:.3f} s")
    total = layers * w.n
    kernels = {}
    for j, (name, _, calls) in enumerate(phases):
        kernels[name] = kernel_entry(name, per[j], len(calls), total // len(calls), bpe[name])
    dom = max(kernels, key=lambda k: kernels[k]["phase_ms_per_pass"])
    d = kernels[dom]
    roofline = {"bound": "hbm", "achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac_of_peak"], "traffic": read_traffic(LAYERED_KERNEL[dom], spec["workload"]),
                "kernel": dom, "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_call"],
                "avg_launch_us": d["avg_us_per_call"]}
    acc = w.acc.cpu().tolist()
    rel = [((sf - sb) / sb) if sb > 0 else math.nan for sb, sf, _ in acc]
    variants = None
    if args.config == "kv":
        # The same K and V tensors one call per tensor (40 calls of [65536,
        # 256], each its own global scale), outside the step: the calls a
        # cache that encodes each tensor as it fills would make.
        variants = {}
        ph, bp, keep1 = kv_per_tensor_phases(lib, tq, w, stream.cuda_stream)
        run_phases(ph)
        _, per_v = timed(torch, ph, max(3, args.steps // 2))
        for j, (name, _, calls) in enumerate(ph):
            variants[name] = kernel_entry(name, per_v[j], len(calls), total // len(calls), bp[name])
        del keep1
        log("bench: per-tensor KV calls timed")
    fails = tq.encode_wait_failures() - fails0
    warn_wait_failures(fails)
    ceiling = copy_ceiling(torch, dev)
    cpu = None
    if not args.no_cpu_baseline:
        try:
            aff = len(os.sched_getaffinity(0))
        except AttributeError:
            aff = os.cpu_count() or 1
        workers = args.cpu_workers or max(1, min(16, aff))
        log(f"bench: cpu baseline (oracle) on {workers} workers")
        cpu = cpu_baseline(torch, w, workers, args.cpu_seconds)
    ms_step = wall * 1e3 / args.steps
    step_bytes = sum(bpe[name] * total for name, _, _ in phases)
    out = {
        "metric": "guided FP4 fake-quant Gelem/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(total * args.steps / wall / 1e9, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": spec["workload"], "layers": layers, "rows": w.rows, "cols": w.cols,
                   "format": "nvfp4" if w.fmt == NV else "mxfp4", "guide_bits": w.bits,
                   "global_scale_rows": w.enc_gr if w.fmt == NV else None,
                   "per_expert_scales": args.config == "moe_expert",
                   "elements_per_side_per_step": total},
        "roofline": roofline,
        "copy_ceiling": ceiling,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "step_GB_s": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
        "encode_wait_failures": fails,
        "rel_excess_mse_guided_per_layer": [round(r, 6) for r in rel],
        "variants": variants,
    }
    del keep
    print(json.dumps(out), flush=True)


# ---------------------------------------------------------------- main

def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} (WORLD_SIZE={world}) is not supported: "
              "the path has no cross-GPU step to run", file=sys.stderr)
        sys.exit(2)

    import torch

    import precision_rl_nvfp4_amd as tq
    import synthetic as syn
    from precision_rl_nvfp4_amd import _abi

    lib = _abi.load()
    if args.encode_batch >= 0:
        lib.trace_set_encode_batch(args.encode_batch)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.config != "stream":
        return main_layered(args, torch, syn, tq, lib, dev)
    fails0 = tq.encode_wait_failures()
    log(f"bench: generating {args.layers} layers x {args.chunks} chunks of [{CHUNK}, {HIDDEN}] pairs")
    t0 = time.perf_counter()
    w = Workload(torch, syn, args.layers, args.chunks, dev)
    qn = int(lib.trace_quant_workspace_bytes(NV, w.layers * w.rows, HIDDEN, CHUNK))
    sn = int(lib.trace_guided_stats_workspace_bytes(NV, w.rows, HIDDEN, CHUNK))
    qwork = torch.empty(max(qn // 8, 1), dtype=torch.float64, device=dev)
    swork = torch.empty(max(sn // 8, 1), dtype=torch.float64, device=dev)
    torch.cuda.synchronize()
    log(f"bench: workload ready in {time.perf_counter() - t0:.1f} s, "
        f"{w.bytes_resident() / 2**30:.1f} GiB resident")

    stream = torch.cuda.current_stream(dev)
    step, per_layer, extra, diag = build_phases(lib, w, stream.cuda_stream, qwork, swork)

    for i in range(args.warmup):
        run_phases(step)
        torch.cuda.synchronize()
        log(f"bench: warmup step {i + 1}/{args.warmup} done")
    # The single-pass encode publishes each chunk's S in its workspace (after
    # the per-chunk slots); the two-pass schedule leaves those words alone.
    if args.warmup > 0:
        G = w.layers * w.chunks
        pub = qwork.view(torch.int32)[G * 1024:G * 2048:1024].cpu()
        s_all = w.gscale[:, :, 0].contiguous().view(torch.int32).reshape(-1).cpu()
        encode_path = "single-pass" if torch.equal(pub, s_all) else "two-pass"
    else:
        encode_path = "unknown"
    log(f"bench: encode schedule {encode_path}")

    wall, per = timed(torch, step, args.steps)
    log(f"bench: {args.steps} timed steps in {wall:.3f} s")
    acc = w.acc.cpu().tolist()               # sums of the last step

    kernels = {name: kernel_entry(name, per[j], len(calls), w.layers * w.n // len(calls))
               for j, (name, _, calls) in enumerate(step)}
    kernels["encode_guidance"]["note"] = (f"one call over the whole stream: {w.layers * w.chunks} groups of "
                                          f"{CHUNK} rows, one S each")
    run_phases(per_layer)
    _, per_l = timed(torch, per_layer, max(3, args.steps // 2))
    kernels["encode_guidance_per_layer"] = kernel_entry("encode_guidance", per_l[0], len(per_layer[0][2]), w.n)
    kernels["encode_guidance_per_layer"]["note"] = (f"timed outside the step: one call per layer "
                                                    f"({w.chunks} groups of {CHUNK} rows)")
    log("bench: per-layer encode timed")
    if not args.no_extra:
        run_phases(extra)
        _, per_x = timed(torch, extra, max(3, args.steps // 2))
        kernels["guided_fake_quant"] = kernel_entry("guided_fake_quant", per_x[0], len(extra[0][2]), w.n)
        kernels["guided_fake_quant"]["note"] = "timed outside the step (no statistics)"
        log("bench: plain guided_fake_quant timed")

    mismatch = None
    if not args.no_diag:
        # Mismatch diagnostics (outside the timed step): the same fused pass
        # with the per-layer code-distance histograms.
        run_phases(diag)
        _, per_d = timed(torch, diag, max(3, args.steps // 4))
        kernels[diag[0][0]] = kernel_entry(diag[0][0], per_d[0], len(diag[0][2]), w.n)
        kernels[diag[0][0]]["note"] = "timed outside the step (statistics + mismatch counts)"
        mismatch = mismatch_report(w.counts.cpu().tolist())
        log("bench: mismatch diagnostics done")

    variants = None
    if not args.no_variants:
        # The record widths of Algorithm 1's parameter b and per-token scales,
        # timed per call like the step, outside it.
        variants = {}
        vph, keep = variant_phases(lib, w, stream.cuda_stream, qwork, torch, dev)
        for name, bpe_e, bpe_g, phases in vph:
            run_phases(phases)
            _, per_v = timed(torch, phases, max(3, args.steps // 4))
            variants[name] = {
                "encode_guidance": kernel_entry("encode_guidance", per_v[0], len(phases[0][2]), w.n, bpe_e),
                "guided_fake_quant": kernel_entry("guided_fake_quant", per_v[1], len(phases[1][2]), w.n,
                                                  bpe_g)}
        del keep
        # The remaining steps of the path on the same layers: the 1-bit record
        # of the step is re-encoded first, since the variants above rewrote
        # the scale plane.
        run_phases(step[:1])
        codes = torch.empty((w.layers, w.rows, HIDDEN // 2), dtype=torch.uint8, device=dev)
        gsq = torch.empty_like(w.gscale)
        dn = int(lib.trace_stats_workspace_bytes(w.n))
        dwork = torch.empty(max(dn // 8, 1), dtype=torch.float64, device=dev)
        other = {}
        for name, bpe, phase in rtn_decode_phases(lib, w, stream.cuda_stream, qwork, codes, gsq, dwork):
            run_phases([phase])
            _, per_o = timed(torch, [phase], max(3, args.steps // 4))
            other[name] = kernel_entry(phase[0], per_o[0], len(phase[2]), w.n, bpe)
            if name == "quantize_rtn":
                run_phases(step[:1])          # the record again (quantize_rtn rewrote the scales)
        variants["other_steps"] = other
        del codes, gsq, dwork
        variants["moe_per_expert"] = moe_per_expert(torch, syn, dev, max(3, args.steps // 4))
        variants["other_configs"] = other_configs(torch, syn, dev, max(3, args.steps // 4))
        log("bench: variants timed")

    record = None
    if not args.no_record:
        record = record_path(torch, w, step, per_layer, stream.cuda_stream, dev, w.layers)
        log("bench: record path timed")

    elems_step = w.layers * w.n
    ms_step = wall * 1e3 / args.steps
    dom = max((k for k, _, _ in step), key=lambda k: kernels[k]["phase_ms_per_pass"])
    d = kernels[dom]
    roofline = {"bound": "hbm", "achieved": d["GB_s"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": d["frac_of_peak"], "traffic": read_traffic(KERNEL_NAME[dom]), "kernel": dom,
                "algorithmic_bytes_per_launch": d["algorithmic_bytes_per_call"],
                "avg_launch_us": d["avg_us_per_call"]}
    rel = [((sf - sb) / sb) if sb > 0 else math.nan for sb, sf, _ in acc]

    fails = tq.encode_wait_failures() - fails0
    warn_wait_failures(fails)
    ceiling = copy_ceiling(torch, dev)
    if args.copy_probe:
        src = torch.empty(2**30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"bench: copy probe, 5 x {src.numel()} bytes device-to-device")

    cpu = None
    if not args.no_cpu_baseline:
        try:
            aff = len(os.sched_getaffinity(0))
        except AttributeError:
            aff = os.cpu_count() or 1
        workers = args.cpu_workers or max(1, min(16, aff))
        log(f"bench: cpu baseline (oracle) on {workers} workers")
        cpu = cpu_baseline(torch, w, workers, args.cpu_seconds)

    out = {
        "metric": "guided FP4 fake-quant Gelem/s + achieved HBM GB/s (% of peak), 1 GPU",
        "value": round(elems_step * args.steps / wall / 1e9, 2),
        "unit": "Gelem/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "stream_nvfp4_136k_tokens", "layers": w.layers, "chunks": w.chunks,
                   "encode_batch": args.encode_batch, "encode_schedule": encode_path,
                   "chunk_tokens": CHUNK, "hidden": HIDDEN, "format": "nvfp4", "guide_bits": 1,
                   "elements_per_side_per_step": elems_step},
        "roofline": roofline,
        "copy_ceiling": ceiling,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "step_GB_s": round(sum(BPE[k] for k, _, _ in step) * elems_step / (ms_step * 1e-3) / 1e9, 1),
        "encode_wait_failures": fails,
        "rel_excess_mse_guided_per_layer": [round(r, 6) for r in rel],
        "mismatch": mismatch,
        "variants": variants,
        "record_path": record,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
