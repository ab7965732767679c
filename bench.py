#!/usr/bin/env python3
"""Throughput of the TurboQuant-style KV-cache hot path on one MI355X.

Default workload (prefill_append, the largest configuration, which exercises
both halves of the metric): quantize and append 131072 new tokens x 8 KV heads
x head_dim 128 of bf16 K and V (N(0,1) with 6 Student-t(4) channels per head)
into a paged cache of 16-token blocks (keys 4-bit Lloyd-Max with fp32 corrected
norm, values 4-bit uniform with fp32 min/scale), then decode attention at batch
1 with 32 query heads over the whole 131072-token context.  One step = one
tq_quantize_append + one tq_decode_attention.  Steps rotate over --layers
independent caches (one per layer), so the 147 MB cache of a step does not stay
in the 256 MB Infinity Cache between steps.  Both kernels get a roofline entry:
`roofline` for the append (the dominant one) and `roofline_decode`.

Other workloads (--workload):
  gqa_decode      batch 16, 32 query heads, 8 KV heads, context 8192 (the
                  Llama-8B-like shape), same codecs: one step = quantize and
                  append the new token of every sequence, then decode attention
                  of the 16 new queries over their 8192 tokens, in one launch
                  (tq_append_decode; --separate: two launches);
  long_3bit       batch 4 x context 32768, 3-bit keys and values, same step;
  qjl             batch 8 x context 16384, 2-bit keys + 1-bit QJL residual signs,
                  same step;
  qjl_build       the qjl workload's whole cache (8 x 16384 tokens x 8 KV heads)
                  quantized and appended in one step, then its decode;
  k3v4_nc         the GQA shape with 3-bit corrected keys and 4-bit values (an
                  asymmetric serving preset), same step;
  k3qjl_v2        batch 8 x context 16384, 3-bit keys + 1-bit QJL residual signs,
                  2-bit values (a second asymmetric preset), same step;
  k8v4            the GQA shape with FP8 (E4M3) keys and 4-bit values (the
                  preset table's k8v4), same step;
  turbo8v3        the GQA shape with 8-bit Lloyd-Max keys (corrected norm) and
                  3-bit values (an on-device default named on the pages), same step;
  polar3          the GQA shape with PolarQuant keys (3-bit angles of the
                  recursive polar transform, fp32 radius) and 4-bit values, same
                  step;
  dequant_layer   the prefill_append cache (131072 tokens x 8 KV heads)
                  reconstructed into a bf16 buffer (--dequant-f32: fp32) in one
                  tq_dequantize_rows call: the whole-cache reconstruction that
                  incremental dequantization replaces by one token per step.
  gqa_d64, gqa_d256, gqa_group8
                  the GQA shape at head_dim 64 and 256 (the generic path: same
                  step, its one-launch step three launches: the new tokens, the
                  decode per split, the merge), and at head_dim 128 with 2 KV
                  heads of 8 query heads each (the tuned kernels, the decode in
                  two head groups of 4 query heads per KV head).

Prints ONE JSON line on stdout; diagnostics go to stderr.  `value` is packed-KV
GB/s: algorithmic bytes of the step (bf16 inputs read, packed rows written,
packed rows of the attended context read, queries, outputs, tables) divided by
the step time, with every input already resident in HBM.  The step time comes
from a timed region with nothing but the steps in it: the steps are captured in a
HIP graph and replayed (--eager: launched one by one from Python, which leaves the
GPU waiting on the host between short kernels).  For the roofline figure a
second pass runs the dominant kernel alone the same number of times back to
back (graph-replayed likewise) between one pair of HIP events on its stream; a
third pass, eager, brackets each step's dominant launch with its own events for
the spread of single launches.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published peak
FP32_MFMA_PEAK_TFS = 157.3     # MI355X dense fp32 matrix peak, published
F16_MFMA_PEAK_TFS = 2500.0     # MI355X dense fp16 matrix peak, published (no sparsity)
# workload -> (synthetic workload, step kind)
MODES = {
    "gqa_decode": ("gqa_decode", "decode"),
    "long_3bit": ("long_3bit", "decode"),
    "qjl": ("qjl", "decode"),
    "prefill_append": ("prefill_append", "append"),
    "qjl_build": ("qjl", "append"),
    "dequant_layer": ("prefill_append", "dequant"),
    "k3v4_nc": ("k3v4_nc", "decode"),
    "k3qjl_v2": ("k3qjl_v2", "decode"),
    "k8v4": ("k8v4", "decode"),
    "turbo8v3": ("turbo8v3", "decode"),
    "polar3": ("polar3", "decode"),
    "gqa_d64": ("gqa_d64", "decode"),
    "gqa_d256": ("gqa_d256", "decode"),
    "gqa_group8": ("gqa_group8", "decode"),
}


def generic_workloads(synth):
    """The GQA shape at head_dim 64 / 256 (the generic path) and with 8 query heads per KV head."""
    import dataclasses
    g = synth.WORKLOADS["gqa_decode"]
    return {"gqa_d64": dataclasses.replace(g, name="gqa_d64", head_dim=64),
            "gqa_d256": dataclasses.replace(g, name="gqa_d256", head_dim=256),
            "gqa_group8": dataclasses.replace(g, name="gqa_group8", num_kv_heads=2, num_q_heads=16)}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def counter_traffic(kernel_key: str, source: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source (else None)."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        data = json.load(open(path))
    except (OSError, ValueError):
        return None
    rec = data.get(kernel_key)
    if not rec:
        return None
    digest = hashlib.sha256(open(os.path.join(ROOT, "kv_cache_vector_randomized_amd", "csrc", source), "rb").read()).hexdigest()
    return rec.get("bytes_per_launch") if rec.get("source_sha256") == digest else None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=4, help="independent layer caches rotated over the steps")
    ap.add_argument("--workload", default="prefill_append", choices=list(MODES))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--separate", action="store_true",
                    help="decode workloads: append and decode as two launches instead of one")
    ap.add_argument("--dequant-f32", action="store_true", help="dequant_layer: fp32 output instead of bf16")
    ap.add_argument("--eager", action="store_true",
                    help="launch every step from Python instead of replaying a HIP graph of the steps")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="also run one plain device-to-device copy of this many MiB (counter calibration)")
    ap.add_argument("--no-stream-ceilings", action="store_true",
                    help="skip the plain read, write and copy streams of the dominant kernel's byte counts")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path.",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from kv_cache_vector_randomized_amd import synth, tq
    from kv_cache_vector_randomized_amd.torch_api import PagedKVCache, bf16_from_bits

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    torch.cuda.init()
    wname, kind = MODES[args.workload]
    w = generic_workloads(synth).get(wname) or synth.WORKLOADS[wname]
    B, T, Hkv, Hq, d = w.batch, w.context, w.num_kv_heads, w.num_q_heads, w.head_dim
    generic = d != 128
    cfg = tq.make_config(d, Hkv, Hq, w.key_bits, w.key_mode, w.val_bits, w.val_mode)
    S = synth.qjl_matrix(d) if w.key_mode == "lloyd_qjl" else None
    ctx = tq.Context(cfg, synth.sign_vector(w.seed, d), S)
    lay = synth.paged_layout(B, [T] * B, w.seed)
    scale = 1.0 / math.sqrt(d)
    log(f"[bench] workload={args.workload} B={B} T={T} Hkv={Hkv} Hq={Hq} page_bytes={ctx.page_bytes}")

    t0 = time.time()
    k_all = synth.kv_tensor(w, B * T, "k")
    v_all = synth.kv_tensor(w, B * T, "v")
    q_np = synth.query_tensor(w)
    log(f"[bench] generated inputs in {time.time() - t0:.1f}s")
    k_dev = bf16_from_bits(k_all)
    v_dev = bf16_from_bits(v_all)
    q_dev = bf16_from_bits(q_np)
    slots_all = torch.from_numpy(np.concatenate([lay.slots(b, 0, T) for b in range(B)])).cuda()
    tables = torch.from_numpy(lay.block_tables).cuda()
    seq_lens = torch.from_numpy(lay.seq_lens).cuda()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    last = torch.tensor([b * T + T - 1 for b in range(B)], device="cuda")
    k_new = k_dev[last].contiguous()
    v_new = v_dev[last].contiguous()
    slots_new = slots_all[last].contiguous()

    th = ctx.layout.token_head_bytes
    second = None          # a second kernel with a roofline of its own (the append workloads' decode)
    n_layers = max(1, args.layers)
    caches = [PagedKVCache(ctx, lay.num_blocks) for _ in range(n_layers)]
    stream = torch.cuda.current_stream()
    decode_bytes = B * Hkv * T * th + B * Hq * d * 2 + B * Hq * d * 4 + lay.block_tables.nbytes + B * 4

    if kind == "decode":
        for c in caches:                               # prefill every layer (not timed)
            c.append(k_dev, v_dev, slots_all)
        torch.cuda.synchronize()
        del k_dev, v_dev
        append_bytes = B * Hkv * (2 * d * 2 + th) + B * 8
        dom_rw = (decode_bytes + append_bytes - B * Hkv * th, B * Hkv * th + B * Hq * d * 4)
        if args.separate:
            dominant, dom_bytes, dom_source = "decode_kernel", decode_bytes, "tq_decode.hip"
            if generic:
                dominant, dom_source = "gen_decode_kernel + gen_merge_kernel", "tq_generic.hip"

            def step(i, ev=None):
                c = caches[i % n_layers]
                c.append(k_new, v_new, slots_new)
                if ev is not None:
                    ev[0].record(stream)
                c.decode(q_dev, tables, seq_lens, T, scale, out=out)
                if ev is not None:
                    ev[1].record(stream)

            def dom(i):
                caches[i % n_layers].decode(q_dev, tables, seq_lens, T, scale, out=out)
        else:
            # one launch: the decode kernel also quantizes and stores the new tokens
            # (their slots are those of position T-1 in the block tables)
            dominant, dom_bytes, dom_source = "decode_kernel (fused append)", decode_bytes + append_bytes, "tq_decode.hip"
            if generic:
                dominant = "gen_append_kernel + gen_decode_kernel + gen_merge_kernel (one-launch step)"
                dom_source = "tq_generic.hip"

            def step(i, ev=None):
                c = caches[i % n_layers]
                if ev is not None:
                    ev[0].record(stream)
                c.append_decode(k_new, v_new, q_dev, tables, seq_lens, T, scale, out=out)
                if ev is not None:
                    ev[1].record(stream)

            def dom(i):
                caches[i % n_layers].append_decode(k_new, v_new, q_dev, tables, seq_lens, T, scale, out=out)
    elif kind == "dequant":
        for c in caches:                               # fill every layer (not timed)
            c.append(k_dev, v_dev, slots_all)
        torch.cuda.synchronize()
        del k_dev, v_dev
        odt = torch.float32 if args.dequant_f32 else torch.bfloat16
        eb = 4 if args.dequant_f32 else 2
        kbuf = torch.empty((B * T, Hkv, d), dtype=odt, device="cuda")
        vbuf = torch.empty_like(kbuf)
        append_bytes = 0
        decode_bytes = B * T * Hkv * (th + 2 * d * eb) + B * T * 8
        dominant, dom_bytes, dom_source = "dequant_kernel", decode_bytes, "tq_dequant.hip"
        dom_rw = (B * T * Hkv * th + B * T * 8, B * T * Hkv * 2 * d * eb)

        def step(i, ev=None):
            c = caches[i % n_layers]
            if ev is not None:
                ev[0].record(stream)
            c.dequantize_rows(slots_all, None, kbuf, vbuf)
            if ev is not None:
                ev[1].record(stream)

        def dom(i):
            caches[i % n_layers].dequantize_rows(slots_all, None, kbuf, vbuf)
    else:
        append_bytes = B * T * Hkv * (2 * d * 2 + th) + B * T * 8
        dominant, dom_bytes, dom_source = "append_page_kernel", append_bytes, "tq_append.hip"
        dom_rw = (B * T * Hkv * 2 * d * 2 + B * T * 8, B * T * Hkv * th)
        for c in caches:                               # every layer holds a full cache before timing
            c.append(k_dev, v_dev, slots_all)
        torch.cuda.synchronize()

        def step(i, ev=None):
            c = caches[i % n_layers]
            if ev is not None:
                ev[0].record(stream)
            c.append(k_dev, v_dev, slots_all)
            if ev is not None:
                ev[1].record(stream)
            c.decode(q_dev, tables, seq_lens, T, scale, out=out)

        def dom(i):
            caches[i % n_layers].append(k_dev, v_dev, slots_all)

        def dom_decode(i):
            caches[i % n_layers].decode(q_dev, tables, seq_lens, T, scale, out=out)
        second = ("decode_kernel", decode_bytes, "tq_decode.hip", dom_decode)
    step_bytes = append_bytes + decode_bytes

    if args.copy_calibration_mb:
        src = torch.empty(args.copy_calibration_mb << 20, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    launch_notes = []

    def timed(fn, base):
        """Milliseconds of `steps` calls of fn between one pair of events on the stream.
        With a graph (the default) the calls are captured once, replayed once untimed
        (the graph's upload), then replayed in the timed region: the GPU then runs the
        launches back to back instead of waiting on the Python side between them."""
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g = None
        if not args.eager:
            try:
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(args.steps):
                        fn(base + i)
                g.replay()
                torch.cuda.synchronize()
            except RuntimeError as e:          # timed eagerly instead, and said so in the record
                log(f"[bench] graph capture failed ({e}); launching eagerly")
                launch_notes.append(f"eager (graph capture failed: {e})")
                g = None
                torch.cuda.synchronize()
        if g is None:
            torch.cuda.synchronize()
            a_ev.record(stream)
            for i in range(args.steps):
                fn(base + i)
            b_ev.record(stream)
        else:
            a_ev.record(stream)
            g.replay()
            b_ev.record(stream)
        torch.cuda.synchronize()
        return a_ev.elapsed_time(b_ev)

    # Timed region: exactly `steps` steps, nothing else on the stream.
    ms_step = timed(step, args.warmup) / args.steps
    value = step_bytes / (ms_step * 1e-3) / 1e9

    # Second pass: the dominant kernel alone, `steps` launches back to back between
    # one pair of events on its stream (per-launch event pairs add their own gaps).
    dom_avg = timed(dom, args.warmup + args.steps) / args.steps
    # Third pass: every step with the dominant kernel bracketed by its own events,
    # for the spread of single launches (these include the events' own overhead).
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + 2 * args.steps + i, evs[i])
    torch.cuda.synchronize()
    dom_ms = [a.elapsed_time(b) for a, b in evs]
    achieved = dom_bytes / (dom_avg * 1e-3) / 1e9
    pct = {p: float(np.percentile(dom_ms, p)) * 1e3 for p in (10, 50, 90)}
    log(f"[bench] step {ms_step * 1e3:.1f} us; {dominant} avg {dom_avg * 1e3:.1f} us "
        f"(p10 {pct[10]:.1f}, p50 {pct[50]:.1f}, p90 {pct[90]:.1f}); "
        f"{achieved:.0f} GB/s = {achieved / HBM_PEAK_GBS:.1%} of HBM peak")
    # The QJL cache build also carries its dense contraction: S r for every
    # token-head, 2 d^2 flops of fp32 arithmetic each, priced at the fp32 MFMA peak;
    # the kernel runs it on the f16 MFMA as three products of split operands.
    roof_mfma = None
    if kind == "append" and w.key_mode == "lloyd_qjl":
        flops = 2.0 * d * d * B * T * Hkv
        tf = flops / (dom_avg * 1e-3) / 1e12
        roof_mfma = {"kernel": dominant, "bound": "mfma", "achieved": round(tf, 2), "peak": FP32_MFMA_PEAK_TFS,
                     "unit": "TFLOP/s", "frac": round(tf / FP32_MFMA_PEAK_TFS, 4),
                     "algorithmic_flops_per_launch": flops,
                     "as_run": {"dtype": "f16 MFMA, three split products", "flops": 3 * flops,
                                "peak": F16_MFMA_PEAK_TFS,
                                "frac": round(3 * tf / F16_MFMA_PEAK_TFS, 4)}}
        log(f"[bench] S r contraction: {tf:.1f} TFLOP/s = {tf / FP32_MFMA_PEAK_TFS:.1%} of the fp32 MFMA peak")
    roof2 = None
    if second is not None:
        name2, bytes2, source2, fn2 = second
        avg2 = timed(fn2, args.warmup + 3 * args.steps) / args.steps
        ach2 = bytes2 / (avg2 * 1e-3) / 1e9
        log(f"[bench] {name2} avg {avg2 * 1e3:.1f} us; {ach2:.0f} GB/s = {ach2 / HBM_PEAK_GBS:.1%} of HBM peak")
        roof2 = {"kernel": name2, "bound": "hbm", "achieved": round(ach2, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(ach2 / HBM_PEAK_GBS, 4),
                 "traffic": counter_traffic(args.workload + ":" + name2, source2),
                 "algorithmic_bytes_per_launch": bytes2, "avg_launch_us": round(avg2 * 1e3, 2)}

    # Plain device streams of each roofline kernel's read and write byte counts
    # (outside the timed region): what the memory system gives a kernel that does
    # nothing but read, write or copy, to set the roofline fractions beside.  Like
    # the kernels, the streams rotate over `--layers` buffers, so that sizes below
    # the 256 MB Infinity Cache are not served from it.
    ceilings = None
    if not args.no_stream_ceilings:
        import ctypes
        sl = ctypes.CDLL(os.path.join(ROOT, "kv_cache_vector_randomized_amd", "libtqstream.so"))
        for f in (sl.tqs_read, sl.tqs_write, sl.tqs_copy, sl.tqs_mix):
            f.restype = ctypes.c_int
        P, SZ, U32, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_uint32, ctypes.c_int
        sl.tqs_read.argtypes = [P, SZ, P, I, P]
        sl.tqs_write.argtypes = [P, SZ, U32, I, P]
        sl.tqs_copy.argtypes = [P, P, SZ, I, P]
        sl.tqs_mix.argtypes = [P, P, SZ, I, I, P]
        hs = lambda: torch.cuda.current_stream().cuda_stream   # the capturing stream inside a graph capture
        blocks = 2048                          # 8 work-groups of 256 threads per compute unit
        nrot = n_layers

        def streams(rd, wr, kernel_us, copy=True):
            rd, wr = rd // 16 * 16, max(wr // 16 * 16, 16)
            cp = min(rd, wr) // 16 * 16
            src = torch.ones(nrot * rd // 4, dtype=torch.int32, device="cuda")
            dst = torch.empty(nrot * wr // 4, dtype=torch.int32, device="cuda")
            sink = torch.zeros(4, dtype=torch.int32, device="cuda")
            s0, d0 = src.data_ptr(), dst.data_ptr()
            t_rd = timed(lambda i: sl.tqs_read(s0 + (i % nrot) * rd, rd, sink.data_ptr(), blocks, hs()), 0) / args.steps
            t_wr = timed(lambda i: sl.tqs_write(d0 + (i % nrot) * wr, wr, i & 7, blocks, hs()), 0) / args.steps
            c = {"read_GBs": round(rd / (t_rd * 1e-3) / 1e9, 1), "read_bytes": rd, "read_us": round(t_rd * 1e3, 2),
                 "write_GBs": round(wr / (t_wr * 1e-3) / 1e9, 1), "write_bytes": wr, "write_us": round(t_wr * 1e3, 2)}
            if copy:
                t_cp = timed(lambda i: sl.tqs_copy(s0 + (i % nrot) * rd, d0 + (i % nrot) * wr, cp, blocks, hs()),
                             0) / args.steps
                c.update({"copy_GBs": round(2 * cp / (t_cp * 1e-3) / 1e9, 1), "copy_bytes": 2 * cp})
                # One kernel reading m words for each word it writes (m = ceil(read / write)), the
                # faster of two grid sizes; its rate applied to this kernel's bytes.
                m = -(-rd // wr)
                if m <= 8:
                    n_out = rd // 16 // m
                    best = None
                    for nb in (2048, 8192):
                        t = timed(lambda i: sl.tqs_mix(s0 + (i % nrot) * rd, d0 + (i % nrot) * wr, rd, m, nb, hs()),
                                  0) / args.steps
                        best = t if best is None or t < best else best
                    mix_bytes = n_out * 16 * (m + 1)
                    rate = mix_bytes / (best * 1e-3)
                    c.update({"mixed_GBs": round(rate / 1e9, 1), "mixed_reads_per_write": m,
                              "mixed_bytes": mix_bytes, "mixed_us": round(best * 1e3, 2),
                              "mixed_projected_us": round((rd + wr) / rate * 1e6, 2)})
            c.update({"read_then_write_us": round((t_rd + t_wr) * 1e3, 2), "kernel_us": round(kernel_us, 2)})
            del src, dst, sink
            return c

        ceilings = streams(*dom_rw, dom_avg * 1e3)
        ceilings["ops"] = ("plain streaming kernels (16-byte nontemporal loads/stores, 2048 work-groups of 256): "
                           "read the kernel's read bytes, write its write bytes, copy min of the two; mixed: one "
                           "kernel with plain 16-byte loads and stores reading m words per word written "
                           "(m = ceil(read/write)), the faster of 2048 and 8192 work-groups, its rate applied to "
                           "the kernel's bytes (mixed_projected_us); each rotated over the layer buffers and "
                           "graph-replayed back to back")
        mixed = (f"; mixed {ceilings['mixed_reads_per_write']}:1 {ceilings['mixed_GBs']} GB/s, "
                 f"{ceilings['mixed_projected_us']} us for these bytes") if "mixed_GBs" in ceilings else ""
        log(f"[bench] streams: read {ceilings['read_GBs']} GB/s ({ceilings['read_us']} us), write "
            f"{ceilings['write_GBs']} GB/s ({ceilings['write_us']} us), copy {ceilings['copy_GBs']} GB/s; "
            f"read then write {ceilings['read_then_write_us']} us{mixed} (kernel {dom_avg * 1e3:.1f} us)")
        if roof2 is not None:
            c2 = streams(roof2["algorithmic_bytes_per_launch"], 16, roof2["avg_launch_us"], copy=False)
            roof2["stream_read"] = {k: c2[k] for k in ("read_GBs", "read_bytes", "read_us")}
            log(f"[bench] {roof2['kernel']}: a plain read of its bytes takes {c2['read_us']} us "
                f"({c2['read_GBs']} GB/s; kernel {roof2['avg_launch_us']} us)")

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, kind, k_all, v_all, q_np, lay, np)

    rec = {
        "metric": "packed-KV GB/s (% HBM peak) for quantize-append and decode attention",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("bf16 in; f64 (new-token append), f32 (decode)" if generic else
                  {"append": "bf16 in; fp32 (append), f16x3/i8 MFMA + fp32 (decode)",
                   "decode": "bf16 in; f16x3/i8 MFMA + fp32 (decode and new-token append)",
                   "dequant": "fp32 (bf16 or fp32 out)"}[kind]),
        "arithmetic": ("generic path: append with the rotation, norms, codes and values in fp64; decode with "
                       "fp32 dot products (one token per lane), softmax and value sums in fp32"
                       if generic else
                       "append: bf16 inputs, rotation on the bf16 MFMA with fp32 sums, codes decided in fp32, "
                       "stored norms from fp64 sums; decode: logits on the f16 MFMA with the query and centroids "
                       "split into f16 terms (about 22 significant bits), value sums on the int8 MFMA with "
                       "fixed-point weights, softmax and accumulation in fp32"),
        "data": "synthetic (seeded; bf16 N(0,1) K/V with outlier channels, N(0,1) queries)",
        "config": {
            "workload": args.workload, "batch": B, "context": T, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": d, "key_bits": w.key_bits, "key_mode": w.key_mode, "val_bits": w.val_bits,
            "val_mode": w.val_mode, "block_tokens": 16, "layer_caches": n_layers,
            "step": ("append 1 token/seq + decode" + (" (two launches)" if args.separate else " (one launch)")
                     if kind == "decode" else "append all tokens + decode" if kind == "append" else
                     "reconstruct every stored token into a " + ("fp32" if args.dequant_f32 else "bf16") + " buffer"),
            "step_bytes": step_bytes,
        },
        "hbm_fraction": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": {"decode_queries": round(B / (ms_step * 1e-3), 1),
                         "context_token_heads": round(B * T * Hkv / (ms_step * 1e-3), 1)},
        "roofline": {
            "kernel": dominant,
            "bound": "hbm",
            "achieved": round(achieved, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": counter_traffic(args.workload + ":" + dominant, dom_source),
            "algorithmic_bytes_per_launch": dom_bytes,
            "avg_launch_us": round(dom_avg * 1e3, 2),
            "p10_p50_p90_us": [round(pct[10], 2), round(pct[50], 2), round(pct[90], 2)],
        },
        "roofline_decode": roof2,
        "roofline_mfma": roof_mfma,
        "stream_ceilings": ceilings,
        "cpu_baseline": cpu,
        "launch": ("eager" if args.eager else "; ".join(launch_notes) if launch_notes
                   else "hip graph of the timed steps (replayed once untimed first)"),
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(w, kind, k_all, v_all, q_np, lay, np):
    """The fp64 oracle (untuned) on a bounded sample of the same step, about 10 s of
    CPU work: one sequence's new-token quantize-append plus its decode attention
    over its context (for the append workloads: the quantize-append of 16384 of
    the step's tokens; dequant_layer: the reconstruction of 16384 tokens)."""
    from oracle import tq_oracle as O
    from kv_cache_vector_randomized_amd import synth
    cores = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    T, Hkv, Hq, d = w.context, w.num_kv_heads, w.num_q_heads, w.head_dim
    cfg = O.Config(d, Hkv, Hq, w.key_bits, w.key_mode, w.val_bits, w.val_mode)
    signs = synth.sign_vector(w.seed, d)
    kcb = O.codebook(w.key_bits, d) if w.key_mode != "fp8" else None   # FP8 keys have no codebook
    S = synth.qjl_matrix(d).astype(np.float64) if w.key_mode == "lloyd_qjl" else None
    f64 = lambda x: synth.bf16_bits_to_f32(x).astype(np.float64)
    th = O.page_bytes(cfg) // 16
    b = 0
    slots = lay.slots(b, 0, T)
    cache = O.new_cache(cfg, lay.num_blocks)
    if kind == "dequant":
        n = 16384
        O.quantize_append(cfg, cache, f64(k_all[:n]), f64(v_all[:n]), slots[:n], signs, kcb, S=S)
        vcb = O.codebook(w.val_bits, d) if w.val_mode == "lloyd" else None
        times = []
        for _ in range(15):
            t0 = time.perf_counter()
            for h in range(Hkv):
                O.dequantize_slots(cfg, cache, slots[:n], h, signs, kcb, vcb)
            times.append(time.perf_counter() - t0)
        sec = statistics.median(times)
        sample_bytes = n * Hkv * (th + 2 * d * 2) + n * 8
        sample = f"reconstruction of {n} tokens x {Hkv} kv heads (bf16-sized output), median of 15 runs, {sec:.2f} s each"
    elif kind == "append":
        # the step's two halves on the first n tokens of sequence 0: their quantize-append,
        # then decode attention of the sequence's queries over those n tokens
        n = min(16384, T)
        lens_n = np.minimum(lay.seq_lens[b:b + 1], n)
        times = []
        for _ in range(3):
            t0 = time.perf_counter()
            O.quantize_append(cfg, cache, f64(k_all[:n]), f64(v_all[:n]), slots[:n], signs, kcb, S=S)
            O.decode_attention(cfg, f64(q_np[b:b + 1]), cache, lay.block_tables[b:b + 1], lens_n,
                               1.0 / math.sqrt(d), signs, kcb, S=S)
            times.append(time.perf_counter() - t0)
        sec = statistics.median(times)
        sample_bytes = (n * Hkv * (2 * d * 2 + th) + n * 8 + n * Hkv * th + Hq * d * 2 + Hq * d * 4
                        + (n // 16) * 4 + 4)
        sample = (f"quantize-append of {n} tokens x {Hkv} kv heads, then decode of {Hq} q heads over those {n} "
                  f"tokens, median of 3 runs, {sec:.2f} s each")
    else:
        t0 = time.time()
        O.quantize_append(cfg, cache, f64(k_all[: T - 1]), f64(v_all[: T - 1]), slots[: T - 1], signs, kcb, S=S)
        log(f"[cpu] oracle prefill of the sample sequence took {time.time() - t0:.1f}s (not timed)")
        times = []
        for _ in range(25):
            t0 = time.perf_counter()
            O.quantize_append(cfg, cache, f64(k_all[T - 1:T]), f64(v_all[T - 1:T]), slots[T - 1:T], signs, kcb, S=S)
            O.decode_attention(cfg, f64(q_np[b:b + 1]), cache, lay.block_tables[b:b + 1], lay.seq_lens[b:b + 1],
                               1.0 / math.sqrt(d), signs, kcb, S=S)
            times.append(time.perf_counter() - t0)
        sec = statistics.median(times)
        sample_bytes = (Hkv * (2 * d * 2 + th) + 8 + Hkv * T * th + Hq * d * 2 + Hq * d * 4
                        + lay.block_tables.shape[1] * 4 + 4)
        sample = (f"one sequence of the step (append 1 token x {Hkv} kv heads, decode {Hq} q heads over {T} "
                  f"tokens), median of 25 runs, {sec:.2f} s each")
    log(f"[cpu] oracle sample {sec:.2f}s -> {sample_bytes / sec / 1e9:.4f} GB/s")
    return {"value": round(sample_bytes / sec / 1e9, 5), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "sample": sample}


if __name__ == "__main__":
    main()
