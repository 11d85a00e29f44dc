#!/usr/bin/env python3
"""Decode-step benchmark of the Kitty 2-bit KV cache on one MI355X.

A step is one decode step of one attention layer over the whole batch:
``kitty_decode_step``, one launch that stores the new token in the fp16
tail (sealing the tail into a quantized page every 32nd token: channel
statistics, ranking, codes, two-plane packing) and runs the fused decode
attention (dequant + QK + online softmax + PV over all pages, then the
split merge).  ``--split`` times the two separate calls instead
(``kitty_append_token`` then ``kitty_decode_attention``).

Workload (default): the memory-budget batch sweep at its largest point --
batch 128, 32 query heads, 8 KV heads, head_dim 128, context 8192,
hi_fraction 0.25, seeded synthetic fp16 K/V/Q (880.8 MB of quantized KV read
per step).  The default run also times the Llama-3-8B-shape step (batch 16,
context 4096) and a read-only kernel over 2 GiB (the read-stream ceiling),
reported beside the headline as context.  ``--workload`` / ``--batch``
select another configuration; ``--lo-bit 4`` runs the (hi_bit 8, lo_bit 4)
pair instead of (4, 2); ``--rank-mode running`` the running-variance ranking
instead of per-page ranking; ``--ceiling`` times only the read-only kernels
over a sweep of launch shapes, and the prefill quantizer's read-and-write
stream without its arithmetic.
To keep reads coming from HBM rather than the 256 MB Infinity Cache, the
steps rotate over L independent layer caches totalling >= 1 GiB.

Steps are replayed from HIP graphs (L steps per graph), so host launch
overhead stays off the GPU timeline.

Printed: one JSON line (metric, value = GB/s of quantized KV read per step,
tokens/s, a roofline object for the decode kernel measured with HIP events
on the launch stream, and the CPU oracle timed on a bounded sample).
"""
import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, published
METRIC = "2-bit-KV decode attention: GB/s KV read vs HBM peak; tokens/s at batch×ctx"


def _workload(name):
    from mixed_precision_bit_kitty_amd import synth
    table = {"llama3_8b": synth.LLAMA3_8B, "qwen3_8b": synth.QWEN3_8B, "batch_sweep": synth.BATCH_SWEEP,
             "prefill_sweep": synth.PREFILL_SWEEP, "tiny": synth.TINY}
    return table[name]


def kv_bytes(seq_lens, n_kv_heads, record_bytes):
    """Algorithmic KV bytes one decode call reads: every sealed page record
    (3072 + 9 n_hi bytes per page and KV head at lo_bit 2, 5120 + 17 n_hi at
    lo_bit 4) plus the fp16 tail tokens (2 x 256 bytes per token and KV
    head)."""
    tot = 0
    for n in seq_lens:
        tot += n_kv_heads * ((n // 32) * record_bytes + (n % 32) * 512)
    return tot


DECODE_SOURCES = ("decode.hip", "page_quant.h", "kitty_internal.h")  # the fused step seals with page_quant.h
QUANTIZE_SOURCES = ("quantize.hip", "page_quant.h", "kitty_internal.h")


def code_text(text):
    """Source text without comments, blank lines and trailing spaces: what
    the compiler sees of it (string literals here hold no comment markers)."""
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = (re.sub(r"//.*", "", l).rstrip() for l in text.splitlines())
    return "\n".join(l for l in lines if l)


def source_hash(files=DECODE_SOURCES, read=None, flags=None):
    """Hash of the kernel sources' code (comments ignored) and of their own
    compile flags (the build's per-file flags; `flags` maps a file to its
    flags in place of those), naming the kernel build that committed counter
    summaries were taken on."""
    if flags is None:
        from mixed_precision_bit_kitty_amd import build as kbuild
        flags = kbuild.SOURCES
    h = hashlib.sha256()
    for f in files:
        if read is None:
            with open(os.path.join(ROOT, "mixed_precision_bit_kitty_amd", "csrc", f)) as fh:
                text = fh.read()
        else:
            text = read(f)
        h.update(code_text(text).encode())
        if f in flags:
            h.update(("\0" + " ".join(flags[f])).encode())
    return h.hexdigest()[:16]


def committed_traffic(kernel_hash, workload, entry, kernel="decode_kernel"):
    """HBM bytes per launch from the committed rocprofv3 counter summary of
    that kernel and entry point (decode: "step" or "attention") on this
    workload, if it was taken on the current kernel source; else None."""
    name = f"{kernel}_{entry}_{workload}" if entry else f"{kernel}_{workload}"
    path = os.path.join(ROOT, "profiles", f"{name}_hbm_counters.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_hash:
        return None
    return d.get("hbm_bytes_per_launch")


def _oracle_decode_rate(w, seconds, lo_bit, rank_mode, threads):
    """Decode steps (append + attention) of the oracle on 2 sequences of the
    workload for about `seconds`, with the BLAS pool limited to `threads`
    (None: its default).  Returns (steps, sequences, bytes read, seconds,
    threads used)."""
    import oracle as O
    from mixed_precision_bit_kitty_amd import synth
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
        limiter = threadpool_limits(threads)
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except ImportError:  # pragma: no cover
        limiter, used = None, threads or 1
    n_seq = 2
    x = synth.batch(w, batch=n_seq, steps=64)
    oc = O.quantize_pages(x["k"], x["v"], w.n_hi, lo_bit=lo_bit, rank_mode=rank_mode)
    rec = O.record_bytes(w.n_hi, lo_bit=lo_bit)
    t0 = time.perf_counter()
    steps = 0
    read = 0
    while True:
        t = steps % 64
        O.append_token(oc, x["k_new"][t], x["v_new"][t])
        O.decode_attention(oc, x["q_new"][t])
        read += kv_bytes([int(n) for n in oc.seq_len], w.n_kv_heads, rec)
        steps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    if limiter is not None:
        limiter.unregister()
    return steps, n_seq, read, el, used


def cpu_baseline(w, seconds, lo_bit=2, rank_mode="page"):
    """The oracle as it stands on a bounded sample of the same workload:
    decode steps (append + attention) on 2 of the sequences, single-threaded
    (the reported value) and with the BLAS pool at its default size (all
    host threads; context)."""
    steps, n_seq, read, el, _ = _oracle_decode_rate(w, seconds, lo_bit, rank_mode, 1)
    s2, _, r2, e2, used = _oracle_decode_rate(w, seconds, lo_bit, rank_mode, None)
    return {"value": round(read / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "tokens_per_s": round(steps * n_seq / el, 3),
            "sample": f"{steps} decode steps (append + attention) of {n_seq} of the {w.batch} sequences, "
                      f"ctx {w.ctx}, numpy oracle single-threaded, {el:.1f} s",
            "all_threads": {"value": round(r2 / e2 / 1e9, 4), "unit": "GB/s", "cores": used,
                            "tokens_per_s": round(s2 * n_seq / e2, 3),
                            "sample": f"{s2} decode steps, BLAS pool of {used} threads "
                                      f"(os.cpu_count() = {os.cpu_count()}), {e2:.1f} s"}}


def bench_quantize(args, w):
    """Prefill quantization of the whole batch (kitty_quantize_pages): K
    statistics, DCPB ranking, codes, two-plane packing, V codes, tail copy.
    Algorithmic bytes: the fp16 K and V read (512 B per token and KV head)
    plus the records written (rec bytes per page and KV head).  Each
    launch quantizes a different one of R input copies (>= 1 GiB in total),
    so reads come from HBM."""
    import torch
    from mixed_precision_bit_kitty_amd import binding, synth

    torch.cuda.set_device(0)
    B = args.batch or w.batch
    print(f"[bench] generating {w.name} batch {B} ctx {w.ctx}", file=sys.stderr, flush=True)
    x = synth.batch(w, batch=B, steps=0)
    k0 = torch.from_numpy(x["k"]).cuda()
    v0 = torch.from_numpy(x["v"]).cuda()
    del x
    _, Hkv, S, D = k0.shape
    in_bytes = 2 * k0.numel() * 2
    R = max(1, math.ceil((1 << 30) / in_bytes))
    ks = [k0] + [k0.clone() for _ in range(R - 1)]
    vs = [v0] + [v0.clone() for _ in range(R - 1)]
    cache = binding.KittyCache(B, Hkv, w.n_hi, S + 32, lo_bit=args.lo_bit, rank_mode=_rank(args))
    rec = cache.record_bytes
    # the running mode also writes each (sequence, KV head)'s 4 KB of sums
    alg = in_bytes + B * Hkv * (S // 32) * rec + (B * Hkv * binding.KITTY_KEY_STATS_BYTES if _rank(args) else 0)
    for i in range(R):
        cache.quantize_pages(ks[i], vs[i])
    torch.cuda.synchronize()
    K = args.steps
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(K):
        cache.quantize_pages(ks[i % R], vs[i % R])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / K
    gbs = alg / (ms * 1e-3) / 1e9
    print(f"[bench] quantize_pages {ms * 1e3:.2f} us ({gbs:.0f} GB/s, {gbs / HBM_PEAK_GBS:.3f} of peak), "
          f"{R} input copies", file=sys.stderr, flush=True)
    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)
        del a, bcopy
    khash = source_hash(QUANTIZE_SOURCES)
    res = {"metric": "kitty_quantize_pages: GB/s of fp16 K/V read + page records written", "value": round(gbs, 1),
           "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": R, "ms_per_step": round(ms, 6),
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "fp32", "data": "synthetic",
           "config": {"workload": f"{w.name}: prefill of batch {B}, {Hkv} KV heads, {S} tokens, n_hi {w.n_hi}"
                                  + ("" if args.lo_bit == 2 else f", hi_bit 8 / lo_bit 4")
                                  + ("" if not _rank(args) else ", running-variance ranking"),
                      "batch": B, "ctx": S, "n_kv_heads": Hkv, "n_hi": w.n_hi, "hi_bit": 2 * args.lo_bit,
                      "lo_bit": args.lo_bit, "rank_mode": args.rank_mode, "input_copies": R},
           "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(gbs / HBM_PEAK_GBS, 4),
                        "traffic": committed_traffic(khash, args.workload + _lo_suffix(args), None,
                                                     "quantize_pages_kernel"),
                        "kernel": "quantize_pages_kernel" if not _rank(args) else
                                  "key_stats_kernel + quantize_pages_kernel (one call)",
                        "bytes_per_launch": int(alg),
                        "avg_launch_us": round(ms * 1e3, 3), "kernel_source_sha256_16": khash}}
    print(json.dumps(res), flush=True)


def _lo_suffix(args):
    """Name suffix of the committed counter summaries of the 4-bit pair and
    of a hi_fraction other than the workload's."""
    return (("" if args.lo_bit == 2 else "_lo4") + ("" if args.hi_fraction is None else f"_hf{args.hi_fraction:g}")
            + ("_running" if _rank(args) else ""))


def _rank(args):
    """The ABI's rank_mode value of --rank-mode."""
    return 1 if args.rank_mode == "running" else 0


def _gpu_inputs(w, B, steps):
    """Seeded synthetic inputs of sequences 0..B-1 (the same per-sequence
    streams as synth.batch), with K and V copied to the GPU in chunks so the
    host holds only a few sequences at a time.  Returns (k, v on the GPU;
    k_new, v_new, q_new [steps, B, ...] on the GPU)."""
    import torch
    from concurrent.futures import ThreadPoolExecutor
    from mixed_precision_bit_kitty_amd import synth
    H, D, Hq = w.n_kv_heads, w.head_dim, w.n_q_heads
    kd = torch.empty((B, H, w.ctx, D), dtype=torch.float16, device="cuda")
    vd = torch.empty_like(kd)
    kn = np.empty((steps, B, H, D), np.float16)
    vn = np.empty_like(kn)
    qn = np.empty((steps, B, Hq, D), np.float16)
    chunk = 16
    with ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as ex:
        for b0 in range(0, B, chunk):
            seqs = list(ex.map(lambda b: synth.sequence(w, b, steps=steps), range(b0, min(B, b0 + chunk))))
            for j, x in enumerate(seqs):
                kd[b0 + j].copy_(torch.from_numpy(x["k"]))
                vd[b0 + j].copy_(torch.from_numpy(x["v"]))
                kn[:, b0 + j], vn[:, b0 + j], qn[:, b0 + j] = x["k_new"], x["v_new"], x["q_new"]
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return kd, vd, dev(kn), dev(vn), dev(qn)


def time_decode(args, w, B, K, W, split=False):
    """K timed decode steps (after W untimed ones) of workload w at batch B
    over L rotated layer caches, replayed from HIP graphs.  Returns the step
    time, the decode kernel's own average launch time and the algorithmic
    bytes of both."""
    import torch
    from mixed_precision_bit_kitty_amd import binding

    ctx, Hkv, Hq, n_hi = w.ctx, w.n_kv_heads, w.n_q_heads, w.n_hi
    print(f"[bench] generating {w.name} batch {B} ctx {ctx}", file=sys.stderr, flush=True)
    n_tok = 64
    kd, vd, k_new, v_new, q_new = _gpu_inputs(w, B, n_tok)

    max_tokens = ctx + K + W + 32
    probe = binding.KittyCache(1, Hkv, n_hi, max_tokens, lo_bit=args.lo_bit, rank_mode=_rank(args))
    layer_bytes = B * probe.max_pages * probe.page_bytes
    del probe
    L = args.layers or max(1, math.ceil((1 << 30) / layer_bytes))
    print(f"[bench] {L} layer caches x {layer_bytes / 1e6:.1f} MB", file=sys.stderr, flush=True)
    layers = [binding.KittyCache(B, Hkv, n_hi, max_tokens, lo_bit=args.lo_bit, rank_mode=_rank(args)) for _ in range(L)]
    layers[0].quantize_pages(kd, vd)
    for c in layers[1:]:
        c.pool.copy_(layers[0].pool)
        c.tail_k.copy_(layers[0].tail_k)
        c.tail_v.copy_(layers[0].tail_v)
        c.seq_lens.copy_(layers[0].seq_lens)
        if c.key_stats is not None:
            c.key_stats.copy_(layers[0].key_stats)
    del kd, vd
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    # Every sequence of a layer has the same length.  Layer l takes its steps
    # i = l, l + L, ...; the decode bound max_seq_len is the longest length
    # the layer reaches in this run, so the page split stays balanced.
    per_layer = (K + W + L - 1) // L
    msl = ctx + per_layer + 1
    outs = [torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda") for _ in range(L)]
    ws = [c.workspace(Hq, msl) for c in layers]

    # One HIP graph per layer (one step of layer l) and one graph of L such
    # steps.  The host only replays graphs, so its launch overhead stays off
    # the GPU timeline.
    def step_eager(l, decode_only=False):
        c, t = layers[l], l % n_tok
        if decode_only:
            c.decode_attention(q_new[t], max_seq_len=msl, out=outs[l], workspace=ws[l])
        elif split:
            c.append_token(k_new[t], v_new[t])
            c.decode_attention(q_new[t], max_seq_len=msl, out=outs[l], workspace=ws[l])
        else:
            c.decode_step(k_new[t], v_new[t], q_new[t], max_seq_len=msl, out=outs[l], workspace=ws[l])

    for l in range(L):
        step_eager(l, decode_only=True)  # first launches outside capture
    torch.cuda.synchronize()
    g_step = []
    for l in range(L):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step_eager(l)
        g_step.append(g)
    g_dec = None
    if split:  # the decode of every layer, back to back (the roofline's kernel alone)
        g_dec = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g_dec):
            for l in range(L):
                step_eager(l, decode_only=True)
    # L consecutive steps (one per layer, in the order the timed loop takes
    # them) in one graph, so the host replays once per L steps
    r0 = W % L
    g_round = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g_round):
        for j in range(L):
            step_eager((r0 + j) % L)
    torch.cuda.synchronize()

    lens = [ctx] * L
    for i in range(W):
        g_step[i % L].replay()
        lens[i % L] += 1
    torch.cuda.synchronize()

    # Graph replays run on torch's current stream, which the events below
    # are recorded on: they bracket exactly the launches of the timed steps.
    rec = layers[0].record_bytes
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(K // L):
        g_round.replay()
    for i in range(K - K % L, K):
        g_step[(W + i) % L].replay()
    end.record()
    torch.cuda.synchronize()
    bytes_steps = []
    for i in range(K):
        li = (W + i) % L
        lens[li] += 1
        bytes_steps.append(kv_bytes([lens[li]] * B, Hkv, rec))
    ms_step = start.elapsed_time(end) / K
    avg_bytes = sum(bytes_steps) / K

    if g_dec is None:
        # The fused step is one decode-kernel launch per step: the timed
        # region is K launches of that kernel back to back.
        dec_ms, dec_bytes = ms_step, avg_bytes
        kernel = "decode_kernel (kitty_decode_step)"
    else:
        # The decode kernel alone: R replays of one graph holding the decode
        # of every layer back to back (R * L launches on one stream), timed
        # with events over the whole region.
        R = max(1, K // L)
        dec_bytes = sum(kv_bytes([n] * B, Hkv, rec) for n in lens) / L
        torch.cuda.synchronize()
        start.record()
        for _ in range(R):
            g_dec.replay()
        end.record()
        torch.cuda.synchronize()
        dec_ms = start.elapsed_time(end) / (R * L)
        kernel = "decode_kernel (kitty_decode_attention)"
    gbs = avg_bytes / (ms_step * 1e-3) / 1e9
    dec_gbs = dec_bytes / (dec_ms * 1e-3) / 1e9
    print(f"[bench] {w.name} batch {B}: step {ms_step * 1e3:.2f} us ({gbs:.0f} GB/s), decode kernel "
          f"{dec_ms * 1e3:.2f} us ({dec_gbs:.0f} GB/s, {dec_gbs / HBM_PEAK_GBS:.3f} of peak)", file=sys.stderr, flush=True)
    del g_step, g_dec, g_round, layers, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return {"ms_step": ms_step, "gbs": gbs, "bytes": avg_bytes, "dec_ms": dec_ms, "dec_gbs": dec_gbs,
            "dec_bytes": dec_bytes, "kernel": kernel, "layers": L, "layer_bytes": layer_bytes}


CEILING_DEFAULT = (0, 8, 4)  # mode, waves per CU, loads in flight per lane: the best of the sweep on MI355X
CEILING_SWEEP = [(0, w, d) for w in (8, 16, 32) for d in (2, 4, 8)] + \
                [(1, w, d) for w in (8, 12) for d in (2, 3, 4) if w * d * 3360 <= 160 * 1024]


def read_ceiling(configs, gib=2, reps=10):
    """GB/s of the read-only kernels over `gib` GiB: per (mode, waves per
    CU, depth), the average of `reps` launches timed with HIP events on the
    launch stream (after one untimed launch)."""
    import torch
    from mixed_precision_bit_kitty_amd import binding
    lib = binding.load_bench()
    nbytes = gib << 30
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    out = []
    for mode, waves, depth in configs:
        used = nbytes if mode == 0 else nbytes // 3360 * 3360

        def launch():
            rc = lib.kitty_read_ceiling(src.data_ptr(), nbytes, mode, waves, depth, sink.data_ptr(), sink.numel(),
                                        stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"kitty_read_ceiling({mode}, {waves}, {depth}) returned {rc}")
        launch()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(reps):
            launch()
        end.record()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / reps
        gbs = used / (ms * 1e-3) / 1e9
        name = ("read_vgpr_kernel" if mode == 0 else "read_lds_kernel") + f"<{depth}>"
        print(f"[bench] ceiling {name}, {waves} waves/CU: {ms * 1e3:.1f} us per {used / 2**30:.2f} GiB, "
              f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of peak)", file=sys.stderr, flush=True)
        out.append({"kernel": name, "mode": "registers" if mode == 0 else "lds_records", "waves_per_cu": waves,
                    "depth": depth, "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                    "us": round(ms * 1e3, 2), "bytes": used})
    del src, sink
    torch.cuda.empty_cache()
    return out


def stream_ceiling(gib=2, read_unit=16384, write_unit=3360, reps=10):
    """GB/s (read + written bytes) of the prefill quantizer's traffic without
    its arithmetic: one block per 16 KiB unit (a page-head's fp16 K and V)
    that writes a 3360-byte record-sized output (kitty_stream_ceiling), over
    `gib` GiB read; the average of `reps` launches timed with HIP events on
    the launch stream (after one untimed launch)."""
    import torch
    from mixed_precision_bit_kitty_amd import binding
    lib = binding.load_bench()
    units = (gib << 30) // read_unit
    src = torch.empty(units * read_unit, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty(units * write_unit, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def launch():
        rc = lib.kitty_stream_ceiling(src.data_ptr(), dst.data_ptr(), units, read_unit, write_unit, stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"kitty_stream_ceiling returned {rc}")
    launch()
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for _ in range(reps):
        launch()
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    moved = units * (read_unit + write_unit)
    gbs = moved / (ms * 1e-3) / 1e9
    print(f"[bench] stream ceiling stream_kernel<{read_unit // 2048}>: {ms * 1e3:.1f} us per {units} units "
          f"({read_unit} B read + {write_unit} B written each), {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of peak)",
          file=sys.stderr, flush=True)
    del src, dst
    torch.cuda.empty_cache()
    return {"kernel": f"stream_kernel<{read_unit // 2048}>", "units": units, "read_bytes": read_unit,
            "write_bytes": write_unit, "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
            "us": round(ms * 1e3, 2), "bytes": moved}


def record_stream_at_size(n_records, waves=12, depth=2, gib=2, reps=20, heads_order=False):
    """The record stream alone (read_lds_kernel: 3360-byte records through a
    per-wave LDS ring, one workgroup per CU as decode runs) at a decode
    workload's size: each launch reads a different slice of `n_records`
    records of a `gib` GiB buffer, so no launch finds its slice in the
    256 MB Infinity Cache; the average of `reps` launches timed with HIP
    events after one untimed launch.  The fixed costs of a launch (the first
    records' latency, the drain) show against the bytes.  heads_order: the
    records in the decode kernel's order (8 interleaved per-head streams, a
    wave reading records 8 apart; KITTY_READ_LDS_HEADS)."""
    import torch
    from mixed_precision_bit_kitty_amd import binding
    lib = binding.load_bench()
    nbytes = n_records * 3360
    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    buf.fill_(1)
    nslices = (gib << 30) // nbytes
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()

    def launch(i):
        rc = lib.kitty_read_ceiling(buf.data_ptr() + (i % nslices) * nbytes, nbytes, 2 if heads_order else 1, waves,
                                    depth, sink.data_ptr(), sink.numel(), stream.cuda_stream)
        if rc != 0:
            raise RuntimeError(f"kitty_read_ceiling returned {rc}")
    launch(nslices - 1)
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    start.record()
    for i in range(reps):
        launch(i)
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / reps
    gbs = nbytes / (ms * 1e-3) / 1e9
    order = ", heads order" if heads_order else ""
    print(f"[bench] record stream read_lds_kernel<{depth}>{order}, {waves} waves/CU: {ms * 1e3:.2f} us per {n_records} records "
          f"({nbytes / 1e6:.1f} MB), {gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f} of peak)", file=sys.stderr, flush=True)
    del buf, sink
    torch.cuda.empty_cache()
    return {"kernel": f"read_lds_kernel<{depth}>", "order": "heads" if heads_order else "contiguous",
            "waves_per_cu": waves, "records": n_records, "bytes": nbytes,
            "us": round(ms * 1e3, 2), "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4)}


# record counts of the decode workloads (page-heads per launch): llama3_8b
# (16 x 8 x 128), qwen3_8b (4 x 8 x 1024), batch_sweep at batch 16 and 128
RECORD_SIZES = {"llama3_8b": 16384, "qwen3_8b": 32768, "batch_sweep_b16": 32768, "batch_sweep_b128": 262144}


def bench_ceiling(args):
    res = read_ceiling(CEILING_SWEEP)
    sized = {k: record_stream_at_size(n) for k, n in RECORD_SIZES.items()}
    sized["batch_sweep_b128_heads_order"] = record_stream_at_size(RECORD_SIZES["batch_sweep_b128"], heads_order=True)
    best = max(res, key=lambda r: r["gbs"])
    best_lds = max((r for r in res if r["mode"] == "lds_records"), key=lambda r: r["gbs"])
    stream = stream_ceiling()
    if args.calibrate_copy:
        import torch
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)
        del a, bcopy
    print(json.dumps({"metric": "HBM read-stream ceiling: GB/s of read-only kernels over 2 GiB",
                      "value": best["gbs"], "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
                      "frac_of_hbm_peak": best["frac"], "best": best, "best_lds_records": best_lds,
                      "sweep": res, "read_write_stream": stream, "record_stream_at_size": sized}), flush=True)


def _workload_key(args, w, B):
    """Name of a configuration in the committed counter summaries."""
    group = "" if args.q_heads is None else f"_g{w.n_q_heads // w.n_kv_heads}"
    return args.workload + ("" if B == w.batch else f"_b{B}") + group + _lo_suffix(args)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="batch_sweep",
                    choices=["llama3_8b", "qwen3_8b", "batch_sweep", "prefill_sweep", "tiny"])
    ap.add_argument("--batch", type=int, default=None,
                    help="override the workload's batch (default: 128 for batch_sweep, the sweep's largest point)")
    ap.add_argument("--layers", type=int, default=0, help="layer caches to rotate (0: enough for >= 1 GiB)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the extra llama3_8b step and read-ceiling measurements of the default run")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one 1 GiB device copy (HBM counter calibration under rocprofv3)")
    ap.add_argument("--split", action="store_true",
                    help="step = kitty_append_token + kitty_decode_attention (two launches) instead of the fused step")
    ap.add_argument("--lo-bit", type=int, default=2, choices=[2, 4],
                    help="bit-width pair: 2 = (hi_bit 4, lo_bit 2), 4 = (hi_bit 8, lo_bit 4)")
    ap.add_argument("--rank-mode", default="page", choices=["page", "running"],
                    help="boosted channels by each page's variance (page) or the head's running variance (running)")
    ap.add_argument("--q-heads", type=int, default=None,
                    help="override the workload's query heads (a multiple of its KV heads: GQA group = q_heads / kv_heads)")
    ap.add_argument("--hi-fraction", type=float, default=None,
                    help="override the workload's hi_fraction (n_hi = hi_fraction x 128)")
    ap.add_argument("--quantize", action="store_true",
                    help="time kitty_quantize_pages (prefill of the whole batch) instead of the decode step")
    ap.add_argument("--ceiling", action="store_true",
                    help="time only the read-only kernels (HBM read-stream ceiling) over a sweep of launch shapes, "
                         "and the prefill quantizer's read-and-write stream without its arithmetic")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import torch
    from mixed_precision_bit_kitty_amd import binding  # noqa: F401  (fails loudly without the library)

    torch.cuda.set_device(0)
    if args.ceiling:
        return bench_ceiling(args)
    w = _workload(args.workload)
    if args.hi_fraction is not None:
        w = w.with_(hi_fraction=args.hi_fraction)
    if args.q_heads is not None:
        if args.q_heads < w.n_kv_heads or args.q_heads % w.n_kv_heads:
            ap.error(f"--q-heads must be a positive multiple of the workload's {w.n_kv_heads} KV heads")
        w = w.with_(n_q_heads=args.q_heads)
    if args.quantize:
        return bench_quantize(args, w)
    B = args.batch or (max(w.sweep) if args.workload == "batch_sweep" else w.batch)
    K, W = args.steps, args.warmup
    r = time_decode(args, w, B, K, W, split=args.split)
    ctx, Hkv, Hq, n_hi = w.ctx, w.n_kv_heads, w.n_q_heads, w.n_hi

    if args.calibrate_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        bcopy = torch.empty_like(a)
        bcopy.copy_(a)
        torch.cuda.synchronize()
        print("[bench] calibration copy: 1 GiB read + 1 GiB written", file=sys.stderr, flush=True)
        del a, bcopy

    khash = source_hash(DECODE_SOURCES)
    roof = {"bound": "hbm", "achieved": round(r["dec_gbs"], 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(r["dec_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": committed_traffic(khash, _workload_key(args, w, B), "attention" if args.split else "step"),
            "kernel": r["kernel"],
            "bytes_per_launch": int(r["dec_bytes"]), "avg_launch_us": round(r["dec_ms"] * 1e3, 3),
            "kernel_source_sha256_16": khash}
    L = r["layers"]
    res = {
        "metric": METRIC if args.lo_bit == 2 else METRIC.replace("2-bit-KV", "4-bit-KV (hi_bit 8, lo_bit 4)"),
        "value": round(r["gbs"], 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(r["ms_step"], 6), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16", "data": "synthetic",
        "tokens_per_s": round(B / (r["ms_step"] * 1e-3), 1),
        "frac_of_hbm_peak": round(r["gbs"] / HBM_PEAK_GBS, 4),
        "config": {"workload": f"{w.name}: one layer, batch {B}, {Hq} query heads, {Hkv} KV heads, head_dim 128, "
                               f"context {ctx}+, hi_fraction {w.hi_fraction} (n_hi {n_hi}), "
                               f"hi_bit {2 * args.lo_bit} / lo_bit {args.lo_bit}, {args.rank_mode} ranking; step = "
                               f"{'append + decode (two launches)' if args.split else 'fused append + decode (one launch)'} "
                               f"(replayed from HIP graphs of {L} steps); {L} layer caches rotated "
                               f"({L * r['layer_bytes'] / 2**30:.2f} GiB)",
                   "batch": B, "ctx": ctx, "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": 128, "n_hi": n_hi,
                   "hi_bit": 2 * args.lo_bit, "lo_bit": args.lo_bit, "rank_mode": args.rank_mode, "layers_rotated": L},
        "roofline": roof,
    }
    default_run = (args.workload == "batch_sweep" and args.batch is None and not args.split and args.lo_bit == 2
                   and args.rank_mode == "page" and args.hi_fraction is None and args.q_heads is None)
    if default_run and not args.no_context:
        # context beside the headline: the Llama-3-8B-shape step and the read-only ceiling
        wl = _workload("llama3_8b")
        r2 = time_decode(args, wl, wl.batch, K, W)
        res["llama3_8b_b16_ctx4096"] = {
            "ms_per_step": round(r2["ms_step"], 6), "value": round(r2["gbs"], 1), "unit": "GB/s",
            "frac_of_hbm_peak": round(r2["gbs"] / HBM_PEAK_GBS, 4), "bytes_per_step": int(r2["bytes"]),
            "tokens_per_s": round(wl.batch / (r2["ms_step"] * 1e-3), 1),
            "traffic": committed_traffic(khash, "llama3_8b", "step")}
        c = read_ceiling([CEILING_DEFAULT])[0]
        res["read_ceiling"] = c
        # the same number of records streamed alone (no arithmetic), and the
        # headline's share of that rate
        n_rec = B * Hkv * (ctx // 32) if args.lo_bit == 2 and n_hi == 32 else None
        if n_rec:
            rs = record_stream_at_size(n_rec)
            rs["headline_share"] = round(r["gbs"] / rs["gbs"], 4)
            res["record_stream_same_size"] = rs
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(w.with_(batch=B), args.cpu_seconds, args.lo_bit, args.rank_mode)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
