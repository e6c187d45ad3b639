"""Benchmark of quantized-KV decode attention on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--gpus 1]

A step is one decode step of the whole hot path: for every layer, append the
new token's K and V (fp16 tail, a key-group flush every G steps) and run
decode attention over the packed cache.  Default workload: 32 layers x 32
heads x head_dim 128 at 1,048,576 tokens of context, K and V at 2 bits (K per
channel in 128-token groups, V per token in 32-channel groups), an fp16 sink
token and a 128-token fp16 tail; the cache (90 GB) is built on the device
from the counter-based synthetic generator.  The 4096-token prefill append
into every layer is timed separately.

Prints one JSON line.  `value` is whole-job algorithmic HBM throughput in
GB/s: the bytes one step must read (packed codes, float32 scales, fp16 sink
and tail rows, queries) over the step time; `roofline` relates the decode
call's bytes to its HIP-event time; `cpu_baseline` times the CPU oracle's
decode (dequant to float64 + float64 attention) on a bounded sample, on one
core and on every core the process may use.  With the default workload the
line also carries `workloads`: the 4K-context 7B-style layer, the 128K GQA
layer (K4V2 and K2V4) and the MixKVQ 32K x 8 batch, each timed the same way
(per decode call, the Infinity Cache evicted before each step) next to a
streaming read of the same number of bytes.
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

import synth

PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="1m_32layer",
                    choices=["1m_32layer", "gqa_128k", "gqa_128k_k2v4",
                             "mixkvq_32k", "7b_layer_4k",
                             "kvquant_3bit_1pct_128k", "kqv_4bit_128k"])
    ap.add_argument("--layers", type=int, default=None,
                    help="layers of the 1m_32layer workload (default 32)")
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="default workload only: skip the sub-records of the "
                         "other workloads")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 3 times (a "
                         "known-size kernel to scale FETCH_SIZE/WRITE_SIZE)")
    return ap.parse_args()


def calibrate_copy(mib):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": n, "launches": 3}), flush=True)


def measured_traffic(workload):
    """Calibrated HBM bytes per decode launch from the committed rocprofv3
    record (profiles/decode_traffic.json), or None if the decode sources
    changed since the counters were taken."""
    import hashlib
    root = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(root, "profiles", "decode_traffic.json")
    try:
        rec = json.load(open(path))
        h = hashlib.sha256()
        for src in rec["sources"]:
            h.update(open(os.path.join(root, src), "rb").read())
        if h.hexdigest() != rec["sha256"]:
            return None
        w = rec["workloads"][workload]
        return int(w["read_bytes"] + w.get("write_bytes", 0))
    except (OSError, KeyError, ValueError):
        return None


def stream_bytes(view, hq):
    """Algorithmic bytes one decode call reads (all streams of the view)."""
    D = view.head_dim
    nq, ns, nt = view.n_quant, view.n_sink, view.n_tail
    G, Gv = view.group_tok, view.group_ch
    if view.k_mixed:
        nb, n4 = view.n_bf16, view.n_int4
        n2 = D - nb - n4
        k = nq * (2 * nb + 4 * math.ceil(n4 / 8) + 4 * math.ceil(n2 / 16))
        k += (nq // G) * (4 * (n4 + n2) + D)
    else:
        k = nq * 4 * math.ceil(D / (32 // view.k_bits)) + (nq // G) * D * 4
    v = nq * 4 * math.ceil(D / (32 // view.v_bits)) + nq * (D // Gv) * 4
    fp16 = (ns + nt) * D * 2 * 2
    per_stream = k + v + fp16
    return view.batch * view.kv_heads * per_stream + view.batch * hq * D * 2


def read_ceiling(torch, kvq, dev, stream, gib=4, reps=5):
    """GB/s of the library's plain streaming-read kernel over `gib` GiB
    (median of `reps` event-timed launches after two untimed ones)."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.empty(kvq.STREAM_READ_BLOCKS, dtype=torch.int32, device=dev)
    for _ in range(2):
        kvq.kvq_stream_read(buf, sink)
    ts = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del buf, sink
    torch.cuda.empty_cache()
    return (gib << 30) / (float(np.median(ts)) * 1e-3) / 1e9


def evict(flush_buf):
    """Evict the 256 MB Infinity Cache by reading 1 GiB: the lines left
    behind are clean, as after the other reads of a model step (a buffer
    rewritten instead leaves dirty lines whose write-back competes with the
    timed reads and halves the read rate even of a plain copy kernel at
    these sizes)."""
    flush_buf.view(__import__("torch").float32).sum()


def size_matched_ceiling(torch, kvq, dev, stream, nbytes, flush_buf, reps=15):
    """GB/s of the plain streaming-read kernel over `nbytes` (the bytes of
    one decode call), evicted before each timed launch like the decode."""
    n = (nbytes + 15) // 16 * 16
    buf = torch.ones(n, dtype=torch.uint8, device=dev)
    sink = torch.empty(kvq.STREAM_READ_BLOCKS, dtype=torch.int32, device=dev)
    ts = []
    for r in range(reps + 2):
        evict(flush_buf)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_stream_read(buf, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        if r >= 2:
            ts.append(e0.elapsed_time(e1))
    del buf, sink
    return n / (float(np.median(ts)) * 1e-3) / 1e9


def build_small(torch, kvq, dev, stream, name, seed, extra_tokens, extra):
    """A workload's cache built from the seeded host inputs: everything but
    the last 4096 tokens appended untimed, those 4096 as one timed prefill
    append; the salience select timed for mixed keys.  Returns the cache,
    q [1][B][Hq][D] and the next tokens' K, V [extra][1][B][Hkv][1][D]."""
    w = dict(synth.WORKLOADS[name])
    B, Hq, Hkv, N, D = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"]
    ikw = {k: w[k] for k in ("outliers", "n_out", "out_factor", "frac",
                             "fmin", "fmax", "sink_factor") if k in w}
    qn, kn, vn = synth.kv_inputs(seed, B, Hq, Hkv, N + extra_tokens, D, **ikw)
    c = kvq.Cache(B, Hkv, D, N + extra_tokens + 8, w["k_bits"], w["v_bits"],
                  w["G"], w["Gv"], w["R"], S=w["S"], mixed=w.get("mixed", False),
                  n_bf16=w.get("n_bf16", 0), n_int4=w.get("n_int4", 0))
    if w.get("mixed"):
        qw = torch.from_numpy(synth.query_window(seed, B, w["W"], Hq, D)).to(dev)
        c.kvq_salience_select(qw)
        # the salience select (I over the last W query rows), timed on its
        # own; a GPU spin ahead of each call keeps the host's launch latency
        # out of the event interval
        sal = []
        for r in range(12):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda._sleep(1 << 18)
            e0.record(stream)
            c.kvq_salience_select(qw)
            e1.record(stream)
            torch.cuda.synchronize()
            if r >= 2:
                sal.append(1000 * e0.elapsed_time(e1))
        extra["salience_select_us"] = round(float(np.median(sal)), 2)
        del qw
    n0 = max(0, N - 4096)
    if n0:
        c.kvq_append(
            torch.from_numpy(np.ascontiguousarray(kn[:, :, :n0])).to(dev),
            torch.from_numpy(np.ascontiguousarray(vn[:, :, :n0])).to(dev))
    kl = torch.from_numpy(np.ascontiguousarray(kn[:, :, n0:N])).to(dev)
    vl = torch.from_numpy(np.ascontiguousarray(vn[:, :, n0:N])).to(dev)
    torch.cuda.synchronize()
    ea = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda._sleep(1 << 21)  # ~1 ms: keeps host launch latency out
    ea[0].record(stream)
    c.kvq_append(kl, vl)
    ea[1].record(stream)
    torch.cuda.synchronize()
    extra[f"append_{N - n0}_us"] = round(1000 * ea[0].elapsed_time(ea[1]), 2)
    del kl, vl
    assert c.kvq_cache_check() == kvq.KVQ_OK
    q = torch.from_numpy(qn).to(dev)[None]
    knew = torch.from_numpy(np.ascontiguousarray(
        kn[:, :, N:].transpose(2, 0, 1, 3)[:, None, :, :, None, :])).to(dev)
    vnew = torch.from_numpy(np.ascontiguousarray(
        vn[:, :, N:].transpose(2, 0, 1, 3)[:, None, :, :, None, :])).to(dev)
    config = {"workload": name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
              "head_dim": D, "context": N,
              "k_bits": "mixed bf16/int4/int2" if w.get("mixed") else w["k_bits"],
              "v_bits": w["v_bits"], "k_group_tokens": w["G"],
              "v_group_channels": w["Gv"], "residual": w["R"], "sink": w["S"]}
    return c, q, knew, vnew, config


def sub_workload(torch, kvq, dev, stream, name, args, flush_buf):
    """One sub-record of the default run: µs per decode call (events around
    kvq_decode_attention, the Infinity Cache evicted before each step),
    GB/s against 8 TB/s and against a streaming read of the same size."""
    steps, warmup = 20, 3
    extra = {}
    c, q, knew, vnew, config = build_small(torch, kvq, dev, stream, name,
                                           args.seed, warmup + steps, extra)
    Hq = q.shape[2]
    view = c.kvq_cache_view()
    ws = torch.empty(2 * kvq.kvq_decode_workspace_bytes(view, Hq, 0) + 65536,
                     dtype=torch.uint8, device=dev)
    out = torch.empty(q.shape[1:], dtype=torch.float32, device=dev)
    calls = []
    for i in range(warmup + steps):
        evict(flush_buf)
        c.kvq_append(knew[i, 0], vnew[i, 0])
        view = c.kvq_cache_view()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_decode_attention(view, q[0], workspace=ws, out=out)
        e1.record(stream)
        if i >= warmup:
            calls.append((e0, e1))
    torch.cuda.synchronize()
    assert c.kvq_cache_check() == kvq.KVQ_OK
    us = [1000 * a.elapsed_time(b) for a, b in calls]
    # the same cache read as keys stored before the rotary embedding
    # (uniform or mixed keys: the dedicated rotary kernel)
    view = c.kvq_cache_view()
    rope_calls = []
    for i in range(6):
        evict(flush_buf)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        kvq.kvq_decode_attention_rope(view, q[0], workspace=ws, out=out)
        e1.record(stream)
        if i:
            rope_calls.append((e0, e1))
    torch.cuda.synchronize()
    rope_us = float(np.median([1000 * a.elapsed_time(b) for a, b in rope_calls]))
    nbytes = stream_bytes(c.kvq_cache_view(), Hq)
    ceil = size_matched_ceiling(torch, kvq, dev, stream, nbytes, flush_buf)
    med = float(np.median(us))
    rec = {"us_per_call": {"mean": round(float(np.mean(us)), 2),
                           "median": round(med, 2),
                           "p10": round(float(np.percentile(us, 10)), 2),
                           "p90": round(float(np.percentile(us, 90)), 2),
                           "calls": len(us)},
           "bytes_per_call": int(nbytes),
           "achieved_gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
           "frac_peak": round(nbytes / (med * 1e-6) / 1e9 / PEAK_GBS, 4),
           "read_ceiling_same_bytes_gbs": round(ceil, 1),
           "frac_read_ceiling": round(nbytes / (med * 1e-6) / 1e9 / ceil, 4),
           "rope_decode_us": round(rope_us, 2),
           "config": config}
    rec.update(extra)
    if "salience_select_us" in extra:
        rec["decode_plus_salience_us"] = round(med + extra["salience_select_us"], 2)
    del c, q, knew, vnew, ws, out
    torch.cuda.empty_cache()
    return rec


def ext_workload(torch, kvq, dev, stream, name, args, flush_buf):
    """A next-row leg on the 128K GQA layer: the codebook datatype with 1%
    per-vector outliers, or the KQV scheme (rotated keys; rotated values
    with the 1-bit residual sketch).  Times the quantization of the whole
    context (the prefill) and the decode call (events, Infinity Cache
    evicted before each call)."""
    w = dict(synth.WORKLOADS[name])
    B, Hq, Hkv, N, D = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"]
    ikw = {k: w[k] for k in ("outliers", "frac", "fmin", "fmax", "sink_factor") if k in w}
    qn, kn, vn = synth.kv_inputs(args.seed, B, Hq, Hkv, N, D, **ikw)
    kt = torch.from_numpy(kn.reshape(B * Hkv, N, D)).to(dev)
    vt = torch.from_numpy(vn.reshape(B * Hkv, N, D)).to(dev)
    qt = torch.from_numpy(qn).to(dev)
    del qn, kn, vn
    jl = None
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if w.get("k_nuq"):
        lk, lv = synth.nuq_codebook(w["k_bits"]), synth.nuq_codebook(w["v_bits"])
        # one untimed pass loads the quantizers' code
        kvq.kvq_quantize_nuq_k(kt[:1, :256], w["k_bits"], w["G"], lk, w["n_out"])
        kvq.kvq_quantize_nuq_v(vt[:1, :256], w["v_bits"], w["Gv"], lv, w["n_out"])
        torch.cuda.synchronize()
        e0.record(stream)
        keys = kvq.kvq_quantize_nuq_k(kt, w["k_bits"], w["G"], lk, w["n_out"])[:3]
        values = kvq.kvq_quantize_nuq_v(vt, w["v_bits"], w["Gv"], lv, w["n_out"])[:3]
        e1.record(stream)
        view = kvq.ext_view(B, Hkv, D, N, keys, values, w["k_bits"], w["v_bits"],
                            w["G"], w["Gv"], k_lut=lk, v_lut=lv)
        keep = (keys, values)
        kernel = ("decode_ext_mfma_kernel (codebook keys and values, outliers) + "
                  "merge_ext_kernel")
    else:
        jl = torch.from_numpy(synth.jl_matrix(args.seed, w["qjl_m"], D)).to(dev)
        kvq.kvq_quantize_k(kvq.kvq_hadamard(kt[:1, :256].contiguous(), out_dtype=torch.float32),
                           w["k_bits"], w["G"])
        kvq.kvq_quantize_v_qjl(kvq.kvq_hadamard(vt[:1, :256].contiguous(),
                                                out_dtype=torch.float32), w["v_bits"], w["Gv"], jl)
        torch.cuda.synchronize()
        e0.record(stream)
        kr = kvq.kvq_hadamard(kt, out_dtype=torch.float32)
        keys = kvq.kvq_quantize_k(kr, w["k_bits"], w["G"])[:2]
        del kr
        vr = kvq.kvq_hadamard(vt, out_dtype=torch.float32)
        c, sc, sk, rn, _ = kvq.kvq_quantize_v_qjl(vr, w["v_bits"], w["Gv"], jl)
        e1.record(stream)
        del vr
        values = (c, sc)
        qt = kvq.kvq_hadamard(qt, out_dtype=torch.float32)
        view = kvq.ext_view(B, Hkv, D, N, keys, values, w["k_bits"], w["v_bits"],
                            w["G"], w["Gv"], sketch=sk, rnorm=rn, jl=jl, v_rotated=True)
        keep = (keys, values, sk, rn, jl)
        kernel = ("decode_ext_mfma_kernel (symmetric keys, values with the sketch) + "
                  "merge_ext_kernel")
    torch.cuda.synchronize()
    quant_us = 1000 * e0.elapsed_time(e1)
    del kt, vt
    ws = torch.empty(kvq.kvq_decode_ext_workspace_bytes(view, Hq, 0), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    calls = []
    for i in range(3 + 20):
        evict(flush_buf)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        kvq.kvq_decode_attention_ext(view, qt, workspace=ws, out=out)
        b.record(stream)
        if i >= 3:
            calls.append((a, b))
    torch.cuda.synchronize()
    us = [1000 * a.elapsed_time(b) for a, b in calls]
    med = float(np.median(us))
    # bytes of one call: codes, scales, outliers, sketch words and norms,
    # the query (and, for the sketch, the projection matrix once)
    streams = B * Hkv
    kw = 4 * math.ceil(D / (32 // w["k_bits"]))
    vw = 4 * math.ceil(D / (32 // w["v_bits"]))
    per = N * (kw + vw) + (N + w["G"] - 1) // w["G"] * D * 4 + N * (D // w["Gv"]) * 4
    if w.get("k_nuq"):
        per += (N + w["G"] - 1) // w["G"] * D * w["n_out"] * 4
        per += N * (D // w["Gv"]) * w["n_out"] * 4
    else:
        per += N * (w["qjl_m"] // 8 + 4)
    nbytes = streams * per + B * Hq * D * 2 + (w.get("qjl_m", 0) * D * 4)
    g = Hq // Hkv
    # the method's arithmetic per token and KV head: the dequantization of
    # K and V (D multiplies each), the scores and the value sums (g D FMA
    # each), and for the sketch the sign sums (g m adds)
    fma = streams * N * (2 * D + 2 * g * D + g * w.get("qjl_m", 0))
    cfg = {k: w[k] for k in w if k not in ("outliers", "fmin", "fmax")}
    cfg["workload"] = name
    del keep, ws, out, view
    torch.cuda.empty_cache()
    return {"us_per_call": {"mean": round(float(np.mean(us)), 2), "median": round(med, 2),
                            "p10": round(float(np.percentile(us, 10)), 2),
                            "p90": round(float(np.percentile(us, 90)), 2), "calls": len(us)},
            "quantize_context_us": round(quant_us, 1),
            "bytes_per_call": int(nbytes),
            "achieved_gbs": round(nbytes / (med * 1e-6) / 1e9, 1),
            "frac_hbm_peak": round(nbytes / (med * 1e-6) / 1e9 / PEAK_GBS, 4),
            "roofline": {"bound": "alu", "fma_per_call": int(fma),
                         "achieved_tflops": round(2 * fma / (med * 1e-6) / 1e12, 2),
                         "peak_tflops": 78.6,
                         "frac": round(2 * fma / (med * 1e-6) / 78.6e12, 4)},
            "kernel": kernel, "config": cfg}


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy)
        return
    import torch
    from quantized_decode_attention_02_amd import kvq

    kvq.lib()  # fail loudly if the library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    w = dict(synth.WORKLOADS[args.workload])
    if args.workload in ("kvquant_3bit_1pct_128k", "kqv_4bit_128k"):
        # a next-row leg on its own (the default run reports it beside the
        # headline)
        flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        print(json.dumps({"workload": args.workload, **ext_workload(
            torch, kvq, dev, stream, args.workload, args, flush_buf)}), flush=True)
        return
    extra = {}

    if args.workload == "1m_32layer":
        layers = args.layers or w["layers"]
        B, Hq, Hkv, N, D = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"]
        chunk = w["chunk"]
        cap = N + args.warmup + args.steps + 8
        caches = []
        build_chunk = 65536
        kbuf = torch.empty(Hkv * build_chunk * D, dtype=torch.float16,
                           device=dev)
        vbuf = torch.empty_like(kbuf)
        t_build = time.time()
        for L in range(layers):
            c = kvq.Cache(B, Hkv, D, cap, w["k_bits"], w["v_bits"], w["G"],
                          w["Gv"], w["R"], S=w["S"])
            t = 0
            while t < N - chunk:
                n = min(build_chunk, N - chunk - t)
                kv = kbuf[:Hkv * n * D].view(1, Hkv, n, D)
                vv = vbuf[:Hkv * n * D].view(1, Hkv, n, D)
                kvq.kvq_synth_normal_f16(kv, args.seed, synth.TENSOR_K, L, 0,
                                         Hkv, t, n, D, n * D)
                kvq.kvq_synth_normal_f16(vv, args.seed, synth.TENSOR_V, L, 0,
                                         Hkv, t, n, D, n * D)
                c.kvq_append(kv, vv)
                t += n
            caches.append(c)
            if L % 8 == 7 or L == layers - 1:
                torch.cuda.synchronize()
                print(f"# built {L + 1}/{layers} layers "
                      f"({time.time() - t_build:.1f}s)", file=sys.stderr,
                      flush=True)
        del kbuf, vbuf
        # the last 4096-token prefill chunk of every layer: timed append
        kc = torch.empty((layers, 1, Hkv, chunk, D), dtype=torch.float16,
                         device=dev)
        vc = torch.empty_like(kc)
        for L in range(layers):
            kvq.kvq_synth_normal_f16(kc[L, 0], args.seed, synth.TENSOR_K, L,
                                     0, Hkv, N - chunk, chunk, D, chunk * D)
            kvq.kvq_synth_normal_f16(vc[L, 0], args.seed, synth.TENSOR_V, L,
                                     0, Hkv, N - chunk, chunk, D, chunk * D)
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        ev[0].record(stream)
        for L in range(layers):
            caches[L].kvq_append(kc[L], vc[L])
        ev[1].record(stream)
        torch.cuda.synchronize()
        append_ms = ev[0].elapsed_time(ev[1])
        extra["append_4096_us_per_layer"] = round(1000 * append_ms / layers,
                                                  2)
        # the optional key rotation of such a chunk (kvq_hadamard: fp16 in
        # and out, 4096 x 32 rows of 128) and of one step's queries
        kr = torch.empty_like(kc[0])
        qh = torch.empty((1, Hq, D), dtype=torch.float16, device=dev)
        rot = {"keys": [], "query": []}
        for r in range(6):
            for name, (src, dst) in (("keys", (kc[r % layers], kr)),
                                     ("query", (qh, qh))):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(1 << 21)
                e0.record(stream)
                kvq.kvq_hadamard(src, out=dst)
                e1.record(stream)
                torch.cuda.synchronize()
                if r:
                    rot[name].append(1000 * e0.elapsed_time(e1))
        extra["rotate_keys_4096_us_per_layer"] = round(float(np.median(rot["keys"])), 2)
        extra["rotate_query_us"] = round(float(np.median(rot["query"])), 2)
        del kr, qh
        del kc, vc
        for c in caches:
            assert c.kvq_cache_check() == kvq.KVQ_OK
        # per-step inputs: queries and the new token of every layer
        n_steps_total = args.warmup + args.steps
        q = torch.empty((layers, B, Hq, D), dtype=torch.float16, device=dev)
        knew = torch.empty((n_steps_total, layers, B, Hkv, 1, D),
                           dtype=torch.float16, device=dev)
        vnew = torch.empty_like(knew)
        for L in range(layers):
            kvq.kvq_synth_normal_f16(q[L, 0], args.seed, synth.TENSOR_Q, L, 0,
                                     Hq, 0, 1, D, D)
            for st in range(n_steps_total):
                kvq.kvq_synth_normal_f16(knew[st, L, 0], args.seed,
                                         synth.TENSOR_K, L, 0, Hkv, N + st, 1,
                                         D, D)
                kvq.kvq_synth_normal_f16(vnew[st, L, 0], args.seed,
                                         synth.TENSOR_V, L, 0, Hkv, N + st, 1,
                                         D, D)
        config = {"workload": "1m_32layer", "layers": layers, "batch": B,
                  "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
                  "context": N, "k_bits": w["k_bits"], "v_bits": w["v_bits"],
                  "k_group_tokens": w["G"], "v_group_channels": w["Gv"],
                  "residual": w["R"], "sink": w["S"]}
    else:
        layers = 1
        B, Hq, Hkv, N, D = w["B"], w["Hq"], w["Hkv"], w["N"], w["D"]
        c, q, knew, vnew, config = build_small(
            torch, kvq, dev, stream, args.workload, args.seed,
            args.warmup + args.steps, extra)
        caches = [c]

    # decode workspaces and outputs (allocated before timing)
    views = [c.kvq_cache_view() for c in caches]
    # room for a few more partials than the first step needs: the automatic
    # split count can grow by one as flushes add key groups
    ws_bytes = 2 * max(kvq.kvq_decode_workspace_bytes(v, Hq, sp)
                       for v in views for sp in {args.splits, 0}) + 65536
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, D), dtype=torch.float32, device=dev)
    flush_buf = None
    if args.workload != "1m_32layer":
        flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)

    def step(i, events=None):
        for L, c in enumerate(caches):
            c.kvq_append(knew[i, L], vnew[i, L])
            view = c.kvq_cache_view()
            if events is not None:
                events[L][0].record(stream)
            kvq.kvq_decode_attention(view, q[L], n_splits=args.splits,
                                     workspace=ws, out=out)
            if events is not None:
                events[L][1].record(stream)

    # (the events are made before the warmup and the caches are checked
    # after the timed steps: host work between the warmup and the timed
    # steps leaves the GPU idle long enough for its clock to drop, and the
    # first timed step then ran ~15% slow)
    dec_events = [[[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in caches] for _ in range(args.steps)]
    step_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in range(args.steps)]
    bytes_step = 0
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        if flush_buf is not None:
            evict(flush_buf)
        step_events[s][0].record(stream)
        step(args.warmup + s, dec_events[s])
        step_events[s][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for c in caches:
        assert c.kvq_cache_check() == kvq.KVQ_OK
    views = [c.kvq_cache_view() for c in caches]
    bytes_step = sum(stream_bytes(v, Hq) for v in views)
    step_ms = [e[0].elapsed_time(e[1]) for e in step_events]
    ms_per_step = float(np.mean(step_ms)) if flush_buf is not None else \
        1000.0 * wall / args.steps
    dec_ms = [e[0].elapsed_time(e[1]) for st in dec_events for e in st]
    dec_avg_ms = float(np.mean(dec_ms))
    ceiling = read_ceiling(torch, kvq, dev, stream)
    bytes_launch = bytes_step / len(caches)
    achieved = bytes_launch / (dec_avg_ms * 1e-3) / 1e9
    value = bytes_step / (ms_per_step * 1e-3) / 1e9

    res = {
        "metric": "quantized-KV decode attention: µs/step + achieved "
                  "HBM GB/s (% of peak)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "us_per_step": round(1000 * ms_per_step, 1),
        "pct_of_hbm_peak": round(100 * value / PEAK_GBS, 1),
        "tokens_per_s": round(B * 1000.0 / ms_per_step, 2),
        "context_tokens_per_s": round(
            sum(v.batch * (v.n_sink + v.n_quant + v.n_tail) for v in views)
            * 1000.0 / ms_per_step, 1),
        "decode_call_us": {
            "mean": round(1000 * dec_avg_ms, 2),
            "median": round(1000 * float(np.median(dec_ms)), 2),
            "p10": round(1000 * float(np.percentile(dec_ms, 10)), 2),
            "p90": round(1000 * float(np.percentile(dec_ms, 90)), 2),
            "calls": len(dec_ms)},
        "read_ceiling": {"value": round(ceiling, 1), "unit": "GB/s",
                         "bytes": 4 << 30, "kernel": "kvq_stream_read"},
        "pct_of_read_ceiling": round(100 * value / ceiling, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int2/int4 codes, fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded; N(0,1)-like bodies, no weights)",
        "config": config,
        "roofline": {
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload),
            "kernel": "kvq_decode_attention (decode_rs_kernel: quantized "
                      "splits + fp16 sink/tail parts; then merge_kernel)",
            "bytes_per_launch": int(bytes_launch),
            "avg_launch_us": round(1000 * dec_avg_ms, 2),
            "frac_of_read_ceiling": round(achieved / ceiling, 4),
        },
        "bytes_per_step": int(bytes_step),
    }
    # The same caches read as keys stored before the rotary embedding
    # (kvq_decode_attention_rope), timed apart from the step.  Vector-ALU
    # bound.  The method's work per quantized token and KV head: turning
    # the key to its position, 2 FMA per channel (shared by the g query
    # heads), then per query head the score (D FMA) and the value sum (D
    # FMA): 2 D + 2 g D.  (The kernel itself spends 4 g D: it folds the
    # turn into the weights of every head.)  The peak is the fp32 vector
    # rate without packed math, 256 CUs x 4 SIMDs x 16 lanes x 2 flops x
    # 2.4 GHz = 78.6 TFLOP/s.
    rope_us = {}
    for pairing in ("half", "interleaved"):
        ts = []
        for r in range(4):
            if flush_buf is not None:
                evict(flush_buf)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
                   for _ in caches]
            for L, c in enumerate(caches):
                view = c.kvq_cache_view()
                evs[L][0].record(stream)
                kvq.kvq_decode_attention_rope(view, q[L], pairing=pairing,
                                              workspace=ws, out=out)
                evs[L][1].record(stream)
            torch.cuda.synchronize()
            if r:
                ts += [1000 * e[0].elapsed_time(e[1]) for e in evs]
        rope_us[pairing] = float(np.median(ts))
    g = Hq // Hkv
    fma = sum((2 + 2 * g) * v.head_dim * v.n_quant * v.batch * v.kv_heads
              for v in views) / len(views)
    fma_kernel = sum(4 * g * v.head_dim * v.n_quant * v.batch * v.kv_heads
                     for v in views) / len(views)
    t_h = rope_us["half"] * 1e-6
    extra["rope_decode"] = {
        "us_per_call": {k: round(x, 2) for k, x in rope_us.items()},
        "bound": "alu",
        "fma_per_launch": int(fma),
        "fma_per_launch_as_computed": int(fma_kernel),
        "achieved_tflops": round(2 * fma / t_h / 1e12, 2),
        "peak_tflops": 78.6,
        "frac": round(2 * fma / t_h / 78.6e12, 4),
        "hbm_gbs": round(bytes_launch / t_h / 1e9, 1),
        "kernel": ("decode_generic_kernel (rotary form: mixed keys) + merge_kernel"
                   if views[0].k_mixed else
                   "decode_rope_kernel (+ general kernel for fp16 sink/tail, "
                   "merge_kernel)")}
    if "salience_select_us" in extra:
        extra["decode_plus_salience_us"] = round(
            res["decode_call_us"]["median"] + extra["salience_select_us"], 2)
    res.update(extra)
    if args.workload == "1m_32layer" and not args.no_workloads:
        del q, knew, vnew, ws, out, caches, views
        torch.cuda.empty_cache()
        flush_buf = torch.zeros(1 << 30, dtype=torch.uint8, device=dev)
        res["workloads"] = {}
        for name in ("7b_layer_4k", "gqa_128k", "gqa_128k_k2v4", "mixkvq_32k"):
            t0w = time.time()
            res["workloads"][name] = sub_workload(torch, kvq, dev, stream, name,
                                                  args, flush_buf)
            print(f"# {name}: {res['workloads'][name]['us_per_call']['median']} "
                  f"us per call ({time.time() - t0w:.1f}s)", file=sys.stderr,
                  flush=True)
        res["next_rows"] = {}
        for name in ("kvquant_3bit_1pct_128k", "kqv_4bit_128k"):
            t0w = time.time()
            res["next_rows"][name] = ext_workload(torch, kvq, dev, stream, name,
                                                  args, flush_buf)
            print(f"# {name}: {res['next_rows'][name]['us_per_call']['median']} "
                  f"us per call ({time.time() - t0w:.1f}s)", file=sys.stderr,
                  flush=True)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(args, w, layers)
    print(json.dumps(res), flush=True)


def _oracle_sample(args, w, layers, n_sample, stream_index=0):
    """The oracle cache of one sampled (batch, KV head) stream, its query
    rows and the factor that scales one pass to a whole step."""
    from oracle import cache as ocache

    D = w["D"]
    if args.workload == "1m_32layer":
        h = stream_index % w["Hkv"]
        k, v = synth.counter_kv(args.seed, 0, w["Hkv"], 0, n_sample, D,
                                heads=[h])
        q = synth.counter_query(args.seed, 0, w["Hq"], D)[h:h + 1]
        scale = (w["N"] / n_sample) * w["Hkv"] * layers * w["B"]
    else:
        qn, kn, vn = synth.kv_inputs(args.seed + stream_index, 1,
                                     w["Hq"] // w["Hkv"], 1, n_sample, D)
        k, v, q = kn[0], vn[0], qn[0]
        scale = (w["N"] / n_sample) * w["Hkv"] * w["B"]
    cfg = ocache.CacheConfig(B=1, Hkv=1, D=D, S=w["S"], R=w["R"], G=w["G"],
                             Gv=w["Gv"], k_bits=w.get("k_bits", 2),
                             v_bits=w["v_bits"], mixed=w.get("mixed", False),
                             n_bf16=w.get("n_bf16", 0),
                             n_int4=w.get("n_int4", 0))
    oc = ocache.Cache(cfg)
    oc.append(k[None], v[None])
    return oc, q, scale


def _oracle_pass(oc, q, g):
    from oracle import attention
    kh, vh = oc.dequantized(0, 0)
    attention.attention(q[:g].astype(np.float64), kh[None], vh[None])


def _pool_worker(job):
    """One process of the all-cores baseline: build its stream's oracle
    cache, wait for every worker, then time `passes` decode passes."""
    args, w, layers, n_sample, idx, g, passes, barrier = job
    from threadpoolctl import threadpool_limits
    with threadpool_limits(limits=1):
        oc, q, _ = _oracle_sample(args, w, layers, n_sample, idx)
        barrier.wait()
        t0 = time.perf_counter()
        for _ in range(passes):
            _oracle_pass(oc, q, g)
        return time.perf_counter() - t0


def cpu_baseline(args, w, layers):
    """The oracle's decode on sampled (batch, KV head) streams, scaled to a
    step: one core (the primary figure), then every core the process may
    use, one stream per process."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits

    g = w["Hq"] // w["Hkv"] if args.workload != "1m_32layer" else 1
    n_sample = 262144 if args.workload == "1m_32layer" else min(w["N"], 131072)
    oc, q, scale = _oracle_sample(args, w, layers, n_sample)
    # repeat the timed decode until about 10 s of CPU work are measured
    times = []
    with threadpool_limits(limits=1):
        while sum(times) < 10.0 or len(times) < 3:
            t0 = time.perf_counter()
            _oracle_pass(oc, q, g)
            times.append(time.perf_counter() - t0)
    del oc
    t = float(np.median(times))
    us_step = t * scale * 1e6
    if args.workload == "1m_32layer":
        sample = (f"1 of {w['Hkv']} KV heads of 1 of {layers} layers at "
                  f"{n_sample} of {w['N']} tokens; scaled x{scale:g}")
    else:
        sample = (f"1 of {w['B'] * w['Hkv']} (batch, KV head) streams at "
                  f"{n_sample} of {w['N']} tokens; scaled x{scale:g}")
    res = {"value": round(us_step, 1), "unit": "us/step", "cores": 1,
           "kind": "oracle", "sample": sample + f"; median of {len(times)} "
           f"passes ({sum(times):.1f} s timed)", "sample_seconds": round(t, 3)}
    # every core: one process per core (at most 16, the CPU share of one
    # GPU on the boxes), each decoding its own stream at a quarter of the
    # sample length; throughput = streams per second over all processes
    avail = len(os.sched_getaffinity(0))
    res["cores_available"] = avail
    P = max(1, min(avail, 16))
    n_par = n_sample // 4
    passes = max(2, int(round(4.0 / max(t / 4, 1e-3))))
    ctx = mp.get_context("fork")
    barrier = ctx.Manager().Barrier(P)
    t0 = time.perf_counter()
    with ctx.Pool(P) as pool:
        walls = pool.map(_pool_worker, [(args, w, layers, n_par, i, g, passes,
                                         barrier) for i in range(P)])
    elapsed = time.perf_counter() - t0
    per_pass = max(walls) / passes          # the slowest process sets the pace
    scale_par = scale * n_sample / n_par    # passes per step at this length
    res["all_cores"] = {
        "value": round(per_pass * scale_par / P * 1e6, 1), "unit": "us/step",
        "cores": P, "kind": "oracle",
        "sample": f"{P} processes, each one stream at {n_par} tokens, "
                  f"{passes} timed passes each ({elapsed:.1f} s wall incl. "
                  f"building); per-step time = slowest process's pass time "
                  f"x {scale_par:g} / {P}"}
    return res


if __name__ == "__main__":
    main()
