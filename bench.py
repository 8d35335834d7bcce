#!/usr/bin/env python3
"""FP8-KV GQA decode attention at 32K context on one MI355X.

Workload: one layer of batch-1 decode with 32 query / 4 KV heads (GQA 8),
head dim 128, 32,768 cached rows scattered over a 33,059-row page-size-1 FP8
pool (seeded permutation), K ~ N(0,1) with 4 x8 outlier channels per head,
V ~ 0.5 N(0,1), bf16 before quantization.  One step = one decode layer:
quantize the new token's K/V row into the pool (its slot is the last table
entry) and attend over all 32,768 positions, as the fused call
fp8kv_decode_attn_append (split-K stage 1 over the cached rows, then a merge
that also quantizes, stores and adds the new token: two kernels); the
three-call form (fp8kv_quantize_rows, then stage 1 + merge) is timed beside it.

Protocol: `--rounds` seeded rounds (workload seed r for round r), each with
its own pool; inside a round the timed items run in a seeded shuffled order,
each as `--warmup` untimed steps followed by exactly `--steps` timed steps
(one HIP graph each, HIP events on the graph's stream).  Cold HBM: the steps
rotate over `--pools` identical copies of the layer's pool (12 x 38.1 MB =
457 MB of 1,152-byte row records, more than the 256 MB Infinity Cache), as
the layers of a model do;
the warm column replays the same step over one pool.  `value` and
`ms_per_step` are the median over rounds; every sample is kept.

Also timed by default: the 48-layer step at 40,000 context (48 distinct
40,290-row pools, 2 GB); the 8K FP8 prefix + 8K chunk prefill with a BF16
prefix beside it; the decode variants (head dim 256, several query rows, a
sliding window, INT8, a 16-request batch); read floors (cold contiguous
reads of 1x, 2x and 8x the layer's bytes, the layer's row records gathered
through its table, a library reduction, and a dependent kernel launch after
stage 1);
and the CPU oracle on the host cores.

Prints one JSON line.  `value` is the effective KV bandwidth of the whole step
(algorithmic KV bytes / step time); `roofline` is for the dominant kernel
(stage 1), timed on its own the same way.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "FP8-KV GQA decode attention: us/layer and KV HBM GB/s (% of peak) at 32K ctx"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
KV_BYTES_PER_ROW_HEAD = 2 * (128 + 4)   # K and V: 128 code bytes + one fp32 scale each
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_stage1_32k_traffic.json")
GUARD_FILE = os.path.join(ROOT, "tests", "golden", "decode_32k_step_seed0.txt")
LAYOUTS = ["separate", "interleaved", "interleaved64", "interleaved128", "split"]


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240, help="timed decode steps (layers) per round and item")
    ap.add_argument("--warmup", type=int, default=24, help="untimed steps before each timed run")
    ap.add_argument("--rounds", type=int, default=5, help="seeded rounds of the headline workload")
    ap.add_argument("--pools", type=int, default=12, help="pool copies rotated per step (cold HBM)")
    ap.add_argument("--max-splits", type=int, default=0)
    ap.add_argument("--layout", default="interleaved128", choices=LAYOUTS,
                    help="pool layout: one row record holding the K codes, V codes, K scales and V scales of all "
                         "KV heads, padded to 128 bytes (1,152 bytes: every KV head's code rows fill whole "
                         "128-byte lines, so the decode reads them with non-temporal loads), the same unpadded "
                         "(1,056 bytes) or padded to 64 bytes, code records + scale records (split), or four "
                         "separate arrays")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="wall-time budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="reuse one pool (Infinity-Cache resident) for everything")
    ap.add_argument("--no-warm-column", action="store_true",
                    help="skip the warm (one-pool) column, so a kernel trace holds only cold stage-1 dispatches")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 8K-prefix + 8K-chunk prefill timing")
    ap.add_argument("--no-variants", action="store_true",
                    help="skip the head-dim-256, multi-row, sliding-window, INT8 and batched decode timings")
    ap.add_argument("--no-model-step", action="store_true",
                    help="skip the 48-layer step at 40,000 context (it runs the headline's stage-1 kernel, so "
                         "kernel traces of the headline are taken without it)")
    ap.add_argument("--model-step-steps", type=int, default=8, help="timed 48-layer steps")
    ap.add_argument("--no-floors", action="store_true", help="skip the read-floor and dependent-launch timings")
    ap.add_argument("--timeline", action="store_true",
                    help="also run the measurement build with per-wave stage-1 timestamps (libfp8kv_timeline.so) "
                         "on the headline workload and report when each wave's data arrives and its work ends")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="first run plain 64 MiB device copies (a known-size kernel for HBM byte counters)")
    return ap.parse_args()


STAGE1_SOURCES = ("decode.hip", "fp8kv_device.h", "fp8kv_launch.h", "fp8kv_api.hip")


def kernel_source_hash() -> str:
    """Hash of the sources the stage-1 kernel and its launch geometry (split
    choice) are built from: its byte counters are only reused while these are
    unchanged."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "fp8_kv_cache_row_amd", "csrc")
    for name in STAGE1_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(layout: str, cold_pools: int):
    """HBM bytes per stage-1 launch from the committed rocprofv3 counter runs
    (taken on the default workload: 12 rotated pool copies, cold), or None when
    they were taken on a different kernel source, pool layout or workload."""
    if cold_pools != 12:
        return None
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash() or rec.get("pool_layout") != layout:
        return None
    return rec.get("bytes_per_launch")


def prefill_timing(fk, wl, dev, reps: int = 6):
    """8,192 historical FP8 rows + an 8,192-token bf16 chunk (32 q / 4 KV heads):
    reconstruct + causal attention in one call, the same attention over the
    prefix's bf16 rows (the BF16-pool comparator), then quantize the chunk.
    Calls are captured in HIP graphs and replayed, so host launch overhead is
    not timed (it would dominate the ~10 us chunk quantize); three alternating
    samples of each of the first two, median reported."""
    import numpy as np
    import torch

    case = wl.chunked_prefill(0)
    P, T, Hq, Hkv = case.prefix_k.shape[0], case.q.shape[0], case.n_q_heads, case.n_kv_heads

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    pool = fk.Fp8KvPool(case.pool_rows, Hkv, device=dev)
    fk.fp8kv_quantize_rows(pool, bf(case.prefix_k), bf(case.prefix_v), torch.from_numpy(case.prefix_rows).to(dev))
    q, kc, vc = bf(case.q), bf(case.k_cur), bf(case.v_cur)
    rows = torch.from_numpy(case.prefix_rows).to(dev)
    slots = torch.from_numpy(case.chunk_slots).to(dev)
    ws_k = torch.empty((P, Hkv, 128), dtype=torch.bfloat16, device=dev)
    ws_v = torch.empty_like(ws_k)
    out = torch.empty_like(q)
    stream = torch.cuda.Stream(device=dev)
    torch.cuda.synchronize()

    bws_k, bws_v = bf(case.prefix_k), bf(case.prefix_v)  # the prefix rows as a BF16 KV cache holds them

    def attn(i):
        fk.fp8kv_prefill_attn(pool, q, kc, vc, rows, ws_k, ws_v, case.sm_scale, out=out, stream=stream)

    def attn_bf16(i):
        fk.fp8kv_prefill_attn_workspace(q, kc, vc, bws_k, bws_v, case.sm_scale, out=out, stream=stream)

    def quant(i):
        fk.fp8kv_quantize_rows(pool, kc, vc, slots, stream=stream)

    # FP8 path and BF16 comparator alternate, so drift on the box affects both alike
    fp8, bf16 = [], []
    for _ in range(3):
        fp8.append(time_exact(stream, attn, reps, 1))
        bf16.append(time_exact(stream, attn_bf16, reps, 1))
    ms, bms = statistics.median(fp8), statistics.median(bf16)
    qms = time_exact(stream, quant, 64, 16)
    pairs = T * P + T * (T + 1) // 2            # causal (query, key) pairs per head
    flop = 4.0 * 128 * pairs * Hq               # QK^T and PV, 2 flop per MAC
    tflops = flop / (ms * 1e-3) / 1e12
    qbytes = T * Hkv * 2 * (128 * 2 + 128 + 4)  # bf16 rows in, codes + scales out
    return {"workload": "8,192 FP8 prefix rows + 8,192-token bf16 chunk, causal, 32 q / 4 KV heads",
            "reconstruct_plus_attention_ms": round(ms, 4),
            "bf16_prefix_attention_ms": round(bms, 4),
            "bf16_prefix_note": "the same attention kernel over the prefix's bf16 rows (a BF16 KV pool, no "
                                "reconstruction): fp8kv_prefill_attn_workspace",
            "fp8_over_bf16": round(ms / bms, 4),
            "samples_ms": {"fp8": [round(x, 4) for x in fp8], "bf16_prefix": [round(x, 4) for x in bf16]},
            "attention_flop": flop,
            "tflops": round(tflops, 2), "mfma_bf16_frac_of_2500": round(tflops / 2500.0, 4),
            "quantize_chunk_us": round(qms * 1e3, 3),
            "quantize_chunk_gbps": round(qbytes / (qms * 1e-3) / 1e9, 1)}


def capture_graph(stream, body, n):
    """A HIP graph of n calls body(i) on `stream` (after one untimed eager pass)."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for i in range(n):
            body(i)
    stream.synchronize()
    with torch.cuda.graph(g, stream=stream):
        for i in range(n):
            body(i)
    return g


def time_graph(stream, g, per_graph, total, warmup):
    """ms per call of a graph holding per_graph calls, replayed to >= total calls;
    HIP events on the graph's stream."""
    import torch
    reps = max(1, -(-total // per_graph))
    for _ in range(max(1, -(-warmup // per_graph))):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * per_graph), reps * per_graph


def rotated_pools(fk, case, layout, n, dev, bf, fmt="e4m3"):
    """n identical copies of a case's quantized pool (cold HBM when rotated)."""
    import torch
    base = fk.Fp8KvPool(case.pool_rows, case.n_kv_heads, layout=layout, device=dev, head_dim=case.head_dim,
                        code_format=fmt)
    fk.fp8kv_quantize_rows(base, bf(case.k_rows), bf(case.v_rows),
                           torch.arange(case.pool_rows, dtype=torch.int32, device=dev))
    pools = [base]
    for _ in range(n - 1):
        p = fk.Fp8KvPool(case.pool_rows, case.n_kv_heads, layout=layout, device=dev, head_dim=case.head_dim,
                         code_format=fmt)
        for dst, src in zip(p._buffers, base._buffers):
            dst.copy_(src)
        pools.append(p)
    torch.cuda.synchronize()
    return pools


def variants_timing(fk, wl, dev, args, bf):
    """The decode variants at 32K context, each over rotated cold pools:
    head dim 256 (fused append step and stage 1 alone), 3 and 8 causal query
    rows per request (and the 8-row step with its new tokens written in the
    same call), the INT8 KV format (fused append step and stage 1
    alone), the 16-request GQA-4 batch (fused step and stage 1 alone), an odd
    4,095-key sliding window (query rows call, and the fused step)."""
    import numpy as np
    import torch
    stream = torch.cuda.Stream(device=dev)
    n = max(1, args.pools)
    steps = max(48, args.steps // 2)
    res = {}

    def run(name, case, body_for, kv_bytes, flop=None, extra=None, fmt="e4m3", copies=None):
        nc = copies or n
        pools = rotated_pools(fk, case, args.layout, nc, dev, bf, fmt)
        body = body_for(case, pools)
        g = capture_graph(stream, body, nc)
        ms, _ = time_graph(stream, g, nc, steps, args.warmup)
        gbps = kv_bytes / (ms * 1e-3) / 1e9
        r = {"us": round(ms * 1e3, 3), "kv_bytes": kv_bytes, "kv_gbps": round(gbps, 1),
             "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4)}
        if flop:
            r["flop"] = flop
            r["tflops"] = round(flop / (ms * 1e-3) / 1e12, 2)
        if extra:
            r.update(extra)
        res[name] = r
        del pools, g
        torch.cuda.synchronize()
        torch.cuda.empty_cache()

    def append_body(case, pools, window=0):
        q, nk, nv = bf(case.q), bf(case.new_k), bf(case.new_v)
        t, sl = torch.from_numpy(case.table).to(dev), torch.from_numpy(case.seq_lens).to(dev)
        # request b's new token sits at its last position
        last = case.table[np.arange(case.table.shape[0]), case.seq_lens.astype(np.int64) - 1]
        slot = torch.from_numpy(np.ascontiguousarray(last, dtype=np.int32)).to(dev)
        ws = fk.decode_workspace(case.table.shape[0], case.n_q_heads, device=dev, head_dim=case.head_dim)
        out = torch.empty_like(q)
        return lambda i: fk.fp8kv_decode_attn_append(pools[i % len(pools)], q, nk, nv, slot, t, sl,
                                                     case.max_seq_len, case.sm_scale, workspace=ws, out=out,
                                                     stream=stream, window=window)

    def stage1_body(case, pools):
        q = bf(case.q)
        t, sl = torch.from_numpy(case.table).to(dev), torch.from_numpy(case.seq_lens).to(dev)
        ws = fk.decode_workspace(case.table.shape[0], case.n_q_heads, device=dev, head_dim=case.head_dim)
        return lambda i: fk.fp8kv_decode_stage1(pools[i % len(pools)], q, t, sl, case.max_seq_len, case.sm_scale,
                                                workspace=ws, stream=stream)

    def rows_body(window):
        def make(case, pools):
            q = bf(case.q if case.q.ndim == 4 else case.q[:, None])
            t, sl = torch.from_numpy(case.table).to(dev), torch.from_numpy(case.seq_lens).to(dev)
            ws = fk.decode_workspace(q.shape[1], case.n_q_heads, device=dev, head_dim=case.head_dim)
            out = torch.empty_like(q)
            return lambda i: fk.fp8kv_decode_attn_rows(pools[i % n], q, t, sl, case.max_seq_len, case.sm_scale,
                                                       window=window, workspace=ws, out=out, stream=stream)
        return make

    c256 = wl.layer_decode(0, head_dim=256)
    kv256 = c256.max_seq_len * c256.n_kv_heads * 2 * (256 + 4)
    run("d256_append_step", c256, append_body, kv256,
        extra={"workload": "32K-context GQA-8 decode step at head dim 256 (32 q / 4 KV heads)"})
    run("d256_stage1", c256, stage1_body, kv256)
    del c256
    def rows_append_body(case, pools):
        nq = case.q.shape[1]
        rng = np.random.default_rng(1)
        shape = (1, nq, case.n_kv_heads, 128)
        nk, nv = bf(wl.bf16_bits(wl.draw_normal(rng, shape))), bf(wl.bf16_bits(wl.draw_normal(rng, shape, 0.5)))
        q = bf(case.q)
        t, sl = torch.from_numpy(case.table).to(dev), torch.from_numpy(case.seq_lens).to(dev)
        slots = torch.from_numpy(np.ascontiguousarray(case.table[:, -nq:])).to(dev)
        ws = fk.decode_workspace(nq, case.n_q_heads, device=dev)
        out = torch.empty_like(q)
        return lambda i: fk.fp8kv_decode_attn_rows_append(pools[i % len(pools)], q, nk, nv, slots, t, sl,
                                                          case.max_seq_len, case.sm_scale, workspace=ws, out=out,
                                                          stream=stream)

    for nq in (3, 8):
        c = wl.layer_decode(0, with_new_token=False, n_qrows=nq)
        kv = c.max_seq_len * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD
        L = c.max_seq_len
        pairs = nq * L - nq * (nq - 1) // 2          # causal (row, key) pairs per head
        run(f"rows{nq}", c, rows_body(0), kv, flop=4.0 * 128 * pairs * c.n_q_heads,
            extra={"workload": f"32K-context GQA-8 decode, {nq} causal query rows per request"})
        if nq == 8:
            run("rows8_append_step", c, rows_append_body, kv, flop=4.0 * 128 * pairs * c.n_q_heads,
                extra={"workload": "32K-context GQA-8 decode step with 8 new tokens quantized on write and "
                                   "attended by their causal query rows"})
    c = wl.layer_decode(0)
    kv = c.max_seq_len * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD
    run("int8_append_step", c, append_body, kv, fmt="int8",
        extra={"workload": "32K-context GQA-8 decode step over an INT8 pool (scale amax/127)"})
    run("int8_stage1", c, stage1_body, kv, fmt="int8")
    # 16 requests with seeded lengths in [1,024, 32,768] (272,568 rows, 288 MB of
    # codes and scales per pool copy: larger than the Infinity Cache, so 4
    # rotated copies keep it cold), 16 q / 4 KV heads
    c = wl.batched_decode(0, with_new_token=True)
    kv = int(c.seq_lens.astype(np.int64).sum()) * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD
    run("batched16_append_step", c, append_body, kv, copies=min(n, 4),
        extra={"workload": "16 requests, lengths 1,024-32,768 (272,568 rows), GQA 4 (16 q / 4 KV heads), "
                           "one decode step with quantize-on-write"})
    run("batched16_stage1", c, stage1_body, kv, copies=min(n, 4))
    if args.layout.startswith("interleaved"):
        # the same rows' whole records gathered through the tables by the read-floor kernel
        FL = floor_lib()
        flat = np.concatenate([c.table[b, :c.seq_lens[b]] for b in range(c.batch)]).astype(np.int32)
        tflat = torch.from_numpy(flat).to(dev)
        sink = torch.zeros(4, dtype=torch.int32, device=dev)

        def gather_body(case, pools):
            rec = pools[0].record.shape[1]
            sp = ctypes.c_void_p(stream.cuda_stream)

            def call(i):
                if FL.fp8kv_floor_gather(pools[i % len(pools)].record.data_ptr(), case.pool_rows, rec,
                                         tflat.data_ptr(), len(flat), 1024, sink.data_ptr(), sp):
                    raise RuntimeError("fp8kv_floor_gather failed")
            return call
        run("batched16_floor_gather_records", c, gather_body, kv, copies=min(n, 4),
            extra={"op": "whole row records of the batch's 272,568 rows read through the tables by the "
                         "read-floor kernel (every byte a page-size-1 reader fetches), 1,024 workgroups"})
    del c
    c = wl.layer_decode(0, with_new_token=False)
    W = 4095
    run("window4095", c, rows_body(W), W * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD,
        extra={"workload": "32K-context GQA-8 decode with a 4,095-key sliding window"})
    c = wl.layer_decode(0)
    run("window4095_append_step", c, lambda case, pools: append_body(case, pools, W),
        W * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD,
        extra={"workload": "32K-context GQA-8 decode step (new token quantized on write) with a 4,095-key "
                           "sliding window"})
    return res


def model_step_timing(fk, wl, dev, args, bf, stream):
    """The 48-layer step at 40,000 context: one fused call per layer over 48
    distinct 40,290-row pools (2 GB, larger than the Infinity Cache, so every
    layer reads its rows from HBM); one layer's draws are copied into all 48
    pools, which does not change the timing.  One warm-up step, then exactly
    --model-step-steps timed steps (48 calls each) in one graph."""
    import torch
    table = wl.model_step_table(0)
    c = wl.model_step_layer(0, table)
    layers = 48
    pools = rotated_pools(fk, c, args.layout, layers, dev, bf)
    q, nk, nv = bf(c.q), bf(c.new_k), bf(c.new_v)
    t, sl = torch.from_numpy(c.table).to(dev), torch.from_numpy(c.seq_lens).to(dev)
    slot = torch.from_numpy(c.table[:, -1].copy()).to(dev)
    ws = fk.decode_workspace(1, c.n_q_heads, device=dev)
    out = torch.empty_like(q)
    K = max(1, args.model_step_steps)
    ms = time_exact(stream, lambda i: fk.fp8kv_decode_attn_append(pools[i % layers], q, nk, nv, slot, t, sl,
                                                                  c.max_seq_len, c.sm_scale, workspace=ws, out=out,
                                                                  stream=stream),
                    layers * K, layers)
    del pools
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    kv = layers * c.max_seq_len * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD
    step_s = ms * layers * 1e-3
    return {"workload": "48-layer decode step at 40,000 context (one token: quantize-on-write + attention per "
                        "layer), 48 x 40,290-row pools, 2.04 GB",
            "steps": K, "us_per_step": round(step_s * 1e6, 2), "us_per_layer": round(ms * 1e3, 3),
            "kv_bytes": kv, "kv_gbps": round(kv / step_s / 1e9, 1),
            "hbm_frac": round(kv / step_s / 1e9 / HBM_PEAK_GBPS, 4)}


def calibration_copies(dev, mib: int = 64, n: int = 4):
    """Plain device-to-device copies of known size, so that rocprofv3 byte
    counters of the decode kernel can be scaled against a kernel whose traffic
    is known (read mib MiB + write mib MiB per copy)."""
    import torch
    bufs = [torch.empty(mib << 20, dtype=torch.uint8, device=dev) for _ in range(2 * n)]
    for i in range(n):
        bufs[2 * i + 1].copy_(bufs[2 * i])
    torch.cuda.synchronize()


def cpu_baseline(case, budget_s: float, with_model_step: bool = True):
    """The oracle (as it stands) on the host: quantize the new K/V row + fp64
    decode attention over all 32,768 rows, repeated until the time budget, on
    all host threads and then on one; and, for the 48-layer 40K step, the same
    per layer over 40,000 rows (per-step figures are 48 layers' worth)."""
    import oracle

    def timed_step(c, budget):
        kc, ks = oracle.quantize_rows(c.k_rows)
        vc, vs = oracle.quantize_rows(c.v_rows)
        row = int(c.table[0, -1])
        reps, t0 = 0, time.perf_counter()
        while True:
            nkc, nks = oracle.quantize_rows(c.new_k)
            nvc, nvs = oracle.quantize_rows(c.new_v)
            kc[row], ks[row], vc[row], vs[row] = nkc[0], nks[0], nvc[0], nvs[0]
            oracle.decode_attention(c.q, kc, vc, ks, vs, c.table, c.seq_lens, c.sm_scale, c.n_kv_heads)
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    kv = case.max_seq_len * case.n_kv_heads * KV_BYTES_PER_ROW_HEAD
    cores = oracle.num_threads()
    reps, el = timed_step(case, budget_s)
    oracle.set_num_threads(1)
    try:
        reps1, el1 = timed_step(case, budget_s / 2)
    finally:
        oracle.set_num_threads(cores)
    res = {"value": round(kv * reps / el / 1e9, 3), "unit": "GB/s", "cores": cores,
           "kind": "oracle",
           "sample": f"full 32K-context layer step (quantize new K/V row + fp64 decode attention, "
                     f"32 q heads x 32,768 rows) repeated {reps} times in {el:.1f} s",
           "us_per_layer": round(el / reps * 1e6, 1),
           "single_core": {"value": round(kv * reps1 / el1 / 1e9, 3), "unit": "GB/s",
                           "us_per_layer": round(el1 / reps1 * 1e6, 1),
                           "sample": f"the same step repeated {reps1} times in {el1:.1f} s on 1 thread"}}
    if with_model_step:
        from fp8_kv_cache_row_amd import workloads as wl
        c = wl.model_step_layer(0, wl.model_step_table(0))
        kv3 = c.max_seq_len * c.n_kv_heads * KV_BYTES_PER_ROW_HEAD
        r3, e3 = timed_step(c, budget_s / 2)
        res["model_step_48x40k"] = {
            "value": round(kv3 * r3 / e3 / 1e9, 3), "unit": "GB/s", "cores": cores,
            "us_per_layer": round(e3 / r3 * 1e6, 1), "us_per_step": round(48 * e3 / r3 * 1e6, 1),
            "sample": f"one 40,000-row layer of the 48-layer step (quantize new K/V row + fp64 decode attention) "
                      f"repeated {r3} times in {e3:.1f} s; a step is 48 such layers"}
    return res


def time_exact(stream, body, steps, warmup, offset=0):
    """ms per call of exactly `steps` calls body(offset + warmup + i), after
    `warmup` untimed calls body(offset + i): one HIP graph each (captured after
    an untimed eager pass), HIP events on the graph's stream."""
    import torch
    g_w = capture_graph(stream, lambda i: body(offset + i), warmup) if warmup > 0 else None
    g_k = capture_graph(stream, lambda i: body(offset + warmup + i), steps)
    torch.cuda.synchronize()
    if g_w is not None:
        g_w.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    with torch.cuda.stream(stream):
        e0.record(stream)
        g_k.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del g_w, g_k
    return ms


def load_guard():
    """The oracle's output of the seed-0 fused step (tests/golden), [Hq][128] fp64."""
    import numpy as np
    rows = [list(map(float, line.split())) for line in open(GUARD_FILE) if line.strip() and not line.startswith("#")]
    return np.array(rows, dtype=np.float64)


def headline_round(fk, B, wl, dev, args, seed, stream, bf):
    """One seeded round of the 32K-context layer: per-item ms (exact step counts)."""
    import numpy as np
    import torch
    case = wl.layer_decode(seed)
    L, Hq, Hkv = case.max_seq_len, case.n_q_heads, case.n_kv_heads
    n_pools = 1 if args.warm else max(1, args.pools)
    pools = rotated_pools(fk, case, args.layout, n_pools, dev, bf)
    q = bf(case.q)
    table = torch.from_numpy(case.table).to(dev)
    lens = torch.from_numpy(case.seq_lens).to(dev)
    new_k, new_v = bf(case.new_k), bf(case.new_v)
    slot = torch.from_numpy(case.table[:, -1].copy()).to(dev)
    ws = fk.decode_workspace(1, Hq, args.max_splits, dev)
    out = torch.empty_like(q)
    one = torch.zeros(1, device=dev)
    torch.cuda.synchronize()
    lib = B.load()
    sp = ctypes.c_void_p(stream.cuda_stream)
    wsb = ws.numel()

    def chk(st, what):
        if st:
            raise B.Fp8KvError(st, what)

    def quant(p):
        chk(lib.fp8kv_quantize_rows(ctypes.byref(p.layer), new_k.data_ptr(), new_v.data_ptr(), Hkv * 128,
                                    slot.data_ptr(), 1, sp), "fp8kv_quantize_rows")

    def stage1(p):
        chk(lib.fp8kv_decode_stage1(ctypes.byref(p.layer), q.data_ptr(), 1, Hq, table.data_ptr(), L, lens.data_ptr(),
                                    L, case.sm_scale, args.max_splits, ws.data_ptr(), wsb, sp), "fp8kv_decode_stage1")

    def stage1_valu(p):
        chk(lib.fp8kv_decode_stage1_valu(ctypes.byref(p.layer), q.data_ptr(), 1, Hq, table.data_ptr(), L,
                                         lens.data_ptr(), L, case.sm_scale, args.max_splits, ws.data_ptr(), wsb, sp),
            "fp8kv_decode_stage1_valu")

    def merge():
        chk(lib.fp8kv_decode_merge(1, Hq, 128, args.max_splits, ws.data_ptr(), wsb, out.data_ptr(), sp),
            "fp8kv_decode_merge")

    def decode(p):
        chk(lib.fp8kv_decode_attn(ctypes.byref(p.layer), q.data_ptr(), 1, Hq, table.data_ptr(), L, lens.data_ptr(),
                                  L, case.sm_scale, args.max_splits, ws.data_ptr(), wsb, out.data_ptr(), sp),
            "fp8kv_decode_attn")

    def append(p):
        chk(lib.fp8kv_decode_attn_append(ctypes.byref(p.layer), q.data_ptr(), 1, Hq, new_k.data_ptr(),
                                         new_v.data_ptr(), Hkv * 128, slot.data_ptr(), table.data_ptr(), L,
                                         lens.data_ptr(), L, case.sm_scale, args.max_splits, ws.data_ptr(), wsb,
                                         out.data_ptr(), sp), "fp8kv_decode_attn_append")

    def tiny():
        with torch.cuda.stream(stream):
            one.add_(1.0)

    P = lambda i: pools[i % n_pools]  # noqa: E731
    items = {
        "step": lambda i: append(P(i)),
        "step_three_calls": lambda i: (quant(P(i)), decode(P(i))),
        "stage1": lambda i: stage1(P(i)),
        "stage1_valu": lambda i: stage1_valu(P(i)),
        "merge": lambda i: merge(),
        "quantize_new_row": lambda i: quant(P(i)),
    }
    if not args.warm and not args.no_warm_column:
        items["step_warm"] = lambda i: append(pools[0])
    if not args.no_floors and seed == 0:
        items["stage1_then_tiny_kernel"] = lambda i: (stage1(P(i)), tiny())
        if args.layout.startswith("interleaved"):
            FL = floor_lib()
            sink = torch.zeros(4, dtype=torch.int32, device=dev)
            rec = pools[0].record.shape[1]

            def gather(p):
                if FL.fp8kv_floor_gather(p.record.data_ptr(), case.pool_rows, rec, table.data_ptr(), L, 256,
                                         sink.data_ptr(), sp):
                    raise RuntimeError("fp8kv_floor_gather failed")
            items["floor_gather_records"] = lambda i: gather(P(i))
    order = list(items)
    np.random.default_rng(1000 + seed).shuffle(order)
    res = {}
    for name in order:
        res[name] = time_exact(stream, items[name], args.steps, args.warmup)
    res["order"] = order

    # correctness guard on the configuration just timed: the fused step (seed 0)
    # against the stored oracle output, and against the two-call decode with
    # another split count over the pool the step has just written into
    append(pools[0])
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)[0]
    ref2 = fk.fp8kv_decode_attn(pools[0], q, table, lens, L, case.sm_scale, max_splits=8)
    torch.cuda.synchronize()
    if not torch.allclose(out.float(), ref2.float(), atol=2e-2, rtol=0):
        raise RuntimeError("bench guard: the fused step disagrees with fp8kv_decode_attn (split cap 8)")
    if seed == 0 and os.path.exists(GUARD_FILE):
        ref = load_guard()
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        mab = float(np.abs(got - ref).max())
        res["guard"] = {"rel_l2": rel, "max_abs": mab}
        if not (rel <= 5e-3 and mab <= 2e-2):
            raise RuntimeError(f"bench guard: fused step vs the stored oracle output rel_l2={rel:.3e} max_abs={mab:.3e}")
    del pools
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res, case


def floor_lib():
    """The benchmark's read-floor kernels (fp8_kv_cache_row_amd/floor/read_floor.hip)."""
    from fp8_kv_cache_row_amd import build as hb
    if not os.path.exists(hb.FLOOR_LIB):
        raise RuntimeError(f"{hb.FLOOR_LIB} is missing: build it first")
    L = ctypes.CDLL(hb.FLOOR_LIB)
    vp, i64, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32
    L.fp8kv_floor_read.argtypes = [vp, i64, i32, vp, vp]
    L.fp8kv_floor_gather.argtypes = [vp, i64, i64, vp, i32, i32, vp, vp]
    return L


def wave_timeline(fk, B, wl, dev, bf, stream, layout: str, launches: int = 24, warm_launches: int = 12):
    """Per-wave timestamps of the 32K-context stage 1 from the measurement
    build (libfp8kv_timeline.so: the same kernels with the 100 MHz real-time
    counter recorded at six points by lane 0 of every wave), one launch at a
    time over the headline's 12 rotated cold pools.  Times are microseconds
    from the launch's first wave entry; the instrumented kernel runs a little
    slower than the product one (each point is a scheduling barrier and a
    counter read)."""
    import numpy as np
    import torch
    path = os.path.join(ROOT, "fp8_kv_cache_row_amd", "libfp8kv_timeline.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it first (python -c 'import __graft_entry__ as g; g.build()')")
    TL = ctypes.CDLL(path)
    main_lib = B.load()
    TL.fp8kv_decode_stage1.argtypes = main_lib.fp8kv_decode_stage1.argtypes
    TL.fp8kv_decode_stage1.restype = main_lib.fp8kv_decode_stage1.restype
    TL.fp8kv_timeline_read.argtypes = [ctypes.c_void_p, ctypes.c_long]
    case = wl.layer_decode(0)
    L, Hq = case.max_seq_len, case.n_q_heads
    pools = rotated_pools(fk, case, layout, 12, dev, bf)
    q = bf(case.q)
    table = torch.from_numpy(case.table).to(dev)
    lens = torch.from_numpy(case.seq_lens).to(dev)
    ws = fk.decode_workspace(1, Hq, 0, dev)
    n_wg, n_w, n_pt = 256, 8, 8  # the 32K layer's grid: 64 splits x 4 KV heads, 8 waves each
    host = np.zeros(n_wg * n_w * n_pt, np.uint64)
    sp = ctypes.c_void_p(stream.cuda_stream)
    runs = []
    for it in range(warm_launches + launches):
        if TL.fp8kv_timeline_clear() != 0:
            raise RuntimeError("fp8kv_timeline_clear failed")
        torch.cuda.synchronize()
        st = TL.fp8kv_decode_stage1(ctypes.byref(pools[it % 12].layer), q.data_ptr(), 1, Hq, table.data_ptr(), L,
                                    lens.data_ptr(), L, case.sm_scale, 0, ws.data_ptr(), ws.numel(), sp)
        if st:
            raise B.Fp8KvError(st, "fp8kv_decode_stage1 (timeline build)")
        torch.cuda.synchronize()
        if TL.fp8kv_timeline_read(host.ctypes.data, host.size) != 0:
            raise RuntimeError("fp8kv_timeline_read failed")
        if it >= warm_launches:
            runs.append(host.reshape(n_wg, n_w, n_pt)[:, :, :6].astype(np.int64).copy())
    T = np.stack(runs)  # [launch, workgroup, wave, point]
    if (T == 0).any():
        raise RuntimeError("timeline: a wave left a point unrecorded")
    rel = (T - T[..., 0].min(axis=(1, 2))[:, None, None, None]) * 1e-2  # 100 MHz ticks -> us
    names = ["entry", "row_indices_in", "scales_in", "step0_done", "steps_done", "partials_stored"]
    by_wave = {nm: [round(float(x), 2) for x in rel[..., k].mean(axis=(0, 1))] for k, nm in enumerate(names)}
    wg_end = rel[..., 5].max(axis=2)
    span = rel[..., 5].max(axis=(1, 2))
    lo, hi = rel[:, :, :4], rel[:, :, 4:]
    return {
        "launches": launches,
        "pool_layout": layout,
        "us_by_wave_index": by_wave,
        "span_us_median": round(float(np.median(span)), 2),
        "workgroup_end_us": {"p10": round(float(np.percentile(wg_end, 10)), 2),
                             "p50": round(float(np.median(wg_end)), 2),
                             "p90": round(float(np.percentile(wg_end, 90)), 2)},
        "scales_in_waves_4_7_minus_0_3_us": round(float(hi[..., 2].mean() - lo[..., 2].mean()), 2),
        "compute_after_scales_in_waves_4_7_us": round(float((hi[..., 4] - hi[..., 2]).mean()), 2),
        "workgroup_merge_after_last_wave_us": round(float((rel[..., 0, 5] - rel[..., 4].max(axis=2)).mean()), 2),
        "workgroup_to_xcd": "workgroup x + 32 y runs on XCD x & 7 (split 8y + (x & 7), KV head x >> 3)",
        "note": "points: wave entry; its first group's row indices in LDS; its scales in (every code load "
                "issued); its first 32-key step done; all its steps done; the workgroup's partials stored",
    }


def read_floors(dev, stream, steps, warmup, nbytes=34603008):
    """Cold reads rotated over distinct buffers: a plain contiguous read kernel
    of 34,603,008 bytes (and of 2x and 8x that, to show how a one-shot read's
    rate grows with its size), and a library reduction of 34,603,008 bytes
    (torch.sum over the rows of an fp32 [33,792][256] tensor, one workgroup per
    row block, no cross-workgroup step) for comparison."""
    import torch
    L = floor_lib()
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    res = {}

    def record(name, ms, nb, what):
        gbps = nb / (ms * 1e-3) / 1e9
        res[name] = {"us": round(ms * 1e3, 3), "bytes": nb, "gbps": round(gbps, 1),
                     "hbm_frac": round(gbps / HBM_PEAK_GBPS, 4), "op": what}

    for mult, n in ((1, 12), (2, 8), (8, 4)):  # every size's rotation exceeds the 256 MB Infinity Cache
        nb = nbytes * mult
        bufs = [torch.full((nb // 4,), float(i + 1), dtype=torch.float32, device=dev) for i in range(n)]

        def contiguous(i, bufs=bufs, nb=nb, n=n):
            if L.fp8kv_floor_read(bufs[i % n].data_ptr(), nb, 512, sink.data_ptr(), sp):
                raise RuntimeError("fp8kv_floor_read failed")

        name = "contiguous_read" if mult == 1 else f"contiguous_read_x{mult}"
        record(name, time_exact(stream, contiguous, steps, warmup), nb,
               f"contiguous 16-byte loads, 512 workgroups x 512 lanes, eight loads in flight per lane, {n} rotated "
               "buffers, graph replay")
        if mult == 1:
            rows = nb // (256 * 4)
            views = [b.view(rows, 256) for b in bufs]
            outs = torch.empty((rows,), dtype=torch.float32, device=dev)

            def reduction(i):
                with torch.cuda.stream(stream):
                    torch.sum(views[i % n], dim=1, out=outs)

            record("library_reduction", time_exact(stream, reduction, steps, warmup), nb,
                   f"torch.sum(dim=1) of an fp32 [{rows}][256] tensor, {n} rotated buffers, graph replay")
            del views
        del bufs
        torch.cuda.empty_cache()
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus} GPUs, WORLD_SIZE={world}); this "
              "path has no multi-GPU decomposition to time.", file=sys.stderr, flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0 or args.rounds < 1:
        print("bench.py: --steps and --rounds must be >= 1, --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp8_kv_cache_row_amd as fk
    from fp8_kv_cache_row_amd import binding as B
    from fp8_kv_cache_row_amd import workloads as wl

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    if args.calibration_copy:
        calibration_copies(dev)

    def bf(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    stream = torch.cuda.Stream(device=dev)
    samples = {}
    guard = None
    case0 = None
    for r in range(args.rounds):
        res, case = headline_round(fk, B, wl, dev, args, r, stream, bf)
        if r == 0:
            case0 = case
            guard = res.pop("guard", None)
        for k, v in res.items():
            samples.setdefault(k, []).append(v)
    med = {k: statistics.median(v) for k, v in samples.items() if k != "order"}
    L, Hq, Hkv = case0.max_seq_len, case0.n_q_heads, case0.n_kv_heads
    kv_bytes = L * Hkv * KV_BYTES_PER_ROW_HEAD
    step_ms, s1_ms = med["step"], med["stage1"]
    s1_gbps = kv_bytes / (s1_ms * 1e-3) / 1e9
    step_gbps = kv_bytes / (step_ms * 1e-3) / 1e9
    n_pools = 1 if args.warm else max(1, args.pools)
    us = lambda ms: round(ms * 1e3, 3)  # noqa: E731
    res = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "single-layer batch-1 GQA-8 FP8 decode at 32K context",
            "n_q_heads": Hq, "n_kv_heads": Hkv, "head_dim": 128, "context": L,
            "pool_rows": case0.pool_rows, "page_size": 1, "pool_layout": args.layout,
            "kv_cache": "E4M3FN codes + fp32 per-row scales", "query": "bf16",
            "hbm_state": "warm (one pool)" if args.warm else f"cold ({n_pools} pool copies rotated)",
            "step": "fp8kv_decode_attn_append: stage 1 + merge that quantizes and adds the new K/V row "
                    "(HIP graph replay)",
        },
        "rounds": args.rounds,
        "round_protocol": f"{args.rounds} seeded rounds (workload seed = round), items in a seeded shuffled order; "
                          f"each item: {args.warmup} untimed steps, then exactly {args.steps} timed steps in one "
                          "graph; value and ms_per_step are medians over rounds",
        "us_per_layer": us(step_ms),
        "pct_hbm_peak": round(100 * step_gbps / HBM_PEAK_GBPS, 2),
        "kv_bytes_per_layer": kv_bytes,
        "us_per_layer_three_calls": us(med["step_three_calls"]),
        "us_per_layer_warm": us(med["step_warm"]) if "step_warm" in med else None,
        "kernels_us": {"quantize_new_row": us(med["quantize_new_row"]), "decode_stage1": us(s1_ms),
                       "decode_merge": us(med["merge"]), "decode_stage1_valu": us(med["stage1_valu"])},
        "stage1_mfma_vs_valu": {"mfma_us": us(s1_ms), "valu_us": us(med["stage1_valu"]),
                                "valu_over_mfma": round(med["stage1_valu"] / s1_ms, 3),
                                "note": "fp8kv_decode_stage1 (bf16 MFMA) against fp8kv_decode_stage1_valu (fp32 "
                                        "vector FMAs), same grid, same cold rotation, same partials"},
        "samples_us": {k: [us(x) for x in v] for k, v in samples.items() if k != "order"},
        "sample_order": samples.get("order"),
        "guard": guard,
        "roofline": {
            "kernel": "decode_stage1",
            "bound": "hbm",
            "achieved": round(s1_gbps, 2),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(s1_gbps / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(args.layout, 0 if args.warm else args.pools),
        },
    }
    if not args.no_floors:
        fl = read_floors(dev, stream, args.steps, args.warmup)
        res["roofline"]["read_floor_us"] = fl["contiguous_read"]["us"]
        res["roofline"]["frac_of_read_floor"] = round(fl["contiguous_read"]["us"] / us(s1_ms), 4)
        res["floors"] = dict(fl)
        if "floor_gather_records" in med:
            g_ms = med["floor_gather_records"]
            rec = res["config"]["pool_layout"]
            res["floors"]["gathered_records"] = {
                "us": us(g_ms), "algorithmic_bytes": kv_bytes, "gbps": round(kv_bytes / (g_ms * 1e-3) / 1e9, 1),
                "hbm_frac": round(kv_bytes / (g_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                "op": f"whole {rec} row records of the 32,768 table rows read through the table (every byte a "
                      "page-size-1 reader fetches), 256 workgroups, the headline's rotated pools"}
        if "stage1_then_tiny_kernel" in med:
            res["floors"]["dependent_launch_after_stage1_us"] = us(med["stage1_then_tiny_kernel"] - s1_ms)
    if args.timeline:
        res["wave_timeline"] = wave_timeline(fk, B, wl, dev, bf, stream, args.layout)
    if not args.no_model_step:
        res["model_step_48x40k"] = model_step_timing(fk, wl, dev, args, bf, stream)
    if not args.no_prefill:
        res["prefill"] = prefill_timing(fk, wl, dev)
    if not args.no_variants:
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        res["variants"] = variants_timing(fk, wl, dev, args, bf)
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(case0, args.cpu_seconds, with_model_step=not args.no_model_step)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
