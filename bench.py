"""Benchmark of the SRFT-rotated int4 KV-cache hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]

One step is one decode step of the hot path over every layer of the workload (layers folded
into the batch): append-quantize the new token's K and V (write path), then fused
dequant + decode attention over the whole cache (read path).  The fp16-KV decode of the same
build and the bulk (prefill) quantize are timed the same way and reported beside it.

The default workload is the long-context serving shard (32 layers x 8 sequences x 8 kv heads,
32 query heads, d = 128, 32768 tokens, int4): the largest configuration that fits one GPU.

Timing: the K timed steps of each measured unit are captured in HIP graphs, step i of graph j
reading cache copy (j K + i) mod R (R copies span >= 1 GB, four times the MI355X Infinity Cache;
the timed replays cycle through the graphs when R > K), so every step reads cold data and host
launch overhead is paid once per graph.  A graph of W warm-up steps runs first; each timed replay
is bracketed by device synchronizations and HIP events.  Inputs are resident in HBM before the
timed region starts.

Prints ONE JSON line (rank 0).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
COLD_BYTES = 1 << 30
MAX_COPIES = 256
METRIC = "decode-attn effective KV GB/s & % HBM peak; quantize Mvectors/s; vs fp16-KV"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0, help="timed steps (default: 4 x the cache copies)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5,
                    help="1 tiny, 2 Qwen-like, 3 Gemma-like (d 256, K8V4), 4 48 L x 16 H, 5 serving shard (default)")
    ap.add_argument("--seq", type=int, default=0, help="override the workload's sequence length (a sweep point)")
    ap.add_argument("--k-bits", type=int, choices=(4, 8), default=0, help="override the workload's K width")
    ap.add_argument("--v-bits", type=int, choices=(4, 8), default=0, help="override the workload's V width")
    ap.add_argument("--transform", choices=("srft", "srht"), default="srft",
                    help="the rotation: SRFT (default) or the SRHT variant")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the CPU oracle sample")
    ap.add_argument("--pmc-run", action="store_true",
                    help="eager decode launches plus a plain copy of known size, for rocprofv3 --pmc passes")
    return ap.parse_args()


class Timer:
    """Time exactly `steps` steps per replay: a HIP graph holds `steps` steps, step i of graph j on
    cache copy (j * steps + i) mod n_copies.  When the copies outnumber the steps, several graphs
    cover them all and the timed replays cycle through the graphs, so the data read between two
    replays of one graph spans every copy (>= 1 GB) whatever `steps` is.  Host launch overhead is
    paid once per graph.  A graph of `warmup` steps runs first, then the timed graphs are replayed
    untimed for at least 100 ms (steady clocks); each timed replay is bracketed by device
    synchronizations and HIP events on the replaying stream, `repeats` replays for the spread."""

    def __init__(self, torch):
        self.torch = torch

    def run(self, step_fn, n_copies, steps, warmup, repeats=7):
        torch = self.torch
        if warmup > 0:
            gw = capture(torch, lambda: [step_fn(i % n_copies) for i in range(warmup)])
            gw.replay()
            torch.cuda.synchronize()
            del gw
        n_graphs = max(1, -(-n_copies // steps))
        graphs = [capture(torch, lambda j=j: [step_fn((j * steps + i) % n_copies) for i in range(steps)])
                  for j in range(n_graphs)]
        repeats = max(repeats, n_graphs)
        # settle: replay for at least 100 ms so that clocks and caches are in steady state
        t_settle, n_settle = time.perf_counter(), 0
        while n_settle < 2 * n_graphs or time.perf_counter() - t_settle < 0.1:
            graphs[n_settle % n_graphs].replay()
            torch.cuda.synchronize()
            n_settle += 1
        times = []
        for r in range(repeats):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            e0.record()
            graphs[r % n_graphs].replay()
            e1.record()
            torch.cuda.synchronize()
            wall = time.perf_counter() - t0
            times.append((e0.elapsed_time(e1), wall))
        del graphs
        per = np.array([t / steps for t, _ in times])
        return {"ms_mean": float(per.mean()), "ms_median": float(np.median(per)),
                "ms_p10": float(np.percentile(per, 10)), "ms_p90": float(np.percentile(per, 90)),
                "ms_min": float(per.min()), "ms_max": float(per.max()), "repeats": repeats, "steps": steps,
                "graphs": n_graphs, "copies": n_copies,
                "wall_ms_per_step": 1e3 * float(np.mean([w for _, w in times])) / steps}


def capture(torch, fn):
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # warm (first-launch work) outside the capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def cpu_info():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    return {"cpu_model": model, "os_cpu_count": os.cpu_count(), "usable_cpus": usable}


def cpu_baseline(w, budget_s, transform="srft"):
    """Time the CPU oracle, as it stands, on a bounded sample of the same workload: units of one
    sequence of one layer (all its kv heads and query heads), drawn with the workload's recipe,
    each quantized (K and V, oracle write path) and decoded (oracle attention over the oracle's
    planes) until `budget_s` of oracle time is spent.  BLAS threads are pinned with threadpoolctl:
    once to one thread, once to every usable CPU (capped by OMP_NUM_THREADS when set)."""
    import dataclasses

    from threadpoolctl import threadpool_limits

    from kv_cache_quantization_srft_amd import synth
    from oracle import kvq_oracle as O

    info = cpu_info()
    all_threads = info["usable_cpus"]
    if os.environ.get("OMP_NUM_THREADS", "").isdigit():
        all_threads = min(all_threads, int(os.environ["OMP_NUM_THREADS"]))
    s = synth.signs(w)
    w1 = dataclasses.replace(w, batch=1)  # one sequence of a layer per unit

    G = w.q_heads // w.kv_heads

    def run(threads, budget):
        units, t_dec, t_q, vec_q, t_start, c_start = 0, 0.0, 0.0, 0, time.perf_counter(), time.process_time()
        with threadpool_limits(limits=threads):
            while units < 1 or time.perf_counter() - t_start < budget:
                layer, j = divmod(units, w.kv_heads)
                layer %= w.layers
                k = synth.kv(w1, layer, synth.K_TENSOR)[:, j:j + 1]
                v = synth.kv(w1, layer, synth.V_TENSOR)[:, j:j + 1]
                q = synth.query(w1, layer)[:, j * G:(j + 1) * G]
                lk = O.calibrate_lambda(k, s, w.n_cal, transform)[:, :, None, :] if w.calibrate else 1.0
                lv = O.calibrate_lambda(v, s, w.n_cal, transform)[:, :, None, :] if w.calibrate else 1.0
                t0 = time.perf_counter()
                kc, ks = O.quantize(k, s, lk, w.k_bits, transform=transform)
                vc, vs = O.quantize(v, s, lv, w.v_bits, transform=transform)
                t1 = time.perf_counter()
                O.decode_attention_quantized(q, kc, ks, vc, vs, s, s, lk, lv, w.seq_len, transform=transform)
                t2 = time.perf_counter()
                t_q += t1 - t0
                t_dec += t2 - t1
                vec_q += k.size // w.head_dim + v.size // w.head_dim
                units += 1
        # cores the run kept busy: process CPU time (all threads) over wall time
        busy = (time.process_time() - c_start) / max(time.perf_counter() - t_start, 1e-9)
        bytes_unit = w.seq_len * (w.head_dim * (w.k_bits + w.v_bits) // 8 + 2 * 2 * w.head_dim // 16)
        return {"decode_GBps": bytes_unit * units / t_dec / 1e9, "decode_ms_per_unit": 1e3 * t_dec / units,
                "quantize_Mvectors_per_s": vec_q / t_q / 1e6, "units": units, "blas_threads": threads,
                "cores_busy": round(busy, 2)}

    single = run(1, budget_s / 2)
    multi = run(all_threads, budget_s / 2)
    units_step = w.layers * w.batch * w.kv_heads
    return {
        "value": round(multi["decode_GBps"], 4), "unit": "GB/s", "cores": max(1, round(multi["cores_busy"])),
        "kind": "oracle", "blas_threads_allowed": all_threads,
        "sample": (f"{multi['units']} units of one (layer, sequence, kv head) with its {G} query heads over "
                   f"{w.seq_len} tokens (a decode step of the workload is {units_step} such units): oracle write "
                   f"path on K and V, then oracle decode (dequantize by the O(d^2) inverse {transform.upper()} + "
                   f"attention); numpy float64 with BLAS pinned to {all_threads} threads (the oracle's DFT is an "
                   f"einsum that runs on one core; `cores` is the measured CPU time over wall time)"),
        "decode_ms_per_step_extrapolated": round(multi["decode_ms_per_unit"] * units_step, 1),
        "quantize_Mvectors_per_s": round(multi["quantize_Mvectors_per_s"], 4),
        "single_thread": {k: (round(v, 4) if isinstance(v, float) else v) for k, v in single.items()},
        "host": info,
    }


PMC_COPY_BYTES = 1 << 30  # the plain copy whose counter readings scale the decode's


def decode_sources_sha():
    """sha256 over the decode kernel's sources: the traffic figure of a profile applies only to
    the kernel it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "csrc")
    for name in ("kvq_decode_q.h", "kvq_decode_q128.hip", "kvq_decode_q256.hip", "kvq_decode_common.h",
                 "kvq_wave_rot.h", "kvq_internal.h", "kvq_device.h", "kvq_plan.cpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def profiled_traffic(workload_name):
    """HBM bytes per decode launch from the committed rocprofv3 --pmc summary of this workload
    (FETCH_SIZE + WRITE_SIZE, each scaled by the same counter's reading for a plain copy of known
    size), or None when there is none or the decode sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"kvq_decode_traffic_{workload_name}.md")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if line.startswith("- `") and "`: " in line:
                k, v = line[3:].split("`: ", 1)
                vals[k] = v.strip()
    if vals.get("decode_sources_sha") != decode_sources_sha():
        return None
    try:
        return int(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1",
                          "detail": "multi-GPU sharding is a design note only (DESIGN.md)"}))
        sys.exit(2)
    import torch

    from kv_cache_quantization_srft_amd import kvq, synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    w = synth.WORKLOADS[args.workload]
    import dataclasses
    if args.seq > 0:
        w = dataclasses.replace(w, seq_len=args.seq)
    if args.k_bits:
        w = dataclasses.replace(w, k_bits=args.k_bits)
    if args.v_bits:
        w = dataclasses.replace(w, v_bits=args.v_bits)
    L, B, H, Hq, d, S = w.layers, w.batch, w.kv_heads, w.q_heads, w.head_dim, w.seq_len
    LB = L * B
    log(f"workload {w.name}: layers {L} batch {B} kv {H} q {Hq} d {d} seq {S} K{w.k_bits}V{w.v_bits}")
    s = torch.from_numpy(synth.signs(w)).cuda()
    lay = kvq.make_layout(LB, H, Hq, d, S, k_bits=w.k_bits, v_bits=w.v_bits, transform=args.transform)

    # ---- synthetic cache, resident in HBM (layers folded into the batch) ----
    t0 = time.perf_counter()
    if w.cid in (4, 5):
        kx = torch.cat([synth.torch_kv(w, l, synth.K_TENSOR, "cuda") for l in range(L)])
        vx = torch.cat([synth.torch_kv(w, l, synth.V_TENSOR, "cuda") for l in range(L)])
    else:
        kx = torch.from_numpy(np.concatenate([synth.kv(w, l, synth.K_TENSOR) for l in range(L)])).cuda()
        vx = torch.from_numpy(np.concatenate([synth.kv(w, l, synth.V_TENSOR) for l in range(L)])).cuda()
    q = torch.from_numpy(np.concatenate([synth.query(w, l) for l in range(L)])).cuda()
    log(f"generated inputs in {time.perf_counter() - t0:.1f}s")

    lam_k = lam_v = None
    if w.calibrate:
        lam_k = torch.empty(LB * H * d, dtype=torch.float32, device="cuda")
        lam_v = torch.empty_like(lam_k)
        kvq.kvq_calibrate_lambda(lay, kx, S, w.n_cal, s, 0, lam_k)
        kvq.kvq_calibrate_lambda(lay, vx, S, w.n_cal, s, 0, lam_v)
    lbs = H * d if w.calibrate else 0

    def new_planes():
        return (torch.empty(kvq.kvq_codes_bytes(lay, w.k_bits), dtype=torch.uint8, device="cuda"),
                torch.empty(kvq.kvq_scales_bytes(lay) // 2, dtype=torch.int16, device="cuda"),
                torch.empty(kvq.kvq_codes_bytes(lay, w.v_bits), dtype=torch.uint8, device="cuda"),
                torch.empty(kvq.kvq_scales_bytes(lay) // 2, dtype=torch.int16, device="cuda"))

    def quantize_all(p, xk, xv):
        kvq.kvq_quantize(lay, w.k_bits, xk, 0, S, s, 0, lam_k, lbs, p[0], p[1])
        kvq.kvq_quantize(lay, w.v_bits, xv, 0, S, s, 0, lam_v, lbs, p[2], p[3])

    base = new_planes()
    quantize_all(base, kx, vx)
    torch.cuda.synchronize()

    q_bytes = sum(t.numel() * t.element_size() for t in base)
    f16_bytes = 2 * kx.numel() * 2
    # enough copies to span COLD_BYTES, at most MAX_COPIES (tiny caches are latency-bound anyway,
    # and every copy is a node of the timing graph)
    n_q = min(MAX_COPIES, max(1, -(-COLD_BYTES // q_bytes)))
    n_f = min(MAX_COPIES, max(1, -(-COLD_BYTES // f16_bytes)))
    planes = [base] + [tuple(t.clone() for t in base) for _ in range(n_q - 1)]
    kv16 = [(kx, vx)] + [(kx.clone(), vx.clone()) for _ in range(n_f - 1)]
    torch.cuda.synchronize()
    log(f"cache copies: {n_q} quantized x {q_bytes / 1e6:.1f} MB, {n_f} fp16 x {f16_bytes / 1e6:.1f} MB")

    ws = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay, S), dtype=torch.uint8, device="cuda")
    out = torch.empty(LB * Hq * d, dtype=torch.float32, device="cuda")
    out16 = torch.empty_like(out)
    # the step's new token: the last cache position of every layer, re-quantized in place
    k_new = kx[:, :, S - 1:S].contiguous()
    v_new = vx[:, :, S - 1:S].contiguous()

    def decode(p):
        kvq.kvq_decode_attn(lay, q, p[0], p[1], p[2], p[3], S, None, s, s, 0, lam_k, lam_v, lbs, 0.0, ws, out)

    if args.pmc_run:
        # counter passes: 20 eager decode launches over the cache copies, then 4 plain copies of
        # PMC_COPY_BYTES (device to device) whose counter readings give the scale factor
        for i in range(20):
            decode(planes[i % len(planes)])
        torch.cuda.synchronize()
        for i in range(20):
            kvq.kvq_decode_attn_fp16(lay, q, kv16[i % len(kv16)][0], kv16[i % len(kv16)][1], S, None, 0.0, ws, out16)
        torch.cuda.synchronize()
        src = torch.empty(PMC_COPY_BYTES, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"pmc_run": w.name, "decode_launches": 20, "fp16_decode_launches": 20,
                          "copy_bytes": PMC_COPY_BYTES,
                          "decode_algorithmic_bytes": q_bytes, "decode_sources_sha": decode_sources_sha()}))
        return

    def step(p):
        # one launch: the new token's K and V go through the write path into position S - 1,
        # then decode attention over all S positions
        kvq.kvq_decode_attn_append(lay, q, k_new, v_new, p[0], p[1], p[2], p[3], S, None, s, s, 0, lam_k, lam_v,
                                   lbs, 0.0, ws, out)

    def step_unfused(p):
        kvq.kvq_quantize(lay, w.k_bits, k_new, S - 1, 1, s, 0, lam_k, lbs, p[0], p[1])
        kvq.kvq_quantize(lay, w.v_bits, v_new, S - 1, 1, s, 0, lam_v, lbs, p[2], p[3])
        decode(p)

    timer = Timer(torch)
    R = len(planes)
    steps = args.steps if args.steps > 0 else 4 * R
    res_step = timer.run(lambda i: step(planes[i]), R, steps, args.warmup)
    res_step3 = timer.run(lambda i: step_unfused(planes[i]), R, steps, args.warmup)
    res_dec = timer.run(lambda i: decode(planes[i]), R, steps, args.warmup)
    # Mode B: the model's cadence, one decode launch per layer (batch B each), L launches a step
    lay_l = kvq.make_layout(B, H, Hq, d, S, k_bits=w.k_bits, v_bits=w.v_bits, transform=args.transform)
    qv_l, out_l = q.view(L, -1), out.view(L, -1)
    lk_l = None if lam_k is None else lam_k.view(L, -1)
    lv_l = None if lam_v is None else lam_v.view(L, -1)
    views = [[tuple(t.view(L, -1)[l] for t in planes[i]) for l in range(L)] for i in range(R)]

    def decode_per_layer(i):
        for l in range(L):
            p = views[i][l]
            kvq.kvq_decode_attn(lay_l, qv_l[l], p[0], p[1], p[2], p[3], S, None, s, s, 0,
                                None if lk_l is None else lk_l[l], None if lv_l is None else lv_l[l], lbs, 0.0, ws,
                                out_l[l])

    steps_b = min(steps, max(8, 4096 // L))
    res_dec_b = timer.run(decode_per_layer, R, steps_b, min(args.warmup, 2))

    # achievable bandwidth: a plain device copy of 1 GiB (read + write)
    src = torch.empty(PMC_COPY_BYTES, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    res_copy = timer.run(lambda i: dst.copy_(src), 1, 4, 1)
    copy_gbps = 2 * PMC_COPY_BYTES / (res_copy["ms_median"] * 1e-3) / 1e9
    del src, dst

    Rf = len(kv16)
    steps_f = args.steps if args.steps > 0 else 4 * Rf
    res_f16 = timer.run(lambda i: kvq.kvq_decode_attn_fp16(lay, q, kv16[i][0], kv16[i][1], S, None, 0.0, ws, out16),
                        Rf, steps_f, args.warmup)
    # mode B for the fp16 comparator: one launch per layer
    out16_l = out16.view(L, -1)
    views16 = [[(kv16[i][0].view(L, -1)[l], kv16[i][1].view(L, -1)[l]) for l in range(L)] for i in range(Rf)]

    def decode_f16_per_layer(i):
        for l in range(L):
            kvq.kvq_decode_attn_fp16(lay_l, qv_l[l], views16[i][l][0], views16[i][l][1], S, None, 0.0, ws, out16_l[l])

    res_f16_b = timer.run(decode_f16_per_layer, Rf, min(steps_f, max(8, 4096 // L)), min(args.warmup, 2))
    # bulk quantize: all layers, K and V, from rotating fp16 copies into rotating planes
    nb = max(R, Rf)
    res_bq = timer.run(lambda i: quantize_all(planes[i % R], *kv16[i % Rf]), nb, 2 * nb, args.warmup)

    # the same write path with the rotation as an in-register FFT (one lane per vector)
    def quantize_all_fft(p, xk, xv):
        kvq.kvq_quantize_fft(lay, w.k_bits, xk, 0, S, s, 0, lam_k, lbs, p[0], p[1])
        kvq.kvq_quantize_fft(lay, w.v_bits, xv, 0, S, s, 0, lam_v, lbs, p[2], p[3])

    res_bqf = timer.run(lambda i: quantize_all_fft(planes[i % R], *kv16[i % Rf]), nb, 2 * nb, args.warmup)

    # paged cache: every copy cut into pages of PAGE tokens, stored in a shuffled page order and
    # addressed through a page table (kvq_decode_attn_paged); same tokens, same bytes read
    page = 256 if S % 256 == 0 else 64
    pps = -(-S // page)
    paged_planes, tables = [], []
    gen = torch.Generator(device="cpu")
    gen.manual_seed(7)
    for i in range(R):
        perm = torch.randperm(LB * pps, generator=gen).to("cuda")
        tbl = perm.view(LB, pps).to(torch.int32).contiguous()
        pp = []
        for t in planes[i]:
            w_ = t.numel() // (LB * H * S)
            nat = t.view(LB, H, S, w_)
            if pps * page != S:
                nat = torch.cat([nat, nat.new_zeros(LB, H, pps * page - S, w_)], 2)
            nat = nat.view(LB, H, pps, page, w_).permute(0, 2, 1, 3, 4).reshape(LB * pps, H, page, w_)
            out_p = torch.empty_like(nat)
            out_p[perm] = nat
            pp.append(out_p.view(-1))
        paged_planes.append(pp)
        tables.append(tbl)
    lay_pg = kvq.make_layout(LB, H, Hq, d, pps * page, k_bits=w.k_bits, v_bits=w.v_bits, transform=args.transform)
    ws_pg = torch.zeros(kvq.kvq_decode_attn_workspace_bytes(lay_pg, S), dtype=torch.uint8, device="cuda")
    out_pg = torch.empty_like(out)

    def decode_paged(i):
        p = paged_planes[i]
        kvq.kvq_decode_attn_paged(lay_pg, q, None, None, p[0], p[1], p[2], p[3], tables[i], pps, page, LB * pps, S,
                                  None, s, s, 0, lam_k, lam_v, lbs, 0.0, ws_pg, out_pg)

    res_pg = timer.run(decode_paged, R, steps, args.warmup)
    decode_paged(0)
    decode(planes[0])
    torch.cuda.synchronize()
    # identical plans give identical bits; a paged chunk is capped at 16384 tokens, so longer
    # single-chunk rows split into more chunks and differ only by the merge's rounding
    paged_diff = float((out_pg - out).abs().max())
    del paged_planes

    # kvq_attn: several query tokens (speculative verification of 4 drafted tokens: the last 4
    # positions attend causally) and a sliding window of 4096 positions, over the same cache
    n_spec = 4
    q_spec = torch.from_numpy(np.concatenate(
        [np.random.default_rng(l).standard_normal((B, n_spec, Hq, d)).astype(np.float16) for l in range(L)])).cuda()
    opts_spec = kvq.make_attn_opts(n_spec, 0)
    ws_spec = torch.zeros(kvq.kvq_attn_workspace_bytes(lay, opts_spec, S), dtype=torch.uint8, device="cuda")
    out_spec = torch.empty(LB * n_spec * Hq * d, dtype=torch.float32, device="cuda")
    win = min(4096, S)
    opts_win = kvq.make_attn_opts(1, win)
    ws_win = torch.zeros(kvq.kvq_attn_workspace_bytes(lay, opts_win, S), dtype=torch.uint8, device="cuda")

    def attn(i, opts, qq, wsp, o):
        p = planes[i]
        kvq.kvq_attn(lay, opts, qq, p[0], p[1], p[2], p[3], None, 0, 0, 0, S, None, s, s, 0, lam_k, lam_v, lbs, 0.0, wsp,
                     o)

    res_spec = timer.run(lambda i: attn(i, opts_spec, q_spec.view(-1), ws_spec, out_spec), R, steps, args.warmup)
    res_win = timer.run(lambda i: attn(i, opts_win, q, ws_win, out), R, steps, args.warmup)
    pl_spec = kvq.kvq_attn_launch_plan(lay, opts_spec, S)
    win_bytes = q_bytes // S * win
    del q_spec, out_spec, ws_spec, ws_win

    # one scale per vector (group = d), the per-token comparison mode of the write path: bulk
    # quantize of K and V, all layers, and the round-trip error of both modes on layer 0's K
    lay_pt = kvq.make_layout(LB, H, Hq, d, S, k_bits=w.k_bits, v_bits=w.v_bits, transform=args.transform,
                             group_size=d)
    pt = (torch.empty(kvq.kvq_codes_bytes(lay_pt, w.k_bits), dtype=torch.uint8, device="cuda"),
          torch.empty(kvq.kvq_scales_bytes(lay_pt) // 2, dtype=torch.int16, device="cuda"),
          torch.empty(kvq.kvq_codes_bytes(lay_pt, w.v_bits), dtype=torch.uint8, device="cuda"),
          torch.empty(kvq.kvq_scales_bytes(lay_pt) // 2, dtype=torch.int16, device="cuda"))

    def quantize_all_pt(xk, xv):
        kvq.kvq_quantize(lay_pt, w.k_bits, xk, 0, S, s, 0, lam_k, lbs, pt[0], pt[1])
        kvq.kvq_quantize(lay_pt, w.v_bits, xv, 0, S, s, 0, lam_v, lbs, pt[2], pt[3])

    res_pt = timer.run(lambda i: quantize_all_pt(*kv16[i % Rf]), Rf, 2 * Rf, args.warmup)
    quantize_all_pt(kx, vx)
    n_err = min(S, 4096)
    x0 = kx[:B, :, :n_err].float()
    round_trip = {}
    for name, lay_e, p in (("group16", lay, base), ("per_token", lay_pt, pt)):
        lay0 = kvq.make_layout(B, H, Hq, d, S, k_bits=w.k_bits, v_bits=w.v_bits, transform=args.transform,
                               group_size=lay_e.group_size)
        rec = torch.empty(B * H * n_err * d, dtype=torch.float32, device="cuda")
        kvq.kvq_dequantize(lay0, w.k_bits, p[0][:kvq.kvq_codes_bytes(lay0, w.k_bits)],
                           p[1][:kvq.kvq_scales_bytes(lay0) // 2], 0, n_err, s, 0,
                           None if lam_k is None else lam_k[:B * H * d], lbs, rec)
        round_trip[name] = float(torch.linalg.vector_norm(rec.view_as(x0) - x0) / torch.linalg.vector_norm(x0))
    del x0, rec

    dec_bytes = q_bytes  # every code and scale byte of the cache is read once per decode step
    n_vec = 2 * LB * H * S
    bq_bytes = n_vec * 2 * d + q_bytes
    dec_gbps = dec_bytes / (res_dec["ms_mean"] * 1e-3) / 1e9
    step_gbps = dec_bytes / (res_step["ms_mean"] * 1e-3) / 1e9
    f16_gbps = f16_bytes / (res_f16["ms_mean"] * 1e-3) / 1e9
    result = {
        "metric": METRIC,
        "value": round(step_gbps, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(res_step["ms_mean"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "layers": L, "batch": B, "kv_heads": H, "q_heads": Hq, "head_dim": d,
                   "seq_len": S, "k_bits": w.k_bits, "v_bits": w.v_bits, "group": 16,
                   "rotation": args.transform,
                   "lambda": "calibrated (first 512 tokens)" if w.calibrate else "1",
                   "storage": f"int{w.k_bits} K / int{w.v_bits} V codes + fp16 group scales",
                   "parallelism": "single GPU; layers folded into the batch", "cold_cache_copies": R},
        "step_breakdown": {"step": res_step, "step_three_launches": res_step3, "decode_only": res_dec,
                           "calls": {"step": "kvq_decode_attn_append (append + decode, one launch)",
                                     "step_three_launches": "kvq_quantize K, kvq_quantize V, kvq_decode_attn",
                                     "decode_only": "kvq_decode_attn"}},
        "decode": {"GBps": round(dec_gbps, 2), "frac_hbm_peak": round(dec_gbps / HBM_PEAK_GBPS, 4),
                   "frac_of_copy_bandwidth": round(dec_gbps / copy_gbps, 4),
                   "bytes_per_step": dec_bytes, "ms": round(res_dec["ms_mean"], 5),
                   "ms_median_p10_p90": [round(res_dec[k], 5) for k in ("ms_median", "ms_p10", "ms_p90")]},
        "decode_per_layer_launches": {
            "launches_per_step": L, "ms": round(res_dec_b["ms_median"], 5),
            "GBps": round(dec_bytes / (res_dec_b["ms_median"] * 1e-3) / 1e9, 2),
            "note": "mode B: one kvq_decode_attn per layer (batch B), all in one HIP graph"},
        "fp16_decode_per_layer_launches": {
            "launches_per_step": L, "ms": round(res_f16_b["ms_median"], 5),
            "GBps": round(f16_bytes / (res_f16_b["ms_median"] * 1e-3) / 1e9, 2),
            "speedup_quantized_vs_fp16_per_layer": round(res_f16_b["ms_median"] / res_dec_b["ms_median"], 3),
            "note": "mode B for the fp16 comparator: one kvq_decode_attn_fp16 per layer, one HIP graph"},
        "copy_1GiB": {"GBps": round(copy_gbps, 2), "frac_hbm_peak": round(copy_gbps / HBM_PEAK_GBPS, 4),
                      "ms": round(res_copy["ms_median"], 5)},
        "fp16_decode": {"GBps": round(f16_gbps, 2), "frac_hbm_peak": round(f16_gbps / HBM_PEAK_GBPS, 4),
                        "bytes_per_step": f16_bytes, "ms": round(res_f16["ms_mean"], 5),
                        "speedup_quantized_vs_fp16": round(res_f16["ms_mean"] / res_dec["ms_mean"], 3),
                        "fp16_equivalent_GBps_of_quantized": round(f16_bytes / (res_dec["ms_mean"] * 1e-3) / 1e9, 2)},
        "quantize_bulk": {"Mvectors_per_s": round(n_vec / (res_bq["ms_mean"] * 1e-3) / 1e6, 2),
                          "GBps_moved": round(bq_bytes / (res_bq["ms_mean"] * 1e-3) / 1e9, 2),
                          "frac_hbm_peak": round(bq_bytes / (res_bq["ms_mean"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                          "vectors": n_vec, "ms": round(res_bq["ms_mean"], 5),
                          "kernel": "quantize_mfma_kernel (rotation as a matrix product on MFMA)"},
        "quantize_bulk_fft": {"Mvectors_per_s": round(n_vec / (res_bqf["ms_mean"] * 1e-3) / 1e6, 2),
                              "GBps_moved": round(bq_bytes / (res_bqf["ms_mean"] * 1e-3) / 1e9, 2),
                              "frac_hbm_peak": round(bq_bytes / (res_bqf["ms_mean"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                              "ms": round(res_bqf["ms_mean"], 5),
                              "kernel": "quantize_fft_kernel (kvq_quantize_fft: in-register FFT, one lane per vector)"},
        "attn_speculative_4": {
            "GBps": round(q_bytes / (res_spec["ms_mean"] * 1e-3) / 1e9, 2), "ms": round(res_spec["ms_mean"], 5),
            "query_tokens": n_spec, "rows_per_work_group": pl_spec.head_tile * pl_spec.query_tile,
            "query_tiles": pl_spec.query_tiles,
            "note": "kvq_attn, 4 query tokens per sequence (the last 4 positions, causal), every layer; bytes = the "
                    "whole cache, read once per tile of query tokens"},
        "attn_window": {
            "GBps": round(win_bytes / (res_win["ms_mean"] * 1e-3) / 1e9, 2), "ms": round(res_win["ms_mean"], 5),
            "window": win, "bytes_per_step": win_bytes,
            "note": "kvq_attn, one query token, sliding window of the latest positions; bytes = the window's codes "
                    "and scales"},
        "decode_paged": {
            "GBps": round(dec_bytes / (res_pg["ms_mean"] * 1e-3) / 1e9, 2), "ms": round(res_pg["ms_mean"], 5),
            "page_tokens": page, "pages": LB * pps, "max_abs_diff_vs_contiguous": paged_diff,
            "note": "kvq_decode_attn_paged over the same cache cut into pages stored in a shuffled order"},
        "quantize_per_token_scale": {
            "Mvectors_per_s": round(n_vec / (res_pt["ms_mean"] * 1e-3) / 1e6, 2), "ms": round(res_pt["ms_mean"], 5),
            "k_relative_error": {k: round(v, 5) for k, v in round_trip.items()},
            "note": "group = head_dim (one fp16 scale per vector), K and V of all layers; the error is "
                    "||dequant(quant(K)) - K|| / ||K|| over layer 0's first tokens, both modes"},
        "roofline": {"bound": "hbm", "kernel": "decode_kernel (one launch per kvq_decode_attn call)",
                     "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4), "traffic": profiled_traffic(w.name),
                     "algorithmic_bytes_per_launch": dec_bytes, "decode_sources_sha": decode_sources_sha()},
    }
    if not args.no_cpu_baseline:
        log("timing the CPU oracle sample")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds, args.transform)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
