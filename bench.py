#!/usr/bin/env python3
"""Benchmark of libsage on one MI355X.

One step = the whole hot path over one batch of synthetic input already
resident in HBM: sage_quant_qkv (K smoothing + per-block INT8 Q/K and
per-channel FP8 V, the K and V statistics in one launch) and sage_attn_fwd
(fused INT8-QK / FP8-PV attention), enqueued on one stream.  Per-token Q
scales and Q smoothing go through sage_quant_qk(_ex/_smooth) + sage_quant_v.  The headline workload is the 720p clip
of a 14B video DiT: B=1, H=40, N=75600 (21 x 45 x 80 latent tokens), d=128.

--mx runs the microscaled path instead: sage_quant_qk_mx_fmt, sage_quant_v_mx_fmt
and sage_attn_fwd_mx_fmt (Q, K, P and V in MXFP6, or MXFP4 with --mx mxfp4),
priced against the dense FP6 = FP4 peak.
--bwd times the 8-bit backward (sage_attn_bwd) over the training forward's
outputs: 10 B H N^2 d ops per step (the five backward products), priced
against the blend of their peaks (four INT8/FP8 products, dP in FP16).

Prints ONE JSON line:
  value       = 4 B H N^2 d * steps / wall time of the timed steps (TOPS),
  roofline    = the attention kernel alone: algorithmic ops per launch (4 B H N^2 d)
                / its mean launch duration (HIP events around each launch on the
                stream it runs on), against the dense INT8 = FP8 MFMA peak,
  cpu_baseline= the CPU oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention TOPS (4·B·H·N²·d/s) & % MFMA peak at N=32760/75600, d=128"
PEAK_TOPS = {"fp8": 5000.0,                       # dense INT8 (QK) = dense FP8 (PV) = 5.0 POPS
             "fp16": 1.0 / (0.5 / 5000.0 + 0.5 / 2500.0),  # INT8 QK half + FP16 PV half
             "mxfp6": 10100.0,                    # dense FP6 (= FP4) MFMA, both products
             "mxfp4": 10100.0,
             # backward: 2d ops each for S, dV, dK, dQ at 5.0 POPS and dP at 2.5
             "bwd": 10.0 / (8.0 / 5000.0 + 2.0 / 2500.0)}
HBM_GBPS = 8000.0
FWD_TARGET_FRAC = 0.50  # the forward's throughput target (fraction of the dense MFMA peak)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
ATTN_SOURCES = [os.path.join(ROOT, "quantized_attention_video_02_amd", "csrc", f)
                for f in ("sage_attn.hip", "sage_common.h", "sage_device.h")]
BWD_SOURCES = [os.path.join(ROOT, "quantized_attention_video_02_amd", "csrc", f)
               for f in ("sage_bwd.hip", "sage_api.hip", "sage_common.h", "sage_device.h")]
QUANT_SOURCES = [os.path.join(ROOT, "quantized_attention_video_02_amd", "csrc", f)
                 for f in ("sage_quant.hip", "sage_api.hip", "sage_common.h")]
# the kernels of one quantization pass (sage_quant_qkv, or sage_quant_qk + sage_quant_v)
QUANT_KERNELS = ("kv_stats_kernel", "kv_combine_kernel", "k_stats_kernel", "k_mean_kernel",
                 "v_stats_kernel", "v_scale_kernel", "quant_qk_kernel", "quant_v_fp8_kernel",
                 "quant_v_fp16_kernel")


def attn_source_hash(bwd=False, quant=False):
    """sha256 of the measured kernels' sources (the attention kernel, the
    backward's kernels and the workspace carving, or the quantization pass):
    HBM byte counts measured on another version of the code are not reported."""
    from quantized_attention_video_02_amd import build as sage_build

    h = hashlib.sha256()
    for f in (QUANT_SOURCES if quant else BWD_SOURCES if bwd else ATTN_SOURCES):
        with open(f, "rb") as fh:
            h.update(fh.read())
        # a source compiled with extra flags is a different kernel
        extra = sage_build.SOURCE_FLAGS.get(os.path.basename(f))
        if extra:
            h.update(" ".join(extra).encode())
    return h.hexdigest()[:16]


def attn_ops(B, H, N, d):
    """Algorithmic work of one launch: 4 d ops per (query, key) pair, 2d INT8
    for Q K^T and 2d FP8 (FP16) for P V."""
    return 4.0 * B * H * N * N * d


def tile_mask_for(wl, keep, seed=11):
    """A seeded block-sparse tile mask (query block x key tile): each tile is
    kept with probability `keep`, plus a local band (|i - j| <= 1) and the
    first key tile, the shape of a sliding-window-plus-sink pattern."""
    import numpy as np

    nb = -(-wl.N // 128)
    rng = np.random.default_rng(seed)
    i, j = np.meshgrid(np.arange(nb), np.arange(nb), indexing="ij")
    m = rng.random((wl.B, wl.H, nb, nb)) < keep
    m |= ((np.abs(i - j) <= 1) | (j == 0))[None, None]
    if wl.causal:
        m &= (j <= i)[None, None]
    return m.astype(np.uint8)


def visited_ops(wl, mask):
    """Algorithmic work of a sparse launch: 4 d ops per visited (query, key)
    pair (causal: pairs with key <= query)."""
    import numpy as np

    nb = mask.shape[-1]
    sizes = np.minimum(128, wl.N - 128 * np.arange(nb)).astype(np.float64)
    pairs = sizes[:, None] * sizes[None, :]
    if wl.causal:  # diagonal tiles hold s (s + 1) / 2 causal pairs
        pairs[np.arange(nb), np.arange(nb)] = sizes * (sizes + 1) / 2
    return 4.0 * wl.d * float((mask.astype(np.float64) * pairs).sum())


def mx_format(mx):
    """The MX element format an `mx` argument names: False / None (the INT8
    path), True (MXFP6), or "mxfp6" / "mxfp4"."""
    return "mxfp6" if mx is True else (mx or None)


def time_gpu(sage, wl, pv, steps, warmup, q_gran="block", tile_mask=None, q_smooth=False,
             mx=False):
    import torch

    mx = mx_format(mx)
    q, k, v = wl.q, wl.k, wl.v
    stream = torch.cuda.current_stream()

    def step(evs=None):
        if evs:
            evs[0].record(stream)
        if mx:
            mz, v6 = sage.quant_qk_mx(q, k, fmt=mx), sage.quant_v_mx(v, fmt=mx)
        elif q_gran == "block" and not q_smooth:
            qz, vq, vs = sage.quant_qkv(q, k, v, pv)
        else:
            qz = sage.quant_qk(q, k, q_gran=q_gran, q_smooth=q_smooth, sm_scale=wl.sm_scale)
            vq, vs = sage.quant_v(v, pv)
        if evs:
            evs[1].record(stream)
        if mx:
            out = sage.attn_fwd_mx(mz, v6, causal=wl.causal, sm_scale=wl.sm_scale)
        else:
            out = sage.attn_fwd(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale, pv=pv,
                                tile_mask=tile_mask)
        if evs:
            evs[2].record(stream)
        return out

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    quant_ms = [e[0].elapsed_time(e[1]) for e in evs]
    attn_ms = [e[1].elapsed_time(e[2]) for e in evs]
    return wall, quant_ms, attn_ms


def time_bwd(sage, wl, steps, warmup):
    """The backward alone, inputs resident: the training forward runs once,
    then each step is one sage_attn_bwd call (events around each)."""
    import torch

    stream = torch.cuda.current_stream()
    do = si_grad(wl)
    qz = sage.quant_qk(wl.q, wl.k)
    vq, vs = sage.quant_v(wl.v, "fp8")
    out, lse = sage.attn_fwd_lse(qz, vq, vs, causal=wl.causal, sm_scale=wl.sm_scale)
    for _ in range(warmup):
        sage.attn_bwd(qz, wl.v, out, do, lse, causal=wl.causal, sm_scale=wl.sm_scale)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i][0].record(stream)
        sage.attn_bwd(qz, wl.v, out, do, lse, causal=wl.causal, sm_scale=wl.sm_scale)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, [e[0].elapsed_time(e[1]) for e in evs]


def si_grad(wl):
    import synthetic_inputs as si

    return si.output_grad(wl)


def cpu_baseline_bwd(wl, cores=None):
    """The oracle on head (0, 0): for a query block, its forward rows (output
    and log-sum-exp) and its dQ over all N keys; ops counted 10 d per pair
    (the forward rows' 4 d and the dQ sweep's 6 d: S, dP, dQ).  First block 0
    on one thread (`single_core_value`), then `cores` threads (default
    host_cores()) on blocks 0 .. cores - 1 at once, wall-clocked; the head's
    quantization is charged pro rata."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synthetic_inputs as si

    q, k, v = (si.bf16_codes(t[0:1, 0:1]) for t in (wl.q, wl.k, wl.v))
    dO = si.bf16_codes(si.output_grad(wl)[0:1, 0:1])
    t0 = time.perf_counter()
    oz = oracle.quant_qk(q, k)
    ovq, ovs = oracle.quant_v(v, "fp8")
    t_quant = time.perf_counter() - t0
    nblk = -(-wl.N // 128)

    def block(qb):
        rows = np.arange(128 * qb, min(wl.N, 128 * qb + 128), dtype=np.int32)
        o_rows, lse_rows = oracle.train_forward_head(oz, ovq, ovs, 0, 0, rows, wl.causal, wl.sm_scale)
        o = np.zeros((wl.N, wl.d), np.uint16)
        o[rows] = o_rows
        lse = np.zeros(wl.N, np.float32)
        lse[rows] = lse_rows
        oracle.bwd_head(oz, v[0, 0], o, dO[0, 0], lse, 0, 0, wl.causal, wl.sm_scale,
                        qblocks=[qb], kblocks=[])
        keys = (rows + 1).sum() if wl.causal else len(rows) * wl.N
        return 10.0 * float(keys) * wl.d, len(rows)

    t0 = time.perf_counter()
    ops, nrows = block(0)
    t1 = time.perf_counter() - t0 + t_quant * nrows / wl.N
    single = ops / t1 / 1e12
    P = min(host_cores() if cores is None else int(cores), nblk)
    sample = (f"head (b=0,h=0) of {wl.name}: for a block of 128 queries, the forward rows (output "
              f"and log-sum-exp) and their dQ over "
              f"{'their causal keys' if wl.causal else f'all {wl.N} keys'}; block 0 on one thread "
              f"({t1:.2f} s incl. the head's quantization pro rata)")
    if P <= 1:
        return {"value": single, "unit": "TOPS", "cores": 1, "kind": "oracle",
                "single_core_value": single, "sample": sample + "; C oracle"}
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=P) as ex:
        done = list(ex.map(block, range(P)))
    wall = time.perf_counter() - t0
    ops_all = sum(x[0] for x in done)
    rows_all = sum(x[1] for x in done)
    t_all = wall + t_quant * rows_all / wl.N / P
    return {"value": ops_all / t_all / 1e12, "unit": "TOPS", "cores": P, "kind": "oracle",
            "single_core_value": single,
            "sample": (f"{sample}; then {P} threads on blocks 0-{P - 1} at once ({wall:.2f} s "
                       f"wall), the quantization pro rata over the threads; C oracle")}


def host_cores():
    """Threads for the all-core oracle run: the CPUs this process may use,
    at most 16 (a one-GPU machine's share of its host)."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def cpu_baseline(wl, pv, target_s=12.0, q_gran="block", q_smooth=False, mx=False, cores=None,
                 all_core_s=None):
    """The oracle as it stands (single-threaded C) on one head of the workload:
    quantization of the whole head, then attention for R query rows against
    all N keys; the head's quantization time is charged pro rata (R / N).
    With Q smoothing the correction rows of the blocks the R rows use are
    computed too (charged to the quantization at the rate per block).  With
    mx ("mxfp6" or "mxfp4") the oracle's MX quantization and attention.

    Then the all-core run: `cores` threads (default host_cores()) each run the
    same single-threaded oracle on disjoint query rows of the head, wall-clocked
    (the C calls release the interpreter lock); the quantization is charged
    pro rata over the threads.  `value` is that run's rate, `cores` its thread
    count, `single_core_value` the one-thread rate."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np

    import oracle
    import synthetic_inputs as si

    mx = mx_format(mx)
    b, h = 0, 0
    q, k, v = (si.bf16_codes(t[b:b + 1, h:h + 1]) for t in (wl.q, wl.k, wl.v))
    t0 = time.perf_counter()
    if mx:
        mz = oracle.mx_quant_qk(q, k, mx)
        vc, ve = oracle.mx_quant_v(v, mx)
    else:
        oz = oracle.quant_qk(q, k, q_gran=q_gran, q_smooth=q_smooth)
        ovq, ovs = oracle.quant_v(v, pv)
    t_quant = time.perf_counter() - t0

    def attn_rows(rows, bias):
        if mx:
            return oracle.mx_attn_rows_head(mz, vc, ve, 0, 0, rows, wl.causal, wl.sm_scale)
        return oracle.attn_rows_head(oz, ovq, ovs, 0, 0, rows, wl.causal, wl.sm_scale, pv,
                                     bias=bias)

    nblk = -(-wl.N // 128)
    bias, t_bias = None, 0.0
    probe = np.arange(8, dtype=np.int32)
    if q_smooth:
        t0 = time.perf_counter()
        bias = oracle.smooth_bias(oz, k, wl.sm_scale, blocks=[0])
        t_bias = time.perf_counter() - t0                       # one block row
    t0 = time.perf_counter()
    attn_rows(probe, bias)
    per_row = (time.perf_counter() - t0) / len(probe)
    R = int(max(8, min(wl.N, target_s / max(per_row + t_bias / 128, 1e-9))))
    rows = np.arange(wl.N - R, wl.N, dtype=np.int32) if wl.causal else np.arange(R, dtype=np.int32)
    if q_smooth:
        used = sorted(set((rows // 128).tolist()))
        t0 = time.perf_counter()
        bias = oracle.smooth_bias(oz, k, wl.sm_scale, blocks=used)
        t_bias = time.perf_counter() - t0
    t0 = time.perf_counter()
    attn_rows(rows, bias)
    t_attn = time.perf_counter() - t0
    keys = (rows + 1).sum() if wl.causal else R * wl.N
    ops = 4.0 * float(keys) * wl.d
    # the whole head's quantization pro rata; the correction for the used
    # blocks, pro rata of their rows
    t_equiv = t_attn + t_quant * R / wl.N
    if q_smooth:
        t_equiv += t_bias * R / (len(used) * 128)
    single = ops / t_equiv / 1e12
    sample = (f"head (b=0,h=0) of {wl.name}: quantization of all {wl.N} tokens "
              f"({t_quant:.2f} s, charged pro rata) + attention for {R} queries x "
              f"{'their causal keys' if wl.causal else f'{wl.N} keys'} ({t_attn:.2f} s)"
              + (f"; Q-smoothing correction of their blocks ({t_bias:.2f} s, pro rata)"
                 if q_smooth else "") + (f"; {mx.upper()} path" if mx else "") + "; C oracle")
    P = host_cores() if cores is None else int(cores)
    if P <= 1:
        return {"value": single, "unit": "TOPS", "cores": 1, "kind": "oracle",
                "single_core_value": single, "sample": sample + ", one thread"}
    # all-core run: P threads, Rt rows each (disjoint; causal: the longest rows)
    per_row = t_attn / R
    budget = 0.6 * target_s if all_core_s is None else all_core_s
    Rt = int(max(1, min(wl.N // P, budget / max(per_row, 1e-9))))
    if wl.causal:
        slices = [np.arange(wl.N - (i + 1) * Rt, wl.N - i * Rt, dtype=np.int32) for i in range(P)]
    else:
        slices = [np.arange(i * Rt, (i + 1) * Rt, dtype=np.int32) for i in range(P)]
    t_bias_all = 0.0
    if q_smooth:
        used_all = sorted(set(np.concatenate(slices) // 128))
        t0 = time.perf_counter()
        bias = oracle.smooth_bias(oz, k, wl.sm_scale, blocks=used_all)
        t_bias_all = time.perf_counter() - t0
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=P) as ex:
        list(ex.map(lambda r: attn_rows(r, bias), slices))
    wall = time.perf_counter() - t0
    rows_all = P * Rt
    keys_all = sum(int((r + 1).sum()) for r in slices) if wl.causal else rows_all * wl.N
    t_all = wall + (t_quant * rows_all / wl.N + t_bias_all) / P
    return {"value": 4.0 * keys_all * wl.d / t_all / 1e12, "unit": "TOPS", "cores": P,
            "kind": "oracle", "single_core_value": single,
            "sample": (f"{sample}; then {P} threads, each the single-threaded oracle on "
                       f"{Rt} disjoint query rows of the same head ({wall:.2f} s wall), the "
                       f"quantization charged pro rata over the threads")}


def measured_mfma_tops():
    """This board's INT8 and FP8 MFMA rates (TOPS) from the register-only
    microbenchmarks (quantized_attention_video_02_amd/microbench), or None
    when that library is not built."""
    import ctypes as ct
    import statistics

    import torch

    from quantized_attention_video_02_amd.microbench import __main__ as mb

    if not os.path.exists(mb.LIB):
        return None
    L = ct.CDLL(mb.LIB)
    L.mb_run.argtypes = [ct.c_int, ct.c_int, ct.c_int, ct.c_void_p, ct.c_void_p]
    L.mb_ops.argtypes = [ct.c_int, ct.c_int, ct.c_int]
    L.mb_ops.restype = ct.c_double
    stream = torch.cuda.current_stream()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count * 12
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    rates = {}
    for kind, name in ((0, "int8"), (1, "fp8")):
        ts = []
        for rep in range(4):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            if L.mb_run(kind, blocks, 1000, ct.c_void_p(out.data_ptr()), ct.c_void_p(stream.cuda_stream)):
                return None
            e1.record(stream)
            torch.cuda.synchronize()
            if rep:
                ts.append(e0.elapsed_time(e1))
        rates[name] = L.mb_ops(kind, blocks, 1000) / (statistics.median(ts) * 1e-3) / 1e12
    return rates


def traffic_key(workload, pv, q_gran="block"):
    return f"{workload}/{pv}" + ("" if q_gran == "block" else f"/{q_gran}")


def attn_kernel_name(mx):
    return "attn_mx_kernel" if mx else "attn_fwd_kernel"


def record_traffic(workload, pv, fetch_dir, write_dir, q_gran="block", mx=False, bwd=False):
    """Write profiles/traffic.json from two rocprofv3 --pmc runs of
    `bench.py --steps 1 --warmup 0 --no-cpu-baseline --calibrate-copy` (one with
    FETCH_SIZE, one with WRITE_SIZE; KiB per dispatch; with --bwd for the
    backward).  Each counter is scaled so that the plain 1 GiB device copy in
    the same run reads (writes) 1 GiB.  The backward's entry is per call: the
    bytes of all its kernels (names with "bwd_") over the number of calls."""
    import csv
    import glob

    mx = mx_format(mx)

    def per_kernel(d, counter):
        rows = []
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                rows += [r for r in csv.DictReader(fh) if r["Counter_Name"] == counter]
        return rows

    res = {}
    kname = "bwd_" if bwd else attn_kernel_name(mx)
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        rows = per_kernel(d, counter)
        attn = [float(r["Counter_Value"]) * 1024 for r in rows if kname in r["Kernel_Name"]]
        # --calibrate-copy's device-to-device copy runs as the HIP runtime's blit kernel
        copy = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]]
        if not attn or not copy:
            raise SystemExit(f"no {kname} or copy dispatch with {counter} under {d}")
        scale = float(1 << 30) / max(copy)
        # one launch of the attention kernel, or one backward call (one dQ sweep each)
        n = sum(1 for r in rows if "bwd_dq_kernel" in r["Kernel_Name"]) if bwd else len(attn)
        if n == 0:
            raise SystemExit(f"no bwd_dq_kernel dispatch with {counter} under {d}")
        res[counter] = (sum(attn) / n * scale, scale)
    entry = {"kernel": "sage_attn_bwd (all its kernels)" if bwd else kname,
             "source_hash": attn_source_hash(bwd),
             "fetch_bytes": res["FETCH_SIZE"][0], "write_bytes": res["WRITE_SIZE"][0],
             "bytes_per_launch": res["FETCH_SIZE"][0] + res["WRITE_SIZE"][0],
             "fetch_scale": res["FETCH_SIZE"][1], "write_scale": res["WRITE_SIZE"][1],
             "note": "rocprofv3 FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by a plain "
                     "1 GiB device copy measured in the same runs"}
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
    data[traffic_key(workload, "bwd" if bwd else (mx if mx else pv), q_gran)] = entry
    if not bwd and not mx:
        # the quantization pass of the same runs: all its kernels, per step
        # (a step launches the quantization kernels once: one quant_qk_kernel)
        qres = {}
        for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
            rows = per_kernel(d, counter)
            copy = [float(r["Counter_Value"]) * 1024 for r in rows if "copyBuffer" in r["Kernel_Name"]]
            scale = float(1 << 30) / max(copy)
            qk = [float(r["Counter_Value"]) * 1024 for r in rows
                  if any(k in r["Kernel_Name"] for k in QUANT_KERNELS)]
            steps = sum(1 for r in rows if "quant_qk_kernel" in r["Kernel_Name"])
            if qk and steps:
                qres[counter] = (sum(qk) / steps * scale, scale)
    if not bwd and not mx and len(qres) == 2:
        qentry = {"kernel": "quantization pass (sage_quant_qkv: all its kernels)",
                  "source_hash": attn_source_hash(quant=True),
                  "fetch_bytes": qres["FETCH_SIZE"][0], "write_bytes": qres["WRITE_SIZE"][0],
                  "bytes_per_step": qres["FETCH_SIZE"][0] + qres["WRITE_SIZE"][0],
                  "note": entry["note"]}
        data[traffic_key(workload, pv, q_gran) + "/quant"] = qentry
        print(json.dumps(qentry))
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(data, f, indent=1)
    print(json.dumps(entry))


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="video_14b_720p")
    ap.add_argument("--pv", default="fp8", choices=["fp8", "fp16"])
    ap.add_argument("--q-gran", default="block", choices=["block", "token"],
                    help="Q scale granularity: per block of 128 queries, or per query row")
    ap.add_argument("--tile-keep", type=float, default=None,
                    help="block-sparse run: keep each (query block, key tile) with this "
                         "probability, plus a local band and the first tile")
    ap.add_argument("--q-smooth", action="store_true",
                    help="Q smoothing: per-block Q means, the FP32 score correction, and the "
                         "attention variant that adds it (all inside the timed step)")
    ap.add_argument("--q-sigma", type=float, default=None,
                    help="give the workload's queries a per-channel offset of this sigma "
                         "(the inputs Q smoothing is for)")
    ap.add_argument("--mx", nargs="?", const="mxfp6", default=None, choices=["mxfp6", "mxfp4"],
                    help="the microscaled path: Q, K, P and V in MXFP6 (the default) or MXFP4 "
                         "(sage_quant_qk_mx_fmt, sage_quant_v_mx_fmt, sage_attn_fwd_mx_fmt)")
    ap.add_argument("--bwd", action="store_true",
                    help="the 8-bit backward (sage_attn_bwd) over the training forward's outputs")
    ap.add_argument("--shape", default=None, metavar="B,H,N",
                    help="override the workload's batch, heads and sequence length (its value "
                         "recipe and head dim stay); the line then carries no traffic figure")
    ap.add_argument("--no-causal", action="store_true",
                    help="run a causal workload without the causal mask")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device-to-device copy (the known-size "
                         "reference for HBM byte counters)")
    ap.add_argument("--record-traffic", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="write profiles/traffic.json for --workload/--pv from two rocprofv3 "
                         "--pmc output folders (FETCH_SIZE, WRITE_SIZE) and exit")
    args = ap.parse_args()
    if args.record_traffic:
        record_traffic(args.workload, args.pv, *args.record_traffic, q_gran=args.q_gran, mx=args.mx,
                       bwd=args.bwd)
        return
    if args.bwd and (args.mx or args.q_smooth or args.tile_keep is not None or
                     args.q_gran != "block" or args.pv != "fp8"):
        print("bench.py: --bwd runs the 8-bit backward alone (no --mx, --q-smooth, "
              "--tile-keep, --q-gran token or --pv fp16)", file=sys.stderr)
        sys.exit(2)
    if args.mx and (args.q_smooth or args.tile_keep is not None or args.q_gran != "block"
                    or args.pv != "fp8"):
        print("bench.py: --mx runs the MX path alone (no --q-smooth, --tile-keep, "
              "--q-gran token or --pv fp16)", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: this build runs on one GPU only (there is no multi-GPU path; "
              "DESIGN.md describes how the work would shard). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import quantized_attention_video_02_amd as sage
    import synthetic_inputs as si

    sage.lib()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dims = {}
    if args.shape:
        dims = dict(zip(("B", "H", "N"), (int(x) for x in args.shape.split(","))))
    wl = si.make(args.workload, device="cuda", q_sigma=args.q_sigma, **dims)
    if args.no_causal:
        wl = dataclasses.replace(wl, causal=False)
    # traffic.json holds counter runs of the named workloads as they are defined
    stock = not dims and not args.no_causal
    torch.cuda.synchronize()
    fmt = args.mx if args.mx else args.pv
    print(f"[bench] {wl.name}: B={wl.B} H={wl.H} N={wl.N} d={wl.d} causal={wl.causal} path={fmt}",
          file=sys.stderr, flush=True)
    if args.calibrate_copy:
        src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.bwd:
        wall, bwd_ms = time_bwd(sage, wl, args.steps, args.warmup)
        ops = 10.0 * wl.B * wl.H * wl.N * wl.N * wl.d
        mean = sum(bwd_ms) / len(bwd_ms)
        srt = sorted(bwd_ms)
        achieved = ops / (mean * 1e-3) / 1e12
        traffic = None
        if stock and os.path.exists(TRAFFIC_FILE):
            with open(TRAFFIC_FILE) as f:
                t = json.load(f).get(traffic_key(wl.name, "bwd"))
            if t and t.get("source_hash") == attn_source_hash(bwd=True):
                traffic = t.get("bytes_per_launch")
        res = {
            "metric": "attention backward TOPS (10·B·H·N²·d/s, the five backward products)",
            "value": ops * args.steps / wall / 1e12, "unit": "TOPS", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall * 1e3 / args.steps,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "int8+fp8+fp16", "data": "synthetic",
            "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                       "causal": wl.causal, "pass": "backward", "seed": wl.seed,
                       "parallelism": "none"},
            "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TOPS["bwd"],
                         "unit": "TFLOP/s", "frac": achieved / PEAK_TOPS["bwd"], "traffic": traffic,
                         "kernel": "sage_attn_bwd (preparation + dQ, dV and dK sweeps)",
                         "ops_per_launch": ops, "mean_launch_ms": mean,
                         "median_launch_ms": srt[len(srt) // 2]},
        }
        if wl.causal:
            # `value` keeps the metric's formula over every (query, key) pair;
            # the kernels compute the N(N+1)/2 pairs the causal mask keeps, so
            # the roofline counts those (as the forward's does)
            useful = 10.0 * wl.B * wl.H * wl.d * wl.N * (wl.N + 1) / 2
            res["roofline"]["all_pairs_tops"] = achieved
            achieved = useful / (mean * 1e-3) / 1e12
            res["roofline"].update({"achieved": achieved, "frac": achieved / PEAK_TOPS["bwd"],
                                    "ops_per_launch": useful,
                                    "ops_counted": "causal pairs (key <= query)"})
        if not args.no_cpu_baseline:
            print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
            res["cpu_baseline"] = cpu_baseline_bwd(wl)
        print(json.dumps(res), flush=True)
        return
    tmask = None
    if args.tile_keep is not None:
        mask_np = tile_mask_for(wl, args.tile_keep)
        tmask = torch.from_numpy(mask_np).cuda()
    wall, quant_ms, attn_ms = time_gpu(sage, wl, args.pv, args.steps, args.warmup, args.q_gran,
                                       tmask, args.q_smooth, args.mx)
    ops = attn_ops(wl.B, wl.H, wl.N, wl.d)
    # roofline work: all pairs when dense; the visited pairs of a sparse run
    work = ops if tmask is None else visited_ops(wl, mask_np)
    ms_per_step = wall * 1e3 / args.steps
    attn_mean = sum(attn_ms) / len(attn_ms)
    srt = sorted(attn_ms)
    attn_med = srt[len(srt) // 2]
    attn_iqr = srt[(3 * len(srt)) // 4] - srt[len(srt) // 4]
    quant_mean = sum(quant_ms) / len(quant_ms)
    achieved = work / (attn_mean * 1e-3) / 1e12
    peak = PEAK_TOPS[fmt]
    bhnd = wl.B * wl.H * wl.N * wl.d
    # quantization bytes, two-pass count: K read twice (statistics, then
    # codes), Q and V once as bf16, the codes written once; the INT8/FP8 path
    # also reads V twice (per-channel scale first): 13 BHNd, MX: 11 BHNd
    qbytes = (11 if args.mx else 13) * bhnd
    traffic, qtraffic = None, None
    if stock and os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tdata = json.load(f)
        t = tdata.get(traffic_key(wl.name, fmt, args.q_gran))
        if t and t.get("source_hash") == attn_source_hash() and not args.q_smooth:
            traffic = t.get("bytes_per_launch")
        t = tdata.get(traffic_key(wl.name, fmt, args.q_gran) + "/quant")
        if t and t.get("source_hash") == attn_source_hash(quant=True) and not args.q_smooth:
            qtraffic = t.get("bytes_per_step")
    res = {
        "metric": METRIC,
        "value": ops * args.steps / wall / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"fp8": "int8+fp8", "fp16": "int8+fp16", "mxfp6": "mxfp6", "mxfp4": "mxfp4"}[fmt],
        "data": "synthetic",
        "config": {"workload": wl.name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d,
                   "causal": wl.causal, "pv": fmt, "q_gran": "mx32" if args.mx else args.q_gran,
                   "seed": wl.seed,
                   "parallelism": "none"},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
                     "frac": achieved / peak, "traffic": traffic,
                     "kernel": attn_kernel_name(args.mx), "ops_per_launch": work,
                     "mean_launch_ms": attn_mean, "median_launch_ms": attn_med,
                     "iqr_launch_ms": attn_iqr,
                     "median_tops": work / (attn_med * 1e-3) / 1e12},
        "quant": {"ms": quant_mean, "bytes_two_pass": qbytes,
                  "gbps_two_pass": qbytes / (quant_mean * 1e-3) / 1e9,
                  "frac_hbm": qbytes / (quant_mean * 1e-3) / 1e9 / HBM_GBPS,
                  "bytes_measured": qtraffic,
                  "gbps_measured": (qtraffic / (quant_mean * 1e-3) / 1e9) if qtraffic else None},
    }
    if args.q_smooth or args.q_sigma is not None:
        res["config"]["q_smooth"] = bool(args.q_smooth)
        res["config"]["q_sigma"] = args.q_sigma
    if args.q_smooth:
        # the quantization phase now includes the correction kernel: its
        # bytes are not the two-pass count above
        res["quant"]["note"] = "includes the Q-smoothing correction kernel (VALU-bound)"
        res["quant"].pop("gbps_two_pass")
        res["quant"].pop("frac_hbm")
    if tmask is not None:
        # value stays the metric's formula over all N^2 pairs (dense-equivalent);
        # the roofline counts the visited pairs only
        res["config"]["tile_keep"] = float(mask_np.mean())
        res["config"]["value_is"] = "dense-equivalent (4 B H N^2 d / s) of a block-sparse run"
        res["roofline"]["traffic"] = None
    if wl.causal and tmask is None:
        # `value` keeps the metric's formula over every (query, key) pair; the
        # kernel computes only the N(N+1)/2 pairs the causal mask keeps (and
        # skips the tiles above the diagonal), so the roofline counts those
        useful = 4.0 * wl.B * wl.H * wl.d * wl.N * (wl.N + 1) / 2
        res["roofline"]["all_pairs_tops"] = achieved
        achieved = useful / (attn_mean * 1e-3) / 1e12
        res["roofline"].update({"achieved": achieved, "frac": achieved / peak,
                                "ops_per_launch": useful,
                                "median_tops": useful / (attn_med * 1e-3) / 1e12,
                                "ops_counted": "causal pairs (key <= query)"})
    if not args.mx and args.pv == "fp8":
        # this board's own matrix-core rates, measured after the timed steps:
        # the kernel does half its work on each, so the blend is its peak here
        m = measured_mfma_tops()
        if m:
            blend = 1.0 / (0.5 / m["int8"] + 0.5 / m["fp8"])
            res["roofline"]["measured_peak"] = {"int8": m["int8"], "fp8": m["fp8"], "blend": blend,
                                                "frac": achieved / blend}
    if not args.mx:
        # the forward's throughput target: half of the dense INT8/FP8 peak
        res["roofline"]["target_frac"] = FWD_TARGET_FRAC
        res["roofline"]["target_met"] = bool(res["roofline"]["frac"] >= FWD_TARGET_FRAC)
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle on a bounded sample", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(wl, args.pv, args.cpu_seconds, args.q_gran,
                                           args.q_smooth, args.mx)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
