#!/usr/bin/env python3
"""Benchmark of the QoQ W4A8 GEMM path on one MI355X.

A step is one pass of the online hot path over one batch of synthetic input
already resident in HBM: per-token INT8 activation quantization followed by the
W4A8 GEMM with its fused FP16 epilogue.  The offline weight encode/pack is not
part of a step (it runs once per weight, on the host).

Default workload: the largest single-GPU configuration, the Qwen1.5-72B-like
FFN at large batch (M=4096 tokens, K=8192, N=24576, g128), compute-bound on the
INT8 matrix cores.  Prints ONE JSON line with the headline numbers, the
roofline of the GEMM kernel, the CPU oracle baseline (all host cores, plus
one-thread legs on the smaller workloads and the oracle's weight encode beside
the library's packer) and a sweep over the other workload shapes
(kernel-level TOPS / GB/s / roofline fraction; the decode shapes against the
HBM roofline).

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-sweep]
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
sys.path.insert(0, ROOT)

METRIC = "W4A8 GEMM TOPS and HBM GB/s on 1 MI355X; % of INT8-MFMA / HBM roofline"
PEAK_INT8_TOPS = 5000.0   # MI355X dense INT8 MFMA peak, 5.0 POP/s
PEAK_HBM_GBS = 8000.0     # MI355X HBM3E, 8 TB/s
MALL_BYTES = 256 * 2 ** 20
SWEEP = ["tiny", "attn_proj", "attn_qkv", "ffn_gateup_prefill", "ffn_down_prefill", "decode_m1", "decode_m16",
         "decode_m64", "ffn_large_g128", "ffn_large_perchannel"]


def algo_bytes(w) -> int:
    """Bytes the method must move per GEMM: W4 codes, group metadata (8-bit
    scale + 4-bit zero per group of 128) or per-channel zero (4 bits), FP16
    channel scale, INT8 activations, FP16 token scales, FP16 output."""
    wq = w.N * w.K // 2
    meta = (w.N * (w.K // 128) * 3) // 2 if w.group_size else w.N // 2
    return wq + meta + 2 * w.N + w.M * w.K + 2 * w.M + 2 * w.M * w.N


def algo_bytes_w8(w) -> int:
    """The same for the W8A8 comparator: INT8 weights and their FP16 scale."""
    return w.N * w.K + 2 * w.N + w.M * w.K + 2 * w.M + 2 * w.M * w.N


def act_bytes(w) -> int:
    return 2 * w.M * w.K + w.M * w.K + 2 * w.M


def producer_bytes(w) -> int:
    """Fused RMS normalization + quantization: FP16 rows and gamma in, INT8
    rows and FP16 scales out (an unfused norm would add 4 bytes per element:
    its FP16 output written and read back)."""
    return 2 * w.M * w.K + 2 * w.K + w.M * w.K + 2 * w.M


def swiglu_bytes(w) -> int:
    """Fused SiLU(gate) * up + quantization: two FP16 [M, K] inputs in, INT8
    rows and FP16 scales out."""
    return 4 * w.M * w.K + w.M * w.K + 2 * w.M


def bound_of(w) -> str:
    t_hbm = algo_bytes(w) / (PEAK_HBM_GBS * 1e9)
    t_mfma = w.ops / (PEAK_INT8_TOPS * 1e12)
    return "mfma" if t_mfma >= t_hbm else "hbm"


def src_hash() -> str:
    """Hash of the kernel sources' code (line comments and blank lines dropped),
    so that a stored traffic measurement goes stale only when code changes."""
    h = hashlib.sha256()
    for f in ("gemm_kernels.h", "gemm_w4.hip", "act_quant.hip"):
        with open(os.path.join(ROOT, "w4a8_quantized_gemm_qoq_amd", "csrc", f), encoding="utf-8") as fh:
            for line in fh:
                code = line.split("//", 1)[0].rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()[:16]


def stored_traffic(name: str):
    """HBM bytes per GEMM launch from the counter profile of this workload
    (profiles/traffic_<name>.json), or None when there is none or the kernel
    code has changed since it was taken."""
    tf = os.path.join(ROOT, "profiles", f"traffic_{name}.json")
    try:
        with open(tf) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    return rec.get("hbm_bytes_per_launch") if rec.get("src_hash") == src_hash() else None


def busy(torch, ms: float):
    """Keep the stream busy so launches queued behind it run back to back."""
    try:
        torch.cuda._sleep(int(ms * 1e-3 * 2.4e9))
    except Exception:
        pass


def time_kernel(torch, launch, reps: int, sleep_ms: float = 20.0) -> float:
    """Average duration (us) of one launch: HIP events recorded on the launch
    stream before and after `reps` back-to-back launches, all queued behind a
    busy kernel so that host submission gaps do not count; divided by reps.
    (Events around every single launch add about 2 us each on this stack.)"""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    busy(torch, sleep_ms)
    e0.record()
    for i in range(reps):
        launch(i)
    e1.record()
    torch.cuda.synchronize()
    return 1e3 * e0.elapsed_time(e1) / reps


def blas_threads() -> int:
    """Threads of the BLAS pool the oracle's matrix product runs on."""
    try:
        from threadpoolctl import threadpool_info
        n = [i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def _time_oracle(O, X, enc, seconds: float):
    """Repeat the oracle's online part (per-token quantization, exact GEMM,
    FP64 epilogue) for about `seconds`; returns (seconds per repetition, reps)."""
    reps = 0
    t0 = time.perf_counter()
    while True:
        O.w4a8_forward(X, enc)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return el / reps, reps


def _column_sample(w, W, max_cols: int):
    """The first `max_cols` output channels of a workload's weight (all tokens,
    all of K): a bounded sample of the same GEMM for the CPU oracle."""
    n = min(w.N, max_cols)
    return W[:n], n


def cpu_baseline(w, X, W, seconds: float, max_cols: int = 2048):
    """The CPU oracle's online part on a bounded sample of the workload (every
    token row and all of K, the first `max_cols` output channels), repeated for
    about `seconds` on all of the host's BLAS threads, in TOPS of that sample."""
    import oracle as O
    Ws, n = _column_sample(w, W, max_cols)
    enc = O.encode_weight_g128(Ws) if w.group_size else O.encode_weight_per_channel(Ws)
    per, reps = _time_oracle(O, X, enc, seconds)
    ops = 2 * w.M * n * w.K
    return {"value": round(ops / per / 1e12, 4), "unit": "TOPS", "cores": blas_threads(), "kind": "oracle",
            "sample": (f"{w.name}: all {w.M} tokens x K={w.K} x the first {n} of {w.N} output channels "
                       f"({ops / 1e9:.0f} G int ops), {reps} repetitions in {per * reps:.1f} s"),
            "seconds_per_repetition": round(per, 4)}


# One-thread and all-thread legs of the oracle on the smaller workloads (the
# tiny GEMM, the attention projections, the prefill FFN and the decode
# shapes), each on at most 1024 output channels.
CPU_LEG_WORKLOADS = ["tiny", "attn_proj", "attn_qkv", "ffn_gateup_prefill", "ffn_down_prefill", "decode_m1",
                     "decode_m16", "decode_m64"]


def cpu_legs(seconds_per_leg: float, max_cols: int = 1024):
    import oracle as O
    import synthetic
    from threadpoolctl import threadpool_limits
    out = []
    for name in CPU_LEG_WORKLOADS:
        w = synthetic.get_workload(name)
        n = min(w.N, max_cols)
        # the first n rows of a workload's weight draw are a draw of n rows
        X, Ws = synthetic.make_x(w.M, w.K, w.outliers), synthetic.make_w(n, w.K)
        enc = O.encode_weight_g128(Ws) if w.group_size else O.encode_weight_per_channel(Ws)
        ops = 2 * w.M * n * w.K
        rec = {"workload": name, "sample": f"all {w.M} tokens x K={w.K} x the first {n} of {w.N} output channels"}
        with threadpool_limits(limits=1, user_api="blas"):
            per1, _ = _time_oracle(O, X, enc, seconds_per_leg)
        perN, _ = _time_oracle(O, X, enc, seconds_per_leg)
        rec.update({"tops_1_thread": round(ops / per1 / 1e12, 5), "tops_all_threads": round(ops / perN / 1e12, 5),
                    "threads": blas_threads(), "ms_1_thread": round(1e3 * per1, 3),
                    "ms_all_threads": round(1e3 * perN, 3)})
        out.append(rec)
    return out


def encode_vs_pack(w, W, q, max_cols: int = 2048):
    """The offline weight encode on the host: the oracle's progressive
    quantization (levels 0 and 1, NumPy) against the library's packer
    (quantization + packing, threaded C++), on the same sample of the
    weight; and the packer on the whole weight."""
    import oracle as O
    Ws, n = _column_sample(w, W, max_cols)
    q.qoq_pack_weights(Ws[:16], w.group_size)  # first call: library load, thread start-up
    t0 = time.perf_counter()
    O.encode_weight_g128(Ws) if w.group_size else O.encode_weight_per_channel(Ws)
    t_o = time.perf_counter() - t0
    t0 = time.perf_counter()
    q.qoq_pack_weights(Ws, w.group_size)
    t_l = time.perf_counter() - t0
    t0 = time.perf_counter()
    q.qoq_pack_weights(W, w.group_size)
    t_full = time.perf_counter() - t0
    return {"sample": f"{w.name} weight, the first {n} of {w.N} output channels x K={w.K}",
            "oracle_encode_s": round(t_o, 4), "library_pack_s": round(t_l, 4),
            "library_pack_full_weight_s": round(t_full, 4), "host_cores": len(os.sched_getaffinity(0))}


def _copies(w, wbytes):
    """Weight copies cycled from launch to launch so that the weights come
    from HBM (one copy of a decode-size weight would stay in the 256 MB
    last-level cache); one copy for the compute-bound prefill shapes."""
    c = 1 if bound_of(w) == "mfma" and w.M >= 1024 else max(1, math.ceil(3 * MALL_BYTES / max(wbytes, 1)))
    return min(c, 64)


def measure_comparators(torch, q, w, W, x8, sx, y, ws, t_g, reps: int, p_host=None):
    """The two comparators on the same inputs and launch plans: the W8A8
    GEMM (INT8 weights, no dequantization) and the saturating-dequantization
    ablation of the g128 GEMM."""
    p8h = q.qoq_pack_weights_w8(W)
    c8 = _copies(w, p8h.qweight.nbytes)
    w8s = [p8h.to(x8.device) for _ in range(c8)]
    for p8 in w8s:
        q.qoq_w8a8_gemm(x8, sx, p8, y=y)
    t8 = time_kernel(torch, lambda i: q.qoq_w8a8_gemm(x8, sx, w8s[i % c8], y=y), reps)
    del w8s
    r = {"w8a8_us": round(t8, 3), "w8a8_tops": round(w.ops / t8 / 1e6, 2),
         "w8a8_gbs": round(algo_bytes_w8(w) / t8 / 1e3, 1), "w8a8_weight_copies": c8,
         "w4a8_over_w8a8": round(t8 / t_g, 3)}
    if w.group_size:
        t_sat = time_kernel(torch, lambda i: q.qoq_w4a8_gemm_saturating(x8, sx, ws[i % len(ws)], y=y), reps)
        r.update({"saturating_us": round(t_sat, 3), "saturating_slowdown": round(t_sat / t_g, 3)})
    if p_host is not None:
        r.update(measure_library_w8a8(torch, q, w, p_host, x8, t_g, reps))
    return r


def plain_w8(q, p_host):
    """The INT8 weights [N, K] that packed W4 weights dequantize to."""
    import numpy as np
    q4, s1, z, _ = q.qoq_unpack_weights(p_host)
    G = q4.shape[1] // 128
    if s1 is None:
        return (q4.astype(np.int16) - z.astype(np.int16)[:, None]).astype(np.int8)
    w = (q4.reshape(q4.shape[0], G, 128).astype(np.int16) - z.astype(np.int16)[:, :, None]) * s1.astype(np.int16)[:, :, None]
    return w.reshape(q4.shape).astype(np.int8)


def measure_library_w8a8(torch, q, w, p_host, x8, t_g, reps: int):
    """The vendor library's INT8 GEMM on the same shape: hipBLASLt through
    torch._int_mm (INT32 output, no scale epilogue: less work than the fused
    FP16 epilogue here), on the INT8 weights the W4 codes dequantize to.  The
    pages set their W4A8 GEMM against the vendor W8A8 GEMM; this is that
    comparison on MI355X.  (The library refuses 16 rows or fewer.)"""
    if w.M <= 16:
        return {"hipblaslt_w8a8_us": None, "hipblaslt_note": "torch._int_mm needs more than 16 rows"}
    w8 = torch.from_numpy(plain_w8(q, p_host)).to(x8.device)
    c = _copies(w, w8.numel())
    w8s = [w8] + [w8.clone() for _ in range(c - 1)]
    try:
        for b in w8s:
            torch._int_mm(x8, b.t())
    except RuntimeError as e:
        return {"hipblaslt_w8a8_us": None, "hipblaslt_note": str(e).splitlines()[0][:120]}
    t = time_kernel(torch, lambda i: torch._int_mm(x8, w8s[i % c].t()), reps)
    del w8s, w8
    return {"hipblaslt_w8a8_us": round(t, 3), "hipblaslt_w8a8_tops": round(w.ops / t / 1e6, 2),
            "hipblaslt_weight_copies": c, "w4a8_over_hipblaslt_w8a8": round(t / t_g, 3)}


KV4_SHAPES = [("llama2_7b_mha", 64, 32, 32, 1024), ("llama3_8b_gqa", 64, 32, 8, 1024),
              ("llama2_7b_mha_b4_t8k", 4, 32, 32, 8192), ("llama3_8b_gqa_b1_t32k", 1, 32, 8, 32768)]


def kv4_bytes(B, H, Hkv, T) -> int:
    """Decode attention over a KV4 cache: K and V codes (64 B per token and
    head), their FP16 scales and byte zeros, the FP16 queries and outputs."""
    return 2 * B * Hkv * T * (64 + 2 + 1) + 2 * 2 * B * H * 128 + 4 * B


def measure_kv4(torch, q, reps: int):
    """KV4 decode attention and KV quantization at 64 sequences x 1024 cached
    tokens (the pages' 64 x 1024 attention input), head_dim 128; and at two
    small-batch long-cache shapes, where the token-split entry is timed too."""
    import numpy as np
    dev = torch.device("cuda")
    out = []
    for name, B, H, Hkv, T in KV4_SHAPES:
        rng = np.random.default_rng(0)
        kv = torch.from_numpy(rng.standard_normal((2, B, Hkv, T, 128)).astype(np.float16)).to(dev)
        t_quant = time_kernel(torch, lambda i: q.qoq_kv4_quant(kv), max(3, reps // 4))
        cache_bytes = 2 * B * Hkv * T * 67
        copies = max(1, min(16, math.ceil(3 * MALL_BYTES / cache_bytes)))
        caches = []
        for _ in range(copies):
            kc, ks, kz = q.qoq_kv4_quant(kv[0])
            vc, vs, vz = q.qoq_kv4_quant(kv[1])
            caches.append(((kc, ks, kz), (vc, vs, vz)))
        del kv
        qq = torch.from_numpy(rng.standard_normal((B, H, 128)).astype(np.float16)).to(dev)
        lengths = torch.full((B,), T, dtype=torch.int32, device=dev)
        o = torch.empty((B, H, 128), dtype=torch.float16, device=dev)
        scale = float(np.float32(1.0 / np.sqrt(128.0)))
        for c in caches:
            q.qoq_kv4_decode_attention(qq, c[0], c[1], lengths, scale, o=o)
        t_attn = time_kernel(torch, lambda i: q.qoq_kv4_decode_attention(qq, caches[i % copies][0],
                                                                         caches[i % copies][1], lengths, scale, o=o),
                             reps)
        nb = kv4_bytes(B, H, Hkv, T)
        rec = {"shape": name, "B": B, "H": H, "Hkv": Hkv, "T": T, "attention_us": round(t_attn, 3),
               "attention_gbs": round(nb / t_attn / 1e3, 1),
               "attention_frac_hbm": round(nb / t_attn / 1e3 / PEAK_HBM_GBS, 4),
               "cache_copies": copies, "kv_quant_us": round(t_quant, 3),
               "kv_quant_gbs": round((2 * B * Hkv * T * (256 + 67)) / t_quant / 1e3, 1)}
        need = q.qoq_kv4_decode_attention_workspace_size(B, H, Hkv, T)
        if need:
            ws = torch.empty(need, dtype=torch.uint8, device=dev)

            def split(i):
                c = caches[i % copies]
                q.qoq_kv4_decode_attention(qq, c[0], c[1], lengths, scale, o=o, split=True, workspace=ws)
            for i in range(copies):
                split(i)
            t_split = time_kernel(torch, split, reps)
            rec.update({"split_attention_us": round(t_split, 3), "split_attention_gbs": round(nb / t_split / 1e3, 1),
                        "split_attention_frac_hbm": round(nb / t_split / 1e3 / PEAK_HBM_GBS, 4)})
        out.append(rec)
        del caches
        torch.cuda.empty_cache()
    return out


def synthetic_gamma(K: int):
    import synthetic
    return synthetic.make_gamma(K)


def measure_gemm(torch, q, w, X, W, reps: int, comparators: bool = False):
    """Kernel-level timing of the act quantizer and the GEMM for one workload
    (and, if asked, of the two comparators on the same inputs)."""
    import numpy as np
    dev = torch.device("cuda")
    packed_host = q.qoq_pack_weights(W, w.group_size)
    wbytes = packed_host.qweight.nbytes + packed_host.meta.nbytes
    copies = _copies(w, wbytes)
    ws = [packed_host.to(dev) for _ in range(copies)]
    x = torch.from_numpy(np.ascontiguousarray(X)).to(dev)
    x8 = torch.empty((w.M, w.K), dtype=torch.int8, device=dev)
    sx = torch.empty((w.M,), dtype=torch.float16, device=dev)
    y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)
    q.qoq_quant_act_per_token(x, x8, sx)
    for p in ws:
        q.qoq_w4a8_gemm(x8, sx, p, y=y)
    torch.cuda.synchronize()
    t_q = time_kernel(torch, lambda i: q.qoq_quant_act_per_token(x, x8, sx), reps)
    gamma = torch.from_numpy(synthetic_gamma(w.K)).to(dev)
    t_n = time_kernel(torch, lambda i: q.qoq_rmsnorm_quant_per_token(x, gamma, 1e-5, x8, sx), reps)
    up = torch.flip(x, dims=(1,)).contiguous()   # a second FP16 operand of the same shape
    t_s = time_kernel(torch, lambda i: q.qoq_swiglu_quant_per_token(x, up, x8, sx), reps)
    del up
    t_g = time_kernel(torch, lambda i: q.qoq_w4a8_gemm(x8, sx, ws[i % copies], y=y), reps)
    b = algo_bytes(w)
    bnd = bound_of(w)
    tops = w.ops / t_g / 1e6
    gbs = b / t_g / 1e3
    frac = tops / PEAK_INT8_TOPS if bnd == "mfma" else gbs / PEAK_HBM_GBS
    r = {"workload": w.name, "M": w.M, "K": w.K, "N": w.N, "group_size": w.group_size,
         "gemm_us": round(t_g, 3), "tops": round(tops, 2), "gbs": round(gbs, 1), "bound": bnd,
         "frac": round(frac, 4), "traffic": stored_traffic(w.name), "weight_copies": copies,
         "act_quant_us": round(t_q, 3),
         "act_quant_gbs": round(act_bytes(w) / t_q / 1e3, 1),
         "rmsnorm_quant_us": round(t_n, 3), "rmsnorm_quant_gbs": round(producer_bytes(w) / t_n / 1e3, 1),
         "swiglu_quant_us": round(t_s, 3), "swiglu_quant_gbs": round(swiglu_bytes(w) / t_s / 1e3, 1)}
    if comparators:
        r.update(measure_comparators(torch, q, w, W, x8, sx, y, ws, t_g, reps, packed_host))
    del ws
    return r


def _counter_rows(d: str, counter: str):
    """(kernel name, grid, dispatch id) -> summed value of one counter, from
    the counter_collection CSV files rocprofv3 wrote under directory d."""
    import csv
    import glob
    vals = {}
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f, newline="") as fh:
            for row in csv.DictReader(fh):
                if row.get("Counter_Name") != counter:
                    continue
                key = (row["Kernel_Name"], int(row["Grid_Size"]), int(row["Dispatch_Id"]))
                vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    return vals


def write_traffic(workload: str, fetch_dir: str, write_dir: str, commands: list[str]) -> dict:
    """profiles/traffic_<workload>.json from the FETCH_SIZE and WRITE_SIZE
    passes of `bench.py --workload <workload> --no-sweep --copy-calib-mb N`:
    both counters in KiB per dispatch, scaled so that the run's device copy
    of known size reads as its size fetched and written; summed over the GEMM
    call's kernels, each the mean over its dispatches."""
    import synthetic
    w = synthetic.get_workload(workload)
    fetch, write = _counter_rows(fetch_dir, "FETCH_SIZE"), _counter_rows(write_dir, "WRITE_SIZE")
    copy_f = [v for (k, _, _), v in fetch.items() if "copyBuffer" in k]
    copy_w = [v for (k, _, _), v in write.items() if "copyBuffer" in k]
    calib_kib = max(copy_w)  # the largest copy is the calibration copy (read and write N bytes)
    fs, ws = calib_kib / max(copy_f), 1.0 * calib_kib / max(copy_w)
    kern = {}
    for src, name in ((fetch, "fetch_kib"), (write, "write_kib")):
        for (k, grid, _), v in src.items():
            if "gemm_" in k or "splitk_reduce" in k:
                short = k.replace("void ", "", 1).replace("qoq::(anonymous namespace)::", "").split("(")[0]
                e = kern.setdefault((short, grid),
                                    {"fetch_kib": [], "write_kib": []})
                e[name].append(v)
    rows = []
    total = 0
    for (k, grid), e in sorted(kern.items()):
        f = sum(e["fetch_kib"]) / max(1, len(e["fetch_kib"]))
        wv = sum(e["write_kib"]) / max(1, len(e["write_kib"]))
        b = int(round((f * fs + wv * ws) * 1024))
        total += b
        rows.append({"kernel": k, "grid": grid, "dispatches": len(e["fetch_kib"]), "fetch_kib": round(f, 1),
                     "write_kib": round(wv, 1), "bytes": b})
    rec = {"workload": workload, "copy_fetch_kib": round(max(copy_f), 2), "copy_write_kib": round(max(copy_w), 2),
           "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "kernels": rows,
           "hbm_bytes_per_launch": total, "algorithmic_bytes": algo_bytes(w),
           "ratio": round(total / algo_bytes(w), 3), "src_hash": src_hash(), "commands": commands,
           "note": "hbm_bytes_per_launch = FETCH_SIZE x fetch_scale + WRITE_SIZE x write_scale (KiB -> bytes) over "
                   "the GEMM call's kernels, mean over its dispatches; the scales make the run's device copy of known "
                   "size read as that size fetched and written.  FETCH_SIZE counts L2 misses, served by the 256 MB "
                   "last-level cache or by HBM."}
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.json"), "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    return rec


def main():
    if len(sys.argv) > 1 and sys.argv[1] == "--traffic-from":
        # bench.py --traffic-from WORKLOAD FETCH_DIR WRITE_DIR: host only, no GPU
        wl, fd, wd = sys.argv[2:5]
        cmd = ("rocprofv3 --pmc {c} --output-format csv -d {d} -o pmc -- python -u bench.py --workload {w} "
               "--no-sweep --no-cpu-baseline --no-kv4 --copy-calib-mb 1024 --steps 5 --warmup 2 --kernel-reps 5")
        rec = write_traffic(wl, fd, wd, [cmd.format(c="FETCH_SIZE", d=fd, w=wl), cmd.format(c="WRITE_SIZE", d=wd, w=wl)])
        print(json.dumps({k: rec[k] for k in ("workload", "fetch_scale", "hbm_bytes_per_launch", "ratio")}))
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="ffn_large_g128")
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--sweep", default=",".join(SWEEP), help="comma-separated workload names")
    ap.add_argument("--sweep-reps", type=int, default=20)
    ap.add_argument("--no-kv4", action="store_true", help="skip the KV4 attention measurement")
    ap.add_argument("--no-comparators", action="store_true",
                    help="skip the W8A8 comparator and the saturating ablation in the sweep")
    ap.add_argument("--kernel-reps", type=int, default=100)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--cpu-leg-seconds", type=float, default=0.5,
                    help="seconds per one-thread / all-thread oracle leg on the smaller workloads")
    ap.add_argument("--no-cpu-legs", action="store_true")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}); "
              "the W4A8 GEMM is measured on one MI355X.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synthetic
    import w4a8_quantized_gemm_qoq_amd as q

    q.load_library()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda")
    w = synthetic.get_workload(args.workload)
    X, W = synthetic.make_inputs(w)

    # resident inputs and outputs
    t_pack0 = time.perf_counter()
    packed = q.qoq_pack_weights(W, w.group_size)
    t_pack = time.perf_counter() - t_pack0
    p = packed.to(dev)
    # Several copies of the packed weights, cycled from step to step, so that
    # the weights come from HBM as they would for the distinct layers of a
    # model (one copy would stay in the 256 MB last-level cache).
    wbytes = packed.qweight.nbytes + packed.meta.nbytes
    copies = max(1, min(64, math.ceil(3 * MALL_BYTES / max(1, wbytes))))
    pw = [p] + [packed.to(dev) for _ in range(copies - 1)]
    x = torch.from_numpy(X).to(dev)
    x8 = torch.empty((w.M, w.K), dtype=torch.int8, device=dev)
    sx = torch.empty((w.M,), dtype=torch.float16, device=dev)
    y = torch.empty((w.M, w.N), dtype=torch.float16, device=dev)

    def step(i=0):
        q.qoq_quant_act_per_token(x, x8, sx)
        q.qoq_w4a8_gemm(x8, sx, pw[i % copies], y=y)

    # eager warmup, then capture the K timed steps in one HIP graph so that
    # host launch overhead does not enter the measurement
    for _ in range(max(1, args.warmup)):
        step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        for i in range(args.steps):
            step(i)
    g.replay()  # warm replay (untimed)
    torch.cuda.synchronize()

    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    wall_s = t1 - t0
    gpu_ms = e0.elapsed_time(e1)
    ms_per_step = 1e3 * wall_s / args.steps

    # correctness of the timed output against a direct launch (same kernels)
    y_graph = y.clone()
    step(args.steps - 1)
    torch.cuda.synchronize()
    assert torch.equal(y_graph.view(torch.int16), y.view(torch.int16)), "graph replay output differs"

    # dominant kernel: the GEMM; average launch duration from HIP events,
    # with the same weight rotation as the timed steps
    gemm_us = time_kernel(torch, lambda i: q.qoq_w4a8_gemm(x8, sx, pw[i % copies], y=y), args.kernel_reps)
    ws_bytes = q.load_library().qoq_w4a8_gemm_workspace_size(w.M, w.N, w.K, w.group_size)
    quant_us = time_kernel(torch, lambda i: q.qoq_quant_act_per_token(x, x8, sx), args.kernel_reps)
    bnd = bound_of(w)
    if bnd == "mfma":
        achieved, peak, unit = w.ops / gemm_us / 1e6, PEAK_INT8_TOPS, "TOPS"
        per_unit = "2*M*N*K int8 ops per launch"
    else:
        achieved, peak, unit = algo_bytes(w) / gemm_us / 1e3, PEAK_HBM_GBS, "GB/s"
        per_unit = "algorithmic bytes per launch"

    traffic = stored_traffic(w.name)

    out = {
        "metric": METRIC,
        "value": round(w.ops * args.steps / wall_s / 1e12, 3),
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8",
        "data": "synthetic",
        "config": {"workload": w.name, "desc": w.desc, "M": w.M, "K": w.K, "N": w.N,
                   "group_size": w.group_size, "step": "per-token INT8 quant + W4A8 GEMM (FP16 out)",
                   "timing": "K steps captured in one HIP graph, replayed once between synchronizations",
                   "weight_copies": copies},
        "gpu_ms_per_step": round(gpu_ms / args.steps, 5),
        "roofline": {"bound": bnd, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "kernel": ("qoq_w4a8_gemm = gemm_large_kernel (K split) + splitk_reduce_kernel" if ws_bytes
                                else "qoq_w4a8_gemm (one kernel)"),
                     "kernel_us": round(gemm_us, 3), "per_unit": per_unit, "weight_copies": copies,
                     "algorithmic_bytes": algo_bytes(w), "ops": w.ops},
        "act_quant_us": round(quant_us, 3),
        "gemm_gbs_algorithmic": round(algo_bytes(w) / gemm_us / 1e3, 1),
        "host_pack_s": round(t_pack, 3),
        "src_hash": src_hash(),
    }

    if not args.no_sweep:
        sweep = []
        for name in [n for n in args.sweep.split(",") if n]:
            sw = synthetic.get_workload(name)
            SX, SW = synthetic.make_inputs(sw)
            try:
                r = measure_gemm(torch, q, sw, SX, SW, args.sweep_reps, comparators=not args.no_comparators)
            except Exception as ex:  # report, do not hide
                r = {"workload": name, "error": repr(ex)}
            print(f"[sweep] {json.dumps(r)}", file=sys.stderr, flush=True)
            sweep.append(r)
            del SX, SW
            torch.cuda.empty_cache()
        out["sweep"] = sweep
        if not args.no_comparators:
            out["comparators"] = {
                "w4a8_over_w8a8": {r["workload"]: r["w4a8_over_w8a8"] for r in sweep if "w4a8_over_w8a8" in r},
                "saturating_slowdown": {r["workload"]: r["saturating_slowdown"] for r in sweep
                                        if "saturating_slowdown" in r},
                "w4a8_over_hipblaslt_w8a8": {r["workload"]: r["w4a8_over_hipblaslt_w8a8"] for r in sweep
                                             if r.get("w4a8_over_hipblaslt_w8a8") is not None},
                "note": "same kernels and plans; W8A8 = per-channel INT8 weights without dequantization; "
                        "saturating = g128 GEMM with a clamping 16-bit-lane dequantization; "
                        "hipblaslt = the vendor library's INT8 GEMM (torch._int_mm, INT32 out) on the same shape",
            }

    if not args.no_kv4:
        try:
            out["kv4"] = measure_kv4(torch, q, args.sweep_reps)
        except Exception as ex:  # report, do not hide
            out["kv4"] = [{"error": repr(ex)}]
        print(f"[kv4] {json.dumps(out['kv4'])}", file=sys.stderr, flush=True)

    if args.copy_calib_mb:
        n = args.copy_calib_mb * 2 ** 20
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        out["copy_calib_bytes"] = n

    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, X, W, args.cpu_seconds)
        print(f"[cpu_baseline] {json.dumps(out['cpu_baseline'])}", file=sys.stderr, flush=True)
        out["host_encode"] = encode_vs_pack(w, W, q)
        print(f"[host_encode] {json.dumps(out['host_encode'])}", file=sys.stderr, flush=True)
        if not args.no_cpu_legs:
            out["cpu_legs"] = cpu_legs(args.cpu_leg_seconds)
            print(f"[cpu_legs] {json.dumps(out['cpu_legs'])}", file=sys.stderr, flush=True)
    else:
        out["cpu_baseline"] = None

    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
