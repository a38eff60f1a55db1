#!/usr/bin/env python3
"""Benchmark of the causal GQA attention hot path on one MI355X.

One step = fa_fwd + fa_bwd_delta + fa_bwd (dQ kernel, then dK/dV kernel) over
one batch of resident synthetic bf16 inputs of the 8192-token training shape
(B=1, 32 query heads, 8 key/value heads, head dim 128, causal).  Prints one
JSON line with the throughput under the FLOP model of the pages (forward
4*B*Hq*Lq*Lk*D, backward 2.5x that, both halved for causal), the roofline
position of the dominant kernel (timed with HIP events on the stream the
kernels run on), peak device memory, and the fp64 CPU oracle timed on a
bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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

METRIC = "fwd+bwd TFLOP/s, causal GQA bf16 attention D=128 L=8192; % of MFMA peak"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU * 4096 FLOP/clk * 2.4 GHz
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
PROFILE_DIR = os.path.join(ROOT, "profiles")


# ------------------------------------------------------------ FLOP accounting

def model_flops(B, Hq, Lq, Lk, D, causal, backward=True):
    """The pages' model: forward 4*B*Hq*Lq*Lk*D, backward 2.5x the forward,
    both halved under a causal mask (VJP page, Background)."""
    fwd = 4.0 * B * Hq * Lq * Lk * D
    if causal:
        fwd /= 2.0
    return fwd * (3.5 if backward else 1.0), fwd


def masked_model_flops(B, Hq, D, pairs, backward=True):
    """The same model counted over the pairs a block mask leaves visible:
    forward 4*D per pair, backward 2.5x that."""
    fwd = 4.0 * B * Hq * D * pairs
    return fwd * (3.5 if backward else 1.0), fwd


def visible_pairs(Lq, Lk, causal):
    """Exact number of (query, key) pairs inside the mask of one head."""
    if not causal:
        return Lq * Lk
    # causal needs Lq <= Lk; row i sees keys 0 .. i + (Lk - Lq), never past Lk - 1
    off = Lk - Lq
    return Lq * (off + 1) + Lq * (Lq - 1) // 2


def visible_pairs_masked(Lq, Lk, causal, mask):
    """Exact number of visible (query, key) pairs of one head under a 64 x 64
    block mask (and the bottom-right causal diagonal, if any)."""
    import numpy as np
    blk = 64
    nkb = mask.shape[1]
    starts = np.arange(nkb) * blk
    ends = np.minimum(starts + blk, Lk)
    rows = np.arange(Lq)
    lim = (rows + (Lk - Lq) + 1) if causal else np.full(Lq, Lk)  # keys < lim are seen
    per = np.clip(np.minimum(ends[None, :], lim[:, None]) - starts[None, :], 0, None)
    return int((per * (mask[rows // blk] != 0)).sum())


def unfused_score_bytes(H, L, bytes_per=2):
    """Bytes of one materialised [H, L, L] score matrix (the unfused backward's
    dominant buffer; VJP page, Memory table, "Attn Matrix Size")."""
    return H * L * L * bytes_per


# per-kernel algorithmic work: MFMA FLOP per visible pair (S, P V | S, dP, dQ |
# S, dP, dV, dK) and HBM bytes for the delta pass
KERNEL_FLOP_PER_PAIR = {"fwd": 4, "dq": 6, "dkv": 8}


def kernel_work(w, pairs):
    bh = w.B * w.Hq
    work = {k: c * w.D * pairs * bh for k, c in KERNEL_FLOP_PER_PAIR.items()}
    work["delta"] = 2 * bh * w.Lq * w.D * 2 + bh * w.Lq * 4  # read O, dO; write delta
    return work


def short_bytes(w):
    """Algorithmic HBM bytes per kernel of the short-query path (each tensor
    read or written once; the fp32 partials in the workspace are the
    implementation's, not the algorithm's)."""
    e = 2  # bytes per element
    kv = w.B * w.Hkv * w.Lk * w.D * e          # one of K, V, dK, dV
    qrow = w.B * w.Hq * w.Lq * w.D * e         # one of Q, O, dO, dQ
    stat = w.B * w.Hq * w.Lq * 4               # LSE or delta
    return {"fwd": 2 * kv + 2 * qrow + stat, "dq": 2 * kv + 3 * qrow + 2 * stat,
            "dkv": 4 * kv + 2 * qrow + 2 * stat, "delta": 2 * qrow + stat}


# ------------------------------------------------------------ traffic record

def _code_only(text):
    """C/C++ source without comments and with whitespace runs collapsed: what
    the compiler sees.  String literals in these sources hold no comment
    markers."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_digest(root=ROOT):
    """Digest of the kernel sources' code (comments and layout ignored)."""
    import glob
    h = hashlib.sha256()
    for p in sorted(glob.glob(os.path.join(root, "causal_gqa_flashattention_amd", "csrc", "*"))):
        if not os.path.isfile(p):
            continue
        with open(p, encoding="utf-8", errors="replace") as f:
            h.update(os.path.basename(p).encode() + b"\0" + _code_only(f.read()).encode())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when
    the kernels changed after the counters were taken."""
    p = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    if not os.path.exists(p):
        return None
    with open(p) as f:
        rec = json.load(f)
    if rec.get("source_digest") != source_digest():
        return None
    k = rec.get("kernels", {}).get(kernel)
    return None if k is None else k.get("hbm_bytes")


COPY_MIB = [256, 1024]


def summarize_pmc(fetch_csv, write_csv, workload):
    """HBM bytes per kernel launch from FETCH_SIZE / WRITE_SIZE (KiB per
    dispatch), each scaled by the factor that maps the same counter to the
    known size of the calibration copies."""
    import csv

    def load(path, counter):
        rows = []
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        return sorted(rows)

    out = {"workload": workload, "source_digest": source_digest(), "kernels": {}, "calibration": {}}
    vals = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = load(path, counter)
        copies = [v for _, n, v in rows if "copy" in n.lower()]
        if len(copies) != len(COPY_MIB):
            raise SystemExit(f"expected {len(COPY_MIB)} copy dispatches in {path}, found {len(copies)}")
        factors = [mib * 1024 / kib for mib, kib in zip(COPY_MIB, copies)]  # true KiB / counted KiB
        factor = sum(factors) / len(factors)
        out["calibration"][counter] = {"copy_mib": COPY_MIB, "counted_kib": copies, "factor": factor}
        for _, n, v in rows:
            # every kernel variant of a stage (e.g. fa_fwd_kernel, fa_fwd_pp_kernel)
            for key, tag in (("fwd", "cgqa::fa_fwd_"), ("delta", "cgqa::fa_delta_"),
                             ("dq", "cgqa::fa_dq_"), ("dkv", "cgqa::fa_dkv_")):
                if tag in n:  # a stage's kernels add up (dK/dV: its split reduction too)
                    d = vals.setdefault(key, {})
                    d[counter] = d.get(counter, 0.0) + v * factor * 1024
    for key, d in vals.items():
        out["kernels"][key] = {"fetch_bytes": round(d.get("FETCH_SIZE", 0.0)),
                               "write_bytes": round(d.get("WRITE_SIZE", 0.0)),
                               "hbm_bytes": round(d.get("FETCH_SIZE", 0.0) + d.get("WRITE_SIZE", 0.0))}
    os.makedirs(PROFILE_DIR, exist_ok=True)
    dst = os.path.join(PROFILE_DIR, f"traffic_{workload}.json")
    with open(dst, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out))
    return 0


# ------------------------------------------------------------ CPU oracle leg

def cpu_baseline(w, bits, budget_s=30.0, mask=None, pairs=None):
    """Time the fp64 oracle on one whole GQA group (its query heads, all rows,
    forward + backward) of the same inputs; report model TFLOP/s of that
    sample.  The group is 1/(B*Hkv) of the workload's model FLOPs.  Under a
    block mask the FLOPs are those of the visible pairs (`pairs` per head)."""
    import numpy as np

    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    G = w.Hq // w.Hkv
    k = oracle.bits_to_f64(bits["k"][0, 0], w.dtype)
    v = oracle.bits_to_f64(bits["v"][0, 0], w.dtype)
    t0 = time.perf_counter()
    heads_done = 0
    for h in range(G):
        q = oracle.bits_to_f64(bits["q"][0, h], w.dtype)
        do = oracle.bits_to_f64(bits["do"][0, h], w.dtype)
        oracle.head_backward(q, k, v, do, w.softmax_scale, w.causal, block_mask=mask)
        heads_done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = time.perf_counter() - t0
    if mask is None:
        total, _ = model_flops(1, heads_done, w.Lq, w.Lk, w.D, w.causal)
        full, _ = model_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal)
    else:
        total, _ = masked_model_flops(1, heads_done, w.D, pairs)
        full, _ = masked_model_flops(w.B, w.Hq, w.D, pairs)
    del np
    if w.Lq <= 8:  # the short-query workloads are measured in algorithmic HBM bytes
        share = sum(short_bytes(w).values()) / (w.B * w.Hkv) * heads_done / G
        full_s = dt * (w.B * w.Hkv) * G / heads_done
        return {"value": share / dt / 1e9, "unit": "GB/s", "cores": int(cores), "kind": "oracle",
                "sample": f"{heads_done} query heads of key/value head 0 (one GQA group), all {w.Lq} rows, "
                          f"fp64 forward+backward, {dt:.2f} s",
                "full_workload_s_extrapolated": round(full_s, 1)}
    return {"value": total / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{heads_done} query heads of key/value head 0 (one GQA group), all {w.Lq} rows, "
                      f"fp64 forward+backward, {dt:.2f} s",
            "full_workload_s_extrapolated": round(dt * full / total, 1)}


def executed_mfma(w, split=None):
    """Matrix work the kernels issue for workload w, following their tilings
    (diagonal tiles run whole, waves past Lq idle), in units of one
    32x32x16 instruction (32768 FLOP; a 16x16x32 one counts half).  Where
    only 32x32x16 instructions run (D <= 128) it is the count SQ_INSTS_MFMA
    should read.  `split`: whether dK/dV runs with a load-balancing
    workspace (bench.py uses one whenever the library plans a split; at head
    dim 256 that is the 64-key kernel; a split shares the same iterations
    between workgroups and changes no count)."""
    cdiv = lambda a, b: -(-a // b)
    D, B, Hq, Hkv, Lq, Lk = w.D, w.B, w.Hq, w.Hkv, w.Lq, w.Lk
    G, off, causal = Hq // Hkv, Lk - Lq, w.causal
    NKD, NDB = D // 16, D // 32

    def kv_end(row_end):  # keys seen by rows < row_end
        return min(Lk, min(row_end, Lq) + off) if causal else Lk

    fwd = 0
    if D in (96, 128):  # 8-wave ping-pong, 256 rows, 64-key tiles
        per_tile = 2 * NKD + NDB * 4
        for qt in range(cdiv(Lq, 256)):
            for wv in range(8):
                r0 = qt * 256 + 32 * wv
                if r0 < Lq:
                    fwd += per_tile * cdiv(kv_end(r0 + 32), 64)
    else:  # 4 waves, 128 rows, 64-key tiles
        per_tile = 2 * NKD + NDB * 4
        for qt in range(cdiv(Lq, 128)):
            fwd += 4 * per_tile * cdiv(kv_end(qt * 128 + 128), 64)
    dq = 0  # 4 waves, 128 rows, 64-key tiles
    for qt in range(cdiv(Lq, 128)):
        dq += 4 * (4 * NKD + NDB * 4) * cdiv(kv_end(qt * 128 + 128), 64)
    # dK/dV, query tiles of 64: 8 waves x 128 keys up to D = 128; at D = 256
    # 4 waves x 64 keys, or x 32 keys (16 rows each) below 512 64-key workgroups
    if split is None:
        split = split_planned(w)
    if D != 256:
        bnk, per_iter = 128, 8 * (2 * NKD + 4 * NDB)
    elif split or B * Hkv * cdiv(Lk, 64) >= 512:
        bnk, per_iter = 64, 4 * (2 * NKD + 4 * NDB)
    else:
        bnk, per_iter = 32, 4 * (2 * (D // 32) + 2 * NDB)
    dkv = 0
    for kt in range(cdiv(Lk, bnk)):
        qfirst = max(0, kt * bnk - off) if causal else 0
        nq = max(0, cdiv(Lq, 64) - qfirst // 64)
        dkv += G * nq * per_iter
    return {"fwd": fwd * B * Hq, "dq": dq * B * Hq, "dkv": dkv * B * Hkv}


def split_planned(w):
    """Whether bench.py runs this workload's dK/dV with a split workspace: the
    library's own plan (fa_bwd_workspace_bytes), mirrored here for the
    counter summaries, which run without a GPU."""
    cdiv = lambda a, b: -(-a // b)
    if w.Lq <= 8:
        return False
    bnk = 64 if w.D > 128 else 128
    wgs = w.B * w.Hkv * cdiv(w.Lk, bnk)
    if w.mask is not None:
        return cdiv(w.Lq, 64) >= 2
    return wgs < 512 and cdiv(w.Lq, 64) >= 2


def summarize_inst(csv_path, workload):
    """SQ_INSTS_MFMA per launch against executed_mfma(); GRBM_GUI_ACTIVE over
    the dispatch duration gives the mean shader clock (summed over XCDs)."""
    import csv
    from fa_synth import WORKLOADS
    w = WORKLOADS[workload]
    want = executed_mfma(w)
    rows = {}
    for r in csv.DictReader(open(csv_path)):
        n = r["Kernel_Name"]
        key = next((k for k, t in (("fwd", "cgqa::fa_fwd_"), ("dq", "cgqa::fa_dq_"), ("dkv", "cgqa::fa_dkv_"))
                    if t in n), None)
        if key is None:
            continue
        # a stage's dispatches add up (dK/dV: its split reduction too); each
        # dispatch's duration counted once
        d = rows.setdefault(key, {"dispatches": set()})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
        if r["Dispatch_Id"] not in d["dispatches"]:
            d["dispatches"].add(r["Dispatch_Id"])
            d["dur_ns"] = d.get("dur_ns", 0) + int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    out = {"workload": workload, "kernels": {}}
    for k, d in rows.items():
        e = {"counted_mfma": int(d.get("SQ_INSTS_MFMA", 0)), "analytic_mfma": want[k]}
        e["ratio"] = round(e["counted_mfma"] / e["analytic_mfma"], 4) if want[k] else None
        if "GRBM_GUI_ACTIVE" in d and d["dur_ns"]:
            e["clock_ghz"] = round(d["GRBM_GUI_ACTIVE"] / 8 / d["dur_ns"], 3)  # 8 XCDs
        if "SQ_INSTS_VALU" in d:
            e["valu_per_mfma"] = round(d["SQ_INSTS_VALU"] / max(1.0, d.get("SQ_INSTS_MFMA", 1.0)), 2)
        out["kernels"][k] = e
    print(json.dumps(out))
    return 0


# ------------------------------------------------------------ main

def realtime_counter_hz(lib, dev):
    """The s_memrealtime counter's rate against HIP events (csrc/probe: one
    wavefront spins on it for 5e6 ticks); the clock figures assume 100 MHz."""
    import ctypes
    import torch
    if not hasattr(lib, "cgqa_counter_rates"):
        return None
    f = lib.cgqa_counter_rates
    f.argtypes = [ctypes.c_void_p, ctypes.c_uint64, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    f.restype = ctypes.c_int
    st = torch.zeros(4, dtype=torch.int64, device=dev)
    rt, mt = ctypes.c_double(), ctypes.c_double()
    rc = f(st.data_ptr(), 5_000_000, ctypes.byref(rt), ctypes.byref(mt))
    torch.cuda.synchronize()
    return round(rt.value) if rc == 0 else None


def mfma_ceiling(dev, cus):
    """Sustained MFMA throughput (csrc/probe) with constant and with random
    bf16 operands: the second is what kernels on real data can approach,
    since the chip lowers its clock as operand toggling raises its power."""
    import ctypes
    import torch
    from causal_gqa_flashattention_amd.build import PKG_DIR, PROBE_LIB_NAME
    from fa_synth import normal_bf16_bits
    path = os.path.join(PKG_DIR, PROBE_LIB_NAME)
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    fn = lib.cgqa_mfma_ceiling
    fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                   ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]
    fn.restype = ctypes.c_int
    bits = torch.from_numpy(normal_bf16_bits((8192 * 8,), seed=7, sigma=1.0).view("int16")).to(dev)
    out = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    c, r = ctypes.c_double(), ctypes.c_double()
    torch.cuda.synchronize()
    rc = fn(bits.data_ptr(), out.data_ptr(), cus, 2048, 10, ctypes.byref(c), ctypes.byref(r))
    torch.cuda.synchronize()
    if rc != 0:
        raise RuntimeError(f"mfma ceiling probe failed: {rc}")
    res = {"constant_operands": round(c.value, 1), "random_operands": round(r.value, 1), "unit": "TFLOP/s",
           "kernel": "v_mfma_f32_32x32x16_bf16, 2 wavefronts/SIMD, 4 accumulators each, operands in registers"}
    # the same loops once more with s_memtime / s_memrealtime stamps: the
    # shader clock they ran at
    if hasattr(lib, "cgqa_mfma_clock"):
        fc = lib.cgqa_mfma_clock
        dbl = ctypes.POINTER(ctypes.c_double)
        fc.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                       ctypes.c_int, ctypes.c_int, ctypes.c_double] + [dbl] * 4
        fc.restype = ctypes.c_int
        stamps = torch.zeros(6 * cus, dtype=torch.int64, device=dev)
        host = (ctypes.c_uint64 * (6 * cus))()
        v = [ctypes.c_double() for _ in range(4)]
        rc = fc(bits.data_ptr(), out.data_ptr(), stamps.data_ptr(), ctypes.addressof(host), cus, 2048, 10, 100e6,
                *(ctypes.byref(x) for x in v))
        torch.cuda.synchronize()
        if rc == 0:
            tc, gc, tr, gr = (x.value for x in v)
            res["clock"] = {
                "realtime_counter_hz": realtime_counter_hz(lib, dev),
                "constant": {"TFLOP/s": round(tc, 1), "shader_ghz": round(gc, 3)},
                "random": {"TFLOP/s": round(tr, 1), "shader_ghz": round(gr, 3)},
                "method": "shader clock = s_memtime ticks per s_memrealtime second (100 MHz) over the loop of "
                          "wave 0 of each workgroup, median over workgroups, in the last of 10 timed launches",
            }
    return res


def power_sample(dev, w, secs=3.0):
    """Board power and shader clock (amd-smi, sampled from a thread) while
    each attention kernel of workload w runs back to back for `secs`
    seconds, and while the matrix-core probe's random- and constant-operand
    loops do: whether a kernel runs at the power limit, and at what clock."""
    import ctypes
    import subprocess
    import threading
    import numpy as np
    import torch
    import causal_gqa_flashattention_amd as fa
    from causal_gqa_flashattention_amd.build import PKG_DIR, PROBE_LIB_NAME
    from fa_synth import make_inputs, normal_bf16_bits

    def smi(stop, recs):
        while not stop.is_set():
            r = subprocess.run(["amd-smi", "metric", "-g", "0", "-p", "-c", "--json"], capture_output=True, text=True)
            try:
                gd = json.loads(r.stdout)["gpu_data"][0]
                recs.append((gd["power"]["socket_power"]["value"],
                             float(np.mean([v["clk"]["value"] for k, v in gd["clock"].items() if k.startswith("gfx_")]))))
            except Exception:  # pragma: no cover - a sample the tool could not give
                pass
            time.sleep(0.05)

    bits = make_inputs(w, with_grad=True)
    g = {n: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for n, b in bits.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sc, causal = w.softmax_scale, w.causal
    fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal)
    fa.fa_bwd_delta(o, do, delta)
    plib = ctypes.CDLL(os.path.join(PKG_DIR, PROBE_LIB_NAME))
    loop = plib.cgqa_mfma_loop
    loop.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int]
    loop.restype = ctypes.c_double
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    pb = torch.from_numpy(normal_bf16_bits((8192 * 8,), seed=7, sigma=1.0).view("int16")).to(dev)
    pout = torch.empty(cus * 512, dtype=torch.float32, device=dev)
    calls = {
        "fwd": lambda: fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal),
        "dq": lambda: fa.fa_bwd_dq(q, k, v, lse, delta, do, dq, scale=sc, causal=causal),
        "dkv": lambda: fa.fa_bwd_dkv(q, k, v, lse, delta, do, dk, dv, scale=sc, causal=causal),
    }
    flops = kernel_work(w, visible_pairs(w.Lq, w.Lk, w.causal))
    out = {}
    for mode in ("idle", "fwd", "dq", "dkv", "mfma_random", "mfma_constant"):
        torch.cuda.synchronize()
        recs, stop = [], threading.Event()
        th = threading.Thread(target=smi, args=(stop, recs))
        th.start()
        time.sleep(0.3)
        t0, ms = time.time(), []
        while time.time() - t0 < secs:
            if mode == "idle":
                time.sleep(0.05)
            elif mode.startswith("mfma"):
                ms.append(loop(pb.data_ptr(), pout.data_ptr(), cus, 2048, 5, int(mode == "mfma_random")) / 5)
            else:
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for _ in range(20):
                    calls[mode]()
                e1.record()
                torch.cuda.synchronize()
                ms.append(e0.elapsed_time(e1) / 20)
        stop.set()
        th.join()
        rec = {"samples": len(recs)}
        if recs:
            W, C = np.array([r[0] for r in recs], dtype=float), np.array([r[1] for r in recs])
            rec.update({"power_w_median": float(np.median(W)), "power_w_max": float(W.max()),
                        "gfx_mhz_median": float(np.median(C))})
        if ms:
            t = float(np.median(ms))
            rec["ms"] = round(t, 4)
            f = 2.0 * 32 * 32 * 16 * 32 * 2048 * cus * 8 if mode.startswith("mfma") else flops[mode]
            rec["TFLOP/s"] = round(f / (t * 1e-3) / 1e12, 1)
        out[mode] = rec
    return out


def gemm_canary(dev, n=4096, reps=10):
    """A plain bf16 n^3 library GEMM timed after the step: a clock and
    contention sanity check for the box (its value is context, not a target)."""
    import torch
    a = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    b = torch.randn((n, n), device=dev, dtype=torch.bfloat16)
    c = a @ b
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b, c
    return {"shape": f"{n}x{n}x{n} bf16", "ms": round(ms, 4), "TFLOP/s": round(2 * n ** 3 / (ms * 1e-3) / 1e12, 1)}


# The other configurations of the path, timed after the headline one: every
# workload of the five configurations that is not the headline shape.
SWEEP = ("dense4k_d64", "dense4k_d96", "d256_8192", "d256_4064x4096", "d256_8200", "long23k")


def workload_sweep(dev, names=SWEEP, min_steps=20, warm_s=0.15, timed_s=0.25):
    """For each workload: fa_fwd, fa_bwd_delta, fa_bwd_dq and fa_bwd_dkv on
    resident inputs (the same seeded recipe as the headline), timed with HIP
    events on the launch stream; medians over the timed steps.  Each
    workload first runs for at least `warm_s` seconds (the clock takes tens
    of milliseconds to settle after the load changes: 25 steps of a 0.7 ms
    workload measured 8% slow), then times at least `min_steps` steps and
    `timed_s` seconds.  Model TFLOP/s use the pages' FLOP model (the
    head-dim-256 shapes are a forward workload: their forward figure is the
    one to read; the backward there is timed as well)."""
    import numpy as np
    import torch

    import causal_gqa_flashattention_amd as fa
    from fa_synth import WORKLOADS, make_inputs

    out = {}
    stream = torch.cuda.current_stream()
    for name in names:
        w = WORKLOADS[name]
        bits = make_inputs(w, with_grad=True)
        g = {n: torch.from_numpy(b.view(np.int16)).view(torch.bfloat16).to(dev) for n, b in bits.items()}
        del bits
        q, k, v, do = g["q"], g["k"], g["v"], g["do"]
        o = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)
        delta = torch.empty_like(lse)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        sc, causal = w.softmax_scale, w.causal
        # dK/dV with the load-balancing workspace where the library plans a
        # split for this shape (allocated here, outside the timed steps)
        ws_bytes = fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D)
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
        torch.cuda.synchronize()
        torch.cuda.reset_peak_memory_stats()
        resident = torch.cuda.memory_allocated()

        def dkv_call():
            if ws is None:
                fa.fa_bwd_dkv(q, k, v, lse, delta, do, dk, dv, scale=sc, causal=causal, stream=stream)
            else:
                fa.fa_bwd_ex(q, k, v, lse, delta, do, None, dk, dv, scale=sc, causal=causal, grads="dkv",
                             workspace=ws, stream=stream)

        def step(ev=None):
            if ev is not None:
                ev[0].record(stream)
            fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal, stream=stream)
            if ev is not None:
                ev[1].record(stream)
            fa.fa_bwd_delta(o, do, delta, stream=stream)
            if ev is not None:
                ev[2].record(stream)
            fa.fa_bwd_dq(q, k, v, lse, delta, do, dq, scale=sc, causal=causal, stream=stream)
            if ev is not None:
                ev[3].record(stream)
            dkv_call()
            if ev is not None:
                ev[4].record(stream)

        t0 = time.perf_counter()
        warmup = 0
        while True:
            step()
            warmup += 1
            if warmup % 4 == 0:
                torch.cuda.synchronize()
                if time.perf_counter() - t0 >= warm_s:
                    break
        steps = max(min_steps, int(math.ceil(timed_s / ((time.perf_counter() - t0) / warmup))))
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        med = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs]))
               for j, n in enumerate(("fwd", "delta", "dq", "dkv"))}
        step_ms = float(np.median([e[0].elapsed_time(e[4]) for e in evs]))
        total, fwd_f = model_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal)
        bwd_f = total - fwd_f
        kind = "causal" if w.causal else "dense"
        out[name] = {
            "shape": f"{kind} GQA bf16, B={w.B} Hq={w.Hq} Hkv={w.Hkv} Lq={w.Lq} Lk={w.Lk} D={w.D}",
            "kernels_median_ms": {n: round(t, 4) for n, t in med.items()},
            "step_median_ms": round(step_ms, 4),
            "fwd_TFLOP/s": round(fwd_f / (med["fwd"] * 1e-3) / 1e12, 1),
            "bwd_TFLOP/s": round(bwd_f / ((med["delta"] + med["dq"] + med["dkv"]) * 1e-3) / 1e12, 1),
            "fwd+bwd_TFLOP/s": round(total / (step_ms * 1e-3) / 1e12, 1),
            "frac_of_peak": round(total / (step_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "fwd_frac_of_peak": round(fwd_f / (med["fwd"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "peak_bytes": int(torch.cuda.max_memory_allocated()),
            "resident_bytes": int(resident),
            "dkv_call": "fa_bwd_dkv" if ws is None else f"fa_bwd_ws ({ws_bytes} bytes of workspace)",
            "warmup_steps": warmup,
            "timed_steps": steps,
        }
        del g, q, k, v, do, o, lse, delta, dq, dk, dv, ws
        torch.cuda.empty_cache()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="train8k")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip timing the other configurations (the 'workloads' key)")
    ap.add_argument("--profile-pass", action="store_true",
                    help="copy kernels of known size plus one step, for counter runs")
    ap.add_argument("--summarize-inst", metavar="CSV",
                    help="SQ_INSTS_MFMA (and GRBM_GUI_ACTIVE, SQ_INSTS_VALU) of a --profile-pass "
                         "counter run against the kernels' analytic MFMA counts")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only run the matrix-core throughput probe and print its JSON")
    ap.add_argument("--power", action="store_true",
                    help="only sample board power and clock (amd-smi) while each kernel, and the "
                         "matrix-core probe, runs back to back; print its JSON")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="turn two rocprofv3 --pmc counter_collection.csv files (FETCH_SIZE, "
                         "WRITE_SIZE) of a --profile-pass run into profiles/traffic_<workload>.json")
    args = ap.parse_args(argv)

    if args.summarize_pmc:
        return summarize_pmc(args.summarize_pmc[0], args.summarize_pmc[1], args.workload)
    if args.summarize_inst:
        return summarize_inst(args.summarize_inst, args.workload)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the path shards by GQA group with no exchange; see the design notes)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import causal_gqa_flashattention_amd as fa
    from fa_synth import WORKLOADS, block_mask_of, make_inputs

    w = WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    if args.mfma_ceiling:
        print(json.dumps({"mfma_ceiling": mfma_ceiling(dev, cus)}), flush=True)
        return 0
    if args.power:
        fa.load_library()
        print(json.dumps({"workload": w.name, "power": power_sample(dev, w)}), flush=True)
        return 0
    fa.load_library()
    bits = make_inputs(w, with_grad=True)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    g = {n: torch.from_numpy(b.view(np.int16)).view(tdt).to(dev) for n, b in bits.items()}
    if w.layout == "bshd":  # [B, L, H, D] buffers seen as [B, H, L, D]; outputs follow (empty_like)
        g = {n: t.transpose(1, 2).contiguous().transpose(1, 2) for n, t in g.items()}
    q, k, v, do = g["q"], g["k"], g["v"], g["do"]
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, w.Lq), dtype=torch.float32, device=dev)
    delta = torch.empty_like(lse)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    sc, causal = w.softmax_scale, w.causal
    stream = torch.cuda.current_stream()
    mask_np = block_mask_of(w)
    mask = None if mask_np is None else torch.from_numpy(mask_np).to(dev)

    general = w.dtype != "bf16" or w.layout != "bhld"  # fp16 or strided: the fa_*_ex calls
    short = w.Lq <= fa.SHORT_MAX_LQ                      # decode-style: the short-query calls
    ws = None
    if short:
        ws = torch.empty(fa.fa_short_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D), dtype=torch.uint8,
                         device=dev)

    # dK/dV through fa_bwd_ws where the library plans a load-balancing split
    # for this shape (never for the 8192-token headline shape); the workspace
    # is allocated before the timed steps and counted as resident
    ws_bytes = 0 if short else fa.fa_bwd_workspace_bytes(w.B, w.Hq, w.Hkv, w.Lq, w.Lk, w.D, mask is not None)
    dkv_ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None

    def step_short(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd_short(q, k, v, o, lse, scale=sc, causal=causal, workspace=ws, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd_delta_ex(o, do, delta, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        fa.fa_bwd_short(q, k, v, lse, delta, do, dq, None, None, scale=sc, causal=causal, grads="dq",
                        workspace=ws, stream=stream)
        if ev is not None:
            ev[3].record(stream)
        fa.fa_bwd_short(q, k, v, lse, delta, do, None, dk, dv, scale=sc, causal=causal, grads="dkv",
                        stream=stream)
        if ev is not None:
            ev[4].record(stream)

    def step_ex(ev=None):
        if ev is not None:
            ev[0].record(stream)
        fa.fa_fwd_ex(q, k, v, o, lse, scale=sc, causal=causal, block_mask=mask, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd_delta_ex(o, do, delta, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        fa.fa_bwd_ex(q, k, v, lse, delta, do, dq, None, None, scale=sc, causal=causal, block_mask=mask,
                     grads="dq", stream=stream)
        if ev is not None:
            ev[3].record(stream)
        fa.fa_bwd_ex(q, k, v, lse, delta, do, None, dk, dv, scale=sc, causal=causal, block_mask=mask,
                     grads="dkv", stream=stream, workspace=False if dkv_ws is None else dkv_ws)
        if ev is not None:
            ev[4].record(stream)

    def step(ev=None):
        if short:
            return step_short(ev)
        if general:
            return step_ex(ev)
        if ev is not None:
            ev[0].record(stream)
        if mask is None:
            fa.fa_fwd(q, k, v, o, lse, scale=sc, causal=causal, stream=stream)
        else:
            fa.fa_fwd_block_sparse(q, k, v, mask, o, lse, scale=sc, causal=causal, stream=stream)
        if ev is not None:
            ev[1].record(stream)
        fa.fa_bwd_delta(o, do, delta, stream=stream)
        if ev is not None:
            ev[2].record(stream)
        if mask is None:
            fa.fa_bwd_dq(q, k, v, lse, delta, do, dq, scale=sc, causal=causal, stream=stream)
        else:
            fa.fa_bwd_dq_block_sparse(q, k, v, lse, delta, do, mask, dq, scale=sc, causal=causal,
                                      stream=stream)
        if ev is not None:
            ev[3].record(stream)
        if dkv_ws is not None:
            fa.fa_bwd_ex(q, k, v, lse, delta, do, None, dk, dv, scale=sc, causal=causal, block_mask=mask,
                         grads="dkv", workspace=dkv_ws, stream=stream)
        elif mask is None:
            fa.fa_bwd_dkv(q, k, v, lse, delta, do, dk, dv, scale=sc, causal=causal, stream=stream)
        else:
            fa.fa_bwd_dkv_block_sparse(q, k, v, lse, delta, do, mask, dk, dv, scale=sc, causal=causal,
                                       stream=stream)
        if ev is not None:
            ev[4].record(stream)

    if args.profile_pass:
        # plain device copies of known sizes (they calibrate the byte
        # counters), then one step of the workload
        for mib in COPY_MIB:
            src = torch.empty(mib * 1024 * 1024, dtype=torch.uint8, device=dev).fill_(1)
            dst = torch.empty_like(src)
            torch.cuda.synchronize()
            dst.copy_(src)
            torch.cuda.synchronize()
            del src, dst
        step()
        torch.cuda.synchronize()
        print(json.dumps({"profile_pass": True, "copy_mib": COPY_MIB, "workload": w.name}))
        return 0

    resident = torch.cuda.memory_allocated()
    torch.cuda.synchronize()
    free_before = torch.cuda.mem_get_info(dev)[0]  # device-wide: sees allocations outside torch too
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    peak = torch.cuda.max_memory_allocated()
    free_after = torch.cuda.mem_get_info(dev)[0]

    names = ["fwd", "delta", "dq", "dkv"]
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    per_med = {n: float(np.median([e[j].elapsed_time(e[j + 1]) for e in evs])) for j, n in enumerate(names)}
    step_ev = np.array([e[0].elapsed_time(e[4]) for e in evs])  # first launch to last, per step
    ms_step = wall * 1e3 / args.steps
    if mask_np is None:
        pairs = visible_pairs(w.Lq, w.Lk, w.causal)
        total_flops, fwd_flops = model_flops(w.B, w.Hq, w.Lq, w.Lk, w.D, w.causal)
    else:
        pairs = visible_pairs_masked(w.Lq, w.Lk, w.causal, mask_np)
        total_flops, fwd_flops = masked_model_flops(w.B, w.Hq, w.D, pairs)
    value = total_flops / (ms_step * 1e-3) / 1e12

    work = kernel_work(w, pairs)
    kernels = {}
    for n in names:
        if n == "delta":
            kernels[n] = {"ms": per[n], "median_ms": per_med[n], "GB/s": work[n] / (per[n] * 1e-3) / 1e9}
        else:
            kernels[n] = {"ms": per[n], "median_ms": per_med[n], "TFLOP/s": work[n] / (per[n] * 1e-3) / 1e12}
    dom = max(("fwd", "dq", "dkv"), key=lambda n: per[n])
    achieved = work[dom] / (per[dom] * 1e-3) / 1e12
    roofline = {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": load_traffic(dom, w.name),
                "flop_per_launch": work[dom], "avg_launch_ms": round(per[dom], 4)}
    if short:  # a handful of query rows: every kernel is bound by HBM, not by the matrix cores
        sb = short_bytes(w)
        for n in names:
            kernels[n] = {"ms": per[n], "GB/s": sb[n] / (per[n] * 1e-3) / 1e9}
        gbs = sb[dom] / (per[dom] * 1e-3) / 1e9
        roofline = {"kernel": dom, "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": load_traffic(dom, w.name),
                    "bytes_per_launch": sb[dom], "avg_launch_ms": round(per[dom], 4)}

    kind = "causal" if w.causal else "dense"
    mask_desc = ""
    if w.mask is not None:
        recipe = (f"sliding window {w.mask[1]} keys" + (f" + {w.mask[2]} sink block(s)" if w.mask[2] else "")
                  if w.mask[0] == "window" else f"random density {w.mask[1]}")
        mask_desc = f", 64x64 block mask: {recipe}, {int(mask_np.sum())}/{mask_np.size} blocks kept"
    if w.layout == "bshd":
        mask_desc += ", every tensor a [B, L, H, D] buffer passed as a strided view"
    metric = METRIC if w.name == "train8k" else (
        f"fwd+bwd TFLOP/s{' over visible pairs' if mask_np is not None else ''}, {kind} GQA {w.dtype} "
        f"attention D={w.D} Lq={w.Lq} Lk={w.Lk}{mask_desc}; % of MFMA peak")
    unit = "TFLOP/s"
    if short:
        total_bytes = sum(short_bytes(w).values())
        value = total_bytes / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
        metric = (f"fwd+bwd algorithmic HBM GB/s (short-query path), {kind} GQA {w.dtype} attention "
                  f"D={w.D} Lq={w.Lq} Lk={w.Lk}; % of HBM peak")
    out = {
        "metric": metric,
        "value": round(value, 2),
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {kind} GQA fwd+bwd, B={w.B} Hq={w.Hq} Hkv={w.Hkv} "
                               f"Lq={w.Lq} Lk={w.Lk} D={w.D}{mask_desc}", "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   "Lq": w.Lq, "Lk": w.Lk, "D": w.D, "causal": w.causal,
                   "visible_pairs_per_head": int(pairs),
                   "dkv_workspace_bytes": int(ws_bytes)},
        "frac_of_peak": round(value / (PEAK_HBM_GBS if short else PEAK_BF16_TFLOPS), 4),
        "model_tflop_per_step": round(total_flops / 1e12, 4),
        "kernels": {n: {kk: round(vv, 4) for kk, vv in d.items()} for n, d in kernels.items()},
        "step_events_ms": {"median": round(float(np.median(step_ev)), 4), "min": round(float(step_ev.min()), 4),
                           "p90": round(float(np.percentile(step_ev, 90)), 4)},
        "roofline": roofline,
        "memory": {"resident_bytes": int(resident), "peak_bytes": int(peak),
                   "extra_over_resident": int(peak - resident),
                   "device_free_bytes_lost": int(free_before - free_after),
                   "unfused_fp32_score_bytes": unfused_score_bytes(w.B * w.Hq, w.Lq, 4)},
    }
    out["gemm_canary"] = gemm_canary(dev)
    ceil = mfma_ceiling(dev, cus)
    if ceil is not None:
        ceil["dominant_kernel_frac_of_random"] = round(achieved / ceil["random_operands"], 4)
        out["mfma_ceiling"] = ceil
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, bits, mask=mask_np, pairs=pairs)
    if w.name == "train8k" and not args.no_workloads:
        del q, k, v, do, o, lse, delta, dq, dk, dv, g
        torch.cuda.empty_cache()
        out["workloads"] = workload_sweep(dev)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
