#!/usr/bin/env python3
"""Benchmark of the top-k block-sparse GQA attention forward on one MI355X.

A step is one full forward call (msa_sparse_fwd, msa_sparse_fwd_varlen for the
ragged-batch workload, or msa_paged_sparse_fwd for the paged decode workload)
over one batch of seeded synthetic inputs already
resident in HBM: for the kv-centric path that includes the k2q CSR build, the
schedule, the per-block kernel and the combine. Prints one JSON line.

Metrics (the pages' benchmark harness, "test_sparse_atten.py"):
  prefill: effective TFLOP/s = 4 * B * Sq * Hq * (topk * 128) * D / time
           (every slot counted as a full 128-token block, -1 and masked included)
  decode:  GB/s of algorithmic bytes = distinct selected K/V blocks of each
           (sequence, KV head) * 64 KiB + Q + O + LSE + q2k + page table

Usage: python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload c3u|c2|vmix|...]
                       [--path auto|q|kv|decode] [--splits N] [--extra c5,c3u]
                       [--lse-temperature T] [--no-cpu-baseline]
(--extra workloads run with the automatic path)
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

MFMA_BF16_PEAK_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 FLOP/clk, dense
HBM_PEAK_GBS = 8000.0
PATHS = {"auto": 0, "q": 1, "kv": 2, "decode": 3, "tile": 4}
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "block_sparse_attention_top_amd", "csrc")
# the source files of each dominant kernel (besides the shared header)
KERNEL_SOURCES = {
    "qcentric_kernel": ("msa_qcentric.hip",),
    "kvcentric_kernel": ("msa_kvcentric.hip",),
    "paged_decode_kernel": ("msa_decode.hip", "msa_lds.hpp"),
    "dense_decode_kernel": ("msa_decode_dense.hip", "msa_lds.hpp"),
    "tile_kernel": ("msa_tile.hip", "msa_lds.hpp"),
}


def _code_only(text: str) -> str:
    """C++ source without comments and with whitespace collapsed: what the compiler
    sees, so that an edit of a comment does not count as a change of the kernel."""
    import re
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":  # string or character literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        else:
            out.append(c)
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_digest(kernel: str) -> str:
    """Hash of the code (comments and layout stripped) of a kernel's sources and the
    shared header: a counter summary is reused only while the kernel it measured is
    unchanged."""
    import hashlib
    srcs = next(f for k, f in KERNEL_SOURCES.items() if kernel.startswith(k))
    h = hashlib.sha256()
    for f in srcs + ("msa_internal.hpp",):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


class HipEvents:
    """Pairs of hipEvent_t created through the HIP runtime (ctypes), for the
    library's profiling hook: the library records them around its dominant
    kernel on the launch stream."""

    def __init__(self, n: int):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.pairs = []
        for _ in range(n):
            a, b = ctypes.c_void_p(), ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(a)) == 0
            assert self.hip.hipEventCreate(ctypes.byref(b)) == 0
            self.pairs.append((a.value, b.value))

    def mean_ms(self) -> float:
        tot = 0.0
        for a, b in self.pairs:
            ms = self.ct.c_float()
            assert self.hip.hipEventElapsedTime(self.ct.byref(ms), a, b) == 0
            tot += ms.value
        return tot / len(self.pairs)

    def close(self) -> None:
        for a, b in self.pairs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dense_decode_algorithmic_bytes(w, inp) -> int:
    """Every page of each sequence's keys (ceil(seqused / 128)) x KV heads x 128 tokens x D x
    element size x 2 (K and V), plus Q, O, LSE, page table and seqused."""
    pages = int(((inp["seqused_k"].astype(np.int64) + 127) // 128).sum())
    kv = pages * w.Hkv * 128 * w.D * inp["k_pool"].itemsize * 2
    q = w.B * w.Sq * w.Hq * w.D  # elements of Q read (bf16 or fp8) and of O written (bf16)
    return int(kv + q * inp["q"].itemsize + q * 2 + w.B * w.Sq * w.Hq * 4 +
               inp["page_table"].nbytes + inp["seqused_k"].nbytes)


def decode_algorithmic_bytes(w, inp) -> int:
    """Distinct valid selected blocks per (b, hkv) x 128 tokens x D x element size x 2
    (K and V; 2 B for bf16, 1 B for the fp8 cache), plus Q, O, LSE, q2k, page table and
    seqused."""
    q2k = inp["q2k"]
    blocks = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            ids = q2k[b, h].reshape(-1)
            ids = ids[(ids >= 0) & (ids < w.max_pages)]
            blocks += np.unique(ids).size
    kv = blocks * 128 * w.D * inp["k_pool"].itemsize * 2
    q = w.B * w.Sq * w.Hq * w.D * 2
    return int(kv + 2 * q + w.B * w.Sq * w.Hq * 4 + q2k.nbytes + inp["page_table"].nbytes +
               inp["seqused_k"].nbytes)


class Case:
    """One workload uploaded to the GPU with a callable that runs one step."""

    def __init__(self, key: str, path: str, splits: int = 0, temperature=None,
                 kv_dtype: str = "bf16"):
        import torch
        import block_sparse_attention_top_amd as msa
        import workloads as wl
        self.varlen = key in wl.VARLEN_WORKLOADS
        self.key = key
        self.temperature = temperature
        # the temperature-scaled LSE as an extra output (computed by the kernels)
        tk = ({} if temperature is None else
              {"return_temperature_lse": True, "lse_temperature_scale": float(temperature),
               "temperature_fast_path": False})
        self.w = wl.VARLEN_WORKLOADS[key] if self.varlen else wl.WORKLOADS[key]
        w = self.w
        t0 = time.time()
        self.inp = wl.make_varlen_workload_inputs(w) if self.varlen else wl.make_inputs(w)
        self.kv_dtype = kv_dtype
        if kv_dtype == "fp8":  # the fp8 e4m3fn K/V cache (bytes, read as fp8 by the library)
            self.inp = wl.with_fp8_kv(self.inp)
            if w.paged and w.dense:  # the pages' fp8 decode: Q fp8 as well
                self.inp["q"] = wl.bf16_bits_to_fp8(self.inp["q"])
        # the fp8 dense decode multiplies on the fp8 matrix cores; every other fp8 path
        # widens the cache to bf16 first
        self.compute_fp8 = kv_dtype == "fp8" and w.paged and w.dense
        log(f"[bench] {key}: inputs generated in {time.time() - t0:.1f}s")
        dev = lambda x: (torch.from_numpy(x).view(torch.bfloat16) if x.dtype == np.uint16
                         else torch.from_numpy(x)).to("cuda")
        self.t = {k: dev(v) for k, v in self.inp.items()}
        t = self.t
        if self.varlen:
            self.o = torch.empty((w.total_q, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
            self.lse = torch.empty((w.total_q, w.Hq), dtype=torch.float32, device="cuda")
            p = msa.msa_sparse_fwd_varlen_path(w.B, w.total_q, w.total_k, w.Hq, w.Hkv, w.topk,
                                               PATHS[path])
            if p not in (1, 2):
                raise SystemExit(f"path {path} does not apply to the varlen workload {key}")
            nb = msa.msa_sparse_fwd_varlen_workspace_size(w.B, w.total_q, w.total_k, w.Hq, w.Hkv,
                                                          w.D, w.topk, w.blk, p)
            ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            self.path_name = {1: "q-centric", 2: "kv-centric"}[p]
            self.splits = 1
            self.step = lambda: msa.msa_sparse_fwd_varlen(
                t["q"], t["k"], t["v"], t["q2k"], t["cu_seqlens_q"], t["cu_seqlens_k"],
                causal=w.causal, path=p, o=self.o, lse=self.lse, workspace=ws, **tk)
            self.bytes = None
            self.flops = w.effective_flops()
            return
        self.o = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
        self.lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
        if w.paged and w.dense:
            # plan once (schedule on the device), then each step is one run
            plan = msa.msa_paged_decode_plan(t["page_table"], t["seqused_k"], seqlen_q=w.Sq,
                                             max_seqlen_k=w.Skv, num_qo_heads=w.Hq,
                                             num_kv_heads=w.Hkv)
            self.plan = plan
            self.path_name = "paged-dense-decode"
            self.splits = plan.info.kv_chunk_size_pages  # pages per chunk
            self.step = lambda: msa.msa_paged_decode_run(
                plan, t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"],
                causal=w.causal, o=self.o, lse=self.lse, **tk)
            self.bytes = dense_decode_algorithmic_bytes(w, self.inp)
        elif w.paged:
            p = msa.msa_paged_sparse_fwd_path(w.B, w.Sq, w.Hkv, w.topk, w.max_pages, PATHS[path])
            if p not in (1, 2, 3):
                raise SystemExit(f"path {path} does not apply to the paged workload {key}")
            nb = msa.msa_paged_sparse_fwd_workspace_size(w.B, w.Sq, w.Hq, w.Hkv, w.D, w.topk,
                                                        w.blk, w.max_pages, splits, p)
            ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            self.path_name = {1: "paged-qcentric", 2: "paged-kv-centric", 3: "paged-decode"}[p]
            self.splits = msa.msa_paged_sparse_fwd_splits(w.B, w.Sq, w.Hkv, w.topk, w.max_pages,
                                                          splits, p)
            self.step = lambda: msa.msa_paged_sparse_fwd(
                t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"], t["q2k"],
                causal=w.causal, num_splits=splits, path=p, o=self.o, lse=self.lse,
                workspace=ws, **tk)
            self.bytes = decode_algorithmic_bytes(w, self.inp) if w.decode else None
        else:
            p = msa.msa_sparse_fwd_path(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.topk, PATHS[path])
            nb = msa.msa_sparse_fwd_workspace_size(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D, w.topk,
                                                   w.blk, p)
            self.path_name = {1: "q-centric", 2: "kv-centric", 4: "query-tile"}[p]
            self.splits = 1
            ws = torch.empty(max(nb, 256), dtype=torch.uint8, device="cuda")
            self.step = lambda: msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"],
                                                   causal=w.causal, path=p, o=self.o,
                                                   lse=self.lse, workspace=ws, **tk)
            self.bytes = None
        self.flops = w.effective_flops()

    def time_steps(self, steps: int, warmup: int) -> tuple:
        """(mean ms per step, mean ms of the dominant kernel) over `steps` back-to-back
        calls each. The step time comes from a plain loop bracketed by events on torch's
        current stream (the launch stream), with nothing else recorded inside it. The
        kernel time comes from a second loop of the same length in which the library
        records a pair of events around its dominant kernel, on the launch stream."""
        import torch
        import block_sparse_attention_top_amd as msa
        for _ in range(warmup):
            self.step()
        torch.cuda.synchronize()
        start = torch.cuda.Event(enable_timing=True)
        end = torch.cuda.Event(enable_timing=True)
        start.record()
        for _ in range(steps):
            self.step()
        end.record()
        end.synchronize()
        step_ms = start.elapsed_time(end) / steps
        ev = HipEvents(steps)
        for i in range(steps):
            msa.msa_set_profiling_events(*ev.pairs[i])
            self.step()
        msa.msa_set_profiling_events(None, None)
        torch.cuda.synchronize()
        kernel_ms = ev.mean_ms()
        ev.close()
        return step_ms, kernel_ms

    def breakdown(self, steps: int, warmup: int):
        """kv-centric only: mean ms of the k2q CSR build alone, of the forward given a
        prebuilt CSR, and of the two together (the timed step)."""
        if self.w.paged or self.path_name != "kv-centric" or self.temperature is not None:
            return None
        import torch
        import block_sparse_attention_top_amd as msa
        w, t = self.w, self.t
        if self.varlen:
            rows = int(sum((k + w.blk - 1) // w.blk for k in w.k_lens))
            cuq, cuk = t["cu_seqlens_q"], t["cu_seqlens_k"]
            csr = msa.msa_build_k2q_csr_varlen(t["q2k"], cuq, cuk, w.total_k, rows)
            build = lambda: msa.msa_build_k2q_csr_varlen(t["q2k"], cuq, cuk, w.total_k, rows,
                                                         row_ptr=csr[0], q_idx=csr[1],
                                                         slot=csr[2])
            fwd = lambda: msa.msa_sparse_fwd_varlen(t["q"], t["k"], t["v"], t["q2k"], cuq, cuk,
                                                    *csr, rows, causal=w.causal, path=2,
                                                    o=self.o, lse=self.lse)
        else:
            nblk = w.Skv // w.blk
            csr = msa.msa_build_k2q_csr(t["q2k"], nblk)
            build = lambda: msa.msa_build_k2q_csr(t["q2k"], nblk, row_ptr=csr[0], q_idx=csr[1],
                                                  slot=csr[2])
            fwd = lambda: msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], *csr,
                                             causal=w.causal, path=2, o=self.o, lse=self.lse)

        def timed(fn, n):
            for _ in range(warmup):
                fn()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(n):
                fn()
            b.record()
            b.synchronize()
            return a.elapsed_time(b) / n

        # The three loops alternate over several rounds and each reports its median: a
        # fixed order (build, then forward, then step) let the clock's drift under
        # sustained load favour whichever loop ran later.
        rounds, n = 3, max(3, steps // 2)
        res = {"csr": [], "fwd": [], "both": []}
        for _ in range(rounds):
            res["csr"].append(timed(build, n))
            res["fwd"].append(timed(fwd, n))
            res["both"].append(timed(self.step, n))
        med = {k: float(np.median(v)) for k, v in res.items()}
        # the CSR build's algorithmic bytes: the index table read, row_ptr written, and
        # q_idx and slot written for every valid entry
        nnz = int(csr[0][:, -1].sum().item())
        csr_bytes = t["q2k"].numel() * 4 + csr[0].numel() * 4 + 2 * nnz * 4
        return {"csr_ms": med["csr"], "fwd_ms": med["fwd"], "csr_plus_fwd_ms": med["both"],
                "fwd_TFLOP_per_s": self.flops / (med["fwd"] * 1e-3) / 1e12,
                "csr_bytes": csr_bytes, "csr_GB_per_s": csr_bytes / (med["csr"] * 1e-3) / 1e9}

    def metric(self, ms: float, kernel_ms: float) -> dict:
        if self.w.decode:
            gbs = self.bytes / (ms * 1e-3) / 1e9
            return {"ms": ms, "GB_per_s": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
                    "kernel_ms": kernel_ms,
                    "kernel_GB_per_s": self.bytes / (kernel_ms * 1e-3) / 1e9,
                    "algorithmic_bytes": self.bytes, "path": self.path_name,
                    "splits": self.splits}
        tf = self.flops / (ms * 1e-3) / 1e12
        return {"ms": ms, "TFLOP_per_s": tf, "mfma_frac": tf / MFMA_BF16_PEAK_TFLOPS,
                "kernel_ms": kernel_ms,
                "kernel_TFLOP_per_s": self.flops / (kernel_ms * 1e-3) / 1e12,
                "effective_flop": self.flops, "path": self.path_name}

    def dominant_kernel(self, temp: bool = False, fp8: bool = False) -> str:
        """Name of the dominant kernel instance (template arguments as the profiler
        prints them; the q-centric kernel runs two waves per row when the rows are
        fewer than 8 per compute unit)."""
        import torch
        t, f = ("true" if temp else "false"), ("true" if fp8 else "false")
        w = self.w
        if self.path_name in ("paged-qcentric", "q-centric"):
            rows = w.total_q if self.varlen else w.B * w.Sq
            items = rows * w.Hkv * self.splits
            cus = torch.cuda.get_device_properties(0).multi_processor_count
            waves = 2 if items < 8 * cus else 1
            paged = "true" if w.paged else "false"
            # paged blocks read about once (fewer than 2 (query, slot) entries per block)
            # take the non-temporal instance
            nblk = w.max_pages if w.paged else w.Skv // w.blk
            nt = not self.varlen and w.Sq * min(w.topk, nblk) < 2 * nblk
            return f"qcentric_kernel<{paged}, {t}, {f}, {waves}, false, {'true' if nt else 'false'}>"
        if self.path_name in ("kv-centric", "paged-kv-centric"):
            paged = "true" if w.paged else "false"
            return f"kvcentric_kernel<{w.qpk}, {t}, {f}, {paged}>"
        if w.paged:
            return decode_instance(w, fp8).replace("TEMP", t)
        return {"query-tile": f"tile_kernel<{w.qpk}, {t}>"}[self.path_name]


def decode_instance(w, fp8: bool = False) -> str:
    """The paged decode kernel instance the launcher picks (TEMP stands for the
    temperature template argument): the dense decode with at most 128 (query, head)
    columns per KV head runs the 32-column kernel (bf16 or the fp8 decode); otherwise
    the union kernel groups queries four to a wave."""
    if w.dense and w.Sq * w.qpk <= 128:
        return f"dense_decode_kernel<TEMP, {'true' if fp8 else 'false'}>"
    return (f"paged_decode_kernel<{(w.Sq + 3) // 4}, TEMP, "
            f"{'true' if w.dense else 'false'}>")


def skew_diagnostics(w, q2k: np.ndarray, varlen_rows=None) -> dict:
    """How the index table spreads over the KV blocks, in the manner of the test page's
    benchmark printout (its q2k fan-out and k2q CSR row summaries): per KV head and
    block, the number of (query, slot) entries that select it (the CSR row lengths),
    the share of block 0 (the sink), and the spread (max / mean, p50) of those counts;
    per query row, the number of valid slots."""
    if varlen_rows is not None:  # packed [Hkv, total_q, topk] with per-query block counts
        hkv_n, nq, topk = q2k.shape
        nb = np.repeat(varlen_rows["nblk"], varlen_rows["q_lens"])[None, :, None]
        base = np.repeat(varlen_rows["rowbase"], varlen_rows["q_lens"])[None, :, None]
        ok = (q2k >= 0) & (q2k < nb)
        rows = (q2k + base)[ok] + np.nonzero(ok)[0] * varlen_rows["nrows"]
        nrows = varlen_rows["nrows"]
        per_row = ok.sum(axis=2).reshape(-1)
        block0 = int(((q2k == 0) & ok).sum())
    else:
        nblk = w.max_pages if w.paged else w.Skv // w.blk
        nrows = w.B * nblk
        ok = (q2k >= 0) & (q2k < nblk)
        b = np.arange(w.B).reshape(-1, 1, 1, 1)
        h = np.arange(w.Hkv).reshape(1, -1, 1, 1)
        rows = (h * nrows + b * nblk + q2k)[ok]
        per_row = ok.sum(axis=3).reshape(-1)
        block0 = int(((q2k == 0) & ok).sum())
    hkv_n = w.Hkv
    counts = np.bincount(rows.reshape(-1), minlength=hkv_n * nrows).astype(np.float64)
    valid = int(counts.sum())
    mean = counts.mean() if counts.size else 0.0
    return {
        "valid_entries": valid,
        "csr_rows": int(counts.size),
        "row_len_max": int(counts.max()) if counts.size else 0,
        "row_len_mean": round(float(mean), 1),
        "row_len_p50": float(np.median(counts)) if counts.size else 0.0,
        "row_len_max_over_mean": round(float(counts.max() / mean), 2) if mean else None,
        "block0_share": round(block0 / valid, 4) if valid else None,
        "empty_rows": int((counts == 0).sum()),
        "fanout_min": int(per_row.min()), "fanout_mean": round(float(per_row.mean()), 2),
        "queries_with_no_slot": int((per_row == 0).sum()),
    }


def measured_traffic(case: "Case"):
    """HBM bytes per launch of the dominant kernel from the committed counter summary
    profiles/traffic_<workload>_<path>.json (FETCH_SIZE and WRITE_SIZE, scaled by a
    plain copy of known size), if it was taken on the current kernel sources."""
    fp8 = case.kv_dtype == "fp8"
    f = os.path.join(PROFILES, f"traffic_{case.key}_{case.path_name}{'-fp8' if fp8 else ''}.json")
    if not os.path.exists(f):
        return None
    with open(f) as fh:
        d = json.load(fh)
    if d.get("source_digest") != source_digest(case.dominant_kernel(False, fp8)):
        return None
    return d.get("hbm_bytes_per_launch")


def copy_calibration(mib: int, reps: int = 3) -> None:
    """A plain device copy of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "reps": reps}), flush=True)


def cpu_baseline(case: Case, budget_s: float = 12.0) -> dict:
    """The oracle (unchanged) on a bounded sample of the same workload's rows."""
    import oracle
    w, inp = case.w, case.inp
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    rng = np.random.default_rng(0)
    total_rows = w.total_q if case.varlen else w.B * w.Sq

    def run(n):
        rows = np.sort(rng.choice(total_rows, size=min(n, total_rows), replace=False))
        t0 = time.perf_counter()
        if case.varlen:
            oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                           inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                           causal=w.causal, rows=rows, nthreads=threads)
        elif w.paged and w.dense and case.kv_dtype == "fp8":  # the pages' fp8 decode
            oracle.paged_decode_fp8(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                    inp["seqused_k"], causal=w.causal, rows=rows,
                                    nthreads=threads)
        elif w.paged and w.dense:  # every block selected
            full = np.ascontiguousarray(np.broadcast_to(
                np.arange(w.max_pages, dtype=np.int32), (w.B, w.Hkv, w.Sq, w.max_pages)))
            oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                          inp["page_table"], inp["seqused_k"], full,
                                          causal=w.causal, rows=rows, nthreads=threads)
        elif w.paged:
            oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                          inp["page_table"], inp["seqused_k"], inp["q2k"],
                                          causal=w.causal, rows=rows, nthreads=threads)
        else:
            oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"], causal=w.causal,
                                    rows=rows, nthreads=threads)
        return rows.size, time.perf_counter() - t0

    # grow the probe until it takes a quarter of the budget (small probes overstate
    # the per-row cost: thread start-up), then size the timed sample from it
    n, dt = run(max(threads, 16))
    while dt < budget_s / 4 and n < total_rows:
        n, dt = run(min(total_rows, n * 4))
    n_target = int(min(total_rows, max(n, n * budget_s / max(dt, 1e-9))))
    if n_target > n:
        n, dt = run(n_target)
    frac = n / total_rows
    if w.decode:
        value = case.bytes * frac / dt / 1e9
        unit = "GB/s"
    else:
        value = w.effective_flops() * frac / dt / 1e12
        unit = "TFLOP/s"
    return {"value": value, "unit": unit, "cores": threads, "kind": "oracle",
            "sample": f"{n} of {total_rows} query rows (all heads) of {w.name}, "
                      f"{dt:.1f} s, fp64 C oracle with OpenMP"}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c3u",
                    help="the workload timed for the headline value (default: B1, Sq=Skv=32768, "
                         "Hq 64 / Hkv 4, topk 16, uniform selections)")
    ap.add_argument("--path", default="auto", choices=sorted(PATHS))
    ap.add_argument("--splits", type=int, default=0,
                    help="KV splits of the paged workload (0 = the library's choice)")
    ap.add_argument("--extra", default="c5,c3p",
                    help="comma-separated workloads reported beside (default: the paged decode "
                         "batch c5 and the paged prefill c3p; '' for none)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="K/V element type (fp8 = the e4m3fn cache)")
    ap.add_argument("--lse-temperature", type=float, default=None, metavar="T",
                    help="also compute the temperature-scaled LSE with this T")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the sparse forward runs on one GPU; sharding is described, not built)", file=sys.stderr)
        return 2

    import torch
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return 0
    case = Case(args.workload, args.path, args.splits, args.lse_temperature, args.kv_dtype)
    skew = None
    w_ = case.w
    if "q2k" in case.inp and not getattr(w_, "dense", False):
        vr = None
        if case.varlen:
            nblk = (np.asarray(w_.k_lens) + w_.blk - 1) // w_.blk
            vr = {"nblk": nblk, "q_lens": np.asarray(w_.q_lens),
                  "rowbase": np.concatenate([[0], np.cumsum(nblk)[:-1]]), "nrows": int(nblk.sum())}
        skew = skew_diagnostics(w_, case.inp["q2k"], vr)
        log(f"[bench] {args.workload}: index skew {skew}")
    log(f"[bench] {args.workload}: timing {args.steps} steps after {args.warmup} warmup "
        f"({case.path_name})")
    ms, kernel_ms = case.time_steps(args.steps, args.warmup)
    m = case.metric(ms, kernel_ms)
    log(f"[bench] {args.workload}: {m}")
    w = case.w
    traffic = measured_traffic(case) if args.lse_temperature is None else None
    if w.decode:
        value, unit = m["GB_per_s"], "GB/s"
        metric = "paged dense decode GB/s" if w.dense else "paged sparse decode GB/s"
        ach = m["kernel_GB_per_s"]
        roof = {"bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": ach / HBM_PEAK_GBS, "traffic": traffic}
    else:
        value, unit = m["TFLOP_per_s"], "TFLOP/s"
        metric = "sparse-attn fwd effective TFLOP/s"
        ach = m["kernel_TFLOP_per_s"]
        roof = {"bound": "mfma", "achieved": ach, "peak": MFMA_BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS, "traffic": traffic}
    # the whole step (every launch of the call) against the same peak, beside the
    # dominant kernel's own fraction
    roof["step_frac"] = (m["hbm_frac"] if w.decode else m["mfma_frac"])
    roof["kernel"] = case.dominant_kernel()
    if args.lse_temperature is not None or args.kv_dtype == "fp8":  # the kernels' variants
        roof["kernel"] = case.dominant_kernel(args.lse_temperature is not None,
                                              args.kv_dtype == "fp8")
    roof["kernel_ms"] = kernel_ms
    brk = case.breakdown(args.steps, args.warmup)
    if brk is not None:
        log(f"[bench] {args.workload}: breakdown {brk}")
    extra = {}
    for key in [k for k in args.extra.split(",") if k]:
        c = Case(key, "auto")
        extra[key] = c.metric(*c.time_steps(args.steps, args.warmup))
        extra[key]["workload"] = c.w.name
        extra[key]["kernel"] = c.dominant_kernel()
        log(f"[bench] {key}: {extra[key]}")
        del c
        torch.cuda.empty_cache()
    cpu = None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle on a row sample)")
        cpu = cpu_baseline(case)
        log(f"[bench] cpu baseline: {cpu}")
    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "fp8" if case.compute_fp8 else "bf16", "data": "synthetic",
        "config": ({"workload": w.name, "B": w.B, "Sq": w.Sq, "Skv": w.Skv, "Hq": w.Hq,
                    "Hkv": w.Hkv, "D": w.D, "topk": w.topk, "blk_kv": w.blk,
                    "causal": w.causal, "path": case.path_name, "splits": case.splits,
                    "lse_temperature": args.lse_temperature, "kv_dtype": args.kv_dtype,
                    "q_dtype": str(case.inp["q"].dtype).replace("uint8", "fp8").replace(
                        "uint16", "bf16"),
                    "parallelism": "none"} if not case.varlen else
                   {"workload": w.name, "B": w.B, "varlen": True, "total_q": w.total_q,
                    "total_k": w.total_k, "q_lens": list(w.q_lens), "k_lens": list(w.k_lens),
                    "Hq": w.Hq, "Hkv": w.Hkv, "D": w.D, "topk": w.topk, "blk_kv": w.blk,
                    "causal": w.causal, "path": case.path_name, "splits": 1,
                    "lse_temperature": args.lse_temperature, "kv_dtype": args.kv_dtype,
                    "parallelism": "none"}),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    if brk is not None:
        line["breakdown"] = brk
    if skew is not None:
        line["index_skew"] = skew
    if extra:
        line["extra"] = extra
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
