"""Seeded synthetic workloads for top-k block-sparse GQA attention.

The shapes follow the workloads of the MSA sparse-attention test and benchmark
harness (page "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py":
the generator ``generate_test_data``, the paged packer ``pack_paged_kv`` and
the benchmark cases ``ring48k`` / ``ulysses384k``). Random numbers come from
the counter-based C generator in ``gen.c``; nothing here computes attention.

Everything returns host numpy arrays: bf16 tensors as ``uint16`` bit
patterns, index tables as ``int32``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libmsa_workloads.so")

# sub-stream ids of one seed
STREAM_Q, STREAM_K, STREAM_V, STREAM_IDX, STREAM_PAGES = 1, 2, 3, 4, 5
MODE_PERM, MODE_SINK, MODE_CAUSAL = 0, 1, 2
DEFAULT_SEED = 42

_lib = None


def build(force: bool = False) -> str:
    """Compile gen.c into libmsa_workloads.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB)
        lib.wl_normal_bf16.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_int64, ctypes.c_void_p]
        lib.wl_normal_bf16.restype = None
        lib.wl_q2k.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int,
                               ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_int,
                               ctypes.c_int, ctypes.c_void_p]
        lib.wl_q2k.restype = ctypes.c_int
        lib.wl_permutation.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64,
                                       ctypes.c_void_p]
        lib.wl_permutation.restype = None
        lib.wl_draw64.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.wl_draw64.restype = ctypes.c_uint64
        lib.wl_stream_key.argtypes = [ctypes.c_uint64, ctypes.c_uint64]
        lib.wl_stream_key.restype = ctypes.c_uint64
        _lib = lib
    return _lib


def normal_bf16(seed: int, stream: int, shape, first: int = 0) -> np.ndarray:
    """N(0,1) values rounded to bf16 (uint16 bit patterns), elements first.. of a stream."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    _load().wl_normal_bf16(seed, stream, first, n, out.ctypes.data)
    return out.reshape(shape)


def q2k_table(seed: int, mode: int, B: int, Hkv: int, Sq: int, kvlen, blk: int, topk: int,
              stream: int = STREAM_IDX) -> np.ndarray:
    """Index table [B, Hkv, Sq, topk] int32 under one of the recipes of gen.c."""
    kv = np.ascontiguousarray(np.broadcast_to(np.asarray(kvlen, dtype=np.int32), (B,)))
    out = np.empty((B, Hkv, Sq, topk), dtype=np.int32)
    rc = _load().wl_q2k(seed, stream, mode, B, Hkv, Sq, kv.ctypes.data, blk, topk, out.ctypes.data)
    if rc != 0:
        raise ValueError("bad q2k generator arguments")
    return out


def permutation(seed: int, stream: int, n: int) -> np.ndarray:
    out = np.empty(n, dtype=np.int32)
    _load().wl_permutation(seed, stream, n, out.ctypes.data)
    return out


def bf16_to_f32(x: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (x.astype(np.uint32) << 16).view(np.float32)


@dataclass
class Workload:
    """One synthetic workload (shapes, masking, index recipe)."""
    name: str
    B: int
    Sq: int
    Skv: int
    Hkv: int
    qpk: int
    topk: int
    causal: bool
    mode: int
    D: int = 128
    blk: int = 128
    paged: bool = False
    seqused_trim: int = 0          # paged: seqused_k = Skv - trim
    shuffle_pages: bool = True
    dense: bool = False            # paged: every key of the sequence (no index table)
    prefill: bool = False          # paged: a prefill (TFLOP/s), not a decode batch (GB/s)
    seed: int = DEFAULT_SEED
    note: str = ""

    @property
    def Hq(self) -> int:
        return self.Hkv * self.qpk

    @property
    def max_pages(self) -> int:
        return (self.Skv + self.blk - 1) // self.blk

    @property
    def decode(self) -> bool:
        """A paged decode batch, measured in GB/s (every other workload in TFLOP/s)."""
        return self.paged and not self.prefill

    @property
    def kvlen(self) -> int:
        return self.Skv - self.seqused_trim if self.paged else self.Skv

    def effective_flops(self) -> int:
        """4 * B * Sq * Hq * (topk * blk) * D: every slot counted as a full block."""
        return 4 * self.B * self.Sq * self.Hq * self.topk * self.blk * self.D

    def scaled(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


WORKLOADS = {
    "c1": Workload("c1_b1_s1k_hq2_hkv1_top4_noncausal", B=1, Sq=1024, Skv=1024, Hkv=1, qpk=2,
                   topk=4, causal=False, mode=MODE_PERM),
    "c2": Workload("c2_b1_s8k_hq64_hkv4_top16_causal", B=1, Sq=8192, Skv=8192, Hkv=4, qpk=16,
                   topk=16, causal=True, mode=MODE_CAUSAL),
    "c3u": Workload("c3_b1_s32k_hq64_hkv4_top16_uniform", B=1, Sq=32768, Skv=32768, Hkv=4,
                    qpk=16, topk=16, causal=False, mode=MODE_PERM),
    "c3s": Workload("c3_b1_s32k_hq64_hkv4_top16_sink", B=1, Sq=32768, Skv=32768, Hkv=4, qpk=16,
                    topk=16, causal=False, mode=MODE_SINK),
    "c4a": Workload("c4a_b1_s48k_hq16_hkv1_top16_causal", B=1, Sq=49152, Skv=49152, Hkv=1,
                    qpk=16, topk=16, causal=True, mode=MODE_CAUSAL),
    "c4b": Workload("c4b_b1_s384k_hq2_hkv1_top16_causal", B=1, Sq=393216, Skv=393216, Hkv=1,
                    qpk=2, topk=16, causal=True, mode=MODE_CAUSAL),
    "c5": Workload("c5_paged_decode_b32_sq8_hq64_hkv4_kv64k_top16", B=32, Sq=8, Skv=65536,
                   Hkv=4, qpk=16, topk=16, causal=True, mode=MODE_CAUSAL, paged=True,
                   seqused_trim=17),
    # the test page's paged prefill benchmark: its default shape, causal, through a
    # shuffled page table of 128-token pages, seqused trimmed by 17
    "c3p": Workload("c3p_paged_prefill_b1_s32k_hq64_hkv4_top16_causal", B=1, Sq=32768,
                    Skv=32768, Hkv=4, qpk=16, topk=16, causal=True, mode=MODE_CAUSAL,
                    paged=True, seqused_trim=17, prefill=True),
    # the same decode batch attending to every key (the dense decode path)
    "c5d": Workload("c5d_paged_dense_decode_b32_sq8_hq64_hkv4_kv64k", B=32, Sq=8, Skv=65536,
                    Hkv=4, qpk=16, topk=16, causal=True, mode=MODE_CAUSAL, paged=True,
                    seqused_trim=17, dense=True),
}


def make_inputs(w: Workload, q2k: Optional[np.ndarray] = None) -> dict:
    """Host inputs for a workload: q, k, v (or k_pool, v_pool, page_table, seqused_k), q2k."""
    out = {}
    out["q"] = normal_bf16(w.seed, STREAM_Q, (w.B, w.Sq, w.Hq, w.D))
    if w.paged:
        num_pages = w.B * w.max_pages
        shape = (num_pages, w.Hkv, w.blk, w.D)
        out["k_pool"] = normal_bf16(w.seed, STREAM_K, shape)
        out["v_pool"] = normal_bf16(w.seed, STREAM_V, shape)
        if w.shuffle_pages:
            pt = permutation(w.seed, STREAM_PAGES, num_pages)
        else:
            pt = np.arange(num_pages, dtype=np.int32)
        out["page_table"] = pt.reshape(w.B, w.max_pages).copy()
        out["seqused_k"] = np.full((w.B,), w.kvlen, dtype=np.int32)
    else:
        out["k"] = normal_bf16(w.seed, STREAM_K, (w.B, w.Skv, w.Hkv, w.D))
        out["v"] = normal_bf16(w.seed, STREAM_V, (w.B, w.Skv, w.Hkv, w.D))
    if q2k is None:
        q2k = q2k_table(w.seed, w.mode, w.B, w.Hkv, w.Sq, w.kvlen, w.blk, w.topk)
    out["q2k"] = q2k
    return out


# ---------------------------------------------------------------------------
# Variable-length batches (the packed form: q [total_q,Hq,D], k/v [total_k,Hkv,D],
# q2k [Hkv,total_q,topk], cu_seqlens [B+1])
# ---------------------------------------------------------------------------
def varlen_lengths(seed: int, B: int, max_q: int, max_k: int, blk: int = 128,
                   k_multiple: bool = True):
    """Ragged lengths in the manner of the test page's samplers: q lengths uniform in
    [1, max_q] and K lengths uniform in [1, max_k] (whole blocks when k_multiple),
    the first sequence at the maximum of each. Uses numpy's PCG64 seeded generator."""
    rng = np.random.default_rng(seed)
    q_lens = rng.integers(1, max_q + 1, size=B)
    q_lens[0] = max_q
    if k_multiple:
        k_lens = rng.integers(1, max_k // blk + 1, size=B) * blk
    else:
        k_lens = rng.integers(1, max_k + 1, size=B)
    k_lens[0] = max_k
    return [int(x) for x in q_lens], [int(x) for x in k_lens]


def cu_seqlens(lengths) -> np.ndarray:
    return np.concatenate([[0], np.cumsum(np.asarray(lengths, dtype=np.int64))]).astype(np.int32)


def make_varlen_inputs(seed: int, q_lens, k_lens, Hkv: int, qpk: int, topk: int, mode: int,
                       D: int = 128, blk: int = 128) -> dict:
    """Host inputs of a variable-length batch; sequence b's index rows come from the
    same recipes as the batched workloads (seed + 1000 + b), block ids local to b."""
    q_lens, k_lens = list(q_lens), list(k_lens)
    total_q, total_k = sum(q_lens), sum(k_lens)
    Hq = Hkv * qpk
    out = {"q": normal_bf16(seed, STREAM_Q, (total_q, Hq, D)),
           "k": normal_bf16(seed, STREAM_K, (total_k, Hkv, D)),
           "v": normal_bf16(seed, STREAM_V, (total_k, Hkv, D)),
           "cu_seqlens_q": cu_seqlens(q_lens), "cu_seqlens_k": cu_seqlens(k_lens)}
    q2k = np.full((Hkv, total_q, topk), -1, dtype=np.int32)
    g = 0
    for b, (sq, sk) in enumerate(zip(q_lens, k_lens)):
        if sq > 0 and sk > 0:
            q2k[:, g:g + sq] = q2k_table(seed + 1000 + b, mode, 1, Hkv, sq, sk, blk, topk)[0]
        g += sq
    out["q2k"] = q2k
    return out



@dataclass
class VarlenWorkload:
    """A variable-length batch: per-sequence query and key lengths, shared heads and
    index recipe (each sequence's index rows as in the uniform workloads)."""
    name: str
    q_lens: tuple
    k_lens: tuple
    Hkv: int
    qpk: int
    topk: int
    causal: bool
    mode: int
    D: int = 128
    blk: int = 128
    seed: int = DEFAULT_SEED
    paged = False  # contiguous K/V only (class attributes, not fields)
    decode = False

    @property
    def Hq(self) -> int:
        return self.Hkv * self.qpk

    @property
    def B(self) -> int:
        return len(self.q_lens)

    @property
    def total_q(self) -> int:
        return int(sum(self.q_lens))

    @property
    def total_k(self) -> int:
        return int(sum(self.k_lens))

    def effective_flops(self) -> int:
        """4 * total_q * Hq * (topk * blk) * D: every slot counted as a full block."""
        return 4 * self.total_q * self.Hq * self.topk * self.blk * self.D


# A ragged prefill batch with the heads and index rule of the 8K causal workload:
# eight sequences of 32 768 tokens in all, five of them ending inside a block.
VARLEN_WORKLOADS = {
    "vmix": VarlenWorkload("vmix_b8_t32k_hq64_hkv4_top16_causal",
                           q_lens=(8192, 7000, 5000, 4096, 3500, 2500, 1500, 980),
                           k_lens=(8192, 7000, 5000, 4096, 3500, 2500, 1500, 980),
                           Hkv=4, qpk=16, topk=16, causal=True, mode=MODE_CAUSAL),
}


def make_varlen_workload_inputs(w: VarlenWorkload) -> dict:
    return make_varlen_inputs(w.seed, w.q_lens, w.k_lens, w.Hkv, w.qpk, w.topk, w.mode, w.D,
                              w.blk)


# ---------------------------------------------------------------------------
# fp8 e4m3fn K/V cache inputs (the fp8 KV cache of `sparse_atten_func`: K/V
# elements stored as OCP float8_e4m3fn, no scale). Conversions use torch's CPU
# float8_e4m3fn dtype: round to nearest even on the way in, exact on the way out.
# ---------------------------------------------------------------------------
_FP8_LUT = None


def bf16_bits_to_fp8(x: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp8 e4m3fn bytes (uint8), round to nearest even: a 65536-entry
    table made once by torch's conversion of every bf16 pattern, then a gather."""
    global _FP8_LUT
    if _FP8_LUT is None:
        import torch
        allbits = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16)
        f = allbits.view(torch.bfloat16).to(torch.float32)
        lut = f.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        _FP8_LUT = np.empty(65536, dtype=np.uint8)
        _FP8_LUT[allbits.numpy().view(np.uint16)] = lut
    return _FP8_LUT[np.ascontiguousarray(x, dtype=np.uint16)]


def fp8_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn bytes -> the bf16 bit patterns of the same values (exact), through a
    256-entry table made by torch's conversion."""
    import torch
    lut = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn)
    lut = lut.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return lut[np.ascontiguousarray(x, dtype=np.uint8)]


def with_fp8_kv(inp: dict) -> dict:
    """A copy of uniform, paged or varlen inputs with K/V (or the pools) as fp8 bytes."""
    out = dict(inp)
    for name in ("k", "v", "k_pool", "v_pool"):
        if name in out:
            out[name] = bf16_bits_to_fp8(out[name])
    return out
