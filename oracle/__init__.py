"""Python access to the CPU oracle (msa_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg. The product path never imports this package.
The oracle is plain double-precision C; see msa_oracle.h for the definitions
it writes out and the passages of the pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "msa_oracle.c")
_HDR = os.path.join(_HERE, "msa_oracle.h")
# MSA_ORACLE_LIB names an already built oracle library to load instead of this one; the
# oracle's mutation test uses it to run the pins against deliberately broken copies
_LIB = os.environ.get("MSA_ORACLE_LIB") or os.path.join(_HERE, "libmsa_oracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    if os.environ.get("MSA_ORACLE_LIB"):
        return _LIB  # given prebuilt
    newest = max(os.path.getmtime(_SRC), os.path.getmtime(_HDR))
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < newest:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                               "-fno-fast-math", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB)
        P, I, I64, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
        lib.oracle_sparse_attention.argtypes = [P, P, P, I, P, P, I, I, I, I, I, I, I, I, I, D,
                                                P, I64, P, P, D, P, I]
        lib.oracle_sparse_attention.restype = I
        lib.oracle_paged_sparse_attention.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, I, I,
                                                      I, I, I, D, P, I64, P, P, D, P, I]
        lib.oracle_paged_sparse_attention.restype = I
        lib.oracle_k2q_csr.argtypes = [P, I, I, I, I, I, P, P, P]
        lib.oracle_k2q_csr.restype = I
        lib.oracle_sparse_attention_varlen.argtypes = [P, P, P, I, P, P, P, I, I, I, I, I, I, I,
                                                       D, P, I64, P, P, D, P, I]
        lib.oracle_sparse_attention_varlen.restype = I
        lib.oracle_k2q_csr_varlen.argtypes = [P, P, P, I, I, I, I, I, P, P, P]
        lib.oracle_k2q_csr_varlen.restype = I
        lib.oracle_fp8_e4m3_decode.argtypes = [P, I64, P]
        lib.oracle_fp8_e4m3_decode.restype = I
        lib.oracle_fp8_e4m3_round.argtypes = [P, I64, P]
        lib.oracle_fp8_e4m3_round.restype = I
        lib.oracle_paged_decode_fp8.argtypes = [P, P, P, P, P, I, I, I, I, I, I, I, I, I, D, P,
                                                I64, P, P, D, P, I]
        lib.oracle_paged_decode_fp8.restype = I
        _lib = lib
    return _lib


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _kv(k, v):
    """K/V as given: uint16 (bf16 bits) or uint8 (fp8 e4m3fn bytes); returns (k, v, fp8)."""
    fp8 = np.asarray(k).dtype == np.uint8
    if fp8 != (np.asarray(v).dtype == np.uint8):
        raise ValueError("k and v must both be bf16 bits (uint16) or both fp8 bytes (uint8)")
    dt = np.uint8 if fp8 else np.uint16
    return _c(k, dt), _c(v, dt), int(fp8)


def fp8_e4m3_decode(x) -> np.ndarray:
    """The oracle's fp8 e4m3fn decoding of a uint8 array (float64, same shape)."""
    a = _c(x, np.uint8)
    out = np.empty(a.shape, dtype=np.float64)
    if _load().oracle_fp8_e4m3_decode(_ptr(a), a.size, _ptr(out)) != 0:
        raise ValueError("oracle_fp8_e4m3_decode: invalid arguments")
    return out


def fp8_e4m3_round(x) -> np.ndarray:
    """The oracle's rounding to the nearest fp8 e4m3fn value (ties to even), float64."""
    a = _c(x, np.float64)
    out = np.empty(a.shape, dtype=np.float64)
    if _load().oracle_fp8_e4m3_round(_ptr(a), a.size, _ptr(out)) != 0:
        raise ValueError("oracle_fp8_e4m3_round: invalid arguments")
    return out


def paged_decode_fp8(q, k_pool, v_pool, page_table, seqused_k, *, causal: bool,
                     softmax_scale: Optional[float] = None, rows=None,
                     temperature: Optional[float] = None, nthreads: int = 0):
    """Oracle fp8 dense paged decode (the test page's `_decode_paged_dense_reference`):
    q [B, Sq, Hq, D], k_pool / v_pool [num_pages, Hkv, page_size, D], all fp8 e4m3fn
    bytes (uint8); every key of the sequence, probabilities rounded to e4m3 before the
    P V product, the row sum unrounded. Returns (O, LSE[, LSE_T]) shaped like
    paged_sparse_attention's."""
    q, k_pool, v_pool = _c(q, np.uint8), _c(k_pool, np.uint8), _c(v_pool, np.uint8)
    page_table, seqused_k = _c(page_table, np.int32), _c(seqused_k, np.int32)
    B, Sq, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    assert page_table.shape[0] == B and seqused_k.shape == (B,) and v_pool.shape == k_pool.shape
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    rws = _c(rows, np.int64)
    n = B * Sq if rws is None else rws.size
    o = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    temp, lse_t = _temperature_out(n, Hq, temperature)
    rc = _load().oracle_paged_decode_fp8(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table), _ptr(seqused_k), B, Sq, Hq, Hkv,
        D, page_size, num_pages, max_pages, int(causal), scale, _ptr(rws), n, _ptr(o), _ptr(lse),
        temp, _ptr(lse_t), nthreads)
    if rc != 0:
        raise ValueError("oracle_paged_decode_fp8: invalid arguments")
    return _shape_out(o, lse, rws, B, Sq, Hq, D, lse_t)


def _shape_out(o, lse, rows, B, Sq, Hq, D, lse_t=None):
    if rows is None:
        o = o.reshape(B, Sq, Hq, D)
        lse = lse.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()
        if lse_t is not None:
            lse_t = lse_t.reshape(B, Sq, Hq).transpose(0, 2, 1).copy()
    return (o, lse) if lse_t is None else (o, lse, lse_t)


def _temperature_out(n, Hq, temperature):
    """(temp, buffer) for the C call: no buffer unless a temperature is asked for."""
    if temperature is None:
        return 1.0, None
    if not temperature > 0:
        raise ValueError("temperature must be positive")
    return float(temperature), np.empty((n, Hq), dtype=np.float64)


def sparse_attention(q, k, v, q2k, *, causal: bool, blk: int = 128,
                     softmax_scale: Optional[float] = None, seqused_k=None, rows=None,
                     temperature: Optional[float] = None, nthreads: int = 0):
    """Oracle forward, contiguous K/V.

    q [B,Sq,Hq,D], k/v [B,Skv,Hkv,D] as uint16 bf16 bits (or uint8 fp8 e4m3fn bytes:
    the fp8 KV cache); q2k [B,Hkv,Sq,topk].
    rows=None: returns O [B,Sq,Hq,D] and LSE [B,Hq,Sq] (float64).
    rows = array of b*Sq+q ids: returns O [n,Hq,D] and LSE [n,Hq].
    temperature: also return the temperature-scaled LSE (same layout as LSE).
    """
    q = _c(q, np.uint16)
    k, v, fp8 = _kv(k, v)
    q2k = _c(q2k, np.int32)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    topk = q2k.shape[-1]
    assert q2k.shape == (B, Hkv, Sq, topk) and v.shape == k.shape
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    seq = _c(seqused_k, np.int32)
    rws = _c(rows, np.int64)
    n = B * Sq if rws is None else rws.size
    o = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    temp, lse_t = _temperature_out(n, Hq, temperature)
    rc = _load().oracle_sparse_attention(_ptr(q), _ptr(k), _ptr(v), fp8, _ptr(q2k), _ptr(seq), B,
                                         Sq,
                                         Skv, Hq, Hkv, D, topk, blk, int(causal), scale,
                                         _ptr(rws), n, _ptr(o), _ptr(lse), temp, _ptr(lse_t),
                                         nthreads)
    if rc != 0:
        raise ValueError("oracle_sparse_attention: invalid arguments")
    return _shape_out(o, lse, rws, B, Sq, Hq, D, lse_t)


def paged_sparse_attention(q, k_pool, v_pool, page_table, seqused_k, q2k, *, causal: bool,
                           softmax_scale: Optional[float] = None, rows=None,
                           temperature: Optional[float] = None, nthreads: int = 0):
    """Oracle forward, paged K/V pool [num_pages,Hkv,page_size,D], page_table [B,max_pages]."""
    q = _c(q, np.uint16)
    k_pool, v_pool, fp8 = _kv(k_pool, v_pool)
    page_table, seqused_k, q2k = (_c(page_table, np.int32), _c(seqused_k, np.int32),
                                  _c(q2k, np.int32))
    B, Sq, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    topk = q2k.shape[-1]
    assert q2k.shape == (B, Hkv, Sq, topk) and page_table.shape[0] == B
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    rws = _c(rows, np.int64)
    n = B * Sq if rws is None else rws.size
    o = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    temp, lse_t = _temperature_out(n, Hq, temperature)
    rc = _load().oracle_paged_sparse_attention(
        _ptr(q), _ptr(k_pool), _ptr(v_pool), fp8, _ptr(page_table), _ptr(seqused_k), _ptr(q2k),
        B, Sq,
        Hq, Hkv, D, topk, page_size, num_pages, max_pages, int(causal), scale, _ptr(rws), n,
        _ptr(o), _ptr(lse), temp, _ptr(lse_t), nthreads)
    if rc != 0:
        raise ValueError("oracle_paged_sparse_attention: invalid arguments")
    return _shape_out(o, lse, rws, B, Sq, Hq, D, lse_t)


def k2q_csr(q2k, nblk: int, with_slot: bool = True):
    """Oracle kv-block -> query CSR of q2k [B,Hkv,Sq,topk].

    Returns (row_ptr [Hkv, B*nblk+1], q_idx [Hkv, B*Sq*topk], slot or None); entries
    past row_ptr[h, -1] are -1.
    """
    q2k = _c(q2k, np.int32)
    B, Hkv, Sq, topk = q2k.shape
    row_ptr = np.empty((Hkv, B * nblk + 1), dtype=np.int32)
    q_idx = np.full((Hkv, B * Sq * topk), -1, dtype=np.int32)
    slot = np.full((Hkv, B * Sq * topk), -1, dtype=np.int32) if with_slot else None
    rc = _load().oracle_k2q_csr(_ptr(q2k), B, Hkv, Sq, topk, nblk, _ptr(row_ptr), _ptr(q_idx),
                                _ptr(slot))
    if rc != 0:
        raise ValueError("oracle_k2q_csr: invalid arguments")
    return row_ptr, q_idx, slot


def sparse_attention_varlen(q, k, v, q2k, cu_seqlens_q, cu_seqlens_k, *, causal: bool,
                            blk: int = 128, softmax_scale: Optional[float] = None, rows=None,
                            temperature: Optional[float] = None, nthreads: int = 0):
    """Oracle forward of a variable-length batch.

    q [total_q,Hq,D], k/v [total_k,Hkv,D] (uint16 bf16 bits), q2k [Hkv,total_q,topk],
    cu_seqlens_q / cu_seqlens_k [B+1]. Returns O [n,Hq,D] and LSE [n,Hq] (the packed
    layout of the interface page) for the given global rows, n = total_q when rows=None;
    with a temperature, also the temperature-scaled LSE [n,Hq].
    """
    q = _c(q, np.uint16)
    k, v, fp8 = _kv(k, v)
    q2k, cq, ck = _c(q2k, np.int32), _c(cu_seqlens_q, np.int32), _c(cu_seqlens_k, np.int32)
    total_q, Hq, D = q.shape
    _, Hkv, _ = k.shape
    topk = q2k.shape[-1]
    B = cq.size - 1
    assert q2k.shape == (Hkv, total_q, topk) and ck.size == B + 1 and cq[-1] == total_q
    scale = D ** -0.5 if softmax_scale is None else float(softmax_scale)
    rws = _c(rows, np.int64)
    n = total_q if rws is None else rws.size
    o = np.empty((n, Hq, D), dtype=np.float64)
    lse = np.empty((n, Hq), dtype=np.float64)
    temp, lse_t = _temperature_out(n, Hq, temperature)
    rc = _load().oracle_sparse_attention_varlen(_ptr(q), _ptr(k), _ptr(v), fp8, _ptr(q2k),
                                                _ptr(cq),
                                                _ptr(ck), B, Hq, Hkv, D, topk, blk, int(causal),
                                                scale, _ptr(rws), n, _ptr(o), _ptr(lse), temp,
                                                _ptr(lse_t), nthreads)
    if rc != 0:
        raise ValueError("oracle_sparse_attention_varlen: invalid arguments")
    return (o, lse) if lse_t is None else (o, lse, lse_t)


def varlen_total_rows(cu_seqlens_k, blk: int = 128) -> int:
    """Number of CSR rows of a variable-length batch: sum of ceil(Skv_b / blk)."""
    ck = np.asarray(cu_seqlens_k, dtype=np.int64)
    return int(((np.diff(ck) + blk - 1) // blk).sum())


def k2q_csr_varlen(q2k, cu_seqlens_q, cu_seqlens_k, *, blk: int = 128, with_slot: bool = True):
    """Oracle CSR of a variable-length batch (q2k [Hkv,total_q,topk]).

    Returns (row_ptr [Hkv, total_rows+1], q_idx [Hkv, total_q*topk], slot or None);
    entries past row_ptr[h, -1] are -1.
    """
    q2k, cq, ck = _c(q2k, np.int32), _c(cu_seqlens_q, np.int32), _c(cu_seqlens_k, np.int32)
    Hkv, total_q, topk = q2k.shape
    B = cq.size - 1
    rows = varlen_total_rows(ck, blk)
    row_ptr = np.empty((Hkv, rows + 1), dtype=np.int32)
    q_idx = np.full((Hkv, total_q * topk), -1, dtype=np.int32)
    slot = np.full((Hkv, total_q * topk), -1, dtype=np.int32) if with_slot else None
    rc = _load().oracle_k2q_csr_varlen(_ptr(q2k), _ptr(cq), _ptr(ck), B, Hkv, topk, blk, rows,
                                       _ptr(row_ptr), _ptr(q_idx), _ptr(slot))
    if rc != 0:
        raise ValueError("oracle_k2q_csr_varlen: invalid arguments")
    return row_ptr, q_idx, slot


