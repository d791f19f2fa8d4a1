"""ctypes marshalling for libmsa.so (see include/msa.h for the contract)."""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libmsa.so")

MSA_OK, MSA_ERR_INVALID_VALUE, MSA_ERR_NOT_SUPPORTED, MSA_ERR_HIP = 0, 1, 2, 3
MSA_PATH_AUTO, MSA_PATH_QCENTRIC, MSA_PATH_KVCENTRIC, MSA_PATH_DECODE, MSA_PATH_TILE = 0, 1, 2, 3, 4
MSA_DTYPE_BF16, MSA_DTYPE_FP8_E4M3 = 0, 1

_lib = None


class MsaError(RuntimeError):
    """A failed libmsa call (status MSA_ERR_HIP or unknown)."""

    def __init__(self, code: int, msg: str):
        super().__init__(f"[msa status {code}] {msg}")
        self.code = code


class MsaValueError(MsaError, ValueError):
    """MSA_ERR_INVALID_VALUE: bad pointer, size or workspace."""


class MsaNotSupportedError(MsaError, NotImplementedError):
    """MSA_ERR_NOT_SUPPORTED: a shape or option outside the supported set."""


class MsaDecodePlan(ctypes.Structure):
    """msa_decode_plan of include/msa.h (host part of a dense-decode plan)."""
    _fields_ = [("batch", ctypes.c_int), ("seqlen_q", ctypes.c_int),
                ("num_qo_heads", ctypes.c_int), ("num_kv_heads", ctypes.c_int),
                ("max_pages", ctypes.c_int), ("kv_chunk_size_pages", ctypes.c_int),
                ("split_kv", ctypes.c_int), ("padded_work_count", ctypes.c_int),
                ("partial_rows", ctypes.c_int64)] + [
        (n, ctypes.c_size_t) for n in ("kv_pages", "split_counts", "o_indptr", "merge_indptr",
                                      "work_offsets", "work_items", "work_count", "o_partial",
                                      "lse_partial", "lse_t_partial", "bytes")]


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Load libmsa.so; raises if it has not been built (no fallback path exists)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with "
                          "`python -m block_sparse_attention_top_amd.build`")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    lib.msa_sparse_fwd_workspace_size.argtypes = [I] * 9
    lib.msa_sparse_fwd_workspace_size.restype = S
    lib.msa_sparse_fwd_path.argtypes = [I] * 7
    lib.msa_sparse_fwd_path.restype = I
    lib.msa_sparse_fwd.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, F, I, I, P, P,
                                   F, P, P, S, P]
    lib.msa_sparse_fwd.restype = I
    lib.msa_build_k2q_csr_workspace_size.argtypes = [I] * 5
    lib.msa_build_k2q_csr_workspace_size.restype = S
    lib.msa_build_k2q_csr.argtypes = [P, I, I, I, I, I, P, P, P, P, S, P]
    lib.msa_build_k2q_csr.restype = I
    lib.msa_sparse_fwd_varlen_workspace_size.argtypes = [I] * 9
    lib.msa_sparse_fwd_varlen_workspace_size.restype = S
    lib.msa_sparse_fwd_varlen_path.argtypes = [I] * 7
    lib.msa_sparse_fwd_varlen_path.restype = I
    lib.msa_sparse_fwd_varlen.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                          I, F, I, I, P, P, F, P, P, S, P]
    lib.msa_sparse_fwd_varlen.restype = I
    lib.msa_build_k2q_csr_varlen_workspace_size.argtypes = [I] * 5
    lib.msa_build_k2q_csr_varlen_workspace_size.restype = S
    lib.msa_build_k2q_csr_varlen.argtypes = [P, P, P, I, I, I, I, I, I, P, P, P, P, S, P]
    lib.msa_build_k2q_csr_varlen.restype = I
    lib.msa_paged_sparse_fwd_workspace_size.argtypes = [I] * 10
    lib.msa_paged_sparse_fwd_workspace_size.restype = S
    lib.msa_paged_sparse_fwd_path.argtypes = [I] * 6
    lib.msa_paged_sparse_fwd_path.restype = I
    lib.msa_paged_sparse_fwd_splits.argtypes = [I] * 7
    lib.msa_paged_sparse_fwd_splits.restype = I
    lib.msa_paged_sparse_fwd.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F, I, I,
                                         I, P, P, F, P, P, S, P]
    lib.msa_paged_sparse_fwd.restype = I
    lib.msa_paged_sparse_fwd_noalloc.argtypes = [P, P, P, P, P, P, I, I, I, I, I, I, I, I, I, I, F,
                                                 I, I, I, P, P, F, P, P]
    lib.msa_paged_sparse_fwd_noalloc.restype = I
    lib.msa_paged_sparse_fwd_varlen_workspace_size.argtypes = [I] * 10
    lib.msa_paged_sparse_fwd_varlen_workspace_size.restype = S
    lib.msa_paged_sparse_fwd_varlen_path.argtypes = [I] * 6
    lib.msa_paged_sparse_fwd_varlen_path.restype = I
    lib.msa_paged_sparse_fwd_varlen_splits.argtypes = [I] * 7
    lib.msa_paged_sparse_fwd_varlen_splits.restype = I
    lib.msa_paged_sparse_fwd_varlen.argtypes = [P, P, P, P, P, P, P, I, I, I, I, I, I, I, I, I,
                                                I, F, I, I, I, P, P, F, P, P, S, P]
    lib.msa_paged_sparse_fwd_varlen.restype = I
    PL = ctypes.POINTER(MsaDecodePlan)
    lib.msa_paged_decode_plan_init.argtypes = [I, I, I, I, I, I, I, I, I, I, PL]
    lib.msa_paged_decode_plan_init.restype = I
    lib.msa_paged_decode_plan.argtypes = [P, PL, P, S, P]
    lib.msa_paged_decode_plan.restype = I
    lib.msa_paged_decode_run.argtypes = [P, P, P, P, P, PL, P, S, I, I, I, F, P, P, F, P, P]
    lib.msa_paged_decode_run.restype = I
    lib.msa_set_profiling_events.argtypes = [P, P]
    lib.msa_set_profiling_events.restype = I
    lib.msa_last_error.argtypes = []
    lib.msa_last_error.restype = ctypes.c_char_p
    lib.msa_version.argtypes = []
    lib.msa_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def msa_set_profiling_events(before=None, after=None) -> None:
    """Record hipEvent handles (ints) around the dominant kernel of later calls."""
    _check(load_library().msa_set_profiling_events(before, after))


def msa_last_error() -> str:
    return load_library().msa_last_error().decode()


def msa_version() -> str:
    return load_library().msa_version().decode()


def _check(rc: int) -> None:
    if rc == MSA_OK:
        return
    msg = msa_last_error()
    if rc == MSA_ERR_INVALID_VALUE:
        raise MsaValueError(rc, msg)
    if rc == MSA_ERR_NOT_SUPPORTED:
        raise MsaNotSupportedError(rc, msg)
    raise MsaError(rc, msg)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, dtype: torch.dtype) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _kv_dtype(k: torch.Tensor, v: torch.Tensor, names=("k", "v")) -> int:
    """bf16 K/V, or the fp8 e4m3fn cache (torch.float8_e4m3fn, or uint8 holding its bytes)."""
    fp8 = {getattr(torch, "float8_e4m3fn", None), torch.uint8}
    for t, nm in zip((k, v), names):
        if not isinstance(t, torch.Tensor) or not t.is_cuda:
            raise ValueError(f"{nm} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{nm} must be contiguous")
    if k.dtype == torch.bfloat16 and v.dtype == torch.bfloat16:
        return MSA_DTYPE_BF16
    if k.dtype in fp8 and v.dtype in fp8:
        return MSA_DTYPE_FP8_E4M3
    raise TypeError(f"{names[0]}/{names[1]} must both be bf16 or both fp8 e4m3fn, "
                    f"got {k.dtype} / {v.dtype}")


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


# |T - 1| at or below this returns the LSE itself as the temperature-scaled LSE,
# as the interface page's binding does
TEMPERATURE_FAST_PATH_ABS_TOL = 1e-12


def _temperature(lse: torch.Tensor, return_temperature_lse: bool, scale, out, fast_path: bool):
    """(T, buffer or None, alias): alias means the LSE itself is the answer (T = 1)."""
    if not return_temperature_lse:
        return 1.0, None, False
    t = 1.0 if scale is None else float(scale)
    if fast_path and abs(t - 1.0) <= TEMPERATURE_FAST_PATH_ABS_TOL and out is None:
        return t, None, True
    if out is None:
        out = torch.empty_like(lse)
    _dev(out, "lse_temperature", torch.float32)
    if tuple(out.shape) != tuple(lse.shape):
        raise ValueError("lse_temperature must have the shape of lse")
    return t, out, False


def _workspace(nbytes: int, device, workspace: Optional[torch.Tensor]):
    if nbytes == 0:
        return None, 0
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    _dev(workspace, "workspace", torch.uint8)
    return workspace, workspace.numel()


def msa_sparse_fwd_workspace_size(B, Sq, Skv, Hq, Hkv, D, topk, blk_kv=128,
                                  path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_sparse_fwd_workspace_size(B, Sq, Skv, Hq, Hkv, D, topk, blk_kv,
                                                            path))


def msa_sparse_fwd_path(B, Sq, Skv, Hq, Hkv, topk, path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_sparse_fwd_path(B, Sq, Skv, Hq, Hkv, topk, path))


def msa_sparse_fwd(q, k, v, q2k, csr_row_ptr=None, csr_q_idx=None, csr_slot=None, *,
                   causal: bool, softmax_scale: float = 0.0, path: int = MSA_PATH_AUTO,
                   blk_kv: int = 128, o=None, lse=None, return_temperature_lse: bool = False,
                   lse_temperature_scale: Optional[float] = None, lse_temperature=None,
                   temperature_fast_path: bool = True, workspace=None, stream=None):
    """Sparse forward with contiguous K/V (bf16, or the fp8 e4m3fn cache). Returns
    (O bf16 [B,Sq,Hq,D], LSE fp32 [B,Hq,Sq]), plus the temperature-scaled LSE (same
    layout) when return_temperature_lse."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16)
    kv_dtype = _kv_dtype(k, v)
    _dev(q2k, "q2k", torch.int32)
    B, Sq, Hq, D = q.shape
    _, Skv, Hkv, _ = k.shape
    topk = q2k.shape[-1]
    for t, nm in ((csr_row_ptr, "csr_row_ptr"), (csr_q_idx, "csr_q_idx"), (csr_slot, "csr_slot")):
        if t is not None:
            _dev(t, nm, torch.int32)
    if o is None:
        o = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    nbytes = int(lib.msa_sparse_fwd_workspace_size(B, Sq, Skv, Hq, Hkv, D, topk, blk_kv, path))
    ws, wsn = _workspace(nbytes, q.device, workspace)
    rc = lib.msa_sparse_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(q2k), _ptr(csr_row_ptr),
                            _ptr(csr_q_idx), _ptr(csr_slot), B, Sq, Skv, Hq, Hkv, D, topk, blk_kv,
                            int(bool(causal)), float(softmax_scale), int(path), kv_dtype, _ptr(o),
                            _ptr(lse), temp, _ptr(lse_t), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse


def msa_build_k2q_csr_workspace_size(B, Hkv, Sq, topk, num_kv_blocks) -> int:
    return int(load_library().msa_build_k2q_csr_workspace_size(B, Hkv, Sq, topk, num_kv_blocks))


def msa_build_k2q_csr(q2k, num_kv_blocks: int, *, row_ptr=None, q_idx=None, slot=None,
                      with_slot: bool = True, workspace=None, stream=None):
    """kv-block -> query CSR of q2k [B,Hkv,Sq,topk]. Returns (row_ptr, q_idx, slot or None)."""
    lib = load_library()
    _dev(q2k, "q2k", torch.int32)
    B, Hkv, Sq, topk = q2k.shape
    dev = q2k.device
    if row_ptr is None:
        row_ptr = torch.empty((Hkv, B * num_kv_blocks + 1), dtype=torch.int32, device=dev)
    if q_idx is None:
        q_idx = torch.empty((Hkv, B * Sq * topk), dtype=torch.int32, device=dev)
    if slot is None and with_slot:
        slot = torch.empty((Hkv, B * Sq * topk), dtype=torch.int32, device=dev)
    nbytes = int(lib.msa_build_k2q_csr_workspace_size(B, Hkv, Sq, topk, num_kv_blocks))
    ws, wsn = _workspace(nbytes, dev, workspace)
    rc = lib.msa_build_k2q_csr(_ptr(q2k), B, Hkv, Sq, topk, num_kv_blocks, _ptr(row_ptr),
                               _ptr(q_idx), _ptr(slot), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    return row_ptr, q_idx, slot


def msa_sparse_fwd_varlen_workspace_size(B, total_q, total_k, Hq, Hkv, D, topk, blk_kv=128,
                                         path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_sparse_fwd_varlen_workspace_size(B, total_q, total_k, Hq, Hkv, D,
                                                                   topk, blk_kv, path))


def msa_sparse_fwd_varlen_path(B, total_q, total_k, Hq, Hkv, topk, path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_sparse_fwd_varlen_path(B, total_q, total_k, Hq, Hkv, topk, path))


def msa_sparse_fwd_varlen(q, k, v, q2k, cu_seqlens_q, cu_seqlens_k, csr_row_ptr=None,
                          csr_q_idx=None, csr_slot=None, csr_total_rows: int = 0, *, causal: bool,
                          softmax_scale: float = 0.0, path: int = MSA_PATH_AUTO, blk_kv: int = 128,
                          o=None, lse=None, return_temperature_lse: bool = False,
                          lse_temperature_scale: Optional[float] = None, lse_temperature=None,
                          temperature_fast_path: bool = True, workspace=None, stream=None):
    """Sparse forward of a variable-length batch (packed q [total_q,Hq,D], k/v
    [total_k,Hkv,D], q2k [Hkv,total_q,topk], cu_seqlens [B+1] on the device).
    Returns (O bf16 [total_q,Hq,D], LSE fp32 [total_q,Hq]). K/V bf16 or fp8 e4m3fn."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16)
    kv_dtype = _kv_dtype(k, v)
    _dev(q2k, "q2k", torch.int32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    total_q, Hq, D = q.shape
    total_k, Hkv, _ = k.shape
    topk = q2k.shape[-1]
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    if tuple(q2k.shape) != (Hkv, total_q, topk):
        raise ValueError("q2k must have shape [Hkv, total_q, topk]")
    for t, nm in ((csr_row_ptr, "csr_row_ptr"), (csr_q_idx, "csr_q_idx"), (csr_slot, "csr_slot")):
        if t is not None:
            _dev(t, nm, torch.int32)
    if o is None:
        o = torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    nbytes = int(lib.msa_sparse_fwd_varlen_workspace_size(B, total_q, total_k, Hq, Hkv, D, topk,
                                                          blk_kv, path))
    ws, wsn = _workspace(nbytes, q.device, workspace)
    rc = lib.msa_sparse_fwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), _ptr(q2k), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k),
        _ptr(csr_row_ptr), _ptr(csr_q_idx), _ptr(csr_slot), int(csr_total_rows), B, total_q,
        total_k, Hq, Hkv, D, topk, blk_kv, int(bool(causal)), float(softmax_scale), int(path),
        kv_dtype, _ptr(o), _ptr(lse), temp, _ptr(lse_t), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse


def msa_build_k2q_csr_varlen_workspace_size(B, Hkv, total_q, topk, total_rows) -> int:
    return int(load_library().msa_build_k2q_csr_varlen_workspace_size(B, Hkv, total_q, topk,
                                                                      total_rows))


def msa_build_k2q_csr_varlen(q2k, cu_seqlens_q, cu_seqlens_k, total_k: int, total_rows: int, *,
                             row_ptr=None, q_idx=None, slot=None, with_slot: bool = True,
                             workspace=None, stream=None):
    """kv-block -> query CSR of a variable-length batch (q2k [Hkv,total_q,topk]) over
    total_rows = sum_b ceil(Skv_b / 128) rows. Returns (row_ptr, q_idx, slot or None)."""
    lib = load_library()
    _dev(q2k, "q2k", torch.int32)
    _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32), _dev(cu_seqlens_k, "cu_seqlens_k", torch.int32)
    Hkv, total_q, topk = q2k.shape
    B = cu_seqlens_q.numel() - 1
    if cu_seqlens_k.numel() != B + 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must have the same length")
    dev = q2k.device
    if row_ptr is None:
        row_ptr = torch.empty((Hkv, total_rows + 1), dtype=torch.int32, device=dev)
    if q_idx is None:
        q_idx = torch.empty((Hkv, total_q * topk), dtype=torch.int32, device=dev)
    if slot is None and with_slot:
        slot = torch.empty((Hkv, total_q * topk), dtype=torch.int32, device=dev)
    nbytes = int(lib.msa_build_k2q_csr_varlen_workspace_size(B, Hkv, total_q, topk, total_rows))
    ws, wsn = _workspace(nbytes, dev, workspace)
    rc = lib.msa_build_k2q_csr_varlen(_ptr(q2k), _ptr(cu_seqlens_q), _ptr(cu_seqlens_k), B, Hkv,
                                      total_q, int(total_k), topk, int(total_rows), _ptr(row_ptr),
                                      _ptr(q_idx), _ptr(slot), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    return row_ptr, q_idx, slot


def msa_paged_sparse_fwd_workspace_size(B, Sq, Hq, Hkv, D, topk, page_size, max_pages,
                                        num_splits=0, path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_workspace_size(B, Sq, Hq, Hkv, D, topk,
                                                                  page_size, max_pages,
                                                                  num_splits, path))


def msa_paged_sparse_fwd_path(B, Sq, Hkv, topk, max_pages, path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_path(B, Sq, Hkv, topk, max_pages, path))


def msa_paged_sparse_fwd_splits(B, Sq, Hkv, topk, max_pages, num_splits=0,
                                path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_splits(B, Sq, Hkv, topk, max_pages,
                                                          num_splits, path))


def msa_paged_sparse_fwd(q, k_pool, v_pool, page_table, seqused_k, q2k, *, causal: bool,
                         softmax_scale: float = 0.0, num_splits: int = 0,
                         path: int = MSA_PATH_AUTO, o=None, lse=None,
                         return_temperature_lse: bool = False,
                         lse_temperature_scale: Optional[float] = None, lse_temperature=None,
                         temperature_fast_path: bool = True, workspace=None, stream=None):
    """Sparse forward through a page table. Returns (O, LSE[, LSE_T]) as msa_sparse_fwd."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16)
    kv_dtype = _kv_dtype(k_pool, v_pool, ("k_pool", "v_pool"))
    _dev(page_table, "page_table", torch.int32)
    _dev(seqused_k, "seqused_k", torch.int32), _dev(q2k, "q2k", torch.int32)
    B, Sq, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    topk = q2k.shape[-1]
    if o is None:
        o = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    nbytes = int(lib.msa_paged_sparse_fwd_workspace_size(B, Sq, Hq, Hkv, D, topk, page_size,
                                                         max_pages, num_splits, path))
    ws, wsn = _workspace(nbytes, q.device, workspace)
    rc = lib.msa_paged_sparse_fwd(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                  _ptr(seqused_k), _ptr(q2k), B, Sq, Hq, Hkv, D, topk, page_size,
                                  num_pages, max_pages, int(bool(causal)), float(softmax_scale),
                                  int(num_splits), int(path), kv_dtype, _ptr(o), _ptr(lse), temp,
                                  _ptr(lse_t), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse


def msa_paged_sparse_fwd_noalloc(q, k_pool, v_pool, page_table, seqused_k, q2k, *,
                                 causal: bool, softmax_scale: float = 0.0, num_splits: int = 0,
                                 path: int = MSA_PATH_AUTO, o=None, lse=None,
                                 return_temperature_lse: bool = False,
                                 lse_temperature_scale: Optional[float] = None,
                                 lse_temperature=None, temperature_fast_path: bool = True,
                                 stream=None):
    """msa_paged_sparse_fwd without a workspace: the split partials use the library's
    own per-GPU scratch array (MSA_NOALLOC_SCRATCH_BYTES). The library allocates
    nothing; outputs are allocated here only when not given."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16)
    kv_dtype = _kv_dtype(k_pool, v_pool, ("k_pool", "v_pool"))
    _dev(page_table, "page_table", torch.int32)
    _dev(seqused_k, "seqused_k", torch.int32), _dev(q2k, "q2k", torch.int32)
    B, Sq, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pool.shape
    max_pages = page_table.shape[1]
    topk = q2k.shape[-1]
    if o is None:
        o = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    rc = lib.msa_paged_sparse_fwd_noalloc(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                          _ptr(seqused_k), _ptr(q2k), B, Sq, Hq, Hkv, D, topk,
                                          page_size, num_pages, max_pages, int(bool(causal)),
                                          float(softmax_scale), int(num_splits), int(path),
                                          kv_dtype, _ptr(o), _ptr(lse), temp, _ptr(lse_t),
                                          _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse


MSA_NOALLOC_SCRATCH_BYTES = 64 << 20


def msa_paged_sparse_fwd_varlen_workspace_size(B, total_q, Hq, Hkv, D, topk, page_size,
                                               max_pages, num_splits=0,
                                               path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_varlen_workspace_size(
        B, total_q, Hq, Hkv, D, topk, page_size, max_pages, num_splits, path))


def msa_paged_sparse_fwd_varlen_splits(B, total_q, Hkv, topk, max_pages, num_splits=0,
                                       path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_varlen_splits(B, total_q, Hkv, topk,
                                                                  max_pages, num_splits, path))


def msa_paged_sparse_fwd_varlen_path(B, total_q, Hkv, topk, max_pages,
                                     path=MSA_PATH_AUTO) -> int:
    return int(load_library().msa_paged_sparse_fwd_varlen_path(B, total_q, Hkv, topk, max_pages,
                                                                path))


def msa_paged_sparse_fwd_varlen(q, k_pool, v_pool, page_table, seqused_k, cu_seqlens_q, q2k, *,
                                causal: bool, softmax_scale: float = 0.0, num_splits: int = 0,
                                path: int = MSA_PATH_AUTO, o=None, lse=None,
                                return_temperature_lse: bool = False,
                                lse_temperature_scale: Optional[float] = None,
                                lse_temperature=None, temperature_fast_path: bool = True,
                                workspace=None, stream=None):
    """Paged K/V with a packed query batch: q [total_q, Hq, D], cu_seqlens_q [B+1],
    q2k [Hkv, total_q, topk]. Returns (O [total_q, Hq, D], LSE [total_q, Hq][, LSE_T])."""
    lib = load_library()
    _dev(q, "q", torch.bfloat16)
    kv_dtype = _kv_dtype(k_pool, v_pool, ("k_pool", "v_pool"))
    _dev(page_table, "page_table", torch.int32)
    _dev(seqused_k, "seqused_k", torch.int32), _dev(cu_seqlens_q, "cu_seqlens_q", torch.int32)
    _dev(q2k, "q2k", torch.int32)
    total_q, Hq, D = q.shape
    num_pages, Hkv, page_size, _ = k_pool.shape
    B, max_pages = page_table.shape
    topk = q2k.shape[-1]
    if cu_seqlens_q.numel() != B + 1 or seqused_k.numel() != B:
        raise ValueError("cu_seqlens_q needs B + 1 entries and seqused_k B (B = page_table rows)")
    if tuple(q2k.shape) != (Hkv, total_q, topk):
        raise ValueError("q2k must be [Hkv, total_q, topk]")
    if o is None:
        o = torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((total_q, Hq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    nbytes = int(lib.msa_paged_sparse_fwd_varlen_workspace_size(B, total_q, Hq, Hkv, D, topk,
                                                                page_size, max_pages,
                                                                num_splits, path))
    ws, wsn = _workspace(nbytes, q.device, workspace)
    rc = lib.msa_paged_sparse_fwd_varlen(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                         _ptr(seqused_k), _ptr(cu_seqlens_q), _ptr(q2k), B,
                                         total_q, Hq, Hkv, D, topk, page_size, num_pages,
                                         max_pages, int(bool(causal)), float(softmax_scale),
                                         int(num_splits), int(path), kv_dtype, _ptr(o),
                                         _ptr(lse), temp,
                                         _ptr(lse_t), _ptr(ws), wsn, _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse


class DecodePlan:
    """A dense paged-decode plan: the host struct and the device plan buffer (schedule
    arrays and partial workspace). The schedule arrays are exposed as int32 views."""

    def __init__(self, info: MsaDecodePlan, buffer: torch.Tensor):
        self.info = info
        self.buffer = buffer

    def _i32(self, off: int, n: int) -> torch.Tensor:
        return self.buffer[off:off + 4 * n].view(torch.int32)

    @property
    def kv_pages(self):
        return self._i32(self.info.kv_pages, self.info.batch)

    @property
    def split_counts(self):
        return self._i32(self.info.split_counts, self.info.batch)

    @property
    def o_indptr(self):
        return self._i32(self.info.o_indptr, self.info.batch + 1)

    @property
    def merge_indptr(self):
        return self._i32(self.info.merge_indptr, self.info.batch * self.info.seqlen_q + 1)

    @property
    def work_count(self):
        return self._i32(self.info.work_count, 1)

    @property
    def work_items(self):
        n = self.info.padded_work_count
        return self._i32(self.info.work_items, 4 * n).view(n, 4)


def msa_paged_decode_plan(page_table, seqused_k, *, seqlen_q: int, max_seqlen_k: int,
                          num_qo_heads: int, num_kv_heads: int, head_dim: int = 128,
                          page_size: int = 128, max_grid_size: int = 0, fixed_split_size: int = 0,
                          disable_split_kv: bool = False, stream=None) -> DecodePlan:
    """Plan of the dense paged decode (q2k = None): sizes on the host, the split-KV
    schedule built on the device from seqused_k."""
    lib = load_library()
    _dev(page_table, "page_table", torch.int32), _dev(seqused_k, "seqused_k", torch.int32)
    B = page_table.shape[0]
    info = MsaDecodePlan()
    _check(lib.msa_paged_decode_plan_init(B, int(seqlen_q), int(num_qo_heads), int(num_kv_heads),
                                          int(head_dim), int(page_size), int(max_seqlen_k),
                                          int(max_grid_size), int(fixed_split_size),
                                          int(bool(disable_split_kv)), ctypes.byref(info)))
    if page_table.shape[1] != info.max_pages:
        raise ValueError(f"page_table must have {info.max_pages} columns (ceil(max_seqlen_k / "
                         f"{page_size}))")
    buf = torch.empty(int(info.bytes), dtype=torch.uint8, device=page_table.device)
    _check(lib.msa_paged_decode_plan(_ptr(seqused_k), ctypes.byref(info), _ptr(buf), buf.numel(),
                                     _stream(stream)))
    return DecodePlan(info, buf)


def msa_paged_decode_run(plan: DecodePlan, q, k_pool, v_pool, page_table, seqused_k, *,
                         causal: bool = True, softmax_scale: float = 0.0, o=None, lse=None,
                         return_temperature_lse: bool = False,
                         lse_temperature_scale: Optional[float] = None, lse_temperature=None,
                         temperature_fast_path: bool = True, stream=None):
    """Run the dense paged decode on a plan. Returns (O bf16 [B,Sq,Hq,D], LSE [B,Hq,Sq]),
    plus the temperature-scaled LSE when asked. Q, K and V all bf16, or all fp8
    e4m3fn (torch.float8_e4m3fn, or uint8 holding its bytes): the pages' fp8 decode,
    probabilities rounded to e4m3 before the P V product."""
    lib = load_library()
    dtype = _kv_dtype(k_pool, v_pool, ("k_pool", "v_pool"))
    if dtype == MSA_DTYPE_BF16:
        _dev(q, "q", torch.bfloat16)
    elif not (isinstance(q, torch.Tensor) and q.is_cuda and q.is_contiguous()
              and q.dtype in (getattr(torch, "float8_e4m3fn", None), torch.uint8)):
        raise TypeError("the fp8 decode takes q as contiguous fp8 e4m3fn on the GPU, like "
                        "k_pool / v_pool")
    _dev(page_table, "page_table", torch.int32)
    _dev(seqused_k, "seqused_k", torch.int32)
    info = plan.info
    B, Sq, Hq, D = q.shape
    if (B, Sq, Hq) != (info.batch, info.seqlen_q, info.num_qo_heads):
        raise ValueError("q does not match the plan")
    if o is None:
        o = torch.empty((B, Sq, Hq, D), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, Hq, Sq), dtype=torch.float32, device=q.device)
    _dev(o, "o", torch.bfloat16), _dev(lse, "lse", torch.float32)
    temp, lse_t, alias = _temperature(lse, return_temperature_lse, lse_temperature_scale,
                                      lse_temperature, temperature_fast_path)
    rc = lib.msa_paged_decode_run(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(page_table),
                                  _ptr(seqused_k), ctypes.byref(info), _ptr(plan.buffer),
                                  plan.buffer.numel(), k_pool.shape[0], dtype, int(bool(causal)),
                                  float(softmax_scale), _ptr(o), _ptr(lse), temp, _ptr(lse_t),
                                  _stream(stream))
    _check(rc)
    if return_temperature_lse:
        return o, lse, (lse if alias else lse_t)
    return o, lse
