"""Top-k block-sparse GQA attention forward for MI355X (gfx950).

A thin ctypes binding over libmsa.so (C ABI in include/msa.h). Functions keep
the C names; they only marshal torch tensors (device memory) and the current
HIP stream into the C call and allocate outputs / workspaces with torch.
Every step of the computation runs in the library's HIP kernels; there is no
fallback: if libmsa.so is missing or the GPU is absent the calls raise.
"""
from __future__ import annotations

from ._ffi import (MSA_DTYPE_BF16, MSA_DTYPE_FP8_E4M3, MSA_PATH_AUTO, MSA_PATH_DECODE,
                   MSA_PATH_KVCENTRIC, MSA_PATH_QCENTRIC, MSA_PATH_TILE,
                   MsaError, MsaNotSupportedError, MsaValueError, lib_path, load_library,
                   msa_build_k2q_csr, msa_build_k2q_csr_workspace_size, msa_last_error,
                   msa_paged_sparse_fwd, msa_paged_sparse_fwd_path, msa_paged_sparse_fwd_splits,
                   msa_paged_sparse_fwd_noalloc, MSA_NOALLOC_SCRATCH_BYTES,
                   msa_paged_sparse_fwd_varlen, msa_paged_sparse_fwd_varlen_path,
                   msa_paged_sparse_fwd_varlen_workspace_size, msa_paged_sparse_fwd_varlen_splits,
                   msa_paged_sparse_fwd_workspace_size, msa_set_profiling_events, msa_sparse_fwd,
                   msa_sparse_fwd_path, msa_sparse_fwd_workspace_size, msa_sparse_fwd_varlen,
                   msa_sparse_fwd_varlen_path, msa_sparse_fwd_varlen_workspace_size,
                   msa_build_k2q_csr_varlen, msa_build_k2q_csr_varlen_workspace_size, msa_version,
                   DecodePlan, MsaDecodePlan, msa_paged_decode_plan, msa_paged_decode_run)

__all__ = [
    "MSA_PATH_AUTO", "MSA_PATH_QCENTRIC", "MSA_PATH_KVCENTRIC", "MSA_PATH_DECODE",
    "MSA_PATH_TILE", "MSA_DTYPE_BF16", "MSA_DTYPE_FP8_E4M3", "MsaError",
    "MsaValueError", "MsaNotSupportedError", "lib_path", "load_library", "msa_sparse_fwd",
    "msa_sparse_fwd_path", "msa_sparse_fwd_workspace_size", "msa_build_k2q_csr",
    "msa_build_k2q_csr_workspace_size", "msa_paged_sparse_fwd", "msa_paged_sparse_fwd_path",
    "msa_paged_sparse_fwd_splits", "msa_paged_sparse_fwd_workspace_size", "msa_last_error",
    "msa_paged_sparse_fwd_noalloc", "MSA_NOALLOC_SCRATCH_BYTES",
    "msa_paged_sparse_fwd_varlen", "msa_paged_sparse_fwd_varlen_path",
    "msa_paged_sparse_fwd_varlen_workspace_size", "msa_paged_sparse_fwd_varlen_splits",
    "msa_set_profiling_events", "msa_version", "msa_sparse_fwd_varlen",
    "msa_sparse_fwd_varlen_path", "msa_sparse_fwd_varlen_workspace_size",
    "msa_build_k2q_csr_varlen", "msa_build_k2q_csr_varlen_workspace_size",
    "DecodePlan", "MsaDecodePlan", "msa_paged_decode_plan", "msa_paged_decode_run",
]
