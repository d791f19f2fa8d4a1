"""Shared helpers of the GPU parity tests: upload seeded host inputs, run the
HIP path through the C ABI, and compare with the oracle.

Tolerances (fixed for bf16 inputs): O max-abs <= 2e-2 against the fp64 oracle;
LSE abs <= 1e-3 where the oracle's LSE is finite; rows the oracle finds empty
(LSE = -inf) must be empty on the GPU too, with O exactly 0; CSR bit-exact.
"""
from __future__ import annotations

import sys

import numpy as np
import torch

O_ATOL = 2e-2
LSE_ATOL = 1e-3


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(x: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    if x.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def bf16_dev_to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def compare(o_gpu: np.ndarray, lse_gpu: np.ndarray, o_ref: np.ndarray, lse_ref: np.ndarray,
            label: str = "") -> dict:
    """o_* [..., Hq, D] rows aligned with lse_* [..., Hq]; returns error stats and asserts."""
    fin = np.isfinite(lse_ref)
    assert not np.isnan(o_gpu).any(), f"{label}: NaN in O"
    assert np.array_equal(np.isneginf(lse_gpu), ~fin), f"{label}: empty-row mask differs"
    empty = ~fin
    if empty.any():
        assert np.all(o_gpu[empty] == 0.0), f"{label}: empty rows not zero"
    o_err = float(np.abs(o_gpu - o_ref).max()) if o_ref.size else 0.0
    lse_err = float(np.abs(lse_gpu[fin] - lse_ref[fin]).max()) if fin.any() else 0.0
    assert o_err <= O_ATOL, f"{label}: O max-abs error {o_err}"
    assert lse_err <= LSE_ATOL, f"{label}: LSE abs error {lse_err}"
    return {"o_err": o_err, "lse_err": lse_err}


def check_lse_t(lt_gpu, lt_ref, label):
    """Temperature-scaled LSE against the oracle: the test page's rule for it,
    |d| <= 1e-3 + 1e-3 |ref| on finite entries, with identical empty-row masks."""
    lt_gpu = np.asarray(lt_gpu, dtype=np.float64)
    fin = np.isfinite(lt_ref)
    assert np.array_equal(np.isneginf(lt_gpu), ~fin), f"{label}: empty-row mask differs"
    err = np.abs(lt_gpu[fin] - lt_ref[fin])
    bound = 1e-3 + 1e-3 * np.abs(lt_ref[fin])
    assert np.all(err <= bound), f"{label}: temperature LSE error {err.max()}"
    return float(err.max()) if err.size else 0.0


def run_contiguous(inp: dict, causal: bool, path: int, softmax_scale: float = 0.0, csr=None):
    import block_sparse_attention_top_amd as msa
    q, k, v, q2k = (to_dev(inp[n]) for n in ("q", "k", "v", "q2k"))
    args = () if csr is None else tuple(csr)
    o, lse = msa.msa_sparse_fwd(q, k, v, q2k, *args, causal=causal, path=path,
                                softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return o, lse


def run_paged(inp: dict, causal: bool, num_splits: int = 0, softmax_scale: float = 0.0,
              path: int = 0):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    o, lse = msa.msa_paged_sparse_fwd(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                      t["seqused_k"], t["q2k"], causal=causal,
                                      num_splits=num_splits, softmax_scale=softmax_scale,
                                      path=path)
    torch.cuda.synchronize()
    return o, lse


def full_compare(o, lse, o_ref, lse_ref, label=""):
    """GPU O [B,Sq,Hq,D] / LSE [B,Hq,Sq] against the full oracle output."""
    og = bf16_dev_to_f64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    return compare(og, lg.transpose(0, 2, 1), o_ref, lse_ref.transpose(0, 2, 1), label)


def sampled_compare(o, lse, o_ref_rows, lse_ref_rows, rows, Sq, label=""):
    """Compare GPU outputs at global rows b*Sq+q against oracle rows [n,Hq,D] / [n,Hq]."""
    rows_t = torch.as_tensor(rows, device=o.device)
    b, s = rows_t // Sq, rows_t % Sq
    og = o[b, s].float().cpu().numpy().astype(np.float64)
    lg = lse[b, :, s].cpu().numpy().astype(np.float64)
    return compare(og, lg, o_ref_rows, lse_ref_rows, label)


def sample_rows(B: int, Sq: int, n: int, seed: int = 0) -> np.ndarray:
    """First, last and evenly spread plus random global rows (sorted, unique)."""
    rng = np.random.default_rng(seed)
    tot = B * Sq
    picks = {0, tot - 1, Sq - 1, min(tot - 1, 127), min(tot - 1, 128)}
    picks.update(np.linspace(0, tot - 1, n // 2).astype(np.int64).tolist())
    picks.update(rng.integers(0, tot, n - len(picks)).tolist() if n > len(picks) else [])
    return np.array(sorted(picks), dtype=np.int64)
