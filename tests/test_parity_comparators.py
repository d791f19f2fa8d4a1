"""The parity comparators reject wrong answers (CPU).

The GPU parity tests judge the HIP path through parity_util's compare, full_compare,
sampled_compare and check_lse_t. Here the oracle's own result, rounded to bf16 the way
the GPU returns O, must pass them; each planted error must be rejected: O off by more
than the tolerance in one element, two heads swapped, one LSE off by 2e-3, an empty row
given a finite LSE or a non-zero O, a NaN, a visible row reported empty, sampled rows
taken from the wrong places, and a temperature LSE past its bound.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import check_lse_t, compare, full_compare, sampled_compare


@pytest.fixture(scope="module")
def case():
    # Sq > Skv with the bottom-right causal limit: the first Sq - Skv rows see no key
    w = wl.Workload("cmp", B=2, Sq=300, Skv=256, Hkv=2, qpk=2, topk=2, causal=True,
                    mode=wl.MODE_CAUSAL, seed=21)
    inp = wl.make_inputs(w)
    o_ref, lse_ref, lse_t_ref = oracle.sparse_attention(
        inp["q"], inp["k"], inp["v"], inp["q2k"], causal=True, temperature=2.0)
    assert np.isneginf(lse_ref).any() and np.isfinite(lse_ref).any()
    return w, o_ref, lse_ref, lse_t_ref


def as_gpu(o_ref, lse_ref):
    """What the GPU returns for an exact answer: O rounded to bf16, LSE in fp32."""
    o = torch.from_numpy(o_ref).to(torch.bfloat16)
    lse = torch.from_numpy(lse_ref).to(torch.float32)
    return o, lse


def visible(lse_ref):
    b, h, q = np.argwhere(np.isfinite(lse_ref))[len(np.argwhere(np.isfinite(lse_ref))) // 2]
    return int(b), int(h), int(q)


def empty(lse_ref):
    b, h, q = np.argwhere(np.isneginf(lse_ref))[0]
    return int(b), int(h), int(q)


def test_exact_answer_passes(case):
    w, o_ref, lse_ref, lse_t_ref = case
    o, lse = as_gpu(o_ref, lse_ref)
    full_compare(o, lse, o_ref, lse_ref, "exact")
    rows = np.array([0, 1, w.Sq - 1, w.Sq, 2 * w.Sq - 1])
    b, s = rows // w.Sq, rows % w.Sq
    sampled_compare(o, lse, o_ref[b, s], lse_ref[b, :, s], rows, w.Sq, "exact sampled")
    check_lse_t(lse_t_ref.astype(np.float32), lse_t_ref, "exact temperature")


def _rejected(o, lse, o_ref, lse_ref):
    with pytest.raises(AssertionError):
        full_compare(o, lse, o_ref, lse_ref, "planted")


def test_o_element_off(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = visible(lse_ref)
    o[b, q, h, 5] += 0.03
    _rejected(o, lse, o_ref, lse_ref)


def test_heads_swapped(case):
    w, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, q = 0, w.Sq - 1  # the last query sees every key of its blocks
    o[b, q, [0, 1]] = o[b, q, [1, 0]]
    assert np.abs(o_ref[b, q, 0] - o_ref[b, q, 1]).max() > 0.05
    _rejected(o, lse, o_ref, lse_ref)


def test_lse_off(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = visible(lse_ref)
    lse[b, h, q] += 2e-3
    _rejected(o, lse, o_ref, lse_ref)


def test_empty_row_given_finite_lse(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = empty(lse_ref)
    lse[b, h, q] = 0.0
    _rejected(o, lse, o_ref, lse_ref)


def test_empty_row_nonzero_o(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = empty(lse_ref)
    o[b, q, h, 0] = 1e-6
    _rejected(o, lse, o_ref, lse_ref)


def test_nan_in_o(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = visible(lse_ref)
    o[b, q, h, 0] = float("nan")
    _rejected(o, lse, o_ref, lse_ref)


def test_visible_row_reported_empty(case):
    _, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    b, h, q = visible(lse_ref)
    lse[b, h, q] = -float("inf")
    o[b, q, h] = 0
    _rejected(o, lse, o_ref, lse_ref)


def test_sampled_rows_misaligned(case):
    w, o_ref, lse_ref, _ = case
    o, lse = as_gpu(o_ref, lse_ref)
    rows = np.array([w.Sq - 2, w.Sq - 1, 2 * w.Sq - 1])
    b, s = rows // w.Sq, rows % w.Sq
    with pytest.raises(AssertionError):  # oracle rows in the wrong order
        sampled_compare(o, lse, o_ref[b, s][::-1], lse_ref[b, :, s][::-1], rows, w.Sq, "planted")


def test_temperature_lse_past_bound(case):
    _, _, _, lse_t_ref = case
    lt = lse_t_ref.copy()
    b, h, q = visible(lse_t_ref)
    lt[b, h, q] += 1e-3 + 1e-3 * abs(lse_t_ref[b, h, q]) + 1e-4
    with pytest.raises(AssertionError):
        check_lse_t(lt, lse_t_ref, "planted")


def test_compare_rejects_row_shift(case):
    """compare on [rows, Hq, D] / [rows, Hq] arrays: the GPU rows one place off."""
    _, o_ref, lse_ref, _ = case
    og = o_ref.reshape(-1, o_ref.shape[2], o_ref.shape[3])
    lg = lse_ref.transpose(0, 2, 1).reshape(-1, lse_ref.shape[1])
    fin = np.isfinite(lg).all(axis=1)
    og, lg = og[fin], lg[fin]
    with pytest.raises(AssertionError):
        compare(np.roll(og, 1, axis=0), np.roll(lg, 1, axis=0), og, lg, "planted")
