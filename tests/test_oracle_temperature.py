"""Pins of the oracle's temperature-scaled LSE: the log-sum-exp of the same masked
scores divided by a temperature T (`lse_temperature_scale` of `sparse_attention_ref`
on the test page; the interface page describes it as the LSE of logits scaled by
softmax_scale / lse_temperature_scale). Each check uses a route independent of the
oracle's own loop: torch's logsumexp over an explicitly masked dense score matrix,
closed forms, the scale identity and the T -> 0 limit."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from test_oracle_pins import BLK, D, block_allowed, rand_inputs


def masked_scores_torch(q, k, allowed, scale):
    """fp64 scores [B,Hq,Sq,Skv] with -inf where the selection does not allow a key."""
    qf = torch.from_numpy(wl.bf16_to_f32(q).astype(np.float64)).permute(0, 2, 1, 3)
    kf = torch.from_numpy(wl.bf16_to_f32(k).astype(np.float64)).permute(0, 2, 1, 3)
    kf = kf.repeat_interleave(qf.shape[1] // kf.shape[1], dim=1).contiguous()
    s = torch.matmul(qf, kf.transpose(-1, -2).contiguous()) * scale
    return s.masked_fill(~torch.from_numpy(allowed), float("-inf"))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("temp", [0.5, 1.7, 3.0])
def test_temperature_lse_matches_masked_logsumexp(causal, temp):
    B, Sq, Skv, Hkv, qpk, topk = 2, 192, 768, 2, 4, 3
    q, k, v = rand_inputs(41, B, Sq, Skv, Hkv * qpk, Hkv)
    mode = wl.MODE_CAUSAL if causal else wl.MODE_PERM
    q2k = wl.q2k_table(42, mode, B, Hkv, Sq, Skv, BLK, topk)
    o, lse, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=causal, temperature=temp)
    allowed = block_allowed(q2k, B, Hkv, qpk, Sq, Skv, causal)
    s = masked_scores_torch(q, k, allowed, D ** -0.5)
    ref = torch.logsumexp(s / temp, dim=-1).numpy()  # [B,Hq,Sq]
    np.testing.assert_allclose(lse_t, ref, rtol=0, atol=1e-11)
    # the ordinary outputs do not change when the temperature LSE is asked for
    o2, lse2 = oracle.sparse_attention(q, k, v, q2k, causal=causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_unit_temperature_is_the_lse():
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 512, 2, 2, 2
    q, k, v = rand_inputs(43, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(44, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    _, lse, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=True, temperature=1.0)
    assert np.array_equal(lse, lse_t)


def test_scale_identity():
    """Logits scaled by scale / T: doubling the scale and taking T = 2 gives the plain
    LSE at the original scale, bit for bit (both factors are powers of two)."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 512, 1, 8, 3
    q, k, v = rand_inputs(45, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(46, wl.MODE_PERM, B, Hkv, Sq, Skv, BLK, topk)
    _, lse = oracle.sparse_attention(q, k, v, q2k, causal=False)
    _, _, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=False,
                                          softmax_scale=2 * D ** -0.5, temperature=2.0)
    assert np.array_equal(lse, lse_t)


def test_zero_queries_give_log_key_count():
    """Q = 0: every score is 0, so the temperature LSE is ln|J| for any T."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 256, 1024, 1, 2, 3
    q, k, v = rand_inputs(47, B, Sq, Skv, Hkv * qpk, Hkv)
    q[:] = 0
    q2k = wl.q2k_table(48, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    _, _, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=True, temperature=0.37)
    allowed = block_allowed(q2k, B, Hkv, qpk, Sq, Skv, True)
    count = allowed.sum(-1)
    np.testing.assert_allclose(lse_t, np.log(count), rtol=0, atol=1e-12)


def test_small_temperature_tends_to_the_max_score():
    """T * LSE_T lies in [max_j s_j, max_j s_j + T ln|J|]."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 512, 1, 4, 2
    q, k, v = rand_inputs(49, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(50, wl.MODE_PERM, B, Hkv, Sq, Skv, BLK, topk)
    temp = 1e-3
    _, _, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=False, temperature=temp)
    allowed = block_allowed(q2k, B, Hkv, qpk, Sq, Skv, False)
    s = masked_scores_torch(q, k, allowed, D ** -0.5)
    smax = s.max(-1).values.numpy()
    lo, hi = smax, smax + temp * np.log(allowed.sum(-1))
    assert np.all(temp * lse_t >= lo - 1e-12) and np.all(temp * lse_t <= hi + 1e-12)


def test_empty_rows_are_minus_infinity():
    """Sq > Skv with the causal rule leaves the first rows without keys."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 384, 256, 1, 2, 2
    q, k, v = rand_inputs(51, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(52, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    _, lse, lse_t = oracle.sparse_attention(q, k, v, q2k, causal=True, temperature=2.5)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lse_t)) and np.isneginf(lse_t).any()


def test_paged_and_varlen_agree_with_contiguous():
    """The temperature LSE goes through the paged and varlen entry points unchanged:
    paged (shuffled pages) and per-sequence varlen equal the contiguous oracle, bit for bit."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 64, 512, 2, 2, 3
    w = wl.Workload("t", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seed=53)
    inp = wl.make_inputs(w)
    _, _, lt_paged = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                                   inp["page_table"], inp["seqused_k"],
                                                   inp["q2k"], causal=True, temperature=1.9)
    # contiguous copy of the pool through the page table
    pool_k, pool_v, pt = inp["k_pool"], inp["v_pool"], inp["page_table"]
    k = pool_k[pt].transpose(0, 1, 3, 2, 4).reshape(B, Skv, Hkv, D)
    v = pool_v[pt].transpose(0, 1, 3, 2, 4).reshape(B, Skv, Hkv, D)
    _, _, lt = oracle.sparse_attention(inp["q"], k, v, inp["q2k"], causal=True, temperature=1.9)
    assert np.array_equal(lt_paged, lt)
    cu_q = np.arange(B + 1, dtype=np.int32) * Sq
    cu_k = np.arange(B + 1, dtype=np.int32) * Skv
    q2k_v = np.ascontiguousarray(inp["q2k"].transpose(1, 0, 2, 3).reshape(Hkv, B * Sq, topk))
    _, _, lt_v = oracle.sparse_attention_varlen(inp["q"].reshape(B * Sq, -1, D),
                                                k.reshape(B * Skv, Hkv, D),
                                                v.reshape(B * Skv, Hkv, D), q2k_v, cu_q, cu_k,
                                                causal=True, temperature=1.9)
    assert np.array_equal(lt_v, lt.transpose(0, 2, 1).reshape(B * Sq, -1))
