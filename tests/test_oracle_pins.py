"""Pins of the CPU oracle against facts fixed by the mathematics and the pages.

The oracle (oracle/msa_oracle.c) writes out the golden definition of the page
"MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py"
(`sparse_attention_ref`). None of these checks retypes that code: each one
compares the oracle with an independent route to the same number --
dense attention from torch's scaled_dot_product_attention (fp64, CPU) where
the selection covers every block, closed forms, invariances the definition
implies, and the logsumexp merge identity.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads as wl

D = 128
BLK = 128


def rand_inputs(seed, B, Sq, Skv, Hq, Hkv):
    q = wl.normal_bf16(seed, wl.STREAM_Q, (B, Sq, Hq, D))
    k = wl.normal_bf16(seed, wl.STREAM_K, (B, Skv, Hkv, D))
    v = wl.normal_bf16(seed, wl.STREAM_V, (B, Skv, Hkv, D))
    return q, k, v


def full_selection(seed, B, Hkv, Sq, nblk):
    """Every row selects all nblk blocks, each row in its own random order."""
    return wl.q2k_table(seed, wl.MODE_PERM, B, Hkv, Sq, nblk * BLK, BLK, nblk)


def dense_torch(q, k, v, allowed, scale):
    """Dense attention in fp64 via torch; allowed [B,Hq,Sq,Skv] bool.

    Returns O [B,Sq,Hq,D], LSE [B,Hq,Sq]; rows with no allowed key are left NaN
    in O (torch's convention) and -inf in LSE.
    """
    qf = torch.from_numpy(wl.bf16_to_f32(q).astype(np.float64)).permute(0, 2, 1, 3)
    kf = torch.from_numpy(wl.bf16_to_f32(k).astype(np.float64)).permute(0, 2, 1, 3)
    vf = torch.from_numpy(wl.bf16_to_f32(v).astype(np.float64)).permute(0, 2, 1, 3)
    rep = qf.shape[1] // kf.shape[1]
    kf = kf.repeat_interleave(rep, dim=1).contiguous()
    vf = vf.repeat_interleave(rep, dim=1).contiguous()
    am = torch.from_numpy(allowed)
    o = F.scaled_dot_product_attention(qf, kf, vf, attn_mask=am, scale=scale)
    s = torch.matmul(qf, kf.transpose(-1, -2).contiguous()) * scale
    lse = torch.logsumexp(s.masked_fill(~am, float("-inf")), dim=-1)
    return o.permute(0, 2, 1, 3).numpy(), lse.numpy()


def bottom_right_allowed(B, Hq, Sq, Skv, causal):
    qi = np.arange(Sq)[:, None]
    kj = np.arange(Skv)[None, :]
    m = (kj <= qi + (Skv - Sq)) if causal else np.ones((Sq, Skv), dtype=bool)
    return np.ascontiguousarray(np.broadcast_to(m, (B, Hq, Sq, Skv)))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sq,Skv,Hkv,qpk", [(256, 256, 2, 2), (256, 256, 1, 16), (64, 256, 2, 4),
                                            (384, 256, 1, 2)])
def test_dense_when_every_block_selected(causal, Sq, Skv, Hkv, qpk):
    """topk == nblk with each row a permutation of all blocks is dense attention
    with the bottom-right causal mask (and rows left of the diagonal empty when Sq > Skv)."""
    B, Hq, nblk = 1, Hkv * qpk, Skv // BLK
    q, k, v = rand_inputs(7, B, Sq, Skv, Hq, Hkv)
    q2k = full_selection(8, B, Hkv, Sq, nblk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=causal)
    allowed = bottom_right_allowed(B, Hq, Sq, Skv, causal)
    o_ref, lse_ref = dense_torch(q, k, v, allowed, D ** -0.5)
    has = allowed.any(-1)  # [B,Hq,Sq]
    has_q = has.transpose(0, 2, 1)  # [B,Sq,Hq]
    np.testing.assert_allclose(o[has_q], o_ref[has_q], rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse[has], lse_ref[has], rtol=0, atol=1e-12)
    # empty rows (Sq > Skv, causal): O = 0 exactly and LSE = -inf
    assert np.all(o[~has_q] == 0.0)
    assert np.all(np.isneginf(lse[~has]))
    if causal and Sq > Skv:
        assert (~has).any()


def test_gqa_head_map_and_scale():
    """Head h reads KV head h // qpk; a non-default softmax scale is honoured."""
    B, Sq, Skv, Hkv, qpk = 2, 128, 256, 2, 4
    Hq, nblk = Hkv * qpk, Skv // BLK
    q, k, v = rand_inputs(11, B, Sq, Skv, Hq, Hkv)
    q2k = full_selection(12, B, Hkv, Sq, nblk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=True, softmax_scale=0.3)
    o_ref, lse_ref = dense_torch(q, k, v, bottom_right_allowed(B, Hq, Sq, Skv, True), 0.3)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def block_allowed(q2k, B, Hkv, qpk, Sq, Skv, causal, kvlen=None):
    """Token mask of a selection: union of the valid selected blocks, restricted by
    kvlen and the bottom-right limit (used with torch's dense attention)."""
    nblk = Skv // BLK
    kvlen = np.full(B, Skv) if kvlen is None else np.asarray(kvlen)
    sel = np.zeros((B, Hkv, Sq, nblk), dtype=bool)
    bb, hh, qq, tt = np.nonzero((q2k >= 0) & (q2k < nblk))
    sel[bb, hh, qq, q2k[bb, hh, qq, tt]] = True
    tok = np.repeat(sel, BLK, axis=-1)
    tok = np.repeat(tok, qpk, axis=1)
    kj = np.arange(Skv)
    for b in range(B):
        tok[b] &= (kj < kvlen[b])[None, None, :]
        if causal:
            lim = np.arange(Sq) + kvlen[b] - Sq
            tok[b] &= (kj[None, :] <= lim[:, None])[None]
    return tok


@pytest.mark.parametrize("causal", [False, True])
def test_sparse_selection_matches_masked_dense(causal):
    """A random top-k selection equals dense attention with the selection's token mask."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 256, 1024, 2, 2, 3
    q, k, v = rand_inputs(21, B, Sq, Skv, Hkv * qpk, Hkv)
    mode = wl.MODE_CAUSAL if causal else wl.MODE_PERM
    q2k = wl.q2k_table(22, mode, B, Hkv, Sq, Skv, BLK, topk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=causal)
    allowed = block_allowed(q2k, B, Hkv, qpk, Sq, Skv, causal)
    o_ref, lse_ref = dense_torch(q, k, v, allowed, D ** -0.5)
    has = allowed.any(-1)
    assert has.all()
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_slot_order_duplicates_and_invalid_ids_do_not_matter():
    """Set semantics: permuting a row, repeating an id, or adding ids outside
    [0, nblk) (or -1) changes nothing, bit for bit."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 1024, 2, 2, 4
    q, k, v = rand_inputs(31, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(32, wl.MODE_PERM, B, Hkv, Sq, Skv, BLK, topk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=False)
    perm = np.ascontiguousarray(q2k[..., ::-1])
    o2, lse2 = oracle.sparse_attention(q, k, v, perm, causal=False)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    nblk = Skv // BLK
    padded = np.concatenate([q2k, np.full_like(q2k, -1)[..., :2], q2k[..., :1],
                             np.full_like(q2k, nblk)[..., :1], np.full_like(q2k, -7)[..., :1]], -1)
    o3, lse3 = oracle.sparse_attention(q, k, v, np.ascontiguousarray(padded), causal=False)
    assert np.array_equal(o, o3) and np.array_equal(lse, lse3)


def test_minus_one_drops_exactly_that_block():
    """Replacing one slot by -1 equals dense attention without that block."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 512, 1, 4, 3
    q, k, v = rand_inputs(41, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(42, wl.MODE_PERM, B, Hkv, Sq, Skv, BLK, topk)
    dropped = q2k.copy()
    dropped[..., 1] = -1
    o, lse = oracle.sparse_attention(q, k, v, dropped, causal=False)
    allowed = block_allowed(dropped, B, Hkv, qpk, Sq, Skv, False)
    o_ref, lse_ref = dense_torch(q, k, v, allowed, D ** -0.5)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)
    o_full, _ = oracle.sparse_attention(q, k, v, q2k, causal=False)
    assert not np.allclose(o, o_full)


def test_single_key_closed_form():
    """Causal, Sq == Skv: query 0 with block 0 selected sees only key 0, so
    O = V_0 exactly and LSE = scale * <Q_0, K_0>."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 256, 256, 2, 2, 2
    q, k, v = rand_inputs(51, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(52, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    assert np.all(q2k[0, :, 0, 0] == 0)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=True)
    qf, kf, vf = (wl.bf16_to_f32(x).astype(np.float64) for x in (q, k, v))
    for h in range(Hkv * qpk):
        hk = h // qpk
        assert np.array_equal(o[0, 0, h], vf[0, 0, hk])
        expect = D ** -0.5 * float(np.dot(qf[0, 0, h], kf[0, 0, hk]))
        assert abs(lse[0, h, 0] - expect) < 1e-12


def test_zero_query_gives_mean_of_values_and_log_count():
    """Q = 0: all visible scores are 0, so O is the mean of the visible values and LSE = ln |J|."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 256, 1024, 2, 2, 3
    Hq = Hkv * qpk
    _, k, v = rand_inputs(61, B, Sq, Skv, Hq, Hkv)
    q = np.zeros((B, Sq, Hq, D), dtype=np.uint16)
    q2k = wl.q2k_table(62, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=True)
    vf = wl.bf16_to_f32(v).astype(np.float64)
    for qi in (0, 1, 127, 128, 200, 255):
        for h in range(Hq):
            hk = h // qpk
            lim = qi + Skv - Sq
            keys = sorted({s * BLK + r for s in q2k[0, hk, qi] if s >= 0 for r in range(BLK)
                           if s * BLK + r <= lim})
            assert abs(lse[0, h, qi] - math.log(len(keys))) < 1e-12
            np.testing.assert_allclose(o[0, qi, h], vf[0, keys, hk].mean(0), rtol=0, atol=1e-12)


def test_logsumexp_merge_of_disjoint_splits():
    """Attention over S1 u S2 equals the LSE-weighted merge of the parts; an
    empty part (0, -inf) is the identity of the merge."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 128, 1024, 2, 2, 4
    q, k, v = rand_inputs(71, B, Sq, Skv, Hkv * qpk, Hkv)
    q2k = wl.q2k_table(72, wl.MODE_PERM, B, Hkv, Sq, Skv, BLK, topk)
    s1, s2 = q2k.copy(), q2k.copy()
    s1[..., 2:] = -1
    s2[..., :2] = -1
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=False)
    o1, l1 = oracle.sparse_attention(q, k, v, s1, causal=False)
    o2, l2 = oracle.sparse_attention(q, k, v, s2, causal=False)
    L = np.logaddexp(l1, l2)
    w1 = np.exp(l1 - L).transpose(0, 2, 1)[..., None]
    w2 = np.exp(l2 - L).transpose(0, 2, 1)[..., None]
    np.testing.assert_allclose(L, lse, rtol=0, atol=1e-12)
    np.testing.assert_allclose(w1 * o1 + w2 * o2, o, rtol=0, atol=1e-12)
    empty = np.full_like(q2k, -1)
    oe, le = oracle.sparse_attention(q, k, v, empty, causal=False)
    assert np.all(oe == 0.0) and np.all(np.isneginf(le))
    Le = np.logaddexp(le, lse)
    assert np.array_equal(Le, lse)


def pack_paged(k, page_table, page_size, num_pages, fill):
    """Dense [B,Skv,H,D] -> pool [num_pages,H,page,D] through a page table; unused
    pool rows get `fill`."""
    B, Skv, H, Dd = k.shape
    pool = np.full((num_pages, H, page_size, Dd), fill, dtype=k.dtype)
    for b in range(B):
        for s in range((Skv + page_size - 1) // page_size):
            n = min(page_size, Skv - s * page_size)
            pool[page_table[b, s], :, :n] = k[b, s * page_size:s * page_size + n].transpose(1, 0, 2)
    return pool


@pytest.mark.parametrize("causal", [False, True])
def test_paged_equals_contiguous_and_ignores_tail(causal):
    """Reading K/V through a shuffled page table equals reading them in place, and
    the contents of keys at or past seqused_k never matter."""
    B, Sq, Skv, Hkv, qpk, topk = 3, 16, 1024, 2, 4, 3
    Hq, max_pages = Hkv * qpk, Skv // BLK
    q, k, v = rand_inputs(81, B, Sq, Skv, Hq, Hkv)
    seqused = np.array([1024 - 17, 700, 129], dtype=np.int32)
    mode = wl.MODE_CAUSAL if causal else wl.MODE_PERM
    # causal rows follow each sequence's seqused_k; non-causal rows may select
    # blocks wholly past seqused_k, which must then contribute nothing
    lens = seqused if causal else np.full(B, Skv)
    q2k = np.concatenate([wl.q2k_table(82 + b, mode, 1, Hkv, Sq, int(lens[b]), BLK, topk)
                          for b in range(B)], 0)
    pt = wl.permutation(83, 1, B * max_pages).reshape(B, max_pages)
    kp = pack_paged(k, pt, BLK, B * max_pages, 0)
    vp = pack_paged(v, pt, BLK, B * max_pages, 0)
    o_c, l_c = oracle.sparse_attention(q, k, v, q2k, causal=causal, seqused_k=seqused)
    o_p, l_p = oracle.paged_sparse_attention(q, kp, vp, pt, seqused, q2k, causal=causal)
    assert np.array_equal(o_c, o_p) and np.array_equal(l_c, l_p)
    # poison everything at or past seqused with large finite values
    k2, v2 = k.copy(), v.copy()
    for b in range(B):
        k2[b, seqused[b]:] = 0x4780  # bf16 65536.0
        v2[b, seqused[b]:] = 0xC780  # bf16 -65536.0
    o_t, l_t = oracle.sparse_attention(q, k2, v2, q2k, causal=causal, seqused_k=seqused)
    assert np.array_equal(o_c, o_t) and np.array_equal(l_c, l_t)
    kp2 = pack_paged(k2, pt, BLK, B * max_pages, 0x4780)
    vp2 = pack_paged(v2, pt, BLK, B * max_pages, 0xC780)
    o_t2, l_t2 = oracle.paged_sparse_attention(q, kp2, vp2, pt, seqused, q2k, causal=causal)
    assert np.array_equal(o_c, o_t2) and np.array_equal(l_c, l_t2)
    # and seqused itself is honoured: with the true tail visible the result changes
    o_full, _ = oracle.sparse_attention(q, k2, v2, q2k, causal=causal)
    assert not np.array_equal(o_full, o_c)


def test_paged_seqused_matches_dense_mask():
    """Paged attention with a trimmed seqused_k equals dense attention over the
    selection's tokens below seqused_k with the limit q + seqused_k - Sq."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 8, 1024, 1, 4, 4
    Hq, max_pages = Hkv * qpk, Skv // BLK
    q, k, v = rand_inputs(91, B, Sq, Skv, Hq, Hkv)
    seqused = np.array([1024 - 17, 300], dtype=np.int32)
    q2k = np.concatenate([wl.q2k_table(92 + b, wl.MODE_CAUSAL, 1, Hkv, Sq, int(seqused[b]), BLK,
                                       topk) for b in range(B)], 0)
    pt = wl.permutation(93, 1, B * max_pages).reshape(B, max_pages)
    kp, vp = pack_paged(k, pt, BLK, B * max_pages, 0), pack_paged(v, pt, BLK, B * max_pages, 0)
    o, lse = oracle.paged_sparse_attention(q, kp, vp, pt, seqused, q2k, causal=True)
    allowed = block_allowed(q2k, B, Hkv, qpk, Sq, Skv, True, kvlen=seqused)
    o_ref, lse_ref = dense_torch(q, k, v, allowed, D ** -0.5)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_out_of_range_page_contributes_nothing():
    """A page-table entry outside [0, num_pages) behaves as an unselected block."""
    B, Sq, Skv, Hkv, qpk, topk = 1, 8, 512, 1, 2, 4
    Hq, max_pages = Hkv * qpk, Skv // BLK
    q, k, v = rand_inputs(95, B, Sq, Skv, Hq, Hkv)
    seqused = np.array([Skv], dtype=np.int32)
    q2k = np.tile(np.arange(4, dtype=np.int32), (B, Hkv, Sq, 1))
    pt = np.arange(max_pages, dtype=np.int32).reshape(1, max_pages)
    kp, vp = pack_paged(k, pt, BLK, max_pages, 0), pack_paged(v, pt, BLK, max_pages, 0)
    bad = pt.copy()
    bad[0, 2] = max_pages + 5
    o_bad, l_bad = oracle.paged_sparse_attention(q, kp, vp, bad, seqused, q2k, causal=False)
    dropped = q2k.copy()
    dropped[..., 2] = -1
    o_ref, l_ref = oracle.paged_sparse_attention(q, kp, vp, pt, seqused, dropped, causal=False)
    assert np.array_equal(o_bad, o_ref) and np.array_equal(l_bad, l_ref)


def test_row_subset_equals_full_run():
    """Evaluating a list of rows gives the same bits as the full run."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 64, 512, 2, 2, 3
    Hq = Hkv * qpk
    q, k, v = rand_inputs(97, B, Sq, Skv, Hq, Hkv)
    q2k = wl.q2k_table(98, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, BLK, topk)
    o, lse = oracle.sparse_attention(q, k, v, q2k, causal=True)
    rows = np.array([0, 5, 63, 64, 100, 127], dtype=np.int64)
    o_r, l_r = oracle.sparse_attention(q, k, v, q2k, causal=True, rows=rows)
    b, s = rows // Sq, rows % Sq
    assert np.array_equal(o_r, o[b, s]) and np.array_equal(l_r, lse[b, :, s])
