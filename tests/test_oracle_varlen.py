"""Pins for the variable-length oracle (packed Q/K/V with cu_seqlens) and its CSR.

The varlen definition is the batched one applied to each sequence (B = 1), with the
sequence's keys starting at cu_seqlens_k[b] and its block ids local to it. Pins:
per-sequence equality with the batched oracle (K padded to a block multiple, the
true length passed as seqused_k), a direct torch SDPA check with the selection's
token mask, brute-force CSR inversion, and equal-length varlen == batched CSR.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def per_sequence_batched(inp, q_lens, k_lens, Hkv, causal):
    """The batched oracle on each sequence alone; returns O [total_q,Hq,D], LSE [total_q,Hq]."""
    os_, ls = [], []
    g0 = k0 = 0
    for sq, sk in zip(q_lens, k_lens):
        if sq == 0:
            k0 += sk
            continue
        Hq, D = inp["q"].shape[1:]
        pad = max(128, -(-sk // 128) * 128)
        kb = np.zeros((1, pad, Hkv, D), np.uint16)
        vb = np.zeros((1, pad, Hkv, D), np.uint16)
        kb[0, :sk] = inp["k"][k0:k0 + sk]
        vb[0, :sk] = inp["v"][k0:k0 + sk]
        qb = inp["q"][g0:g0 + sq][None]
        q2k = inp["q2k"][:, g0:g0 + sq][None]
        # block ids >= ceil(sk/128) are unused slots in the varlen reading; the padded
        # batched run would accept ids < pad/128, so mask them the same way
        nb = -(-sk // 128)
        q2k = np.where(q2k < nb, q2k, -1).astype(np.int32)
        o, l = oracle.sparse_attention(qb, kb, vb, q2k, causal=causal,
                                       seqused_k=np.array([sk], np.int32))
        os_.append(o[0])
        ls.append(l[0].T)
        g0 += sq
        k0 += sk
    return np.concatenate(os_, 0), np.concatenate(ls, 0)


@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("k_multiple", [True, False])
def test_varlen_equals_per_sequence_batched(causal, k_multiple):
    q_lens, k_lens = wl.varlen_lengths(3, 5, 40, 640, k_multiple=k_multiple)
    mode = wl.MODE_CAUSAL if causal else wl.MODE_PERM
    topk = 4
    if not causal:  # PERM needs at least topk blocks per sequence
        k_lens = [max(k, topk * 128) for k in k_lens]
    inp = wl.make_varlen_inputs(11, q_lens, k_lens, 2, 4, topk, mode)
    o, l = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                          inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                          causal=causal)
    o_ref, l_ref = per_sequence_batched(inp, q_lens, k_lens, 2, causal)
    assert np.array_equal(o, o_ref)
    assert np.array_equal(l, l_ref)


def test_varlen_against_torch_sdpa():
    """Independent route: fp64 SDPA per sequence with the selection's token mask."""
    q_lens, k_lens = [7, 1, 12], [300, 128, 200]  # 300 and 200 end inside a block
    Hkv, qpk, topk = 2, 2, 2
    inp = wl.make_varlen_inputs(5, q_lens, k_lens, Hkv, qpk, topk, wl.MODE_CAUSAL)
    o, l = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                          inp["cu_seqlens_q"], inp["cu_seqlens_k"], causal=True)
    f = lambda x: torch.from_numpy(wl.bf16_to_f32(x)).double()
    g0 = k0 = 0
    for sq, sk in zip(q_lens, k_lens):
        q = f(inp["q"][g0:g0 + sq])            # [sq, Hq, D]
        k = f(inp["k"][k0:k0 + sk])
        v = f(inp["v"][k0:k0 + sk])
        for h in range(Hkv * qpk):
            hk = h // qpk
            mask = torch.zeros(sq, sk, dtype=torch.bool)
            for qq in range(sq):
                for s in inp["q2k"][hk, g0 + qq]:
                    if 0 <= s < -(-sk // 128):
                        mask[qq, s * 128:min(sk, s * 128 + 128)] = True
                mask[qq, qq + sk - sq + 1:] = False  # bottom-right causal
            sc = (q[:, h] @ k[:, hk].T) * (128 ** -0.5)
            sc = sc.masked_fill(~mask, float("-inf"))
            for qq in range(sq):
                if mask[qq].any():
                    p = torch.softmax(sc[qq], -1)
                    assert np.allclose(o[g0 + qq, h], (p @ v[:, hk]).numpy(), atol=1e-12)
                    assert abs(l[g0 + qq, h] - torch.logsumexp(sc[qq], -1).item()) < 1e-12
                else:
                    assert np.all(o[g0 + qq, h] == 0) and l[g0 + qq, h] == -np.inf
        g0 += sq
        k0 += sk


def test_varlen_empty_sequences_and_rows():
    """A sequence without keys gives empty rows; a sequence without queries is skipped."""
    q_lens, k_lens = [5, 0, 3], [256, 384, 0]
    inp = wl.make_varlen_inputs(2, q_lens, k_lens, 1, 8, 2, wl.MODE_CAUSAL)
    inp["q2k"][:, 5:8] = np.array([0, 1], np.int32)  # ids point at blocks that do not exist
    o, l = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                          inp["cu_seqlens_q"], inp["cu_seqlens_k"], causal=False)
    assert np.all(np.isneginf(l[5:8])) and np.all(o[5:8] == 0)
    assert np.all(np.isfinite(l[:5]))


def test_varlen_rows_subset():
    q_lens, k_lens = wl.varlen_lengths(8, 4, 30, 512)
    inp = wl.make_varlen_inputs(8, q_lens, k_lens, 2, 2, 3, wl.MODE_CAUSAL)
    args = (inp["q"], inp["k"], inp["v"], inp["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    o, l = oracle.sparse_attention_varlen(*args, causal=True)
    rows = np.array([0, 3, 29, 30, sum(q_lens) - 1])
    o2, l2 = oracle.sparse_attention_varlen(*args, causal=True, rows=rows)
    assert np.array_equal(o2, o[rows]) and np.array_equal(l2, l[rows])


def brute_csr_varlen(q2k, cu_q, cu_k, blk=128):
    Hkv, total_q, topk = q2k.shape
    B = len(cu_q) - 1
    nblk = [-(-(cu_k[b + 1] - cu_k[b]) // blk) for b in range(B)]
    base = np.concatenate([[0], np.cumsum(nblk)])
    rows = int(base[-1])
    out = []
    for h in range(Hkv):
        lists = {r: [] for r in range(rows)}
        for b in range(B):
            for g in range(cu_q[b], cu_q[b + 1]):
                for t in range(topk):
                    s = int(q2k[h, g, t])
                    if 0 <= s < nblk[b]:
                        lists[int(base[b]) + s].append((g, t))
        out.append(lists)
    return rows, out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_varlen_csr_brute_force(seed):
    q_lens, k_lens = wl.varlen_lengths(seed, 4, 50, 768, k_multiple=seed != 1)
    q_lens[2] = 0
    inp = wl.make_varlen_inputs(seed, q_lens, k_lens, 2, 4, 5, wl.MODE_CAUSAL)
    rng = np.random.default_rng(seed)
    q2k = inp["q2k"]
    q2k[rng.random(q2k.shape) < 0.05] = 99  # out of range for every sequence
    rp, qi, sl = oracle.k2q_csr_varlen(q2k, inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    rows, lists = brute_csr_varlen(q2k, inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    assert rp.shape == (2, rows + 1)
    for h in range(2):
        assert rp[h, 0] == 0
        for r in range(rows):
            ent = lists[h][r]
            assert rp[h, r + 1] - rp[h, r] == len(ent)
            seg = slice(rp[h, r], rp[h, r + 1])
            assert list(zip(qi[h, seg].tolist(), sl[h, seg].tolist())) == ent


def test_varlen_csr_equal_lengths_is_batched():
    B, Hkv, Sq, Skv, topk = 3, 2, 40, 512, 4
    inp = wl.make_varlen_inputs(4, [Sq] * B, [Skv] * B, Hkv, 2, topk, wl.MODE_CAUSAL)
    rp, qi, sl = oracle.k2q_csr_varlen(inp["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    batched = inp["q2k"].reshape(Hkv, B, Sq, topk).transpose(1, 0, 2, 3).copy()
    rp2, qi2, sl2 = oracle.k2q_csr(batched, Skv // 128)
    assert np.array_equal(rp, rp2) and np.array_equal(qi, qi2) and np.array_equal(sl, sl2)
