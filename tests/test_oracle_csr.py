"""Pins of the oracle's kv-block -> query CSR (page "MSA interface.py",
`build_k2q_csr`; its test on the page "test_sparse_atten.py" checks it bit-exact).

Brute force on tiny tables plus the invariants any correct inversion obeys.
"""
import numpy as np
import pytest

import oracle
import workloads as wl


def brute_force_csr(q2k, nblk):
    """Dictionary inversion: row (b, s) -> list of (b*Sq+q, t) in (q, t) order."""
    B, Hkv, Sq, topk = q2k.shape
    out = []
    for h in range(Hkv):
        rows = {(b, s): [] for b in range(B) for s in range(nblk)}
        for b in range(B):
            for q in range(Sq):
                for t in range(topk):
                    s = int(q2k[b, h, q, t])
                    if 0 <= s < nblk:
                        rows[(b, s)].append((b * Sq + q, t))
        out.append([rows[(b, s)] for b in range(B) for s in range(nblk)])
    return out


@pytest.mark.parametrize("mode", [wl.MODE_PERM, wl.MODE_SINK, wl.MODE_CAUSAL])
@pytest.mark.parametrize("B,Hkv,Sq,Skv,topk", [(1, 1, 64, 512, 4), (3, 2, 50, 1024, 3),
                                               (2, 2, 300, 256, 2)])
def test_csr_matches_brute_force(mode, B, Hkv, Sq, Skv, topk):
    nblk = Skv // 128
    q2k = wl.q2k_table(5, mode, B, Hkv, Sq, Skv, 128, topk)
    # sprinkle -1 and out-of-range ids: both are unused slots
    rng = np.random.default_rng(0)
    m = rng.random(q2k.shape) < 0.1
    q2k[m] = -1
    m2 = rng.random(q2k.shape) < 0.03
    q2k[m2] = nblk + 3
    row_ptr, q_idx, slot = oracle.k2q_csr(q2k, nblk)
    ref = brute_force_csr(q2k, nblk)
    for h in range(Hkv):
        assert row_ptr[h, 0] == 0
        for r, entries in enumerate(ref[h]):
            lo, hi = row_ptr[h, r], row_ptr[h, r + 1]
            assert hi - lo == len(entries)
            assert list(zip(q_idx[h, lo:hi].tolist(), slot[h, lo:hi].tolist())) == entries


def test_csr_duplicate_ids_in_slot_order():
    """A block named twice in one index row gives that CSR row two entries of the query,
    in slot order: the CSR lists every valid (q, t) slot in ascending (q, t) order."""
    B, Hkv, Sq, Skv, topk = 2, 2, 60, 1024, 6
    nblk = Skv // 128
    q2k = wl.q2k_table(13, wl.MODE_PERM, B, Hkv, Sq, Skv, 128, topk)
    rng = np.random.default_rng(1)
    rows = rng.random((B, Hkv, Sq)) < 0.4
    for b, h, q in zip(*np.nonzero(rows)):
        t1, t2 = sorted(rng.choice(topk, size=2, replace=False))
        q2k[b, h, q, t2] = q2k[b, h, q, t1]
    row_ptr, q_idx, slot = oracle.k2q_csr(q2k, nblk)
    ref = brute_force_csr(q2k, nblk)
    repeats = 0
    for h in range(Hkv):
        for r, entries in enumerate(ref[h]):
            lo, hi = row_ptr[h, r], row_ptr[h, r + 1]
            got = list(zip(q_idx[h, lo:hi].tolist(), slot[h, lo:hi].tolist()))
            assert got == entries
            qs = [e[0] for e in entries]
            repeats += len(qs) - len(set(qs))
    assert repeats == int(rows.sum())  # every planted repeat shows up as a second entry


def test_csr_invariants_and_empty_rows():
    B, Hkv, Sq, Skv, topk = 2, 2, 200, 2048, 4
    nblk = Skv // 128
    q2k = wl.q2k_table(9, wl.MODE_CAUSAL, B, Hkv, Sq, Skv, 128, topk)
    # force block 3 of sequence 0 to be unused, as the pages' empty-tile test does
    q2k[0][q2k[0] == 3] = -1
    row_ptr, q_idx, slot = oracle.k2q_csr(q2k, nblk)
    valid = (q2k >= 0) & (q2k < nblk)
    for h in range(Hkv):
        rp = row_ptr[h]
        assert rp[0] == 0 and np.all(np.diff(rp) >= 0)
        assert rp[-1] == valid[:, h].sum()
        assert rp[3 + 1] - rp[3] == 0  # the emptied row
        nnz = rp[-1]
        # every entry points back at a slot holding its row's block
        for r in range(B * nblk):
            b, s = divmod(r, nblk)
            qs = q_idx[h, rp[r]:rp[r + 1]]
            ts = slot[h, rp[r]:rp[r + 1]]
            assert np.all(qs // Sq == b)
            assert np.all(q2k[b, h, qs % Sq, ts] == s)
            keys = (qs.astype(np.int64) * 64 + ts)
            assert np.all(np.diff(keys) > 0)  # ascending q, then t
        # the multiset of (q, t) is exactly the valid slots
        got = np.sort(q_idx[h, :nnz].astype(np.int64) * 64 + slot[h, :nnz])
        bb, qq, tt = np.nonzero(valid[:, h])
        want = np.sort((bb * Sq + qq).astype(np.int64) * 64 + tt)
        assert np.array_equal(got, want)
        assert np.all(q_idx[h, nnz:] == -1)
