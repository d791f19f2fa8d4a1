"""GPU checks that a caller's k2q CSR is not trusted by the kv-centric path.

A forward given a prebuilt CSR reads it as data: an entry whose query lies outside its
row's sequence, or whose slot lies outside [0, topk), is skipped, and a row_ptr that is
not non-decreasing within [0, rows * topk] voids the kv-centric pass. In each case the
call returns MSA_OK with every access inside the tensors. The outputs of the (query,
KV head) rows whose partials the corrupted entries would have written are unspecified;
every other row must be bit-identical to the call with the intact CSR (each (query,
slot) partial has exactly one writer, and a row's arithmetic does not depend on which
rows share its work item). The row_ptr cases check that the call returns and that an
intact call afterwards still gives the same bits.
"""
import pytest
import torch

import workloads as wl
import oracle
from parity_util import run_contiguous, say, to_dev

pytestmark = pytest.mark.gpu

KV = 2


def contiguous_case(B, Sq, Skv, Hkv, qpk, topk, seed):
    w = wl.Workload("csr", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=True,
                    mode=wl.MODE_CAUSAL, seed=seed)
    return w, wl.make_inputs(w)


def run_varlen(inp, csr):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k", "cu_seqlens_q", "cu_seqlens_k")}
    o, lse = msa.msa_sparse_fwd_varlen(t["q"], t["k"], t["v"], t["q2k"], t["cu_seqlens_q"],
                                       t["cu_seqlens_k"], *csr, causal=True, path=KV)
    torch.cuda.synchronize()
    return o, lse


def _intact(inp, nblk):
    import block_sparse_attention_top_amd as msa
    csr = msa.msa_build_k2q_csr(to_dev(inp["q2k"]), nblk)
    torch.cuda.synchronize()
    return csr


def _rows_equal_except(o, lse, o_ref, lse_ref, Sq, qpk, skip):
    """O [B,Sq,Hq,D] and LSE [B,Hq,Sq] equal bit for bit outside the (global query,
    KV head) pairs in skip."""
    keep_o = torch.ones(o.shape[:3], dtype=torch.bool)
    keep_l = torch.ones(lse.shape, dtype=torch.bool)
    for gq, hkv in skip:
        b, q = divmod(gq, Sq)
        keep_o[b, q, hkv * qpk:(hkv + 1) * qpk] = False
        keep_l[b, hkv * qpk:(hkv + 1) * qpk, q] = False
    oc, orf = o.cpu(), o_ref.cpu()
    lc, lrf = lse.cpu(), lse_ref.cpu()
    assert torch.equal(oc[keep_o], orf[keep_o])
    assert torch.equal(lc[keep_l], lrf[keep_l])
    return int(keep_o.sum()), int(keep_o.numel())


def test_contiguous_bad_entries_skipped():
    w, inp = contiguous_case(2, 300, 2048, 2, 8, 8, seed=9)
    rp, qi, sl = _intact(inp, w.Skv // w.blk)
    o_ref, l_ref = run_contiguous(inp, True, KV, csr=(rp, qi, sl))
    n0, n1 = int(rp[0, -1]), int(rp[1, -1])
    qi2, sl2 = qi.clone(), sl.clone()
    e = [n0 // 7, (3 * n0) // 5, n1 // 3, n1 - 1]
    skip = {(int(qi[0, e[0]]), 0), (int(qi[0, e[1]]), 0), (int(qi[1, e[2]]), 1),
            (int(qi[1, e[3]]), 1)}
    qi2[0, e[0]] = 2**31 - 1       # past the last query
    qi2[0, e[1]] = -3              # negative
    sl2[1, e[2]] = w.topk          # slot past the index row
    sl2[1, e[3]] = -1
    say(f"[csr] contiguous, bad entries at {e}: rows {sorted(skip)} unspecified")
    o, lse = run_contiguous(inp, True, KV, csr=(rp, qi2, sl2))
    kept, total = _rows_equal_except(o, lse, o_ref, l_ref, w.Sq, w.qpk, skip)
    say(f"[csr] {kept} of {total} (query, head) rows bit-identical")


@pytest.mark.parametrize("kind", ["descent", "negative", "past_cap"])
def test_contiguous_bad_row_ptr_voids_pass(kind):
    w, inp = contiguous_case(2, 300, 2048, 2, 8, 8, seed=10)
    rp, qi, sl = _intact(inp, w.Skv // w.blk)
    o_ref, l_ref = run_contiguous(inp, True, KV, csr=(rp, qi, sl))
    rp2 = rp.clone()
    nrows = rp.shape[1] - 1
    if kind == "descent":
        r = nrows // 2
        rp2[1, r], rp2[1, r + 1] = rp[1, r + 1] + 5, rp[1, r]
    elif kind == "negative":
        rp2[0, 0] = -5
    else:
        rp2[1, nrows] = w.B * w.Sq * w.topk + 1
    say(f"[csr] contiguous, row_ptr {kind}")
    run_contiguous(inp, True, KV, csr=(rp2, qi, sl))  # returns; outputs unspecified
    o, lse = run_contiguous(inp, True, KV, csr=(rp, qi, sl))
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)


def test_varlen_entry_from_other_sequence_skipped():
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens = [100, 257, 31], [700, 1024, 129]
    inp = wl.make_varlen_inputs(4, q_lens, k_lens, 2, 4, 4, wl.MODE_CAUSAL)
    total_rows = oracle.varlen_total_rows(inp["cu_seqlens_k"])
    cuq, cuk = to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"])
    rp, qi, sl = msa.msa_build_k2q_csr_varlen(to_dev(inp["q2k"]), cuq, cuk, sum(k_lens),
                                              total_rows)
    torch.cuda.synchronize()
    o_ref, l_ref = run_varlen(inp, (rp, qi, sl, total_rows))
    cu = inp["cu_seqlens_q"]
    qi_h = qi.cpu().numpy()
    n = int(rp[0, -1])
    # entries of sequence 1 pointed at a query of sequence 0, and one of sequence 0 at
    # a query of sequence 2: both in range globally, outside their rows' sequences
    e1 = next(i for i in range(n) if cu[1] <= qi_h[0, i] < cu[2])
    e0 = next(i for i in range(n) if cu[0] <= qi_h[0, i] < cu[1])
    skip = {(int(qi_h[0, e1]), 0), (int(qi_h[0, e0]), 0)}
    qi2 = qi.clone()
    qi2[0, e1] = int(cu[0]) + 3
    qi2[0, e0] = int(cu[2]) + 1
    say(f"[csr] varlen, entries {e1}, {e0} moved to other sequences")
    o, lse = run_varlen(inp, (rp, qi2, sl, total_rows))
    # varlen layouts: O [total_q, Hq, D], LSE [total_q, Hq]
    qpk = inp["q"].shape[1] // inp["k"].shape[1]
    keep = torch.ones(o.shape[:2], dtype=torch.bool)
    for gq, hkv in skip:
        keep[gq, hkv * qpk:(hkv + 1) * qpk] = False
    assert torch.equal(o.cpu()[keep], o_ref.cpu()[keep])
    assert torch.equal(lse.cpu()[keep], l_ref.cpu()[keep])
    say(f"[csr] {int(keep.sum())} of {keep.numel()} (query, head) rows bit-identical")
