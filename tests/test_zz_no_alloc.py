"""The no-allocation paged entry point (msa_paged_sparse_fwd_noalloc) against the
entry point with a caller workspace (msa_paged_sparse_fwd), through the C ABI.

Both run the same kernels, so the outputs must agree bit for bit; the second call of
each pair uses a smaller input than the first, so that anything the scratch array
keeps from the previous call would show. The small case is also checked against the
oracle at the parity tolerances (O max-abs 2e-2, LSE 1e-3)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import full_compare, say, to_dev

pytestmark = pytest.mark.gpu

PQ, PK, PD = 1, 2, 3  # paged q-centric, kv-centric and decode (union of blocks) paths


def paged_inputs(B, Sq, Skv, Hkv, qpk, topk, trims, seed):
    w = wl.Workload("paged", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seed=seed)
    inp = wl.make_inputs(w, q2k=np.zeros((1,), np.int32))
    inp["seqused_k"] = np.array([Skv - t for t in trims], dtype=np.int32)
    inp["q2k"] = np.concatenate([wl.q2k_table(seed + b, w.mode, 1, Hkv, Sq,
                                              int(inp["seqused_k"][b]), 128, topk)
                                 for b in range(B)], 0)
    return w, inp


def both(inp, splits, path, **kw):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    args = (t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"], t["q2k"])
    B, Sq, Hq, D = t["q"].shape
    Hkv = t["k_pool"].shape[1]
    nbytes = msa.msa_paged_sparse_fwd_workspace_size(B, Sq, Hq, Hkv, D, t["q2k"].shape[-1], 128,
                                                     t["page_table"].shape[1], splits, path)
    assert 0 < nbytes <= msa.MSA_NOALLOC_SCRATCH_BYTES  # the scratch array is in use
    ws = torch.full((nbytes,), 255, dtype=torch.uint8, device="cuda")  # NaN bytes
    ref = msa.msa_paged_sparse_fwd(*args, causal=True, num_splits=splits, path=path,
                                   workspace=ws, **kw)
    got = msa.msa_paged_sparse_fwd_noalloc(*args, causal=True, num_splits=splits, path=path, **kw)
    torch.cuda.synchronize()
    return ref, got


CASES = [  # (B, Sq, Skv, Hkv, qpk, topk, trims)
    (32, 8, 16384, 4, 16, 16, [17] * 32),   # the decode batch shape at 16K keys
    (3, 4, 2048, 2, 8, 8, [5, 0, 700]),     # smaller: fewer rows, heads and splits
]


@pytest.mark.parametrize("path,splits", [(PQ, 4), (PD, 0), (PD, 3)])
def test_noalloc_matches_workspace_entry_point(path, splits):
    for i, (B, Sq, Skv, Hkv, qpk, topk, trims) in enumerate(CASES):
        say(f"[noalloc] path={path} splits={splits} call {i}: B={B} Sq={Sq} Skv={Skv} "
            f"Hkv={Hkv} qpk={qpk} topk={topk}")
        w, inp = paged_inputs(B, Sq, Skv, Hkv, qpk, topk, trims, seed=31 + i)
        (o1, l1), (o2, l2) = both(inp, splits, path)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "no-alloc output differs"
        if i == 1:
            o_ref, lse_ref = oracle.paged_sparse_attention(
                inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"], inp["seqused_k"],
                inp["q2k"], causal=True)
            say(f"[noalloc] oracle: {full_compare(o2, l2, o_ref, lse_ref, 'noalloc-small')}")


KV_CASES = [  # small enough for the kv-centric workspace to fit the scratch array
    (2, 64, 4096, 2, 8, 8, [0, 1000]),
    (1, 32, 2048, 1, 4, 4, [100]),
]


def test_noalloc_kv_centric_path():
    """The kv-centric path asked for explicitly: its CSR, work items and partials in the
    scratch array, two calls in a row, the second smaller."""
    for i, (B, Sq, Skv, Hkv, qpk, topk, trims) in enumerate(KV_CASES):
        say(f"[noalloc] path={PK} call {i}: B={B} Sq={Sq} Skv={Skv} Hkv={Hkv} qpk={qpk} "
            f"topk={topk}")
        w, inp = paged_inputs(B, Sq, Skv, Hkv, qpk, topk, trims, seed=51 + i)
        (o1, l1), (o2, l2) = both(inp, 0, PK)
        assert torch.equal(o1, o2) and torch.equal(l1, l2), "no-alloc output differs"


def test_noalloc_auto_never_takes_the_kv_path():
    """A paged prefill whose automatic path is the kv-centric one: through the no-alloc
    entry point, auto runs the q-centric kernel (one split, no scratch) instead."""
    import block_sparse_attention_top_amd as msa
    w, inp = paged_inputs(1, 2048, 16384, 2, 2, 16, [300], seed=60)
    assert msa.msa_paged_sparse_fwd_path(1, 2048, 2, 16, w.max_pages) == PK
    say("[noalloc] auto on a kv-centric-sized paged prefill")
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    args = (t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"], t["q2k"])
    ref = msa.msa_paged_sparse_fwd(*args, causal=True, path=PQ)
    got = msa.msa_paged_sparse_fwd_noalloc(*args, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(ref[0], got[0]) and torch.equal(ref[1], got[1])


def test_noalloc_temperature_lse():
    w, inp = paged_inputs(3, 4, 2048, 2, 8, 8, [5, 0, 700], seed=40)
    say("[noalloc] temperature-scaled LSE, path=1 splits=4")
    (o1, l1, t1), (o2, l2, t2) = both(inp, 4, PQ, return_temperature_lse=True,
                                      lse_temperature_scale=2.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(t1, t2)


def test_noalloc_rejects_more_than_its_scratch():
    """Split partials beyond MSA_NOALLOC_SCRATCH_BYTES are refused before any launch:
    the outputs keep what they held."""
    import block_sparse_attention_top_amd as msa
    w, inp = paged_inputs(32, 8, 16384, 4, 16, 16, [17] * 32, seed=31)
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    need = msa.msa_paged_sparse_fwd_workspace_size(32, 8, 64, 4, 128, 16, 128, 128, 16, PQ)
    assert need > msa.MSA_NOALLOC_SCRATCH_BYTES
    o = torch.full((32, 8, 64, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((32, 64, 8), 5.0, dtype=torch.float32, device="cuda")
    with pytest.raises(msa.MsaValueError):
        msa.msa_paged_sparse_fwd_noalloc(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                         t["seqused_k"], t["q2k"], causal=True, num_splits=16,
                                         path=PQ, o=o, lse=lse)
    torch.cuda.synchronize()
    assert bool((o == 3.0).all()) and bool((lse == 5.0).all())
