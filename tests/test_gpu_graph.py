"""The library's calls captured in a HIP graph (through torch.cuda.graph) and replayed.

The library launches only kernels on the caller's stream: no allocation, no
synchronisation and no memset nodes (scratch memory is cleared by fill kernels), so its
calls can be captured. Each case captures one call with every output, workspace and plan
buffer given, then replays the graph three times. Between replays the program does its
own eager work (another library call on other inputs, a torch fill of the graph's
outputs) and synchronises; every replay must reproduce the eager call's O and LSE bit
for bit (each path is deterministic: the kv-centric kernel decides its rescale per row,
so the order-free CSR's grouping does not change a row's bits).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu

Q, KV = 1, 2


def capture(fn):
    s = torch.cuda.Stream()  # default priority
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(2):
            fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, refs, eager_other, label):
    for rep in range(3):
        for t in outs:  # the program's own eager work between replays
            t.fill_(float("nan") if t.dtype == torch.float32 else 7.0)
        eager_other()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, r in zip(outs, refs):
            assert torch.equal(t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32),
                               r.view(torch.int16) if r.dtype == torch.bfloat16 else r.view(torch.int32)), \
                f"{label}: replay {rep} differs from the eager call"
        say(f"[graph] {label}: replay {rep} bit-identical")


def contiguous(seed, Sq, Hkv, qpk, topk):
    w = wl.Workload("g", B=1, Sq=Sq, Skv=Sq, Hkv=Hkv, qpk=qpk, topk=topk, causal=True,
                    mode=wl.MODE_CAUSAL, seed=seed)
    inp = wl.make_inputs(w)
    return w, {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k")}


@pytest.mark.parametrize("path", [KV, Q])
def test_contiguous_forward_in_graph(path):
    import block_sparse_attention_top_amd as msa
    w, t = contiguous(61, 2048, 2, 8, 8)
    _, t2 = contiguous(62, 1024, 2, 8, 8)
    nbytes = msa.msa_sparse_fwd_workspace_size(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.D, w.topk,
                                               w.blk, path)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    fn = lambda: msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=True, path=path,
                                    o=o, lse=lse, workspace=ws)
    fn()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    say(f"[graph] contiguous path {path}: capturing")
    g = capture(fn)
    other = lambda: msa.msa_sparse_fwd(t2["q"], t2["k"], t2["v"], t2["q2k"], causal=True,
                                       path=path)
    replay_and_check(g, [o, lse], [o_ref, l_ref], other, f"contiguous path {path}")


def paged(seed, B, Sq, Skv, trims):
    w = wl.Workload("g", B=B, Sq=Sq, Skv=Skv, Hkv=4, qpk=16, topk=16, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seed=seed)
    inp = wl.make_inputs(w, q2k=np.zeros((1,), np.int32))
    inp["seqused_k"] = np.array([Skv - x for x in trims], dtype=np.int32)
    inp["q2k"] = np.concatenate([wl.q2k_table(seed + b, w.mode, 1, w.Hkv, Sq,
                                              int(inp["seqused_k"][b]), 128, w.topk)
                                 for b in range(B)], 0)
    return w, {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k",
                                           "q2k")}


def test_paged_noalloc_in_graph():
    """The entry point meant for capture: split partials in the library's own scratch."""
    import block_sparse_attention_top_amd as msa
    w, t = paged(63, 4, 8, 8192, [0, 300, 5000, 8191])
    _, t2 = paged(64, 2, 8, 4096, [0, 17])
    args = (t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"], t["q2k"])
    o = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    fn = lambda: msa.msa_paged_sparse_fwd_noalloc(*args, causal=True, num_splits=4, path=Q,
                                                  o=o, lse=lse)
    fn()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    say("[graph] paged no-alloc, 4 splits: capturing")
    g = capture(fn)
    other = lambda: msa.msa_paged_sparse_fwd_noalloc(
        t2["q"], t2["k_pool"], t2["v_pool"], t2["page_table"], t2["seqused_k"], t2["q2k"],
        causal=True, num_splits=3, path=Q)
    replay_and_check(g, [o, lse], [o_ref, l_ref], other, "paged no-alloc")


def test_dense_decode_run_in_graph():
    """A dense decode plan built eagerly, its run captured."""
    import block_sparse_attention_top_amd as msa
    w, t = paged(65, 6, 8, 4096, [0, 100, 4000, 4095, 1, 2048])
    plan = msa.msa_paged_decode_plan(t["page_table"], t["seqused_k"], seqlen_q=w.Sq,
                                     max_seqlen_k=w.Skv, num_qo_heads=w.Hq,
                                     num_kv_heads=w.Hkv, fixed_split_size=4)
    o = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    fn = lambda: msa.msa_paged_decode_run(plan, t["q"], t["k_pool"], t["v_pool"],
                                          t["page_table"], t["seqused_k"], causal=True,
                                          o=o, lse=lse)
    fn()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    say("[graph] dense decode run: capturing")
    g = capture(fn)
    _, t2 = paged(66, 2, 8, 2048, [0, 5])
    plan2 = msa.msa_paged_decode_plan(t2["page_table"], t2["seqused_k"], seqlen_q=8,
                                      max_seqlen_k=2048, num_qo_heads=64, num_kv_heads=4)
    other = lambda: msa.msa_paged_decode_run(plan2, t2["q"], t2["k_pool"], t2["v_pool"],
                                             t2["page_table"], t2["seqused_k"], causal=True)
    replay_and_check(g, [o, lse], [o_ref, l_ref], other, "dense decode run")


def test_paged_kv_centric_in_graph():
    """The paged prefill on the kv-centric path (CSR, items, partials and combine in the
    caller's workspace), captured and replayed."""
    import block_sparse_attention_top_amd as msa
    w, t = paged(67, 2, 1024, 4096, [0, 700])
    args = (t["q"], t["k_pool"], t["v_pool"], t["page_table"], t["seqused_k"], t["q2k"])
    nbytes = msa.msa_paged_sparse_fwd_workspace_size(w.B, w.Sq, w.Hq, w.Hkv, w.D, w.topk, w.blk,
                                                     w.max_pages, 0, KV)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((w.B, w.Sq, w.Hq, w.D), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.B, w.Hq, w.Sq), dtype=torch.float32, device="cuda")
    fn = lambda: msa.msa_paged_sparse_fwd(*args, causal=True, path=KV, o=o, lse=lse,
                                          workspace=ws)
    fn()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    say("[graph] paged kv-centric: capturing")
    g = capture(fn)
    _, t2 = paged(68, 1, 512, 2048, [100])
    other = lambda: msa.msa_paged_sparse_fwd(
        t2["q"], t2["k_pool"], t2["v_pool"], t2["page_table"], t2["seqused_k"], t2["q2k"],
        causal=True, path=KV)
    replay_and_check(g, [o, lse], [o_ref, l_ref], other, "paged kv-centric")


def test_paged_varlen_kv_centric_in_graph():
    """A ragged batch through the paged varlen entry point on the kv-centric path (its
    per-sequence tables, CSR, items, partials and combine), captured and replayed."""
    import block_sparse_attention_top_amd as msa
    inp = wl.make_varlen_inputs(69, [300, 0, 700], [1000, 500, 2000], 2, 8, 8, wl.MODE_CAUSAL)
    B, mp = 3, 16
    k_lens = np.diff(inp["cu_seqlens_k"])
    pool_k = np.zeros((B * mp, 2, 128, 128), dtype=np.uint16)
    pool_v = np.zeros_like(pool_k)
    pt = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    for b in range(B):
        for s in range((int(k_lens[b]) + 127) // 128):
            lo = int(inp["cu_seqlens_k"][b]) + 128 * s
            hi = min(int(inp["cu_seqlens_k"][b + 1]), lo + 128)
            pool_k[pt[b, s], :, :hi - lo] = inp["k"][lo:hi].transpose(1, 0, 2)
            pool_v[pt[b, s], :, :hi - lo] = inp["v"][lo:hi].transpose(1, 0, 2)
    t = {n: to_dev(x) for n, x in dict(q=inp["q"], kp=pool_k, vp=pool_v, pt=pt,
                                        su=k_lens.astype(np.int32), cu=inp["cu_seqlens_q"],
                                        q2k=inp["q2k"]).items()}
    total_q = int(inp["cu_seqlens_q"][-1])
    nbytes = msa.msa_paged_sparse_fwd_varlen_workspace_size(B, total_q, 16, 2, 128, 8, 128, mp,
                                                            0, KV)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    o = torch.empty((total_q, 16, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((total_q, 16), dtype=torch.float32, device="cuda")
    fn = lambda: msa.msa_paged_sparse_fwd_varlen(t["q"], t["kp"], t["vp"], t["pt"], t["su"],
                                                 t["cu"], t["q2k"], causal=True, path=KV, o=o,
                                                 lse=lse, workspace=ws)
    fn()
    torch.cuda.synchronize()
    o_ref, l_ref = o.clone(), lse.clone()
    say("[graph] paged varlen kv-centric: capturing")
    g = capture(fn)
    w2, t2 = paged(70, 1, 256, 2048, [0])
    other = lambda: msa.msa_paged_sparse_fwd(
        t2["q"], t2["k_pool"], t2["v_pool"], t2["page_table"], t2["seqused_k"], t2["q2k"],
        causal=True, path=KV)
    replay_and_check(g, [o, lse], [o_ref, l_ref], other, "paged varlen kv-centric")
