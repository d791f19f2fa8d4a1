"""GPU parity of variable-length batches (packed Q/K/V with cu_seqlens): the HIP
q-centric and kv-centric paths and the varlen k2q CSR, through the C ABI,
against the CPU oracle on the same seeded ragged inputs. Tolerances and
comparison rules are in parity_util."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import bf16_dev_to_f64, compare, say, to_dev

pytestmark = pytest.mark.gpu

Q, KV = 1, 2


def run_varlen(inp, causal, path, csr=None, softmax_scale=0.0):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k", "cu_seqlens_q", "cu_seqlens_k")}
    extra = () if csr is None else tuple(csr)
    o, lse = msa.msa_sparse_fwd_varlen(t["q"], t["k"], t["v"], t["q2k"], t["cu_seqlens_q"],
                                       t["cu_seqlens_k"], *extra, causal=causal, path=path,
                                       softmax_scale=softmax_scale)
    torch.cuda.synchronize()
    return o, lse


def check_varlen(inp, causal, path, label, rows=None):
    say(f"[varlen] {label} path={path} q_lens={np.diff(inp['cu_seqlens_q']).tolist()} "
        f"k_lens={np.diff(inp['cu_seqlens_k']).tolist()} causal={causal}")
    o, lse = run_varlen(inp, causal, path)
    o_ref, lse_ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                                    causal=causal, rows=rows)
    og = bf16_dev_to_f64(o)
    lg = lse.cpu().numpy().astype(np.float64)
    if rows is not None:
        og, lg = og[rows], lg[rows]
    return compare(og, lg, o_ref, lse_ref, label), (o, lse)


@pytest.mark.parametrize("path", [Q, KV])
@pytest.mark.parametrize("qpk", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("topk", [8, 16])
def test_varlen_pages_grid(path, qpk, topk):
    """B = 3 ragged sequences, Hkv = 2, causal: the forward test grid of the test page
    (qhead_per_kv 1..16, topk 8 / 16), K lengths on and off block boundaries."""
    q_lens, k_lens = wl.varlen_lengths(17 + qpk, 3, 200, 1536, k_multiple=(qpk % 2 == 0))
    inp = wl.make_varlen_inputs(qpk * 100 + topk, q_lens, k_lens, 2, qpk, topk, wl.MODE_CAUSAL)
    check_varlen(inp, True, path, f"grid-qpk{qpk}-topk{topk}")


@pytest.mark.parametrize("path", [Q, KV])
@pytest.mark.parametrize("causal", [True, False])
def test_varlen_ragged_tails(path, causal):
    """Key lengths ending inside a block, queries longer than keys, one-token sequences."""
    q_lens, k_lens = [37, 1, 300, 129, 5], [300, 1, 200, 1000, 127]
    inp = wl.make_varlen_inputs(5, q_lens, k_lens, 2, 8, 4, wl.MODE_CAUSAL)
    check_varlen(inp, causal, path, f"tails-causal{int(causal)}")


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_empty_sequences(path):
    """A sequence with no queries, one with no keys (its rows are empty), ids past a
    sequence's own blocks (unused slots) and -1 rows."""
    q_lens, k_lens = [20, 0, 9, 33], [512, 384, 0, 250]
    inp = wl.make_varlen_inputs(9, q_lens, k_lens, 2, 4, 4, wl.MODE_CAUSAL)
    q2k = inp["q2k"]
    q2k[:, 20:29] = np.array([0, 1, 2, 3], np.int32)  # keyless sequence: every id is invalid
    q2k[0, 30, :] = -1
    q2k[1, 31, 0] = 2  # sequence 3 has 2 blocks: id 2 is unused
    inp["q2k"] = q2k
    _, (o, lse) = check_varlen(inp, True, path, "empty-seqs")
    assert torch.isneginf(lse[20:29]).all() and (o[20:29] == 0).all()


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_no_keys_at_all(path):
    """total_k == 0: every row is empty (O = 0, LSE = -inf); K/V are empty tensors."""
    import block_sparse_attention_top_amd as msa
    inp = wl.make_varlen_inputs(1, [4, 6], [0, 0], 1, 2, 4, wl.MODE_CAUSAL)
    o, lse = run_varlen(inp, True, path)
    assert torch.isneginf(lse).all() and (o == 0).all()
    assert msa.msa_sparse_fwd_varlen_path(2, 10, 0, 2, 1, 4) == Q
    assert msa.msa_sparse_fwd_varlen_workspace_size(2, 10, 0, 2, 1, 128, 4, 128, path) == 0


def test_varlen_matches_uniform_batch():
    """Equal lengths: the varlen result equals the uniform-batch one. The q-centric
    path runs the same per-row arithmetic, so bit for bit; the kv-centric path
    groups a row's entries into wave steps in CSR order, which the unordered
    internal CSR leaves open, so within the parity tolerances."""
    import block_sparse_attention_top_amd as msa
    B, Sq, Skv, Hkv, qpk, topk = 3, 160, 640, 2, 8, 4
    w = wl.Workload("eq", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=True,
                    mode=wl.MODE_CAUSAL, seed=12)
    inp = wl.make_inputs(w)
    q = to_dev(inp["q"]).reshape(B * Sq, Hkv * qpk, 128)
    k = to_dev(inp["k"]).reshape(B * Skv, Hkv, 128)
    v = to_dev(inp["v"]).reshape(B * Skv, Hkv, 128)
    q2k_b = to_dev(inp["q2k"])
    q2k_v = q2k_b.permute(1, 0, 2, 3).reshape(Hkv, B * Sq, topk).contiguous()
    cuq = torch.arange(0, B + 1, device="cuda", dtype=torch.int32) * Sq
    cuk = torch.arange(0, B + 1, device="cuda", dtype=torch.int32) * Skv
    for path in (Q, KV):
        say(f"[varlen] uniform-equivalence path={path}")
        ob, lb = msa.msa_sparse_fwd(to_dev(inp["q"]), to_dev(inp["k"]), to_dev(inp["v"]), q2k_b,
                                    causal=True, path=path)
        ov, lv = msa.msa_sparse_fwd_varlen(q, k, v, q2k_v, cuq, cuk, causal=True, path=path)
        torch.cuda.synchronize()
        ob = ob.reshape(B * Sq, -1, 128)
        lb = lb.permute(0, 2, 1).reshape(B * Sq, -1)
        if path == Q:
            assert torch.equal(ov.view(torch.int16), ob.view(torch.int16))
            assert torch.equal(lv, lb)
        else:
            compare(bf16_dev_to_f64(ov), lv.cpu().numpy().astype(np.float64), bf16_dev_to_f64(ob),
                    lb.cpu().numpy().astype(np.float64), "uniform-kv")


@pytest.mark.parametrize("seed,k_multiple", [(0, True), (1, False), (2, False)])
def test_varlen_csr_bit_exact(seed, k_multiple):
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens = wl.varlen_lengths(seed, 5, 300, 2000, k_multiple=k_multiple)
    q_lens[3] = 0
    inp = wl.make_varlen_inputs(seed, q_lens, k_lens, 2, 4, 8, wl.MODE_CAUSAL)
    rng = np.random.default_rng(seed)
    q2k = inp["q2k"]
    q2k[rng.random(q2k.shape) < 0.05] = -1
    q2k[rng.random(q2k.shape) < 0.02] = 99  # past every sequence's blocks
    total_rows = oracle.varlen_total_rows(inp["cu_seqlens_k"])
    say(f"[varlen] csr seed={seed} total_rows={total_rows}")
    rp, qi, sl = msa.msa_build_k2q_csr_varlen(to_dev(q2k), to_dev(inp["cu_seqlens_q"]),
                                              to_dev(inp["cu_seqlens_k"]), sum(k_lens), total_rows)
    torch.cuda.synchronize()
    rp_ref, qi_ref, sl_ref = oracle.k2q_csr_varlen(q2k, inp["cu_seqlens_q"], inp["cu_seqlens_k"])
    rp, qi, sl = rp.cpu().numpy(), qi.cpu().numpy(), sl.cpu().numpy()
    assert np.array_equal(rp, rp_ref)
    for h in range(q2k.shape[0]):
        n = rp_ref[h, -1]
        assert np.array_equal(qi[h, :n], qi_ref[h, :n])
        assert np.array_equal(sl[h, :n], sl_ref[h, :n])


def test_varlen_prebuilt_csr():
    """The kv-centric path fed the public (ordered) varlen CSR matches the oracle."""
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens = [100, 257, 31], [700, 1024, 129]
    inp = wl.make_varlen_inputs(4, q_lens, k_lens, 2, 4, 4, wl.MODE_CAUSAL)
    total_rows = oracle.varlen_total_rows(inp["cu_seqlens_k"])
    cuq, cuk = to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"])
    csr = msa.msa_build_k2q_csr_varlen(to_dev(inp["q2k"]), cuq, cuk, sum(k_lens), total_rows)
    say(f"[varlen] prebuilt csr total_rows={total_rows}")
    o, lse = run_varlen(inp, True, KV, csr=(*csr, total_rows))
    o_ref, lse_ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                                    causal=True)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "prebuilt")


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_prefill_mix_sampled(path):
    """A prefill-sized ragged batch (eight sequences, 45 056 tokens, Hkv 4, qpk 16,
    topk 16, causal) checked on sampled rows of every sequence."""
    q_lens = [16384, 8192, 8192, 4096, 4096, 2048, 1536, 512]
    k_lens = [16384, 8192, 8300, 4096, 4000, 2048, 1536, 700]
    inp = wl.make_varlen_inputs(21, q_lens, k_lens, 4, 16, 16, wl.MODE_CAUSAL)
    cu = inp["cu_seqlens_q"]
    rng = np.random.default_rng(3)
    rows = sorted({int(x) for b in range(len(q_lens)) for x in
                   [cu[b], cu[b + 1] - 1, *rng.integers(cu[b], cu[b + 1], 6)]})
    check_varlen(inp, True, path, "prefill-mix", rows=np.array(rows, dtype=np.int64))
