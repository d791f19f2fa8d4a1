"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the same
seeded inputs. Tolerances and comparison rules are in parity_util."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import (bf16_dev_to_f64, full_compare, run_contiguous, run_paged, sample_rows,
                         sampled_compare, say, to_dev)

pytestmark = pytest.mark.gpu

Q, KV, TILE = 1, 2, 4  # paths: q-centric, kv-centric, query-tile


def contiguous_case(B, Sq, Skv, Hkv, qpk, topk, causal, mode, seed=42):
    w = wl.Workload("case", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=causal,
                    mode=mode, seed=seed)
    return w, wl.make_inputs(w)


def tile_ok(qpk, topk):
    """Shapes the query-tile kernel takes: qpk 8 or 16, (256 / qpk) * topk <= 512."""
    return qpk in (8, 16) and (256 // qpk) * topk <= 512


def expect_not_supported(inp, causal, path):
    import block_sparse_attention_top_amd as msa
    with pytest.raises(msa.MsaNotSupportedError):
        run_contiguous(inp, causal, path)


def check_contiguous(w, inp, path, label, softmax_scale=0.0):
    say(f"[parity] {label} path={path} B={w.B} Sq={w.Sq} Skv={w.Skv} Hkv={w.Hkv} qpk={w.qpk} "
        f"topk={w.topk} causal={w.causal}")
    o, lse = run_contiguous(inp, w.causal, path, softmax_scale=softmax_scale)
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             causal=w.causal,
                                             softmax_scale=softmax_scale or None)
    return full_compare(o, lse, o_ref, lse_ref, label), (o, lse)


@pytest.mark.parametrize("path", [Q, KV, TILE])
@pytest.mark.parametrize("name,B,Sq,Skv,Hkv,qpk,topk,causal,mode", [
    ("c1-full", 1, 1024, 1024, 1, 2, 4, False, wl.MODE_PERM),
    ("c2-small", 1, 1152, 1152, 2, 16, 8, True, wl.MODE_CAUSAL),
    ("c3u-small", 1, 1024, 1024, 2, 16, 4, False, wl.MODE_PERM),
    ("c3s-small", 1, 1024, 1024, 2, 16, 4, False, wl.MODE_SINK),
    ("c4b-small", 1, 2048, 2048, 1, 2, 16, True, wl.MODE_CAUSAL),
    ("batch3", 3, 200, 512, 2, 4, 3, True, wl.MODE_CAUSAL),
    ("sq-gt-skv", 1, 400, 256, 1, 8, 2, True, wl.MODE_CAUSAL),
    ("sq-lt-skv", 2, 72, 1024, 2, 16, 5, True, wl.MODE_CAUSAL),
    ("topk1", 1, 256, 512, 1, 16, 1, False, wl.MODE_PERM),
    ("topk32", 1, 64, 4096, 1, 4, 32, False, wl.MODE_PERM),
])
def test_contiguous_small(path, name, B, Sq, Skv, Hkv, qpk, topk, causal, mode):
    w, inp = contiguous_case(B, Sq, Skv, Hkv, qpk, topk, causal, mode)
    if path == TILE and not tile_ok(qpk, topk):
        expect_not_supported(inp, causal, path)
        return
    check_contiguous(w, inp, path, name)


@pytest.mark.parametrize("path", [Q, KV])
@pytest.mark.parametrize("Hkv", [3, 5, 12, 16])
def test_kv_head_counts(path, Hkv):
    """KV head counts whose item streams do not line up with the heads: the kv-centric
    items are cut into 1, 2, 4 or 8 streams of equal key ranges, so 3, 5 and 12 heads
    put stream boundaries inside a head's query range, and 16 heads share streams."""
    w, inp = contiguous_case(2, 300, 1024, Hkv, 2, 4, True, wl.MODE_CAUSAL, seed=8 + Hkv)
    check_contiguous(w, inp, path, f"hkv{Hkv}")


@pytest.mark.parametrize("path", [Q, KV, TILE])
@pytest.mark.parametrize("qpk", [1, 2, 4, 8, 16])
def test_qhead_per_kv_sweep(path, qpk):
    w, inp = contiguous_case(2, 300, 640, 2, qpk, 3, True, wl.MODE_CAUSAL, seed=7)
    if path == TILE and not tile_ok(qpk, 3):
        expect_not_supported(inp, True, path)
        return
    check_contiguous(w, inp, path, f"qpk{qpk}")


@pytest.mark.parametrize("path", [Q, KV, TILE])
def test_unused_slots_invalid_ids_and_empty_blocks(path):
    """-1 rows, ids outside [0, nblk), a block nobody selects, and a custom scale."""
    w, inp = contiguous_case(1, 256, 1024, 2, 8, 4, False, wl.MODE_PERM, seed=3)
    q2k = inp["q2k"].copy()
    nblk = w.Skv // 128
    q2k[:, :, :17] = -1                     # rows with nothing selected
    q2k[:, :, 20:40, 1] = nblk + 5          # out-of-range ids
    q2k[:, :, 40:60, 2] = -3
    q2k[q2k == 5] = -1                      # block 5 selected by nobody: empty CSR row
    inp["q2k"] = q2k
    check_contiguous(w, inp, path, "edge-ids", softmax_scale=0.05)


@pytest.mark.parametrize("temp", [None, 0.5])
def test_kv_rescale_per_row_deterministic(temp):
    """Scores spread wide (Q scaled by 16, exact in bf16), so that the kv-centric kernel's
    lazy second-half rescale fires often. Each (query, head) row's result must depend
    on its own scores only: two calls with the library's own order-free CSR (its wave
    steps group rows differently from call to call) and one with the public ordered
    CSR agree bit for bit, and all match the oracle. V is scaled by 1/4 (exact): such
    peaked rows put O near a single V row, and this keeps |O| at the magnitudes the
    absolute O tolerance is stated for (bf16 partials and output round relative to |O|)."""
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous_case(1, 2048, 4096, 2, 16, 8, True, wl.MODE_CAUSAL, seed=91)

    def scaled(bits, f):
        x = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(f)
        return (x.view(np.uint32) >> 16).astype(np.uint16)

    inp = dict(inp)
    inp["q"] = scaled(inp["q"], 16)
    inp["v"] = scaled(inp["v"], 0.25)
    say(f"[rescale] kv path, Q x 16, T={temp}")
    q, k, v, q2k = (to_dev(inp[n]) for n in ("q", "k", "v", "q2k"))
    tk = {} if temp is None else dict(return_temperature_lse=True, lse_temperature_scale=temp)
    # the order-free CSR's grouping varies with the timing of its atomics, so several
    # calls give a grouping-dependent result more than one chance to show
    own = [msa.msa_sparse_fwd(q, k, v, q2k, causal=True, path=KV, **tk) for _ in range(4)]
    csr = msa.msa_build_k2q_csr(q2k, w.Skv // w.blk)
    ordered = msa.msa_sparse_fwd(q, k, v, q2k, *csr, causal=True, path=KV, **tk)
    torch.cuda.synchronize()
    r1 = own[0]
    for other in own[1:] + [ordered]:
        assert all(torch.equal(a, b) for a, b in zip(r1, other))
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             causal=True)
    full_compare(r1[0], r1[1], o_ref, lse_ref, "rescale")


@pytest.mark.parametrize("path", [Q, KV, TILE])
def test_deterministic(path):
    w, inp = contiguous_case(1, 512, 1024, 2, 16, 4, True, wl.MODE_CAUSAL, seed=5)
    o1, l1 = run_contiguous(inp, True, path)
    o2, l2 = run_contiguous(inp, True, path)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("other", [KV, TILE])
def test_paths_agree(other):
    w, inp = contiguous_case(1, 640, 1024, 2, 16, 8, True, wl.MODE_CAUSAL, seed=9)
    oq, lq = run_contiguous(inp, True, Q)
    ok, lk = run_contiguous(inp, True, other)
    assert (oq.float() - ok.float()).abs().max().item() <= 2e-2
    fin = torch.isfinite(lq)
    assert torch.equal(fin, torch.isfinite(lk))
    assert (lq[fin] - lk[fin]).abs().max().item() <= 1e-3


@pytest.mark.parametrize("B,Sq,Skv,Hkv,qpk,topk,causal", [
    (1, 200, 4096, 1, 16, 32, True),   # 16 x 32 = 512 index entries per tile, ragged tail
    (1, 100, 2048, 2, 8, 16, False),   # 32-query tiles, 512 entries
    (3, 77, 1024, 3, 16, 4, True),     # 9 (b, hkv) pairs: plain placement
    (2, 130, 640, 1, 8, 5, True),      # 2 pairs over XCD groups of 4, Sq > Skv
    (1, 16, 128, 1, 16, 1, True),      # one tile, one block
])
def test_tile_shapes(B, Sq, Skv, Hkv, qpk, topk, causal):
    w, inp = contiguous_case(B, Sq, Skv, Hkv, qpk, topk, causal,
                             wl.MODE_CAUSAL if causal else wl.MODE_PERM, seed=31)
    check_contiguous(w, inp, TILE, f"tile-B{B}-Sq{Sq}-qpk{qpk}-k{topk}")


def test_tile_rejects_large_index_sets():
    w, inp = contiguous_case(1, 64, 4096, 1, 8, 17, False, wl.MODE_PERM, seed=2)
    expect_not_supported(inp, False, TILE)


def test_tile_duplicate_ids_count_once():
    """The query-tile path takes each selected block once per row (set semantics,
    as the oracle): a row listing a block twice equals the row listing it once."""
    w, inp = contiguous_case(1, 256, 1024, 2, 16, 6, True, wl.MODE_CAUSAL, seed=12)
    q2k = inp["q2k"].copy()
    q2k[:, :, :, -1] = q2k[:, :, :, 0]
    check_contiguous(w, dict(inp, q2k=q2k), TILE, "tile-duplicates")


# ---------------------------------------------------------------------------
# CSR
# ---------------------------------------------------------------------------
def csr_gpu(q2k_np, nblk):
    import block_sparse_attention_top_amd as msa
    rp, qi, sl = msa.msa_build_k2q_csr(to_dev(q2k_np), nblk)
    torch.cuda.synchronize()
    return rp.cpu().numpy(), qi.cpu().numpy(), sl.cpu().numpy()


def assert_csr_equal(q2k_np, nblk, label):
    say(f"[csr] {label} shape={q2k_np.shape} nblk={nblk}")
    rp, qi, sl = csr_gpu(q2k_np, nblk)
    rp_o, qi_o, sl_o = oracle.k2q_csr(q2k_np, nblk)
    assert np.array_equal(rp, rp_o), f"{label}: row_ptr differs"
    for h in range(rp.shape[0]):
        nnz = rp_o[h, -1]
        assert np.array_equal(qi[h, :nnz], qi_o[h, :nnz]), f"{label}: q_idx differs (h={h})"
        assert np.array_equal(sl[h, :nnz], sl_o[h, :nnz]), f"{label}: slot differs (h={h})"


@pytest.mark.parametrize("B", [1, 3])
@pytest.mark.parametrize("topk", [4, 8, 16, 32])
@pytest.mark.parametrize("Sq,Skv", [(2048, 4096), (4096, 4096), (1024, 4096), (4096, 2048)])
def test_csr_bit_exact_causal(B, topk, Sq, Skv):
    q2k = wl.q2k_table(17, wl.MODE_CAUSAL, B, 2, Sq, Skv, 128, topk)
    assert_csr_equal(q2k, Skv // 128, f"causal B{B} k{topk}")


@pytest.mark.parametrize("mode", [wl.MODE_PERM, wl.MODE_SINK])
def test_csr_bit_exact_patterns_with_holes(mode):
    q2k = wl.q2k_table(19, mode, 2, 3, 3000, 8192, 128, 16)
    rng = np.random.default_rng(1)
    q2k[rng.random(q2k.shape) < 0.05] = -1
    q2k[rng.random(q2k.shape) < 0.01] = 64 + 7
    q2k[q2k == 9] = -1
    assert_csr_equal(q2k, 64, f"mode{mode}-holes")


@pytest.mark.parametrize("key", ["c2", "c4b"])
def test_csr_bit_exact_full_size(key):
    """The public (ordered) CSR at the full workload sizes: c4b has 3072 rows and 6.3M
    entries, c2 4 KV heads x 64 rows."""
    w = wl.WORKLOADS[key]
    q2k = wl.q2k_table(w.seed, w.mode, w.B, w.Hkv, w.Sq, w.Skv, w.blk, w.topk)
    assert_csr_equal(q2k, w.Skv // w.blk, f"{key} full size")


def test_csr_bit_exact_with_duplicate_ids():
    """A repeated id in a row gives two entries of that row, in slot order (the
    definition's (query, slot) order); the scatter ranks equal rows by lane."""
    q2k = wl.q2k_table(23, wl.MODE_PERM, 1, 2, 2000, 4096, 128, 16)
    q2k[..., 5] = q2k[..., 2]
    q2k[..., 11] = q2k[..., 2]
    assert_csr_equal(q2k, 32, "duplicates")


def test_csr_deterministic_and_prebuilt_csr_used():
    w, inp = contiguous_case(1, 700, 2048, 2, 8, 8, True, wl.MODE_CAUSAL, seed=4)
    import block_sparse_attention_top_amd as msa
    q2k = to_dev(inp["q2k"])
    a = msa.msa_build_k2q_csr(q2k, 16)
    b = msa.msa_build_k2q_csr(q2k, 16)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)
    o1, l1 = run_contiguous(inp, True, KV)
    o2, l2 = run_contiguous(inp, True, KV, csr=a)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# paged
# ---------------------------------------------------------------------------
def paged_case(B, Sq, Skv, Hkv, qpk, topk, causal, trims, seed=42, shuffle=True):
    w = wl.Workload("paged", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=causal,
                    mode=wl.MODE_CAUSAL if causal else wl.MODE_PERM, paged=True,
                    shuffle_pages=shuffle, seed=seed)
    inp = wl.make_inputs(w, q2k=np.zeros((1,), np.int32))
    seqused = np.array([Skv - t for t in trims], dtype=np.int32)
    inp["seqused_k"] = seqused
    lens = seqused if causal else np.full(B, Skv, dtype=np.int32)
    inp["q2k"] = np.concatenate([wl.q2k_table(seed + b, w.mode, 1, Hkv, Sq, int(lens[b]), 128,
                                              topk) for b in range(B)], 0)
    return w, inp


def check_paged(w, inp, splits, label, path=0):
    say(f"[paged] {label} path={path} splits={splits} B={w.B} Sq={w.Sq} Skv={w.Skv} "
        f"qpk={w.qpk} topk={w.topk} causal={w.causal}")
    o, lse = run_paged(inp, w.causal, num_splits=splits, path=path)
    o_ref, lse_ref = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                                   inp["page_table"], inp["seqused_k"],
                                                   inp["q2k"], causal=w.causal)
    full_compare(o, lse, o_ref, lse_ref, label)
    return o, lse


PQ, PK, PD = 1, 2, 3  # paged q-centric, kv-centric and decode (union of blocks) paths


@pytest.mark.parametrize("path,splits", [(PQ, 0), (PQ, 1), (PQ, 3), (PQ, 8), (PK, 0),
                                         (PD, 0), (PD, 1), (PD, 3), (PD, 8), (PD, 64)])
@pytest.mark.parametrize("causal", [True, False])
def test_paged_small(path, splits, causal):
    w, inp = paged_case(4, 8, 2048, 2, 16, 8, causal, trims=[17, 0, 1000, 2047])
    check_paged(w, inp, splits, "c5-small", path)


@pytest.mark.parametrize("Sq,topk,qpk,causal", [
    (1, 16, 16, True),    # one query: three of four waves idle
    (1, 32, 8, False),
    (5, 12, 4, True),     # ragged query count per wave
    (13, 8, 1, True),
    (16, 32, 2, True),    # the largest index set one workgroup holds (512 entries)
    (16, 4, 16, False),
])
def test_paged_decode_shapes(Sq, topk, qpk, causal):
    w, inp = paged_case(3, Sq, 4096, 2, qpk, topk, causal, trims=[0, 77, 2500], seed=5 + Sq)
    check_paged(w, inp, 0, f"decode-Sq{Sq}-topk{topk}", PD)
    check_paged(w, inp, 2, f"decode-Sq{Sq}-topk{topk}-2split", PD)


def test_paged_decode_shared_blocks():
    """Every query selects the same blocks (the sink/recent pattern of decode):
    the union holds topk blocks, each read once for all Sq queries, and duplicate
    ids inside a row count once, as in the oracle's set semantics."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 8, 2048, 2, 16, 8
    w, inp = paged_case(B, Sq, Skv, Hkv, qpk, topk, True, trims=[0, 3], seed=7)
    q2k = inp["q2k"].copy()
    q2k[:, :, :, :] = q2k[:, :, -1:, :]  # the last query's row for every query
    q2k[:, :, :, -1] = q2k[:, :, :, 0]   # one duplicate id per row
    inp = dict(inp, q2k=q2k)
    for splits in (0, 1, 5):
        check_paged(w, inp, splits, "decode-shared", PD)


def test_paged_decode_rejects_long_query_sets():
    import block_sparse_attention_top_amd as msa
    w, inp = paged_case(1, 17, 1024, 1, 16, 4, True, trims=[0])
    with pytest.raises(msa.MsaNotSupportedError):
        run_paged(inp, True, path=PD)
    assert msa.msa_paged_sparse_fwd_path(1, 17, 1, 4, 8) == PQ
    assert msa.msa_paged_sparse_fwd_path(1, 16, 1, 4, 8, PD) == PD


@pytest.mark.parametrize("path", [0, PK])
@pytest.mark.parametrize("qpk", [1, 4, 16])
def test_paged_prefill_ragged(qpk, path):
    w, inp = paged_case(3, 150, 1024, 2, qpk, 4, True, trims=[0, 100, 900])
    check_paged(w, inp, 0, f"paged-prefill-qpk{qpk}", path)


@pytest.mark.parametrize("path", [PQ, PK, PD])
def test_paged_tail_poison_and_bad_page(path):
    """NaN and huge values past seqused_k change nothing; an out-of-range page id
    drops that block (as the oracle does)."""
    w, inp = paged_case(2, 8, 1024, 1, 16, 4, True, trims=[17, 300], seed=11)
    o0, l0 = check_paged(w, inp, 0, "tail-clean", path)
    kp, vp, pt = inp["k_pool"].copy(), inp["v_pool"].copy(), inp["page_table"]
    for b in range(w.B):
        used = int(inp["seqused_k"][b])
        for s in range(w.max_pages):
            lo = max(0, used - s * 128)
            if lo < 128:
                kp[pt[b, s], :, lo:] = 0x7FC0  # NaN
                vp[pt[b, s], :, lo:] = 0x7F80  # +inf
    inp2 = dict(inp, k_pool=kp, v_pool=vp)
    o1, l1 = run_paged(inp2, True, path=path)
    assert torch.equal(o0, o1) and torch.equal(l0, l1)
    bad = pt.copy()
    bad[0, int(inp["q2k"][0, 0, 0, 0])] = 1 << 20
    check_paged(w, dict(inp, page_table=bad), 0, "bad-page", path)


@pytest.mark.parametrize("path", [PQ, PK, PD])
def test_paged_shuffled_equals_identity_bitwise(path):
    """The same logical K/V through a shuffled and through an identity page table."""
    B, Sq, Skv, Hkv, qpk, topk = 3, 8, 1024, 2, 16, 6
    w, inp = paged_case(B, Sq, Skv, Hkv, qpk, topk, True, trims=[5, 0, 200], seed=13)
    pt = inp["page_table"]
    ident = np.arange(B * w.max_pages, dtype=np.int32).reshape(B, w.max_pages)
    k2 = np.empty_like(inp["k_pool"])
    v2 = np.empty_like(inp["v_pool"])
    k2[ident.reshape(-1)] = inp["k_pool"][pt.reshape(-1)]
    v2[ident.reshape(-1)] = inp["v_pool"][pt.reshape(-1)]
    o1, l1 = run_paged(inp, True, path=path)
    o2, l2 = run_paged(dict(inp, k_pool=k2, v_pool=v2, page_table=ident), True, path=path)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_paged_equals_contiguous():
    """Paged with seqused == Skv and the identity table matches the contiguous path."""
    B, Sq, Skv, Hkv, qpk, topk = 2, 64, 1024, 2, 16, 4
    w, inp = contiguous_case(B, Sq, Skv, Hkv, qpk, topk, True, wl.MODE_CAUSAL, seed=21)
    mp = Skv // 128
    pool_k = inp["k"].reshape(B, mp, 128, Hkv, 128).transpose(0, 1, 3, 2, 4).reshape(
        B * mp, Hkv, 128, 128)
    pool_v = inp["v"].reshape(B, mp, 128, Hkv, 128).transpose(0, 1, 3, 2, 4).reshape(
        B * mp, Hkv, 128, 128)
    pin = dict(q=inp["q"], k_pool=pool_k, v_pool=pool_v, q2k=inp["q2k"],
               page_table=np.arange(B * mp, dtype=np.int32).reshape(B, mp),
               seqused_k=np.full(B, Skv, dtype=np.int32))
    op, lp = run_paged(pin, True, num_splits=1, path=PQ)
    oc, lc = run_contiguous(inp, True, Q)
    assert torch.equal(op, oc) and torch.equal(lp, lc)
    # the kv-centric path through the page table: the same items, the same bits
    op, lp = run_paged(pin, True, path=PK)
    oc, lc = run_contiguous(inp, True, KV)
    assert torch.equal(op, oc) and torch.equal(lp, lc)


# ---------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark times
# ---------------------------------------------------------------------------
def expected_nonempty(w, q2k: np.ndarray) -> np.ndarray:
    """[B, Hkv, Sq] bool: the row has at least one key (a valid slot whose block holds a
    key at or before the causal limit), computed from the index table alone."""
    nblk = (w.kvlen + w.blk - 1) // w.blk if w.paged else w.Skv // w.blk
    ok = (q2k >= 0) & (q2k < nblk)
    if w.causal:
        lim = np.arange(w.Sq).reshape(1, 1, -1, 1) + w.kvlen - w.Sq  # last visible key
        ok &= q2k.astype(np.int64) * w.blk <= lim
    return ok.any(axis=3)


def poisoned_workspace(nbytes: int) -> torch.Tensor:
    """A workspace whose every byte is 0xFF, a NaN pattern for bf16 and fp32: a partial
    the kernels read without having written it shows up as a non-finite output."""
    return torch.full((max(nbytes, 256),), 255, dtype=torch.uint8, device="cuda")


def check_any_size_properties(w, q2k, o, lse, label):
    """Properties that hold at any size: O finite everywhere, LSE finite exactly on the
    rows with a key, and O exactly 0 on the others."""
    assert torch.isfinite(o.float()).all(), f"{label}: non-finite O"
    want = torch.as_tensor(np.repeat(expected_nonempty(w, q2k), w.qpk, axis=1), device=o.device)
    got = torch.isfinite(lse)
    assert torch.equal(got, want), f"{label}: rows with a finite LSE differ from the index table"
    assert not torch.isnan(lse).any(), f"{label}: NaN in LSE"
    if not bool(want.all()):
        empty = (~want).permute(0, 2, 1)  # [B, Sq, Hq]
        assert bool((o[empty] == 0).all()), f"{label}: empty rows not zero"


# every row against the oracle where it finishes in seconds on the host (c1, c2),
# sampled rows elsewhere; the at-any-size properties on every row of every workload
FULL_ROWS = {"c1", "c2"}


@pytest.mark.parametrize("key", ["c1", "c2", "c3u", "c3s", "c4a", "c4b"])
def test_full_size(key):
    import block_sparse_attention_top_amd as msa
    w = wl.WORKLOADS[key]
    say(f"[full] {key} {w.name}: generating inputs")
    inp = wl.make_inputs(w)
    q, k, v, q2k = (to_dev(inp[n]) for n in ("q", "k", "v", "q2k"))
    path = msa.msa_sparse_fwd_path(w.B, w.Sq, w.Skv, w.Hq, w.Hkv, w.topk, 0)
    ws = poisoned_workspace(msa.msa_sparse_fwd_workspace_size(w.B, w.Sq, w.Skv, w.Hq, w.Hkv,
                                                              w.D, w.topk, w.blk, path))
    say(f"[full] {key}: running GPU (auto path = {path}, poisoned workspace)")
    o, lse = msa.msa_sparse_fwd(q, k, v, q2k, causal=w.causal, path=0, workspace=ws)
    torch.cuda.synchronize()
    check_any_size_properties(w, inp["q2k"], o, lse, key)
    del ws
    if key in FULL_ROWS:
        say(f"[full] {key}: oracle on all {w.B * w.Sq} query rows")
        o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                 causal=w.causal)
        stats = full_compare(o, lse, o_ref, lse_ref, key)
    else:
        rows = sample_rows(w.B, w.Sq, 48, seed=1)
        o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                 causal=w.causal, rows=rows)
        stats = sampled_compare(o, lse, o_ref, lse_ref, rows, w.Sq, key)
    say(f"[full] {key}: {stats}")


def test_full_size_paged_prefill():
    """The paged prefill (32768 causal queries through a shuffled page table, seqused
    trimmed by 17) at full size, on the path the benchmark times (auto = kv-centric),
    with a poisoned workspace: the at-any-size properties on every row, sampled rows
    against the oracle."""
    import block_sparse_attention_top_amd as msa
    w = wl.WORKLOADS["c3p"]
    say(f"[full] c3p {w.name}: generating inputs")
    inp = wl.make_inputs(w)
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    path = msa.msa_paged_sparse_fwd_path(w.B, w.Sq, w.Hkv, w.topk, w.max_pages)
    assert path == PK
    ws = poisoned_workspace(msa.msa_paged_sparse_fwd_workspace_size(
        w.B, w.Sq, w.Hq, w.Hkv, w.D, w.topk, w.blk, w.max_pages, 0, path))
    say("[full] c3p: running GPU (auto path = kv-centric, poisoned workspace)")
    o, lse = msa.msa_paged_sparse_fwd(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                      t["seqused_k"], t["q2k"], causal=True, workspace=ws)
    torch.cuda.synchronize()
    check_any_size_properties(w, inp["q2k"], o, lse, "c3p")
    del ws
    rows = sample_rows(w.B, w.Sq, 48, seed=1)
    o_ref, lse_ref = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                                   inp["page_table"], inp["seqused_k"],
                                                   inp["q2k"], causal=True, rows=rows)
    say(f"[full] c3p: {sampled_compare(o, lse, o_ref, lse_ref, rows, w.Sq, 'c3p')}")


@pytest.mark.parametrize("key", ["c2", "c4b"])
def test_full_size_prebuilt_csr_bit_identical(key):
    """The forward given the public ordered CSR equals the forward that builds its own
    order-free CSR (entries stored as index-table positions), bit for bit: every
    (query, slot) partial depends only on its own row, whatever the item it runs in."""
    import block_sparse_attention_top_amd as msa
    w = wl.WORKLOADS[key]
    say(f"[full] {key} {w.name}: own CSR against the public ordered CSR")
    inp = wl.make_inputs(w)
    q, k, v, q2k = (to_dev(inp[n]) for n in ("q", "k", "v", "q2k"))
    o1, l1 = msa.msa_sparse_fwd(q, k, v, q2k, causal=w.causal, path=KV)
    csr = msa.msa_build_k2q_csr(q2k, w.Skv // w.blk)
    o2, l2 = msa.msa_sparse_fwd(q, k, v, q2k, *csr, causal=w.causal, path=KV)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.fixture(scope="module")
def c5_case():
    w = wl.WORKLOADS["c5"]
    say(f"[full] c5 {w.name}: generating inputs and the oracle over all {w.B * w.Sq} rows")
    inp = wl.make_inputs(w)
    ref = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                        inp["page_table"], inp["seqused_k"], inp["q2k"],
                                        causal=True)
    return w, inp, ref


# auto (q-centric, one split), q-centric with a forced split-and-merge, the union decode
# kernel with its automatic split count and with one split
@pytest.mark.parametrize("path,splits", [(0, 0), (PQ, 4), (PD, 0), (PD, 1)])
def test_full_size_paged_decode(c5_case, path, splits):
    import block_sparse_attention_top_amd as msa
    w, inp, (o_ref, lse_ref) = c5_case
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    p = msa.msa_paged_sparse_fwd_path(w.B, w.Sq, w.Hkv, w.topk, w.max_pages, path)
    ns = msa.msa_paged_sparse_fwd_splits(w.B, w.Sq, w.Hkv, w.topk, w.max_pages, splits, p)
    ws = poisoned_workspace(msa.msa_paged_sparse_fwd_workspace_size(
        w.B, w.Sq, w.Hq, w.Hkv, w.D, w.topk, w.blk, w.max_pages, splits, p))
    say(f"[full] c5: running GPU (path {p}, {ns} splits, poisoned workspace)")
    o, lse = msa.msa_paged_sparse_fwd(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                      t["seqused_k"], t["q2k"], causal=True, num_splits=splits,
                                      path=p, workspace=ws)
    torch.cuda.synchronize()
    check_any_size_properties(w, inp["q2k"], o, lse, "c5")
    stats = full_compare(o, lse, o_ref, lse_ref, f"c5 path {p} splits {ns}")
    say(f"[full] c5: {stats}")


def test_kv_centric_at_max_csr_rows():
    """B * Skv / 128 = 16384 CSR rows, the most the kv-centric path takes: the order-free
    CSR scatter then keeps exactly 64 KiB of row cursors in LDS."""
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous_case(8, 64, 262144, 1, 1, 4, False, wl.MODE_PERM, seed=5)
    assert w.B * (w.Skv // w.blk) == 16384
    o, lse = check_contiguous(w, inp, KV, "max-csr-rows")[1]
    del o, lse
    # one sequence of 16385 blocks is too many rows for the kv-centric passes: refused on
    # the host before any launch (contents unused); the automatic path takes q-centric
    Skv2 = (16384 + 1) * 128
    kv0 = torch.zeros((1, Skv2, 1, 128), dtype=torch.bfloat16, device="cuda")
    q0 = torch.zeros((1, 8, 1, 128), dtype=torch.bfloat16, device="cuda")
    q2k0 = torch.zeros((1, 1, 8, 4), dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MsaNotSupportedError):
        msa.msa_sparse_fwd(q0, kv0, kv0, q2k0, causal=False, path=KV)
    assert msa.msa_sparse_fwd_path(1, 8, Skv2, 1, 1, 4, 0) == Q
    del kv0


def test_kv_centric_sub_batches():
    """B * Skv / 128 = 3 x 5500 = 16500 CSR rows, past the 16384 the kv-centric passes
    hold: the path runs sub-batches of two sequences and one. Sampled rows of every
    sequence against the oracle, and every row against the q-centric path."""
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous_case(3, 64, 5500 * 128, 1, 2, 8, True, wl.MODE_CAUSAL, seed=6)
    assert w.B * (w.Skv // w.blk) == 16500
    say(f"[sub-batch] {w.B} x {w.Skv // w.blk} blocks: kv-centric in sub-batches")
    o, lse = run_contiguous(inp, True, KV)
    rows = np.array([0, 1, 31, 63, 64, 100, 127, 128, 150, 191])  # all three sequences
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             causal=True, rows=rows)
    sampled_compare(o, lse, o_ref, lse_ref, rows, w.Sq, "sub-batches")
    oq, lq = run_contiguous(inp, True, Q)
    full_compare(o, lse, bf16_dev_to_f64(oq).astype(np.float64),
                 lq.cpu().numpy().astype(np.float64), "sub-batches vs q-centric")
    # a prebuilt CSR covers the whole batch, so it must fit the CSR passes: refused
    nr = w.B * (w.Skv // w.blk)
    rp = torch.zeros((1, nr + 1), dtype=torch.int32, device="cuda")
    qi = torch.zeros((1, w.B * w.Sq * w.topk), dtype=torch.int32, device="cuda")
    with pytest.raises(msa.MsaNotSupportedError):
        run_contiguous(inp, True, KV, csr=(rp, qi, qi))


def to_pool(inp, perm=None):
    """Contiguous K/V [B, Skv, Hkv, D] as page pools [B * Skv / 128, Hkv, 128, D] with a
    page table: identity, or page i of the identity layout stored at perm[i]."""
    B, Skv, Hkv, D = inp["k"].shape
    mp = Skv // 128
    def pool(x):
        p = x.reshape(B, mp, 128, Hkv, D).transpose(0, 1, 3, 2, 4).reshape(B * mp, Hkv, 128, D)
        if perm is None:
            return np.ascontiguousarray(p)
        out = np.empty_like(p)
        out[perm] = p
        return out
    ids = np.arange(B * mp, dtype=np.int32) if perm is None else perm.astype(np.int32)
    return dict(q=inp["q"], k_pool=pool(inp["k"]), v_pool=pool(inp["v"]), q2k=inp["q2k"],
                page_table=ids.reshape(B, mp), seqused_k=np.full(B, Skv, dtype=np.int32))


def test_paged_kv_centric_sub_batches():
    """3 sequences of 5500 pages (16500 CSR rows): the paged kv-centric path runs
    sub-batches of two sequences and one, through a shuffled page table, and gives the
    contiguous kv-centric path's bits (itself checked against the oracle above)."""
    w, inp = contiguous_case(3, 64, 5500 * 128, 1, 2, 8, True, wl.MODE_CAUSAL, seed=6)
    say("[paged-kv] 3 x 5500 pages, shuffled: sub-batches")
    perm = np.random.default_rng(9).permutation(w.B * 5500)
    op, lp = run_paged(to_pool(inp, perm), True, path=PK)
    oc, lc = run_contiguous(inp, True, KV)
    assert torch.equal(op, oc) and torch.equal(lp, lc)


@pytest.mark.parametrize("qpk", [2, 16])
def test_paged_kv_centric_prefill(qpk):
    """A paged prefill the automatic path sends to the kv-centric path (two sequences of
    16384 keys, trimmed by 0 and 5000, 2048 causal queries each): sampled rows against the
    oracle, every row against the paged q-centric kernel."""
    import block_sparse_attention_top_amd as msa
    w, inp = paged_case(2, 2048, 16384, 2, qpk, 16, True, trims=[0, 5000], seed=31)
    assert msa.msa_paged_sparse_fwd_path(w.B, w.Sq, w.Hkv, w.topk, w.max_pages) == PK
    say(f"[paged-kv] prefill qpk={qpk}: auto path")
    o, lse = run_paged(inp, True)
    rows = np.array([0, 1, 100, 1023, 2047, 2048, 2049, 3000, 4095])
    o_ref, lse_ref = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                                   inp["page_table"], inp["seqused_k"],
                                                   inp["q2k"], causal=True, rows=rows)
    sampled_compare(o, lse, o_ref, lse_ref, rows, w.Sq, f"paged-kv qpk{qpk}")
    oq, lq = run_paged(inp, True, num_splits=1, path=PQ)
    full_compare(o, lse, bf16_dev_to_f64(oq).astype(np.float64),
                 lq.cpu().numpy().astype(np.float64), f"paged-kv vs q-centric qpk{qpk}")


# the test page's paged forward grid (test_sparse_page_atten: causal, Hkv 2, page 128,
# no trim), batch 3, qhead_per_kv 1 and 16, topk 4 and 16, all six length pairs
@pytest.mark.parametrize("Sq,Skv", [(8192, 8192), (4096, 8192), (2048, 8192), (1024, 8192),
                                    (8192, 4096), (4096, 4096)])
@pytest.mark.parametrize("qpk,topk", [(1, 4), (1, 16), (16, 4), (16, 16)])
def test_paged_kv_centric_page_grid(Sq, Skv, qpk, topk):
    """The paged kv-centric path through a shuffled page table: bit for bit the
    contiguous kv-centric path on the same K/V, and sampled rows against the oracle."""
    w, inp = contiguous_case(3, Sq, Skv, 2, qpk, topk, True, wl.MODE_CAUSAL, seed=Sq + qpk)
    say(f"[paged-grid] Sq={Sq} Skv={Skv} qpk={qpk} topk={topk}")
    perm = np.random.default_rng(Skv + topk).permutation(3 * (Skv // 128))
    op, lp = run_paged(to_pool(inp, perm), True, path=PK)
    oc, lc = run_contiguous(inp, True, KV)
    assert torch.equal(op, oc) and torch.equal(lp, lc)
    rows = sample_rows(w.B, w.Sq, 24, seed=qpk)
    o_ref, lse_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             causal=True, rows=rows)
    sampled_compare(op, lp, o_ref, lse_ref, rows, w.Sq, f"paged-grid {Sq}/{Skv}")
