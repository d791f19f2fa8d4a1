"""GPU parity of paged K/V with a packed query batch (msa_paged_sparse_fwd_varlen, the
paged form of sparse_atten_func with cu_seqlens_q), through the C ABI.

Each case starts from a ragged contiguous batch (wl.make_varlen_inputs), stores every
sequence's 128-token blocks as pages of a pool in a shuffled order, and gives
seqused_k = the sequence's key count. The rows of a page past seqused_k hold NaN and
+inf, and the page-table entries past a sequence's blocks hold page ids outside the
pool: neither may change anything. The paged results must equal, bit for bit, the
contiguous varlen path of the same kernel family on the contiguous batch (the same
arithmetic on the same keys), and match the varlen oracle under the parity rules."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import bf16_dev_to_f64, check_lse_t, compare, say, to_dev

pytestmark = pytest.mark.gpu

AUTO, Q, KV = 0, 1, 2
# poison for the rows past seqused_k: NaN in K, +inf (bf16) or 448 (fp8 e4m3fn) in V
POISON = {np.dtype(np.uint16): (0x7FC0, 0x7F80), np.dtype(np.uint8): (0x7F, 0x7E)}


def to_paged(inp, seed, spare_pages=0):
    """The contiguous varlen batch as page pools, a shuffled page table and seqused_k."""
    cu_k = inp["cu_seqlens_k"]
    k_lens = np.diff(cu_k)
    B = len(k_lens)
    nb = (k_lens + 127) // 128
    mp = max(1, int(nb.max())) + spare_pages
    Hkv, D = inp["k"].shape[1], inp["k"].shape[2]
    n_pages = int(nb.sum()) + 3  # three pages no sequence uses
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n_pages)
    pk, pv = POISON[inp["k"].dtype]
    kp = np.full((n_pages, Hkv, 128, D), pk, dtype=inp["k"].dtype)
    vp = np.full((n_pages, Hkv, 128, D), pv, dtype=inp["v"].dtype)
    pt = np.full((B, mp), 1 << 20, dtype=np.int32)  # outside the pool
    i = 0
    for b in range(B):
        for s in range(int(nb[b])):
            page = int(perm[i])
            i += 1
            lo, hi = int(cu_k[b]) + 128 * s, min(int(cu_k[b + 1]), int(cu_k[b]) + 128 * (s + 1))
            kp[page, :, :hi - lo] = inp["k"][lo:hi].transpose(1, 0, 2)
            vp[page, :, :hi - lo] = inp["v"][lo:hi].transpose(1, 0, 2)
            pt[b, s] = page
    return dict(q=inp["q"], k_pool=kp, v_pool=vp, page_table=pt,
                seqused_k=k_lens.astype(np.int32), cu_seqlens_q=inp["cu_seqlens_q"],
                q2k=inp["q2k"])


def run_paged_varlen(pin, causal, path, fp8=False, **kw):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(pin[n]) for n in ("q", "page_table", "seqused_k", "cu_seqlens_q", "q2k")}
    kp, vp = to_dev(pin["k_pool"]), to_dev(pin["v_pool"])
    if fp8:
        kp, vp = kp.view(torch.float8_e4m3fn), vp.view(torch.float8_e4m3fn)
    out = msa.msa_paged_sparse_fwd_varlen(t["q"], kp, vp, t["page_table"], t["seqused_k"],
                                          t["cu_seqlens_q"], t["q2k"], causal=causal, path=path,
                                          **kw)
    torch.cuda.synchronize()
    return out


def run_varlen(inp, causal, path, **kw):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k", "cu_seqlens_q", "cu_seqlens_k")}
    out = msa.msa_sparse_fwd_varlen(t["q"], t["k"], t["v"], t["q2k"], t["cu_seqlens_q"],
                                    t["cu_seqlens_k"], causal=causal, path=path, **kw)
    torch.cuda.synchronize()
    return out


CASES = [  # (q_lens, k_lens, Hkv, qpk, topk, causal)
    ([150, 3, 260, 0, 64], [800, 129, 300, 256, 1000], 2, 8, 8, True),
    ([1, 1, 1, 1], [4000, 17, 128, 2600], 4, 16, 16, True),      # decode-like
    ([700, 300], [700, 2500], 1, 2, 4, False),
    ([33, 0, 513], [0, 90, 3000], 2, 4, 16, True),               # a sequence with no keys
]


@pytest.mark.parametrize("path", [Q, KV])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_paged_varlen_equals_contiguous_varlen(case, path):
    q_lens, k_lens, Hkv, qpk, topk, causal = CASES[case]
    mode = wl.MODE_CAUSAL if causal or any(0 < k < 128 * topk for k in k_lens) else wl.MODE_PERM
    inp = wl.make_varlen_inputs(70 + case, q_lens, k_lens, Hkv, qpk, topk, mode)
    pin = to_paged(inp, seed=case, spare_pages=case % 2)
    say(f"[paged-varlen] case {case} path={path} q_lens={q_lens} k_lens={k_lens} Hkv={Hkv} "
        f"qpk={qpk} topk={topk} causal={causal}")
    o, lse = run_paged_varlen(pin, causal, path, num_splits=1)  # as the contiguous varlen path
    oc, lc = run_varlen(inp, causal, path)
    assert torch.equal(o, oc) and torch.equal(lse, lc), "paged differs from contiguous"
    o_ref, lse_ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                                    causal=causal)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
            f"paged-varlen case {case}")


def test_paged_varlen_auto_path_and_large_prefill():
    """A ragged prefill big enough for the kv-centric path (auto), sampled rows against
    the oracle and every row bit for bit against the contiguous varlen kv path."""
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens = [4096, 1000, 3000], [4096, 9000, 3000]
    inp = wl.make_varlen_inputs(91, q_lens, k_lens, 2, 16, 16, wl.MODE_CAUSAL)
    pin = to_paged(inp, seed=5)
    mp = pin["page_table"].shape[1]
    assert msa.msa_paged_sparse_fwd_varlen_path(3, sum(q_lens), 2, 16, mp) == KV
    say("[paged-varlen] ragged prefill, auto path")
    o, lse = run_paged_varlen(pin, True, AUTO)
    oc, lc = run_varlen(inp, True, KV)
    assert torch.equal(o, oc) and torch.equal(lse, lc)
    rows = np.array([0, 1, 2047, 4095, 4096, 5095, 5096, 8095])
    o_ref, lse_ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                                    causal=True, rows=rows)
    compare(bf16_dev_to_f64(o)[rows], lse.cpu().numpy().astype(np.float64)[rows], o_ref,
            lse_ref, "paged-varlen prefill")
    # decode-like batches stay on the q-centric kernel
    assert msa.msa_paged_sparse_fwd_varlen_path(64, 64, 4, 16, 512) == Q


@pytest.mark.parametrize("path", [Q, KV])
def test_paged_varlen_fp8_and_temperature(path):
    """The fp8 cache with the temperature-scaled LSE: bit for bit the bf16 run on the
    dequantized pools, and the oracle on the fp8 inputs."""
    q_lens, k_lens = [150, 3, 260], [800, 129, 1000]
    inp = wl.with_fp8_kv(wl.make_varlen_inputs(77, q_lens, k_lens, 2, 8, 8, wl.MODE_CAUSAL))
    pin = to_paged(inp, seed=3)  # fp8 byte pools
    say(f"[paged-varlen] fp8 + temperature path={path}")
    tk = dict(return_temperature_lse=True, lse_temperature_scale=0.5)
    o8, l8, t8 = run_paged_varlen(pin, True, path, fp8=True, num_splits=2, **tk)
    deq = dict(pin, k_pool=to_dev(pin["k_pool"]).view(torch.float8_e4m3fn).to(torch.bfloat16)
               .view(torch.uint16).cpu().numpy(),
               v_pool=to_dev(pin["v_pool"]).view(torch.float8_e4m3fn).to(torch.bfloat16)
               .view(torch.uint16).cpu().numpy())
    od, ld, td = run_paged_varlen(deq, True, path, num_splits=2, **tk)
    assert torch.equal(o8, od) and torch.equal(l8, ld) and torch.equal(t8, td)
    o_ref, lse_ref, lt_ref = oracle.sparse_attention_varlen(
        inp["q"], inp["k"], inp["v"], inp["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
        causal=True, temperature=0.5)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().astype(np.float64), o_ref, lse_ref,
            "paged-varlen fp8")
    check_lse_t(t8.cpu().numpy(), lt_ref, f"paged-varlen fp8 T0.5 path{path}")


def test_paged_varlen_empty_batch_and_refusals():
    import block_sparse_attention_top_amd as msa
    inp = wl.make_varlen_inputs(5, [0, 0], [300, 0], 1, 2, 4, wl.MODE_CAUSAL)
    pin = to_paged(inp, seed=1)
    o, lse = run_paged_varlen(pin, True, AUTO)  # total_q = 0: nothing to do
    assert o.shape[0] == 0 and lse.shape[0] == 0
    inp = wl.make_varlen_inputs(6, [4, 4], [300, 200], 1, 2, 4, wl.MODE_CAUSAL)
    pin = to_paged(inp, seed=2)
    with pytest.raises(msa.MsaNotSupportedError):  # no union decode for packed queries
        run_paged_varlen(pin, True, 3)


@pytest.mark.parametrize("splits", [0, 3, 16])
@pytest.mark.parametrize("case", [0, 1, 3])
def test_paged_varlen_q_centric_splits(case, splits):
    """The q-centric path with its slots split (automatic, 3 and 16) and merged by
    log-sum-exp, with the temperature LSE: against the varlen oracle."""
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens, Hkv, qpk, topk, causal = CASES[case]
    inp = wl.make_varlen_inputs(80 + case, q_lens, k_lens, Hkv, qpk, topk, wl.MODE_CAUSAL)
    pin = to_paged(inp, seed=10 + case)
    ns = msa.msa_paged_sparse_fwd_varlen_splits(len(q_lens), sum(q_lens), Hkv, topk,
                                                pin["page_table"].shape[1], splits, Q)
    say(f"[paged-varlen] case {case} q-centric splits={splits} ({ns} used)")
    if case == 1 and splits == 0:
        assert ns == 8  # 16 (query, KV head) rows: the automatic rule splits
    o, lse, lt = run_paged_varlen(pin, True, Q, num_splits=splits, return_temperature_lse=True,
                                  lse_temperature_scale=2.0)
    o_ref, lse_ref, lt_ref = oracle.sparse_attention_varlen(
        inp["q"], inp["k"], inp["v"], inp["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
        causal=True, temperature=2.0)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
            f"paged-varlen splits case {case}")
    check_lse_t(lt.cpu().numpy(), lt_ref, f"paged-varlen splits {splits} T2")


def draw_random_cases(n=16, seed=2031):
    """Seeded ragged batches for the paged varlen entry point: lengths (empty sequences
    and sequences without keys included), heads, topk, causality, path, splits, the fp8
    cache and the temperature LSE."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        B = int(rng.integers(1, 6))
        c = dict(q_lens=[0 if rng.random() < 0.15 else int(rng.integers(1, 300)) for _ in range(B)],
                 k_lens=[0 if rng.random() < 0.1 else int(rng.integers(1, 2500)) for _ in range(B)],
                 Hkv=int(rng.choice([1, 2, 4])), qpk=int(rng.choice([1, 2, 4, 8, 16])),
                 topk=int(rng.choice([1, 4, 8, 16, 32])), causal=bool(rng.random() < 0.7),
                 path=int(rng.choice([AUTO, Q, KV])), splits=int(rng.choice([0, 1, 4])),
                 fp8=bool(rng.random() < 0.3), temp=[None, 0.5, 2.0][int(rng.integers(3))],
                 seed=int(rng.integers(1, 1 << 30)))
        c["q_lens"][0] = max(c["q_lens"][0], 1)
        out.append(c)
    return out


RANDOM = draw_random_cases()


@pytest.mark.parametrize("i", range(len(RANDOM)))
def test_paged_varlen_random(i):
    c = RANDOM[i]
    say(f"[paged-varlen] random {i}: { {k: v for k, v in c.items() if k != 'seed'} }")
    short = any(0 < k < 128 * c["topk"] for k in c["k_lens"])
    mode = wl.MODE_CAUSAL if c["causal"] or short else wl.MODE_PERM
    inp = wl.make_varlen_inputs(c["seed"], c["q_lens"], c["k_lens"], c["Hkv"], c["qpk"],
                                c["topk"], mode)
    if c["fp8"]:
        inp = wl.with_fp8_kv(inp)
    pin = to_paged(inp, seed=c["seed"] % 1000, spare_pages=i % 3)
    tk = {} if c["temp"] is None else dict(return_temperature_lse=True,
                                           lse_temperature_scale=c["temp"])
    out = run_paged_varlen(pin, c["causal"], c["path"], fp8=c["fp8"], num_splits=c["splits"],
                           **tk)
    ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                         inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                         causal=c["causal"], temperature=c["temp"])
    compare(bf16_dev_to_f64(out[0]), out[1].cpu().numpy().astype(np.float64), ref[0], ref[1],
            f"paged-varlen random {i}")
    if c["temp"] is not None:
        check_lse_t(out[2].cpu().numpy(), ref[2], f"paged-varlen random {i} T")
