"""Dense paged decode (q2k = None) with its plan/run split-KV schedule, on the GPU.

Schedule checks follow the properties the test page's decode schedule tests state:
page counts per sequence, chunk counts, work items = sum of chunk counts,
o_indptr advancing by (queries x chunks) rows, merge_indptr giving each query row
its sequence's chunk count, longer sequences taking more chunks. Expected values
are worked out here from the lengths and the plan's chunk size. Forward checks
compare with the oracle, which has no dense mode of its own: a dense decode is the
sparse definition with every block of the sequence selected (the oracle's P-dense
pin ties that to plain dense attention)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import bf16_dev_to_f64, compare, say, to_dev

pytestmark = pytest.mark.gpu

B, SQ, HKV, QPK = 32, 8, 4, 16


def plan_for(page_table, seqused, max_kv, **kw):
    import block_sparse_attention_top_amd as msa
    p = msa.msa_paged_decode_plan(page_table, seqused, seqlen_q=SQ, max_seqlen_k=max_kv,
                                  num_qo_heads=HKV * QPK, num_kv_heads=HKV, **kw)
    torch.cuda.synchronize()
    return p


def identity_table(b, pages):
    return torch.arange(b * pages, device="cuda", dtype=torch.int32).view(b, pages)


@pytest.mark.parametrize("kv_tokens", [8, 128, 1000, 8192, 65536, 1 << 20])
def test_schedule_uniform_lengths(kv_tokens):
    pages = -(-kv_tokens // 128)
    seqused = torch.full((B,), kv_tokens, dtype=torch.int32, device="cuda")
    p = plan_for(identity_table(B, pages), seqused, kv_tokens)
    chunk = p.info.kv_chunk_size_pages
    chunks = -(-pages // chunk) if p.info.split_kv else 1
    assert p.info.padded_work_count >= int(p.work_count.item()) == B * chunks
    assert torch.equal(p.kv_pages.cpu(), torch.full((B,), pages, dtype=torch.int32))
    assert torch.equal(p.split_counts.cpu(), torch.full((B,), chunks, dtype=torch.int32))
    o_indptr = p.o_indptr.cpu()
    assert int(o_indptr[0]) == 0 and int(o_indptr[-1]) == B * SQ * chunks
    assert torch.equal(o_indptr[1:] - o_indptr[:-1], torch.full((B,), SQ * chunks, dtype=torch.int32))
    items = p.work_items.cpu()[:B * chunks]
    # every (sequence, chunk) once, chunks cover the sequence's pages exactly
    for b in (0, B - 1):
        mine = items[items[:, 0] == b]
        assert mine[:, 1].tolist() == list(range(chunks))
        assert int(mine[:, 3].sum()) == pages and int(mine[0, 2]) == 0


def test_schedule_forced_single_page_chunks():
    seqused = torch.full((B,), 3 * 128, dtype=torch.int32, device="cuda")
    p = plan_for(identity_table(B, 3), seqused, 3 * 128, fixed_split_size=1)
    assert p.info.split_kv == 1 and p.info.kv_chunk_size_pages == 1
    o_indptr = p.o_indptr.cpu()
    assert int(o_indptr[-1]) == B * SQ * 3
    assert torch.equal(o_indptr[1:] - o_indptr[:-1], torch.full((B,), SQ * 3, dtype=torch.int32))


def test_schedule_varlen_balance():
    lens = torch.tensor([8, 128, 1024, 1 << 20] * (B // 4), dtype=torch.int32, device="cuda")
    max_kv = int(lens.max())
    max_pages = -(-max_kv // 128)
    p = plan_for(identity_table(B, max_pages), lens, max_kv, max_grid_size=256)
    assert p.info.split_kv == 1
    kv_pages, counts = p.kv_pages.cpu(), p.split_counts.cpu()
    assert int(kv_pages[0]) == 1 and int(kv_pages[3]) == max_pages
    assert int(counts[3]) > int(counts[0])
    assert int(p.work_count.item()) == int(counts.sum())
    row_counts = p.merge_indptr.cpu()
    row_counts = row_counts[1:] - row_counts[:-1]
    for b in range(B):
        assert torch.equal(row_counts[b * SQ:(b + 1) * SQ],
                           torch.full((SQ,), int(counts[b]), dtype=torch.int32))


def dense_inputs(seed, batch, max_kv, lens, hkv=2, qpk=16, sq=SQ):
    """Paged pool with a shuffled page table; seqused_k = lens (the tails hold
    finite N(0,1) data that must not matter)."""
    w = wl.Workload("dd", B=batch, Sq=sq, Skv=-(-max_kv // 128) * 128, Hkv=hkv, qpk=qpk, topk=1,
                    causal=True, mode=wl.MODE_CAUSAL, paged=True, seed=seed)
    inp = wl.make_inputs(w)
    inp["seqused_k"] = np.asarray(lens, dtype=np.int32)
    return w, inp


def run_dense(inp, w, max_kv, causal=True, **kw):
    import block_sparse_attention_top_amd as msa
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k")}
    tk = {k: kw.pop(k) for k in list(kw) if k in ("return_temperature_lse",
                                                  "lse_temperature_scale", "softmax_scale")}
    p = msa.msa_paged_decode_plan(t["page_table"], t["seqused_k"], seqlen_q=w.Sq,
                                  max_seqlen_k=max_kv, num_qo_heads=w.Hq, num_kv_heads=w.Hkv,
                                  **kw)
    out = msa.msa_paged_decode_run(p, t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                   t["seqused_k"], causal=causal, **tk)
    torch.cuda.synchronize()
    return p, out


def oracle_dense(inp, w, causal=True, rows=None, temperature=None, softmax_scale=None):
    full = np.broadcast_to(np.arange(w.max_pages, dtype=np.int32),
                           (w.B, w.Hkv, w.Sq, w.max_pages))
    return oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                         inp["page_table"], inp["seqused_k"],
                                         np.ascontiguousarray(full), causal=causal, rows=rows,
                                         temperature=temperature, softmax_scale=softmax_scale)


@pytest.mark.parametrize("kv_tokens", [1, 8, 127, 128, 1000, 4096])
@pytest.mark.parametrize("causal", [True, False])
def test_dense_decode_small(kv_tokens, causal):
    w, inp = dense_inputs(90 + kv_tokens, 3, kv_tokens, [kv_tokens] * 3)
    say(f"[dense] kv={kv_tokens} causal={causal}")
    p, (o, lse) = run_dense(inp, w, kv_tokens, causal=causal)
    o_ref, lse_ref = oracle_dense(inp, w, causal=causal)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), f"dense-{kv_tokens}")


@pytest.mark.parametrize("mode", ["forced", "disabled", "auto"])
def test_dense_decode_split_modes(mode):
    """The same inputs through one chunk per sequence, single-page chunks and the
    automatic chunking agree with the oracle."""
    lens = [300, 128, 1, 2000, 0, 1500]
    w, inp = dense_inputs(95, len(lens), 2048, lens)
    kw = {"forced": {"fixed_split_size": 1}, "disabled": {"disable_split_kv": True},
          "auto": {"max_grid_size": 64}}[mode]
    say(f"[dense] split mode {mode}")
    p, (o, lse) = run_dense(inp, w, 2048, **kw)
    o_ref, lse_ref = oracle_dense(inp, w)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), f"dense-{mode}")
    assert torch.isneginf(lse[4]).all() and (o[4] == 0).all()  # seqused 0: no keys


def test_dense_decode_temperature_and_qpk():
    lens = [700, 1024, 33]
    w, inp = dense_inputs(96, 3, 1024, lens, hkv=3, qpk=4, sq=5)
    say("[dense] temperature, qpk 4, Sq 5")
    p, (o, lse, lt) = run_dense(inp, w, 1024, fixed_split_size=2, return_temperature_lse=True,
                                lse_temperature_scale=2.0)
    o_ref, lse_ref, lt_ref = oracle_dense(inp, w, temperature=2.0)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "dense-temp")
    lt_g = lt.cpu().numpy().astype(np.float64)
    fin = np.isfinite(lt_ref)
    assert np.array_equal(np.isfinite(lt_g), fin)
    assert np.all(np.abs(lt_g[fin] - lt_ref[fin]) <= 1e-3 + 1e-3 * np.abs(lt_ref[fin]))


def test_dense_decode_long_sequences_sampled():
    """32 sequences x 8 queries, 64 heads over 4 KV heads, mixed lengths up to 64K
    tokens (the decode workload's shape with dense attention), on sampled rows."""
    rng = np.random.default_rng(7)
    lens = rng.integers(1, 65536, size=32)
    lens[0] = 65519
    w, inp = dense_inputs(97, 32, 65536, lens, hkv=4, qpk=16)
    say("[dense] 64K mixed, sampled")
    p, (o, lse) = run_dense(inp, w, 65536)
    rows = np.array([0, 7, 8, 100, 129, 255], dtype=np.int64)
    o_ref, lse_ref = oracle_dense(inp, w, rows=rows)
    b, s = rows // w.Sq, rows % w.Sq
    og = o.float().cpu().numpy()[b, s].astype(np.float64)
    lg = lse.cpu().numpy()[b, :, s].astype(np.float64)
    compare(og, lg, o_ref, lse_ref, "dense-64k")


def test_dense_equals_sparse_with_every_block():
    """The dense decode and the paged sparse forward given every block agree."""
    import block_sparse_attention_top_amd as msa
    lens = [900, 1024, 40, 512]
    w, inp = dense_inputs(98, 4, 1024, lens, hkv=2, qpk=8)
    _, (o, lse) = run_dense(inp, w, 1024)
    full = np.ascontiguousarray(np.broadcast_to(np.arange(w.max_pages, dtype=np.int32),
                                                (w.B, w.Hkv, w.Sq, w.max_pages)))
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k")}
    o2, lse2 = msa.msa_paged_sparse_fwd(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                        t["seqused_k"], to_dev(full), causal=True)
    torch.cuda.synchronize()
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), bf16_dev_to_f64(o2),
            lse2.cpu().numpy().astype(np.float64), "dense-vs-sparse")


@pytest.mark.parametrize("causal", [True, False])
def test_dense_decode_bad_pages_and_nan_tails(causal):
    """Page ids outside the pool drop their keys (as in the oracle); keys at or past
    seqused_k never matter, even when they hold NaN."""
    lens = [1000, 700, 257]
    w, inp = dense_inputs(99, 3, 1024, lens)
    pt = inp["page_table"].copy()
    pt[0, 2] = -1
    num_pages = inp["k_pool"].shape[0]
    pt[1, 1] = num_pages + 5
    inp["page_table"] = pt
    for b, n in enumerate(lens):
        pg = pt[b, (n - 1) // 128]
        if 0 <= pg < num_pages and n % 128:
            inp["k_pool"][pg, :, n % 128:] = 0x7FC0  # bf16 NaN
            inp["v_pool"][pg, :, n % 128:] = 0x7FC0
    say(f"[dense] bad pages, NaN tails, causal={causal}")
    p, (o, lse) = run_dense(inp, w, 1024, causal=causal)
    o_ref, lse_ref = oracle_dense(inp, w, causal=causal)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "dense-bad-pages")
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("sq", [16, 12])
def test_dense_decode_wide_columns(sq):
    """More than 128 (query, head) columns per KV head (16 heads x 12 or 16 queries) run
    through the union kernel's dense mode (up to 4 queries per wave)."""
    lens = [2000, 300, 1024]
    w, inp = dense_inputs(100 + sq, 3, 2048, lens, sq=sq)
    say(f"[dense] wide columns Sq={sq}")
    p, (o, lse) = run_dense(inp, w, 2048, max_grid_size=48)
    o_ref, lse_ref = oracle_dense(inp, w)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), f"dense-wide-{sq}")


def draw_dense_cases(n=24, seed=2028, fp8=False):
    """Seeded random dense decodes: KV heads, qhead_per_kv, query count, batch, ragged
    seqused_k (zero included), split mode, causality, temperature and scale. The fp8
    decode serves at most 128 (query, head) columns per KV head; bf16 takes wider
    ones through the union kernel's dense mode."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        c = dict(hkv=int(rng.choice([1, 2, 3, 4, 8])), qpk=int(rng.choice([1, 2, 4, 8, 16])),
                 sq=int(rng.integers(1, 17)), batch=int(rng.integers(1, 9)),
                 max_kv=int(rng.integers(1, 4000)), causal=bool(rng.random() < 0.7),
                 temp=[None, None, 0.5, 2.0][int(rng.integers(4))],
                 scale=0.0 if rng.random() < 0.7 else float(rng.uniform(0.02, 0.2)),
                 seed=int(rng.integers(1, 1 << 30)))
        if fp8 and c["sq"] * c["qpk"] > 128:
            continue
        if not fp8 and rng.random() < 0.25:  # wider than 128 columns: the union kernel
            c["qpk"], c["sq"] = 16, int(rng.integers(9, 17))
        lens = [0 if rng.random() < 0.15 else int(rng.integers(1, c["max_kv"] + 1))
                for _ in range(c["batch"])]
        lens[int(rng.integers(c["batch"]))] = c["max_kv"]
        c["lens"] = lens
        c["split"] = [{}, {"fixed_split_size": int(rng.integers(1, 9))},
                      {"disable_split_kv": True},
                      {"max_grid_size": int(rng.choice([16, 64, 256]))}][int(rng.integers(4))]
        if c["batch"] * c["sq"] * c["hkv"] * c["qpk"] * c["max_kv"] * 128 * 4 > 5e9:
            continue
        cases.append(c)
    return cases


DENSE_CASES = draw_dense_cases()


@pytest.mark.parametrize("i", range(len(DENSE_CASES)))
def test_dense_decode_random(i):
    c = DENSE_CASES[i]
    say(f"[dense sweep] case {i}: { {k: v for k, v in c.items() if k != 'seed'} }")
    w, inp = dense_inputs(c["seed"], c["batch"], c["max_kv"], c["lens"], hkv=c["hkv"],
                          qpk=c["qpk"], sq=c["sq"])
    kw = dict(c["split"], softmax_scale=c["scale"])
    if c["temp"]:
        kw.update(return_temperature_lse=True, lse_temperature_scale=c["temp"])
    p, out = run_dense(inp, w, c["max_kv"], causal=c["causal"], **kw)
    ref = oracle_dense(inp, w, causal=c["causal"], temperature=c["temp"],
                       softmax_scale=c["scale"] if c["scale"] > 0 else None)
    o, lse = out[0], out[1]
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), ref[0],
            ref[1].transpose(0, 2, 1), f"dense-random-{i}")
    if c["temp"]:
        lt_g = out[2].cpu().numpy().astype(np.float64)
        lt_ref = ref[2]
        fin = np.isfinite(lt_ref)
        assert np.array_equal(np.isfinite(lt_g), fin)
        assert np.all(np.abs(lt_g[fin] - lt_ref[fin]) <= 1e-3 + 1e-3 * np.abs(lt_ref[fin]))
