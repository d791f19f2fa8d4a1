"""The fp8 dense paged decode (Q, K and V fp8 e4m3fn; probabilities rounded to e4m3
before P V) on the GPU against the oracle's fp8 decode, the test page's
`_decode_paged_dense_reference`.

Tolerance: the test page's own fp8 rule for this decode (`_assert_fp8_forward_close`):
O within max(0.125, 4 x the bf16 rounding of the reference) in max-abs, LSE within
atol = rtol = 2e-3 on finite entries. The kernel rounds the probabilities relative to
its running reference maximum instead of the row's final maximum, so its e4m3
rounding points differ from the reference's; the LSE (unrounded sums) and the
temperature LSE are held tighter (1e-3), and a zero query, whose probabilities are
all exactly 1, must average the visible values to bf16 precision."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import say, to_dev

pytestmark = pytest.mark.gpu

SQ = 8


def fp8_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").view(torch.float8_e4m3fn)


def fp8_inputs(seed, batch, max_kv, lens, hkv=2, qpk=16, sq=SQ):
    """Paged pools with a shuffled page table, Q and K/V as fp8 bytes (the bf16
    N(0, 1) inputs rounded to e4m3)."""
    w = wl.Workload("df8", B=batch, Sq=sq, Skv=-(-max_kv // 128) * 128, Hkv=hkv, qpk=qpk, topk=1,
                    causal=True, mode=wl.MODE_CAUSAL, paged=True, seed=seed)
    inp = wl.make_inputs(w)
    inp["seqused_k"] = np.asarray(lens, dtype=np.int32)
    for n in ("q", "k_pool", "v_pool"):
        inp[n] = wl.bf16_bits_to_fp8(inp[n])
    return w, inp


def run_fp8(inp, w, max_kv, causal=True, **kw):
    import block_sparse_attention_top_amd as msa
    pt, seq = to_dev(inp["page_table"]), to_dev(inp["seqused_k"])
    tk = {k: kw.pop(k) for k in list(kw) if k in ("return_temperature_lse",
                                                  "lse_temperature_scale")}
    p = msa.msa_paged_decode_plan(pt, seq, seqlen_q=w.Sq, max_seqlen_k=max_kv, num_qo_heads=w.Hq,
                                  num_kv_heads=w.Hkv, **kw)
    out = msa.msa_paged_decode_run(p, fp8_dev(inp["q"]), fp8_dev(inp["k_pool"]),
                                   fp8_dev(inp["v_pool"]), pt, seq, causal=causal, **tk)
    torch.cuda.synchronize()
    return out


def check(o_gpu, lse_gpu, o_ref, lse_ref, label, lse_abs=1e-3):
    """o_* [rows, Hq, D], lse_* [rows, Hq]; the page's fp8 rule plus an absolute LSE
    bound (lse_abs; None keeps the page's relative rule alone)."""
    o_g = np.asarray(o_gpu, dtype=np.float64)
    o_bf = torch.from_numpy(o_ref).to(torch.bfloat16).double().numpy()
    floor = np.abs(o_bf - o_ref).max()
    o_err = np.abs(o_g - o_bf).max()
    fin = np.isfinite(lse_ref)
    lse_g = np.asarray(lse_gpu, dtype=np.float64)
    assert np.array_equal(np.isfinite(lse_g), fin), f"{label}: empty-row mask differs"
    lse_err = np.abs(lse_g[fin] - lse_ref[fin]).max() if fin.any() else 0.0
    say(f"[{label}] O max-abs {o_err:.4f} (bf16 floor {floor:.4f}), LSE max-abs {lse_err:.2e}")
    assert o_err <= max(0.125, 4 * floor), f"{label}: O error {o_err}"
    assert np.all(np.abs(lse_g[fin] - lse_ref[fin]) <= 2e-3 + 2e-3 * np.abs(lse_ref[fin]))
    if lse_abs is not None:
        assert lse_err <= lse_abs, f"{label}: LSE error {lse_err}"
    assert not np.any(o_g[~fin]), f"{label}: empty rows must be zero"


def as_rows(o, lse):
    """O [B, Sq, Hq, D] and LSE [B, Hq, Sq] -> [B*Sq, Hq, D] and [B*Sq, Hq]."""
    o = o.float().cpu().numpy()
    B, Sq, Hq, D = o.shape
    return o.reshape(B * Sq, Hq, D), lse.cpu().numpy().transpose(0, 2, 1).reshape(B * Sq, Hq)


def oracle_rows(inp, causal=True, rows=None, temperature=None):
    out = oracle.paged_decode_fp8(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                  inp["seqused_k"], causal=causal, rows=rows,
                                  temperature=temperature)
    if rows is not None:
        return out
    o, lse = out[0], out[1]
    B, Sq, Hq, D = o.shape
    res = (o.reshape(B * Sq, Hq, D), lse.transpose(0, 2, 1).reshape(B * Sq, Hq))
    if temperature is not None:
        res += (out[2].transpose(0, 2, 1).reshape(B * Sq, Hq),)
    return res


@pytest.mark.parametrize("kv_tokens", [1, 8, 127, 128, 1000, 4096])
@pytest.mark.parametrize("causal", [True, False])
def test_fp8_decode_small(kv_tokens, causal):
    w, inp = fp8_inputs(110 + kv_tokens, 3, kv_tokens, [kv_tokens] * 3)
    say(f"[fp8 dense] kv={kv_tokens} causal={causal}")
    o, lse = run_fp8(inp, w, kv_tokens, causal=causal)
    check(*as_rows(o, lse), *oracle_rows(inp, causal=causal), f"fp8-{kv_tokens}-{causal}")


@pytest.mark.parametrize("mode", ["forced", "disabled", "auto"])
def test_fp8_decode_split_modes(mode):
    lens = [300, 128, 1, 2000, 0, 1500]
    w, inp = fp8_inputs(115, len(lens), 2048, lens)
    kw = {"forced": {"fixed_split_size": 1}, "disabled": {"disable_split_kv": True},
          "auto": {"max_grid_size": 64}}[mode]
    say(f"[fp8 dense] split mode {mode}")
    o, lse = run_fp8(inp, w, 2048, **kw)
    check(*as_rows(o, lse), *oracle_rows(inp), f"fp8-{mode}")
    assert torch.isneginf(lse[4]).all() and (o[4] == 0).all()  # seqused 0: no keys


def test_fp8_decode_temperature_and_small_qpk():
    lens = [700, 1024, 33]
    w, inp = fp8_inputs(116, 3, 1024, lens, hkv=3, qpk=4, sq=5)
    say("[fp8 dense] temperature, qpk 4, Sq 5")
    o, lse, lt = run_fp8(inp, w, 1024, fixed_split_size=2, return_temperature_lse=True,
                         lse_temperature_scale=2.0)
    o_ref, lse_ref, lt_ref = oracle_rows(inp, temperature=2.0)
    check(*as_rows(o, lse), o_ref, lse_ref, "fp8-temp")
    lt_g = lt.cpu().numpy().transpose(0, 2, 1).reshape(lt_ref.shape).astype(np.float64)
    fin = np.isfinite(lt_ref)
    assert np.array_equal(np.isfinite(lt_g), fin)
    assert np.all(np.abs(lt_g[fin] - lt_ref[fin]) <= 1e-3 + 1e-3 * np.abs(lt_ref[fin]))


def test_fp8_zero_query_averages_the_values():
    """A zero query scores every key 0, so every probability is exactly 1 in e4m3 and
    O is the mean of the visible values; LSE = log(visible keys)."""
    lens = [1000, 130]
    w, inp = fp8_inputs(117, 2, 1024, lens)
    inp["q"] = np.zeros_like(inp["q"])
    o, lse = run_fp8(inp, w, 1024)
    o_ref, lse_ref = oracle_rows(inp)
    o_g, lse_g = as_rows(o, lse)
    for b, n0 in enumerate(lens):
        for s in range(w.Sq):
            n = n0 - w.Sq + s + 1
            assert np.allclose(lse_g[b * w.Sq + s], math.log(n), atol=1e-5, rtol=0)
    assert np.abs(o_g - o_ref).max() <= 2 ** -8 * np.abs(o_ref).max() + 1e-6


def test_fp8_decode_workload_sampled():
    """32 sequences x 8 queries, 64 heads over 4 KV heads, mixed lengths up to 64K
    tokens (the decode workload's shape, dense, fp8), on sampled rows."""
    rng = np.random.default_rng(8)
    lens = rng.integers(1, 65536, size=32)
    lens[0] = 65519
    w, inp = fp8_inputs(118, 32, 65536, lens, hkv=4, qpk=16)
    say("[fp8 dense] 64K mixed, sampled")
    o, lse = run_fp8(inp, w, 65536)
    rows = np.array([0, 7, 8, 100, 129, 255], dtype=np.int64)
    o_ref, lse_ref = oracle_rows(inp, rows=rows)
    o_g, lse_g = as_rows(o, lse)
    check(o_g[rows], lse_g[rows], o_ref, lse_ref, "fp8-64k")


def test_fp8_decode_refusals():
    import block_sparse_attention_top_amd as msa
    lens = [256] * 2
    w, inp = fp8_inputs(119, 2, 256, lens, sq=16)  # 16 queries x 16 heads: 256 columns
    pt, seq = to_dev(inp["page_table"]), to_dev(inp["seqused_k"])
    p = msa.msa_paged_decode_plan(pt, seq, seqlen_q=16, max_seqlen_k=256, num_qo_heads=w.Hq,
                                  num_kv_heads=w.Hkv)
    with pytest.raises(msa.MsaNotSupportedError):
        msa.msa_paged_decode_run(p, fp8_dev(inp["q"]), fp8_dev(inp["k_pool"]),
                                 fp8_dev(inp["v_pool"]), pt, seq)
    qb = torch.zeros(inp["q"].shape, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(TypeError):  # fp8 pools need an fp8 query
        msa.msa_paged_decode_run(p, qb, fp8_dev(inp["k_pool"]), fp8_dev(inp["v_pool"]), pt, seq)


def test_fp8_decode_bad_pages_and_nan_tails():
    """Page ids outside the pool drop their keys (as in the oracle); keys at or past
    seqused_k never matter, even when their bytes are the e4m3fn NaN code."""
    lens = [1000, 700, 257]
    w, inp = fp8_inputs(120, 3, 1024, lens)
    pt = inp["page_table"].copy()
    pt[0, 2] = -1
    num_pages = inp["k_pool"].shape[0]
    pt[1, 1] = num_pages + 5
    inp["page_table"] = pt
    for b, n in enumerate(lens):  # NaN in every unused row of the last page
        pg = pt[b, (n - 1) // 128]
        if 0 <= pg < num_pages and n % 128:
            inp["k_pool"][pg, :, n % 128:] = 0x7F
            inp["v_pool"][pg, :, n % 128:] = 0x7F
    say("[fp8 dense] bad pages, NaN tails")
    o, lse = run_fp8(inp, w, 1024)
    check(*as_rows(o, lse), *oracle_rows(inp), "fp8-bad-pages")
    assert torch.isfinite(o.float()).all()


def test_fp8_decode_peaked():
    """Peaked scores (Q x 16 and V / 4, applied before the e4m3 rounding): the decode's
    lazy reference max moves often, which is where its rounding of P against the running
    max departs most from the reference's rounding against the final max. Still within
    the page's fp8 rule. The LSEs here are ~50: the fp32 accumulation of dot products
    of that size alone is ~1e-3 in natural-log units, so the test keeps the page's
    relative LSE rule (2e-3 + 2e-3 |LSE|) without the absolute 1e-3 bound of the
    N(0, 1) cases."""
    from test_gpu_peaked import scaled
    w = wl.Workload("df8p", B=3, Sq=SQ, Skv=3072, Hkv=2, qpk=16, topk=1, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seed=96)
    inp = wl.make_inputs(w)
    inp["seqused_k"] = np.asarray([3000, 1, 2500], dtype=np.int32)
    inp["q"] = scaled(inp["q"], 16)
    inp["v_pool"] = scaled(inp["v_pool"], 0.25)
    for n in ("q", "k_pool", "v_pool"):
        inp[n] = wl.bf16_bits_to_fp8(inp[n])
    say("[fp8 dense] peaked scores")
    o, lse = run_fp8(inp, w, 3000)
    check(*as_rows(o, lse), *oracle_rows(inp), "fp8-peaked", lse_abs=None)


@pytest.mark.parametrize("i", range(24))
def test_fp8_decode_random(i):
    """Seeded random fp8 decodes (the bf16 sweep's generator, limited to the fp8
    decode's 128 columns per KV head) under the page's fp8 rule."""
    import block_sparse_attention_top_amd as msa
    from test_gpu_decode_dense import draw_dense_cases
    c = draw_dense_cases(seed=2029, fp8=True)[i]
    say(f"[fp8 dense sweep] case {i}: { {k: v for k, v in c.items() if k != 'seed'} }")
    w, inp = fp8_inputs(c["seed"], c["batch"], c["max_kv"], c["lens"], hkv=c["hkv"],
                        qpk=c["qpk"], sq=c["sq"])
    pt, seq = to_dev(inp["page_table"]), to_dev(inp["seqused_k"])
    p = msa.msa_paged_decode_plan(pt, seq, seqlen_q=w.Sq, max_seqlen_k=c["max_kv"],
                                  num_qo_heads=w.Hq, num_kv_heads=w.Hkv, **c["split"])
    tk = dict(return_temperature_lse=True, lse_temperature_scale=c["temp"]) if c["temp"] else {}
    out = msa.msa_paged_decode_run(p, fp8_dev(inp["q"]), fp8_dev(inp["k_pool"]),
                                   fp8_dev(inp["v_pool"]), pt, seq, causal=c["causal"],
                                   softmax_scale=c["scale"], **tk)
    torch.cuda.synchronize()
    ref = oracle.paged_decode_fp8(inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"],
                                  inp["seqused_k"], causal=c["causal"],
                                  softmax_scale=c["scale"] if c["scale"] > 0 else None,
                                  temperature=c["temp"])
    o, lse = as_rows(out[0], out[1])
    B, Sq, Hq, D = ref[0].shape
    check(o, lse, ref[0].reshape(B * Sq, Hq, D), ref[1].transpose(0, 2, 1).reshape(B * Sq, Hq),
          f"fp8-random-{i}")
    if c["temp"]:
        lt_g = out[2].cpu().numpy().astype(np.float64)
        fin = np.isfinite(ref[2])
        assert np.array_equal(np.isfinite(lt_g), fin)
        assert np.all(np.abs(lt_g[fin] - ref[2][fin]) <= 1e-3 + 1e-3 * np.abs(ref[2][fin]))
