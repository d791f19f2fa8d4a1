"""GPU parity of the fp8 e4m3fn K/V cache (the fp8 KV cache of `sparse_atten_func`).
The test page's own check: the fp8 path equals the bf16 path run on the dequantized
K/V bit for bit (atol = rtol = 0). Both kernels widen e4m3fn to bf16 exactly
before the products, so this holds by construction: the q-centric kernel's rows are
fixed per call, and the kv-centric kernel decides its lazy second-half rescale per row,
so a row's result does not depend on how the order-free CSR grouped it into wave steps.
Every case is also compared with the oracle on the fp8 inputs, under the usual parity
rules."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import bf16_dev_to_f64, check_lse_t, compare, sample_rows, say, to_dev

pytestmark = pytest.mark.gpu

Q, KV, DEC, TILE = 1, 2, 3, 4


def fp8_dev(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").view(torch.float8_e4m3fn)


def bits_equal(a: torch.Tensor, b: torch.Tensor) -> bool:
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("path", [Q, KV])
@pytest.mark.parametrize("causal", [True, False])
def test_contiguous_fp8_equals_dequantized(path, causal):
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("f", B=2, Sq=300, Skv=1024, Hkv=2, qpk=8, topk=4, causal=causal,
                    mode=wl.MODE_CAUSAL if causal else wl.MODE_PERM, seed=81)
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    say(f"[fp8] contiguous path={path} causal={causal}")
    q, q2k = to_dev(inp["q"]), to_dev(inp["q2k"])
    k8, v8 = fp8_dev(f8["k"]), fp8_dev(f8["v"])
    o8, l8, t8 = msa.msa_sparse_fwd(q, k8, v8, q2k, causal=causal, path=path,
                                    return_temperature_lse=True, lse_temperature_scale=2.0)
    kd, vd = k8.to(torch.bfloat16).contiguous(), v8.to(torch.bfloat16).contiguous()
    od, ld, td = msa.msa_sparse_fwd(q, kd, vd, q2k, causal=causal, path=path,
                                    return_temperature_lse=True, lse_temperature_scale=2.0)
    torch.cuda.synchronize()
    assert bits_equal(o8, od) and bits_equal(l8, ld) and bits_equal(t8, td)
    o_ref, lse_ref = oracle.sparse_attention(f8["q"], f8["k"], f8["v"], f8["q2k"], causal=causal)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "fp8")


def test_uint8_bytes_are_accepted_as_fp8():
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("f", B=1, Sq=64, Skv=512, Hkv=1, qpk=4, topk=2, causal=True,
                    mode=wl.MODE_CAUSAL, seed=82)
    inp = wl.with_fp8_kv(wl.make_inputs(w))
    q, q2k = to_dev(inp["q"]), to_dev(inp["q2k"])
    a = msa.msa_sparse_fwd(q, fp8_dev(inp["k"]), fp8_dev(inp["v"]), q2k, causal=True, path=Q)
    b = msa.msa_sparse_fwd(q, to_dev(inp["k"]), to_dev(inp["v"]), q2k, causal=True, path=Q)
    torch.cuda.synchronize()
    assert bits_equal(a[0], b[0]) and bits_equal(a[1], b[1])


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_fp8(path):
    import block_sparse_attention_top_amd as msa
    inp = wl.make_varlen_inputs(83, [100, 1, 257, 0, 40], [700, 129, 300, 128, 1024], 2, 16, 8,
                                wl.MODE_CAUSAL)
    f8 = wl.with_fp8_kv(inp)
    say(f"[fp8] varlen path={path}")
    q, q2k = to_dev(inp["q"]), to_dev(inp["q2k"])
    cu = (to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"]))
    k8, v8 = fp8_dev(f8["k"]), fp8_dev(f8["v"])
    o8, l8 = msa.msa_sparse_fwd_varlen(q, k8, v8, q2k, *cu, causal=True, path=path)
    od, ld = msa.msa_sparse_fwd_varlen(q, k8.to(torch.bfloat16).contiguous(),
                                       v8.to(torch.bfloat16).contiguous(), q2k, *cu, causal=True,
                                       path=path)
    torch.cuda.synchronize()
    assert bits_equal(o8, od) and bits_equal(l8, ld)
    o_ref, lse_ref = oracle.sparse_attention_varlen(f8["q"], f8["k"], f8["v"], f8["q2k"],
                                                    inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                                    causal=True)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().astype(np.float64), o_ref, lse_ref, "varlen")


@pytest.mark.parametrize("path,splits", [(Q, 1), (Q, 4), (KV, 0)])
def test_paged_fp8(path, splits):
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("fp", B=4, Sq=8, Skv=8192, Hkv=2, qpk=16, topk=16, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seqused_trim=17, seed=84)
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    say(f"[fp8] paged path={path} splits={splits}")
    t = {n: to_dev(inp[n]) for n in ("q", "page_table", "seqused_k", "q2k")}
    k8, v8 = fp8_dev(f8["k_pool"]), fp8_dev(f8["v_pool"])
    args = (t["page_table"], t["seqused_k"], t["q2k"])
    o8, l8 = msa.msa_paged_sparse_fwd(t["q"], k8, v8, *args, causal=True, num_splits=splits,
                                      path=path)
    od, ld = msa.msa_paged_sparse_fwd(t["q"], k8.to(torch.bfloat16).contiguous(),
                                      v8.to(torch.bfloat16).contiguous(), *args, causal=True,
                                      num_splits=splits, path=path)
    torch.cuda.synchronize()
    assert bits_equal(o8, od) and bits_equal(l8, ld)
    o_ref, lse_ref = oracle.paged_sparse_attention(f8["q"], f8["k_pool"], f8["v_pool"],
                                                   f8["page_table"], f8["seqused_k"], f8["q2k"],
                                                   causal=True)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "paged")


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_fp8_temperature(path):
    """fp8 cache with the temperature-scaled LSE on a ragged batch (the fp8 and
    temperature variants of both varlen kernels together): bit for bit the bf16 run on
    the dequantized K/V, and the oracle on the fp8 inputs."""
    import block_sparse_attention_top_amd as msa
    inp = wl.make_varlen_inputs(87, [150, 3, 260, 0, 64], [800, 129, 300, 256, 1000], 2, 8, 8,
                                wl.MODE_CAUSAL)
    f8 = wl.with_fp8_kv(inp)
    say(f"[fp8] varlen + temperature path={path}")
    q, q2k = to_dev(inp["q"]), to_dev(inp["q2k"])
    cu = (to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"]))
    k8, v8 = fp8_dev(f8["k"]), fp8_dev(f8["v"])
    tk = dict(return_temperature_lse=True, lse_temperature_scale=0.5)
    o8, l8, t8 = msa.msa_sparse_fwd_varlen(q, k8, v8, q2k, *cu, causal=True, path=path, **tk)
    od, ld, td = msa.msa_sparse_fwd_varlen(q, k8.to(torch.bfloat16).contiguous(),
                                           v8.to(torch.bfloat16).contiguous(), q2k, *cu,
                                           causal=True, path=path, **tk)
    torch.cuda.synchronize()
    assert bits_equal(o8, od) and bits_equal(l8, ld) and bits_equal(t8, td)
    o_ref, lse_ref, lt_ref = oracle.sparse_attention_varlen(
        f8["q"], f8["k"], f8["v"], f8["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
        causal=True, temperature=0.5)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().astype(np.float64), o_ref, lse_ref, "varlen")
    check_lse_t(t8.cpu().numpy(), lt_ref, f"varlen-fp8-T0.5-path{path}")


@pytest.mark.parametrize("path,splits", [(Q, 1), (Q, 4), (KV, 0)])
def test_paged_fp8_temperature(path, splits):
    """fp8 cache with the temperature-scaled LSE on the paged q-centric kernel, one split
    and four (the split combine merges both LSEs), and on the paged kv-centric path."""
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("fpt", B=3, Sq=8, Skv=4096, Hkv=2, qpk=16, topk=8, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seqused_trim=60, seed=88)
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    say(f"[fp8] paged + temperature path={path} splits={splits}")
    t = {n: to_dev(inp[n]) for n in ("q", "page_table", "seqused_k", "q2k")}
    k8, v8 = fp8_dev(f8["k_pool"]), fp8_dev(f8["v_pool"])
    args = (t["page_table"], t["seqused_k"], t["q2k"])
    tk = dict(return_temperature_lse=True, lse_temperature_scale=2.0)
    o8, l8, t8 = msa.msa_paged_sparse_fwd(t["q"], k8, v8, *args, causal=True,
                                          num_splits=splits, path=path, **tk)
    od, ld, td = msa.msa_paged_sparse_fwd(t["q"], k8.to(torch.bfloat16).contiguous(),
                                          v8.to(torch.bfloat16).contiguous(), *args, causal=True,
                                          num_splits=splits, path=path, **tk)
    torch.cuda.synchronize()
    assert bits_equal(o8, od) and bits_equal(l8, ld) and bits_equal(t8, td)
    o_ref, lse_ref, lt_ref = oracle.paged_sparse_attention(
        f8["q"], f8["k_pool"], f8["v_pool"], f8["page_table"], f8["seqused_k"], f8["q2k"],
        causal=True, temperature=2.0)
    compare(bf16_dev_to_f64(o8), l8.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "paged")
    check_lse_t(t8.cpu().numpy(), lt_ref, f"paged-fp8-T2-path{path}-splits{splits}")


def test_fp8_rejected_by_the_bf16_only_paths():
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("fr", B=1, Sq=8, Skv=1024, Hkv=1, qpk=16, topk=4, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seed=85)
    inp = wl.with_fp8_kv(wl.make_inputs(w))
    t = {n: to_dev(inp[n]) for n in ("q", "page_table", "seqused_k", "q2k")}
    with pytest.raises(msa.MsaNotSupportedError):
        msa.msa_paged_sparse_fwd(t["q"], fp8_dev(inp["k_pool"]), fp8_dev(inp["v_pool"]),
                                 t["page_table"], t["seqused_k"], t["q2k"], causal=True, path=DEC)
    wc = wl.Workload("fr", B=1, Sq=64, Skv=512, Hkv=1, qpk=16, topk=2, causal=True,
                     mode=wl.MODE_CAUSAL, seed=86)
    ic = wl.with_fp8_kv(wl.make_inputs(wc))
    with pytest.raises(msa.MsaNotSupportedError):
        msa.msa_sparse_fwd(to_dev(ic["q"]), fp8_dev(ic["k"]), fp8_dev(ic["v"]), to_dev(ic["q2k"]),
                           causal=True, path=TILE)


def test_decode_workload_fp8_sampled():
    """The 32 x 8-query paged decode workload (64K-token sequences, 17 keys trimmed)
    with an fp8 cache, automatic path, on sampled rows."""
    import block_sparse_attention_top_amd as msa
    w = wl.WORKLOADS["c5"]
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    say("[fp8] c5 sampled")
    t = {n: to_dev(inp[n]) for n in ("q", "page_table", "seqused_k", "q2k")}
    o, lse = msa.msa_paged_sparse_fwd(t["q"], fp8_dev(f8["k_pool"]), fp8_dev(f8["v_pool"]),
                                      t["page_table"], t["seqused_k"], t["q2k"], causal=True)
    torch.cuda.synchronize()
    rows = sample_rows(w.B, w.Sq, 48, seed=1)
    o_ref, lse_ref = oracle.paged_sparse_attention(f8["q"], f8["k_pool"], f8["v_pool"],
                                                   f8["page_table"], f8["seqused_k"], f8["q2k"],
                                                   causal=True, rows=rows)
    b, s = rows // w.Sq, rows % w.Sq
    og = o.float().cpu().numpy()[b, s].astype(np.float64)
    lg = lse.cpu().numpy()[b, :, s].astype(np.float64)
    compare(og, lg, o_ref, lse_ref, "c5-fp8")
