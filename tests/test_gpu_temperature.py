"""GPU parity of the temperature-scaled LSE (log-sum-exp of the masked scores divided by
T) on every forward path, against the oracle on the same seeded inputs. Tolerance: the
test page's rule for it, |d| <= 1e-3 + 1e-3 |ref| on finite entries, with identical
empty-row masks; O and the plain LSE keep the parity rules of parity_util."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import bf16_dev_to_f64, check_lse_t, compare, say, to_dev

pytestmark = pytest.mark.gpu

Q, KV, DEC, TILE = 1, 2, 3, 4


def contiguous(B, Sq, Skv, Hkv, qpk, topk, causal, mode, seed):
    w = wl.Workload("t", B=B, Sq=Sq, Skv=Skv, Hkv=Hkv, qpk=qpk, topk=topk, causal=causal,
                    mode=mode, seed=seed)
    return w, wl.make_inputs(w)


@pytest.mark.parametrize("path", [Q, KV, TILE])
@pytest.mark.parametrize("temp", [2.0, 0.5, 0.03])
def test_contiguous_temperature(path, temp):
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous(2, 320, 1024, 2, 16, 4, True, wl.MODE_CAUSAL, seed=61)
    say(f"[temp] contiguous path={path} T={temp}")
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k")}
    o, lse, lt = msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=True, path=path,
                                    return_temperature_lse=True, lse_temperature_scale=temp)
    torch.cuda.synchronize()
    o_ref, lse_ref, lt_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                                     causal=True, temperature=temp)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), f"T{temp}")
    check_lse_t(lt.cpu().numpy(), lt_ref, f"path{path}-T{temp}")
    # the plain outputs do not depend on whether the temperature LSE is asked for
    o2, lse2 = msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=True, path=path)
    torch.cuda.synchronize()
    if path in (Q, TILE) and temp >= 1.0:
        assert torch.equal(o.view(torch.int16), o2.view(torch.int16)) and torch.equal(lse, lse2)
    else:
        compare(bf16_dev_to_f64(o2), lse2.cpu().numpy().transpose(0, 2, 1).astype(np.float64),
                o_ref, lse_ref.transpose(0, 2, 1), "plain")


@pytest.mark.parametrize("path", [Q, KV, TILE])
def test_unit_temperature_gives_the_lse_bits(path):
    """T = 1 computed by the kernels equals the LSE bit for bit; the binding's fast
    path returns the LSE tensor itself, as the interface page's binding does."""
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous(1, 256, 768, 2, 8, 3, False, wl.MODE_PERM, seed=62)
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k")}
    say(f"[temp] unit T path={path}")
    _, lse, lt = msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=False, path=path,
                                    return_temperature_lse=True, lse_temperature_scale=1.0,
                                    temperature_fast_path=False)
    torch.cuda.synchronize()
    assert lt.data_ptr() != lse.data_ptr() and torch.equal(lt, lse)
    _, lse, lt = msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=False, path=path,
                                    return_temperature_lse=True)
    assert lt.data_ptr() == lse.data_ptr()


def test_empty_rows_and_invalid_ids():
    """Sq > Skv (causal) leaves rows without keys; -1 rows too: -inf on every path."""
    import block_sparse_attention_top_amd as msa
    w, inp = contiguous(1, 400, 256, 1, 16, 2, True, wl.MODE_CAUSAL, seed=63)
    inp["q2k"][0, 0, 300:310] = -1
    _, _, lt_ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"], causal=True,
                                           temperature=3.0)
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k")}
    for path in (Q, KV, TILE):
        say(f"[temp] empty rows path={path}")
        _, _, lt = msa.msa_sparse_fwd(t["q"], t["k"], t["v"], t["q2k"], causal=True, path=path,
                                      return_temperature_lse=True, lse_temperature_scale=3.0)
        torch.cuda.synchronize()
        check_lse_t(lt.cpu().numpy(), lt_ref, f"empty-path{path}")


@pytest.mark.parametrize("path", [Q, KV])
def test_varlen_temperature(path):
    import block_sparse_attention_top_amd as msa
    q_lens, k_lens = [130, 7, 300, 0, 64], [900, 129, 300, 256, 1000]
    inp = wl.make_varlen_inputs(64, q_lens, k_lens, 2, 4, 8, wl.MODE_CAUSAL)
    say(f"[temp] varlen path={path}")
    t = {n: to_dev(inp[n]) for n in ("q", "k", "v", "q2k", "cu_seqlens_q", "cu_seqlens_k")}
    o, lse, lt = msa.msa_sparse_fwd_varlen(t["q"], t["k"], t["v"], t["q2k"], t["cu_seqlens_q"],
                                           t["cu_seqlens_k"], causal=True, path=path,
                                           return_temperature_lse=True, lse_temperature_scale=2.0)
    torch.cuda.synchronize()
    o_ref, lse_ref, lt_ref = oracle.sparse_attention_varlen(
        inp["q"], inp["k"], inp["v"], inp["q2k"], inp["cu_seqlens_q"], inp["cu_seqlens_k"],
        causal=True, temperature=2.0)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref, "varlen")
    check_lse_t(lt.cpu().numpy(), lt_ref, f"varlen-path{path}")


@pytest.mark.parametrize("path,splits", [(Q, 1), (Q, 4), (KV, 0), (DEC, 1), (DEC, 5)])
@pytest.mark.parametrize("temp", [2.0, 0.25])
def test_paged_temperature(path, splits, temp):
    import block_sparse_attention_top_amd as msa
    w = wl.Workload("tp", B=3, Sq=8, Skv=4096, Hkv=2, qpk=16, topk=8, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seqused_trim=100, seed=65)
    inp = wl.make_inputs(w)
    say(f"[temp] paged path={path} splits={splits} T={temp}")
    t = {n: to_dev(inp[n]) for n in ("q", "k_pool", "v_pool", "page_table", "seqused_k", "q2k")}
    o, lse, lt = msa.msa_paged_sparse_fwd(t["q"], t["k_pool"], t["v_pool"], t["page_table"],
                                          t["seqused_k"], t["q2k"], causal=True,
                                          num_splits=splits, path=path,
                                          return_temperature_lse=True,
                                          lse_temperature_scale=temp)
    torch.cuda.synchronize()
    o_ref, lse_ref, lt_ref = oracle.paged_sparse_attention(
        inp["q"], inp["k_pool"], inp["v_pool"], inp["page_table"], inp["seqused_k"], inp["q2k"],
        causal=True, temperature=temp)
    compare(bf16_dev_to_f64(o), lse.cpu().numpy().transpose(0, 2, 1).astype(np.float64), o_ref,
            lse_ref.transpose(0, 2, 1), "paged")
    check_lse_t(lt.cpu().numpy(), lt_ref, f"paged-{path}-{splits}-T{temp}")
