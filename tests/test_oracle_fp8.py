"""Pins of the oracle's fp8 e4m3fn K/V cache reads (the fp8 KV cache of
`sparse_atten_func` on the interface page, checked on the test page against the
bf16 path on dequantized K/V). The decoder is checked against torch's own
float8_e4m3fn conversion and against values worked out from the format; the
attention on fp8 K/V must equal the attention on the dequantized bf16 K/V."""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def test_decoder_matches_torch_float8_e4m3fn():
    b = np.arange(256, dtype=np.uint8)
    mine = oracle.fp8_e4m3_decode(b)
    ref = torch.from_numpy(b).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan) and nan.sum() == 2  # 0x7f and 0xff
    assert np.array_equal(mine[~nan], ref[~nan])


@pytest.mark.parametrize("bits,value", [
    (0x38, 1.0), (0x40, 2.0), (0x3C, 1.5), (0x7E, 448.0), (0xFE, -448.0),
    (0x01, 2.0 ** -9), (0x07, 7 * 2.0 ** -9), (0x08, 2.0 ** -6), (0x00, 0.0), (0xB8, -1.0),
])
def test_decoder_worked_values(bits, value):
    """(1 + m/8) 2^(e-7) for normal codes, m 2^-9 for e = 0."""
    assert oracle.fp8_e4m3_decode(np.array([bits], np.uint8))[0] == value


def test_negative_zero():
    v = oracle.fp8_e4m3_decode(np.array([0x80], np.uint8))[0]
    assert v == 0.0 and np.signbit(v)


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_kv_equals_dequantized_bf16(causal):
    w = wl.Workload("f", B=2, Sq=96, Skv=512, Hkv=2, qpk=4, topk=3, causal=causal,
                    mode=wl.MODE_CAUSAL if causal else wl.MODE_PERM, seed=71)
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    deq = dict(inp, k=wl.fp8_to_bf16_bits(f8["k"]), v=wl.fp8_to_bf16_bits(f8["v"]))
    a = oracle.sparse_attention(f8["q"], f8["k"], f8["v"], f8["q2k"], causal=causal,
                                temperature=2.0)
    b = oracle.sparse_attention(deq["q"], deq["k"], deq["v"], deq["q2k"], causal=causal,
                                temperature=2.0)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    # and quantizing changed something (the pin is not vacuous)
    c = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"], causal=causal)
    assert not np.array_equal(a[0], c[0])


def test_fp8_paged_and_varlen_equal_dequantized():
    w = wl.Workload("fp", B=2, Sq=8, Skv=1024, Hkv=2, qpk=8, topk=4, causal=True,
                    mode=wl.MODE_CAUSAL, paged=True, seqused_trim=17, seed=72)
    inp = wl.make_inputs(w)
    f8 = wl.with_fp8_kv(inp)
    deq = dict(inp, k_pool=wl.fp8_to_bf16_bits(f8["k_pool"]),
               v_pool=wl.fp8_to_bf16_bits(f8["v_pool"]))
    args = ("page_table", "seqused_k", "q2k")
    a = oracle.paged_sparse_attention(f8["q"], f8["k_pool"], f8["v_pool"],
                                      *(f8[n] for n in args), causal=True)
    b = oracle.paged_sparse_attention(deq["q"], deq["k_pool"], deq["v_pool"],
                                      *(deq[n] for n in args), causal=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    vin = wl.make_varlen_inputs(73, [30, 5, 64], [300, 129, 512], 2, 4, 4, wl.MODE_CAUSAL)
    vf = wl.with_fp8_kv(vin)
    cu = (vin["cu_seqlens_q"], vin["cu_seqlens_k"])
    a = oracle.sparse_attention_varlen(vf["q"], vf["k"], vf["v"], vf["q2k"], *cu, causal=True)
    b = oracle.sparse_attention_varlen(vf["q"], wl.fp8_to_bf16_bits(vf["k"]),
                                       wl.fp8_to_bf16_bits(vf["v"]), vf["q2k"], *cu, causal=True)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


def test_quantizer_rounds_to_nearest_even():
    """Input preparation: bf16 values on the fp8 grid are kept; a midpoint goes to the
    even neighbour (1 + 1/16 lies between 1 and 1 + 1/8)."""
    vals = np.array([1.0, 1.0625, 1.1875, -2.5, 448.0], np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    q = wl.bf16_bits_to_fp8(bits)
    assert list(oracle.fp8_e4m3_decode(q)) == [1.0, 1.0, 1.25, -2.5, 448.0]
