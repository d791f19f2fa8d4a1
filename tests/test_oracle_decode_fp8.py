"""Pins of the oracle's e4m3 rounding and of its fp8 dense paged decode (the test
page's `_decode_paged_dense_reference`: fp8 Q/K/V, probabilities rounded to e4m3 before
P V, unrounded row sum).

Rounding is pinned against an independent brute-force nearest-code search over every
finite e4m3fn value (ties to the even code) and against torch's float8_e4m3fn cast.
The decode is pinned by closed forms (a zero query averages the visible values; two
keys with scores 0 and -1 weight the second value by e4m3(e^-1) = 0.375) and against
the already-pinned paged oracle: the LSE does not depend on the rounding (equal to
1e-12), the output differs from the unrounded one by at most the rounding bound and
does differ somewhere."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl


def finite_codes():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.fp8_e4m3_decode(codes)
    ok = np.isfinite(vals)
    return codes[ok], vals[ok]


def brute_round(x):
    """Nearest finite e4m3fn value by exhaustive search; ties go to the code whose
    mantissa's last bit is 0; beyond 464 (and 464 itself, the tie with the missing
    next code) NaN, as the non-saturating cast gives."""
    codes, vals = finite_codes()
    out = np.empty_like(x)
    for i, v in enumerate(x):
        if abs(v) >= 464.0:
            out[i] = np.nan
            continue
        d = np.abs(vals - v)
        best = d.min()
        cand = codes[d == best]
        if len(cand) > 1:
            cand = cand[(cand & 1) == 0]
        # +0 and -0 tie for v = 0; either has value 0
        out[i] = oracle.fp8_e4m3_decode(cand[:1])[0]
    return out


def test_round_fixes_every_code():
    _, vals = finite_codes()
    assert np.array_equal(oracle.fp8_e4m3_round(vals), vals)


def test_round_matches_brute_force_nearest():
    _, vals = finite_codes()
    pos = np.unique(vals[vals >= 0])
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(3)
    x = np.concatenate([mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                        rng.uniform(0, 470, 3000), rng.uniform(0, 0.02, 2000),
                        -rng.uniform(0, 300, 500)])
    got, want = oracle.fp8_e4m3_round(x), brute_round(x)
    both_nan = np.isnan(got) & np.isnan(want)
    assert np.array_equal(got[~both_nan], want[~both_nan]) and np.array_equal(np.isnan(got), np.isnan(want))


def test_round_matches_torch_cast():
    rng = np.random.default_rng(4)
    x = np.concatenate([rng.uniform(0, 440, 20000), np.geomspace(1e-6, 1.0, 20000),
                        -rng.uniform(0, 440, 5000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    assert np.array_equal(oracle.fp8_e4m3_round(x.astype(np.float64)), ref)


def fp8_bytes(a: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(
        torch.float8_e4m3fn).view(torch.uint8).numpy()


def pools(rng, num_pages, Hkv, D=128):
    k = fp8_bytes(rng.standard_normal((num_pages, Hkv, 128, D)))
    v = fp8_bytes(rng.standard_normal((num_pages, Hkv, 128, D)))
    return k, v


def test_zero_query_averages_the_visible_values():
    rng = np.random.default_rng(5)
    B, Sq, Hkv, qpk, pages = 2, 3, 2, 4, 3
    k, v = pools(rng, B * pages, Hkv)
    pt = rng.permutation(B * pages).astype(np.int32).reshape(B, pages)
    seq = np.array([300, 129], dtype=np.int32)
    q = np.zeros((B, Sq, Hkv * qpk, 128), dtype=np.uint8)  # e4m3 0x00 = +0
    o, lse = oracle.paged_decode_fp8(q, k, v, pt, seq, causal=True)
    vd = oracle.fp8_e4m3_decode(v)
    for b in range(B):
        for s in range(Sq):
            n = seq[b] - Sq + s + 1  # causal: keys 0 .. q + seqused - Sq
            rows = np.concatenate([vd[pt[b, j // 128], :, j % 128][None] for j in range(n)])
            mean = rows.mean(axis=0)  # [Hkv, D]
            for h in range(Hkv * qpk):
                assert np.allclose(o[b, s, h], mean[h // qpk], rtol=0, atol=1e-12)
                assert abs(lse[b, h, s] - math.log(n)) < 1e-12


def test_two_keys_weight_the_second_value_by_the_rounded_probability():
    """q = e_0, k_0 = 0, k_1 = -e_0, scale 1: scores 0 and -1, probabilities 1 and
    e^-1 = 0.3679, which rounds to 0.375 (1.5 x 2^-2) in e4m3; the row sum keeps
    1 + e^-1."""
    rng = np.random.default_rng(6)
    D = 128
    kf = np.zeros((1, 1, 128, D), dtype=np.float32)
    kf[0, 0, 1, 0] = -1.0
    k = fp8_bytes(kf)
    v = fp8_bytes(rng.standard_normal((1, 1, 128, D)))
    qf = np.zeros((1, 1, 1, D), dtype=np.float32)
    qf[0, 0, 0, 0] = 1.0
    q = fp8_bytes(qf)
    o, lse = oracle.paged_decode_fp8(q, k, v, np.zeros((1, 1), np.int32), np.array([2], np.int32),
                                     causal=False, softmax_scale=1.0)
    vd = oracle.fp8_e4m3_decode(v)[0, 0]
    want = (vd[0] + 0.375 * vd[1]) / (1 + math.exp(-1))
    assert np.allclose(o[0, 0, 0], want, rtol=0, atol=1e-12)
    assert abs(lse[0, 0, 0] - math.log(1 + math.exp(-1))) < 1e-12


@pytest.mark.parametrize("causal", [True, False])
def test_against_the_unrounded_paged_oracle(causal):
    rng = np.random.default_rng(7)
    B, Sq, Hkv, qpk, max_pages = 3, 5, 2, 4, 4
    k, v = pools(rng, B * max_pages + 2, Hkv)
    pt = rng.permutation(B * max_pages + 2)[:B * max_pages].astype(np.int32).reshape(B, max_pages)
    pt[1, 2] = -1  # a page outside the pool contributes nothing
    seq = np.array([450, 200, 3], dtype=np.int32)
    q8 = fp8_bytes(rng.standard_normal((B, Sq, Hkv * qpk, 128)))
    o, lse, lt = oracle.paged_decode_fp8(q8, k, v, pt, seq, causal=causal, temperature=2.0)
    # the same scores through the paged oracle: Q's fp8 values are exact in bf16
    qb = wl.fp8_to_bf16_bits(q8)
    full = np.ascontiguousarray(np.broadcast_to(np.arange(max_pages, dtype=np.int32),
                                                (B, Hkv, Sq, max_pages)))
    o_ref, lse_ref, lt_ref = oracle.paged_sparse_attention(qb, k, v, pt, seq, full, causal=causal,
                                                           temperature=2.0)
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert np.max(np.abs(lse[fin] - lse_ref[fin])) < 1e-12
    assert np.max(np.abs(lt[fin] - lt_ref[fin])) < 1e-12
    # rounding bound: |e4m3(p) - p| <= max(p / 16, 2^-10) with p <= 1, and the row sum >= 1
    vmax = np.abs(oracle.fp8_e4m3_decode(v)).max()
    diff = np.abs(o - o_ref).max()
    assert diff <= (1 / 16 + 512 * 2 ** -10) * vmax
    assert diff > 0  # the rounding is applied
