"""Seeded random sweep: many small problems of mixed shape against the oracle.

The other GPU tests vary one or two parameters at a time over fixed grids. Here 60
cases are drawn from a seeded generator, each mixing what those grids keep apart: the
layout (contiguous, paged, varlen), the path (auto, q-centric with 0-8 splits,
kv-centric, query tile, union decode), batch, query and key lengths (empty
sequences, partial last blocks, seqused_k trims down to zero keys), KV heads 1-4,
qhead_per_kv 1-16, topk 1-32, causal or not, index recipe, an fp8 e4m3fn K/V cache, a
temperature-scaled LSE and a custom softmax scale. Sixteen more cases are large enough
(at least 2^20 (query, head, slot) triples) that the automatic path takes the kv-centric
kernel, with 1-8 KV heads (1, 2, 4 or 8 item streams), and are compared on sampled
rows. Each case is printed before it runs and compared with the oracle under the usual
parity rules (O max-abs 2e-2, LSE 1e-3, identical empty rows with O = 0, the
temperature LSE within 1e-3 + 1e-3 |ref|).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from parity_util import (bf16_dev_to_f64, check_lse_t, compare, full_compare, say, to_dev)

pytestmark = pytest.mark.gpu

AUTO, Q, KV, DEC, TILE = 0, 1, 2, 3, 4
N_CASES = 60
MAX_ORACLE_FLOP = 3e9


def tile_ok(qpk, topk):
    return qpk in (8, 16) and (256 // qpk) * topk <= 512


def draw_cases(n=N_CASES, seed=2026):
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        c = dict(kind=str(rng.choice(["contig", "paged", "varlen"], p=[0.45, 0.3, 0.25])),
                 qpk=int(rng.choice([1, 2, 4, 8, 16])), Hkv=int(rng.choice([1, 2, 3, 4])),
                 topk=int(rng.choice([1, 2, 3, 4, 5, 8, 11, 16, 32])),
                 causal=bool(rng.random() < 0.6), fp8=bool(rng.random() < 0.25),
                 temp=[None, None, 0.5, 2.0][int(rng.integers(4))],
                 scale=0.0 if rng.random() < 0.7 else float(rng.uniform(0.02, 0.2)),
                 seed=int(rng.integers(1, 1 << 30)))
        Hq = c["Hkv"] * c["qpk"]
        if c["kind"] == "contig":
            c["B"], nblk = int(rng.integers(1, 4)), int(rng.integers(1, 17))
            c["Skv"], c["Sq"] = 128 * nblk, int(rng.integers(1, 400))
            c["mode"] = wl.MODE_CAUSAL if c["causal"] else int(rng.choice([wl.MODE_PERM,
                                                                           wl.MODE_SINK]))
            if c["mode"] != wl.MODE_CAUSAL and c["topk"] > nblk:
                c["mode"] = wl.MODE_CAUSAL
            paths = [AUTO, Q, KV] + ([TILE] if tile_ok(c["qpk"], c["topk"]) and not c["fp8"]
                                     else [])
            c["path"] = int(rng.choice(paths))
            rows, keys = c["B"] * c["Sq"], min(c["topk"], nblk) * 128
        elif c["kind"] == "paged":
            c["B"], nblk = int(rng.integers(1, 5)), int(rng.integers(1, 33))
            c["Skv"] = 128 * nblk
            c["Sq"] = int(rng.integers(1, 17)) if rng.random() < 0.6 else int(rng.integers(17, 300))
            c["trims"] = [int(rng.integers(0, c["Skv"] + 1)) if rng.random() < 0.5 else 0
                          for _ in range(c["B"])]
            if not c["causal"] and c["topk"] > nblk:
                c["causal"] = True  # the causal recipe pads short rows with -1
            dec_ok = c["Sq"] <= 16 and c["Sq"] * c["topk"] <= 512 and not c["fp8"]
            u = rng.random()
            c["path"] = DEC if dec_ok and u < 0.4 else (KV if u >= 0.7 else Q)
            c["splits"] = 0 if c["path"] in (DEC, KV) else int(rng.choice([0, 1, 2, 3, 5, 8]))
            rows, keys = c["B"] * c["Sq"], min(c["topk"], nblk) * 128
        else:
            B = int(rng.integers(1, 5))
            q_lens = [int(rng.integers(0, 200)) if rng.random() < 0.85 else 0 for _ in range(B)]
            k_lens = [int(rng.integers(0, 1500)) if rng.random() < 0.9 else 0 for _ in range(B)]
            q_lens[0], k_lens[0] = max(q_lens[0], 1), max(k_lens[0], 1)
            c.update(q_lens=q_lens, k_lens=k_lens, path=int(rng.choice([AUTO, Q, KV])))
            short = any(0 < k < 128 * c["topk"] for k in k_lens)
            c["mode"] = wl.MODE_CAUSAL if c["causal"] or short else wl.MODE_PERM
            rows, keys = sum(q_lens), 128 * c["topk"]
        if rows * Hq * keys * 128 * 4 > MAX_ORACLE_FLOP:
            continue
        cases.append(c)
    return cases


CASES = draw_cases()


def draw_large_cases(n=16, seed=2027):
    """Problems past the automatic kv-centric threshold (2^20 (query, head, slot)
    triples), contiguous or varlen, compared on sampled rows."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        c = dict(kind=str(rng.choice(["contig", "varlen"])),
                 qpk=int(rng.choice([1, 2, 4, 8, 16])), Hkv=int(rng.choice([1, 2, 3, 4, 6, 8])),
                 topk=int(rng.choice([4, 8, 13, 16, 32])), causal=bool(rng.random() < 0.6),
                 fp8=bool(rng.random() < 0.25), temp=[None, None, 0.5, 2.0][int(rng.integers(4))],
                 scale=0.0 if rng.random() < 0.7 else float(rng.uniform(0.02, 0.2)),
                 path=int(rng.choice([AUTO, KV])), seed=int(rng.integers(1, 1 << 30)))
        Hq = c["Hkv"] * c["qpk"]
        if c["kind"] == "contig":
            c["B"] = int(rng.integers(1, 4))
            nblk = int(rng.integers(max(2, c["topk"] // 2), 65))
            c["Skv"], c["Sq"] = 128 * nblk, int(rng.integers(256, 8193))
            c["mode"] = wl.MODE_CAUSAL if c["causal"] or c["topk"] > nblk else int(
                rng.choice([wl.MODE_PERM, wl.MODE_SINK]))
            nq = c["B"] * c["Sq"]
        else:
            B = int(rng.integers(2, 7))
            c["q_lens"] = [int(rng.integers(0, 4000)) for _ in range(B)]
            c["k_lens"] = [int(rng.integers(1, 9000)) for _ in range(B)]
            short = any(k < 128 * c["topk"] for k in c["k_lens"])
            c["mode"] = wl.MODE_CAUSAL if c["causal"] or short else wl.MODE_PERM
            nq = sum(c["q_lens"])
        if nq * Hq * c["topk"] < (1 << 20) or nq * Hq * 128 * 2 > (3 << 30):
            continue
        cases.append(c)
    return cases


LARGE = draw_large_cases()


def describe(i, c):
    keys = {k: v for k, v in c.items() if k != "seed"}
    return f"[sweep] case {i}: {keys}"


def fp8_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to("cuda").view(torch.float8_e4m3fn)


def kv_dev(inp, names, fp8):
    return [fp8_dev(inp[n]) if fp8 else to_dev(inp[n]) for n in names]


def temp_kw(c):
    return dict(return_temperature_lse=True, lse_temperature_scale=c["temp"]) if c["temp"] else {}


def oracle_scale(c):
    return c["scale"] if c["scale"] > 0 else None


@pytest.mark.parametrize("i", range(len(CASES)))
def test_random_case(i):
    import block_sparse_attention_top_amd as msa
    c = CASES[i]
    say(describe(i, c))
    Hq = c["Hkv"] * c["qpk"]
    if c["kind"] == "contig":
        w = wl.Workload("sweep", B=c["B"], Sq=c["Sq"], Skv=c["Skv"], Hkv=c["Hkv"], qpk=c["qpk"],
                        topk=c["topk"], causal=c["causal"], mode=c["mode"], seed=c["seed"])
        inp = wl.make_inputs(w)
        if c["fp8"]:
            inp = wl.with_fp8_kv(inp)
        k, v = kv_dev(inp, ("k", "v"), c["fp8"])
        out = msa.msa_sparse_fwd(to_dev(inp["q"]), k, v, to_dev(inp["q2k"]), causal=c["causal"],
                                 path=c["path"], softmax_scale=c["scale"], **temp_kw(c))
        ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                      causal=c["causal"], softmax_scale=oracle_scale(c),
                                      temperature=c["temp"])
    elif c["kind"] == "paged":
        mode = wl.MODE_CAUSAL if c["causal"] else wl.MODE_PERM
        w = wl.Workload("sweep", B=c["B"], Sq=c["Sq"], Skv=c["Skv"], Hkv=c["Hkv"], qpk=c["qpk"],
                        topk=c["topk"], causal=c["causal"], mode=mode, paged=True,
                        shuffle_pages=True, seed=c["seed"])
        inp = wl.make_inputs(w, q2k=np.zeros((1,), np.int32))
        seqused = np.array([c["Skv"] - t for t in c["trims"]], dtype=np.int32)
        inp["seqused_k"] = seqused
        lens = seqused if c["causal"] else np.full(c["B"], c["Skv"], dtype=np.int32)
        inp["q2k"] = np.concatenate([wl.q2k_table(c["seed"] + b, mode, 1, c["Hkv"], c["Sq"],
                                                  int(lens[b]), 128, c["topk"])
                                     for b in range(c["B"])], 0)
        if c["fp8"]:
            inp = wl.with_fp8_kv(inp)
        kp, vp = kv_dev(inp, ("k_pool", "v_pool"), c["fp8"])
        out = msa.msa_paged_sparse_fwd(to_dev(inp["q"]), kp, vp, to_dev(inp["page_table"]),
                                       to_dev(inp["seqused_k"]), to_dev(inp["q2k"]),
                                       causal=c["causal"], num_splits=c["splits"],
                                       path=c["path"], softmax_scale=c["scale"], **temp_kw(c))
        ref = oracle.paged_sparse_attention(inp["q"], inp["k_pool"], inp["v_pool"],
                                            inp["page_table"], inp["seqused_k"], inp["q2k"],
                                            causal=c["causal"], softmax_scale=oracle_scale(c),
                                            temperature=c["temp"])
    else:
        inp = wl.make_varlen_inputs(c["seed"], c["q_lens"], c["k_lens"], c["Hkv"], c["qpk"],
                                    c["topk"], c["mode"])
        if c["fp8"]:
            inp = wl.with_fp8_kv(inp)
        k, v = kv_dev(inp, ("k", "v"), c["fp8"])
        out = msa.msa_sparse_fwd_varlen(to_dev(inp["q"]), k, v, to_dev(inp["q2k"]),
                                        to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"]),
                                        causal=c["causal"], path=c["path"],
                                        softmax_scale=c["scale"], **temp_kw(c))
        ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                             causal=c["causal"], softmax_scale=oracle_scale(c),
                                             temperature=c["temp"])
    torch.cuda.synchronize()
    o, lse = out[0], out[1]
    o_ref, lse_ref = ref[0], ref[1]
    if c["kind"] == "varlen":  # packed layouts: O [total_q,Hq,D], LSE [total_q,Hq]
        compare(bf16_dev_to_f64(o), lse.cpu().numpy().astype(np.float64), o_ref, lse_ref,
                f"case {i}")
    else:
        full_compare(o, lse, o_ref, lse_ref, f"case {i}")
    if c["temp"]:
        check_lse_t(out[2].cpu().numpy(), ref[2], f"case {i} temperature")
    assert o.shape[-2] == Hq


@pytest.mark.parametrize("i", range(len(LARGE)))
def test_random_large_case(i):
    """Sampled rows (first, last, spread and random) of a problem the automatic path
    sends to the kv-centric kernel; the path it took is checked too."""
    import block_sparse_attention_top_amd as msa
    c = LARGE[i]
    say(describe(i, c).replace("[sweep]", "[sweep-large]"))
    Hq = c["Hkv"] * c["qpk"]
    if c["kind"] == "contig":
        assert msa.msa_sparse_fwd_path(c["B"], c["Sq"], c["Skv"], Hq, c["Hkv"], c["topk"],
                                       c["path"]) == KV
        w = wl.Workload("sweep", B=c["B"], Sq=c["Sq"], Skv=c["Skv"], Hkv=c["Hkv"], qpk=c["qpk"],
                        topk=c["topk"], causal=c["causal"], mode=c["mode"], seed=c["seed"])
        inp = wl.make_inputs(w)
        nq = c["B"] * c["Sq"]
    else:
        assert msa.msa_sparse_fwd_varlen_path(len(c["q_lens"]), sum(c["q_lens"]),
                                              sum(c["k_lens"]), Hq, c["Hkv"], c["topk"],
                                              c["path"]) == KV
        inp = wl.make_varlen_inputs(c["seed"], c["q_lens"], c["k_lens"], c["Hkv"], c["qpk"],
                                    c["topk"], c["mode"])
        nq = sum(c["q_lens"])
    if c["fp8"]:
        inp = wl.with_fp8_kv(inp)
    k, v = kv_dev(inp, ("k", "v"), c["fp8"])
    rng = np.random.default_rng(i)
    rows = np.unique(np.concatenate([[0, nq - 1], np.linspace(0, nq - 1, 48).astype(np.int64),
                                     rng.integers(0, nq, 46)]))
    if c["kind"] == "contig":
        out = msa.msa_sparse_fwd(to_dev(inp["q"]), k, v, to_dev(inp["q2k"]), causal=c["causal"],
                                 path=c["path"], softmax_scale=c["scale"], **temp_kw(c))
        ref = oracle.sparse_attention(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                      causal=c["causal"], softmax_scale=oracle_scale(c),
                                      temperature=c["temp"], rows=rows)
        torch.cuda.synchronize()
        b, s = rows // c["Sq"], rows % c["Sq"]
        og = out[0][b, s].float().cpu().numpy().astype(np.float64)
        lg = out[1][b, :, s].cpu().numpy().astype(np.float64)
        lt = out[2][b, :, s].cpu().numpy() if c["temp"] else None
    else:
        out = msa.msa_sparse_fwd_varlen(to_dev(inp["q"]), k, v, to_dev(inp["q2k"]),
                                        to_dev(inp["cu_seqlens_q"]), to_dev(inp["cu_seqlens_k"]),
                                        causal=c["causal"], path=c["path"],
                                        softmax_scale=c["scale"], **temp_kw(c))
        ref = oracle.sparse_attention_varlen(inp["q"], inp["k"], inp["v"], inp["q2k"],
                                             inp["cu_seqlens_q"], inp["cu_seqlens_k"],
                                             causal=c["causal"], softmax_scale=oracle_scale(c),
                                             temperature=c["temp"], rows=rows)
        torch.cuda.synchronize()
        og = out[0][rows].float().cpu().numpy().astype(np.float64)
        lg = out[1][rows].cpu().numpy().astype(np.float64)
        lt = out[2][rows].cpu().numpy() if c["temp"] else None
    compare(og, lg, ref[0], ref[1], f"large case {i}")
    if c["temp"]:
        check_lse_t(lt, ref[2], f"large case {i} temperature")


def draw_csr_cases(n=24, seed=2030):
    """Random index tables for the public k2q CSR builders: ids uniform with
    replacement (so repeats within a row occur), holes (-1) and ids past the blocks,
    CSR row counts in each of the ordered builder's three scatters (per-row lane masks
    in LDS up to 2048 rows, per-wave hash slots up to 9216, one wave per tile up to
    the builders' 16384); contiguous or varlen (empty sequences included)."""
    rng = np.random.default_rng(seed)
    out = []
    while len(out) < n:
        c = dict(varlen=bool(rng.random() < 0.35), Hkv=int(rng.integers(1, 5)),
                 topk=int(rng.integers(1, 33)), p_hole=float(rng.choice([0.0, 0.05, 0.3])),
                 p_oob=float(rng.choice([0.0, 0.02])), seed=int(rng.integers(1, 1 << 30)))
        if c["varlen"]:
            B = int(rng.integers(1, 7))
            c["q_lens"] = [0 if rng.random() < 0.15 else int(rng.integers(1, 1500))
                           for _ in range(B)]
            c["k_lens"] = [0 if rng.random() < 0.15 else int(rng.integers(1, 150000))
                           for _ in range(B)]
            c["k_lens"][0] = max(c["k_lens"][0], 1)
            entries = sum(c["q_lens"]) * c["Hkv"] * c["topk"]
        else:
            c["B"], c["Sq"] = int(rng.integers(1, 5)), int(rng.integers(1, 3000))
            # CSR rows (B * nblk): 45% ranked by masks, 40% by hash slots, 15% past both
            u = rng.random()
            rows = (int(rng.integers(1, 2049)) if u < 0.45 else
                    int(rng.integers(2049 + c["B"], 9217)) if u < 0.85 else
                    int(rng.integers(9217 + c["B"], 16385)))  # the builders take 16384 rows
            c["nblk"] = max(1, rows // c["B"])
            entries = c["B"] * c["Sq"] * c["Hkv"] * c["topk"]
        if entries == 0 or entries > (2 << 20):
            continue
        out.append(c)
    return out


CSR_CASES = draw_csr_cases()


def _holes(rng, q2k, c, nblk_max):
    q2k[rng.random(q2k.shape) < c["p_hole"]] = -1
    q2k[rng.random(q2k.shape) < c["p_oob"]] = nblk_max + int(rng.integers(0, 5))
    return q2k


@pytest.mark.parametrize("i", range(len(CSR_CASES)))
def test_random_csr(i):
    import block_sparse_attention_top_amd as msa
    c = CSR_CASES[i]
    say(f"[sweep-csr] case {i}: { {k: v for k, v in c.items() if k != 'seed'} }")
    rng = np.random.default_rng(c["seed"])
    if c["varlen"]:
        cu_q, cu_k = wl.cu_seqlens(c["q_lens"]), wl.cu_seqlens(c["k_lens"])
        total_q = int(cu_q[-1])
        q2k = np.full((c["Hkv"], total_q, c["topk"]), -1, dtype=np.int32)
        for b in range(len(c["q_lens"])):
            nb = -(-c["k_lens"][b] // 128)
            if nb and c["q_lens"][b]:
                q2k[:, cu_q[b]:cu_q[b + 1]] = rng.integers(0, nb, (c["Hkv"], c["q_lens"][b],
                                                                   c["topk"]))
        q2k = _holes(rng, q2k, c, max(-(-k // 128) for k in c["k_lens"]))
        total_rows = oracle.varlen_total_rows(cu_k)
        rp, qi, sl = msa.msa_build_k2q_csr_varlen(to_dev(q2k), to_dev(cu_q), to_dev(cu_k),
                                                  int(cu_k[-1]), total_rows)
        ref = oracle.k2q_csr_varlen(q2k, cu_q, cu_k)
    else:
        q2k = rng.integers(0, c["nblk"], (c["B"], c["Hkv"], c["Sq"], c["topk"])).astype(np.int32)
        q2k = _holes(rng, q2k, c, c["nblk"])
        rp, qi, sl = msa.msa_build_k2q_csr(to_dev(q2k), c["nblk"])
        ref = oracle.k2q_csr(q2k, c["nblk"])
    torch.cuda.synchronize()
    rp, qi, sl = rp.cpu().numpy(), qi.cpu().numpy(), sl.cpu().numpy()
    assert np.array_equal(rp, ref[0]), "row_ptr differs"
    for h in range(c["Hkv"]):
        n = ref[0][h, -1]
        assert np.array_equal(qi[h, :n], ref[1][h, :n]), f"q_idx differs (h={h})"
        assert np.array_equal(sl[h, :n], ref[2][h, :n]), f"slot differs (h={h})"
