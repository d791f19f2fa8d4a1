"""Host-side logic of the library that needs no GPU.

query_bucket (msa_internal.hpp) assigns each kv-centric work item to one of 256
query ranges by its first query; the item-table and item-order kernels must agree
on it for every query count the API accepts, including query ids past 2^23, where
q * 256 no longer fits in 32 bits. The helper is compiled into a host program and
compared with exact integer arithmetic.

kv_item_slot (msa_internal.hpp) gives each kv-centric work item (a chunk of a CSR row)
a fixed slot in the unsorted item table, so that the scatter can list items without a
shared counter; two items must never share a slot, and every slot must fit the table.
"""
import os
import subprocess

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "host", "query_bucket_check.cpp")


def _build(tmp_path_factory, src, name):
    exe = str(tmp_path_factory.mktemp("host") / name)
    subprocess.check_call(["/opt/rocm/bin/hipcc", "-O1", "-std=c++17", "-x", "hip",
                           "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
                           "-packed-fp32-ops", src, "-o", exe],
                          stderr=subprocess.DEVNULL)
    return exe


@pytest.fixture(scope="module")
def bucket_exe(tmp_path_factory):
    return _build(tmp_path_factory, SRC, "query_bucket_check")


@pytest.fixture(scope="module")
def slot_exe(tmp_path_factory):
    return _build(tmp_path_factory, os.path.join(HERE, "host", "kv_item_slot_check.cpp"),
                  "kv_item_slot_check")


def _run(exe, triples):
    inp = "".join(f"{q} {nq} {b}\n" for q, nq, b in triples)
    out = subprocess.run([exe], input=inp, capture_output=True, text=True, check=True).stdout
    return [int(x) for x in out.split()]


def test_query_bucket_exact_past_2_pow_23(bucket_exe):
    rng = np.random.default_rng(7)
    triples = []
    # query counts the API accepts (B*Sq*topk < 2^31 with topk >= 1), around and past 2^23
    for nq in (1, 3, 8192, 393216, (1 << 23) - 1, 1 << 23, 9_000_000, 134_217_727,
               (1 << 31) - 1):
        qs = {0, nq - 1, nq // 2, min(nq - 1, 1 << 23), min(nq - 1, (1 << 23) + 1)}
        qs |= set(int(x) for x in rng.integers(0, nq, size=16))
        triples += [(q, nq, 256) for q in sorted(qs)]
    got = _run(bucket_exe, triples)
    want = [min(q * b // nq, b - 1) for q, nq, b in triples]
    assert got == want


def test_query_bucket_monotone_and_in_range(bucket_exe):
    nq = 9_000_000
    qs = list(range(0, nq, 4099)) + [nq - 1]
    got = _run(bucket_exe, [(q, nq, 256) for q in qs])
    assert min(got) == 0 and max(got) == 255
    assert all(a <= b for a, b in zip(got, got[1:]))


@pytest.mark.parametrize("Hkv,shift,nrows,seed", [(1, 7, 64, 0), (4, 7, 200, 1), (2, 9, 300, 2),
                                                   (3, 8, 50, 3), (1, 9, 3072, 4)])
def test_kv_item_slots_distinct_and_in_range(slot_exe, Hkv, shift, nrows, seed):
    rng = np.random.default_rng(seed)
    chunk = 1 << shift
    # rows of every kind: empty, one entry, a chunk and one more (a last chunk of one
    # entry, followed at once by the next row's first chunk), exact multiples, long rows
    kinds = [0, 1, chunk, chunk + 1, 2 * chunk - 1, 3 * chunk]
    lens = [int(rng.choice(kinds)) if rng.random() < 0.5 else int(rng.integers(0, 6 * chunk))
            for _ in range(Hkv * nrows)]
    inp = f"len {Hkv} {shift} {nrows}\n" + " ".join(map(str, lens)) + "\n"
    out = subprocess.run([slot_exe], input=inp, capture_output=True, text=True,
                         check=True).stdout.split()
    per_head = int(out[0])
    slots = [int(x) for x in out[1:]]
    n_items = sum((n + chunk - 1) // chunk for n in lens)
    assert len(slots) == n_items
    assert len(set(slots)) == n_items
    assert min(slots, default=0) >= 0 and max(slots, default=0) < Hkv * per_head


@pytest.mark.parametrize("kind", ["valid", "descent", "negative", "past_cap", "huge",
                                  "random"])
def test_kv_caller_row_ptr_checked(slot_exe, kind):
    """A caller's CSR row_ptr is not trusted by the kv-centric item kernel: a row is
    listed only if 0 <= row_ptr[r] <= row_ptr[r + 1] <= cap (kv_row_ok), any failing
    row voids the item order, and every listed chunk must then lie in [0, cap) with
    its slot inside the table; with no failing row the slots must be distinct."""
    rng = np.random.default_rng(11)
    Hkv, shift, nrows, cap = 3, 7, 60, 60 * 200
    chunk = 1 << shift
    rp = []
    for _ in range(Hkv):
        lens = rng.integers(0, 4 * chunk, size=nrows)
        lens = (lens * cap // max(int(lens.sum()), cap)).astype(np.int64)
        rp.append(np.concatenate([[0], np.cumsum(lens)]))
    rp = np.stack(rp)
    if kind == "descent":
        rp[1, 17], rp[1, 18] = rp[1, 18] + 5, rp[1, 17]
    elif kind == "negative":
        rp[0, 0] = -5
    elif kind == "past_cap":
        rp[2, nrows] = cap + 1
    elif kind == "huge":
        rp[1, 30:] = (1 << 31) - 1
    elif kind == "random":
        rp = rng.integers(-cap, 2 * cap, size=rp.shape)
    want_bad = any(not (0 <= rp[h, r] <= rp[h, r + 1] <= cap)
                   for h in range(Hkv) for r in range(nrows))
    assert want_bad == (kind != "valid")
    inp = f"ptr {Hkv} {shift} {nrows} {cap}\n" + " ".join(map(str, rp.ravel())) + "\n"
    out = subprocess.run([slot_exe], input=inp, capture_output=True, text=True,
                         check=True).stdout.split()
    per_head, bad = int(out[0]), int(out[1])
    assert per_head == cap // chunk + nrows + 1
    assert bad == int(want_bad)
    items = np.array([int(x) for x in out[2:]], dtype=np.int64).reshape(-1, 3)
    if len(items):
        slot, beg, end = items[:, 0], items[:, 1], items[:, 2]
        assert slot.min() >= 0 and slot.max() < Hkv * per_head
        assert beg.min() >= 0 and end.max() <= cap and (beg < end).all()
    if not want_bad:
        assert len(set(items[:, 0].tolist())) == len(items)
        n_items = sum(-(-int(rp[h, r + 1] - rp[h, r]) // chunk)
                      for h in range(Hkv) for r in range(nrows))
        assert len(items) == n_items


def test_bench_skew_diagnostics_brute_force():
    """bench.py's index-skew summary (CSR row lengths, block-0 share, per-query fan-out)
    against a brute-force count over a small table with -1 and out-of-range ids."""
    import sys
    sys.path.insert(0, os.path.dirname(HERE))
    import bench
    import workloads as wl
    w = wl.Workload("tiny", B=2, Sq=40, Skv=640, Hkv=2, qpk=2, topk=4, causal=True,
                    mode=wl.MODE_CAUSAL)
    rng = np.random.default_rng(3)
    q2k = rng.integers(-2, 7, size=(w.B, w.Hkv, w.Sq, w.topk)).astype(np.int32)  # 5 blocks
    d = bench.skew_diagnostics(w, q2k)
    nblk = w.Skv // w.blk
    counts = {}
    per_row = []
    b0 = 0
    for b in range(w.B):
        for h in range(w.Hkv):
            for q in range(w.Sq):
                n = 0
                for t in range(w.topk):
                    s = int(q2k[b, h, q, t])
                    if 0 <= s < nblk:
                        counts[(h, b * nblk + s)] = counts.get((h, b * nblk + s), 0) + 1
                        n += 1
                        b0 += s == 0
                per_row.append(n)
    allc = [counts.get((h, r), 0) for h in range(w.Hkv) for r in range(w.B * nblk)]
    assert d["valid_entries"] == sum(allc) == sum(per_row)
    assert d["csr_rows"] == len(allc)
    assert d["row_len_max"] == max(allc)
    assert d["empty_rows"] == sum(c == 0 for c in allc)
    assert abs(d["row_len_mean"] - np.mean(allc)) < 0.06
    assert d["block0_share"] == round(b0 / sum(allc), 4)
    assert d["fanout_min"] == min(per_row)
    assert d["queries_with_no_slot"] == sum(n == 0 for n in per_row)
