"""The C ABI library loads, exports every entry point include/msa.h declares, and
rejects bad arguments on the host before any launch (no GPU needed: every call
here fails validation, so no device memory is touched)."""
import ctypes
import os
import re

import pytest

import block_sparse_attention_top_amd as msa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(msa_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert {"msa_sparse_fwd", "msa_build_k2q_csr", "msa_paged_sparse_fwd",
            "msa_last_error"} <= set(names)
    lib = ctypes.CDLL(msa.lib_path())
    for name in names:
        assert hasattr(lib, name), name


def test_version():
    assert msa.msa_version().startswith("msa-gfx950")


FAKE = 0x10000  # never dereferenced: every call below fails host validation first


def fwd(**kw):
    lib = msa.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, q2k=FAKE, rp=None, qi=None, sl=None, B=1, Sq=256, Skv=256,
             Hq=16, Hkv=1, D=128, topk=4, blk=128, causal=1, scale=0.0, path=0, kvd=0, o=FAKE,
             lse=FAKE, temp=1.0, lset=None, ws=None, wsb=0)
    a.update(kw)
    return lib.msa_sparse_fwd(a["q"], a["k"], a["v"], a["q2k"], a["rp"], a["qi"], a["sl"], a["B"],
                              a["Sq"], a["Skv"], a["Hq"], a["Hkv"], a["D"], a["topk"], a["blk"],
                              a["causal"], a["scale"], a["path"], a["kvd"], a["o"], a["lse"],
                              a["temp"], a["lset"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), 2), (dict(blk=64), 2), (dict(Hq=3, Hkv=1), 2), (dict(Hq=32, Hkv=1), 2),
    (dict(Hq=6, Hkv=4), 1), (dict(topk=33), 2), (dict(topk=0), 1), (dict(B=0), 1),
    (dict(Sq=0), 1), (dict(Skv=200), 1), (dict(q=None), 1), (dict(o=FAKE + 8), 1),
    (dict(lse=FAKE + 2), 1), (dict(path=7), 1), (dict(rp=FAKE), 1),
    # temperature-scaled LSE: T must be positive and finite, the buffer aligned
    (dict(lset=FAKE, temp=0.0), 1), (dict(lset=FAKE, temp=-2.0), 1),
    (dict(lset=FAKE, temp=float("inf")), 1), (dict(lset=FAKE, temp=float("nan")), 1),
    (dict(lset=FAKE + 2, temp=2.0), 1),
    # K/V dtype: unknown code; fp8 on the query-tile path
    (dict(kvd=2), 1), (dict(kvd=-1), 1), (dict(kvd=1, path=4), 2),
    # kv-centric without (enough) workspace
    (dict(path=2), 1), (dict(path=2, ws=FAKE, wsb=16), 1),
    # kv-centric with too many CSR rows for the LDS-resident passes
    (dict(path=2, Skv=128 * 20000), 2),
])
def test_sparse_fwd_rejects(kw, code):
    assert fwd(**kw) == code
    assert msa.msa_last_error() != ""


def test_workspace_queries():
    # q-centric needs none; kv-centric needs partials (topk * rows * heads * 256 B) and more
    assert msa.msa_sparse_fwd_workspace_size(1, 1024, 1024, 64, 4, 128, 16, 128, 1) == 0
    n = msa.msa_sparse_fwd_workspace_size(1, 1024, 1024, 64, 4, 128, 16, 128, 2)
    assert n >= 1024 * 16 * 64 * 128 * 2
    assert msa.msa_sparse_fwd_workspace_size(1, 1024, 1000, 64, 4, 128, 16, 128, 2) == 0
    assert msa.msa_build_k2q_csr_workspace_size(1, 4, 8192, 16, 64) > 0
    # paged: one split needs no workspace, several need fp32 partials
    for path in (0, 1, 3):
        assert msa.msa_paged_sparse_fwd_workspace_size(32, 8, 64, 4, 128, 16, 128, 512, 1,
                                                       path) == 0
        assert msa.msa_paged_sparse_fwd_workspace_size(32, 8, 64, 4, 128, 16, 128, 512, 4,
                                                       path) >= 4 * 32 * 8 * 64 * 128 * 4
    # the decode kernel splits the union of a (b, hkv)'s blocks: up to min(Sq*topk, 64) splits
    assert msa.msa_paged_sparse_fwd_splits(1, 8, 1, 16, 512, 100, 3) == 64
    assert msa.msa_paged_sparse_fwd_splits(1, 8, 1, 16, 512, 100, 1) == 16
    assert msa.msa_paged_sparse_fwd_splits(1, 1, 1, 4, 512, 0, 3) == 4
    assert msa.msa_paged_sparse_fwd_splits(1, 8, 1, 16, 512, 100, 2) == 1  # kv: no splits
    assert msa.msa_paged_sparse_fwd_workspace_size(1, 8, 16, 1, 128, 16, 128, 512, 64, 3) >= \
        64 * 8 * 16 * 128 * 4
    # the paged kv-centric path takes the contiguous one's workspace over max_pages blocks
    assert msa.msa_paged_sparse_fwd_workspace_size(1, 8, 16, 1, 128, 16, 128, 512, 4, 2) == \
        msa.msa_sparse_fwd_workspace_size(1, 8, 512 * 128, 16, 1, 128, 16, 128, 2) > 0
    assert msa.msa_paged_sparse_fwd_workspace_size(1, 8, 16, 1, 128, 16, 128, 512, 4, 4) == 0


def test_csr_and_paged_reject():
    lib = msa.load_library()
    assert lib.msa_build_k2q_csr(FAKE, 1, 1, 16, 33, 8, FAKE, FAKE, None, FAKE, 1 << 20,
                                 None) == 2
    assert lib.msa_build_k2q_csr(FAKE, 1, 1, 16, 4, 8, FAKE, FAKE, None, None, 0, None) == 1
    assert lib.msa_build_k2q_csr(None, 1, 1, 16, 4, 8, FAKE, FAKE, None, FAKE, 1 << 20,
                                 None) == 1
    # paged: page_size != 128, missing seqused_k, forced splits without workspace,
    # negative splits, unknown or kv-centric path, decode path with Sq > 16
    args = [FAKE] * 6 + [32, 8, 64, 4, 128, 16, 128, 16384, 512, 1, 0.0, 0, 0, 0, FAKE, FAKE,
                         1.0, None, None, 0, None]
    a = list(args); a[12] = 64
    assert lib.msa_paged_sparse_fwd(*a) == 2
    a = list(args); a[4] = None
    assert lib.msa_paged_sparse_fwd(*a) == 1
    for path in (0, 1, 3):
        a = list(args); a[17] = 4; a[18] = path
        assert lib.msa_paged_sparse_fwd(*a) == 1
    a = list(args); a[17] = -1
    assert lib.msa_paged_sparse_fwd(*a) == 1
    a = list(args); a[18] = 2
    assert lib.msa_paged_sparse_fwd(*a) == 1
    a = list(args); a[18] = 3; a[7] = 17
    assert lib.msa_paged_sparse_fwd(*a) == 2
    a = list(args); a[22] = 0.0; a[23] = FAKE  # temperature buffer with T = 0
    assert lib.msa_paged_sparse_fwd(*a) == 1
    a = list(args); a[18] = 3; a[19] = 1  # fp8 K/V on the decode path
    assert lib.msa_paged_sparse_fwd(*a) == 2
    a = list(args); a[19] = 5  # unknown K/V dtype
    assert lib.msa_paged_sparse_fwd(*a) == 1


def test_missing_library_raises(monkeypatch, tmp_path):
    from block_sparse_attention_top_amd import _ffi
    monkeypatch.setattr(_ffi, "_lib", None)
    monkeypatch.setattr(_ffi, "_LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(ImportError):
        _ffi.load_library()


def test_profiling_events_must_pair():
    lib = msa.load_library()
    assert lib.msa_set_profiling_events(FAKE, None) == 1
    assert lib.msa_set_profiling_events(None, FAKE) == 1
    assert lib.msa_set_profiling_events(None, None) == 0


def test_auto_path_resolution():
    # small problems take the q-centric path, large ones the kv-centric path
    assert msa.msa_sparse_fwd_path(1, 1024, 1024, 2, 1, 4, 0) == 1
    assert msa.msa_sparse_fwd_path(1, 8192, 8192, 64, 4, 16, 0) == 2
    # the switch is at 32768 (query, KV head, block) units, B * Sq * Hkv * min(topk, nblk),
    # whatever qhead_per_kv is
    assert msa.msa_sparse_fwd_path(1, 1024, 1024, 4, 4, 8, 0) == 2    # 1024 * 4 * 8
    assert msa.msa_sparse_fwd_path(1, 1023, 1024, 4, 4, 8, 0) == 1    # one query fewer
    assert msa.msa_sparse_fwd_path(1, 1024, 1024, 64, 4, 16, 0) == 2  # min(16, 8 blocks)
    assert msa.msa_sparse_fwd_path(1, 512, 512, 64, 4, 16, 0) == 1    # 512 * 4 * 4
    assert msa.msa_sparse_fwd_path(1, 8192, 8192, 4, 4, 16, 0) == 2   # qhead_per_kv 1
    # one sequence with more blocks than the kv-centric passes hold -> q-centric; a batch
    # with more rows in all stays kv-centric (sub-batches of whole sequences)
    assert msa.msa_sparse_fwd_path(1, 8192, 128 * 20000, 64, 4, 16, 0) == 1
    assert msa.msa_sparse_fwd_path(4, 4096, 128 * 8192, 64, 4, 16, 0) == 2
    # short query sets over long keys: each block serves about Sq * topk / nblk entries,
    # and the kv-centric path needs two or more per block on average
    assert msa.msa_sparse_fwd_path(64, 8, 65536, 64, 4, 16, 0) == 1    # 0.25 per block
    assert msa.msa_sparse_fwd_path(16, 32, 65536, 64, 4, 16, 0) == 1   # 1
    assert msa.msa_sparse_fwd_path(8, 64, 65536, 64, 4, 16, 0) == 2    # 2
    assert msa.msa_sparse_fwd_path(64, 8, 8192, 64, 4, 16, 0) == 2     # 2
    ws4 = msa.msa_sparse_fwd_workspace_size(4, 4096, 128 * 8192, 64, 4, 128, 16, 128, 2)
    ws2 = msa.msa_sparse_fwd_workspace_size(2, 4096, 128 * 8192, 64, 4, 128, 16, 128, 2)
    assert ws4 == ws2 > 0  # sized for one sub-batch of two sequences
    assert msa.msa_sparse_fwd_workspace_size(1, 8192, 128 * 20000, 64, 4, 128, 16, 128, 2) == 0
    assert msa.msa_sparse_fwd_path(1, 8192, 8192, 64, 4, 16, 1) == 1
    # paged: automatic is the q-centric kernel on decode batches, the kv-centric path on
    # prefills under the contiguous rule; the decode kernel is asked for
    assert msa.msa_paged_sparse_fwd_path(32, 8, 4, 16, 512) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_paged_sparse_fwd_path(64, 8, 4, 16, 512) == msa.MSA_PATH_QCENTRIC  # 0.25
    assert msa.msa_paged_sparse_fwd_path(32, 8, 4, 16, 512, 3) == msa.MSA_PATH_DECODE
    assert msa.msa_paged_sparse_fwd_splits(32, 8, 4, 16, 512) == 1
    assert msa.msa_paged_sparse_fwd_path(1, 32768, 4, 16, 256) == msa.MSA_PATH_KVCENTRIC
    assert msa.msa_paged_sparse_fwd_path(1, 32768, 4, 16, 20000) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_paged_sparse_fwd_path(4, 4096, 4, 16, 8192) == msa.MSA_PATH_KVCENTRIC
    # paged with packed queries: the same rule over B * max_pages rows, no sub-batches
    assert msa.msa_paged_sparse_fwd_varlen_path(3, 8096, 2, 16, 71) == msa.MSA_PATH_KVCENTRIC
    assert msa.msa_paged_sparse_fwd_varlen_path(64, 64, 4, 16, 512) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_paged_sparse_fwd_varlen_path(64, 65536, 4, 16, 512) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_paged_sparse_fwd_varlen_path(2, 8, 1, 4, 8, 2) == msa.MSA_PATH_KVCENTRIC
    assert msa.msa_paged_sparse_fwd_varlen_workspace_size(3, 8096, 32, 2, 128, 16, 128, 71) > 0
    assert msa.msa_paged_sparse_fwd_varlen_workspace_size(3, 8096, 32, 2, 128, 16, 64, 71) == 0
    # q-centric: the uniform split rule over total_q rows (1024 rows here: one split)
    assert msa.msa_paged_sparse_fwd_varlen_splits(64, 256, 4, 16, 512) == 1
    assert msa.msa_paged_sparse_fwd_varlen_workspace_size(64, 256, 64, 4, 128, 16, 128, 512) == 0
    assert msa.msa_paged_sparse_fwd_varlen_splits(4, 4, 4, 16, 512) == 8
    assert msa.msa_paged_sparse_fwd_varlen_workspace_size(4, 4, 64, 4, 128, 16, 128, 512) >= \
        8 * 4 * 64 * 128 * 4
    assert msa.msa_paged_sparse_fwd_varlen_splits(4, 4, 4, 16, 512, 100) == 16
    assert msa.msa_paged_sparse_fwd_varlen_splits(3, 8096, 2, 16, 71) == 1  # kv-centric
    # contiguous: the query tile is asked for
    assert msa.msa_sparse_fwd_path(1, 8192, 8192, 64, 4, 16, 4) == msa.MSA_PATH_TILE


def fwd_varlen(**kw):
    lib = msa.load_library()
    a = dict(q=FAKE, k=FAKE, v=FAKE, q2k=FAKE, cuq=FAKE, cuk=FAKE, rp=None, qi=None, sl=None,
             rows=0, B=3, tq=300, tk=900, Hq=16, Hkv=1, D=128, topk=4, blk=128, causal=1,
             scale=0.0, path=0, kvd=0, o=FAKE, lse=FAKE, temp=1.0, lset=None, ws=None, wsb=0)
    a.update(kw)
    return lib.msa_sparse_fwd_varlen(a["q"], a["k"], a["v"], a["q2k"], a["cuq"], a["cuk"],
                                     a["rp"], a["qi"], a["sl"], a["rows"], a["B"], a["tq"],
                                     a["tk"], a["Hq"], a["Hkv"], a["D"], a["topk"], a["blk"],
                                     a["causal"], a["scale"], a["path"], a["kvd"], a["o"],
                                     a["lse"], a["temp"], a["lset"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(D=64), 2), (dict(blk=64), 2), (dict(Hq=3), 2), (dict(topk=33), 2), (dict(B=0), 1),
    (dict(tq=-1), 1), (dict(tk=-1), 1), (dict(cuq=None), 1), (dict(cuk=FAKE + 2), 1),
    (dict(q=None), 1), (dict(o=FAKE + 8), 1), (dict(path=4), 2), (dict(path=3), 2),
    (dict(path=9), 1), (dict(rp=FAKE), 1),
    # a prebuilt CSR needs its row count, at most floor(total_k / 128) + B
    (dict(rp=FAKE, qi=FAKE, sl=FAKE, rows=0, path=2), 1),
    (dict(rp=FAKE, qi=FAKE, sl=FAKE, rows=7 + 3 + 1, path=2), 1),
    # kv-centric without workspace / with too many CSR rows
    (dict(path=2), 1), (dict(path=2, tk=128 * 20000), 2),
    # keys may be absent only when total_k == 0
    (dict(k=None), 1),
    (dict(lset=FAKE, temp=0.0), 1), (dict(kvd=3), 1),
])
def test_sparse_fwd_varlen_rejects(kw, code):
    assert fwd_varlen(**kw) == code
    assert msa.msa_last_error() != ""


def test_sparse_fwd_varlen_empty_batch_is_a_no_op():
    # total_q == 0: nothing to compute, no pointer is needed
    assert fwd_varlen(q=None, o=None, lse=None, q2k=None, tq=0) == 0


def test_varlen_workspace_and_paths():
    # small batches run q-centric (no workspace), large ones kv-centric
    assert msa.msa_sparse_fwd_varlen_path(3, 300, 900, 16, 1, 4) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(4, 32768, 32768, 64, 4, 16) == msa.MSA_PATH_KVCENTRIC
    # units: total_q * Hkv * min(topk, ceil(total_k / 128))
    assert msa.msa_sparse_fwd_varlen_path(2, 2048, 4096, 4, 4, 4, 0) == msa.MSA_PATH_KVCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(2, 2047, 4096, 4, 4, 4, 0) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(2, 2048, 384, 4, 4, 16, 0) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(4, 32768, 0, 64, 4, 16) == msa.MSA_PATH_QCENTRIC
    # 512 queries over 8208 rows (bound): 8192 entries, fewer than 2 per row
    assert msa.msa_sparse_fwd_varlen_path(16, 512, 16 * 65536, 64, 4, 16) == msa.MSA_PATH_QCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(4, 2048, 4 * 65536, 64, 4, 16) == msa.MSA_PATH_KVCENTRIC
    assert msa.msa_sparse_fwd_varlen_path(2, 8192, 128 * 20000, 64, 4, 16) == \
        msa.MSA_PATH_QCENTRIC
    assert msa.msa_sparse_fwd_varlen_workspace_size(3, 300, 900, 16, 1, 128, 4, 128, 1) == 0
    n = msa.msa_sparse_fwd_varlen_workspace_size(3, 300, 900, 16, 1, 128, 4, 128, 2)
    assert n >= 300 * 4 * 16 * 128 * 2
    # the varlen CSR workspace holds the per-sequence tables and the count passes
    assert msa.msa_build_k2q_csr_varlen_workspace_size(3, 2, 300, 4, 9) > 300 * 8


def test_csr_varlen_rejects():
    lib = msa.load_library()
    base = [FAKE, FAKE, FAKE, 3, 2, 300, 900, 4, 9, FAKE, FAKE, None, FAKE, 1 << 20, None]
    a = list(base); a[8] = 0  # total_rows
    assert lib.msa_build_k2q_csr_varlen(*a) == 1
    a = list(base); a[8] = 20000
    assert lib.msa_build_k2q_csr_varlen(*a) == 2
    a = list(base); a[7] = 33
    assert lib.msa_build_k2q_csr_varlen(*a) == 2
    a = list(base); a[1] = None
    assert lib.msa_build_k2q_csr_varlen(*a) == 1
    a = list(base); a[12] = None; a[13] = 0
    assert lib.msa_build_k2q_csr_varlen(*a) == 1


def test_decode_plan_init():
    import ctypes
    lib = msa.load_library()
    P = msa.MsaDecodePlan()
    # 32 sequences x 4 KV heads of 64K tokens: split so that ~2 items per compute unit
    assert lib.msa_paged_decode_plan_init(32, 8, 64, 4, 128, 128, 65536, 512, 0, 0,
                                          ctypes.byref(P)) == 0
    assert P.max_pages == 512 and P.kv_chunk_size_pages == 128 and P.split_kv == 1
    assert P.padded_work_count == 32 * 4 and P.partial_rows == 32 * 4 * 8
    assert P.bytes >= P.partial_rows * 64 * 128 * 4
    # enough sequences: no split; forced single-page chunks; chunks capped at 512 pages
    assert lib.msa_paged_decode_plan_init(512, 8, 64, 4, 128, 128, 4096, 512, 0, 0,
                                          ctypes.byref(P)) == 0
    assert P.split_kv == 0 and P.kv_chunk_size_pages == 32 and P.partial_rows == 512 * 8
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 384, 0, 1, 0,
                                          ctypes.byref(P)) == 0
    assert P.kv_chunk_size_pages == 1 and P.padded_work_count == 12
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 1 << 20, 16, 0, 0,
                                          ctypes.byref(P)) == 0
    assert P.kv_chunk_size_pages == 512
    # rejected: Sq > 16, chunk > 512 pages, one chunk for a 1M-token sequence, bad sizes
    assert lib.msa_paged_decode_plan_init(4, 17, 64, 4, 128, 128, 4096, 0, 0, 0,
                                          ctypes.byref(P)) == 2
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 4096, 0, 513, 0,
                                          ctypes.byref(P)) == 2
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 1 << 20, 0, 0, 1,
                                          ctypes.byref(P)) == 2
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 0, 0, 0, 0,
                                          ctypes.byref(P)) == 1
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 64, 128, 4096, 0, 0, 0,
                                          ctypes.byref(P)) == 2
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 4096, 0, 0, 0, None) == 1


def test_decode_plan_and_run_reject_bad_buffers():
    import ctypes
    lib = msa.load_library()
    P = msa.MsaDecodePlan()
    assert lib.msa_paged_decode_plan_init(4, 8, 64, 4, 128, 128, 4096, 0, 0, 0,
                                          ctypes.byref(P)) == 0
    assert lib.msa_paged_decode_plan(FAKE, ctypes.byref(P), FAKE, P.bytes - 1, None) == 1
    assert lib.msa_paged_decode_plan(FAKE, ctypes.byref(P), FAKE + 16, P.bytes, None) == 1
    assert lib.msa_paged_decode_plan(None, ctypes.byref(P), FAKE, P.bytes, None) == 1
    Z = msa.MsaDecodePlan()  # never initialised
    assert lib.msa_paged_decode_plan(FAKE, ctypes.byref(Z), FAKE, 1 << 30, None) == 1
    run = [FAKE] * 5 + [ctypes.byref(P), FAKE, P.bytes, 16, 0, 1, 0.0, FAKE, FAKE, 1.0, None,
                        None]
    a = list(run); a[8] = 0  # num_pages
    assert lib.msa_paged_decode_run(*a) == 1
    a = list(run); a[0] = None
    assert lib.msa_paged_decode_run(*a) == 1
    a = list(run); a[14] = 0.0; a[15] = FAKE  # temperature buffer with T = 0
    assert lib.msa_paged_decode_run(*a) == 1
    a = list(run); a[9] = 7  # unknown dtype
    assert lib.msa_paged_decode_run(*a) == 1
    # the fp8 decode covers Sq * qpk <= 128 columns: 16 queries x 16 heads is refused
    P16 = msa.MsaDecodePlan()
    assert lib.msa_paged_decode_plan_init(4, 16, 64, 4, 128, 128, 4096, 0, 0, 0,
                                          ctypes.byref(P16)) == 0
    a = list(run); a[5] = ctypes.byref(P16); a[7] = P16.bytes; a[9] = 1
    assert lib.msa_paged_decode_run(*a) == 2


def paged_noalloc(**kw):
    lib = msa.load_library()
    a = dict(B=32, Sq=8, Hq=64, Hkv=4, D=128, topk=16, page=128, num_pages=4096, max_pages=128,
             splits=0, path=1, kvd=0)
    a.update(kw)
    return lib.msa_paged_sparse_fwd_noalloc(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, a["B"], a["Sq"],
                                            a["Hq"], a["Hkv"], a["D"], a["topk"], a["page"],
                                            a["num_pages"], a["max_pages"], 1, 0.0, a["splits"],
                                            a["path"], a["kvd"], FAKE, FAKE, 1.0, None, None)


@pytest.mark.parametrize("kw,code", [
    # split partials beyond the scratch array: 16 splits x 16384 rows x 512 B = 128 MiB
    (dict(splits=16), 1),
    # argument errors reported as by msa_paged_sparse_fwd
    (dict(D=64), 2), (dict(topk=33), 2), (dict(Hq=6), 1), (dict(path=2), 1),
    (dict(splits=-1), 1), (dict(num_pages=0), 1),
])
def test_paged_noalloc_rejects_on_host(kw, code):
    assert paged_noalloc(**kw) == code
    assert msa.msa_last_error()


def test_noalloc_scratch_size_matches_header():
    text = open(os.path.join(ROOT, "include", "msa.h")).read()
    m = re.search(r"#define MSA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == msa.MSA_NOALLOC_SCRATCH_BYTES
