"""The seeded generators produce the index recipes the workloads state."""
import numpy as np

import workloads as wl


def test_deterministic_and_slice_consistent():
    a = wl.normal_bf16(42, wl.STREAM_Q, (1000,))
    b = wl.normal_bf16(42, wl.STREAM_Q, (1000,))
    c = wl.normal_bf16(42, wl.STREAM_Q, (600,), first=400)
    assert np.array_equal(a, b) and np.array_equal(a[400:], c)
    assert not np.array_equal(a, wl.normal_bf16(42, wl.STREAM_K, (1000,)))


def test_normal_moments():
    x = wl.bf16_to_f32(wl.normal_bf16(42, wl.STREAM_V, (1 << 20,))).astype(np.float64)
    assert abs(x.mean()) < 5e-3 and abs(x.std() - 1.0) < 5e-3
    assert np.all(np.isfinite(x))


def test_perm_rows_distinct_in_range():
    t = wl.q2k_table(1, wl.MODE_PERM, 1, 2, 500, 1024, 128, 4)
    assert t.min() >= 0 and t.max() < 8
    s = np.sort(t, -1)
    assert np.all(np.diff(s, axis=-1) > 0)
    # not sorted in general (permutation order)
    assert not np.all(np.diff(t, axis=-1) > 0)


def test_sink_rows():
    t = wl.q2k_table(1, wl.MODE_SINK, 1, 2, 500, 32768, 128, 16)
    assert np.all(t[..., 0] == 0)
    assert np.all(np.diff(t, axis=-1) > 0) and t.max() < 256


def test_causal_rows_follow_visible_rule():
    Sq = Skv = 8192
    t = wl.q2k_table(3, wl.MODE_CAUSAL, 1, 4, Sq, Skv, 128, 16)
    for q in range(0, Sq, 97):
        vis = min(max((q + Skv - Sq) // 128 + 1, 0), 64)
        row = t[0, 1, q]
        if vis <= 16:
            assert list(row[:vis]) == list(range(vis)) and np.all(row[vis:] == -1)
        else:
            assert row[-1] == vis - 1 and np.all(np.diff(row) > 0) and row[0] >= 0


def test_causal_rows_when_sq_exceeds_skv_use_floor_division():
    # q + Skv - Sq < 0 for the first rows: floor division gives visible <= 0
    t = wl.q2k_table(3, wl.MODE_CAUSAL, 1, 1, 400, 256, 128, 2)
    assert np.all(t[0, 0, :144] == -1)        # limits -144..-1: nothing visible
    assert list(t[0, 0, 144]) == [0, -1]      # limit 0: block 0 only
    assert list(t[0, 0, 399]) == [0, 1]


def test_page_table_is_a_permutation():
    p = wl.permutation(42, wl.STREAM_PAGES, 32 * 512)
    assert np.array_equal(np.sort(p), np.arange(32 * 512))
    assert not np.array_equal(p, np.arange(32 * 512))


def test_paged_workload_recipe():
    w = wl.WORKLOADS["c5"]
    t = wl.q2k_table(w.seed, w.mode, w.B, w.Hkv, w.Sq, w.kvlen, w.blk, w.topk)
    assert w.kvlen == 65519 and w.max_pages == 512
    assert np.all(t[..., -1] == 511)
    assert np.all(np.diff(t, axis=-1) > 0)
