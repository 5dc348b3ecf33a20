"""The seeded input generators: determinism, slice independence, shapes."""
import numpy as np
import pytest

import workloads as wl


def test_table_slices_do_not_depend_on_request():
    full = wl.table_rows(1, 3000, 16, "bf16", 0, 3000)
    part = wl.table_rows(1, 3000, 16, "bf16", 1000, 2500)
    assert part.tobytes() == full[1000:2500].tobytes()
    again = wl.table_rows(1, 3000, 16, "bf16", 0, 3000)
    assert again.tobytes() == full.tobytes()


def test_table_statistics_and_dtype():
    t = wl.table_rows(2, 4096, 64, "f32", 0, 4096)
    assert t.dtype == np.float32 and t.shape == (4096, 64)
    assert abs(float(t.std()) - 0.02) < 5e-4
    b = wl.table_rows(2, 4096, 64, "bf16", 0, 4096)
    assert b.dtype == np.uint16
    assert np.allclose(wl.bf16_bits_to_f32(b), t, rtol=2 ** -8, atol=0)


def test_generator_bf16_encoding_matches_torch():
    torch = pytest.importorskip("torch")
    v = np.random.default_rng(0).standard_normal(10000).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(wl.f32_to_bf16_bits(v), ref)


def test_zipf_ids_are_skewed_and_in_range():
    ids = wl.token_ids(3, 151936, 65536, "zipf")
    assert ids.dtype == np.int32
    assert ids.min() >= 0 and ids.max() < 151936
    counts = np.bincount(ids, minlength=151936)
    assert counts[0] == counts.max()
    assert counts[0] > 10 * counts[100]


def test_uniform_ids_cover_both_halves():
    ids = wl.token_ids(4, 151936, 8192)
    lo = np.count_nonzero(ids < 75968)
    assert 3800 < lo < 4400


def test_cu_seqlens():
    cu = wl.cu_seqlens_uniform(32, 2048)
    assert cu[0] == 0 and cu[-1] == 65536 and np.all(np.diff(cu) == 2048)
    r = wl.cu_seqlens_ragged(5, 9, 1, 7)
    assert r[0] == 0 and np.all(np.diff(r) >= 1) and np.all(np.diff(r) <= 7)


def test_workload_table_matches_page_shapes():
    w = wl.WORKLOADS["qwen3_0p6b_tp2_rank0"]
    assert (w.vocab, w.dim, w.shard_rows, w.rank_start(0)) == (151936, 1024, 75968, 0)
    w5 = wl.WORKLOADS["large_v151936_d4096_tp4_rank2"]
    assert (w5.shard_rows, w5.rank_start(2)) == (37984, 75968)


def test_tables_hold_no_negative_zero():
    w = wl.WORKLOADS["qwen3_0p6b_tp2_all_ranks"]
    t = wl.table_rows(wl.table_seed(w), w.vocab, w.dim, "bf16", 0, 8192)
    assert not np.any(t == 0x8000)
    f = wl.table_rows(5, 40000, 64, "f32", 0, 40000)
    assert not np.any(np.signbit(f) & (f == 0))
