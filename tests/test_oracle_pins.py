"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these re-types the oracle's formulas: each compares it with values the
pages print, with hand-derived closed forms, with library routines (numpy
take / float64 matmul / fancy indexing, torch's bf16 conversion) or with
invariants the pages state (the sum of masked partials is the full lookup;
the concatenation of shard logits is the full product).
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# printed page values
# ---------------------------------------------------------------------------
def test_twelve_word_demo_every_printed_step():
    g = _golden("vllm11_twelve_word_demo.json")
    V, D, tp = g["vocab"], g["dim"], g["tp"]
    ids = np.array(g["ids"], dtype=np.int64)
    partials = []
    for rank in range(tp):
        start, end = oracle.shard_range(V, tp, rank)
        assert [start, end] == g[f"rank{rank}"]["range"]
        # the page's shard recipe: row for global id i holds 10*i + j
        shard = (np.arange(start, end, dtype=np.float32)[:, None] * 10.0
                 + np.arange(D, dtype=np.float32)[None, :])
        mask, local = oracle.mask_shift(ids, start, end)
        if rank == 0:
            assert mask.tolist() == g["rank0"]["mask"]
            assert local.tolist() == g["rank0"]["local"]
            # step 3 of the page looks up the placeholder row 0 for the masked id
            assert shard[local].tolist() == g["rank0"]["lookup"]
        part = oracle.embed(ids, shard, start)
        assert part.tolist() == g[f"rank{rank}"]["partial"]
        partials.append(part)
    total = oracle.sum_partials(partials)
    assert total.tolist() == g["sum"]
    assert total.tolist() == g["standard_embedding"]


def test_arange_4x2_ownership_and_partials():
    g = _golden("tpvocab_arange_4x2.json")
    full = np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    assert list(oracle.shard_range(4, 2, 0)) == g["printed"]["rank0_range"]
    tok = np.array(g["stated"]["tokens"], dtype=np.int64)
    parts = []
    for rank in range(2):
        s, e = oracle.shard_range(4, 2, rank)
        p = oracle.embed(tok, full[s:e], s)
        nonzero_tokens = [int(t) for t, row in zip(tok, p) if np.any(row != 0)]
        assert nonzero_tokens == g["stated"][f"rank{rank}_nonzero_tokens"]
        assert p.tolist() == g["derived_by_hand"][f"rank{rank}_partial"]
        parts.append(p)
    assert oracle.sum_partials(parts).tolist() == g["derived_by_hand"]["sum"]


def test_arange_4x2_lmhead_shapes_words_and_closed_form():
    g = _golden("tpvocab_arange_4x2.json")
    W = np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    # integer-valued x so that every product is exact in fp32 and fp64
    x = np.array([[1, 2], [-3, 5], [7, 0]], dtype=np.float32)
    full = np.zeros((3, 4), dtype=np.float64)
    for rank in range(2):
        s, e = oracle.shard_range(4, 2, rank)
        z = oracle.lmhead_f64(x, W[s:e])
        assert list(z.shape) == g["printed"][f"lm_rank{rank}_shape"]
        assert list(range(s, e)) == g["printed"][f"lm_rank{rank}_words"]
        oracle.lmhead_f64(x, W[s:e], out=full, col_offset=s)
    a, b = x[:, 0].astype(np.float64), x[:, 1].astype(np.float64)
    closed = np.stack([a + 2 * b, 3 * a + 4 * b, 5 * a + 6 * b, 7 * a + 8 * b], axis=1)
    assert np.array_equal(full, closed)


def test_qwen3_shard_shapes():
    g = _golden("tpmath_qwen3_shapes.json")
    V, tp = g["vocab"], g["tp"]
    s0, e0 = oracle.shard_range(V, tp, 0)
    s1, e1 = oracle.shard_range(V, tp, 1)
    assert e0 - s0 == g["vocab_per_card"] and e1 - s1 == g["vocab_per_card"]
    assert (s0, e0, s1, e1) == (0, 75968, 75968, 151936)
    # the tp=4 rank-2 shard of the hidden-4096 workload
    assert oracle.shard_range(V, 4, 2) == (75968, 113952)


# ---------------------------------------------------------------------------
# ownership rule
# ---------------------------------------------------------------------------
def test_shard_range_rejects_bad_splits():
    for args in [(10, 3, 0), (12, 2, 2), (12, 2, -1), (12, 0, 0), (0, 1, 0)]:
        with pytest.raises(oracle.OracleError):
            oracle.shard_range(*args)


@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_every_valid_id_has_exactly_one_owner(itype):
    for V in range(1, 9):
        ids = np.arange(-2, V + 2, dtype=itype)
        for tp in [t for t in range(1, V + 1) if V % t == 0]:
            owners = np.zeros(ids.size, dtype=np.int64)
            for r in range(tp):
                s, e = oracle.shard_range(V, tp, r)
                mask, local = oracle.mask_shift(ids, s, e)
                owners += mask
                assert np.all(local[mask] == ids[mask] - s)
                assert np.all(local[~mask] == 0)
                assert np.all((local >= 0) & (local < V // tp))
            valid = (ids >= 0) & (ids < V)
            assert np.array_equal(owners, valid.astype(np.int64))


# ---------------------------------------------------------------------------
# invariant: sum over ranks of masked partials == full lookup (library take)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("tp", [1, 2, 4, 8])
def test_sum_of_partials_is_full_lookup(dtype, tp):
    V, D = 64, 24
    full = wl.table_rows(7, V, D, dtype, 0, V)
    rng = np.random.default_rng(tp)
    ids = rng.integers(-5, V + 5, size=300).astype(np.int64)
    parts = []
    for r in range(tp):
        s, e = oracle.shard_range(V, tp, r)
        parts.append(oracle.embed(ids, full[s:e], s))
    total = oracle.sum_partials(parts)
    valid = (ids >= 0) & (ids < V)
    ref = np.zeros_like(total)
    ref[valid] = np.take(full, ids[valid], axis=0)
    assert total.tobytes() == ref.tobytes()
    # and the full-table call of the same lookup (start 0, all rows) agrees
    assert oracle.embed(ids, full, 0).tobytes() == ref.tobytes()


@pytest.mark.parametrize("dim", [1, 2, 3, 8])
def test_brute_force_tiny_vocabularies(dim):
    for V in range(1, 9):
        full = wl.table_rows(11, V, dim, "f32", 0, V)
        ids = np.arange(-2, V + 2, dtype=np.int32)
        for tp in [t for t in range(1, V + 1) if V % t == 0]:
            for r in range(tp):
                s, e = oracle.shard_range(V, tp, r)
                p = oracle.embed(ids, full[s:e], s)
                for i, x in enumerate(ids):
                    if s <= x < e:
                        assert p[i].tobytes() == full[x].tobytes()
                    else:
                        assert p[i].tobytes() == bytes(4 * dim)


def test_masked_rows_are_positive_zero_and_placeholder_unread():
    # row 0 of the shard holds -0.0, NaN and -inf: the formula mask*y would
    # give -0 / NaN for masked ids; the reading taken writes +0 bits.
    shard = np.array([[-0.0, np.nan, -np.inf, -1.5], [1, 2, 3, 4]], dtype=np.float32)
    ids = np.array([5, 0, -1, 1, 2], dtype=np.int64)
    out = oracle.embed(ids, shard, 0)
    zero = bytes(16)
    assert out[0].tobytes() == zero and out[2].tobytes() == zero and out[4].tobytes() == zero
    assert out[1].tobytes() == shard[0].tobytes()
    assert out[3].tobytes() == shard[1].tobytes()


def test_embed_empty_input():
    out = oracle.embed(np.zeros(0, dtype=np.int32), np.ones((4, 8), np.float32), 0)
    assert out.shape == (0, 8)


# ---------------------------------------------------------------------------
# sum of partials: rounding rule and fp32 order
# ---------------------------------------------------------------------------
def test_bf16_rounding_textbook_values():
    one = 0x3F80
    cases = [  # a list, not a dict: 0.0 and -0.0 are equal dict keys
        (1.0, one),
        (1.0 + 2.0 ** -8, one),                    # halfway, even neighbour is 1.0
        (1.0 + 3 * 2.0 ** -8, one + 2),            # halfway, even neighbour is 1+2^-6
        (1.0 + 2.0 ** -8 + 2.0 ** -20, one + 1),   # just above halfway rounds up
        (-2.0, 0xC000),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (float(np.float32(3.4e38)), 0x7F80),       # rounds past the largest bf16 -> inf
        (float("inf"), 0x7F80),
    ]
    for v, bits in cases:
        assert int(oracle.round_bf16([v])[0]) == bits, v
    nan_bits = int(oracle.round_bf16([float("nan")])[0])
    assert (nan_bits & 0x7F80) == 0x7F80 and (nan_bits & 0x7F) != 0


def test_bf16_rounding_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),   # subnormals
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
    ])
    ours = oracle.round_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(oracle.widen_bf16(ours),
                          torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).float().numpy())


def test_sum_partials_fp32_rank_order_matches_numpy():
    rng = np.random.default_rng(5)
    parts = [rng.standard_normal(1000).astype(np.float32) * 10 ** k for k in range(4)]
    ref = parts[0].copy()
    for p in parts[1:]:
        ref = np.add(ref, p, dtype=np.float32)
    assert oracle.sum_partials(parts).tobytes() == ref.tobytes()


def test_sum_partials_bf16_matches_torch_fp32_then_round():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(6)
    parts = [wl.f32_to_bf16_bits(rng.standard_normal(2000).astype(np.float32) * 2.0 ** (3 * k))
             for k in range(3)]
    tp = [torch.from_numpy(p.view(np.int16)).view(torch.bfloat16).float() for p in parts]
    acc = tp[0]
    for t in tp[1:]:
        acc = acc + t
    ref = acc.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.sum_partials(parts), ref)


def test_sum_single_partial_is_identity():
    rng = np.random.default_rng(8)
    p = wl.f32_to_bf16_bits(rng.standard_normal(100).astype(np.float32))
    p[0] = 0x8000  # -0.0 survives a one-partial sum
    assert oracle.sum_partials([p]).tobytes() == p.tobytes()


def test_sum_with_negative_zero_documented_case():
    # (+0) + (-0) = +0: the sum invariant is bitwise only for tables without -0.0
    a = np.array([0.0], dtype=np.float32)
    b = np.array([-0.0], dtype=np.float32)
    assert oracle.sum_partials([b, a]).tobytes() == np.float32(0.0).tobytes()


# ---------------------------------------------------------------------------
# last-position select
# ---------------------------------------------------------------------------
def test_select_closed_form_uniform_prefill():
    T, D, S = 32 * 64, 8, 32
    H = wl.hidden_states(9, T, D, "bf16")
    cu = wl.cu_seqlens_uniform(S, 64)
    out = oracle.last_token_select(H, cu)
    rows = [63 + 64 * s for s in range(S)]
    assert out.tobytes() == H[rows].tobytes()


def test_select_ragged_matches_fancy_indexing():
    cu = wl.cu_seqlens_ragged(10, 17, 1, 40)
    T = int(cu[-1])
    H = wl.hidden_states(12, T, 12, "f32")
    out = oracle.last_token_select(H, cu)
    assert out.tobytes() == H[cu[1:].astype(np.int64) - 1].tobytes()


def test_select_rejects_malformed_cu_seqlens():
    H = np.zeros((10, 4), np.float32)
    for cu in ([1, 10], [0, 5, 5, 10], [0, 4, 9], [0, 6, 3, 10]):
        with pytest.raises(oracle.OracleError):
            oracle.last_token_select(H, np.array(cu, np.int32))


# ---------------------------------------------------------------------------
# logits: concatenation of shard products == full product (library matmul)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_lmhead_concat_equals_full_product(dtype):
    V, D, M, tp = 48, 40, 7, 4
    W = wl.table_rows(13, V, D, dtype, 0, V)
    X = wl.hidden_states(14, M, D, dtype)
    Wf = W.astype(np.float64) if dtype == "f32" else wl.bf16_bits_to_f32(W).astype(np.float64)
    Xf = X.astype(np.float64) if dtype == "f32" else wl.bf16_bits_to_f32(X).astype(np.float64)
    ref = Xf @ Wf.T
    cat = np.zeros((M, V), np.float64)
    for r in range(tp):
        s, e = oracle.shard_range(V, tp, r)
        oracle.lmhead_f64(X, W[s:e], out=cat, col_offset=s)
    np.testing.assert_allclose(cat, ref, rtol=1e-12, atol=1e-15)
    # the oracle's concat equals its own full product bitwise (same k order)
    full = oracle.lmhead_f64(X, W)
    assert cat.tobytes() == full.tobytes()


def test_lmhead_not_transposed_on_nonsquare():
    # distinguishes X.W^T from X^T.W / W.X^T and a dropped or extra term
    X = np.array([[1, 0, 2]], dtype=np.float32)
    W = np.array([[1, 1, 1], [0, 1, 0], [3, 0, -1]], dtype=np.float32)
    out = oracle.lmhead_f64(X, W)
    assert out.tolist() == [[3.0, 0.0, 1.0]]


def test_lmhead_threads_do_not_change_values():
    W = wl.table_rows(15, 64, 32, "bf16", 0, 64)
    X = wl.hidden_states(16, 5, 32, "bf16")
    a = oracle.lmhead_f64(X, W, nthreads=1)
    b = oracle.lmhead_f64(X, W, nthreads=3)
    c = oracle.lmhead_f64(X, W, nthreads=8)
    assert a.tobytes() == b.tobytes() == c.tobytes()
    assert oracle.logit_f64(X, W, 3, 17) == a[3, 17]


def test_lmhead_rejects_offset_past_row():
    X = np.zeros((2, 4), np.float32)
    W = np.zeros((3, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.lmhead_f64(X, W, out=np.zeros((2, 4)), col_offset=2)


# ---------------------------------------------------------------------------
# greedy pick over logits
# ---------------------------------------------------------------------------
def test_argmax_rows_matches_numpy_first_maximum():
    rng = np.random.default_rng(31)
    z = rng.integers(-5, 6, size=(40, 57)).astype(np.float64)  # many exact ties
    mx, idx = oracle.argmax_rows(z)
    assert np.array_equal(idx, np.argmax(z, axis=1))            # numpy: first maximum
    assert np.array_equal(mx, z.max(axis=1))


def test_argmax_of_concatenated_shards_is_global_argmax():
    V, D, M, tp = 96, 16, 9, 3
    W = wl.table_rows(32, V, D, "f32", 0, V, std=1.0)
    X = wl.hidden_states(33, M, D, "f32")
    full = oracle.lmhead_f64(X, W)
    cat = np.zeros((M, V))
    for r in range(tp):
        s, e = oracle.shard_range(V, tp, r)
        oracle.lmhead_f64(X, W[s:e], out=cat, col_offset=s)
    assert np.array_equal(oracle.argmax_rows(cat)[1], oracle.argmax_rows(full)[1])
    # per-shard maxima combined by value (ties to the lower id) give the same pick
    best = [max((oracle.argmax_rows(cat[:, s:e])[0][m], -(oracle.argmax_rows(cat[:, s:e])[1][m] + s))
                for s, e in (oracle.shard_range(V, tp, r) for r in range(tp))) for m in range(M)]
    assert [-b[1] for b in best] == list(oracle.argmax_rows(full)[1])


# ---------------------------------------------------------------------------
# shard loading (each rank's weight_loader keeps rows [rank*R, rank*R + R))
# ---------------------------------------------------------------------------
def test_load_shard_arange_4x2_demo():
    g = _golden("tpvocab_arange_4x2.json")
    full = np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    for rank in range(2):
        assert oracle.load_shard(full, 2, rank).tolist() == g["derived_by_hand"][f"rank{rank}_shard"]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_load_shard_is_numpy_slice_and_shards_tile_the_table(dtype):
    for vocab, dim in [(1, 1), (12, 4), (96, 3), (1000, 40)]:
        full = wl.table_rows(70 + vocab, vocab, dim, dtype, 0, vocab)
        for tp in [t for t in range(1, 9) if vocab % t == 0]:
            shards = []
            for rank in range(tp):
                sh = oracle.load_shard(full, tp, rank)
                r = vocab // tp
                assert sh.tobytes() == full[rank * r:(rank + 1) * r].tobytes()
                shards.append(sh)
            assert np.concatenate(shards).tobytes() == full.tobytes()


def test_load_shard_rejects_uneven_split():
    full = np.zeros((10, 4), np.float32)
    with pytest.raises(oracle.OracleError):
        oracle.load_shard(full, 3, 0)
    with pytest.raises(oracle.OracleError):
        oracle.load_shard(full, 2, 2)


# ---------------------------------------------------------------------------
# log-sum-exp of the logits rows (the softmax normaliser the sampler needs)
# ---------------------------------------------------------------------------
def test_logsumexp_closed_forms():
    # n equal logits c: log(n e^c) = c + ln n  (a dropped or doubled term moves it by ln(1 +- 1/n))
    for n in (1, 2, 3, 7, 1000, 151936):
        for c in (0.0, -3.25, 17.5):
            got = oracle.logsumexp_rows(np.full((1, n), c))[0]
            assert abs(got - (c + math.log(n))) <= 1e-12 * max(1.0, abs(c) + math.log(n)), (n, c)
    # one logit: the logit itself, exactly
    assert oracle.logsumexp_rows(np.array([[-2.5]]))[0] == -2.5
    # two logits a, b: max + log(1 + e^-|a-b|)
    for a, b in [(0.0, 1.0), (5.0, -5.0), (-1e3, -1e3 + 2.0), (3.0, 3.0)]:
        want = max(a, b) + math.log1p(math.exp(-abs(a - b)))
        assert abs(oracle.logsumexp_rows(np.array([[a, b]]))[0] - want) <= 1e-12 * max(1, abs(want))


def test_logsumexp_matches_library_routine():
    from scipy.special import logsumexp
    rng = np.random.default_rng(71)
    for shape, scale in [((5, 1), 1.0), ((8, 333), 3.0), ((3, 151936), 2.0), ((4, 50), 300.0)]:
        z = rng.standard_normal(shape) * scale
        got = oracle.logsumexp_rows(z)
        want = logsumexp(z, axis=1)
        assert np.allclose(got, want, rtol=1e-12, atol=1e-12), shape


def test_logsumexp_no_overflow_and_shift_invariance():
    # logits past exp's range: the factored maximum keeps the value finite
    z = np.array([[1000.0, 999.0, 998.0], [-1000.0, -1001.0, -1e4]])
    got = oracle.logsumexp_rows(z)
    assert np.all(np.isfinite(got))
    assert abs(got[0] - (1000.0 + math.log(1 + math.exp(-1) + math.exp(-2)))) < 1e-12 * 1000
    rng = np.random.default_rng(72)
    z = rng.standard_normal((6, 200))
    for c in (-50.0, 0.5, 123.0):
        assert np.allclose(oracle.logsumexp_rows(z + c), oracle.logsumexp_rows(z) + c,
                           rtol=0, atol=1e-12 * (1 + abs(c)))


def test_logsumexp_of_concatenated_shards_combines_shard_values():
    # the full row's value from its shards' values: log(sum_r exp(lse_r)),
    # factored by the largest shard value (the combine across tp ranks)
    rng = np.random.default_rng(73)
    z = rng.standard_normal((5, 4 * 97)) * 4
    full = oracle.logsumexp_rows(z)
    parts = np.stack([oracle.logsumexp_rows(z[:, r * 97:(r + 1) * 97]) for r in range(4)], axis=1)
    mx = parts.max(axis=1)
    comb = mx + np.log(np.exp(parts - mx[:, None]).sum(axis=1))
    assert np.allclose(full, comb, rtol=1e-12, atol=1e-12)
    # and a shard's value never exceeds the full row's (every term is positive)
    assert np.all(parts <= full[:, None] + 1e-12)
