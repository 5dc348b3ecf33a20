"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Embedding rows, partial sums and selected rows must match bit for bit; logits
(bf16 or fp32 inputs, fp32 accumulation) must satisfy
|gpu - ref| <= 1e-2 + 1e-2 |ref| against the oracle's fp64 products.
Every workload's LM head is compared in full, logit by logit.
"""
import json
import os
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

import oracle  # noqa: E402
import workloads as wl  # noqa: E402
import vocab_sharded_embedding_amd as vpe  # noqa: E402
from _gpu import as_f64, assert_logits_close, dev, oracle_threads, to_dev, to_host  # noqa: E402

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# ---------------------------------------------------------------------------
# cached workload inputs (generation of the large tables takes seconds)
# ---------------------------------------------------------------------------
_cache = {}


def _inputs(name):
    if name in _cache:
        return _cache[name]
    w = wl.WORKLOADS[name]
    d = {"w": w, "ids": wl.workload_ids(w), "hidden": wl.workload_hidden(w),
         "cu": wl.workload_cu_seqlens(w)}
    d["shards"] = {r: wl.shard_table(w, r) for r in w.ranks}
    _cache.clear()  # keep at most one workload's tables in host memory
    _cache[name] = d
    return d


def _lm_rows(d):
    """The LM head's input rows on the host (prefill: last position of each sequence)."""
    w = d["w"]
    if w.seqs:
        return d["hidden"][d["cu"][1:].astype(np.int64) - 1]
    return d["hidden"]


# ---------------------------------------------------------------------------
# the pages' worked examples, run on the GPU
# ---------------------------------------------------------------------------
def test_twelve_word_demo_on_gpu():
    with open(os.path.join(GOLDEN, "vllm11_twelve_word_demo.json")) as f:
        g = json.load(f)
    V, D, tp = g["vocab"], g["dim"], g["tp"]
    ids = to_dev(np.array(g["ids"], dtype=np.int64))
    parts = []
    for rank in range(tp):
        start, end = vpe.vpe_shard_range(V, tp, rank)
        shard = (np.arange(start, end, dtype=np.float32)[:, None] * 10.0
                 + np.arange(D, dtype=np.float32)[None, :])
        p = vpe.vpe_embed(ids, to_dev(shard), start)
        assert to_host(p).tolist() == g[f"rank{rank}"]["partial"]
        parts.append(p)
    total = vpe.vpe_sum_partials(parts)
    torch.cuda.synchronize()
    assert to_host(total).tolist() == g["sum"]


def test_arange_4x2_demo_on_gpu():
    with open(os.path.join(GOLDEN, "tpvocab_arange_4x2.json")) as f:
        g = json.load(f)
    full = np.arange(1, 9, dtype=np.float32).reshape(4, 2)
    tok = to_dev(np.array(g["stated"]["tokens"], dtype=np.int32))
    parts = []
    for rank in range(2):
        s, e = vpe.vpe_shard_range(4, 2, rank)
        p = vpe.vpe_embed(tok, to_dev(full[s:e]), s)
        assert to_host(p).tolist() == g["derived_by_hand"][f"rank{rank}_partial"]
        parts.append(p)
    assert to_host(vpe.vpe_sum_partials(parts)).tolist() == g["derived_by_hand"]["sum"]
    # LM head: shard logits at their vocab offsets give the closed form
    x = np.array([[1, 2], [-3, 5], [7, 0]], dtype=np.float32)
    logits = torch.full((3, 4), float("nan"), device=dev())
    for rank in range(2):
        s, e = vpe.vpe_shard_range(4, 2, rank)
        vpe.vpe_lmhead(to_dev(x), to_dev(full[s:e]), logits, col_offset=s)
    a, b = x[:, 0].astype(np.float64), x[:, 1].astype(np.float64)
    closed = np.stack([a + 2 * b, 3 * a + 4 * b, 5 * a + 6 * b, 7 * a + 8 * b], axis=1)
    assert np.array_equal(as_f64(to_host(logits)), closed)


# ---------------------------------------------------------------------------
# embedding lookup at every workload, every rank it runs: bit-exact
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER)
def test_embed_matches_oracle(name):
    d = _inputs(name)
    w = d["w"]
    ids_d = to_dev(d["ids"])
    for rank in w.ranks:
        _say(f"embed {name} rank {rank}: n={w.n_ids} dim={w.dim} {w.dtype}")
        start = w.rank_start(rank)
        out = vpe.vpe_embed(ids_d, to_dev(d["shards"][rank]), start)
        ref = oracle.embed(d["ids"], d["shards"][rank], start, nthreads=oracle_threads())
        got = to_host(out)
        assert got.shape == ref.shape
        assert got.tobytes() == ref.tobytes(), f"{name} rank {rank}: embedding differs"
        owned = (d["ids"] >= start) & (d["ids"] < start + w.shard_rows)
        assert np.all(got[~owned] == 0)


@pytest.mark.parametrize("name", ["tiny_v4096_d64_f32_tp2", "qwen3_0p6b_tp2_all_ranks"])
def test_sum_of_partials_is_full_lookup(name):
    d = _inputs(name)
    w = d["w"]
    ids_d = to_dev(d["ids"])
    parts = [vpe.vpe_embed(ids_d, to_dev(d["shards"][r]), w.rank_start(r)) for r in w.ranks]
    total = to_host(vpe.vpe_sum_partials(parts))
    full = np.concatenate([d["shards"][r] for r in w.ranks], axis=0)
    ref_full = oracle.embed(d["ids"], full, 0, nthreads=oracle_threads())
    ref_sum = oracle.sum_partials([to_host(p) for p in parts])
    assert total.tobytes() == ref_full.tobytes()
    assert total.tobytes() == ref_sum.tobytes()
    assert total.tobytes() == np.take(full, d["ids"], axis=0).tobytes()


def test_sum_with_negative_zero_entry_follows_the_oracle():
    # (+0) + (-0) = +0: a -0.0 table entry is the one case where the sum of
    # masked partials differs (in sign only) from the full lookup
    V, D = 64, 16
    full = wl.table_rows(90, V, D, "bf16", 0, V)
    full[40, 3] = 0x8000
    ids = np.arange(V, dtype=np.int32)
    ids_d = to_dev(ids)
    parts = [vpe.vpe_embed(ids_d, to_dev(full[r * 32:(r + 1) * 32]), r * 32) for r in range(2)]
    got = to_host(vpe.vpe_sum_partials(parts))
    assert got.tobytes() == oracle.sum_partials([to_host(p) for p in parts]).tobytes()
    assert got[40, 3] == 0 and full[40, 3] == 0x8000
    got[40, 3] = 0x8000
    assert got.tobytes() == full.tobytes()


def test_sum_in_place_and_general_values():
    # partials that are all non-zero exercise the fp32 add order and the rounding
    rng = np.random.default_rng(21)
    for dtype in ("f32", "bf16"):
        for n in (1, 7, 4096 + 5):
            parts_h = [wl.hidden_states(30 + r, 1, n, dtype).reshape(-1) for r in range(3)]
            parts = [to_dev(p) for p in parts_h]
            ref = oracle.sum_partials(parts_h)
            got = to_host(vpe.vpe_sum_partials(parts))
            assert got.tobytes() == ref.tobytes(), (dtype, n)
            vpe.vpe_sum_partials(parts, out=parts[0])  # in place into partial 0
            assert to_host(parts[0]).tobytes() == ref.tobytes(), (dtype, n)
    del rng


def test_sum_every_part_count():
    # one to six partials, general (all non-zero) values, sizes spanning
    # several blocks with ragged vector and element tails; in place as well
    for dtype in ("f32", "bf16"):
        epv = 8 if dtype == "bf16" else 4
        for n_parts in (1, 2, 3, 4, 5, 6):
            for n in (epv * 512 * 3 + 5 * epv + 3, epv * 1024):
                parts_h = [wl.hidden_states(60 + 7 * n_parts + r, 1, n, dtype).reshape(-1)
                           for r in range(n_parts)]
                parts = [to_dev(p) for p in parts_h]
                ref = oracle.sum_partials(parts_h)
                what = (dtype, n_parts, n)
                assert to_host(vpe.vpe_sum_partials(parts)).tobytes() == ref.tobytes(), what
                # in place into the last partial
                vpe.vpe_sum_partials(parts, out=parts[-1])
                assert to_host(parts[-1]).tobytes() == ref.tobytes(), what


# ---------------------------------------------------------------------------
# last-position select
# ---------------------------------------------------------------------------
def test_select_prefill_workload():
    d = _inputs("qwen3_0p6b_tp1_prefill")
    out = vpe.vpe_last_token_select(to_dev(d["hidden"]), to_dev(d["cu"]))
    ref = oracle.last_token_select(d["hidden"], d["cu"])
    assert to_host(out).tobytes() == ref.tobytes()


@pytest.mark.parametrize("dtype,dim", [("bf16", 1024), ("bf16", 3), ("f32", 4), ("f32", 130)])
def test_select_ragged(dtype, dim):
    cu = wl.cu_seqlens_ragged(40 + dim, 37, 1, 50)
    H = wl.hidden_states(41, int(cu[-1]), dim, dtype)
    out = vpe.vpe_last_token_select(to_dev(H), to_dev(cu))
    assert to_host(out).tobytes() == oracle.last_token_select(H, cu).tobytes()


def test_select_out_of_range_index_gives_zero_row():
    H = np.arange(40, dtype=np.float32).reshape(10, 4) + 1
    cu = np.array([0, 0, 4, 10, 12], dtype=np.int32)  # an empty first sequence; 12 > 10 tokens
    out = to_host(vpe.vpe_last_token_select(to_dev(H), to_dev(cu)))
    assert np.all(out[0] == 0) and np.all(out[3] == 0)
    assert out[1].tobytes() == H[3].tobytes() and out[2].tobytes() == H[9].tobytes()


# ---------------------------------------------------------------------------
# LM head: small and ragged shapes, full oracle comparison
# ---------------------------------------------------------------------------
LM_SHAPES = [
    # (m, n, k): tile multiples, ragged tails in every dimension, K not a multiple of 8
    (1, 1, 8), (3, 5, 7), (16, 128, 64), (17, 129, 65), (32, 1000, 200), (64, 777, 1024),
    (65, 300, 96), (128, 256, 128), (130, 515, 264), (257, 131, 40), (300, 2100, 1024),
    # past 128 rows with K not a multiple of 8: the 256 x 128 tile staged through registers
    (200, 300, 37), (300, 700, 45),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,k", LM_SHAPES)
def test_lmhead_shapes(dtype, m, n, k):
    X = wl.hidden_states(50 + m, m, k, dtype)
    W = wl.table_rows(60 + n, n, k, dtype, 0, n, std=0.5)
    got = to_host(vpe.vpe_lmhead(to_dev(X), to_dev(W)))
    ref = oracle.lmhead_f64(X, W, nthreads=oracle_threads())
    assert_logits_close(got, ref, f"lmhead {dtype} {m}x{n}x{k}")


def _shifted(a, on):
    """a on the device, one element past a 16-byte boundary when `on` (the
    boundary requires element alignment only)."""
    if not on:
        return to_dev(a)
    src = to_dev(a)
    flat = torch.empty(src.numel() + 1, dtype=src.dtype, device=dev())
    view = flat[1:].view(src.shape)
    view.copy_(src)
    assert view.data_ptr() % 16 != 0
    return view


@pytest.mark.parametrize("m", [8, 40, 100, 200, 300])
@pytest.mark.parametrize("which", ["x", "w", "both"])
def test_lmhead_unaligned_operands(m, which):
    # bf16 operands that cannot take 16-byte loads (K a multiple of 8): every
    # tile shape then stages them through registers
    n, k = 700, 72
    X = wl.hidden_states(80 + m, m, k, "bf16")
    W = wl.table_rows(81, n, k, "bf16", 0, n, std=0.5)
    x_d, w_d = _shifted(X, which in ("x", "both")), _shifted(W, which in ("w", "both"))
    got = to_host(vpe.vpe_lmhead(x_d, w_d))
    assert_logits_close(got, oracle.lmhead_f64(X, W), f"lmhead unaligned {which} m={m}")


@pytest.mark.parametrize("m", [8, 24, 40])
def test_lmhead_unaligned_long_shard(m):
    # a 70000-row shard takes the 192-row decode tiles; unaligned operands
    # stage them through registers
    n, k = 70000, 72
    X = wl.hidden_states(90 + m, m, k, "bf16")
    W = wl.table_rows(91, n, k, "bf16", 0, n, std=0.5)
    got = to_host(vpe.vpe_lmhead(_shifted(X, True), _shifted(W, True)))
    assert_logits_close(got, oracle.lmhead_f64(X, W, nthreads=oracle_threads()),
                        f"lmhead unaligned long shard m={m}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("ld,col", [(1500, 0), (1500, 500), (1501, 3), (1003, 1)])
def test_lmhead_writes_only_its_columns(dtype, ld, col):
    m, n, k = 40, 1000, 128
    X = wl.hidden_states(70, m, k, dtype)
    W = wl.table_rows(71, n, k, dtype, 0, n, std=0.5)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    logits = torch.full((m, ld), -1536.0, dtype=tdt, device=dev())  # exact in bf16
    vpe.vpe_lmhead(to_dev(X), to_dev(W), logits, col_offset=col)
    got = to_host(logits)
    ref = oracle.lmhead_f64(X, W)
    assert_logits_close(got[:, col:col + n], ref, f"lmhead {dtype} ld={ld} col={col}")
    sentinel = as_f64(got)
    assert np.all(sentinel[:, :col] == -1536.0) and np.all(sentinel[:, col + n:] == -1536.0)


# ---------------------------------------------------------------------------
# LM head at the workloads
# ---------------------------------------------------------------------------
def _lm_run(d, logits_cols, col_of):
    w = d["w"]
    x_h = _lm_rows(d)
    tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    logits = torch.empty((x_h.shape[0], logits_cols), dtype=tdt, device=dev())
    x_d = to_dev(x_h)
    for r in w.ranks:
        vpe.vpe_lmhead(x_d, to_dev(d["shards"][r]), logits, col_offset=col_of(r))
    return x_h, to_host(logits)


@pytest.mark.parametrize("name", wl.WORKLOAD_ORDER)
def test_lmhead_workload_full(name):
    # every logit of every workload against the fp64 oracle, the concatenated
    # workloads over the whole [M, V] buffer (the shard logits concatenated
    # must equal the full product everywhere: [TP-vocab] section 6).  The
    # largest, [4096, 37984] x 4096, is 1.27 TFLOP of fp64 loops: about half
    # a minute on 16 host threads.
    d = _inputs(name)
    w = d["w"]
    _say(f"lmhead {name}: M={w.lm_rows} shard rows={w.shard_rows} dim={w.dim}")
    if w.concat:
        x_h, got = _lm_run(d, w.vocab, w.rank_start)
    else:
        x_h, got = _lm_run(d, w.shard_rows, lambda r: 0)
    ref = np.zeros(got.shape, dtype=np.float64)
    for r in w.ranks:
        oracle.lmhead_f64(x_h, d["shards"][r], out=ref,
                          col_offset=w.rank_start(r) if w.concat else 0,
                          nthreads=oracle_threads())
    _say(f"lmhead {name}: oracle done")
    assert_logits_close(got, ref, name)


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------
def test_empty_calls_are_no_ops():
    W = to_dev(np.ones((8, 16), np.float32))
    out = vpe.vpe_embed(to_dev(np.zeros(0, np.int32)), W, 0)
    assert out.shape == (0, 16)
    logits = vpe.vpe_lmhead(to_dev(np.zeros((0, 16), np.float32)), W)
    assert logits.shape == (0, 8)
    sel = vpe.vpe_last_token_select(to_dev(np.zeros((0, 16), np.float32)),
                                    to_dev(np.zeros(1, np.int32)))
    assert sel.shape == (0, 16)
    torch.cuda.synchronize()


@pytest.mark.parametrize("dtype,dim", [("bf16", 1), ("bf16", 3), ("bf16", 8), ("bf16", 520),
                                       ("f32", 1), ("f32", 2), ("f32", 6), ("f32", 300),
                                       ("bf16", 8200)])
@pytest.mark.parametrize("itype", [np.int32, np.int64])
def test_embed_odd_dims_and_out_of_range_ids(dtype, dim, itype):
    V, tp, rank = 96, 3, 1
    start = V // tp * rank
    shard = wl.table_rows(80, V, dim, dtype, start, start + V // tp)
    rng = np.random.default_rng(dim)
    ids = rng.integers(-1000, V + 1000, size=333).astype(itype)
    ids[:4] = [start, start + V // tp - 1, start - 1, start + V // tp]
    if itype == np.int64:
        ids[4:6] = [-(2 ** 40), 2 ** 40 + start]  # would alias into the shard if truncated
    got = to_host(vpe.vpe_embed(to_dev(ids), to_dev(shard), start))
    assert got.tobytes() == oracle.embed(ids, shard, start).tobytes()


def test_binding_rejects_bad_arguments():
    W = to_dev(np.ones((8, 16), np.float32))
    x = to_dev(np.ones((2, 16), np.float32))
    with pytest.raises(vpe.VpeError) as e:
        vpe.vpe_lmhead(x, W, torch.empty((2, 10), device=dev()), col_offset=4)
    assert e.value.status == vpe.VPE_ERR_RANGE
    with pytest.raises(TypeError):
        vpe.vpe_lmhead(x.to(torch.bfloat16), W)
    with pytest.raises(vpe.VpeError) as e:
        vpe.vpe_shard_range(151936, 3, 0)
    assert e.value.status == vpe.VPE_ERR_SHARD


# ---------------------------------------------------------------------------
# prefill LM head with the last-position select folded in
# ---------------------------------------------------------------------------
def test_lmhead_prefill_workload():
    d = _inputs("qwen3_0p6b_tp1_prefill")
    w = d["w"]
    _say(f"lmhead_prefill {w.name}: T={d['hidden'].shape[0]} S={w.seqs} rows={w.shard_rows}")
    H = to_dev(d["hidden"])
    cu = to_dev(d["cu"])
    Wd = to_dev(d["shards"][0])
    got_t = vpe.vpe_lmhead_prefill(H, cu, Wd)
    unfused = vpe.vpe_lmhead(vpe.vpe_last_token_select(H, cu), Wd)
    got = to_host(got_t)
    # same tiles, same k order: the fused call is the composition, bit for bit
    assert got.tobytes() == to_host(unfused).tobytes()
    ref = oracle.lmhead_f64(oracle.last_token_select(d["hidden"], d["cu"]), d["shards"][0],
                            nthreads=oracle_threads())
    assert_logits_close(got, ref, "lmhead_prefill qwen3 prefill")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seqs,dim,rows", [(1, 64, 100), (7, 200, 333), (37, 1024, 1000),
                                          (130, 96, 700), (300, 72, 515)])
def test_lmhead_prefill_ragged(dtype, seqs, dim, rows):
    cu = wl.cu_seqlens_ragged(200 + seqs, seqs, 1, 40)
    H = wl.hidden_states(201 + seqs, int(cu[-1]), dim, dtype)
    W = wl.table_rows(202 + seqs, rows, dim, dtype, 0, rows, std=0.5)
    ld, col = rows + 9, 5
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    logits = torch.full((seqs, ld), -1536.0, dtype=tdt, device=dev())
    vpe.vpe_lmhead_prefill(to_dev(H), to_dev(cu), to_dev(W), logits, col_offset=col)
    got = to_host(logits)
    ref = oracle.lmhead_f64(oracle.last_token_select(H, cu), W)
    assert_logits_close(got[:, col:col + rows], ref, f"prefill {dtype} S={seqs} D={dim}")
    g = as_f64(got)
    assert np.all(g[:, :col] == -1536.0) and np.all(g[:, col + rows:] == -1536.0)


@pytest.mark.parametrize("seqs,dim,rows,seq_len", [
    (32, 1024, 151936, 2048),  # the prefill workload's shape, 4 MB between rows
    (17, 520, 3000, 700),      # K past two 256-column chunks, the last one partial
    (1, 72, 640, 50),          # K inside one chunk, not a multiple of 64
    (32, 4096, 3001, 300),     # 16 chunks; ragged tile tail
    (5, 256, 129, 9),          # exactly one chunk
])
def test_prefill_gathered_rows_equal_select_then_lmhead(seqs, dim, rows, seq_len):
    # up to 32 gathered rows take the kernel that keeps X resident in LDS in
    # chunks of 256 columns: logits and greedy-pick keys must equal those of
    # the select followed by the LM head bit for bit, and the oracle's
    cu = wl.cu_seqlens_ragged(240 + seqs, seqs, max(1, seq_len // 2), seq_len)
    H = wl.hidden_states(241 + seqs, int(cu[-1]), dim, "bf16")
    W = wl.table_rows(242 + seqs, rows, dim, "bf16", 0, rows, std=0.5)
    _say(f"prefill gathered S={seqs} D={dim} R={rows} T={int(cu[-1])}")
    H_d, cu_d, W_d = to_dev(H), to_dev(cu), to_dev(W)
    ld, col = rows + 11, 3
    fused = torch.full((seqs, ld), -1536.0, dtype=torch.bfloat16, device=dev())
    vpe.vpe_lmhead_prefill(H_d, cu_d, W_d, fused, col_offset=col)
    sel = vpe.vpe_last_token_select(H_d, cu_d)
    plain = torch.full((seqs, ld), -1536.0, dtype=torch.bfloat16, device=dev())
    vpe.vpe_lmhead(sel, W_d, plain, col_offset=col)
    got = to_host(fused)
    assert got.tobytes() == to_host(plain).tobytes()
    ref = oracle.lmhead_f64(oracle.last_token_select(H, cu), W, nthreads=oracle_threads())
    assert_logits_close(got[:, col:col + rows], ref, f"gathered prefill S={seqs} D={dim}")
    g = as_f64(got)
    assert np.all(g[:, :col] == -1536.0) and np.all(g[:, col + rows:] == -1536.0)
    keys = []
    for fn in ("fused", "plain"):
        best = torch.empty(seqs, dtype=torch.int64, device=dev())
        vpe.vpe_argmax_init(best)
        if fn == "fused":
            vpe.vpe_lmhead_prefill_argmax(H_d, cu_d, W_d, 7, best)
        else:
            vpe.vpe_lmhead_argmax(sel, W_d, 7, best)
        keys.append(to_host(best))
    assert np.array_equal(keys[0], keys[1])
    _, tok = vpe.vpe_argmax_decode(torch.from_numpy(keys[0]).to(dev()))
    assert np.array_equal(to_host(tok), np.argmax(g[:, col:col + rows], axis=1) + 7)


def test_lmhead_prefill_out_of_range_sequence_gives_zero_logits():
    H = wl.hidden_states(210, 10, 64, "bf16")
    W = wl.table_rows(211, 50, 64, "bf16", 0, 50, std=0.5)
    cu = np.array([0, 0, 4, 10, 12], dtype=np.int32)  # empty first sequence; 12 > 10 tokens
    got = as_f64(to_host(vpe.vpe_lmhead_prefill(to_dev(H), to_dev(cu), to_dev(W))))
    assert np.all(got[0] == 0) and np.all(got[3] == 0)
    ref = oracle.lmhead_f64(H[[3, 9]], W)
    assert_logits_close(got[1:3].astype(np.float64), ref, "prefill valid rows")


@pytest.mark.parametrize("seqs", [5, 300])
def test_lmhead_prefill_hidden_past_the_masked_load_offset(seqs):
    # packed activations of 1048560 x 1024 bf16 (2147450880 bytes) lie past
    # the byte offset 0x7FFF0000 at which masked buffer loads are issued and
    # below 2^31: the launcher must stage X element-wise there, so that a
    # sequence ending past the tokens still gets zero logits (a buffer load at
    # the masked offset would read row 1048544 instead).  5 sequences take a
    # decode-size tile, 300 the large-M kernels.
    T, D, n = 1048560, 1024, 200
    assert 0x7FFF0000 < T * D * 2 < 2 ** 31
    rng = np.random.default_rng(230 + seqs)
    ends = np.sort(rng.choice(np.arange(1, T), size=seqs - 2, replace=False))
    ends = np.concatenate([ends, [T]])  # the last valid sequence reads the last row
    cu = np.concatenate([[0], ends, [T + 10]]).astype(np.int32)
    _say(f"lmhead_prefill past the masked offset: T={T} S={seqs}")
    Xv = wl.hidden_states(231 + seqs, seqs - 1, D, "bf16")
    W = wl.table_rows(232, n, D, "bf16", 0, n, std=0.5)
    H = torch.ones((T, D), dtype=torch.bfloat16, device=dev())  # non-zero everywhere else
    H[torch.from_numpy(ends - 1).to(dev())] = to_dev(Xv)
    cu_d, W_d = to_dev(cu), to_dev(W)
    got = as_f64(to_host(vpe.vpe_lmhead_prefill(H, cu_d, W_d)))
    assert np.all(got[-1] == 0), "sequence past the tokens read real rows"
    assert_logits_close(got[:-1], oracle.lmhead_f64(Xv, W), "prefill rows past 0x7FFF0000")
    best = torch.empty(seqs, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    vpe.vpe_lmhead_prefill_argmax(H, cu_d, W_d, 0, best)
    val, tok = vpe.vpe_argmax_decode(best)
    assert np.array_equal(to_host(tok), np.argmax(got, axis=1))
    assert to_host(val)[-1] == 0 and to_host(tok)[-1] == 0
    del H
    torch.cuda.empty_cache()


def test_parallel_lmhead_layer_prefill_and_decode():
    V, D, tp = 512, 128, 2
    full = wl.table_rows(220, V, D, "bf16", 0, V)
    cu = wl.cu_seqlens_ragged(221, 5, 1, 9)
    H = wl.hidden_states(222, int(cu[-1]), D, "bf16")
    full_d = to_dev(full).view(torch.bfloat16)
    logits = torch.empty((5, V), dtype=torch.bfloat16, device=dev())
    for r in range(tp):
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev())
        head.weight_loader(head.weight, full_d)
        head(to_dev(H), cu_seqlens=to_dev(cu), logits=logits)
    ref = oracle.lmhead_f64(oracle.last_token_select(H, cu), full)
    assert_logits_close(to_host(logits), ref, "ParallelLMHead prefill")
    emb = [vpe.VocabParallelEmbedding(V, D, tp_size=tp, tp_rank=r, device=dev()) for r in range(tp)]
    ids = wl.token_ids(223, V, 77)
    parts = []
    for e in emb:
        e.weight_loader(e.weight, full_d)
        parts.append(e(to_dev(ids)))
    total = to_host(vpe.VocabParallelEmbedding.sum_partials(parts))
    assert total.tobytes() == oracle.embed(ids, full, 0).tobytes()


# ---------------------------------------------------------------------------
# greedy pick over the vocabulary without materialising the logits
# ---------------------------------------------------------------------------
def _int_inputs(seed, m, n, k, dtype, lo=-1, hi=1):
    """Small-integer X and W: every logit is an integer of magnitude <= k, exact
    in fp32 accumulation and (k <= 256) in bf16, so both sides decide on the
    same values and equal logits are common."""
    rng = np.random.default_rng(seed)
    X = rng.integers(lo, hi + 1, size=(m, k)).astype(np.float32)
    W = rng.integers(lo, hi + 1, size=(n, k)).astype(np.float32)
    if dtype == "bf16":
        X, W = wl.f32_to_bf16_bits(X), wl.f32_to_bf16_bits(W)
    return X, W


def _pick(x_d, shards, starts, order=None):
    best = torch.empty(x_d.shape[0], dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    for r in (order if order is not None else range(len(shards))):
        vpe.vpe_lmhead_argmax(x_d, shards[r], starts[r], best)
    val, tok = vpe.vpe_argmax_decode(best)
    return to_host(val).astype(np.float64), to_host(tok)


ARGMAX_SHAPES = [(1, 1, 8), (3, 5, 7), (16, 128, 64), (17, 129, 65), (40, 1000, 128),
                 (64, 777, 256), (100, 515, 96), (257, 1300, 64), (300, 2100, 200)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,k", ARGMAX_SHAPES)
def test_argmax_exact_on_integer_logits(dtype, m, n, k):
    # integer logits: the oracle's first maximum is the unique right answer
    X, W = _int_inputs(300 + m + n, m, n, k, dtype)
    val, tok = _pick(to_dev(X), [to_dev(W)], [0])
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, W))
    assert np.array_equal(tok, ref_idx), f"{dtype} {m}x{n}x{k}"
    assert np.array_equal(val, ref_max)


@pytest.mark.parametrize("m", [1, 300, 5000])
def test_argmax_decode_clear_leaves_keys_ready(m):
    # the clearing decode returns what the plain decode returns and leaves
    # every key at 0, so a second round of folds needs no init
    n, k = 700, 64
    X1, W = _int_inputs(500 + m, m, n, k, "bf16")
    X2, _ = _int_inputs(600 + m, m, n, k, "bf16")
    w_d = to_dev(W)
    best = torch.empty(m, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    vpe.vpe_lmhead_argmax(to_dev(X1), w_d, 0, best)
    keys = best.clone()
    val1, tok1 = vpe.vpe_argmax_decode_clear(best)
    val0, tok0 = vpe.vpe_argmax_decode(keys)
    assert np.array_equal(to_host(tok1), to_host(tok0))
    assert to_host(val1).tobytes() == to_host(val0).tobytes()
    assert int(torch.count_nonzero(best)) == 0
    vpe.vpe_lmhead_argmax(to_dev(X2), w_d, 0, best)
    val2, tok2 = vpe.vpe_argmax_decode_clear(best)
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X2, W))
    assert np.array_equal(to_host(tok2), ref_idx)
    assert np.array_equal(to_host(val2).astype(np.float64), ref_max)
    assert int(torch.count_nonzero(best)) == 0


@pytest.mark.parametrize("m", [8, 100, 300])
def test_argmax_unaligned_operands(m):
    # the greedy pick on operands one element past a 16-byte boundary
    n, k = 900, 64
    X, W = _int_inputs(400 + m, m, n, k, "bf16")
    val, tok = _pick(_shifted(X, True), [_shifted(W, True)], [0])
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, W))
    assert np.array_equal(tok, ref_idx) and np.array_equal(val, ref_max), f"m={m}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("tp,order", [(2, "forward"), (2, "reverse"), (4, "reverse"), (3, "forward")])
def test_argmax_shards_combine_to_global_first_maximum(dtype, tp, order):
    m, V, k = 70, 3001, 64
    X, W = _int_inputs(330 + tp, m, V, k, dtype, lo=0, hi=1)
    # plant equal maxima in every shard for a few rows: the smallest id must win
    per = -(-V // tp)
    starts = [min(r * per, V) for r in range(tp)]
    ends = [min((r + 1) * per, V) for r in range(tp)]
    one = np.float32(1) if dtype == "f32" else wl.f32_to_bf16_bits(np.ones((1, 1), np.float32))[0, 0]
    for r in range(tp):
        W[ends[r] - 1, :] = one  # logit = row sum of X, the largest possible
    x_d = to_dev(X)
    shards = [to_dev(W[s:e]) for s, e in zip(starts, ends)]
    seq = list(range(tp)) if order == "forward" else list(reversed(range(tp)))
    val, tok = _pick(x_d, shards, starts, seq)
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, W))
    assert np.array_equal(tok, ref_idx) and np.array_equal(val, ref_max)
    # X >= 0, so shard 0's planted row reaches every row's maximum
    assert np.all(tok <= ends[0] - 1)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n", [(5, 130), (33, 321), (129, 333)])
def test_argmax_ignores_padding_columns_when_all_logits_are_negative(dtype, m, n):
    # every logit < 0: a padded column read as zero would win if it were not excluded
    X, W = _int_inputs(360 + m, m, n, 64, dtype, lo=1, hi=2)
    Wn = W ^ np.uint16(0x8000) if dtype == "bf16" else -W
    val, tok = _pick(to_dev(X), [to_dev(Wn)], [0])
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, Wn))
    assert np.all(ref_max < 0)
    assert np.array_equal(tok, ref_idx) and np.array_equal(val, ref_max)


def test_argmax_matches_the_stored_logits_bit_for_bit():
    # the pick is the first maximum of exactly the logits vpe_lmhead stores
    for m, n, k in [(16, 2000, 1024), (64, 1500, 1024), (100, 1000, 512), (300, 1700, 256)]:
        X = wl.hidden_states(380 + m, m, k, "bf16")
        W = wl.table_rows(381 + m, n, k, "bf16", 0, n, std=0.5)
        x_d, w_d = to_dev(X), to_dev(W)
        stored = as_f64(to_host(vpe.vpe_lmhead(x_d, w_d)))
        val, tok = _pick(x_d, [w_d], [1000])
        assert np.array_equal(tok - 1000, np.argmax(stored, axis=1)), f"{m}x{n}x{k}"
        assert np.array_equal(val, stored.max(axis=1))


def _first_max_in_key_order(stored_bits):
    """Per row: (bf16 bits, first column) of the largest 16-bit order code
    (-0 below +0, a positive NaN above +Inf, a negative one below -Inf)."""
    h = stored_bits.astype(np.uint32)
    code = np.where(h & 0x8000, ~h & 0xFFFF, h | 0x8000)
    col = np.argmax(code, axis=1)
    return h[np.arange(h.shape[0]), col], col


@pytest.mark.parametrize("m", [8, 40, 200, 300])
@pytest.mark.parametrize("case", ["ties", "inf", "nan", "zero_rows", "tiny"])
def test_argmax_special_rows_match_stored_logits(m, case):
    # Rows built so that many distinct fp32 logits round to the same bf16 top
    # value (the first of them must win), and rows with infinite or NaN logits
    # or a maximum that rounds to +-0, which the kernels decide on a separate
    # exact path.  The reference is the first maximum, in key order, of the
    # logits vpe_lmhead stores for the same inputs.  n = 700 leaves a partial
    # last tile in every kernel.
    rng = np.random.default_rng(500 + m)
    n, k = 700, 32
    X = np.zeros((m, k), np.float32)
    W = rng.standard_normal((n, k)).astype(np.float32)
    X[:, 0] = 1.0
    X[:, 1] = np.float32(2.0 ** -6)
    W[:, 0] = rng.integers(0, 4, size=n).astype(np.float32)  # coarse part: many equal tops
    W[:, 1] = rng.uniform(-1, 1, size=n).astype(np.float32)   # fine part: about one bf16 ulp
    W[:, 2:] = 0.0
    Xb, Wb = wl.f32_to_bf16_bits(X), wl.f32_to_bf16_bits(W)
    if case == "inf":
        Wb[123, 2] = 0x7F80                     # +Inf: rows with x[2] != 0 see +-Inf, others NaN
        Xb[::3, 2] = wl.f32_to_bf16_bits(np.float32([[1.0]]))[0, 0]
    elif case == "nan":
        Wb[456, 3] = 0x7FC0                     # a NaN column in every row
    elif case == "zero_rows":
        Xb[::2, :] = 0                          # +0 rows: every logit is +-0
        Xb[1::4, :] = 0x8000                    # -0 rows
    elif case == "tiny":
        Xb[:, :] = 0
        Xb[:, 0] = wl.f32_to_bf16_bits(np.float32([[2.0 ** -70]]))[0, 0]
        Wb[:, 0] = wl.f32_to_bf16_bits(-np.float32(2.0 ** -70) *
                                       rng.integers(1, 4, size=(n, 1)).astype(np.float32))[:, 0]
    x_d, w_d = to_dev(Xb), to_dev(Wb)
    stored = to_host(vpe.vpe_lmhead(x_d, w_d))
    top, col = _first_max_in_key_order(stored)
    best = torch.empty(m, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    vpe.vpe_lmhead_argmax(x_d, w_d, 5000, best)
    val, tok = vpe.vpe_argmax_decode(best)
    tok = to_host(tok)
    bits = to_host(val).view(np.uint32)
    assert np.array_equal(tok - 5000, col), f"{case} m={m}"
    assert np.array_equal(bits >> 16, top) and not np.any(bits & 0xFFFF), f"{case} m={m}"


@pytest.mark.parametrize("name", ["qwen3_0p6b_tp2_rank0", "qwen3_0p6b_tp2_all_ranks"])
def test_argmax_workload_is_a_valid_greedy_pick(name):
    d = _inputs(name)
    w = d["w"]
    _say(f"argmax {name}: M={w.lm_rows} ranks={list(w.ranks)} rows={w.shard_rows}")
    x_h = _lm_rows(d)
    x_d = to_dev(x_h)
    shards = [to_dev(d["shards"][r]) for r in w.ranks]
    starts = [w.rank_start(r) for r in w.ranks]
    val, tok = _pick(x_d, shards, starts, list(reversed(range(len(shards)))))
    # against the logits the library stores: exact
    stored = np.full((x_h.shape[0], w.vocab), -np.inf)
    for s, wd in zip(starts, shards):
        stored[:, s:s + w.shard_rows] = as_f64(to_host(vpe.vpe_lmhead(x_d, wd)))
    assert np.array_equal(tok, np.argmax(stored, axis=1))
    assert np.array_equal(val, stored.max(axis=1))
    # against the oracle on sampled rows: the pick's fp64 logit is within the
    # logit tolerance of the fp64 maximum, and the reported value within
    # tolerance of the pick's fp64 logit
    rng = np.random.default_rng(7)
    M = x_h.shape[0]
    nt = oracle_threads()
    for m in sorted({0, M - 1, *rng.integers(0, M, size=6).tolist()}):
        ref = np.full((1, w.vocab), -np.inf)
        for r, s in zip(w.ranks, starts):
            ref[:, s:s + w.shard_rows] = oracle.lmhead_f64(x_h[m:m + 1], d["shards"][r],
                                                           nthreads=nt)
        ref_max, _ = oracle.argmax_rows(ref)
        at_pick = ref[0, tok[m]]
        tol = 1e-2 + 1e-2 * abs(ref_max[0])
        assert ref_max[0] - at_pick <= 2 * tol, f"{name} row {m}"
        assert abs(val[m] - at_pick) <= 1e-2 + 1e-2 * abs(at_pick), f"{name} row {m}"


def _keys(fn):
    """Run fn(best) on fresh keys and return the raw keys (uint64 as int64)."""
    def run(m):
        best = torch.empty(m, dtype=torch.int64, device=dev())
        vpe.vpe_argmax_init(best)
        fn(best)
        return to_host(best)
    return run


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("seqs,dim,V,tp", [(1, 64, 100, 1), (7, 200, 999, 3), (37, 1024, 2000, 2),
                                          (130, 96, 700, 1), (300, 72, 1030, 2)])
def test_prefill_argmax_equals_select_then_argmax(dtype, seqs, dim, V, tp):
    # the fused pick reads each sequence's last position itself; its keys must
    # equal those of the select followed by the pick on the selected rows, for
    # every shard split, folded in reverse order; one sequence ends past the
    # tokens (a row of zero logits) and one is empty
    cu = wl.cu_seqlens_ragged(600 + seqs, seqs, 1, 40).astype(np.int64)
    if seqs > 2:
        cu[2] = cu[1]                      # empty sequence 1: its last index is cu[1] - 1
        cu[-1] = cu[-1] + 5                # last sequence ends past the tokens
    cu = cu.astype(np.int32)
    T = int(cu[-2]) + 3 if seqs > 2 else int(cu[-1])
    H = wl.hidden_states(601 + seqs, T, dim, dtype)
    full = wl.table_rows(602 + seqs, V, dim, dtype, 0, V, std=0.5)
    H_d, cu_d = to_dev(H), to_dev(cu)
    per = V // tp
    shards = [(r * per, to_dev(full[r * per:(r + 1) * per])) for r in range(tp)]
    fused = _keys(lambda best: [vpe.vpe_lmhead_prefill_argmax(H_d, cu_d, w, s, best)
                                for s, w in reversed(shards)])(seqs)
    X_d = vpe.vpe_last_token_select(H_d, cu_d)
    unfused = _keys(lambda best: [vpe.vpe_lmhead_argmax(X_d, w, s, best)
                                  for s, w in reversed(shards)])(seqs)
    assert np.array_equal(fused, unfused), f"{dtype} S={seqs} D={dim} V={V} tp={tp}"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_prefill_argmax_exact_on_integer_logits(dtype):
    # integer hidden states and table: the oracle's first maximum over the
    # selected rows' exact logits is the unique right answer
    seqs, dim, V = 45, 64, 1500
    cu = wl.cu_seqlens_ragged(620, seqs, 1, 30)
    T = int(cu[-1])
    rng = np.random.default_rng(621)
    H = rng.integers(-1, 2, size=(T, dim)).astype(np.float32)
    W = rng.integers(-1, 2, size=(V, dim)).astype(np.float32)
    if dtype == "bf16":
        H, W = wl.f32_to_bf16_bits(H), wl.f32_to_bf16_bits(W)
    best = torch.empty(seqs, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    vpe.vpe_lmhead_prefill_argmax(to_dev(H), to_dev(cu), to_dev(W), 0, best)
    val, tok = vpe.vpe_argmax_decode(best)
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(oracle.last_token_select(H, cu), W))
    assert np.array_equal(to_host(tok), ref_idx)
    assert np.array_equal(to_host(val).astype(np.float64), ref_max)


def test_prefill_argmax_workload():
    d = _inputs("qwen3_0p6b_tp1_prefill")
    w = d["w"]
    _say(f"prefill argmax {w.name}: T={d['hidden'].shape[0]} S={w.seqs} rows={w.shard_rows}")
    H, cu, Wd = to_dev(d["hidden"]), to_dev(d["cu"]), to_dev(d["shards"][0])
    fused = _keys(lambda best: vpe.vpe_lmhead_prefill_argmax(H, cu, Wd, 0, best))(w.seqs)
    stored = as_f64(to_host(vpe.vpe_lmhead_prefill(H, cu, Wd)))
    val, tok = vpe.vpe_argmax_decode(torch.from_numpy(fused).to(dev()))
    assert np.array_equal(to_host(tok), np.argmax(stored, axis=1))
    assert np.array_equal(to_host(val).astype(np.float64), stored.max(axis=1))


def test_parallel_lmhead_layer_fold_argmax():
    V, D, tp, m = 1000, 64, 4, 9
    X, full = _int_inputs(390, m, V, D, "bf16")
    full_d = to_dev(full)
    best = torch.empty(m, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    for r in reversed(range(tp)):
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev())
        head.weight_loader(head.weight, full_d)
        head.fold_argmax(to_dev(X), best)
    val, tok = vpe.vpe_argmax_decode(best)
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, full))
    assert np.array_equal(to_host(tok), ref_idx)
    assert np.array_equal(to_host(val).astype(np.float64), ref_max)
    # packed sequences: each rank folds in every sequence's last position
    cu = wl.cu_seqlens_ragged(391, 6, 1, 5)
    H, _ = _int_inputs(392, int(cu[-1]), 1, D, "bf16")
    best = torch.empty(6, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    for r in range(tp):
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev())
        head.weight_loader(head.weight, full_d)
        head.fold_argmax(to_dev(H), best, cu_seqlens=to_dev(cu))
    val, tok = vpe.vpe_argmax_decode(best)
    ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(oracle.last_token_select(H, cu), full))
    assert np.array_equal(to_host(tok), ref_idx)
    assert np.array_equal(to_host(val).astype(np.float64), ref_max)


# ---------------------------------------------------------------------------
# decode-size LM heads (a handful of rows against a whole shard)
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("m", [1, 2, 5, 8, 16, 25, 32])
@pytest.mark.parametrize("name", ["qwen3_0p6b_tp1_prefill", "large_v151936_d4096_tp4_rank2"])
def test_lmhead_decode_rows(name, m):
    _decode_rows(name, m)


@pytest.mark.parametrize("m", [1, 5, 16, 17, 24, 25, 32, 33, 48, 64, 65, 96, 128, 129])
def test_lmhead_decode_rows_tp2_shard(m):
    # the 75968-row shard takes 192-row decode tiles and 320 x 128 tiles up to
    # M = 128 (one round over the CUs)
    _decode_rows("qwen3_0p6b_tp2_rank0", m)


def _decode_rows(name, m):
    d = _inputs(name)
    w = d["w"]
    W = d["shards"][w.ranks[0]]
    _say(f"lmhead decode {name}: M={m} rows={w.shard_rows} dim={w.dim}")
    X = wl.hidden_states(600 + m, m, w.dim, w.dtype)
    x_d, w_d = to_dev(X), to_dev(W)
    got = to_host(vpe.vpe_lmhead(x_d, w_d))
    ref = oracle.lmhead_f64(X, W, nthreads=oracle_threads())
    assert_logits_close(got, ref, f"decode {name} M={m}")
    # the greedy pick agrees with the stored logits exactly
    val, tok = _pick(x_d, [w_d], [w.rank_start(w.ranks[0])])
    g = as_f64(got)
    assert np.array_equal(tok - w.rank_start(w.ranks[0]), np.argmax(g, axis=1))
    assert np.array_equal(val, g.max(axis=1))


# ---------------------------------------------------------------------------
# a table past 2 GiB: row offsets beyond the 32-bit range
# ---------------------------------------------------------------------------
def test_table_past_2gib():
    n, k, seed = 140000, 8192, 77  # 2.29 GB of bf16; row 131072 starts at byte 2^31
    w_d = torch.empty((n, k), dtype=torch.bfloat16, device=dev())
    for lo in range(0, n, 16384):
        hi = min(n, lo + 16384)
        w_d[lo:hi] = to_dev(wl.table_rows(seed, n, k, "bf16", lo, hi, std=0.5))
    ranges = [(0, 32), (131040, 131104), (n - 64, n)]
    cols = np.concatenate([np.arange(a, b) for a, b in ranges])
    w_cols = np.concatenate([wl.table_rows(seed, n, k, "bf16", a, b, std=0.5) for a, b in ranges])
    for m in (4, 300):
        _say(f"table past 2 GiB: lmhead M={m}")
        x = wl.hidden_states(900 + m, m, k, "bf16")
        got = to_host(vpe.vpe_lmhead(to_dev(x), w_d))
        assert_logits_close(got[:, cols], oracle.lmhead_f64(x, w_cols, nthreads=oracle_threads()),
                            f"past 2 GiB M={m}")
    _say("table past 2 GiB: lookup")
    ids = np.concatenate([cols, [131071, 131072, n - 1, n, -1]]).astype(np.int64)
    out = to_host(vpe.vpe_embed(to_dev(ids), w_d, 0))
    assert out[:len(cols)].tobytes() == w_cols.tobytes()
    assert np.all(out[-2:] == 0)  # ids n and -1 are outside the table
    del w_d
    torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# shard loading on the device, and one tied table for both calls
# ---------------------------------------------------------------------------
def test_load_shard_full_vocab_every_rank():
    d = _inputs("qwen3_0p6b_tp1_prefill")  # its only shard is the full 151936 x 1024 table
    full = d["shards"][0]
    full_d = to_dev(full)
    for tp in (2, 4):
        for r in range(tp):
            _say(f"load_shard full table tp={tp} rank={r}")
            got = to_host(vpe.vpe_load_shard(full_d, tp, r))
            assert got.tobytes() == oracle.load_shard(full, tp, r).tobytes(), (tp, r)


@pytest.mark.parametrize("dtype,dim,rows", [("bf16", 8, 40), ("bf16", 24, 17), ("f32", 3, 5)])
def test_lmhead_most_rows(dtype, dim, rows):
    # the largest M the LM head accepts (2**21 hidden rows): 8192 row tiles of
    # the large-M kernel, or 32768 row blocks of the fp32 kernel's grid
    m = 1 << 21
    x = wl.hidden_states(4300 + dim, m, dim, dtype)
    w = wl.table_rows(4301 + dim, rows, dim, dtype, 0, rows, std=0.5)
    _say(f"lmhead most rows: m={m} dim={dim} rows={rows} {dtype}")
    got = to_host(vpe.vpe_lmhead(to_dev(x), to_dev(w)))
    assert_logits_close(got, oracle.lmhead_f64(x, w, nthreads=oracle_threads()), "most rows")
    with pytest.raises(vpe.VpeError):
        vpe.vpe_lmhead(to_dev(np.zeros((m + 1, dim), dtype=x.dtype)), to_dev(w))


def test_embed_past_one_grid():
    # more rows than one grid takes (2**24 per launch): the lookup is split into
    # several grids, each starting at its own row of ids and output.  Short rows
    # (one 4-byte vector) compared in full; rows of 1040 bytes (the multi-row
    # wave path) sampled around the split and at random, row by row against the
    # oracle on the same ids.
    rng = np.random.default_rng(4242)
    n = (1 << 24) + 1000
    start, rows = 7000, 50000
    ids = rng.integers(start - 20000, start + rows + 20000, size=n).astype(np.int32)
    ids_d = to_dev(ids)
    shard = wl.table_rows(4243, 80000, 2, "bf16", start, start + rows)
    _say(f"embed past one grid: n={n} dim=2 bf16")
    got = to_host(vpe.vpe_embed(ids_d, to_dev(shard), start))
    assert got.tobytes() == oracle.embed(ids, shard, start, nthreads=oracle_threads()).tobytes()
    del got
    shard = wl.table_rows(4244, 80000, 520, "bf16", start, start + rows)
    _say(f"embed past one grid: n={n} dim=520 bf16")
    out = vpe.vpe_embed(ids_d, to_dev(shard), start)
    split = 1 << 24
    pick = np.concatenate([np.arange(split - 40, split + 40), np.arange(n - 8, n),
                           rng.integers(0, n, size=2000)])
    got = to_host(out[torch.from_numpy(pick).to(dev())])
    del out
    assert got.tobytes() == oracle.embed(ids[pick], shard, start).tobytes()


@pytest.mark.parametrize("dtype,dim", [("bf16", 4096), ("bf16", 2056), ("f32", 1030)])
def test_embed_many_long_rows(dtype, dim):
    # enough ids for several rows per wave on rows longer than 4 KB, with a
    # ragged last wave (n % 4 == 3), rows that need two passes of the wave
    # (2056 bf16 = 257 vectors), 8-byte vectors (1030 fp32), and ids below,
    # inside and past the shard
    rng = np.random.default_rng(900 + dim)
    rows, start, n = 3001, 5000, 4 * 8 * 4 * 256 + 3
    shard = wl.table_rows(910 + dim, 9000, dim, dtype, start, start + rows)
    ids = rng.integers(start - 2000, start + rows + 2000, size=n).astype(np.int32)
    _say(f"embed many long rows {dtype} dim={dim} n={n}")
    got = to_host(vpe.vpe_embed(to_dev(ids), to_dev(shard), start))
    assert got.tobytes() == oracle.embed(ids, shard, start, nthreads=oracle_threads()).tobytes()


@pytest.mark.parametrize("dtype,vocab,dim", [("f32", 12, 3), ("f32", 96, 5), ("bf16", 30, 7),
                                             ("bf16", 64, 8), ("bf16", 4096, 1000),
                                             ("f32", 6, 1)])
def test_load_shard_odd_rows(dtype, vocab, dim):
    # rows whose byte length is not a multiple of 16: shard starts and ends fall
    # off 16-byte boundaries (bytewise path) or leave a tail after the vectors
    full = wl.table_rows(700 + vocab, vocab, dim, dtype, 0, vocab)
    full_d = to_dev(full)
    for tp in [t for t in (1, 2, 3, 4, 6) if vocab % t == 0]:
        for r in range(tp):
            out = torch.full((vocab // tp, dim), -1536.0, dtype=full_d.dtype, device=dev())
            vpe.vpe_load_shard(full_d, tp, r, out=out)
            assert to_host(out).tobytes() == oracle.load_shard(full, tp, r).tobytes()


def test_weight_loader_and_tied_head():
    V, D, tp = 1024, 96, 4
    full = wl.table_rows(710, V, D, "bf16", 0, V)
    full_d = to_dev(full)
    ids = wl.token_ids(711, V, 300)
    X = wl.hidden_states(712, 7, D, "bf16")
    parts = []
    logits = torch.empty((7, V), dtype=torch.bfloat16, device=dev())
    for r in range(tp):
        emb = vpe.VocabParallelEmbedding(V, D, tp_size=tp, tp_rank=r, device=dev())
        emb.weight_loader(emb.weight, full_d)  # device table: the library's copy kernel
        assert to_host(emb.weight.data).tobytes() == oracle.load_shard(full, tp, r).tobytes()
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev()).tie_to(emb)
        assert head.weight.data_ptr() == emb.weight.data_ptr()
        parts.append(emb(to_dev(ids)))
        head(to_dev(X), logits=logits)
    total = to_host(vpe.VocabParallelEmbedding.sum_partials(parts))
    assert total.tobytes() == oracle.embed(ids, full, 0).tobytes()
    assert_logits_close(to_host(logits), oracle.lmhead_f64(X, full), "tied heads")
    with pytest.raises(ValueError):
        vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=0, device=dev()).tie_to(
            vpe.VocabParallelEmbedding(V, D, tp_size=tp, tp_rank=1, device=dev()))


# ---------------------------------------------------------------------------
# the path captured in a HIP graph: replays match eager launches bit for bit
# ---------------------------------------------------------------------------
def test_graph_replays_match_eager():
    V, D, tp, n_ids, m = 4096, 256, 2, 999, 40
    full = wl.table_rows(800, V, D, "bf16", 0, V)
    ids_d = to_dev(wl.token_ids(801, V, n_ids))
    x_d = to_dev(wl.hidden_states(802, m, D, "bf16"))
    shards = [to_dev(full[r * V // tp:(r + 1) * V // tp]) for r in range(tp)]
    starts = [r * V // tp for r in range(tp)]

    def path(parts, total, logits, best):
        for r in range(tp):
            vpe.vpe_embed(ids_d, shards[r], starts[r], out=parts[r])
        vpe.vpe_sum_partials(parts, out=total)
        for r in range(tp):
            vpe.vpe_lmhead(x_d, shards[r], logits, col_offset=starts[r])
        vpe.vpe_argmax_init(best)
        for r in range(tp):
            vpe.vpe_lmhead_argmax(x_d, shards[r], starts[r], best)
        return vpe.vpe_argmax_decode(best)

    def buffers():
        return ([torch.empty((n_ids, D), dtype=torch.bfloat16, device=dev()) for _ in range(tp)],
                torch.empty((n_ids, D), dtype=torch.bfloat16, device=dev()),
                torch.empty((m, V), dtype=torch.bfloat16, device=dev()),
                torch.empty(m, dtype=torch.int64, device=dev()))

    eb = buffers()
    e_val, e_tok = path(*eb)
    torch.cuda.synchronize()
    gb = buffers()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev())
    with torch.cuda.graph(g, stream=side):
        g_val, g_tok = path(*gb)
    for rep in range(3):
        # eager work between replays, including clearing every output
        for t in gb[0] + [gb[1], gb[2], gb[3]]:
            t.zero_()
        g_val.zero_()
        g_tok.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(eb[0] + [eb[1], eb[2]], gb[0] + [gb[1], gb[2]]):
            assert to_host(a).tobytes() == to_host(b).tobytes(), f"replay {rep}"
        assert torch.equal(e_tok, g_tok) and torch.equal(e_val, g_val), f"replay {rep}"
    # and the eager results are right
    assert to_host(eb[1]).tobytes() == oracle.embed(to_host(ids_d), full, 0).tobytes()


def test_graph_decode_loop_with_clearing_decode():
    # a captured decode step (every shard's fold, then the clearing decode)
    # replayed as a loop: the keys are set once, eagerly, before the loop, and
    # each replay leaves them cleared for the next one (no init in the graph)
    V, D, tp, m = 4096, 128, 2, 24
    _, W = _int_inputs(810, 1, V, D, "bf16")
    shards = [to_dev(W[r * V // tp:(r + 1) * V // tp]) for r in range(tp)]
    starts = [r * V // tp for r in range(tp)]
    x_d = torch.zeros((m, D), dtype=torch.bfloat16, device=dev())
    best = torch.empty(m, dtype=torch.int64, device=dev())
    vpe.vpe_argmax_init(best)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream(device=dev())
    with torch.cuda.graph(g, stream=side):
        for r in range(tp):
            vpe.vpe_lmhead_argmax(x_d, shards[r], starts[r], best)
        val, tok = vpe.vpe_argmax_decode_clear(best)
    for step in range(4):
        X, _ = _int_inputs(820 + step, m, 1, D, "bf16")
        x_d.copy_(to_dev(X))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_max, ref_idx = oracle.argmax_rows(oracle.lmhead_f64(X, W))
        assert np.array_equal(to_host(tok), ref_idx), f"step {step}"
        assert np.array_equal(to_host(val).astype(np.float64), ref_max), f"step {step}"
        assert int(torch.count_nonzero(best)) == 0, f"step {step}"


# ---------------------------------------------------------------------------
# seeded random shapes: every kernel variant's edges, many times over
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_random_lmhead_shapes_and_windows(dtype):
    rng = np.random.default_rng(900 if dtype == "bf16" else 901)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for case in range(24):
        m = int(rng.choice([1, 2, 7, 16, 17, 33, 64, 65, 129, 256, 257, 300, 513]))
        n = int(rng.integers(1, 1400))
        k = int(rng.choice([1, 8, 24, 40, 64, 72, 100, 128, 200, 264, 520]))
        col = int(rng.integers(0, 20)) * (8 if rng.random() < 0.7 else 1)
        ld = col + n + int(rng.integers(0, 24))
        X = wl.hidden_states(1000 + case, m, k, dtype)
        W = wl.table_rows(1100 + case, n, k, dtype, 0, n, std=0.5)
        logits = torch.full((m, ld), -1536.0, dtype=tdt, device=dev())
        vpe.vpe_lmhead(to_dev(X), to_dev(W), logits, col_offset=col)
        got = to_host(logits)
        what = f"{dtype} case {case}: m={m} n={n} k={k} ld={ld} col={col}"
        assert_logits_close(got[:, col:col + n], oracle.lmhead_f64(X, W, nthreads=oracle_threads()),
                            what)
        g = as_f64(got)
        assert np.all(g[:, :col] == -1536.0) and np.all(g[:, col + n:] == -1536.0), what
        if dtype == "bf16":
            # the greedy pick agrees with the stored logits
            val, tok = _pick(to_dev(X), [to_dev(W)], [col])
            assert np.array_equal(tok - col, np.argmax(g[:, col:col + n], axis=1)), what
            assert np.array_equal(val, g[:, col:col + n].max(axis=1)), what


def test_random_prefill_and_lookups():
    rng = np.random.default_rng(902)
    for case in range(16):
        dtype = "bf16" if case % 2 == 0 else "f32"
        seqs = int(rng.integers(1, 400))
        dim = int(rng.choice([8, 16, 24, 64, 96, 136]))
        rows = int(rng.integers(1, 900))
        cu = wl.cu_seqlens_ragged(1200 + case, seqs, 1, 30)
        H = wl.hidden_states(1300 + case, int(cu[-1]), dim, dtype)
        W = wl.table_rows(1400 + case, rows, dim, dtype, 0, rows, std=0.5)
        what = f"case {case}: {dtype} seqs={seqs} dim={dim} rows={rows}"
        H_d, cu_d, W_d = to_dev(H), to_dev(cu), to_dev(W)
        got = to_host(vpe.vpe_lmhead_prefill(H_d, cu_d, W_d))
        sel = oracle.last_token_select(H, cu)
        assert_logits_close(got, oracle.lmhead_f64(sel, W, nthreads=oracle_threads()), what)
        assert to_host(vpe.vpe_last_token_select(H_d, cu_d)).tobytes() == sel.tobytes(), what
        # lookups over the same table as a vocabulary, ids spilling past both ends
        vocab_start = int(rng.integers(0, 5000))
        ids = rng.integers(vocab_start - 50, vocab_start + rows + 50, size=int(rng.integers(1, 3000)))
        ids = ids.astype(np.int64 if case % 3 == 0 else np.int32)
        got = to_host(vpe.vpe_embed(to_dev(ids), W_d, vocab_start))
        assert got.tobytes() == oracle.embed(ids, W, vocab_start).tobytes(), what
        parts = [got, oracle.embed(ids, W, vocab_start + 1)]
        tot = to_host(vpe.vpe_sum_partials([to_dev(p) for p in parts]))
        assert tot.tobytes() == oracle.sum_partials(parts).tobytes(), what
