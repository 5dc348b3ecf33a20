"""GPU parity of the log-sum-exp of the logits rows (per shard, and combined
over shards) against the CPU oracle, through the C ABI.

Two kinds of input:
  - small-integer X and W (entries -1, 0, 1): every logit is an integer of
    magnitude <= K, exact in fp32 accumulation and in bf16, so the GPU and the
    oracle take the log-sum-exp of the same numbers and differ only by fp32
    exp / sum / log rounding (well under 1e-4 at these sizes); one W tile left
    out of a row would move the value by about log(1 - 1/tiles), far more.
    The shapes pick each LM-head kernel the workloads use.
  - the workloads' own normal inputs: the oracle's fp64 logits are the
    reference, and the GPU's value comes from logits rounded to the logits
    dtype, so the bound is the rounding's: |d lse| <= max_j |d z_j| <=
    2^-9 max_j |z_j| per row (taken as 2^-8 max|z| + 1e-4); and the value must
    be the log-sum-exp of the logits the same call stored (a property of the
    output, checked in fp64 to 1e-5).
"""
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
from _gpu import as_f64, dev, oracle_threads, to_dev, to_host  # noqa: E402

TIGHT = 1e-4  # integer logits: fp32 exp / sum / log rounding only


def _int_inputs(seed, m, n, k, dtype):
    rng = np.random.default_rng(seed)
    X = rng.integers(-1, 2, size=(m, k)).astype(np.float32)
    W = rng.integers(-1, 2, size=(n, k)).astype(np.float32)
    if dtype == "bf16":
        X, W = wl.f32_to_bf16_bits(X), wl.f32_to_bf16_bits(W)
    return X, W


def _lse(x_h, w_h, store=True, col_offset=0, ld=None):
    x_d, w_d = to_dev(x_h), to_dev(w_h)
    logits = None
    if store:
        tdt = x_d.dtype
        logits = torch.empty((x_h.shape[0], ld or w_h.shape[0] + col_offset), dtype=tdt,
                             device=dev())
    lg, lse = vpe.vpe_lmhead_logsumexp(x_d, w_d, logits=logits, col_offset=col_offset,
                                       store_logits=store)
    torch.cuda.synchronize()
    return (to_host(lg) if lg is not None else None), to_host(lse).astype(np.float64)


# shapes that take each LM-head kernel: decode tiles (M <= 16, 32, 64 on short
# and long shards), 320 x 128 and 256 x 128 (M <= 128), the two-stage 320 x 256
# (M <= 256), the X-in-registers kernel (M > 256); ragged N and M tails
INT_SHAPES = [
    (1, 1, 8), (3, 5, 40), (16, 777, 64), (17, 1000, 64), (32, 4100, 32), (40, 300, 64),
    (8, 75968, 64), (32, 151936, 64), (64, 75968, 64), (64, 1025, 16), (100, 2000, 64),
    (128, 75968, 64), (129, 3000, 40), (256, 75968, 64), (200, 640, 64), (300, 2100, 64),
    (1024, 75968, 64), (4096, 37984, 64), (257, 131, 40),
    # K not a multiple of 8: operands staged element-wise through registers
    (40, 300, 37), (300, 700, 45),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("m,n,k", INT_SHAPES)
def test_logsumexp_exact_on_integer_logits(dtype, m, n, k):
    X, W = _int_inputs(300 + m + n, m, n, k, dtype)
    logits, lse = _lse(X, W)
    ref_logits = oracle.lmhead_f64(X, W, nthreads=oracle_threads())
    assert np.array_equal(as_f64(logits), ref_logits), "integer logits must be exact"
    ref = oracle.logsumexp_rows(ref_logits)
    err = np.abs(lse - ref)
    assert np.all(err <= TIGHT * np.maximum(1.0, np.abs(ref))), (
        f"{dtype} {m}x{n}x{k}: max err {err.max()} at row {int(err.argmax())}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_logsumexp_without_logits_equals_with_logits(dtype):
    for m, n, k in [(8, 75968, 64), (40, 3000, 72), (256, 75968, 64), (300, 2100, 64)]:
        X, W = _int_inputs(400 + m, m, n, k, dtype)
        _, with_logits = _lse(X, W, store=True)
        _, alone = _lse(X, W, store=False)
        assert with_logits.tobytes() == alone.tobytes(), (dtype, m, n, k)


def test_logsumexp_logits_written_at_their_columns_only():
    m, n, k, ld, col = 40, 1000, 64, 1507, 251
    X, W = _int_inputs(410, m, n, k, "bf16")
    tdt = torch.bfloat16
    logits = torch.full((m, ld), -1536.0, dtype=tdt, device=dev())
    _, lse = vpe.vpe_lmhead_logsumexp(to_dev(X), to_dev(W), logits=logits, col_offset=col)
    got = as_f64(to_host(logits))
    ref = oracle.lmhead_f64(X, W)
    assert np.array_equal(got[:, col:col + n], ref)
    assert np.all(got[:, :col] == -1536.0) and np.all(got[:, col + n:] == -1536.0)
    assert np.all(np.abs(to_host(lse) - oracle.logsumexp_rows(ref)) <= TIGHT * 10)


@pytest.mark.parametrize("tp", [2, 3, 4])
def test_combined_shards_equal_the_full_row(tp):
    # each rank's value over its shard, combined in rank order, against the
    # oracle over the concatenated row
    m, R, k = 37, 1700, 64
    X, W = _int_inputs(420 + tp, m, R * tp, k, "bf16")
    x_d = to_dev(X)
    parts = []
    for r in range(tp):
        _, lse = vpe.vpe_lmhead_logsumexp(x_d, to_dev(W[r * R:(r + 1) * R]), store_logits=False)
        parts.append(lse)
    full = to_host(vpe.vpe_logsumexp_combine(parts)).astype(np.float64)
    ref = oracle.logsumexp_rows(oracle.lmhead_f64(X, W))
    assert np.all(np.abs(full - ref) <= TIGHT * np.maximum(1.0, np.abs(ref)))
    # the combine is in place-safe and order-fixed: same bits when run twice
    again = to_host(vpe.vpe_logsumexp_combine(parts, out=parts[0]))
    assert again.tobytes() == full.astype(np.float32).tobytes()


def test_combine_special_values():
    # a shard whose values are all -inf adds nothing; NaN propagates
    a = torch.tensor([0.0, 1.0, float("-inf"), 2.0, float("nan")], device=dev())
    b = torch.tensor([0.0, float("-inf"), float("-inf"), 2.0, 0.0], device=dev())
    got = to_host(vpe.vpe_logsumexp_combine([a, b])).astype(np.float64)
    assert abs(got[0] - np.log(2.0)) < 1e-6
    assert got[1] == np.float32(1.0)
    assert got[2] == -np.inf
    assert abs(got[3] - (2.0 + np.log(2.0))) < 1e-6
    assert np.isnan(got[4])


def test_logsumexp_nan_row():
    X, W = _int_inputs(430, 4, 500, 64, "f32")
    X[2, 5] = np.nan
    _, lse = _lse(X, W)
    assert np.isnan(lse[2]) and np.all(np.isfinite(lse[[0, 1, 3]]))


def test_logsumexp_workspace_too_small_is_refused():
    X, W = _int_inputs(440, 8, 1000, 64, "bf16")
    need = vpe.vpe_lmhead_logsumexp_workspace(8, 1000)
    assert need == 8 * 16 * 8
    small = torch.empty(need - 8, dtype=torch.uint8, device=dev())
    with pytest.raises(vpe.VpeError) as e:
        vpe.vpe_lmhead_logsumexp(to_dev(X), to_dev(W), workspace=small)
    assert e.value.status == vpe.VPE_ERR_WORKSPACE
    ok = torch.empty(need, dtype=torch.uint8, device=dev())
    _, lse = vpe.vpe_lmhead_logsumexp(to_dev(X), to_dev(W), workspace=ok)
    ref = oracle.logsumexp_rows(oracle.lmhead_f64(X, W))
    assert np.all(np.abs(to_host(lse) - ref) <= TIGHT * np.maximum(1, np.abs(ref)))


# ---------------------------------------------------------------------------
# the workloads' shapes and normal inputs
# ---------------------------------------------------------------------------
def _workload_rows(w):
    hidden = wl.workload_hidden(w)
    if w.seqs:
        cu = wl.workload_cu_seqlens(w)
        return hidden[cu[1:].astype(np.int64) - 1]
    return hidden


@pytest.mark.parametrize("name", ["qwen3_0p6b_tp2_rank0", "qwen3_0p6b_tp1_prefill",
                                  "qwen3_0p6b_tp2_all_ranks", "large_v151936_d4096_tp4_rank2"])
def test_logsumexp_workloads(name):
    w = wl.WORKLOADS[name]
    x_h = _workload_rows(w)
    print(f"logsumexp {name}: M={x_h.shape[0]} R={w.shard_rows} D={w.dim}", flush=True)
    x_d = to_dev(x_h)
    M = x_h.shape[0]
    ref_logits = np.zeros((M, w.shard_rows * len(w.ranks)), dtype=np.float64)
    parts, stored = [], []
    for i, r in enumerate(w.ranks):
        W = wl.shard_table(w, r)
        oracle.lmhead_f64(x_h, W, out=ref_logits, col_offset=i * w.shard_rows,
                          nthreads=oracle_threads())
        lg, lse = vpe.vpe_lmhead_logsumexp(x_d, to_dev(W))
        parts.append(lse)
        stored.append(as_f64(to_host(lg)))
        del W
    got = to_host(vpe.vpe_logsumexp_combine(parts)).astype(np.float64)
    ref = oracle.logsumexp_rows(ref_logits)
    bound = 2.0 ** -8 * np.abs(ref_logits).max(axis=1) + 1e-4
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{name}: max err {err.max()} (bound {bound.min()})"
    # the value is the log-sum-exp of the logits the calls stored
    from scipy.special import logsumexp
    own = logsumexp(np.concatenate(stored, axis=1), axis=1)
    assert np.all(np.abs(got - own) <= 1e-5 * np.maximum(1, np.abs(own))), name


def test_parallel_lmhead_layer_logsumexp():
    V, D, tp, m = 512, 64, 2, 9
    X, Wf = _int_inputs(450, m, V, D, "bf16")
    full_d = to_dev(Wf)
    logits = torch.empty((m, V), dtype=torch.bfloat16, device=dev())
    parts = []
    for r in range(tp):
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev())
        head.weight_loader(head.weight, full_d)
        _, lse = head.logsumexp(to_dev(X), logits=logits)
        parts.append(lse)
    ref_logits = oracle.lmhead_f64(X, Wf)
    assert np.array_equal(as_f64(to_host(logits)), ref_logits)
    got = to_host(vpe.ParallelLMHead.combine_logsumexp(parts)).astype(np.float64)
    ref = oracle.logsumexp_rows(ref_logits)
    assert np.all(np.abs(got - ref) <= TIGHT * np.maximum(1, np.abs(ref)))


# ---------------------------------------------------------------------------
# prefill: the last position of every packed sequence, select folded in
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("dtype,seqs,dim,rows,seq_len", [
    ("bf16", 32, 1024, 151936, 2048),  # the prefill workload's shape
    ("bf16", 17, 520, 3000, 700),      # decode-size tiles, K not a multiple of 64
    ("bf16", 64, 256, 2100, 40),       # 128-row decode tiles
    ("bf16", 200, 128, 1000, 9),       # 320 x 256 tiles
    ("bf16", 300, 64, 2100, 5),        # X in registers, gathered
    ("f32", 9, 64, 700, 30),
    ("f32", 70, 40, 300, 12),
])
def test_prefill_logsumexp_equals_select_then_logsumexp(dtype, seqs, dim, rows, seq_len):
    cu = wl.cu_seqlens_ragged(500 + seqs, seqs, max(1, seq_len // 2), seq_len)
    H = wl.hidden_states(501 + seqs, int(cu[-1]), dim, dtype)
    W = wl.table_rows(502 + seqs, rows, dim, dtype, 0, rows, std=0.5)
    print(f"prefill logsumexp {dtype} S={seqs} D={dim} R={rows} T={int(cu[-1])}", flush=True)
    H_d, cu_d, W_d = to_dev(H), to_dev(cu), to_dev(W)
    lg_f, lse_f = vpe.vpe_lmhead_prefill_logsumexp(H_d, cu_d, W_d)
    sel = vpe.vpe_last_token_select(H_d, cu_d)
    lg_p, lse_p = vpe.vpe_lmhead_logsumexp(sel, W_d)
    _, lse_alone = vpe.vpe_lmhead_prefill_logsumexp(H_d, cu_d, W_d, store_logits=False)
    torch.cuda.synchronize()
    assert to_host(lg_f).tobytes() == to_host(lg_p).tobytes()
    assert to_host(lse_f).tobytes() == to_host(lse_p).tobytes()
    assert to_host(lse_alone).tobytes() == to_host(lse_f).tobytes()
    from scipy.special import logsumexp
    own = logsumexp(as_f64(to_host(lg_f)), axis=1)
    got = to_host(lse_f).astype(np.float64)
    assert np.all(np.abs(got - own) <= 1e-5 * np.maximum(1, np.abs(own)))


def test_prefill_logsumexp_exact_on_integer_logits():
    seqs, dim, rows = 40, 64, 3000
    cu = wl.cu_seqlens_ragged(520, seqs, 1, 30)
    rng = np.random.default_rng(521)
    H = wl.f32_to_bf16_bits(rng.integers(-1, 2, size=(int(cu[-1]), dim)).astype(np.float32))
    W = wl.f32_to_bf16_bits(rng.integers(-1, 2, size=(rows, dim)).astype(np.float32))
    lg, lse = vpe.vpe_lmhead_prefill_logsumexp(to_dev(H), to_dev(cu), to_dev(W))
    ref_logits = oracle.lmhead_f64(oracle.last_token_select(H, cu), W)
    assert np.array_equal(as_f64(to_host(lg)), ref_logits)
    ref = oracle.logsumexp_rows(ref_logits)
    assert np.all(np.abs(to_host(lse) - ref) <= TIGHT * np.maximum(1, np.abs(ref)))


def test_prefill_logsumexp_out_of_range_sequence():
    # an empty first sequence and one ending past the tokens: zero logits, so
    # the value is log(shard rows)
    H = wl.hidden_states(530, 10, 64, "bf16")
    W = wl.table_rows(531, 50, 64, "bf16", 0, 50, std=0.5)
    cu = np.array([0, 0, 4, 10, 12], dtype=np.int32)
    lg, lse = vpe.vpe_lmhead_prefill_logsumexp(to_dev(H), to_dev(cu), to_dev(W))
    got, val = as_f64(to_host(lg)), to_host(lse).astype(np.float64)
    assert np.all(got[0] == 0) and np.all(got[3] == 0)
    assert abs(val[0] - np.log(50)) < 1e-5 and abs(val[3] - np.log(50)) < 1e-5
    ref = oracle.logsumexp_rows(oracle.lmhead_f64(H[[3, 9]], W))
    assert np.all(np.abs(val[1:3] - ref) <= 2.0 ** -8 * np.abs(got[1:3]).max(axis=1) + 1e-4)


def test_prefill_logsumexp_workspace_too_small_is_refused():
    cu = np.array([0, 3, 7], dtype=np.int32)
    H = wl.hidden_states(540, 7, 64, "bf16")
    W = wl.table_rows(541, 1000, 64, "bf16", 0, 1000)
    need = vpe.vpe_lmhead_logsumexp_workspace(2, 1000)
    small = torch.empty(need - 8, dtype=torch.uint8, device=dev())
    with pytest.raises(vpe.VpeError) as e:
        vpe.vpe_lmhead_prefill_logsumexp(to_dev(H), to_dev(cu), to_dev(W), workspace=small)
    assert e.value.status == vpe.VPE_ERR_WORKSPACE


def test_prefill_logsumexp_workload():
    w = wl.WORKLOADS["qwen3_0p6b_tp1_prefill"]
    hidden = wl.workload_hidden(w)
    cu = wl.workload_cu_seqlens(w)
    W = wl.shard_table(w, w.ranks[0])
    print(f"prefill logsumexp workload: S={w.seqs} R={w.shard_rows} D={w.dim}", flush=True)
    lg, lse = vpe.vpe_lmhead_prefill_logsumexp(to_dev(hidden), to_dev(cu), to_dev(W))
    ref_logits = oracle.lmhead_f64(oracle.last_token_select(hidden, cu), W,
                                   nthreads=oracle_threads())
    got = to_host(lse).astype(np.float64)
    ref = oracle.logsumexp_rows(ref_logits)
    bound = 2.0 ** -8 * np.abs(ref_logits).max(axis=1) + 1e-4
    assert np.all(np.abs(got - ref) <= bound)
    from scipy.special import logsumexp
    own = logsumexp(as_f64(to_host(lg)), axis=1)
    assert np.all(np.abs(got - own) <= 1e-5 * np.maximum(1, np.abs(own)))


def test_parallel_lmhead_layer_prefill_logsumexp():
    V, D, tp = 512, 64, 2
    cu = wl.cu_seqlens_ragged(550, 6, 1, 9)
    rng = np.random.default_rng(551)
    H = wl.f32_to_bf16_bits(rng.integers(-1, 2, size=(int(cu[-1]), D)).astype(np.float32))
    Wf = wl.f32_to_bf16_bits(rng.integers(-1, 2, size=(V, D)).astype(np.float32))
    full_d, H_d, cu_d = to_dev(Wf), to_dev(H), to_dev(cu)
    logits = torch.empty((6, V), dtype=torch.bfloat16, device=dev())
    parts = []
    for r in range(tp):
        head = vpe.ParallelLMHead(V, D, tp_size=tp, tp_rank=r, device=dev())
        head.weight_loader(head.weight, full_d)
        _, lse = head.logsumexp(H_d, logits=logits, cu_seqlens=cu_d)
        parts.append(lse)
    ref_logits = oracle.lmhead_f64(oracle.last_token_select(H, cu), Wf)
    assert np.array_equal(as_f64(to_host(logits)), ref_logits)
    got = to_host(vpe.ParallelLMHead.combine_logsumexp(parts)).astype(np.float64)
    ref = oracle.logsumexp_rows(ref_logits)
    assert np.all(np.abs(got - ref) <= TIGHT * np.maximum(1, np.abs(ref)))
