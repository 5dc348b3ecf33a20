"""The allocation-free log-sum-exp (vpe_lmhead_logsumexp_noalloc), through the
C ABI, against the entry point that takes a workspace: both run the same
kernels, so logits and values must be equal bit for bit.  Calls follow each
other on one GPU, each smaller than the one before, so every call after the
first runs over what the previous one left in the library's static array.
A call that needs more than the array holds is refused before anything runs.
"""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a HIP GPU"),
]

import workloads as wl  # noqa: E402
import vocab_sharded_embedding_amd as vpe  # noqa: E402
from _gpu import dev, to_dev, to_host  # noqa: E402

# (dtype, M, shard rows, K, store logits): largest first, so each call lands on
# pairs an earlier, larger call wrote
CALLS = [
    ("bf16", 1024, 75968, 1024, True),   # X-in-registers tiles, 238 W tiles
    ("bf16", 256, 75968, 1024, False),   # 320 x 256 tiles, no logits stored
    ("bf16", 40, 3000, 72, True),        # decode-size tiles
    ("f32", 17, 1000, 64, True),         # fp32 tiles
]


def _inputs(i, dtype, m, n, k):
    X = wl.hidden_states(500 + i, m, k, dtype)
    W = wl.table_rows(510 + i, n, k, dtype, 0, n, std=0.5)
    return to_dev(X), to_dev(W)


def test_noalloc_equals_workspace_entry_point_on_consecutive_calls():
    for rep in range(2):
        for i, (dtype, m, n, k, store) in enumerate(CALLS):
            print(f"noalloc call {rep}.{i}: {dtype} M={m} R={n} K={k} logits={store}", flush=True)
            x_d, w_d = _inputs(i, dtype, m, n, k)
            lg_a, lse_a = vpe.vpe_lmhead_logsumexp(x_d, w_d, store_logits=store)
            lse_b = torch.full((m,), float("nan"), dtype=torch.float32, device=dev())
            lg_b = torch.full_like(lg_a, float("nan")) if store else None
            vpe.vpe_lmhead_logsumexp_noalloc(x_d, w_d, lse_b, logits=lg_b)
            torch.cuda.synchronize()
            assert np.all(np.isfinite(to_host(lse_b)))
            assert to_host(lse_a).tobytes() == to_host(lse_b).tobytes(), (rep, i)
            if store:
                assert to_host(lg_a).tobytes() == to_host(lg_b).tobytes(), (rep, i)


def test_noalloc_refuses_a_call_past_the_array():
    # 2^21 rows over a 400-row shard take the X-in-registers kernel's 320-row
    # tiles: 2 tiles x 2^21 rows x 8 bytes = 32 MiB > 16 MiB
    m, n, k = 1 << 21, 400, 8
    assert 2 * m * 8 > vpe.VPE_NOALLOC_SCRATCH_BYTES
    x_d = torch.zeros((m, k), dtype=torch.bfloat16, device=dev())
    w_d = torch.zeros((n, k), dtype=torch.bfloat16, device=dev())
    lse = torch.full((m,), 7.0, dtype=torch.float32, device=dev())
    with pytest.raises(vpe.VpeError) as e:
        vpe.vpe_lmhead_logsumexp_noalloc(x_d, w_d, lse)
    assert e.value.status == vpe.VPE_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert bool((lse == 7.0).all())  # nothing ran
    # the same shard with half the rows fits exactly (16 MiB) and runs
    half = m // 2
    lse_h = torch.empty(half, dtype=torch.float32, device=dev())
    vpe.vpe_lmhead_logsumexp_noalloc(x_d[:half], w_d, lse_h)
    torch.cuda.synchronize()
    # all-zero logits: log(400 * e^0) = ln 400 for every row
    assert np.allclose(to_host(lse_h), np.log(400.0), rtol=0, atol=1e-5)
