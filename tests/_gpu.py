"""Helpers shared by the GPU tests: moving seeded numpy inputs to the device
and reading results back as the same host representation the oracle uses
(float32 arrays, or uint16 bf16 bit patterns)."""
import os

import numpy as np
import torch


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(dev()).view(torch.bfloat16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bf16 as uint16 bits)."""
    t = t.detach().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def as_f64(a: np.ndarray) -> np.ndarray:
    """Host values of a result, widened exactly to float64."""
    if a.dtype == np.uint16:
        return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def oracle_threads() -> int:
    # a GPU host may grant a process a 16-core share whatever its affinity mask says
    return max(1, min(16, len(os.sched_getaffinity(0))))


def assert_logits_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    """|got - ref| <= 1e-2 + 1e-2 |ref| element by element (ref in fp64)."""
    g = as_f64(got)
    err = np.abs(g - ref)
    bound = 1e-2 + 1e-2 * np.abs(ref)
    bad = ~(err <= bound)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} logits out of tolerance; first at "
            f"{idx.tolist()}: got {g[tuple(idx[0])]}, ref {ref[tuple(idx[0])]}; "
            f"max err {float(err.max())}")
