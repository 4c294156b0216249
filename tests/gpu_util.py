"""Helpers for the GPU tests: host <-> device copies of bf16 bit patterns and
payload words, block-wise downloads for the full-size checks, and a thread
pool that runs an oracle function over slices of a block.  No arithmetic of
the method lives here."""
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

DEV = torch.device("cuda:0")


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says where."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def up16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def down16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def up64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int64)).to(DEV)


def down64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().numpy().view(np.uint64)


def empty16(n: int) -> torch.Tensor:
    return torch.empty(n, dtype=torch.int16, device=DEV)


def new_err() -> torch.Tensor:
    import tensor_all_reduce_amd as tar
    e = torch.empty(2, dtype=torch.int64, device=DEV)
    tar.ar_err_init(e)
    return e


def err_host(e: torch.Tensor):
    v = down64(e)
    return int(v[0]), int(v[1])


def bits16(t: torch.Tensor) -> torch.Tensor:
    """View a bf16/int16 tensor as int16 bit patterns (no conversion)."""
    return t.view(torch.int16) if t.dtype != torch.int16 else t


def sample_indices(n: int, k: int, seed: int) -> np.ndarray:
    g = np.random.default_rng([seed, n])
    idx = np.concatenate([np.arange(min(n, 4096)), np.arange(max(0, n - 4096), n),
                          g.integers(0, n, size=k)])
    return np.unique(idx)


def gather_ranks(ins, idx: np.ndarray):
    """Copy element idx of every rank buffer to the host (uint16)."""
    ti = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    return [down16(bits16(x)[ti]) for x in ins]


def gather(t: torch.Tensor, idx: np.ndarray) -> np.ndarray:
    ti = torch.from_numpy(idx.astype(np.int64)).to(DEV)
    return down16(bits16(t)[ti])


def blocks(n: int, step: int):
    """[a, b) ranges of at most `step` covering [0, n)."""
    for a in range(0, n, step):
        yield a, min(n, a + step)


def down16_range(t: torch.Tensor, a: int, b: int) -> np.ndarray:
    return down16(bits16(t)[a:b])


def down64_range(t: torch.Tensor, a: int, b: int) -> np.ndarray:
    return down64(t[a:b])


def host_threads() -> int:
    """Threads for the host-side oracle: the cores this process may use,
    at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


_POOL = None


def pmap_slices(fn, arrays, n: int, parts: int | None = None):
    """fn applied to aligned slices [a, b) of every array in `arrays` (each
    of length n), split over host threads; returns the list of results in
    slice order.  The oracle is a ctypes library, which releases the GIL."""
    global _POOL
    parts = parts or host_threads()
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=host_threads())
    step = -(-n // parts)
    step += (-step) % 8
    cuts = [(a, min(n, a + step)) for a in range(0, n, step)]
    futs = [_POOL.submit(fn, [x[a:b] for x in arrays]) for a, b in cuts]
    return [f.result() for f in futs]


def first_mismatch(got: np.ndarray, want: np.ndarray):
    """(count, first index) of elements where got != want; (0, None) if none."""
    bad = np.flatnonzero(got != want)
    return (int(bad.size), int(bad[0])) if bad.size else (0, None)
