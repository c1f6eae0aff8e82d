"""Shared helpers for the GPU parity tests (test infrastructure)."""
from __future__ import annotations

import functools
import sys

import numpy as np

import synth
from oracle import reference as ref


def torch():
    import torch as _t

    return _t


def dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def say(*a):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[gpu-case]", *a, flush=True)
    sys.stdout.flush()


def assert_within(y_gpu, y_ref, A, what):
    y = np.asarray(y_gpu).astype(np.float64)
    ok = ref.within_tolerance(y, y_ref, A)
    if not ok.all():
        idx = np.argwhere(~ok)[:5]
        detail = [(tuple(i), float(y[tuple(i)]), float(y_ref[tuple(i)]), float(A[tuple(i)])) for i in idx]
        raise AssertionError(f"{what}: {int((~ok).sum())} of {ok.size} outside tolerance; first {detail}; "
                             f"worst ratio {ref.worst_ratio(y, y_ref, A):.3g}")


def sample_rows(N, n_random=24, seed=0):
    rng = np.random.default_rng(seed + N)
    fixed = [0, 1, 15, 16, 17, 31, 63, 64, N // 2, N - 17, N - 2, N - 1]
    rows = sorted({r for r in fixed if 0 <= r < N} | set(rng.integers(0, N, n_random).tolist()))
    return np.array(rows, dtype=np.int64)


@functools.lru_cache(maxsize=1)
def uniform_weights(seed, N, K, bits):
    """Host case (codes/scales/zeros + x for up to 16 rows) and its device upload."""
    import gemm_unpack_bit_amd as q

    c = synth.uniform_case(seed, 16, N, K, bits)
    wq = q.pack(dev(c["codes"]), bits)
    zq = q.pack_zeros(dev(c["zeros"]), bits)
    s = dev(c["scales"])
    return c, wq, s, zq
