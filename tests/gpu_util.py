"""Host <-> device plumbing and comparison helpers for the GPU parity tests."""
from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")

P_RTOL = 1e-5       # probabilities: relative tolerance
P_ATOL = 1e-30      # ... and an absolute floor for values far below fp32's range of interest
TIE_TOL = 1e-6      # decisions within this of their threshold may go either way


def dev(x: np.ndarray) -> torch.Tensor:
    if x.dtype == np.uint16:                     # bf16 bit patterns
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def check_sample_sequence(z64, q, d, u, T, out_row, a_gpu, pd_row=None, tol=TIE_TOL):
    """Compare one sequence's GPU result with the oracle.

    Returns (matches_canonical, n_flags).  Raises AssertionError when the GPU
    outcome is not among the oracle's acceptable outcomes, or when the output
    row is malformed, or when p_k(d_k) is off by more than the tolerance.
    """
    K = len(d)
    canon, allowed, flags = oracle.sample_outcomes(z64, q, d, u, T, tol=tol)
    a_gpu = int(a_gpu)
    assert 0 <= a_gpu <= K
    c_gpu = int(out_row[a_gpu])
    assert (a_gpu, c_gpu) in allowed, (a_gpu, c_gpu, canon, allowed)
    assert np.array_equal(out_row[:a_gpu], np.asarray(d[:a_gpu], np.int32))
    assert np.all(out_row[a_gpu + 1:] == -1)
    if pd_row is not None:
        want = np.array([oracle.target_distribution(z64[k], T)[int(d[k])] for k in range(K)])
        assert np.allclose(pd_row, want, rtol=P_RTOL, atol=P_ATOL), (pd_row, want)
    return (a_gpu, c_gpu) == canon, flags
