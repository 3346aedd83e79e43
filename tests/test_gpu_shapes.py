"""GPU parity over a seeded sweep of shapes around the kernels' boundaries.

Vocabularies just below, at and just above multiples of the 2048-element CDF
tile (and so of the 8-element octet), with batch sizes and draft counts drawn
so that the row kernel's split count and the draw's chunk count vary from
case to case; both logit dtypes.  Each case runs the greedy, the sampled and
the mixed verify against the oracle with the checks of the single-shape
tests (exact tokens and counts; near ties within 1e-6 may go either way;
p_k(d_k) within 1e-5).
"""
from types import SimpleNamespace

import numpy as np
import pytest

from tests.test_gpu_mixed import _mixed_parity
from tests.test_gpu_verify import _greedy_parity, _random_case, _sample_parity

pytestmark = pytest.mark.gpu

VOCABS = [2047, 2048, 2049, 4095, 4096, 4097, 6143, 8191, 10241, 16383, 16385, 30721, 65535,
          65537]


def _case(i):
    rng = np.random.default_rng(7000 + i)
    V = VOCABS[i]
    B = int(rng.integers(1, 24))
    K = int(rng.integers(1, 10))
    dtype = ("f32", "bf16")[i % 2]
    T = float(rng.choice([0.6, 0.9, 1.2]))
    return rng, B, K, V, dtype, T


@pytest.mark.parametrize("i", range(len(VOCABS)))
def test_boundary_shapes(gpu, i):
    rng, B, K, V, dtype, T = _case(i)
    logits, q, d, u = _random_case(rng, B, K, V, dtype, T=T)
    _greedy_parity(gpu, logits, dtype, d)
    _sample_parity(gpu, logits, dtype, q, d, u, T)
    temps = rng.choice(np.array([0.0, 0.5, 0.8, 1.1], dtype=np.float32), size=B)
    vi = SimpleNamespace(logits=logits, draft_probs=q, draft_tokens=d, uniforms=u,
                         spec=SimpleNamespace(B=B, dtype=dtype))
    _mixed_parity(gpu, vi, temps)
