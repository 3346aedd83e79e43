"""GPU: spec_verify_sample_noalloc (its workspace is a fixed device array held
by the library) against spec_verify_sample with a caller workspace, on the
same inputs: tokens, accept counts and p_k(d_k) bit for bit, over calls in a
row whose shapes shrink and grow again, so every call sees the scratch the
previous one left behind.  The small case is also checked against the oracle."""
import numpy as np
import pytest
import torch

import synth
from tests.gpu_util import DEV, check_sample_sequence, dev
from tests.test_gpu_verify import _random_case

pytestmark = pytest.mark.gpu


def _compare(gpu, logits, q, d, u, T):
    B, K1, V = logits.shape
    K = K1 - 1
    z, qd, dd, ud = dev(logits), dev(q), dev(d), dev(u)
    ws = torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
    o1, a1, p1 = gpu.spec_verify_sample(z, qd, dd, ud, T, want_draft_target_prob=True,
                                        workspace=ws)
    o2 = torch.full((B, K + 1), -7, dtype=torch.int32, device=DEV)
    a2 = torch.full((B,), -7, dtype=torch.int32, device=DEV)
    p2 = torch.full((B, K), float("nan"), dtype=torch.float32, device=DEV)
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    gpu.spec_verify_sample_noalloc(z, qd, dd, ud, T, o2, a2, p2, device_error=err)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(a1, a2)
    assert torch.equal(p1.view(torch.int32), p2.view(torch.int32))
    assert int(err.item()) == 0
    assert int(ws.count_nonzero().item()) == 0
    return o2.cpu().numpy(), a2.cpu().numpy(), p2.cpu().numpy()


def test_noalloc_equals_sample_on_calls_in_a_row(gpu):
    assert gpu.noalloc_scratch_bytes() == 8 << 20
    rng = np.random.default_rng(4242)
    big = _random_case(rng, 48, 7, 50000, "bf16", T=0.8)         # several CDF tiles per row
    print("noalloc: B=48 K=7 V=50000 bf16", flush=True)
    first = _compare(gpu, *big, 0.8)
    # a smaller call: the mid-size verify (B=8, K=5, V=32000 fp32)
    vi = synth.make_verify_inputs(synth.verify_config(2))
    print("noalloc: B=8 K=5 V=32000 f32", flush=True)
    out, acc, _ = _compare(gpu, vi.logits, vi.draft_probs, vi.draft_tokens, vi.uniforms,
                           vi.temperature)
    for b in range(vi.spec.B):
        check_sample_sequence(vi.logits_f64(b), vi.draft_probs[b], vi.draft_tokens[b],
                              vi.uniforms[b], vi.temperature, out[b], acc[b])
    # smaller still, with a ragged vocabulary (element loads), then the first again
    tiny = _random_case(rng, 3, 4, 1001, "bf16", T=1.3)
    print("noalloc: B=3 K=4 V=1001 bf16", flush=True)
    _compare(gpu, *tiny, 1.3)
    print("noalloc: B=48 K=7 V=50000 bf16 again", flush=True)
    again = _compare(gpu, *big, 0.8)
    for x, y in zip(first, again):
        assert np.array_equal(x.view(np.int32), y.view(np.int32))
