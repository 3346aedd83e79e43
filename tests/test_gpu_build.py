"""GPU parity: peagle_build_draft_batch against the oracle, bit for bit.

The P-EAGLE build workload (B=64, K=7, H=2880 bf16) at full size, plus K=1,
K=63, odd hidden sizes (element copy path), fp32 / fp16 hidden states, the
extreme accept counts, out-of-range accept counts and block tables (device
error bits), and an empty batch.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests.gpu_util import DEV, dev, host_bits
from tests.test_oracle_build import _case, check_invariants

pytestmark = pytest.mark.gpu


def _run(sv, case, hidden_dtype=torch.bfloat16, device_error=None):
    hid = case["target_hidden"]
    hs = case["h_shared"]
    if hidden_dtype == torch.float32:
        th = torch.from_numpy(hid.view(np.float32)).to(DEV)
        hh = torch.from_numpy(hs.view(np.float32)).to(DEV)
    else:
        th = torch.from_numpy(hid.view(np.int16)).to(DEV).view(hidden_dtype)
        hh = torch.from_numpy(hs.view(np.int16)).to(DEV).view(hidden_dtype)
    res = sv.peagle_build_draft_batch(dev(case["out_tokens"]), dev(case["num_accepted"]),
                                      dev(case["draft_tokens"]), dev(case["start_pos"]),
                                      dev(case["block_table"]), case["block_size"], th, hh,
                                      case["mask_token_id"], device_error=device_error)
    torch.cuda.synchronize()
    out = {k: (host_bits(v) if k == "hidden" else v.cpu().numpy()) for k, v in res.items()}
    if hidden_dtype == torch.float32:
        out["hidden"] = np.ascontiguousarray(out["hidden"]).view(np.uint32)
    return out


def _compare(got, want):
    for key in ("input_ids", "positions", "slot_mapping", "sample_rows"):
        assert np.array_equal(got[key], want[key]), key
    assert got["hidden"].tobytes() == np.ascontiguousarray(want["hidden"]).tobytes()


def test_build_workload(gpu):
    bi = synth.make_build_inputs(synth.build_config(3))
    case = dict(out_tokens=bi.out_tokens, num_accepted=bi.num_accepted,
                draft_tokens=bi.draft_tokens, start_pos=bi.start_pos,
                block_table=bi.block_table, block_size=bi.spec.block_size,
                target_hidden=bi.target_hidden, h_shared=bi.h_shared,
                mask_token_id=bi.mask_token_id)
    got = _run(gpu, case)
    want = oracle.build_draft_batch(**case)
    _compare(got, want)
    check_invariants(got, case, bi.spec.K)


@pytest.mark.parametrize("B,K,H,bs,seed", [(3, 1, 8, 16, 0), (5, 63, 64, 16, 1), (7, 7, 2047, 4, 2),
                                           (2, 3, 1, 1, 3), (130, 5, 2880, 16, 4)])
def test_build_shapes(gpu, B, K, H, bs, seed):
    rng = np.random.default_rng(seed)
    case = _case(rng, B, K, H, bs)
    _compare(_run(gpu, case), oracle.build_draft_batch(**case))


@pytest.mark.parametrize("dtype", [torch.float32, torch.float16])
def test_build_hidden_dtypes(gpu, dtype):
    rng = np.random.default_rng(9)
    K, H = 4, 100
    # fp32: each element is a pair of the case's 16-bit words (same bytes)
    case = _case(rng, 6, K, 2 * H if dtype == torch.float32 else H, 16)
    got = _run(gpu, case, hidden_dtype=dtype)
    want = oracle.build_draft_batch(**case)
    for key in ("input_ids", "positions", "slot_mapping", "sample_rows"):
        assert np.array_equal(got[key], want[key]), key
    assert got["hidden"].tobytes() == np.ascontiguousarray(want["hidden"]).tobytes()


@pytest.mark.parametrize("a", [0, 7])
def test_build_extreme_accepts(gpu, a):
    rng = np.random.default_rng(20 + a)
    case = _case(rng, 9, 7, 256, 16, a=a)
    _compare(_run(gpu, case), oracle.build_draft_batch(**case))


def test_build_bad_data_flags(gpu):
    rng = np.random.default_rng(30)
    K = 3
    case = _case(rng, 4, K, 16, 4)
    case["num_accepted"] = case["num_accepted"].copy()
    case["num_accepted"][1] = 9                       # > K: clamped to K
    case["out_tokens"][1, K] = 77
    bt = case["block_table"].copy()
    bt[2, :] = -1                                     # sequence 2 has no pages
    case["block_table"] = bt
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    got = _run(gpu, case, device_error=err)
    flags = int(err.item())
    assert flags & gpu.DEVERR_ACCEPT_COUNT and flags & gpu.DEVERR_BLOCK_TABLE
    seg1 = slice(2 * K, 4 * K)
    assert np.sum(got["slot_mapping"][seg1] == -1) == 0          # a clamped to K: nothing rejected
    assert got["input_ids"][2 * K + K] == 77
    assert np.all(got["slot_mapping"][4 * K:6 * K] == -1)        # no pages: every slot -1


def test_build_empty(gpu):
    e32 = torch.zeros((0, 4), dtype=torch.int32, device=DEV)
    res = gpu.peagle_build_draft_batch(torch.zeros((0, 5), dtype=torch.int32, device=DEV),
                                       torch.zeros(0, dtype=torch.int32, device=DEV), e32,
                                       torch.zeros(0, dtype=torch.int64, device=DEV),
                                       torch.zeros((0, 1), dtype=torch.int32, device=DEV), 16,
                                       torch.zeros((0, 8), dtype=torch.bfloat16, device=DEV),
                                       torch.zeros(8, dtype=torch.bfloat16, device=DEV), 5)
    assert res["input_ids"].shape == (0,)
