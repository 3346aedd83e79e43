"""GPU: calls on two streams at once, each with its own workspace.

The library keeps no device state between calls except the no-alloc entry
point's fixed array (not used here): a sampled verify + P-EAGLE build on one
stream and a mixed verify, a tree verify and drafter sampling on another,
enqueued alternately without waiting, must give exactly the results of the
same calls made one after another on one stream.
"""
import numpy as np
import pytest
import torch

import synth
from synth import TREE_CONFIGS, make_tree_inputs
from tests.gpu_util import DEV, dev
from tests.test_gpu_graph import _build_inputs, _outputs

pytestmark = pytest.mark.gpu


def _work(sv, vi, ti, temps, b, outs, ws, ws_t, dsrc):
    """The calls, each on the current stream; returns the output tensors."""
    z, q, d, u = vi
    o = outs
    r = [sv.spec_verify_sample(z, q, d, u, 0.9, out_tokens=o["tok"], out_num_accepted=o["acc"],
                               workspace=ws[0])]
    sv.peagle_build_draft_batch(o["tok"], o["acc"], d, b["start_pos"], b["block_table"],
                                b["block_size"], b["target_hidden"], b["h_shared"],
                                b["mask_token_id"], outputs=o["build"])
    r.append(sv.spec_verify_mixed(z, q, d, u, temps, workspace=ws[1]))
    r.append(sv.spec_verify_tree(ti[0], ti[1], ti[2], 0.8, draft_probs=ti[3], uniforms=ti[4],
                                 workspace=ws_t))
    r.append(sv.spec_draft_sample(dsrc, 3, 0.7, uniforms=ti[5]))
    return r


def test_two_streams(gpu):
    rng = np.random.default_rng(404)
    vi = synth.make_verify_inputs(synth.verify_config(2))
    B, K, V = vi.spec.B, vi.spec.K, vi.spec.V
    args = (dev(vi.logits), dev(vi.draft_probs), dev(vi.draft_tokens), dev(vi.uniforms))
    temps = dev(synth.make_temperatures(B, 404))
    t = make_tree_inputs(TREE_CONFIGS["tree-mid"])
    Bt, N, Vt = t.spec.B, t.spec.N, t.spec.V
    ud = rng.random((Bt * 2, 3), dtype=np.float32)
    tree = (dev(t.logits), dev(t.parents), dev(t.tokens), dev(t.draft_probs), dev(t.uniforms),
            dev(ud))
    dsrc = dev(t.logits.reshape(-1, Vt)[: Bt * 2 * 3])
    b = _build_inputs(B, K, V)
    b.pop("host")

    def fresh():
        ws = [torch.zeros(gpu.spec_verify_workspace_bytes(B, K, V), dtype=torch.uint8, device=DEV)
              for _ in range(2)]
        ws_t = torch.zeros(gpu.spec_verify_workspace_bytes(Bt, N, Vt), dtype=torch.uint8,
                           device=DEV)
        return _outputs(B, K, V, 512), ws, ws_t

    # reference: one stream, one call after another
    o_ref, ws_r, wst_r = fresh()
    ref = _work(gpu, args, tree, temps, b, o_ref, ws_r, wst_r, dsrc)
    torch.cuda.synchronize()
    # two streams, two independent sets of buffers, calls interleaved
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    sets = [fresh(), fresh()]
    res = [None, None]
    for rep in range(3):
        for i, st in enumerate((s1, s2)):
            with torch.cuda.stream(st):
                o, ws, wst = sets[i]
                res[i] = _work(gpu, args, tree, temps, b, o, ws, wst, dsrc)
        torch.cuda.synchronize()
        for i in range(2):
            o = sets[i][0]
            assert torch.equal(o["tok"], o_ref["tok"]) and torch.equal(o["acc"], o_ref["acc"])
            for k in o["build"]:
                assert torch.equal(o["build"][k], o_ref["build"][k]), k
            for got, want in zip(res[i][1:], ref[1:]):
                for x, y in zip(got, want):
                    if x is not None:
                        assert torch.equal(x, y)
            for w in sets[i][1] + [sets[i][2]]:
                assert int(w.count_nonzero().item()) == 0
