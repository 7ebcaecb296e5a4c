"""kda_prefill_noalloc (the workspace-free prefill for callers that cannot allocate) against
kda_prefill with a caller-provided workspace, through the C ABI: two calls in a row on the
segment-parallel path, the second with a smaller input, must give byte-identical outputs,
final states and rings (the same kernels run on the same plan; only the workspace's
location differs).  A problem with enough (sequence, head) units for the whole-sequence
path, which needs no scratch, goes through the same entry point."""
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _run(prob, noalloc):
    import gated_delta_rule_05_amd as kda
    layer = kda.Layer(**prob["layer"])
    res = kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"], prob["gate"],
                      prob["cu_seqlens"].to(DEV), prob["cu_seqlens"], state_in=prob.get("state_in"),
                      ring_in=prob.get("ring_in"), noalloc=noalloc)
    torch.cuda.synchronize()
    return res


def _split_bytes(prob):
    import gated_delta_rule_05_amd as kda
    return kda.prefill_workspace_bytes(kda.Layer(**prob["layer"]), torch.bfloat16, prob["cu_seqlens"])


def test_noalloc_matches_prefill_two_calls():
    import gated_delta_rule_05_amd as kda
    big = synthetic.make_prefill([2048], H=8, io="bf16", seed=401, device=DEV, init_state=True,
                                 init_ring=True)
    small = synthetic.make_prefill([700, 300], H=2, io="bf16", seed=402, device=DEV,
                                   init_state=True, init_ring=True)
    assert 0 < _split_bytes(small) < _split_bytes(big) <= kda.NOALLOC_SCRATCH_BYTES
    for prob in (big, small):
        ref = _run(prob, False)
        got = _run(prob, True)
        for name, r, g in zip(("out", "state", "ring"), ref, got):
            assert torch.equal(r, g), name


def test_noalloc_whole_sequence_path():
    prob = synthetic.make_prefill([100, 37], H=48, io="bf16", seed=403, device=DEV,
                                  init_state=True, init_ring=True)
    assert _split_bytes(prob) == 0
    ref = _run(prob, False)
    got = _run(prob, True)
    for name, r, g in zip(("out", "state", "ring"), ref, got):
        assert torch.equal(r, g), name
