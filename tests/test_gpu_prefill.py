"""GPU parity of kda_prefill against the fp64 oracle (through the C ABI)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from kda_testutil import D, assert_close, check_all_units, head_layer, io_code, oracle_units, unit_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _kda():
    import gated_delta_rule_05_amd as kda
    return kda


def _prefill(prob, **kw):
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    res = kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"],
                      prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"],
                      state_in=prob.get("state_in"), ring_in=prob.get("ring_in"), **kw)
    torch.cuda.synchronize()
    return res


def _check(prob, res, units, label):
    out, state, ring = res
    bf16 = prob["q"].dtype == torch.bfloat16
    cu = prob["cu_seqlens"].tolist()
    H = prob["layer"]["num_heads"]
    Hd = H * D
    refs = oracle_units(prob, units)
    worst = 0.0
    for (n, h), (o_ref, s_ref, r_ref) in zip(units, refs):
        got = out[cu[n]:cu[n + 1], h * D:(h + 1) * D].float().cpu().numpy()
        if got.size:
            worst = max(worst, assert_close(got, o_ref, bf16, f"{label} out (n={n}, h={h})", stored_bf16=bf16))
        if state is not None:
            worst = max(worst, assert_close(state[n, h].cpu().numpy(), s_ref, bf16,
                                            f"{label} state (n={n}, h={h})"))
        if ring is not None:
            r = ring[n].cpu().numpy()
            got_r = np.stack([r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])
            assert np.array_equal(got_r.astype(np.float64), r_ref), f"{label} ring (n={n}, h={h})"
    print(f"{label}: worst error = {worst:.3f} x tolerance")
    return worst


def _all_units(prob):
    N = len(prob["cu_seqlens"]) - 1
    return [(n, h) for n in range(N) for h in range(prob["layer"]["num_heads"])]


def test_tiny_prefill_fp32():
    """1 sequence x 64 tokens, 2 heads, fp32 io, zero state and ring: max relative error
    below 1e-4."""
    prob = synthetic.make_workload("tiny_prefill_fp32", device=DEV)
    _check(prob, _prefill(prob), _all_units(prob), "tiny_prefill_fp32")


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_varlen_ragged_with_state_and_ring(io):
    """Several sequences of ragged lengths (chunk tails, sequences shorter than the conv
    window, an empty one), carried state and ring."""
    lens = [37, 1, 0, 16, 2, 70, 33]
    prob = synthetic.make_prefill(lens, H=3, io=io, seed=201, device=DEV, init_state=True,
                                  init_ring=True)
    _check(prob, _prefill(prob), _all_units(prob), f"varlen_{io}")


@pytest.mark.parametrize("softplus,low_rank", [(False, False), (True, False), (False, True), (True, True)])
def test_chunk_boundary_lengths(softplus, low_rank):
    """Sequence lengths on either side of one, two and three 16-token chunks, and just past
    the conv window: the pipelined kernel's first and last iterations (prefetch two chunks
    ahead, ragged last chunk with 1..15 live rows, the ring taken from the last chunk or
    from the history before it), with carried state and ring."""
    lens = [3, 4, 15, 16, 17, 18, 31, 32, 33, 47, 48, 49]
    prob = synthetic.make_prefill(lens, H=2, io="bf16", seed=211, device=DEV, init_state=True,
                                  init_ring=True, softplus_gate=softplus, low_rank_gate=low_rank)
    label = ("softplus" if softplus else "bounded") + ("_low_rank" if low_rank else "")
    _check(prob, _prefill(prob), _all_units(prob), f"chunk_boundaries_{label}")


def test_in_place_state_and_ring():
    """state_out may equal state_in and ring_out may equal ring_in."""
    prob = synthetic.make_prefill([40, 19], H=2, io="bf16", seed=202, device=DEV,
                                  init_state=True, init_ring=True)
    ref = _prefill(prob)
    st = prob["state_in"].clone()
    rg = prob["ring_in"].clone()
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    out, st2, rg2 = kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"],
                                prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"],
                                state_in=st, ring_in=rg, state_out=st, ring_out=rg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref[0]) and torch.equal(st, ref[1]) and torch.equal(rg, ref[2])


def test_no_final_state():
    prob = synthetic.make_prefill([50], H=2, io="bf16", seed=203, device=DEV)
    out, st, rg = _prefill(prob, final_state=False)
    assert st is None and rg is None
    ref = _prefill(prob)
    assert torch.equal(out, ref[0])


def test_deterministic():
    prob = synthetic.make_prefill([100, 60], H=4, io="bf16", seed=204, device=DEV,
                                  init_state=True, init_ring=True)
    a = _prefill(prob)
    b = _prefill(prob)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


@pytest.mark.parametrize("zval,bval", [(1e4, 0.0), (-1e4, -6.0)])
def test_extreme_gates(zval, bval):
    """z = +1e4: g at the lower bound on every channel (the e^40 reference bound inside a
    tile).  z = -1e4: g = 0 exactly with beta ~ 0.0025, so the initial state is carried
    across every chunk of a long sequence."""
    for io in ("f32", "bf16"):
        prob = synthetic.make_prefill([200, 67], H=2, io=io, seed=205, device=DEV,
                                      init_state=True, init_ring=True)
        prob["z"].fill_(zval)
        prob["beta"].fill_(bval)
        _check(prob, _prefill(prob), _all_units(prob), f"extreme_{zval}_{io}")


@pytest.mark.parametrize("gate_kind", [0, synthetic.GATE_SOFTPLUS])
def test_many_short_sequences(gate_kind):
    """600 packed sequences of 0..40 tokens (more than the 512 the launch orders longest
    first, so the grid takes them in index order), carried state and ring, bf16: every
    unit against the oracle, for both decay gates."""
    rng = np.random.default_rng(206)
    lens = [int(x) for x in rng.integers(0, 41, size=600)]
    prob = synthetic.make_prefill(lens, H=2, io="bf16", seed=206, device=DEV, init_state=True,
                                  init_ring=True, softplus_gate=gate_kind == synthetic.GATE_SOFTPLUS)
    _check(prob, _prefill(prob), _all_units(prob), f"many_short_{gate_kind}")


def test_prefill_t4096_h32():
    """1 sequence x 4096 tokens, 32 heads, bf16 io: every unit against the oracle.  With 32
    (sequence, head) units this runs the segment-parallel path (8 segments)."""
    prob = synthetic.make_workload("prefill_t4096_h32", device=DEV)
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    assert kda.prefill_workspace_bytes(layer, torch.bfloat16, prob["cu_seqlens"]) > 0
    out, state, ring = _prefill(prob)
    check_all_units(prob, out.cpu(), state.cpu(), _all_units(prob), "prefill_t4096_h32", batch=32,
                    ring=ring.cpu())


def _split_problem(seed):
    """Ragged sequences long enough to be cut into 256-token segments (and two that are
    not: an empty one and a 2-token one), carried state and ring, and a quarter of the
    channels at g = 0 exactly (z = -1e4), so that state crosses every segment boundary
    undecayed."""
    lens = [1000, 2, 0, 700, 300]
    prob = synthetic.make_prefill(lens, H=3, io="bf16", seed=seed, device=DEV, init_state=True,
                                  init_ring=True)
    z = prob["z"].view(sum(lens), 3, D)
    z[:, :, ::4] = -1e4
    return prob


def test_segment_parallel_path():
    """The segment-parallel path (Transfer pass, combine, Final pass) against the oracle on
    every unit, final states and rings included."""
    prob = _split_problem(206)
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    assert kda.prefill_workspace_bytes(layer, torch.bfloat16, prob["cu_seqlens"]) > 0
    _check(prob, _prefill(prob), _all_units(prob), "segment_parallel")
    _ring_exact(prob, _prefill(prob)[2])


def test_segment_parallel_in_place():
    """The segment-parallel path with state_out == state_in and ring_out == ring_in: the
    sequence's first segment reads its start state and ring in the same launch in which its
    last segment writes the final ones, so it reads the copies the Transfer pass keeps in
    the workspace.  Byte-identical to the run with separate output buffers."""
    prob = _split_problem(210)
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    assert kda.prefill_workspace_bytes(layer, torch.bfloat16, prob["cu_seqlens"]) > 0
    ref = _prefill(prob)
    st = prob["state_in"].clone()
    rg = prob["ring_in"].clone()
    out, st2, rg2 = kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"],
                                prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"],
                                state_in=st, ring_in=rg, state_out=st, ring_out=rg)
    torch.cuda.synchronize()
    assert st2.data_ptr() == st.data_ptr() and rg2.data_ptr() == rg.data_ptr()
    assert torch.equal(out, ref[0]) and torch.equal(st, ref[1]) and torch.equal(rg, ref[2])


def test_segment_parallel_eight_units():
    """Eight (sequence, head) units, a multiple of the eight XCDs, so the combine deals each
    unit's column blocks to one XCD; the two sequences have different segment counts (8
    and 4 segments of 256 tokens).  Every unit against the oracle."""
    prob = synthetic.make_prefill([2000, 900], H=4, io="bf16", seed=208, device=DEV,
                                  init_state=True, init_ring=True)
    z = prob["z"].view(2900, 4, D)
    z[:, :, ::4] = -1e4  # g = 0 on a quarter of the channels: state crosses every boundary
    kda = _kda()
    assert kda.prefill_workspace_bytes(kda.Layer(**prob["layer"]), torch.bfloat16, prob["cu_seqlens"]) > 0
    _check(prob, _prefill(prob), _all_units(prob), "segment_parallel_8_units")


@pytest.mark.parametrize("gate_kind", [0, synthetic.GATE_SOFTPLUS])
def test_single_head_long_sequence(gate_kind):
    """One head, one 3,000-token sequence: the segment-parallel path with a single unit
    (twelve 256-token segments, the last one short), carried state and ring, every output
    row and the final state against the oracle."""
    prob = synthetic.make_prefill([3000], H=1, io="bf16", seed=209, device=DEV, init_state=True,
                                  init_ring=True, softplus_gate=gate_kind == synthetic.GATE_SOFTPLUS)
    kda = _kda()
    assert kda.prefill_workspace_bytes(kda.Layer(**prob["layer"]), torch.bfloat16, prob["cu_seqlens"]) > 0
    _check(prob, _prefill(prob), _all_units(prob), f"single_head_{gate_kind}")


def test_segment_parallel_matches_whole_path():
    """Both paths meet the oracle; with the same inputs their outputs differ only by
    rounding (the segment path forms start states as M S + B)."""
    prob = _split_problem(207)
    split = _prefill(prob)
    whole = _prefill(prob, allow_split=False)
    _check(prob, whole, _all_units(prob), "whole_path")
    assert torch.equal(split[2], whole[2])  # rings: pure data movement
    d = (split[0].float() - whole[0].float()).abs().max().item()
    rms = whole[0].float().pow(2).mean().sqrt().item()
    assert d <= 0.05 * rms, (d, rms)


def test_prefill_2x8192_h96():
    """2 sequences x 8192 tokens, 96 heads, bf16 io, final states: every (sequence, head)
    unit's output rows, final state and ring against the oracle."""
    prob = synthetic.make_workload("prefill_2x8192_h96", device=DEV)
    out, state, ring = _prefill(prob)
    assert torch.isfinite(out.float()).all() and torch.isfinite(state).all()
    check_all_units(prob, out.cpu(), state.cpu(), _all_units(prob), "prefill_2x8192_h96",
                    ring=ring.cpu())
    _ring_exact(prob, ring)


def _ring_exact(prob, ring):
    cu = prob["cu_seqlens"].tolist()
    Hd = prob["layer"]["num_heads"] * D
    for n in range(len(cu) - 1):
        if cu[n + 1] - cu[n] < 3:
            continue
        for p, name in enumerate(("q", "k", "v")):
            exp = prob[name][cu[n + 1] - 3:cu[n + 1]].float().T
            assert torch.equal(ring[n, p * Hd:(p + 1) * Hd], exp), (n, name)


def test_varlen16_h64_then_decode():
    """16 packed sequences with lengths ~ U[512, 16384], 64 heads, nonzero initial state
    and ring; then 32 decode steps from the returned states and rings.  Every unit of both
    phases against the oracle: the prefill's output rows, final states and rings; then the
    decode outputs and final states against the oracle continued from its own prefill
    states and rings (nothing of the GPU's prefill result enters the reference)."""
    kda = _kda()
    w = synthetic.WORKLOADS["varlen16_h64"]
    prob = synthetic.make_workload("varlen16_h64", device=DEV)
    out, state, ring = _prefill(prob)
    N, H = len(w.seqlens), w.heads
    assert torch.isfinite(out.float()).all() and torch.isfinite(state).all()
    units = _all_units(prob)
    _, (s_ref, r_ref) = check_all_units(prob, out.cpu(), state.cpu(), units, "varlen16_h64",
                                        ring=ring.cpu(), keep_final=True)
    _ring_exact(prob, ring)
    # decode continuation: 32 steps from the returned states and rings
    g = synthetic.gen(w.seed + 1, DEV)
    steps = w.decode_after
    acts = synthetic.activations(N, H, w.io, g, DEV, lead=(steps,))
    layer = kda.Layer(**prob["layer"])
    st = state.clone()
    rg = ring.clone()
    outs = []
    for s in range(steps):
        outs.append(kda.decode_step(layer, acts["q"][s], acts["k"][s], acts["v"][s], acts["z"][s],
                                    acts["beta"][s], acts["gate"][s], st, rg))
    torch.cuda.synchronize()
    outs = torch.stack(outs)  # [steps, N, H*d]
    # the reference: the decode tokens as a packed problem of N sequences x 32 tokens from
    # the oracle's own final states and rings (prefill == repeated decode is pinned in the
    # oracle tests)
    Hd = H * D
    dprob = {name: acts[name].transpose(0, 1).reshape(N * steps, -1).contiguous()
             for name in ("q", "k", "v", "z", "beta", "gate")}
    dprob["layer"] = prob["layer"]
    dprob["cu_seqlens"] = synthetic.cu_seqlens([steps] * N)
    sref = np.empty((N, H, D, D))
    rref = np.empty((N, 3, H, D, 3))
    for i, (n, h) in enumerate(units):
        sref[n, h] = s_ref[i]
        rref[n, :, h] = r_ref[i]
    dprob["state_in"] = torch.from_numpy(sref)
    dprob["ring_in"] = torch.from_numpy(rref.reshape(N, 3 * Hd, 3).astype(np.float32))
    check_all_units(dprob, outs.transpose(0, 1).reshape(N * steps, Hd).cpu(), st.cpu(),
                    _all_units(dprob), "varlen16_h64 decode continuation", batch=64)


def test_fp16_operand_range():
    """Activations 8192x larger than the configs' (raw q, k, v and the ring scaled up) and a
    quarter of the channels at g = 0, so that the state accumulates: the state pass's fp16
    operands -- the state itself and log2(e) times the SiLU conv outputs of q and k -- reach
    over half of fp16's largest finite value 65504 (asserted below from the oracle's trace)
    while staying under it.  Whole-sequence and segment-parallel paths, every unit against
    the oracle."""
    scale = 8192.0
    prob = synthetic.make_prefill([600, 300], H=2, io="bf16", seed=302, device=DEV,
                                  init_state=True, init_ring=True)
    for name in ("q", "k", "v"):
        prob[name] = (prob[name].float() * scale).to(torch.bfloat16)
    prob["ring_in"] *= scale
    z = prob["z"].view(900, 2, D)
    z[:, :, ::4] = -1e4
    # the regime, from the oracle's trace of one unit: SiLU outputs (v, whose distribution
    # q and k share) and state entries
    acts, st, rg = unit_inputs(prob, 0, 0)
    tr = oracle.prefill_units(head_layer(prob["layer"], 0), io_code(torch.bfloat16), [0, 600],
                              acts["q"], acts["k"], acts["v"], acts["z"], acts["beta"], acts["gate"],
                              st, rg, units=[(0, 0)], nthreads=1, trace=True)["trace"]
    assert np.abs(tr["v"]).max() * 1.4426950408889634 > 0.5 * 65504
    assert np.abs(tr["S"]).max() > 8000
    kda = _kda()
    assert kda.prefill_workspace_bytes(kda.Layer(**prob["layer"]), torch.bfloat16, prob["cu_seqlens"]) > 0
    for split in (False, True):
        out, state, ring = _prefill(prob, allow_split=split)
        assert torch.isfinite(out.float()).all() and torch.isfinite(state).all()
        check_all_units(prob, out.cpu(), state.cpu(), _all_units(prob),
                        f"fp16_range ({'segment-parallel' if split else 'whole-sequence'})", ring=ring.cpu())
