"""GPU parity of the chunked prefill with Kimi-Linear's unbounded softplus decay gate,
g = -exp(A_log) softplus(z + dt_bias) ("Kimi Delta Attention (KDA) -- analysis & C kernel
plan", status note), against the fp64 oracle through the C ABI.  Without the lower bound a
chunk's decay range is unbounded ("Kimi K3 - Retention gate", "Why": the position-pair
diagonal tiles); the cases below span in-chunk ranges from a fraction of a nat to
thousands, far past what one reference row per chunk could hold in fp32."""
import math

import numpy as np
import pytest
import torch

import synthetic
from kda_testutil import D, assert_close, oracle_units

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
    cu = prob["cu_seqlens"].tolist()
    Hd = prob["layer"]["num_heads"] * D
    worst = 0.0
    for (n, h), (o_ref, s_ref, r_ref) in zip(units, oracle_units(prob, units)):
        got = out[cu[n]:cu[n + 1], h * D:(h + 1) * D].float().cpu().numpy()
        assert np.isfinite(got).all(), f"{label} out (n={n}, h={h}) not finite"
        if got.size:
            worst = max(worst, assert_close(got, o_ref, True, f"{label} out (n={n}, h={h})", stored_bf16=True))
        worst = max(worst, assert_close(state[n, h].cpu().numpy(), s_ref, True, f"{label} state (n={n}, h={h})"))
        r = ring[n].cpu().numpy()
        got_r = np.stack([r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])
        assert np.array_equal(got_r.astype(np.float64), r_ref), f"{label} ring (n={n}, h={h})"
    print(f"{label}: worst error = {worst:.3f} x tolerance", flush=True)
    return worst


def _all_units(prob):
    return [(n, h) for n in range(len(prob["cu_seqlens"]) - 1) for h in range(prob["layer"]["num_heads"])]


def _chunk_range_nats(prob, h):
    """The largest decay range of any channel of head h over an aligned 16-token chunk, in
    nats (from the fp64 gate on the host, for the test's own coverage claim)."""
    p = prob["layer"]
    z = prob["z"][:, h * D:(h + 1) * D].double().cpu()
    x = z + p["dt_bias"][h * D:(h + 1) * D].double().cpu()
    g = -math.exp(float(p["A_log"][h])) * torch.nn.functional.softplus(x)
    worst = 0.0
    cu = prob["cu_seqlens"].tolist()
    for n in range(len(cu) - 1):
        for c0 in range(cu[n], cu[n + 1], 16):
            blk = g[c0 + 1:min(c0 + 16, cu[n + 1])]
            if blk.numel():
                worst = max(worst, float(-blk.sum(0).min()))
    return worst


def test_softplus_prefill_varlen():
    """Ragged sequences (chunk tails, shorter than the conv window, empty), carried state and
    ring, the synthetic gate distribution (A_log = log U(1, 16), z ~ N(0, 1)): every unit."""
    lens = [37, 1, 0, 16, 2, 130, 33]
    prob = synthetic.make_prefill(lens, H=3, io="bf16", seed=501, device=DEV, init_state=True,
                                  init_ring=True, softplus_gate=True)
    _check(prob, _prefill(prob, allow_split=False), _all_units(prob), "softplus_varlen")


def test_softplus_prefill_decay_ranges():
    """Four heads whose decay scales e^A_log run from 0.05 to 60: in-chunk ranges from under a
    nat (state carried across many chunks) to thousands of nats (every factor of a single
    reference row would leave fp32), all against the oracle."""
    prob = synthetic.make_prefill([300, 77], H=4, io="bf16", seed=502, device=DEV,
                                  init_state=True, init_ring=True, softplus_gate=True)
    prob["layer"]["A_log"] = torch.log(torch.tensor([0.05, 1.0, 16.0, 60.0], device=DEV))
    ranges = [_chunk_range_nats(prob, h) for h in range(4)]
    assert ranges[0] < 5.0 and ranges[3] > 1000.0, ranges
    _check(prob, _prefill(prob, allow_split=False), _all_units(prob), "softplus_ranges")


def test_softplus_prefill_segment_parallel():
    """Few (sequence, head) units: the segment-parallel path (Transfer pass, combine, Final
    pass) with the softplus gate, every unit against the oracle, beside the whole-sequence
    path."""
    prob = synthetic.make_prefill([1500, 300], H=2, io="bf16", seed=503, device=DEV,
                                  init_state=True, init_ring=True, softplus_gate=True)
    prob["layer"]["A_log"] = torch.log(torch.tensor([0.2, 4.0], device=DEV))
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    assert kda.prefill_workspace_bytes(layer, torch.bfloat16, prob["cu_seqlens"]) > 0
    split = _prefill(prob)
    _check(prob, split, _all_units(prob), "softplus_segment_parallel")
    whole = _prefill(prob, allow_split=False)
    assert torch.equal(split[2], whole[2])
    d = (split[0].float() - whole[0].float()).abs().max().item()
    rms = whole[0].float().pow(2).mean().sqrt().item()
    assert d <= 0.05 * rms, (d, rms)


def test_softplus_prefill_2x8192_h96():
    """The 2 x 8192-token, 96-head prefill with the softplus gate: sampled units against the
    oracle (the bench's softplus workload)."""
    prob = synthetic.make_workload("prefill_2x8192_h96_softplus", device=DEV)
    res = _prefill(prob)
    assert torch.isfinite(res[0].float()).all() and torch.isfinite(res[1]).all()
    rng = np.random.default_rng(9)
    units = sorted({(0, 0), (1, 95)} | {(int(rng.integers(0, 2)), int(rng.integers(0, 96))) for _ in range(3)})
    _check(prob, res, units, "softplus_2x8192_h96")


def test_softplus_low_rank_prefill_varlen():
    """Kimi-Linear's pairing: the softplus gate with the low-rank pre-activation z_low f_b^T
    formed inside the kernel (the position pairs then run in interval 2), ragged sequences,
    carried state and ring, every unit; then decode steps from the returned states."""
    from kda_testutil import decode_as_prefill
    kda = _kda()
    lens = [37, 1, 0, 16, 2, 130, 33]
    prob = synthetic.make_prefill(lens, H=3, io="bf16", seed=504, device=DEV, init_state=True,
                                  init_ring=True, low_rank_gate=True, softplus_gate=True)
    assert prob["z"].shape == (sum(lens), D)
    res = _prefill(prob, allow_split=False)
    _check(prob, res, _all_units(prob), "softplus_low_rank_varlen")
    layer = kda.Layer(**prob["layer"])
    dec = synthetic.make_decode(B=len(lens), H=3, io="bf16", steps=3, seed=505, device=DEV,
                                low_rank_gate=True)
    dec["layer"] = prob["layer"]
    dec["state"], dec["ring"] = res[1].clone(), res[2].clone()
    st, rg = dec["state"].clone(), dec["ring"].clone()
    outs = torch.stack([kda.decode_step(layer, dec["q"][s], dec["k"][s], dec["v"][s], dec["z"][s],
                                        dec["beta"][s], dec["gate"][s], st, rg) for s in range(3)])
    torch.cuda.synchronize()
    for b in (0, 5):
        for h in range(3):
            (o_ref, s_ref, _), = oracle_units(decode_as_prefill(dec, 3, b, h), [(0, 0)], workers=1)
            assert_close(outs[:, b, h * D:(h + 1) * D].float().cpu().numpy(), o_ref, True,
                         f"softplus low-rank decode out (b={b}, h={h})", stored_bf16=True)
            assert_close(st[b, h].cpu().numpy(), s_ref, True, f"softplus low-rank decode state (b={b}, h={h})")


def test_softplus_low_rank_segment_parallel():
    """The softplus and low-rank gates together on the segment-parallel path, every unit."""
    prob = synthetic.make_prefill([1500, 300], H=2, io="bf16", seed=506, device=DEV,
                                  init_state=True, init_ring=True, low_rank_gate=True,
                                  softplus_gate=True)
    kda = _kda()
    assert kda.prefill_workspace_bytes(kda.Layer(**prob["layer"]), torch.bfloat16, prob["cu_seqlens"]) > 0
    _check(prob, _prefill(prob), _all_units(prob), "softplus_low_rank_segment_parallel")


def test_softplus_low_rank_prefill_2x8192_h96():
    """2 x 8192 tokens, 96 heads, softplus and low-rank gates (the bench's Kimi-Linear
    workload): sampled units against the oracle."""
    prob = synthetic.make_workload("prefill_2x8192_h96_softplus_lowrank", device=DEV)
    res = _prefill(prob)
    assert torch.isfinite(res[0].float()).all() and torch.isfinite(res[1]).all()
    rng = np.random.default_rng(10)
    units = sorted({(0, 0), (1, 95)} | {(int(rng.integers(0, 2)), int(rng.integers(0, 96))) for _ in range(3)})
    _check(prob, res, units, "softplus_low_rank_2x8192_h96")


@pytest.mark.parametrize("low_rank", [False, True])
def test_softplus_prefill_fp32_runs_the_scan(low_rank):
    """fp32 io with the softplus gate (and with the low-rank gate too): kda_prefill runs the
    sequential scan, equal bit for bit to the explicit scan arm, and meets the oracle."""
    kda = _kda()
    lens = [45, 3, 0, 60]
    prob = synthetic.make_prefill(lens, H=2, io="f32", seed=507, device=DEV, init_state=True,
                                  init_ring=True, low_rank_gate=low_rank, softplus_gate=True)
    res = _prefill(prob)
    scan = _prefill(prob, scan=True)
    for x, y in zip(res, scan):
        assert torch.equal(x, y)
    out, state, ring = res
    cu = prob["cu_seqlens"].tolist()
    for (n, h), (o_ref, s_ref, _) in zip(_all_units(prob), oracle_units(prob, _all_units(prob))):
        got = out[cu[n]:cu[n + 1], h * D:(h + 1) * D].cpu().numpy()
        if got.size:
            assert_close(got, o_ref, False, f"softplus fp32 out (n={n}, h={h})")
        assert_close(state[n, h].cpu().numpy(), s_ref, False, f"softplus fp32 state (n={n}, h={h})")
