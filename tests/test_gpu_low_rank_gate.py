"""GPU parity of the low-rank decay gate (kda_layer.f_b) against the fp64 oracle, through the
C ABI: z is z_low [rows, 128] and the gate's pre-activation z_low f_b^T ("Kimi Delta
Attention (KDA) -- analysis & C kernel plan", "The KDA layer, precisely", fact 2; the
Retention-gate page's f_b_proj(f_a_proj(.))).  The bf16 chunked prefill forms the
projection on MFMA inside the kernel, fp32 io runs the sequential scan, and decode forms it
per channel."""
import numpy as np
import pytest
import torch

import synthetic
from kda_testutil import D, assert_close, decode_as_prefill, oracle_units

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
    Hd = prob["layer"]["num_heads"] * D
    worst = 0.0
    for (n, h), (o_ref, s_ref, r_ref) in zip(units, oracle_units(prob, units)):
        got = out[cu[n]:cu[n + 1], h * D:(h + 1) * D].float().cpu().numpy()
        if got.size:
            worst = max(worst, assert_close(got, o_ref, bf16, f"{label} out (n={n}, h={h})", stored_bf16=bf16))
        worst = max(worst, assert_close(state[n, h].cpu().numpy(), s_ref, bf16, f"{label} state (n={n}, h={h})"))
        r = ring[n].cpu().numpy()
        got_r = np.stack([r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])
        assert np.array_equal(got_r.astype(np.float64), r_ref), f"{label} ring (n={n}, h={h})"
    print(f"{label}: worst error = {worst:.3f} x tolerance", flush=True)
    return worst


def _all_units(prob):
    return [(n, h) for n in range(len(prob["cu_seqlens"]) - 1) for h in range(prob["layer"]["num_heads"])]


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_low_rank_prefill_varlen(io):
    """Ragged sequences (chunk tails, shorter than the conv window, empty), carried state and
    ring, three heads (f_b rows h*128 + i): every unit.  bf16 runs the chunked kernel's MFMA
    projection on the whole-sequence path; fp32 runs the sequential scan."""
    lens = [37, 1, 0, 16, 2, 130, 33]
    prob = synthetic.make_prefill(lens, H=3, io=io, seed=301, device=DEV, init_state=True,
                                  init_ring=True, low_rank_gate=True)
    assert prob["z"].shape == (sum(lens), D)
    _check(prob, _prefill(prob, allow_split=False), _all_units(prob), f"low_rank_varlen_{io}")


def test_low_rank_prefill_segment_parallel():
    """Few (sequence, head) units: the segment-parallel path (Transfer pass, combine, Final
    pass) with the low-rank gate, every unit against the oracle, and beside the
    whole-sequence path."""
    prob = synthetic.make_prefill([1500, 300], H=2, io="bf16", seed=302, device=DEV,
                                  init_state=True, init_ring=True, low_rank_gate=True)
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    assert kda.prefill_workspace_bytes(layer, torch.bfloat16, prob["cu_seqlens"]) > 0
    split = _prefill(prob)
    _check(prob, split, _all_units(prob), "low_rank_segment_parallel")
    whole = _prefill(prob, allow_split=False)
    assert torch.equal(split[2], whole[2])
    d = (split[0].float() - whole[0].float()).abs().max().item()
    rms = whole[0].float().pow(2).mean().sqrt().item()
    assert d <= 0.05 * rms, (d, rms)


def test_low_rank_prefill_2x8192_h96():
    """The 2 x 8192-token, 96-head prefill with the low-rank gate: sampled units against the
    oracle (the bench's low-rank workload)."""
    prob = synthetic.make_workload("prefill_2x8192_h96_lowrank", device=DEV)
    res = _prefill(prob)
    assert torch.isfinite(res[0].float()).all() and torch.isfinite(res[1]).all()
    rng = np.random.default_rng(8)
    units = sorted({(0, 0), (1, 95)} | {(int(rng.integers(0, 2)), int(rng.integers(0, 96))) for _ in range(3)})
    _check(prob, res, units, "low_rank_2x8192_h96")


@pytest.mark.parametrize("io", ["bf16", "f32"])
def test_low_rank_decode_steps_and_multi(io):
    """Decode with the low-rank gate: six chained one-token steps against the oracle on
    sampled units, and one six-row kda_decode_multi launch bit-identical to the chain."""
    kda = _kda()
    B, H, steps = 6, 4, 6
    dec = synthetic.make_decode(B, H, io, steps, seed=303, device=DEV, low_rank_gate=True)
    layer = kda.Layer(**dec["layer"])
    st0, rg0 = dec["state"].clone(), dec["ring"].clone()
    st, rg = st0.clone(), rg0.clone()
    outs = []
    for s in range(steps):
        outs.append(kda.decode_step(layer, dec["q"][s], dec["k"][s], dec["v"][s], dec["z"][s],
                                    dec["beta"][s], dec["gate"][s], st, rg))
    torch.cuda.synchronize()
    bf16 = io == "bf16"
    for b, h in [(0, 0), (B - 1, H - 1), (2, 1)]:
        p = decode_as_prefill(dec, steps, b, h)
        (o_ref, s_ref, _), = oracle_units(p, [(0, 0)], workers=1)
        got = torch.stack([o[b, h * D:(h + 1) * D] for o in outs]).float().cpu().numpy()
        assert_close(got, o_ref, bf16, f"decode out (b={b}, h={h})", stored_bf16=bf16)
        assert_close(st[b, h].cpu().numpy(), s_ref, bf16, f"decode state (b={b}, h={h})")
    # the same rows in one multi-token launch
    t = lambda x: x.transpose(0, 1).contiguous()
    st2, rg2 = st0.clone(), rg0.clone()
    out = kda.decode_multi(layer, t(dec["q"]), t(dec["k"]), t(dec["v"]), t(dec["z"]), t(dec["beta"]),
                           t(dec["gate"]), st2, rg2)
    torch.cuda.synchronize()
    assert torch.equal(out, torch.stack(outs, dim=1))
    assert torch.equal(st2, st) and torch.equal(rg2, rg)


def test_low_rank_prefill_then_decode():
    """A fused-gate prefill's returned state and ring, continued by fused-gate decode steps:
    the decode outputs against the oracle run over the joined tokens."""
    kda = _kda()
    H, steps = 2, 4
    lens = [70, 45]
    prob = synthetic.make_prefill(lens, H=H, io="bf16", seed=304, device=DEV, init_state=True,
                                  init_ring=True, low_rank_gate=True)
    layer = kda.Layer(**prob["layer"])
    _, st, rg = _prefill(prob)
    dec = synthetic.make_decode(len(lens), H, "bf16", steps, seed=305, device=DEV, low_rank_gate=True)
    outs = []
    for s in range(steps):
        outs.append(kda.decode_step(layer, dec["q"][s], dec["k"][s], dec["v"][s], dec["z"][s],
                                    dec["beta"][s], dec["gate"][s], st, rg))
    torch.cuda.synchronize()
    cu = prob["cu_seqlens"].tolist()
    for n in range(len(lens)):
        # the joined problem: the prefill tokens of sequence n, then its decode tokens
        joined = {name: torch.cat([prob[name][cu[n]:cu[n + 1]], dec[name][:, n]]).contiguous()
                  for name in ("q", "k", "v", "z", "gate", "beta")}
        joined.update(layer=prob["layer"], cu_seqlens=torch.tensor([0, lens[n] + steps], dtype=torch.int32),
                      state_in=prob["state_in"][n:n + 1], ring_in=prob["ring_in"][n:n + 1])
        for h in range(H):
            (o_ref, _, _), = oracle_units(joined, [(0, h)], workers=1)
            got = torch.stack([o[n, h * D:(h + 1) * D] for o in outs]).float().cpu().numpy()
            assert_close(got, o_ref[lens[n]:], True, f"continued decode (n={n}, h={h})", stored_bf16=True)


def test_low_rank_gate_argument_checks():
    """f_b must be 16-byte aligned; z must have 128 columns and f_b the io dtype."""
    kda = _kda()
    prob = synthetic.make_prefill([20], H=2, io="bf16", seed=306, device=DEV, low_rank_gate=True)
    params = dict(prob["layer"])
    with pytest.raises(TypeError):
        kda.prefill(kda.Layer(**params), prob["q"].float(), prob["k"].float(), prob["v"].float(),
                    prob["z"].float(), prob["beta"].float(), prob["gate"].float(),
                    prob["cu_seqlens"].to(DEV), prob["cu_seqlens"])
    full = synthetic.make_prefill([20], H=2, io="bf16", seed=306, device=DEV)
    with pytest.raises(ValueError):
        kda.prefill(kda.Layer(**params), full["q"], full["k"], full["v"], full["z"], full["beta"],
                    full["gate"], full["cu_seqlens"].to(DEV), full["cu_seqlens"])
    buf = torch.empty(params["f_b"].numel() + 8, dtype=torch.bfloat16, device=DEV)
    params["f_b"] = buf[1:1 + params["f_b"].numel()].view(2 * D, D)
    with pytest.raises(kda.KdaError):
        kda.prefill(kda.Layer(**params), prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"],
                    prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"])
