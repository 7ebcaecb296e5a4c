"""GPU tests of kda_prefill_scan, the sequential-scan prefill arm (docs.rs
"memra_engine::kda": memra_kda_scan_s128 runs prefill and decode alike): parity with the
fp64 oracle, and bit-identity with decode steps."""
import pytest
import torch

import synthetic
from test_gpu_prefill import _all_units, _check, _ring_exact

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def _kda():
    import gated_delta_rule_05_amd as kda
    return kda


def _scan(prob, **kw):
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    res = kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"],
                      prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"],
                      state_in=prob.get("state_in"), ring_in=prob.get("ring_in"), scan=True, **kw)
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_scan_against_oracle(io):
    """Ragged lengths (an empty sequence, ones shorter than the conv window), carried
    state and ring."""
    lens = [37, 1, 0, 16, 2, 70, 33]
    prob = synthetic.make_prefill(lens, H=3, io=io, seed=401, device=DEV, init_state=True,
                                  init_ring=True)
    res = _scan(prob)
    _check(prob, res, _all_units(prob), f"scan_{io}")
    _ring_exact(prob, res[2])


def test_scan_is_bit_identical_to_decode_steps():
    """A prefill through the scan arm equals feeding its tokens one by one through
    kda_decode_step, bit for bit (outputs, final state, ring)."""
    kda = _kda()
    lens = [23, 9]
    prob = synthetic.make_prefill(lens, H=2, io="bf16", seed=402, device=DEV, init_state=True,
                                  init_ring=True)
    out, st, rg = _scan(prob)
    layer = kda.Layer(**prob["layer"])
    cu = prob["cu_seqlens"].tolist()
    for n in range(len(lens)):
        s = prob["state_in"][n:n + 1].clone()
        r = prob["ring_in"][n:n + 1].clone()
        for t in range(cu[n], cu[n + 1]):
            o = kda.decode_step(layer, *(prob[x][t:t + 1] for x in ("q", "k", "v", "z", "beta", "gate")), s, r)
            assert torch.equal(o[0], out[t]), (n, t)
        torch.cuda.synchronize()
        assert torch.equal(s[0], st[n]) and torch.equal(r[0], rg[n]), n


def test_scan_null_state_and_ring_mean_zeros():
    prob = synthetic.make_prefill([40, 7], H=2, io="bf16", seed=403, device=DEV)
    a = _scan(prob)
    prob["state_in"] = torch.zeros((2, 2, 128, 128), device=DEV)
    prob["ring_in"] = torch.zeros((2, 3 * 2 * 128, 3), device=DEV)
    b = _scan(prob)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_scan_takes_any_lower_bound():
    """The chunked kernel needs lower_bound >= -5 (its 16-token tile bound); the scan arm
    has no tile and runs, e.g., -8 against the oracle."""
    prob = synthetic.make_prefill([50, 31], H=2, io="bf16", seed=404, device=DEV, init_state=True)
    prob["layer"]["lower_bound"] = -8.0
    _check(prob, _scan(prob), _all_units(prob), "scan_lb8")
    kda = _kda()
    layer = kda.Layer(**prob["layer"])
    with pytest.raises(kda.KdaError):
        kda.prefill(layer, prob["q"], prob["k"], prob["v"], prob["z"], prob["beta"], prob["gate"],
                    prob["cu_seqlens"].to(DEV), prob["cu_seqlens"], state_in=prob["state_in"])


def test_softplus_gate_prefill_and_decode():
    """Kimi-Linear's unbounded gate g = -exp(A_log) softplus(z + dt_bias) with slow decay
    (the state carried over many chunks): the chunked kda_prefill and the scan arm both
    against the oracle, the same ring bits, and decode steps continuing from the states."""
    import gated_delta_rule_05_amd as kda
    from kda_testutil import assert_close, decode_as_prefill, oracle_units
    lens = [45, 3, 0, 60]
    prob = synthetic.make_prefill(lens, H=2, io="bf16", seed=405, device=DEV, init_state=True,
                                  init_ring=True)
    prob["layer"]["gate_kind"] = kda.GATE_SOFTPLUS
    prob["z"].mul_(0.25).sub_(3.0)  # softplus(z - 3) ~ 0.05: slow decay, state carried
    res = _kda().prefill(kda.Layer(**prob["layer"]), prob["q"], prob["k"], prob["v"], prob["z"],
                         prob["beta"], prob["gate"], prob["cu_seqlens"].to(DEV), prob["cu_seqlens"],
                         state_in=prob["state_in"], ring_in=prob["ring_in"])
    torch.cuda.synchronize()
    scan = _scan(prob)
    assert torch.equal(res[2], scan[2])
    _check(prob, res, _all_units(prob), "softplus_prefill")
    _check(prob, scan, _all_units(prob), "softplus_scan")
    # decode from the returned states: 5 steps on 4 sequences, against the oracle run over
    # the decode tokens from those states (which the prefill check pinned)
    layer = kda.Layer(**prob["layer"])
    dec = synthetic.make_decode(B=4, H=2, io="bf16", steps=5, seed=406, device=DEV)
    dec["layer"] = prob["layer"]
    dec["z"].mul_(0.25).sub_(3.0)
    dec["state"], dec["ring"] = res[1].clone(), res[2].clone()
    st, rg = dec["state"].clone(), dec["ring"].clone()
    outs = torch.stack([kda.decode_step(layer, dec["q"][s], dec["k"][s], dec["v"][s], dec["z"][s],
                                        dec["beta"][s], dec["gate"][s], st, rg) for s in range(5)])
    torch.cuda.synchronize()
    for b in range(4):
        for h in range(2):
            (o_ref, s_ref, _), = oracle_units(decode_as_prefill(dec, 5, b, h), [(0, 0)], workers=1)
            assert_close(outs[:, b, h * 128:(h + 1) * 128].float().cpu().numpy(), o_ref, True,
                         f"softplus decode out (b={b}, h={h})", stored_bf16=True)
            assert_close(st[b, h].cpu().numpy(), s_ref, True, f"softplus decode state (b={b}, h={h})")
