"""GPU tests of kda_decode_multi: several decode tokens per sequence in one launch (the
batched verify of speculative decoding) and rollback by replay (docs.rs
"memra_engine::kda": kda_verify_rows_cached, kda_verify_rollback_rows, kda_scan_replay).

Two properties: each row is bit-identical to chaining one-token decode steps (the pages
require per-row bit-identity of the verify with the t = 1 chain), and the results match
the fp64 oracle like any decode step."""
import numpy as np
import pytest
import torch

import synthetic
from kda_testutil import D, assert_close, decode_as_prefill, oracle_units

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
NAMES = ("q", "k", "v", "z", "beta", "gate")


def _kda():
    import gated_delta_rule_05_amd as kda
    return kda


def _rows(dec, t):
    """The first t steps of a decode problem as [B, t, ...] rows (the multi-token layout)."""
    return {n: dec[n][:t].transpose(0, 1).contiguous() for n in NAMES}


def _chain(layer, dec, t, state, ring, ntok=None):
    """Chained one-token steps on copies; sequence b stops after ntok[b] steps.  Returns
    the outputs [B, t, H*d] (rows past a sequence's count are zero) and final buffers."""
    kda = _kda()
    B = state.shape[0]
    st, rg = state.clone(), ring.clone()
    outs = torch.zeros((B, t, dec["q"].shape[-1]), dtype=dec["q"].dtype, device=DEV)
    counts = [t] * B if ntok is None else list(ntok)
    for b in range(B):
        for s in range(counts[b]):
            o = kda.decode_step(layer, *(dec[n][s, b:b + 1] for n in NAMES), st[b:b + 1], rg[b:b + 1])
            outs[b, s] = o[0]
    torch.cuda.synchronize()
    return outs, st, rg


@pytest.mark.parametrize("t", [4, 6])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_multi_is_bit_identical_to_chained_steps(io, t):
    """Ping-pong and in place, at the speculative verify's 4 tokens and at 6."""
    kda = _kda()
    B, H = 5, 3
    dec = synthetic.make_decode(B=B, H=H, io=io, steps=t, seed=301, device=DEV)
    layer = kda.Layer(**dec["layer"])
    ref_out, ref_st, ref_rg = _chain(layer, dec, t, dec["state"], dec["ring"])
    rows = _rows(dec, t)
    st_out = torch.empty_like(dec["state"])
    rg_out = torch.empty_like(dec["ring"])
    st_in, rg_in = dec["state"].clone(), dec["ring"].clone()
    out = kda.decode_multi(layer, *(rows[n] for n in NAMES), st_in, rg_in, st_out, rg_out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out)
    assert torch.equal(st_out, ref_st)
    assert torch.equal(rg_out, ref_rg)
    # the inputs of a ping-pong call are untouched
    assert torch.equal(st_in, dec["state"]) and torch.equal(rg_in, dec["ring"])
    # in place gives the same bits
    out2 = kda.decode_multi(layer, *(rows[n] for n in NAMES), st_in, rg_in)
    torch.cuda.synchronize()
    assert torch.equal(out2, ref_out) and torch.equal(st_in, ref_st) and torch.equal(rg_in, ref_rg)


@pytest.mark.parametrize("t,counts", [(7, [7, 0, 1, 4, 3, 7]), (4, [4, 0, 1, 2, 3, 4])])
def test_multi_against_oracle_with_ragged_counts(t, counts):
    """bf16, per-sequence token counts 0..t: outputs of the run rows and final states match
    the oracle over each sequence's own prefix; rows past the count are not written; a
    sequence with 0 rows passes its state and ring through."""
    kda = _kda()
    B, H = 6, 2
    dec = synthetic.make_decode(B=B, H=H, io="bf16", steps=t, seed=302, device=DEV)
    layer = kda.Layer(**dec["layer"])
    ntok = torch.tensor(counts, dtype=torch.int32, device=DEV)
    rows = _rows(dec, t)
    sentinel = torch.full((B, t, H * D), 7.0, dtype=torch.bfloat16, device=DEV)
    st_out = torch.empty_like(dec["state"])
    rg_out = torch.empty_like(dec["ring"])
    kda.decode_multi(layer, *(rows[n] for n in NAMES), dec["state"], dec["ring"], st_out, rg_out,
                     ntok=ntok, out=sentinel)
    torch.cuda.synchronize()
    for b, c in enumerate(counts):
        assert torch.all(sentinel[b, c:] == 7.0), f"rows past the count written (b={b})"
        if c == 0:
            assert torch.equal(st_out[b], dec["state"][b]) and torch.equal(rg_out[b], dec["ring"][b])
            continue
        for h in range(H):
            (o_ref, s_ref, r_ref), = oracle_units(decode_as_prefill(dec, c, b, h), [(0, 0)], workers=1)
            got = sentinel[b, :c, h * D:(h + 1) * D].float().cpu().numpy()
            assert_close(got, o_ref, True, f"out (b={b}, h={h})", stored_bf16=True)
            assert_close(st_out[b, h].cpu().numpy(), s_ref, True, f"state (b={b}, h={h})")
            ring_b = rg_out[b].cpu().numpy()
            got_r = np.stack([ring_b[p * H * D + h * D:p * H * D + (h + 1) * D] for p in range(3)])
            assert np.array_equal(got_r, r_ref), f"ring (b={b}, h={h})"


def test_verify_then_rollback_by_replay():
    """A speculative round on the 256 x 32 decode shape: verify t = K + 1 = 4 rows per
    sequence from the pre-round buffers into a second pair (ping-pong), accept a random
    prefix per sequence, and rebuild the accepted state by replaying the same launch from
    the untouched pre-round buffers.  The rebuilt state and ring are byte-identical to
    chaining the accepted one-token steps; the verify's outputs are byte-identical to the
    chained outputs."""
    kda = _kda()
    B, H, t = 256, 32, 4
    dec = synthetic.make_decode(B=B, H=H, io="bf16", steps=t, seed=303, device=DEV)
    layer = kda.Layer(**dec["layer"])
    rows = _rows(dec, t)
    s0, r0 = dec["state"], dec["ring"]               # pre-round (never written below)
    s1, r1 = torch.empty_like(s0), torch.empty_like(r0)
    out = kda.decode_multi(layer, *(rows[n] for n in NAMES), s0, r0, s1, r1)
    g = torch.Generator().manual_seed(304)
    keep = torch.randint(0, t + 1, (B,), generator=g).to(torch.int32)
    kda.decode_multi(layer, *(rows[n] for n in NAMES), s0, r0, s1, r1, ntok=keep.to(DEV),
                     write_out=False)
    torch.cuda.synchronize()
    # reference: chained one-token steps over the accepted prefix, on a sample of sequences
    idx = [0, 1, 2] + sorted(torch.randperm(B, generator=g)[:13].tolist())
    for b in idx:
        k = int(keep[b])
        st, rg = s0[b:b + 1].clone(), r0[b:b + 1].clone()
        for s in range(t):
            o = kda.decode_step(layer, *(dec[n][s, b:b + 1] for n in NAMES), st, rg)
            assert torch.equal(o[0], out[b, s]), f"verify row {s} of sequence {b}"
            if s + 1 == k:
                st_k, rg_k = st.clone(), rg.clone()
        if k == 0:
            st_k, rg_k = s0[b:b + 1], r0[b:b + 1]
        assert torch.equal(s1[b:b + 1], st_k), f"rolled-back state of sequence {b} (keep {k})"
        assert torch.equal(r1[b:b + 1], rg_k), f"rolled-back ring of sequence {b} (keep {k})"


def test_zero_tokens_copies_through():
    kda = _kda()
    dec = synthetic.make_decode(B=2, H=2, io="bf16", steps=1, seed=305, device=DEV)
    layer = kda.Layer(**dec["layer"])
    empty = {n: dec[n][:0].transpose(0, 1).contiguous() for n in NAMES}
    s1, r1 = torch.zeros_like(dec["state"]), torch.zeros_like(dec["ring"])
    out = kda.decode_multi(layer, *(empty[n] for n in NAMES), dec["state"], dec["ring"], s1, r1)
    torch.cuda.synchronize()
    assert out.shape[1] == 0
    assert torch.equal(s1, dec["state"]) and torch.equal(r1, dec["ring"])


@pytest.mark.parametrize("t", [3, 5])
@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_multi_softplus_gate_is_bit_identical_to_chained_steps(io, t):
    """The same per-row bit-identity with the unbounded softplus gate (its fast decays make
    the state forget within a few rows, so every row's own arithmetic shows)."""
    kda = _kda()
    B, H = 4, 2
    dec = synthetic.make_decode(B=B, H=H, io=io, steps=t, seed=307, device=DEV)
    dec["layer"]["gate_kind"] = synthetic.GATE_SOFTPLUS
    layer = kda.Layer(**dec["layer"])
    ref_out, ref_st, ref_rg = _chain(layer, dec, t, dec["state"], dec["ring"])
    rows = _rows(dec, t)
    st, rg = dec["state"].clone(), dec["ring"].clone()
    out = kda.decode_multi(layer, *(rows[n] for n in NAMES), st, rg)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_out) and torch.equal(st, ref_st) and torch.equal(rg, ref_rg)
    for b in (0, B - 1):
        for h in range(H):
            (o_ref, s_ref, _), = oracle_units(decode_as_prefill(dec, t, b, h), [(0, 0)], workers=1)
            assert_close(out[b, :, h * D:(h + 1) * D].float().cpu().numpy(), o_ref, io == "bf16",
                         f"softplus multi out (b={b}, h={h})", stored_bf16=io == "bf16")
            assert_close(st[b, h].cpu().numpy(), s_ref, io == "bf16", f"softplus multi state (b={b}, h={h})")
