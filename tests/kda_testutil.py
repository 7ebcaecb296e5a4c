"""Helpers shared by the tests: oracle runs on sampled (sequence, head) units and the
parity metrics.  Imports the oracle (test infrastructure) and never the HIP library."""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import oracle

D = 128


def _cpu(x):
    return None if x is None else x.detach().to("cpu")


def head_layer(params: dict, h: int) -> oracle.Layer:
    """The oracle layer of head h alone (H = 1), cut from the full layer's parameters."""
    H = params["num_heads"]
    Hd = H * D
    cw = _cpu(params["conv_w"]).numpy()
    rows = np.concatenate([cw[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])
    f_b = params.get("f_b")
    return oracle.Layer(1, D, conv_w=rows,
                        dt_bias=_cpu(params["dt_bias"]).numpy()[h * D:(h + 1) * D],
                        A_log=_cpu(params["A_log"]).numpy()[h:h + 1],
                        norm_w=_cpu(params["norm_w"]).numpy(),
                        lower_bound=params["lower_bound"], l2_eps=params["l2_eps"],
                        rms_eps=params["rms_eps"], gate_kind=params.get("gate_kind", 0),
                        f_b=None if f_b is None else _cpu(f_b[h * D:(h + 1) * D]).contiguous())


def io_code(dtype) -> int:
    return oracle.BF16 if dtype == torch.bfloat16 else oracle.F32


def unit_inputs(prob: dict, n: int, h: int):
    """Slices of one (sequence, head) unit of a packed prefill problem, on the CPU."""
    cu = prob["cu_seqlens"].tolist()
    H = prob["layer"]["num_heads"]
    Hd = H * D
    lo, hi = cu[n], cu[n + 1]
    cols = slice(h * D, (h + 1) * D)
    acts = {name: _cpu(prob[name][lo:hi, cols]).contiguous() for name in ("q", "k", "v", "gate")}
    # the low-rank gate's z_low is shared by every head
    low_rank = prob["layer"].get("f_b") is not None
    acts["z"] = _cpu(prob["z"][lo:hi] if low_rank else prob["z"][lo:hi, cols]).contiguous()
    acts["beta"] = _cpu(prob["beta"][lo:hi, h:h + 1]).contiguous()
    st = None if prob.get("state_in") is None else _cpu(prob["state_in"][n, h]).double().numpy()[None, None]
    rg = None
    if prob.get("ring_in") is not None:
        r = _cpu(prob["ring_in"][n]).numpy()
        rg = np.concatenate([r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])[None]
    return acts, st, rg


def oracle_units(prob: dict, units, workers: int | None = None):
    """Run the oracle on each listed (n, h) unit of a prefill problem.  Returns a list of
    (out [T_n, 128], state [128, 128], ring [3, 128, 3]) in fp64."""
    params = prob["layer"]
    io = io_code(prob["q"].dtype)

    def one(u):
        n, h = u
        acts, st, rg = unit_inputs(prob, n, h)
        T = acts["q"].shape[0]
        res = oracle.prefill_units(head_layer(params, h), io, [0, T], acts["q"], acts["k"],
                                   acts["v"], acts["z"], acts["beta"], acts["gate"], st, rg,
                                   units=[(0, 0)], nthreads=1)
        return res["out"][0], res["state"][0], res["ring"][0]

    workers = workers or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(workers) as ex:
        return list(ex.map(one, list(units)))


def decode_as_prefill(dec: dict, steps: int, b: int, h: int) -> dict:
    """A decode run of `steps` tokens for sequence b, head h, rewritten as a one-sequence
    prefill problem with H = 1 (prefill == repeated decode is pinned in the oracle tests)."""
    H = dec["layer"]["num_heads"]
    Hd = H * D
    cols = slice(h * D, (h + 1) * D)
    prob = {name: _cpu(dec[name][:steps, b, cols]) for name in ("q", "k", "v", "gate")}
    low_rank = dec["layer"].get("f_b") is not None
    prob["z"] = _cpu(dec["z"][:steps, b] if low_rank else dec["z"][:steps, b, cols])
    prob["beta"] = _cpu(dec["beta"][:steps, b, h:h + 1])
    prob["state_in"] = _cpu(dec["state"][b:b + 1, h:h + 1])
    r = _cpu(dec["ring"][b]).numpy()
    prob["ring_in"] = torch.from_numpy(np.concatenate(
        [r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])[None].copy())
    prob["cu_seqlens"] = torch.tensor([0, steps], dtype=torch.int32)
    lay = head_layer(dec["layer"], h)
    prob["layer"] = dict(num_heads=1, conv_w=torch.from_numpy(lay.conv_w),
                         dt_bias=torch.from_numpy(lay.dt_bias), A_log=torch.from_numpy(lay.A_log),
                         norm_w=torch.from_numpy(lay.norm_w), lower_bound=lay.lower_bound,
                         l2_eps=lay.l2_eps, rms_eps=lay.rms_eps, gate_kind=lay.gate_kind,
                         f_b=lay.f_b)
    return prob


def full_layer(params: dict) -> oracle.Layer:
    """The oracle layer with every head of a problem's parameters."""
    f_b = params.get("f_b")
    return oracle.Layer(params["num_heads"], D, conv_w=_cpu(params["conv_w"]).numpy(),
                        dt_bias=_cpu(params["dt_bias"]).numpy(), A_log=_cpu(params["A_log"]).numpy(),
                        norm_w=_cpu(params["norm_w"]).numpy(), lower_bound=params["lower_bound"],
                        l2_eps=params["l2_eps"], rms_eps=params["rms_eps"],
                        gate_kind=params.get("gate_kind", 0),
                        f_b=None if f_b is None else _cpu(f_b).contiguous())


def check_all_units(prob: dict, out, state, units, label: str, batch: int = 16, ring=None,
                    keep_final: bool = False):
    """Every listed (n, h) unit of a packed prefill problem against the oracle, streamed:
    the oracle runs `batch` units at a time on all host cores, each unit's output rows and
    final state are compared with the GPU's (out [T, H*d], state [N, H, d, d], both already
    on the host) and only the metrics are kept.  Asserts every unit within tolerance;
    returns the worst ratios (charged / raw / rne for bf16 outputs, see
    bf16_output_metrics) and prints them.  With keep_final, also the oracle's own final
    states [units, d, d] and rings [units, 3, d, 3] (fp64), in the order of `units`."""
    params = prob["layer"]
    io = io_code(prob["q"].dtype)
    bf16 = prob["q"].dtype == torch.bfloat16
    cu = prob["cu_seqlens"].tolist()
    H = params["num_heads"]
    Hd = H * D
    lay = full_layer(params)
    cpu = {name: _cpu(prob[name]).contiguous() for name in ("q", "k", "v", "z", "beta", "gate")}
    st_in = None if prob.get("state_in") is None else _cpu(prob["state_in"]).double().numpy()
    rg_in = None if prob.get("ring_in") is None else _cpu(prob["ring_in"]).numpy()
    units = list(units)
    worst = dict(out=0.0, out_raw=0.0, out_rne=0.0, state=0.0)
    finals = (np.empty((len(units), D, D)), np.empty((len(units), 3, D, 3))) if keep_final else None
    for b0 in range(0, len(units), batch):
        part = units[b0:b0 + batch]
        res = oracle.prefill_units(lay, io, cu, cpu["q"], cpu["k"], cpu["v"], cpu["z"], cpu["beta"],
                                   cpu["gate"], st_in, rg_in, units=part,
                                   nthreads=min(len(part), os.cpu_count() or 1))
        for i, (n, h) in enumerate(part):
            got = out[cu[n]:cu[n + 1], h * D:(h + 1) * D].float().numpy()
            ref = res["out"][i]
            if got.size:
                assert np.all(np.isfinite(got)), f"{label} out (n={n}, h={h}): non-finite values"
                if bf16:
                    m = bf16_output_metrics(got, ref)
                    worst["out_raw"] = max(worst["out_raw"], m["raw"])
                    worst["out_rne"] = max(worst["out_rne"], m["rne"])
                    e = m["charged"]
                else:
                    e = error_ratio(got, ref, False)
                assert e <= 1.0, f"{label} out (n={n}, h={h}): error is {e:.3g} x the tolerance"
                worst["out"] = max(worst["out"], e)
            if state is not None:
                worst["state"] = max(worst["state"], assert_close(state[n, h].numpy(), res["state"][i], bf16,
                                                                  f"{label} state (n={n}, h={h})"))
            if ring is not None:
                r = ring[n].numpy()
                got_r = np.stack([r[p * Hd + h * D:p * Hd + (h + 1) * D] for p in range(3)])
                assert np.array_equal(got_r.astype(np.float64), res["ring"][i]), f"{label} ring (n={n}, h={h})"
        if keep_final:
            finals[0][b0:b0 + len(part)] = res["state"]
            finals[1][b0:b0 + len(part)] = res["ring"]
        del res
    print(f"{label}: {len(units)} units; worst out {worst['out']:.3f} x tolerance (raw {worst['out_raw']:.3f}, "
          f"vs rounded reference {worst['out_rne']:.3f}), state {worst['state']:.3f}", flush=True)
    return (worst, finals) if keep_final else worst


# --------------------------------------------------------------------------- parity metrics

FP32_REL_TOL = 1e-4   # max |gpu - ref| / max |ref|, fp32 io
BF16_RMS_TOL = 2e-2   # max |gpu - ref| / RMS(ref), bf16 io


def bf16_rne(x):
    """fp64 values rounded to the nearest bf16 value (8 significant bits, ties to even),
    returned as fp64: the output a kernel that rounds the exact result once would store."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)  # |x| in [2^(e-1), 2^e)
    sp = np.ldexp(1.0, e - 8)
    return np.where(x == 0, 0.0, np.rint(x / sp) * sp)


def bf16_half_ulp(x):
    """Half the bf16 spacing at each fp64 value: the largest error that rounding the exact
    value to bf16 (nearest) can make there, |bf16_rne(x) - x| <= bf16_half_ulp(x)."""
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    return np.where(x == 0, 0.0, np.ldexp(1.0, e - 9))


def bf16_output_metrics(got, ref) -> dict:
    """Three forms of the bf16-output error, each as a fraction of 2e-2 RMS(ref):
      charged  max(|g - r| - h(r), 0): the error beyond the output's own rounding, with
               h(r) the exact half-ulp of bf16 at the reference value (a kernel that
               rounds the exact value once scores 0);
      raw      max |g - r|: includes that rounding, which alone reaches 1.6-1.7x the
               tolerance on outputs at 15-16x their RMS after the per-row normalisation;
      rne      max |g - bf16_rne(r)|: any one-ulp difference on such an output is over 1.5x
               the tolerance, so fp32-level noise that flips a rounding fails it."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    d = np.abs(g - r)

    def frac(err):
        return err / (BF16_RMS_TOL * rms) if rms > 0 else (0.0 if err == 0 else np.inf)

    if not g.size:
        return dict(charged=0.0, raw=0.0, rne=0.0)
    return dict(charged=frac(float(np.max(np.maximum(d - bf16_half_ulp(r), 0.0)))),
                raw=frac(float(np.max(d))), rne=frac(float(np.max(np.abs(g - bf16_rne(r))))))


def error_ratio(got, ref, io_is_bf16: bool, stored_bf16: bool = False) -> float:
    """The parity metric for one tensor, as a fraction of its tolerance (<= 1 passes).

    fp32 io: max |g - r| / max |r| against 1e-4.  bf16 io: max |g - r| / RMS(r) against
    2e-2; for tensors stored in bf16 (the output) the error is the part beyond the
    output's own rounding, max(|g - r| - h(r), 0) with h(r) the exact bf16 half-ulp at the
    reference value (bf16_output_metrics)."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if not g.size:
        return 0.0
    if io_is_bf16 and stored_bf16:
        return bf16_output_metrics(g, r)["charged"]
    d = np.abs(g - r)
    if io_is_bf16:
        rms = float(np.sqrt(np.mean(r * r)))
        err = float(np.max(d))
        return err / (BF16_RMS_TOL * rms) if rms > 0 else (0.0 if err == 0 else np.inf)
    mx = float(np.max(np.abs(r)))
    err = float(np.max(d))
    return err / (FP32_REL_TOL * mx) if mx > 0 else (0.0 if err == 0 else np.inf)


def rms_error(got, ref) -> float:
    """RMS(g - r) / RMS(r), reported beside the max-based metric."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    den = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    return float(np.sqrt(np.mean((g - r) ** 2))) / den if den > 0 else 0.0


def assert_close(got, ref, io_is_bf16: bool, what: str, stored_bf16: bool = False):
    g = np.asarray(got, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"{what}: non-finite values"
    e = error_ratio(g, ref, io_is_bf16, stored_bf16)
    assert e <= 1.0, (f"{what}: error is {e:.3g} x the tolerance "
                      f"(rms error {rms_error(g, ref):.3g} of rms)")
    return e
