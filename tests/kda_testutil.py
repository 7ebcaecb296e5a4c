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


# --------------------------------------------------------------------------- parity metrics

FP32_REL_TOL = 1e-4   # max |gpu - ref| / max |ref|, fp32 io
BF16_RMS_TOL = 2e-2   # max |gpu - ref| / RMS(ref), bf16 io
# A value stored in bf16 carries its own rounding, up to half a unit in the last place,
# i.e. at most 2^-8 of its magnitude; that part of the difference is not charged.
BF16_HALF_ULP = 2.0 ** -8


def error_ratio(got, ref, io_is_bf16: bool, stored_bf16: bool = False) -> float:
    """The parity metric for one tensor, as a fraction of its tolerance (<= 1 passes).

    fp32 io: max |g - r| / max |r| against 1e-4.  bf16 io: max |g - r| / RMS(r) against
    2e-2, where for tensors stored in bf16 each element's difference is first reduced by
    its own rounding allowance 2^-8 |g|."""
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if not g.size:
        return 0.0
    d = np.abs(g - r)
    if io_is_bf16:
        if stored_bf16:
            d = np.maximum(d - BF16_HALF_ULP * np.abs(g), 0.0)
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
