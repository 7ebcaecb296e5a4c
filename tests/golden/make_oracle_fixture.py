"""Writes tests/golden/oracle_tiny.json: a small fp32 problem and the oracle's answer.

Calls only the oracle.  The fixture guards the oracle against unintended change; it is
not independent evidence (the pins in tests/test_oracle_pins.py are).
Run from the repository root:  python tests/golden/make_oracle_fixture.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402


def problem():
    r = np.random.default_rng(777)
    H, d, lens = 2, 8, [5, 3]
    T = sum(lens)
    p = dict(H=H, d=d, seqlens=lens,
             conv_w=r.uniform(-0.5, 0.5, (3 * H * d, 4)).astype(np.float32),
             dt_bias=r.normal(0, 0.1, H * d).astype(np.float32),
             A_log=np.log(r.uniform(1, 16, H)).astype(np.float32),
             norm_w=(1 + r.normal(0, 0.02, d)).astype(np.float32))
    for n in ("q", "k", "v", "z", "gate"):
        p[n] = r.normal(0, 1, (T, H * d)).astype(np.float32)
    p["beta"] = r.normal(0, 1, (T, H)).astype(np.float32)
    p["state_in"] = r.normal(0, 0.02, (len(lens), H, d, d)).astype(np.float32)
    p["ring_in"] = r.normal(0, 1, (len(lens), 3 * H * d, 3)).astype(np.float32)
    return p


def run(p):
    L = oracle.Layer(p["H"], p["d"], p["conv_w"], p["dt_bias"], p["A_log"], p["norm_w"])
    cu = np.concatenate([[0], np.cumsum(p["seqlens"])])
    return oracle.prefill(L, oracle.F32, cu, p["q"], p["k"], p["v"], p["z"], p["beta"],
                          p["gate"], p["state_in"].astype(np.float64), p["ring_in"])


if __name__ == "__main__":
    p = problem()
    out, state, ring = run(p)
    doc = {k: (v.tolist() if isinstance(v, np.ndarray) else v) for k, v in p.items()}
    doc.update(expected_out=out.tolist(), expected_state=state.tolist(),
               expected_ring=ring.tolist())
    with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_tiny.json"), "w") as f:
        json.dump(doc, f)
    print("wrote oracle_tiny.json")
