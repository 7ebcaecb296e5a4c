"""Golden fixtures: figures the pages print (layouts and bounds) and a small oracle
regression fixture written by tests/golden/make_oracle_fixture.py (oracle only)."""
import json
import math
import os

import numpy as np

import oracle
import synthetic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _facts():
    with open(os.path.join(GOLDEN, "page_facts.json")) as f:
        return json.load(f)


def state_bytes_per_head(d=synthetic.HEAD_DIM):
    """fp32 [d_k][d_v] per (sequence, head): the state layout the library uses."""
    return d * d * 4


def ring_bytes_per_sequence(H, d=synthetic.HEAD_DIM, kconv=synthetic.CONV_KERNEL):
    """fp32 [3 planes * H * d][kconv - 1]: the fused conv ring layout."""
    return 3 * H * d * (kconv - 1) * 4


def test_state_layout_reproduces_the_pages_budget():
    f = _facts()
    for key in ("recurrent_state_mib_k3", "recurrent_state_mib_45x32"):
        e = f[key]
        mib = e["layers"] * e["heads"] * state_bytes_per_head() / 2 ** 20
        assert round(mib) == e["value"], (key, mib)


def test_ring_layout_reproduces_the_pages_snapshot_size():
    e = _facts()["ring_snapshot_kib_64_heads"]
    assert ring_bytes_per_sequence(e["heads"]) / 1024 == e["value"]


def test_decode_mac_count():
    e = _facts()["decode_macs_per_token_layer"]
    d = synthetic.HEAD_DIM
    assert 3 * d * d * e["heads"] == e["value"]
    assert abs(e["value"] / 1e6 - e["approx_mflop"]) < 0.05


def test_constants_match_the_pages():
    f = _facts()
    assert synthetic.LOWER_BOUND == f["gate_lower_bound"]["value"]
    assert synthetic.HEAD_DIM == f["head_dim"]["value"]
    assert synthetic.CONV_KERNEL == f["conv_kernel"]["value"]
    assert synthetic.L2_EPS == f["l2_eps"]["value"]
    # the tile bound: 16 tokens at |g| <= 5 rescale by at most e^80, inside bf16/fp32 range
    assert f["tile_tokens"]["value"] * -f["gate_lower_bound"]["value"] == f["tile_rescale_log_bound"]["value"]
    assert math.exp(f["tile_rescale_log_bound"]["value"]) < np.finfo(np.float32).max


def test_oracle_regression_fixture():
    with open(os.path.join(GOLDEN, "oracle_tiny.json")) as f:
        doc = json.load(f)
    arr = {k: np.asarray(v, dtype=np.float32) for k, v in doc.items()
           if k not in ("H", "d", "seqlens") and not k.startswith("expected")}
    L = oracle.Layer(doc["H"], doc["d"], arr["conv_w"], arr["dt_bias"], arr["A_log"], arr["norm_w"])
    cu = np.concatenate([[0], np.cumsum(doc["seqlens"])])
    out, state, ring = oracle.prefill(L, oracle.F32, cu, arr["q"], arr["k"], arr["v"], arr["z"],
                                      arr["beta"], arr["gate"],
                                      arr["state_in"].astype(np.float64), arr["ring_in"])
    assert np.max(np.abs(out - np.asarray(doc["expected_out"]))) < 1e-12
    assert np.max(np.abs(state - np.asarray(doc["expected_state"]))) < 1e-12
    assert np.array_equal(ring, np.asarray(doc["expected_ring"]))
