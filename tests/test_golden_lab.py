"""The oracle against the values the "fp8_parity.py" lab page fixes
(tests/golden/lab_smoke_checks.json, each entry citing its place on the page)."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "lab_smoke_checks.json")))
FMT = {"E4M3": oracle.E4M3, "E5M2": oracle.E5M2}


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_format_constants(name):
    c = GOLDEN["constants"]
    f = FMT[name]
    assert oracle.fmax(f) == c["fmax"][name]
    assert oracle.smallest_normal(f) == c["smallest_normal"][name]
    finite = [v for v in oracle.decode_table(f) if np.isfinite(v)]
    assert max(finite) == c["fmax"][name]
    assert min(v for v in finite if v > 0 and v >= c["smallest_normal"][name]) == c["smallest_normal"][name]
    assert oracle.scale_from_amax(0.0, f) == np.float32(c["scale_floor"])


@pytest.mark.parametrize("name", ["E4M3", "E5M2"])
def test_check1_roundtrip(name):
    c, k1 = GOLDEN["constants"], GOLDEN["check1"]
    f = FMT[name]
    x = workloads.lab_smoke_inputs()["x"].numpy()
    assert x.size == k1["n"] and abs(x.std() - k1["std"]) < 0.2
    q, s, _ = oracle.quantize_per_tensor(x, f)
    y = (oracle.decode_array(q, f).astype(np.float32) * s).astype(np.float64)
    normal = np.abs(x / s) >= c["smallest_normal"][name]
    assert (np.abs(y - x) / np.abs(x))[normal].max() <= c["roundtrip_rel_bound"][name]


def test_check2_unscaled_cast():
    k = GOLDEN["check2"]
    big = np.array(k["input"], np.float32)
    plain = oracle.decode_array(oracle.cast(big, 1.0, oracle.E4M3), oracle.E4M3)
    with np.errstate(invalid="ignore"):
        rel = np.abs(plain - big) / np.abs(big)
    assert not np.any(rel < k["rel_err_must_not_be_below"])


def test_check3_spike():
    k, fmax = GOLDEN["check3"], GOLDEN["constants"]["fmax"]["E4M3"]
    d = workloads.lab_smoke_inputs()
    assert len(d["history"]) == k["history_len"] and d["act"].numel() == k["n"]
    act = d["act"].numpy()
    assert act[k["spike_index"]] == k["spike"]
    s_del = np.float32(max(float(np.abs(h.numpy()).max()) for h in d["history"])) / np.float32(fmax)
    y_del = oracle.decode_array(oracle.cast(act, s_del, oracle.E4M3), oracle.E4M3) * s_del
    q, s_cur, _ = oracle.quantize_per_tensor(act, oracle.E4M3)
    y_cur = oracle.decode_array(q, oracle.E4M3) * s_cur
    i = k["spike_index"]
    assert not (abs(y_del[i] - k["spike"]) < k["delayed_abs_err_must_not_be_below"])
    assert abs(y_cur[i] - k["spike"]) <= k["spike"] * k["current_rel_bound"]


def test_check4_tiles_beat_tensor():
    k = GOLDEN["check4"]
    a = workloads.lab_smoke_inputs()["a"].numpy()
    assert list(a.shape) == k["shape"]
    q, s, _ = oracle.quantize_per_tensor(a, oracle.E4M3)
    y_t = oracle.decode_array(q, oracle.E4M3) * s
    qt, st = oracle.quantize_tiles(a, 0, k["shape"][1], oracle.E4M3)
    y_r = oracle.decode_array(qt, oracle.E4M3) * st.reshape(-1, 1)
    rows = [r for r in range(k["shape"][0]) if r != k["outlier_row"]]
    assert ((y_r - a)[rows] ** 2).mean() < ((y_t - a)[rows] ** 2).mean()


def test_check5_shapes_and_gap():
    from oracle import fp8_train
    k = GOLDEN["check5"]
    d = workloads.lab_mlp_inputs()
    assert list(d["X"].shape) == k["X"] and list(d["W1"].shape) == k["W1"] and list(d["W2"].shape) == k["W2"]
    l32 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=False, steps=k["steps"], lr=k["lr"])
    l8 = fp8_train.train_mlp(d["X"], d["Y"], d["W1"], d["W2"], fp8=True, steps=k["steps"], lr=k["lr"])
    assert abs(l8[-1] - l32[-1]) / l32[-1] < k["max_rel_gap"]
