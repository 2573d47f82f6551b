"""The seeded input generators: offsets recipes, shapes, determinism."""
import numpy as np
import pytest

import workloads as wl


@pytest.mark.parametrize("idx", [1, 2, 3, 4, 5])
def test_offsets_well_formed(idx):
    w = wl.WORKLOADS[idx]
    off = wl.make_offsets(idx, np.random.default_rng(idx))
    assert off.dtype == np.int32 and off.shape == (w.E + 1,)
    assert off[0] == 0 and off[-1] == w.M and np.all(np.diff(off) >= 0)
    again = wl.make_offsets(idx, np.random.default_rng(idx))
    assert np.array_equal(off, again)


def test_fixed_offsets():
    assert list(wl.make_offsets(1, None)) == [0, 128, 256]
    assert list(np.diff(wl.make_offsets(3, None))) == [256] * 8
    assert list(np.diff(wl.make_offsets(4, None))) == [3200, 1536, 1024, 640, 512, 512, 384, 384]
    assert list(wl.zipf_units(64, 8, 1.1)) == [25, 12, 8, 5, 4, 4, 3, 3]


def test_ragged_multinomial_has_one_empty_expert():
    for seed in range(20):
        off = wl.make_offsets(2, np.random.default_rng(seed))
        counts = np.diff(off)
        assert (counts == 0).sum() >= 1 and counts.sum() == 4096


def test_many_small_units():
    for seed in range(20):
        off = wl.make_offsets(5, np.random.default_rng(seed))
        counts = np.diff(off)
        assert np.all(counts % 128 == 0)
        assert counts.min() == 0 and counts.max() == 640 and counts.sum() == 16384


def test_small_inputs_shapes_and_determinism():
    a = wl.make_wgrad_inputs(1)
    b = wl.make_wgrad_inputs(1)
    assert a["gT"].shape == (256, 256) and a["xT"].shape == (256, 256)
    assert a["gT"].flags.c_contiguous and a["gT"].dtype == np.float32
    assert np.array_equal(a["gT"], b["gT"])
    d = wl.make_dgrad_inputs(1)
    assert d["g"].shape == (256, 256) and d["W"].shape == (2, 256, 256)
    # the tiny workload's wgrad and dgrad passes share g
    assert np.array_equal(d["g"].T, a["gT"])
    d2 = wl.make_dgrad_inputs(2)
    assert d2["W"].shape == (8, 1024, 2048)
    assert abs(float(d2["W"].std()) - 1 / 32) < 1e-3
    w3 = wl.make_wgrad_inputs(3)
    assert w3["gT"].shape == (2048, 2048)


def test_forward_inputs_shapes_offsets_and_determinism():
    a = wl.make_forward_inputs(1)
    b = wl.make_forward_inputs(1)
    assert a["x"].shape == (256, 256) and a["W"].shape == (2, 256, 256)
    assert a["x"].dtype == np.float32 and a["x"].flags.c_contiguous
    assert np.array_equal(a["x"], b["x"]) and np.array_equal(a["W"], b["W"])
    # the offsets are the workload's own draw, shared with its other passes
    assert np.array_equal(wl.make_forward_inputs(2)["off"], wl.make_dgrad_inputs(2)["off"])
    assert abs(float(a["W"].std()) - 0.02) < 2e-3
