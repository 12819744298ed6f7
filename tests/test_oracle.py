"""The CPU oracle against its pins (hand-worked goldens, brute force, torch,
mpmath, closed forms, invariances) and against the synthetic workloads."""
import math

import numpy as np
import pytest

import oracle
import synthetic
from tests import oracle_pins


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda c: c.__name__)
def test_pin(check):
    check(oracle)


def test_auto_block_sizes():
    assert oracle.auto_block_sizes(80) == (80, 80)
    assert oracle.auto_block_sizes(1200) == (240, 80)
    assert oracle.auto_block_sizes(3600) == (240, 80)
    assert oracle.auto_block_sizes(16) == (16, 16)
    assert oracle.auto_block_sizes(4096) == (256, 128)
    assert oracle.aligned_block_sizes(1200) == [16, 48, 80, 240, 400, 1200]


def test_plan_rejects():
    with pytest.raises(ValueError):
        oracle.plan(5, 72, 1, 0)            # T not a multiple of 16
    with pytest.raises(ValueError):
        oracle.plan(5, 80, 1, 5)            # reference frame out of range
    with pytest.raises(ValueError):
        oracle.plan(5, 80, 1, 0, 32, 16)    # 32 does not divide 80
    with pytest.raises(ValueError):
        oracle.plan(0, 80, 1, 0)


def test_tiny_workload_bound_path_exact():
    """The tiny workload: bound-shift and max-subtract agree in fp64 and every
    head is eligible."""
    wl = synthetic.WORKLOADS["tiny"]
    q, k, v = (synthetic.to_f64(t) for t in synthetic.make_inputs(wl))
    args = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
    bnd = oracle.bounds(q, k, *args)
    assert bnd["eligible"].tolist() == [[1, 1]]
    a = oracle.attention(q, k, v, *args)
    b = oracle.attention_bound_shift(q, k, v, *args, bnd["row_bound"])
    assert np.abs(a - b).max() < 1e-12
    rows = synthetic.sample_rows(wl, 40)
    np.testing.assert_allclose(oracle.attention_rows(q, k, v, rows, *args),
                               np.stack([a[b_, h, i] for b_, h, i in rows]), rtol=0, atol=1e-13)


@pytest.mark.slow
@pytest.mark.parametrize("name", ["sr720", "sr1080", "dense"])
def test_large_workload_bound_shift_rows(name):
    """On the N(0,1) workloads the largest row bound stays below 32, and the
    bound-shift form equals max-subtract within 1e-12 on sampled rows."""
    wl = synthetic.WORKLOADS[name]
    q, k, v = (synthetic.to_f64(t) for t in synthetic.make_inputs(wl))
    args = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
    bnd = oracle.bounds(q, k, *args)
    assert np.all(bnd["eligible"] == 1)
    assert 10.0 < bnd["bmax"].max() < 32.0
    rows = synthetic.sample_rows(wl, 24)
    a = oracle.attention_rows(q, k, v, rows, *args)
    b = oracle.attention_rows(q, k, v, rows, *args, row_bound=bnd["row_bound"])
    assert np.abs(a - b).max() < 1e-12


@pytest.mark.slow
def test_bound_stress_is_ineligible():
    """The heavy-tailed workload pushes every head's bound far above 32, and the
    fp64 bound-shift form underflows on most rows (the hazard the online
    fallback covers)."""
    wl = synthetic.WORKLOADS["bound_stress"]
    q, k, v = (synthetic.to_f64(t) for t in synthetic.make_inputs(wl))
    args = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
    bnd = oracle.bounds(q, k, *args)
    assert np.all(bnd["eligible"] == 0)
    assert bnd["bmax"].min() > 1e3
    rows = synthetic.sample_rows(wl, 24)
    with np.errstate(all="ignore"):
        b = oracle.attention_rows(q, k, v, rows, *args, row_bound=bnd["row_bound"])
    assert np.isnan(b).any()


@pytest.mark.slow
def test_key_offset_centring_restores_eligibility():
    """Keys sharing a 40-long offset push every plain bound above 32; centring
    the keys brings it back under 32, and the centred shift equals
    max-subtract within 1e-12 on sampled rows."""
    wl = synthetic.WORKLOADS["key_offset"]
    q, k, v = (synthetic.to_f64(t) for t in synthetic.make_inputs(wl))
    args = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)
    plain = oracle.bounds(q, k, *args)
    cent = oracle.bounds(q, k, *args, center=True)
    assert np.all(plain["eligible"] == 0) and plain["bmax"].min() > 40.0
    assert np.all(cent["eligible"] == 1) and cent["bmax"].max() < 25.0
    rows = synthetic.sample_rows(wl, 24)
    a = oracle.attention_rows(q, k, v, rows, *args)
    b = oracle.attention_rows(q, k, v, rows, *args, row_bound=cent["row_shift"])
    assert np.abs(a - b).max() < 1e-12


def test_active_flops():
    assert oracle.active_flops(1, 2, 64, 5, 80, 1, 0) == 52_428_800
    assert oracle.active_flops(1, 8, 128, 21, 1200, 1, 0) == 471_859_200_000
    assert oracle.active_flops(1, 8, 128, 13, 3600, 2, 0) == 3_662_807_040_000
    assert oracle.active_flops(1, 8, 128, 14, 1200, 13, 0) == 1_156_055_040_000


def test_metrics():
    ref = np.array([1.0, -2.0, 2.0])
    got = np.array([1.0, -2.0, 2.03])
    m, r = oracle.max_abs_and_rel_l2(got, ref)
    assert abs(m - 0.03) < 1e-12 and abs(r - 0.01) < 1e-12
