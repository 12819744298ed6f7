"""fsa_plan (C++, through the C ABI) against the oracle's brute-force plan:
bit-exact headers, row pointers and column indices."""
import ctypes
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import frame_windowed_block_amd as fsa
import oracle
from tests.conftest import GOLDEN


def _same(frames, t, w, r, bq=0, bk=0):
    info, row_ptr, col_idx = fsa.plan(frames, t, w, r, bq, bk)
    oinfo, orow, ocol = oracle.plan(frames, t, w, r, bq, bk)
    assert info.as_dict() == oinfo
    assert row_ptr.dtype == np.int32 and col_idx.dtype == np.int32
    assert row_ptr.tobytes() == orow.tobytes()
    assert col_idx.tobytes() == ocol.tobytes()
    return info


@pytest.mark.parametrize("name", ["tiny", "sr720", "sr1080", "dense"])
def test_workload_plans(name):
    import synthetic
    wl = synthetic.WORKLOADS[name]
    info = _same(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    want = {"tiny": (80, 80, 5, 5, 16), "sr720": (240, 80, 105, 315, 6000),
            "sr1080": (240, 80, 195, 585, 46575), "dense": (240, 80, 70, 210, 14700)}[name]
    assert (info.block_q, info.block_k, info.n_qblocks, info.n_kblocks, info.nnz) == want


@pytest.mark.parametrize("fname", ["plan_5x80_w1_r0.json", "plan_5x80_w1_r0_bq16.json"])
def test_golden(fname):
    with open(os.path.join(GOLDEN, fname)) as fh:
        g = json.load(fh)
    info, row_ptr, col_idx = fsa.plan(g["frames"], g["tokens_per_frame"], g["window"],
                                      g["ref_frame"], g["block_q"], g["block_k"])
    assert row_ptr.tolist() == g["row_ptr"] and col_idx.tolist() == g["col_idx"]
    assert info.nnz == g["nnz"]


@settings(max_examples=120, deadline=None)
@given(frames=st.integers(1, 9), tq=st.sampled_from([16, 32, 48, 80, 96, 144, 240]),
       w=st.integers(0, 10), rsel=st.integers(0, 1000), bsel=st.integers(0, 10_000))
def test_hypothesis_sweep(frames, tq, w, rsel, bsel):
    r = rsel % frames
    sizes = [0] + [b for b in range(16, tq + 1, 16) if tq % b == 0]
    bq = sizes[bsel % len(sizes)]
    bk = sizes[(bsel // 7) % len(sizes)]
    _same(frames, tq, w, r, bq, bk)


def test_auto_sizes_match_oracle():
    for t in (16, 32, 48, 80, 112, 240, 256, 272, 1200, 3600, 4096):
        info, _, _ = fsa.plan(1, t, 0, 0)
        assert (info.block_q, info.block_k) == oracle.auto_block_sizes(t)


@pytest.mark.parametrize("args,want", [
    ((0, 80, 1, 0), fsa.FSA_ERR_INVALID_ARG),
    ((5, 0, 1, 0), fsa.FSA_ERR_INVALID_ARG),
    ((5, 72, 1, 0), fsa.FSA_ERR_UNALIGNED),
    ((5, 8, 1, 0), fsa.FSA_ERR_UNALIGNED),
    ((5, 80, -1, 0), fsa.FSA_ERR_INVALID_ARG),
    ((5, 80, 1, 5), fsa.FSA_ERR_INVALID_ARG),
    ((5, 80, 1, -1), fsa.FSA_ERR_INVALID_ARG),
    ((5, 80, 1, 0, 32, 16), fsa.FSA_ERR_UNALIGNED),
    ((5, 80, 1, 0, 16, 24), fsa.FSA_ERR_UNALIGNED),
    ((5, 80, 1, 0, -16, 16), fsa.FSA_ERR_INVALID_ARG),
    ((2**20, 2**12, 1, 0), fsa.FSA_ERR_INVALID_ARG),       # N overflows int32
])
def test_plan_rejects(args, want):
    with pytest.raises(fsa.FsaError) as ei:
        fsa.plan(*args)
    assert ei.value.status == want


def test_buffer_too_small_and_sizing():
    L = fsa.lib()
    info = fsa.PlanInfo()
    assert L.fsa_plan(5, 80, 1, 0, 0, 0, ctypes.byref(info), None, 0, None, 0) == 0
    assert info.nnz == 16 and info.n_qblocks == 5
    rp = np.full(6, -7, dtype=np.int32)
    ci = np.full(15, -7, dtype=np.int32)
    P = ctypes.POINTER(ctypes.c_int32)
    st = L.fsa_plan(5, 80, 1, 0, 0, 0, ctypes.byref(info), rp.ctypes.data_as(P), 6,
                    ci.ctypes.data_as(P), 15)
    assert st == fsa.FSA_ERR_BUFFER_TOO_SMALL
    assert np.all(rp == -7) and np.all(ci == -7)
    st = L.fsa_plan(5, 80, 1, 0, 0, 0, ctypes.byref(info), rp.ctypes.data_as(P), 6, None, 0)
    assert st == fsa.FSA_ERR_INVALID_ARG
    assert L.fsa_plan(5, 80, 1, 0, 0, 0, None, None, 0, None, 0) == fsa.FSA_ERR_INVALID_ARG


def test_large_window_and_single_frame():
    _same(1, 16, 0, 0)
    _same(3, 16, 2**30, 2)
    info = _same(14, 1200, 13, 0)
    assert info.nnz == info.n_qblocks * info.n_kblocks


@pytest.mark.parametrize("r", [0, 2, 3])
def test_largest_window_is_dense(r):
    """w = 2^31 - 1 (no overflow in the frame arithmetic) lists every key block
    of every row, the same plan as w = F - 1."""
    info = _same(4, 48, 2**31 - 1, r, 48, 16)
    dense, drow, dcol = fsa.plan(4, 48, 3, r, 48, 16)
    _, row_ptr, col_idx = fsa.plan(4, 48, 2**31 - 1, r, 48, 16)
    assert info.nnz == info.n_qblocks * info.n_kblocks == dense.nnz
    assert row_ptr.tobytes() == drow.tobytes() and col_idx.tobytes() == dcol.tobytes()
