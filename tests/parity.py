"""Whole-output parity helpers for the GPU tests (no GPU needed to import).

``reference`` runs the fp64 oracle over every (batch, head) of a workload in
a thread pool (numpy releases the GIL in its BLAS calls and array loops; BLAS
is held to one thread per worker) and returns the output with what the
per-element bar needs: the second moment of v under each row's weights, the
row's Cauchy-Schwarz score bound over its visible keys, and its visible key
count. ``assert_close`` applies the bars: every element within
``oracle.element_bar`` (1e-2, or more only where bf16 / fp32 arithmetic can
exceed it) and the whole tensor within relative L2 5e-3.
"""
from __future__ import annotations

import contextlib
import os
import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synthetic


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def reference(wl, qc, kc, vc) -> dict:
    """Oracle output of the whole workload, fp64, plus bar inputs."""
    q, k, v = (synthetic.to_f64(x) for x in (qc, kc, vc))
    bsz, heads, n, d = q.shape
    o = np.empty_like(q)
    m2 = np.empty_like(v)
    args = (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)

    def one(bh):
        b, h = bh
        ob, mb = oracle.attention_visible(q[b:b + 1, h:h + 1], k[b:b + 1, h:h + 1],
                                          v[b:b + 1, h:h + 1], *args, moments=True)
        o[b, h] = ob[0, 0]
        m2[b, h] = mb[0, 0]

    jobs = [(b, h) for b in range(bsz) for h in range(heads)]
    try:
        from threadpoolctl import threadpool_limits
        one_blas_thread = threadpool_limits(limits=1)
    except Exception:                                  # noqa: BLE001
        one_blas_thread = contextlib.nullcontext()
    with one_blas_thread, ThreadPoolExecutor(min(workers(), max(1, len(jobs)))) as ex:
        list(ex.map(one, jobs))
    sb = oracle.row_bound_by_frames(q, k, *args)
    nk = np.array([len(oracle.visible_frames(i // wl.tokens_per_frame, wl.frames, wl.window,
                                             wl.ref_frame)) * wl.tokens_per_frame for i in range(n)])
    return {"o": o, "m2": m2, "score_bound": sb, "n_keys": np.broadcast_to(nk, sb.shape),
            "head_dim": d}


def select_heads(ref: dict, sel) -> dict:
    """The reference of a head subset (every output of those heads)."""
    return {"o": ref["o"][:, sel], "m2": ref["m2"][:, sel], "score_bound": ref["score_bound"][:, sel],
            "n_keys": ref["n_keys"][:, sel], "head_dim": ref["head_dim"]}


def assert_close(got, ref: dict, what: str):
    """Every element within its bar, relative L2 within 5e-3; prints the
    figures (max-abs, rel-L2, the worst excess over the bar, how many
    elements have a bar above 1e-2 and the max-abs over those that do not)."""
    want = ref["o"]
    assert got.shape == want.shape, (what, got.shape, want.shape)
    m, r = oracle.max_abs_and_rel_l2(got, want)
    bar = oracle.element_bar(want, ref["m2"], ref["score_bound"], ref["n_keys"], ref["head_dim"])
    err = np.abs(got - want)
    excess = float((err - bar).max()) if got.size else 0.0
    wide = bar > oracle.MAX_ABS_BAR
    plain = float(err[~wide].max()) if (~wide).any() else 0.0
    _say(f"{what}: max_abs={m:.3e} rel_l2={r:.3e} worst excess over the bar={excess:.3e} "
         f"elements={got.size} bar>1e-2 on {int(wide.sum())} (max_abs elsewhere {plain:.3e})")
    assert np.isfinite(got).all(), what
    assert excess <= 0.0, (what, m, excess)
    assert r <= oracle.REL_L2_BAR, (what, r)
