"""Pin checks for the CPU oracle, written against an oracle namespace.

Each ``check_*`` function raises AssertionError when the oracle it is given
disagrees with something fixed independently of it: values worked by hand
(``tests/golden/``), brute force with Python loops, a library routine
(``torch``'s scaled-dot-product attention), mpmath at 50 digits, closed forms
and invariances. ``test_oracle.py`` runs them on the real oracle, and
``test_oracle_mutants.py`` runs them on copies of the oracle with planted
mistakes, each of which must be caught by at least one check.

Nothing here imports the HIP library.
"""
from __future__ import annotations

import itertools
import json
import math
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def _rand(shape, seed):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float64).numpy()


# ---------------------------------------------------------------- brute force
def brute_visible(f, frames, window, ref_frame):
    """Independent restatement of the mask rule with explicit loops."""
    out = []
    for g in range(frames):
        if abs(g - f) <= window or g == ref_frame:
            out.append(g)
    return out


def brute_attention(q, k, v, frames, t, window, ref_frame, scale, moments=False):
    """Masked softmax attention with Python loops and math.exp (tiny inputs);
    with ``moments`` also the weighted mean of v squared."""
    bsz, heads, n, d = q.shape
    o = np.zeros_like(q)
    m2 = np.zeros_like(q)
    for b in range(bsz):
        for h in range(heads):
            for i in range(n):
                vis = brute_visible(i // t, frames, window, ref_frame)
                keys = [j for j in range(n) if (j // t) in vis]
                s = [scale * sum(q[b, h, i, c] * k[b, h, j, c] for c in range(d)) for j in keys]
                m = max(s)
                w = [math.exp(x - m) for x in s]
                z = sum(w)
                for c in range(d):
                    o[b, h, i, c] = sum(wj * v[b, h, j, c] for wj, j in zip(w, keys)) / z
                    m2[b, h, i, c] = sum(wj * v[b, h, j, c] ** 2 for wj, j in zip(w, keys)) / z
    return (o, m2) if moments else o


def check_golden_attention(orc):
    g = _load("attention_hand_worked.json")
    q = np.array(g["q"])[None, None]
    k = np.array(g["k"])[None, None]
    v = np.array(g["v"])[None, None]
    for case in g["cases"]:
        o = orc.attention(q, k, v, case["frames"], case["tokens_per_frame"], case["window"],
                          case["ref_frame"], g["scale"])
        np.testing.assert_allclose(o[0, 0], np.array(case["o"]), rtol=0, atol=1e-12)


def check_golden_plans(orc):
    for name in ("plan_5x80_w1_r0.json", "plan_5x80_w1_r0_bq16.json"):
        g = _load(name)
        info, row_ptr, col_idx = orc.plan(g["frames"], g["tokens_per_frame"], g["window"],
                                          g["ref_frame"], g["block_q"], g["block_k"])
        for key in ("n_qblocks", "n_kblocks", "nnz", "block_q", "block_k"):
            assert info[key] == g[key], (name, key)
        assert row_ptr.tolist() == g["row_ptr"], name
        assert col_idx.tolist() == g["col_idx"], name


BRUTE_CASES = [
    # frames, T, D, window, ref
    (1, 16, 8, 0, 0),
    (2, 16, 8, 1, 1),
    (3, 16, 8, 0, 0),
    (4, 16, 16, 1, 0),
    (4, 32, 8, 2, 3),
    (4, 16, 8, 5, 3),
    (3, 32, 16, 0, 2),
    (4, 16, 8, 1, 2),
]


def check_brute_force(orc, cases=BRUTE_CASES):
    for idx, (frames, t, d, w, r) in enumerate(cases):
        n = frames * t
        q, k, v = (_rand((1, 2, n, d), 100 * idx + s) for s in range(3))
        scale = 1.0 / math.sqrt(d)
        ref, ref_m2 = brute_attention(q, k, v, frames, t, w, r, scale, moments=True)
        got = orc.attention(q, k, v, frames, t, w, r, scale)
        np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
        # the same definition over the visible keys only, and the second moment
        for fn in (orc.attention, orc.attention_visible):
            got, got_m2 = fn(q, k, v, frames, t, w, r, scale, moments=True)
            np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)
            np.testing.assert_allclose(got_m2, ref_m2, rtol=0, atol=1e-12)
        np.testing.assert_allclose(orc.attention_visible(q, k, v, frames, t, w, r, scale), ref,
                                   rtol=0, atol=1e-12)
        rows = [(0, 1, 0), (0, 0, n - 1), (0, 1, n // 2)]
        got_rows = orc.attention_rows(q, k, v, rows, frames, t, w, r, scale)
        for x, (b, h, i) in enumerate(rows):
            np.testing.assert_allclose(got_rows[x], ref[b, h, i], rtol=0, atol=1e-12)


def check_weights(orc):
    frames, t, d, w, r = 4, 16, 8, 1, 2
    n = frames * t
    q, k = _rand((1, 2, n, d), 7), _rand((1, 2, n, d), 8)
    p = orc.attention_weights(q, k, frames, t, w, r, 1.0 / math.sqrt(d))
    np.testing.assert_allclose(p.sum(-1), 1.0, rtol=0, atol=1e-12)
    # each row equals the brute-force weights, exp(s - max) / sum, scale included
    for b_h in range(2):
        for i in (0, t - 1, n // 2, n - 1):
            vis = brute_visible(i // t, frames, w, r)
            keys = [j for j in range(n) if (j // t) in vis]
            s = [sum(q[0, b_h, i, c] * k[0, b_h, j, c] for c in range(d)) / math.sqrt(d) for j in keys]
            e = [math.exp(x - max(s)) for x in s]
            np.testing.assert_allclose(p[0, b_h, i, keys], np.array(e) / sum(e), rtol=0, atol=1e-13)
    for i in range(n):
        vis = brute_visible(i // t, frames, w, r)
        for j in range(n):
            if (j // t) not in vis:
                assert p[0, 0, i, j] == 0.0 and p[0, 1, i, j] == 0.0
            else:
                assert p[0, 0, i, j] > 0.0


def check_dense_limit(orc):
    """Window >= F - 1 makes the mask all-ones: plain attention (torch, fp64)."""
    frames, t, d = 3, 16, 16
    n = frames * t
    q, k, v = (_rand((1, 2, n, d), 20 + s) for s in range(3))
    scale = 1.0 / math.sqrt(d)
    want = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q), torch.from_numpy(k), torch.from_numpy(v), scale=scale).numpy()
    for w in (frames - 1, frames + 4):
        got = orc.attention(q, k, v, frames, t, w, 1, scale)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)
    info, row_ptr, col_idx = orc.plan(frames, t, frames - 1, 0, 16, 16)
    assert info["nnz"] == info["n_qblocks"] * info["n_kblocks"]


def check_closed_forms(orc):
    frames, t, d, w, r = 5, 16, 5, 1, 0
    n = frames * t
    scale = 0.25
    rng_v = _rand((1, 1, n, d), 30)
    zero_q = np.zeros((1, 1, n, d))
    k = _rand((1, 1, n, d), 31)
    # q = 0: uniform weights over the visible keys -> mean of v over them; B_i = 0
    o = orc.attention(zero_q, k, rng_v, frames, t, w, r, scale)
    for i in range(n):
        vis = brute_visible(i // t, frames, w, r)
        keys = [j for j in range(n) if j // t in vis]
        np.testing.assert_allclose(o[0, 0, i], rng_v[0, 0, keys].mean(0), rtol=0, atol=1e-12)
    bnd = orc.bounds(zero_q, k, frames, t, w, r, scale, 16, 16)
    assert np.all(bnd["row_bound"] == 0.0) and np.all(bnd["qnorm"] == 0.0)
    # constant v rows -> that constant
    q = _rand((1, 1, n, d), 32)
    const_v = np.broadcast_to(np.array([1.5, -2.0, 0.0, 3.25, 7.0]), (1, 1, n, d)).copy()
    o = orc.attention(q, k, const_v, frames, t, w, r, scale)
    np.testing.assert_allclose(o, const_v, rtol=0, atol=1e-12)
    for fn in (orc.attention, orc.attention_visible):
        o, m2 = fn(q, k, const_v, frames, t, w, r, scale, moments=True)
        np.testing.assert_allclose(o, const_v, rtol=0, atol=1e-12)
        np.testing.assert_allclose(m2, const_v ** 2, rtol=1e-13, atol=1e-12)
    # frame-indicator v: column c = [frame(j) == c] -> attention mass per frame
    ind_v = np.zeros((1, 1, n, frames))
    for j in range(n):
        ind_v[0, 0, j, j // t] = 1.0
    o = orc.attention(q[..., :frames], k[..., :frames], ind_v, frames, t, w, r, scale)
    np.testing.assert_allclose(o.sum(-1), 1.0, rtol=0, atol=1e-12)
    for i in range(n):
        vis = brute_visible(i // t, frames, w, r)
        for c in range(frames):
            if c not in vis:
                assert o[0, 0, i, c] == 0.0
    o0 = orc.attention(zero_q[..., :frames], k[..., :frames], ind_v, frames, t, w, r, scale)
    for i in range(n):
        vis = brute_visible(i // t, frames, w, r)
        for c in vis:
            assert abs(o0[0, 0, i, c] - 1.0 / len(vis)) < 1e-12


def check_bound_shift_exact(orc):
    """Norm-bound softmax equals max-subtract softmax: mpmath at 50 digits on a
    tiny case (the identity itself), then the oracle's fp64 bound-shift form."""
    import mpmath
    mpmath.mp.dps = 50
    frames, t, d, w, r = 3, 2, 4, 0, 0
    n = frames * t
    q, k, v = (_rand((1, 1, n, d), 40 + s) for s in range(3))
    scale = 0.5
    bnd = orc.bounds(np.zeros((1, 1, 16 * frames, d)), np.zeros((1, 1, 16 * frames, d)),
                     frames, 16, w, r, scale, 16, 16)      # exercised for shape only
    assert bnd["bmax"].shape == (1, 1)
    for i in range(n):
        vis = brute_visible(i // t, frames, w, r)
        keys = [j for j in range(n) if j // t in vis]
        s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[0, 0, i, c]) * mpmath.mpf(k[0, 0, j, c])
                                             for c in range(d)) for j in keys]
        qn = mpmath.sqrt(mpmath.fsum(mpmath.mpf(x) ** 2 for x in q[0, 0, i]))
        kn = max(mpmath.sqrt(mpmath.fsum(mpmath.mpf(x) ** 2 for x in k[0, 0, j])) for j in keys)
        bound = mpmath.mpf(scale) * qn * kn
        assert all(x <= bound for x in s)
        m = max(s)
        for c in range(d):
            a = mpmath.fsum(mpmath.exp(x - m) * mpmath.mpf(v[0, 0, j, c]) for x, j in zip(s, keys)) \
                / mpmath.fsum(mpmath.exp(x - m) for x in s)
            b = mpmath.fsum(mpmath.exp(x - bound) * mpmath.mpf(v[0, 0, j, c]) for x, j in zip(s, keys)) \
                / mpmath.fsum(mpmath.exp(x - bound) for x in s)
            assert abs(a - b) < mpmath.mpf("1e-40")
    # fp64: the oracle's bound-shift form against its max-subtract form
    frames, t, d, w, r = 4, 16, 16, 1, 0
    n = frames * t
    q, k, v = (_rand((1, 2, n, d), 50 + s) for s in range(3))
    scale = 1.0 / math.sqrt(d)
    bnd = orc.bounds(q, k, frames, t, w, r, scale, 16, 16)
    a = orc.attention(q, k, v, frames, t, w, r, scale)
    b = orc.attention_bound_shift(q, k, v, frames, t, w, r, scale, bnd["row_bound"])
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)


def check_cauchy_schwarz(orc):
    frames, t, d, w, r = 4, 32, 8, 1, 3
    n = frames * t
    q, k = _rand((1, 2, n, d), 60), _rand((1, 2, n, d), 61)
    k[0, 1, 5] *= 30.0          # one long key in frame 0
    scale = 0.3
    mask = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            mask[i, j] = (j // t) in brute_visible(i // t, frames, w, r)
    s = scale * np.einsum("bhid,bhjd->bhij", q, k)
    ref_bound = None
    for bq, bk in ((16, 16), (16, 32), (32, 16), (32, 32)):
        bnd = orc.bounds(q, k, frames, t, w, r, scale, bq, bk)
        rb = bnd["row_bound"]
        assert np.all(np.where(mask, s <= rb[..., None] * (1 + 1e-12), True))
        # tight: the row bound uses the largest visible key norm, no other
        qn = np.sqrt((q * q).sum(-1))
        kn = np.sqrt((k * k).sum(-1))
        want = np.empty_like(qn)
        for i in range(n):
            want[:, :, i] = scale * qn[:, :, i] * np.where(mask[i], kn, 0.0).max(-1)
        np.testing.assert_allclose(rb, want, rtol=1e-14, atol=0)
        if ref_bound is not None:
            np.testing.assert_array_equal(rb, ref_bound)
        ref_bound = rb
        np.testing.assert_allclose(bnd["bmax"], want.max(-1), rtol=1e-14, atol=0)
        np.testing.assert_allclose(
            bnd["kmax"], kn.reshape(1, 2, n // bk, bk).max(-1), rtol=1e-15, atol=0)
    np.testing.assert_allclose(orc.row_bound_by_frames(q, k, frames, t, w, r, scale), ref_bound,
                               rtol=1e-14, atol=0)
    # eligibility: head 1 holds the long key, so its bound exceeds a limit head 0 meets
    limit = float(ref_bound[0, 0].max()) * 1.01
    bnd = orc.bounds(q, k, frames, t, w, r, scale, 16, 16, bound_limit=limit)
    assert bnd["eligible"].tolist() == [[1, 0]]


def plan_nnz_closed_form(frames, t, w, r, bq, bk):
    pairs = 0
    for f in range(frames):
        pairs += len(brute_visible(f, frames, w, r))
    return pairs * (t // bq) * (t // bk)


def check_plan_closed_form(orc):
    for frames, t, w, r in ((5, 80, 1, 0), (21, 1200, 1, 0), (13, 3600, 2, 0), (14, 1200, 13, 0),
                            (6, 48, 2, 5), (3, 16, 0, 1), (1, 32, 0, 0)):
        sizes = [b for b in range(16, t + 1, 16) if t % b == 0]
        if frames * t > 4000:       # brute force costs ~N^2 per plan: two plans only
            combos = [orc.auto_block_sizes(t), (sizes[-1], sizes[0])]
        else:
            picks = sorted({sizes[0], sizes[-1], sizes[len(sizes) // 2]})
            combos = list(itertools.product(picks, picks))
        for bq, bk in combos:
            info, row_ptr, col_idx = orc.plan(frames, t, w, r, bq, bk)
            assert info["nnz"] == plan_nnz_closed_form(frames, t, w, r, bq, bk)
            assert row_ptr[-1] == info["nnz"] == len(col_idx)
            # every listed block is inside the mask, keys ascending per row
            for qb in range(info["n_qblocks"]):
                kbs = col_idx[row_ptr[qb]:row_ptr[qb + 1]]
                assert np.all(np.diff(kbs) > 0)
                f = qb * bq // t
                vis = brute_visible(f, frames, w, r)
                assert all((kb * bk) // t in vis for kb in kbs)
    pairs = {(5, 1, 0): 16, (21, 1, 0): 80, (13, 2, 0): 69, (14, 13, 0): 196}
    for (frames, w, r), want in pairs.items():
        assert sum(len(brute_visible(f, frames, w, r)) for f in range(frames)) == want
        assert orc.active_pairs(frames, 16, w, r) == want * 256


def check_plan_negative_control(orc):
    """128-token blocks on 1200-token frames straddle frame edges: partial blocks."""
    cls = orc.block_classes(21, 1200, 1, 0, 128, 128)
    assert (cls == 2).sum() > 0
    cls = orc.block_classes(21, 1200, 1, 0, 240, 80)
    assert (cls == 2).sum() == 0


def check_invariances(orc):
    frames, t, d, w, r = 4, 16, 8, 1, 0
    n = frames * t
    q, k, v = (_rand((1, 3, n, d), 70 + s) for s in range(3))
    scale = 0.35
    base = orc.attention(q, k, v, frames, t, w, r, scale)
    # permuting keys (with their values) inside each frame leaves o unchanged
    perm = np.concatenate([f * t + np.random.default_rng(f).permutation(t) for f in range(frames)])
    o = orc.attention(q, k[:, :, perm], v[:, :, perm], frames, t, w, r, scale)
    np.testing.assert_allclose(o, base, rtol=0, atol=1e-12)
    # heads are independent: any head subset computed alone gives the same rows
    for sel in ([0], [2], [1, 2]):
        o = orc.attention(q[:, sel], k[:, sel], v[:, sel], frames, t, w, r, scale)
        np.testing.assert_array_equal(o, base[:, sel])
    # moving keys across a frame edge changes the result (the mask is not key-symmetric)
    perm2 = np.arange(n)
    perm2[[t - 1, t]] = perm2[[t, t - 1]]
    o = orc.attention(q, k[:, :, perm2], v[:, :, perm2], frames, t, 0, 3, scale)
    o0 = orc.attention(q, k, v, frames, t, 0, 3, scale)
    assert np.abs(o - o0).max() > 1e-6


def check_centering(orc):
    """Key mean-centring [vi:Softmax] on keys whose mean and centred lengths are
    known by construction: a shared offset mu0 of length 40 plus deviations
    +dev_j (first half of the keys) and -dev_j (second half), so the mean is
    exactly mu0 and ||k_j - mu0|| is the drawn length. The pairs straddle every
    block, so a per-block mean would differ from mu0."""
    frames, t, d, w, r = 4, 32, 8, 1, 2
    n = frames * t
    scale = 0.3
    rng = np.random.default_rng(5)
    mu0 = rng.standard_normal((1, 2, d))
    mu0 *= 40.0 / np.linalg.norm(mu0, axis=-1, keepdims=True)
    u = rng.standard_normal((1, 2, n // 2, d))
    u /= np.linalg.norm(u, axis=-1, keepdims=True)
    length = rng.uniform(0.5, 2.0, (1, 2, n // 2))
    dev = u * length[..., None]
    k = mu0[:, :, None, :] + np.concatenate([dev, -dev], axis=2)
    klen = np.concatenate([length, length], axis=2)
    q, v = _rand((1, 2, n, d), 90), _rand((1, 2, n, d), 91)
    for bq, bk in ((16, 16), (32, 16), (16, 32)):
        c = orc.bounds(q, k, frames, t, w, r, scale, bq, bk, center=True)
        np.testing.assert_allclose(c["kmean"], mu0, rtol=0, atol=1e-12)
        np.testing.assert_allclose(c["kmax"], klen.reshape(1, 2, n // bk, bk).max(-1),
                                   rtol=1e-10, atol=0)
        for h in range(2):
            for i in range(n):
                vis = brute_visible(i // t, frames, w, r)
                on = np.array([(j // t) in vis for j in range(n)])
                qi = q[0, h, i]
                bprime = scale * math.sqrt(sum(x * x for x in qi)) * klen[0, h, on].max()
                shift = scale * sum(a * b for a, b in zip(qi, mu0[0, h])) + bprime
                assert abs(c["row_bound"][0, h, i] - bprime) <= 1e-10 * bprime
                assert abs(c["row_shift"][0, h, i] - shift) <= 1e-9 * (abs(shift) + 1.0)
                s = scale * (k[0, h] @ qi)
                assert np.all(s[on] <= c["row_shift"][0, h, i] + 1e-9)
                assert np.all(s[on] >= c["row_shift"][0, h, i] - 2.0 * bprime - 1e-9)
    # the offset makes the plain bound loose; centring makes it tight enough
    plain = orc.bounds(q, k, frames, t, w, r, scale, 16, 16)
    c = orc.bounds(q, k, frames, t, w, r, scale, 16, 16, center=True)
    assert plain["eligible"].tolist() == [[0, 0]] and c["eligible"].tolist() == [[1, 1]]
    assert np.all(plain["kmean"] == 0.0) and np.array_equal(plain["row_shift"], plain["row_bound"])
    # the shifted softmax is the max-subtract softmax
    a = orc.attention(q, k, v, frames, t, w, r, scale)
    b = orc.attention_bound_shift(q, k, v, frames, t, w, r, scale, c["row_shift"])
    np.testing.assert_allclose(b, a, rtol=0, atol=1e-12)
    # translating every key by a vector moves the mean and the shift, not the bound
    off = 10.0 * rng.standard_normal((1, 2, d))
    c2 = orc.bounds(q, k + off[:, :, None, :], frames, t, w, r, scale, 16, 16, center=True)
    np.testing.assert_allclose(c2["kmean"], c["kmean"] + off, rtol=0, atol=1e-11)
    for key in ("kmax", "row_bound", "bmax"):
        np.testing.assert_allclose(c2[key], c[key], rtol=1e-9, atol=0)
    np.testing.assert_allclose(c2["row_shift"] - c["row_shift"],
                               scale * np.einsum("bhnd,bhd->bhn", q, off), rtol=0, atol=1e-9)
    # keys that already have mean zero: centring changes nothing
    k0 = np.concatenate([dev, -dev], axis=2)
    c0 = orc.bounds(q, k0, frames, t, w, r, scale, 16, 16, center=True)
    p0 = orc.bounds(q, k0, frames, t, w, r, scale, 16, 16)
    np.testing.assert_allclose(c0["kmean"], 0.0, rtol=0, atol=1e-15)
    for key in ("kmax", "row_bound", "row_shift", "bmax"):
        np.testing.assert_allclose(c0[key], p0[key], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- pre-attention
def brute_pre_attention(x, gain, w, heads, head_dim, eps, base):
    """RMS norm, projection, rotary embedding and head packing with Python loops."""
    bsz, n, c = x.shape
    out = [np.zeros((bsz, heads, n, head_dim)) for _ in range(3)]
    half = head_dim // 2
    for b in range(bsz):
        for t in range(n):
            ms = sum(x[b, t, i] ** 2 for i in range(c)) / c
            xn = [x[b, t, i] / math.sqrt(ms + eps) * gain[i] for i in range(c)]
            y = [sum(w[o, i] * xn[i] for i in range(c)) for o in range(3 * heads * head_dim)]
            for part in range(3):
                for h in range(heads):
                    row = y[(part * heads + h) * head_dim:(part * heads + h + 1) * head_dim]
                    for j in range(head_dim):
                        out[part][b, h, t, j] = row[j]
                    if part == 2:
                        continue
                    for j in range(half):
                        a = t * base ** (-2.0 * j / head_dim)
                        lo, hi = row[j], row[j + half]
                        out[part][b, h, t, j] = lo * math.cos(a) - hi * math.sin(a)
                        out[part][b, h, t, j + half] = hi * math.cos(a) + lo * math.sin(a)
    return out


def check_pre_attention(orc):
    """The fused pre-attention chain [vi:Layout]: brute force, a hand-derived
    rotary embedding, head packing by construction, and the invariances of the
    normalisation and of the rotation."""
    # brute force on tiny shapes
    for seed, (bsz, n, c, heads, d, eps, base) in enumerate(
            [(1, 3, 4, 1, 2, 1e-6, 10000.0), (2, 4, 6, 2, 4, 1e-3, 100.0), (1, 5, 8, 1, 8, 0.0, 10000.0)]):
        x = _rand((bsz, n, c), 300 + seed)
        gain = 0.5 + np.abs(_rand((c,), 310 + seed))
        w = _rand((3 * heads * d, c), 320 + seed)
        want = brute_pre_attention(x, gain, w, heads, d, eps, base)
        got = orc.pre_attention(x, gain, w, heads, d, eps, base)
        for a, b in zip(got, want):
            np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # rotary embedding of hand-derived cases (D = 4, position 2)
    g = _load("rope_d4_p2.json")
    t = np.zeros((1, 1, 3, 4))
    for case in g["cases"]:
        t[0, 0, 2] = case["in"]
        np.testing.assert_allclose(orc.rope(t, g["base"])[0, 0, 2], case["out"], rtol=0, atol=2e-9)
    # head packing: constant tokens, W row o = (o + 1) e_0, one token (no rotation)
    heads, d, c = 3, 4, 5
    w = np.zeros((3 * heads * d, c))
    w[:, 0] = np.arange(1, 3 * heads * d + 1)
    q, k, v = orc.pre_attention(np.ones((2, 1, c)), np.ones(c), w, heads, d, 0.0)
    for part, t in enumerate((q, k, v)):
        for h in range(heads):
            np.testing.assert_allclose(t[:, h, 0], np.broadcast_to(
                part * heads * d + h * d + 1 + np.arange(d), (2, d)), rtol=0, atol=1e-12)
    # normalisation: identity projection shows x / rms(x) * gain; scale-free at eps = 0
    heads, d = 2, 4
    c = heads * d
    x = _rand((1, 6, c), 330)
    gain = 0.5 + np.abs(_rand((c,), 331))
    w = np.concatenate([np.eye(c)] * 3)
    _, _, v = orc.pre_attention(x, gain, w, heads, d, 0.0)
    vv = v.transpose(0, 2, 1, 3).reshape(1, 6, c)
    np.testing.assert_allclose((vv / gain) ** 2 @ np.ones(c), c, rtol=1e-12)
    np.testing.assert_allclose(vv / gain * np.sqrt((x * x).mean(-1, keepdims=True)), x, rtol=0, atol=1e-12)
    for a, b in zip(orc.pre_attention(7.5 * x, gain, w, heads, d, 0.0),
                    orc.pre_attention(x, gain, w, heads, d, 0.0)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # rotation: pair norms are kept, and with the same token at every position
    # q_n . k_m depends on n - m only
    w = _rand((3 * heads * d, c), 332)
    row = _rand((1, 1, c), 333)
    xs = np.repeat(row, 7, axis=1)
    q, k, v = orc.pre_attention(xs, np.ones(c), w, heads, d, 1e-6)
    half = d // 2
    pn = q[..., :half] ** 2 + q[..., half:] ** 2
    np.testing.assert_allclose(pn, np.broadcast_to(pn[:, :, :1], pn.shape), rtol=1e-12)
    for h in range(heads):
        dots = q[0, h] @ k[0, h].T
        for s_ in range(-6, 7):
            diag = np.diagonal(dots, offset=s_)
            np.testing.assert_allclose(diag, diag[0], rtol=0, atol=1e-11)
    # v is not rotated: the same token gives the same v at every position
    np.testing.assert_allclose(v, np.broadcast_to(v[:, :, :1], v.shape), rtol=0, atol=1e-12)
    # a norm gain folded into the weight gives the same outputs (the form the
    # kernel takes): (r x * g) W^T = r x (W diag g)^T
    x = _rand((2, 5, c), 335)
    gain = 0.5 + np.abs(_rand((c,), 336))
    for a, b in zip(orc.pre_attention(x, gain, w, heads, d, 1e-6),
                    orc.pre_attention(x, np.ones(c), w * gain[None, :], heads, d, 1e-6)):
        np.testing.assert_allclose(a, b, rtol=0, atol=1e-12)
    # a subset of tokens with their positions gives the same rows
    x = _rand((2, 9, c), 334)
    full = orc.pre_attention(x, gain, w, heads, d, 1e-6)
    sel = np.array([8, 0, 5])
    part = orc.pre_attention(x[:, sel], gain, w, heads, d, 1e-6, positions=sel)
    for a, b in zip(part, full):
        np.testing.assert_allclose(a, b[:, :, sel], rtol=0, atol=1e-12)
    # q at position 0 is the plain projection of the normalised token
    xn = row[0, 0] / np.sqrt((row[0, 0] ** 2).mean() + 1e-6)
    np.testing.assert_allclose(q[0, :, 0].reshape(-1), w[:heads * d] @ xn, rtol=0, atol=1e-12)


def _bf16(x):
    """Round to bf16 (RNE) and back to fp32."""
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float32).numpy()


def emulate_bf16_kernel(q, k, v, frames, t, window, ref_frame, scale, shift="bound"):
    """Masked attention in the arithmetic of a bf16 MFMA kernel, emulated with
    numpy fp32 on bf16-valued inputs (independent of the oracle): fp32 scores,
    weights exp2(s c - shift) with c = scale log2(e), rounded to bf16; values
    accumulated in fp32 sixteen keys at a time, the row sum of the same bf16
    weights in fp32 pairs; o = O / l rounded to bf16. ``shift`` is the row's
    Cauchy-Schwarz bound times log2(e) ("bound") or the row max ("max")."""
    f32 = np.float32
    bsz, heads, n, d = q.shape
    c = f32(f32(scale) * f32(math.log2(math.e)))
    out = np.zeros(q.shape)
    qf, kf, vf = (np.asarray(x, dtype=np.float32) for x in (q, k, v))
    for b in range(bsz):
        for h in range(heads):
            kn = np.sqrt((kf[b, h].astype(np.float64) ** 2).sum(-1)).astype(np.float32)
            for i in range(n):
                keys = [j for j in range(n) if (j // t) in brute_visible(i // t, frames, window, ref_frame)]
                sc = (kf[b, h, keys] @ qf[b, h, i]).astype(np.float32)
                if shift == "bound":
                    qn = f32(np.sqrt((qf[b, h, i].astype(np.float64) ** 2).sum()))
                    sh = f32(c * f32(qn * kn[keys].max()))
                else:
                    sh = f32((sc * c).max())
                x = (sc.astype(np.float64) * float(c) - float(sh)).astype(np.float32)
                p = _bf16(np.exp2(x))
                acc = np.zeros(d, dtype=np.float32)
                lsum = f32(0.0)
                for j0 in range(0, len(keys), 16):
                    part = p[j0:j0 + 16].astype(np.float64) @ vf[b, h, keys[j0:j0 + 16]].astype(np.float64)
                    acc = (acc + part.astype(np.float32)).astype(np.float32)
                for j0 in range(0, len(keys), 2):
                    lsum = f32(lsum + f32(p[j0:j0 + 2].sum()))
                out[b, h, i] = _bf16(acc / lsum)
    return out


def check_element_bar(orc):
    """The per-element bar admits correct bf16 / fp32 arithmetic and nothing
    looser where it counts: an emulation of that arithmetic stays inside it on
    plain, heavy-tailed and large-output inputs; the bar is 1e-2 on almost
    every plain element; where |o| >= 4 it stays below one bf16 spacing, so an
    output one rounding step off fails it."""
    frames, t, d, w, r = 4, 32, 16, 1, 0
    n = frames * t
    scale = 1.0 / math.sqrt(d)
    cases = []
    q, k, v = (_bf16(_rand((1, 2, n, d), 500 + s)) for s in range(3))
    cases.append(("normal", q, k, v, "bound"))
    zq, zk = _rand((1, 2, n, 1), 510), _rand((1, 2, n, 1), 511)
    big = np.ones((1, 2, n, 1))
    big[:, :, ::20] = 8.0
    cases.append(("heavy", _bf16(q * np.exp(zq)), _bf16(k * np.exp(zk) * big), v, "max"))
    # nearly one-hot rows over values of spread 6: outputs reach |o| >= 4
    cases.append(("large", _bf16(10.0 * q), k, _bf16(6.0 * v), "max"))
    for name, qq, kk, vv, sh in cases:
        ref, m2 = orc.attention(qq, kk, vv, frames, t, w, r, scale, moments=True)
        sb = orc.row_bound_by_frames(qq, kk, frames, t, w, r, scale)
        nk = np.array([len(brute_visible(i // t, frames, w, r)) * t for i in range(n)])
        bar = orc.element_bar(ref, m2, sb, np.broadcast_to(nk, sb.shape), d)
        emu = emulate_bf16_kernel(qq, kk, vv, frames, t, w, r, scale, sh)
        assert np.all(np.abs(emu - ref) <= bar), (name, float((np.abs(emu - ref) - bar).max()))
        if name == "normal":
            assert np.all(bar == 1e-2), name
        if name == "large":
            # where |o| >= 4 and the row is nearly one-hot the bar stays under
            # one bf16 spacing, and correct arithmetic does exceed 1e-2 there
            hi = (np.abs(ref) >= 4.0) & (m2 - ref * ref < 0.25)
            assert hi.sum() >= 100, name
            assert np.all(bar[hi] < orc.bf16_ulp(ref[hi])), name
            assert np.any(np.abs(emu - ref)[hi] > 1e-2), name
    # a zero-spread element: the bar is 1e-2 below |o| = 2 and half a spacing above 4
    ref = np.array([[0.3, 3.0, 5.0, -6.5]])
    bar = orc.element_bar(ref, ref * ref, np.ones(1), np.full(1, 64), 128)
    np.testing.assert_allclose(bar[0], [1e-2, 1e-2, 2.0 ** -6 / 2 * 2, 2.0 ** -6 / 2 * 2], rtol=1e-3)


ALL_CHECKS = [
    check_golden_attention, check_golden_plans, check_brute_force, check_weights,
    check_dense_limit, check_closed_forms, check_bound_shift_exact, check_cauchy_schwarz,
    check_plan_closed_form, check_plan_negative_control, check_invariances, check_centering,
    check_pre_attention, check_element_bar,
]
