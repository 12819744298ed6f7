"""HIP path against the fp64 oracle, through the C ABI (needs an MI355X).

Bars: block plans bit-exact (CPU tests), bounds within 1e-5 relative, and
attention outputs (bf16) within relative L2 5e-3 of the oracle and, element
by element, within the bar of ``oracle.element_bar``: max-abs 1e-2, raised
only where correct bf16 / fp32 arithmetic can itself exceed it (half a bf16
spacing of the result plus the worst-case error of bf16 weights and fp32
accumulation, which matters only at |o| >= 4 on nearly one-hot rows). Every
output element of every shape is compared, the full-size workloads included.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
import synthetic
from tests import parity

pytestmark = pytest.mark.gpu

BOUND_RTOL = 1e-5


def _fsa():
    import frame_windowed_block_amd as fsa
    fsa.lib()
    return fsa


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _run(wl, q, k, v, bq=0, bk=0, bound_limit=0.0, head_offset=0, head_count=0, out=None,
         center=False):
    fsa = _fsa()
    dplan = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, bq, bk)
    o, b = fsa.forward(dplan, q, k, v, wl.scale, bound_limit, head_offset, head_count, out=out,
                       center=center)
    torch.cuda.synchronize()
    return o, b, dplan


def _oracle_args(wl):
    return (wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame, wl.scale)


def _assert_close(got, ref, what):
    parity.assert_close(got, ref, what)


def _check_bounds(wl, qc, kc, b, dplan, bq, bk, bound_limit=0.0, center=False):
    qnorm, kmax, eligible, bmax = (t.cpu().numpy() for t in b[:4])
    ref = oracle.bounds(synthetic.to_f64(qc), synthetic.to_f64(kc), *_oracle_args(wl),
                        dplan.info.block_q, dplan.info.block_k, bound_limit, center=center)
    np.testing.assert_allclose(qnorm, ref["qnorm"], rtol=BOUND_RTOL, atol=0)
    if center:
        # fp32 sums of N keys: error well under 1e-6 of the largest key entry
        kmean = b[4].cpu().numpy()
        scale_k = float(np.abs(synthetic.to_f64(kc)).max())
        np.testing.assert_allclose(kmean, ref["kmean"], rtol=0, atol=1e-6 * scale_k)
        # the centred norms inherit that error as an absolute one
        np.testing.assert_allclose(kmax, ref["kmax"], rtol=BOUND_RTOL, atol=2e-6 * scale_k)
    else:
        assert b[4] is None
        np.testing.assert_allclose(kmax, ref["kmax"], rtol=BOUND_RTOL, atol=0)
    np.testing.assert_allclose(bmax, ref["bmax"], rtol=BOUND_RTOL if not center else 1e-4, atol=0)
    limit = oracle.effective_bound_limit(bound_limit)
    tie = np.abs(ref["bmax"] - limit) <= 1e-4 * limit
    assert np.all((eligible == ref["eligible"]) | tie)
    return ref


# ----------------------------------------------------------------- small shapes, every output
SMALL = [
    # name, B, H, D, F, T, w, r, bq, bk
    ("tiny", 1, 2, 64, 5, 80, 1, 0, 0, 0),
    ("t240_w1", 1, 2, 128, 3, 240, 1, 0, 240, 80),
    ("t48_w0_rlast", 2, 3, 128, 4, 48, 0, 3, 48, 16),
    ("t16_pair", 1, 1, 128, 2, 16, 0, 0, 16, 16),
    ("t80_bq16", 1, 2, 64, 5, 80, 2, 4, 16, 80),
    ("t512_subtiles", 1, 2, 128, 3, 512, 1, 1, 512, 128),
    ("t1200_small", 1, 1, 128, 3, 1200, 1, 0, 240, 80),
    ("t144_d64_b2", 2, 2, 64, 4, 144, 1, 2, 144, 48),
    ("t32_dense", 1, 2, 128, 6, 32, 9, 0, 32, 32),
    ("wmax_dense", 1, 2, 128, 4, 48, 2**31 - 1, 1, 48, 16),    # largest window: dense mask
    # rows whose 16-key tile counts sit at the edges of the walk's 64-tile
    # offset tables: 64 and 128 tiles (frames 0 and 1), 65, 126 (D = 64,
    # three tiles per block) and 129 (one tile per block, a 688-row query
    # block taking three passes)
    ("tab64_128", 1, 2, 128, 2, 1024, 0, 0, 256, 128),
    ("tab65", 1, 1, 128, 1, 1040, 0, 0, 208, 80),
    ("tab126_d64", 1, 2, 64, 2, 1008, 1, 0, 112, 48),
    ("tab129_bk16", 1, 1, 128, 3, 688, 1, 0, 688, 16),
]


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
def test_small_parity(case):
    name, bsz, heads, d, frames, t, w, r, bq, bk = case
    wl = synthetic.Workload(name, bsz, heads, d, frames, t, w, r, seed=len(name))
    _say(f"case {name}: B={bsz} H={heads} D={d} F={frames} T={t} w={w} r={r} bq={bq} bk={bk}")
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    o, b, dplan = _run(wl, q, k, v, bq, bk)
    _check_bounds(wl, qc, kc, b, dplan, bq, bk)
    ref = parity.reference(wl, qc, kc, vc)
    _assert_close(synthetic.to_f64(o), ref, name)
    # online fallback forced on every head: same result within tolerance
    o2, b2, _ = _run(wl, q, k, v, bq, bk, bound_limit=1e-30)
    assert int(b2[2].sum()) == 0
    _assert_close(synthetic.to_f64(o2), ref, name + " (online)")


# ----------------------------------------------------------------- key mean-centring
CENTRED = [
    # name, B, H, D, F, T, w, r, bq, bk: one key chunk per head (N <= 2D), several
    # chunks with a ragged last one, D = 64, and a multi-tile query block
    ("c_t16_pair", 1, 1, 128, 2, 16, 0, 0, 16, 16),
    ("c_t240_w1", 1, 2, 128, 3, 240, 1, 0, 240, 80),
    ("c_t144_d64_b2", 2, 2, 64, 4, 144, 1, 2, 144, 48),
    ("c_t48_w0_rlast", 2, 3, 128, 4, 48, 0, 3, 48, 16),
    ("c_t1200_small", 1, 2, 128, 3, 1200, 1, 0, 240, 80),
]


@pytest.mark.parametrize("case", CENTRED, ids=[c[0] for c in CENTRED])
def test_centred_parity(case):
    """Keys sharing a 40-long offset: the plain bound is too loose (every head
    falls back), the centred one is tight (every head takes the bound path),
    and both outputs match the oracle."""
    name, bsz, heads, d, frames, t, w, r, bq, bk = case
    wl = synthetic.Workload(name, bsz, heads, d, frames, t, w, r, dist="key_offset", seed=len(name))
    _say(f"case {name}: B={bsz} H={heads} D={d} F={frames} T={t} w={w} r={r} bq={bq} bk={bk} centred")
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    ref = parity.reference(wl, qc, kc, vc)
    o, b, dplan = _run(wl, q, k, v, bq, bk, center=True)
    rb = _check_bounds(wl, qc, kc, b, dplan, bq, bk, center=True)
    assert np.all(rb["eligible"] == 1)
    _assert_close(synthetic.to_f64(o), ref, name + " (centred)")
    o0, b0, _ = _run(wl, q, k, v, bq, bk)
    rb0 = _check_bounds(wl, qc, kc, b0, dplan, bq, bk)
    assert np.all(rb0["eligible"] == 0)
    _assert_close(synthetic.to_f64(o0), ref, name + " (plain)")


def test_centred_on_zero_mean_keys_matches_plain():
    """On N(0,1) keys the centred path gives the same output within tolerance,
    and both runs are bitwise repeatable."""
    wl = synthetic.Workload("c_plain", 1, 2, 128, 3, 240, 1, 1, seed=11)
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    o1, b1, dplan = _run(wl, q, k, v, center=True)
    o2, b2, _ = _run(wl, q, k, v, center=True)
    assert torch.equal(o1, o2) and torch.equal(b1[4], b2[4])
    _check_bounds(wl, qc, kc, b1, dplan, 0, 0, center=True)
    ref = parity.reference(wl, qc, kc, vc)
    _assert_close(synthetic.to_f64(o1), ref, "centred on zero-mean keys")


def test_centred_head_range_and_grouping():
    """Centred calls on a head range write only that range (kmean included),
    and per-group calls equal the ungrouped call bitwise."""
    wl = synthetic.Workload("c_hr", 2, 5, 128, 3, 240, 1, 2, dist="key_offset", seed=4)
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    fsa = _fsa()
    dplan = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    full_o, full_b, _ = _run(wl, q, k, v, center=True)
    sentinel = torch.full_like(q, 7.0)
    qn = torch.full((2, 5, wl.seq_len), -1.0, device="cuda")
    km = torch.full((2, 5, dplan.info.n_kblocks), -1.0, device="cuda")
    el = torch.full((2, 5), -3, dtype=torch.int32, device="cuda")
    bm = torch.full((2, 5), -1.0, device="cuda")
    mu = torch.full((2, 5, 128), -5.0, device="cuda")
    fsa.bounds(dplan, q, k, wl.scale, 0.0, 1, 3, qn, km, el, bm, kmean=mu)
    fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, 1, 3, out=sentinel, kmean=mu)
    torch.cuda.synchronize()
    for h in (0, 4):
        assert torch.all(sentinel[:, h] == 7.0) and torch.all(mu[:, h] == -5.0)
        assert torch.all(qn[:, h] == -1.0) and torch.all(km[:, h] == -1.0)
        assert torch.all(el[:, h] == -3) and torch.all(bm[:, h] == -1.0)
    for h0 in (0, 4):
        fsa.bounds(dplan, q, k, wl.scale, 0.0, h0, 1, qn, km, el, bm, kmean=mu)
        fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, h0, 1, out=sentinel, kmean=mu)
    torch.cuda.synchronize()
    assert torch.equal(sentinel, full_o)
    for x, y in zip((qn, km, el, bm, mu), full_b):
        assert torch.equal(x, y)


# ----------------------------------------------------------------- seeded sweep of small shapes
def _random_cases(n=24, seed=20261203, t_max=512, n_max=1536, f_max=6, prefix="rnd"):
    """Seeded random small shapes: T a multiple of 16 up to 512, block sizes
    drawn from the multiples of 16 dividing T, 1-6 frames, window 0-3, any
    reference frame, D 64 or 128, 1-2 batch items, 1-3 heads, normal or
    heavy-tailed inputs; N stays <= 1536 so the oracle is quick. This walks
    the kernel through stage counts of every residue of its 3-way unrolled
    loop, odd and even 16-key tile counts, query blocks with idle wavefronts
    and query blocks taking several passes."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        t = 16 * int(rng.integers(1, t_max // 16 + 1))
        frames = int(rng.integers(1, f_max + 1))
        if frames * t > n_max:
            continue
        divs = [16 * m for m in range(1, t // 16 + 1) if t % (16 * m) == 0]
        cases.append((f"{prefix}{len(cases)}", int(rng.integers(1, 3)), int(rng.integers(1, 4)),
                      int(rng.choice([64, 128])), frames, t, int(rng.integers(0, 4)),
                      int(rng.integers(0, frames)), int(rng.choice(divs)), int(rng.choice(divs)),
                      str(rng.choice(["normal", "normal", "bound_stress"]))))
    return cases


RANDOM = _random_cases()
# longer rows (N up to 4096: up to 256 16-key tiles per row), so the walk's
# 64-tile offset tables are refilled several times at many different offsets
WIDE = _random_cases(16, 20261205, t_max=2048, n_max=4096, f_max=8, prefix="wide")


@pytest.mark.parametrize("case", RANDOM, ids=[c[0] for c in RANDOM])
def test_random_small_parity(case):
    name, bsz, heads, d, frames, t, w, r, bq, bk, dist = case
    wl = synthetic.Workload(name, bsz, heads, d, frames, t, w, r, dist=dist, seed=1000 + len(name) + t)
    _say(f"case {name}: B={bsz} H={heads} D={d} F={frames} T={t} w={w} r={r} bq={bq} bk={bk} {dist}")
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    o, b, dplan = _run(wl, q, k, v, bq, bk)
    _check_bounds(wl, qc, kc, b, dplan, bq, bk)
    ref = parity.reference(wl, qc, kc, vc)
    _assert_close(synthetic.to_f64(o), ref, name)
    if int(name[3:]) % 3 == 0:
        o2, b2, _ = _run(wl, q, k, v, bq, bk, bound_limit=1e-30)
        assert int(b2[2].sum()) == 0
        _assert_close(synthetic.to_f64(o2), ref, name + " (online)")


@pytest.mark.parametrize("case", WIDE, ids=[c[0] for c in WIDE])
def test_random_wide_parity(case):
    name, bsz, heads, d, frames, t, w, r, bq, bk, dist = case
    wl = synthetic.Workload(name, bsz, heads, d, frames, t, w, r, dist=dist, seed=2000 + int(name[4:]) + t)
    _say(f"case {name}: B={bsz} H={heads} D={d} F={frames} T={t} w={w} r={r} bq={bq} bk={bk} {dist}")
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    ref = parity.reference(wl, qc, kc, vc)
    o, b, dplan = _run(wl, q, k, v, bq, bk)
    _check_bounds(wl, qc, kc, b, dplan, bq, bk)
    _assert_close(synthetic.to_f64(o), ref, name)
    o2, b2, _ = _run(wl, q, k, v, bq, bk, bound_limit=1e-30)
    assert int(b2[2].sum()) == 0
    _assert_close(synthetic.to_f64(o2), ref, name + " (online)")


# ----------------------------------------------------------------- full-size workloads
FULL = ["tiny", "sr720", "sr1080", "bound_stress", "dense", "key_offset"]
_cache = {}


def _full(name):
    if name not in _cache:
        wl = synthetic.WORKLOADS[name]
        qc, kc, vc = synthetic.make_inputs(wl)
        _cache.clear()
        _cache[name] = (wl, qc, kc, vc)
    return _cache[name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_parity(name):
    """Every output element of the full-size workload against the oracle."""
    wl, qc, kc, vc = _full(name)
    _say(f"workload {name}: N={wl.seq_len} H={wl.heads} D={wl.head_dim}")
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    ref = parity.reference(wl, qc, kc, vc)
    # the key-offset workload needs centring for the bound path; run it both ways
    for center in ((False, True) if name == "key_offset" else (False,)):
        o, b, dplan = _run(wl, q, k, v, center=center)
        _check_bounds(wl, qc, kc, b, dplan, 0, 0, center=center)
        eligible = b[2].cpu().numpy()
        if name == "bound_stress" or (name == "key_offset" and not center):
            assert np.all(eligible == 0)
        else:
            assert np.all(eligible == 1)
        _assert_close(synthetic.to_f64(o), ref, name + (" (centred)" if center else ""))


def test_deterministic_and_grouping_bitwise():
    """Repeated runs are bitwise equal, and four 2-head calls on four streams
    equal one 8-head call bitwise (each group sees the ungrouped mask)."""
    wl, qc, kc, vc = _full("dense")
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    fsa = _fsa()
    o1, b1, dplan = _run(wl, q, k, v)
    o2, _, _ = _run(wl, q, k, v)
    assert torch.equal(o1, o2)
    og = torch.full_like(q, float("nan"))
    qn, km, el, bm = b1[:4]
    streams = [torch.cuda.Stream() for _ in range(4)]
    start = torch.cuda.Event()
    start.record()
    for gi, s in enumerate(streams):
        s.wait_event(start)
        with torch.cuda.stream(s):
            fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, 2 * gi, 2, out=og, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(og, o1)
    # grouped bounds match ungrouped bounds too
    b2 = [torch.zeros_like(x) for x in b1[:4]]
    for gi in range(4):
        fsa.bounds(dplan, q, k, wl.scale, 0.0, 2 * gi, 2, *b2)
    torch.cuda.synchronize()
    for x, y in zip(b1[:4], b2):
        assert torch.equal(x, y)


def test_head_range_leaves_other_heads_untouched():
    wl = synthetic.Workload("hr", 2, 5, 128, 3, 240, 1, 2, seed=3)
    qc, kc, vc = synthetic.make_inputs(wl)
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    fsa = _fsa()
    dplan = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    sentinel = torch.full_like(q, 7.0)
    qn = torch.full((2, 5, wl.seq_len), -1.0, device="cuda")
    km = torch.full((2, 5, dplan.info.n_kblocks), -1.0, device="cuda")
    el = torch.full((2, 5), -3, dtype=torch.int32, device="cuda")
    bm = torch.full((2, 5), -1.0, device="cuda")
    fsa.bounds(dplan, q, k, wl.scale, 0.0, 1, 3, qn, km, el, bm)
    fsa.attention(dplan, q, k, v, qn, km, el, wl.scale, 1, 3, out=sentinel)
    torch.cuda.synchronize()
    for h in (0, 4):
        assert torch.all(sentinel[:, h] == 7.0)
        assert torch.all(qn[:, h] == -1.0) and torch.all(km[:, h] == -1.0)
        assert torch.all(el[:, h] == -3) and torch.all(bm[:, h] == -1.0)
    assert torch.all(el[:, 1:4] == 1)
    ref = parity.select_heads(parity.reference(wl, qc, kc, vc), slice(1, 4))
    _assert_close(synthetic.to_f64(sentinel[:, 1:4]), ref, "head range")


def test_unsafe_bound_underflows_on_stress_data():
    """Forcing the bound path on the heavy-tailed workload (limit = +inf)
    drives whole rows to exp underflow: their sums vanish and the output turns
    non-finite. This is the hazard the per-head eligibility check guards."""
    wl, qc, kc, vc = _full("bound_stress")
    q, k, v = (x.cuda() for x in (qc, kc, vc))
    o, b, _ = _run(wl, q, k, v, bound_limit=float("inf"))
    assert int(b[2].sum()) == wl.heads
    assert not torch.isfinite(o).all().item()


def test_empty_batch_is_noop():
    fsa = _fsa()
    wl = synthetic.Workload("e", 0, 2, 128, 2, 16, 0, 0)
    dplan = fsa.DevicePlan(2, 16, 0, 0)
    q = torch.empty((0, 2, 32, 128), dtype=torch.bfloat16, device="cuda")
    o, _ = fsa.forward(dplan, q, q.clone(), q.clone(), wl.scale)
    torch.cuda.synchronize()
    assert o.shape == q.shape


# ----------------------------------------------------------------- the largest accepted head
def _frame_reference(q, k, v, f, t, scale):
    """Oracle output (and bar inputs) of frame f's rows when every frame sees
    only itself and reference frame 0 (window 0): the attention of a one- or
    two-frame problem made of frame 0 and frame f."""
    sl = [slice(0, t)] if f == 0 else [slice(0, t), slice(f * t, (f + 1) * t)]
    sub = [torch.cat([x[:, :, s] for s in sl], dim=2).cpu() for x in (q, k, v)]
    wl = synthetic.Workload("frame_sub", 1, 1, q.shape[-1], len(sl), t, 0, 0)
    assert wl.scale == scale
    ref = parity.reference(wl, *sub)
    rows = slice(0, t) if f == 0 else slice(t, 2 * t)
    return {"o": ref["o"][:, :, rows], "m2": ref["m2"][:, :, rows], "score_bound": ref["score_bound"][:, :, rows],
            "n_keys": ref["n_keys"][:, :, rows], "head_dim": ref["head_dim"]}


def test_largest_head_slab():
    """The largest head the boundary accepts: N * D * 2 just below 2 GiB (N =
    8,388,592 tokens at D = 128 in 16-token frames, window 0, reference frame
    0), so the kernels' 32-bit byte offsets inside the head reach their top.
    Sampled frames (the first, the last and a spread between) on the bound path
    and on the forced fallback, against the oracle on the frames each row sees;
    norms of the same rows and key blocks against fp64."""
    fsa = _fsa()
    d, t = 128, 16
    frames = ((1 << 31) // (2 * d) - 1) // t
    n = frames * t
    assert n * d * 2 < (1 << 31) <= (n + t) * d * 2
    _say(f"case largest_head_slab: F={frames} T={t} N={n} D={d}")
    q, k, v = synthetic.make_device_normal((1, 1, n, d), seed=11, device="cuda")
    wl = synthetic.Workload("largest", 1, 1, d, frames, t, 0, 0)
    dplan = fsa.DevicePlan(frames, t, 0, 0, 16, 16)
    o, b = fsa.forward(dplan, q, k, v, wl.scale)
    o2, b2 = fsa.forward(dplan, q, k, v, wl.scale, bound_limit=1e-30)
    torch.cuda.synchronize()
    assert int(b2[2].sum()) == 0
    rng = np.random.default_rng(5)
    sample = sorted({0, 1, 2, frames // 2, frames - 2, frames - 1, *rng.integers(0, frames, 8).tolist()})
    qnorm, kmax = b[0][0, 0], b[1][0, 0]
    for f in sample:
        rows = slice(f * t, (f + 1) * t)
        ref = _frame_reference(q, k, v, f, t, wl.scale)
        _assert_close(synthetic.to_f64(o[:, :, rows].cpu()), ref, f"frame {f}")
        _assert_close(synthetic.to_f64(o2[:, :, rows].cpu()), ref, f"frame {f} (online)")
        qf = synthetic.to_f64(q[0, 0, rows].cpu())
        kf = synthetic.to_f64(k[0, 0, rows].cpu())
        np.testing.assert_allclose(qnorm[rows].cpu().numpy(), np.linalg.norm(qf, axis=-1), rtol=BOUND_RTOL, atol=0)
        np.testing.assert_allclose(float(kmax[f]), np.linalg.norm(kf, axis=-1).max(), rtol=BOUND_RTOL, atol=0)
    del q, k, v, o, o2, b, b2
    torch.cuda.empty_cache()


# ----------------------------------------------------------------- a wider seeded sweep
SWEEP = (_random_cases(160, 777001, prefix="sw") +
         _random_cases(24, 777002, t_max=2048, n_max=4096, f_max=8, prefix="sww"))


@pytest.mark.timeout(600)
def test_random_sweep_centring_and_head_ranges():
    """184 more seeded shapes in one test (so a failure lists them all): every
    fifth with centred keys (some on offset keys), every second also on the
    forced fallback, and every third with more than one head also as a call on
    heads 1.. alone, whose rows must equal the whole call's bitwise while head 0
    stays untouched."""
    fails = []
    for idx, (name, bsz, heads, d, frames, t, w, r, bq, bk, dist) in enumerate(SWEEP):
        center = idx % 5 == 4
        if center and dist == "normal" and idx % 10 == 9:
            dist = "key_offset"
        wl = synthetic.Workload(name, bsz, heads, d, frames, t, w, r, dist=dist, seed=5000 + idx)
        _say(f"case {name}: B={bsz} H={heads} D={d} F={frames} T={t} w={w} r={r} bq={bq} bk={bk} {dist} "
             f"center={center}")
        try:
            qc, kc, vc = synthetic.make_inputs(wl)
            q, k, v = (x.cuda() for x in (qc, kc, vc))
            ref = parity.reference(wl, qc, kc, vc)
            o, b, dplan = _run(wl, q, k, v, bq, bk, center=center)
            _check_bounds(wl, qc, kc, b, dplan, bq, bk, center=center)
            _assert_close(synthetic.to_f64(o), ref, name)
            if idx % 2 == 0:
                o2, b2, _ = _run(wl, q, k, v, bq, bk, bound_limit=1e-30, center=center)
                assert int(b2[2].sum()) == 0
                _assert_close(synthetic.to_f64(o2), ref, name + " (online)")
            if heads > 1 and idx % 3 == 0:
                o3 = torch.zeros_like(q)
                _run(wl, q, k, v, bq, bk, head_offset=1, head_count=heads - 1, out=o3, center=center)
                assert torch.equal(o3[:, 1:], o[:, 1:]), "head range differs from the whole call"
                assert not (o3[:, :1] != 0).any().item(), "a head outside the range was written"
        except AssertionError as e:
            fails.append(f"{name}: {str(e)[:200]}")
    assert not fails, fails
