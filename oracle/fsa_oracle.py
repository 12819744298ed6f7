"""CPU oracle for frame-windowed sparse attention.

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, fp64 statement of
what the HIP library computes. Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it. It shares no code,
table or constant with ``frame_windowed_block_amd/`` and imports nothing from
it; the only module both use is ``synthetic`` (seeded input draws).

Sources (the pages reporting the HeyGen / Google Cloud Avatar IV port):

* [vi:Mask]    aihot.vn, "HeyGen tối ưu hóa mô hình Avatar IV trên Google
               Cloud Trillium TPU", section "Xóa bỏ mặt nạ (Mask)" and Fig. 3.
* [vi:Softmax] same page, section "Giải phóng Softmax" and Fig. 4.
* [vi:Coll]    same page, section "Ẩn đi các tập lệnh tập thể (Collective)" (head
               groups keep the token order, so each group sees the ungrouped mask).
* [vi:Layout]  same page, section "Bố cục là ABI" and Fig. 5 (normalisation,
               rotary embedding, projection and head packing fused into one
               kernel that writes the layout its consumer reads).
* [uk:Mask], [uk:Softmax]  bib.com.ua, "HeyGen прискорила Avatar IV на TPU у
               1,86 раза", sections "Маску sparse attention прибрали
               конструктивно" and "Як розірвали послідовний ланцюг softmax"
               (corroborating text).

What the method computes, in the pages' terms: each query frame attends to a
window of neighbouring frames plus one global reference frame [vi:Mask]; the
tile grid is cut in steps of 16 tokens that divide a frame, so every block is
fully inside or fully outside the mask [vi:Mask, Fig. 3]; and the running max
of online softmax is replaced by a per-row Cauchy-Schwarz bound built from
norms computed beforehand, which leaves the output unchanged in exact arithmetic
[vi:Softmax]. The method therefore reaches exactly masked softmax attention,
and this oracle is that definition written out: dense scores over all keys,
the frame mask applied, a standard max-subtract softmax, in fp64.

Readings where the pages are silent (each is restated where it is used):

* window: half-width ``w`` in frames, clipped at the sequence ends (no wrap);
* the reference frame is global as a key only; its query rows follow the same
  window rule as every other frame; if it also lies in the window it counts once;
* token order is frame-major: token ``i`` belongs to frame ``i // T``;
* automatic block sizes: ``bq`` is the largest multiple of 16 dividing ``T``
  that is <= 256, ``bk`` the largest that is <= 128;
* the row bound is taken over the row's active key blocks (a tighter valid
  bound than the global largest key norm), and a head is eligible for the bound
  path iff its largest row bound is <= ``bound_limit`` (default 32);
* key mean-centring (optional): the mean is over all N keys of a head; the
  row's exponent is shifted by scale q_i.mean plus the centred bound, and
  eligibility checks the centred bound.

Pins (``tests/test_oracle.py``): brute force with Python loops on tiny inputs,
weight rows summing to one with exact zeros off the mask, the full window
reproducing ``torch``'s fp64 scaled-dot-product attention, the bound-shift
softmax equal to max-subtract (mpmath at 50 digits and fp64), closed forms
(q = 0, constant v, frame-indicator v), Cauchy-Schwarz on every active pair,
the plan's closed-form block count and a hand-derived plan under
``tests/golden/``, key-permutation / head-independence invariances, and for
centring: keys built as an offset plus +/- pairs of known length (so the mean
and the centred norms are known by construction), translation invariance of
the centred bound, and the shift bounding every active score.
``attention_visible`` (the same definition over the visible keys only, for
whole full-size outputs) and the second moments both attention forms return
are pinned by the same brute force and by the constant-v closed form;
``element_bar`` (the per-element comparison bar) by an emulation of bf16
weights with fp32 accumulation that must stay inside it, and by outputs one
bf16 rounding step off that must fall outside it.
"""
from __future__ import annotations

import numpy as np

DEFAULT_BOUND_LIMIT = 32.0
TILE = 16            # finest bf16 tile along the sequence [vi:Mask]
AUTO_BQ_CAP = 256
AUTO_BK_CAP = 128


# --------------------------------------------------------------------------
# Mask [vi:Mask], [uk:Mask]
# --------------------------------------------------------------------------
def visible_frames(f: int, frames: int, window: int, ref_frame: int) -> list[int]:
    """Key frames that query frame ``f`` attends: the clipped window of
    neighbouring frames plus the reference frame, each once, ascending."""
    lo = max(0, f - window)
    hi = min(frames - 1, f + window)
    vis = set(range(lo, hi + 1))
    vis.add(ref_frame)
    return sorted(vis)


def frame_visibility(frames: int, window: int, ref_frame: int) -> np.ndarray:
    """Boolean [F, F]: entry (f, g) is True iff query frame f sees key frame g."""
    vis = np.zeros((frames, frames), dtype=bool)
    for f in range(frames):
        vis[f, visible_frames(f, frames, window, ref_frame)] = True
    return vis


def token_mask_rows(rows, frames: int, tokens_per_frame: int, window: int,
                    ref_frame: int) -> np.ndarray:
    """Token-level mask rows: bool [len(rows), N], M(i, j) = [frame(j) in V(frame(i))]
    with frame(t) = t // T (frame-major token order)."""
    rows = np.asarray(rows, dtype=np.int64)
    n = frames * tokens_per_frame
    vis = frame_visibility(frames, window, ref_frame)
    key_frame = np.arange(n) // tokens_per_frame
    return vis[rows // tokens_per_frame][:, key_frame]


def token_mask(frames: int, tokens_per_frame: int, window: int, ref_frame: int) -> np.ndarray:
    """Full token-level mask bool [N, N] (small shapes only)."""
    n = frames * tokens_per_frame
    return token_mask_rows(np.arange(n), frames, tokens_per_frame, window, ref_frame)


# --------------------------------------------------------------------------
# Attention: dense masked softmax with max-subtract, fp64 [vi:Mask], [vi:Softmax]
# --------------------------------------------------------------------------
def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def attention(q, k, v, frames: int, tokens_per_frame: int, window: int,
              ref_frame: int, scale: float, moments: bool = False):
    """o[b,h,i] = sum_j p_ij v_j / sum_j p_ij with p_ij = exp(s_ij - m_i) on the
    mask and 0 off it, s_ij = scale * q_i . k_j, m_i = max of s_ij over the mask.

    q, k, v: [B, H, N, D] (any float dtype, promoted to fp64). Computed dense,
    one query frame at a time: a T x N score block over every key, masked.
    Returns fp64 [B, H, N, D], not rounded. With ``moments`` it returns
    (o, m2), m2[b,h,i,d] = sum_j w_ij v_jd^2 with the same weights
    w_ij = p_ij / sum_j p_ij (the second moment of v under row i's attention,
    used by ``element_bar``).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, heads, n, _ = q.shape
    t = tokens_per_frame
    assert n == frames * t
    vis = frame_visibility(frames, window, ref_frame)
    key_frame = np.arange(n) // t
    out = np.empty_like(q)
    m2 = np.empty_like(v) if moments else None
    for b in range(bsz):
        for h in range(heads):
            kt = k[b, h].T
            for f in range(frames):
                rows = slice(f * t, (f + 1) * t)
                s = scale * (q[b, h, rows] @ kt)                  # [T, N]
                on = vis[f][key_frame]                            # [N]
                s = np.where(on[None, :], s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)                                 # exactly 0 off the mask
                z = p.sum(axis=1, keepdims=True)
                out[b, h, rows] = (p @ v[b, h]) / z
                if moments:
                    m2[b, h, rows] = (p @ (v[b, h] * v[b, h])) / z
    return (out, m2) if moments else out


def attention_visible(q, k, v, frames: int, tokens_per_frame: int, window: int,
                      ref_frame: int, scale: float, moments: bool = False):
    """The same masked softmax attention as ``attention``, with each query
    frame's scores formed only against the keys of its visible frames V(f)
    (the window plus the reference frame, [vi:Mask]). Off-mask weights are
    exactly zero in the definition, so leaving those keys out changes nothing
    but the order in which fp64 sums meet their exact zeros. It needs a
    fraction (the mask density) of the dense form's work, which makes whole
    full-size outputs affordable to check. Returns what ``attention`` does.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    bsz, heads, n, _ = q.shape
    t = tokens_per_frame
    assert n == frames * t
    out = np.empty_like(q)
    m2 = np.empty_like(v) if moments else None
    for f in range(frames):
        rows = slice(f * t, (f + 1) * t)
        keys = np.concatenate([np.arange(g * t, (g + 1) * t)
                               for g in visible_frames(f, frames, window, ref_frame)])
        for b in range(bsz):
            for h in range(heads):
                kk, vv = k[b, h, keys], v[b, h, keys]
                s = scale * (q[b, h, rows] @ kk.T)                # [T, |V(f)| T]
                p = np.exp(s - s.max(axis=1, keepdims=True))
                z = p.sum(axis=1, keepdims=True)
                out[b, h, rows] = (p @ vv) / z
                if moments:
                    m2[b, h, rows] = (p @ (vv * vv)) / z
    return (out, m2) if moments else out


def attention_rows(q, k, v, rows, frames: int, tokens_per_frame: int, window: int,
                   ref_frame: int, scale: float, row_bound=None) -> np.ndarray:
    """The same definition as ``attention`` for selected (b, h, i) query rows.

    With ``row_bound`` ([B, H, N], optional) each row's exponent is shifted by
    that fixed value instead of by the row max (the norm-bound form of
    [vi:Softmax]; see ``attention_bound_shift``). Returns fp64 [len(rows), D].
    """
    t = tokens_per_frame
    n = frames * t
    vis = frame_visibility(frames, window, ref_frame)
    key_frame = np.arange(n) // t
    out = np.empty((len(rows), q.shape[-1]), dtype=np.float64)
    by_head = {}
    for r, (b, h, i) in enumerate(rows):
        by_head.setdefault((b, h), []).append((r, i))
    for (b, h), items in by_head.items():
        kk = _f64(k[b, h])
        vv = _f64(v[b, h])
        for r, i in items:
            s = scale * (kk @ _f64(q[b, h, i]))                   # [N]
            on = vis[i // t][key_frame]
            shift = s[on].max() if row_bound is None else float(row_bound[b, h, i])
            p = np.exp(np.where(on, s - shift, -np.inf))         # exactly 0 off the mask
            out[r] = (p @ vv) / p.sum()
    return out


def attention_weights(q, k, frames: int, tokens_per_frame: int, window: int,
                      ref_frame: int, scale: float) -> np.ndarray:
    """Softmax weights [B, H, N, N] of the masked attention (small shapes only)."""
    q, k = _f64(q), _f64(k)
    mask = token_mask(frames, tokens_per_frame, window, ref_frame)
    s = scale * (q @ np.swapaxes(k, -1, -2))
    s = np.where(mask, s, -np.inf)
    p = np.exp(s - s.max(axis=-1, keepdims=True))
    return p / p.sum(axis=-1, keepdims=True)


def attention_bound_shift(q, k, v, frames: int, tokens_per_frame: int, window: int,
                          ref_frame: int, scale: float, row_bound) -> np.ndarray:
    """The norm-bound form [vi:Softmax]: the same masked softmax, but each row's
    exponent is shifted by a fixed per-row value ``row_bound`` [B, H, N] chosen
    before the keys are visited, instead of by the row's running max. In exact
    arithmetic the result equals ``attention`` for any finite shift; in fp64 it
    stays close as long as exp(s - B) does not underflow."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    bound = _f64(row_bound)
    bsz, heads, n, _ = q.shape
    t = tokens_per_frame
    vis = frame_visibility(frames, window, ref_frame)
    key_frame = np.arange(n) // t
    out = np.empty_like(q)
    for b in range(bsz):
        for h in range(heads):
            kt = k[b, h].T
            for f in range(frames):
                rows = slice(f * t, (f + 1) * t)
                s = scale * (q[b, h, rows] @ kt)
                on = vis[f][key_frame]
                p = np.where(on[None, :], np.exp(s - bound[b, h, rows][:, None]), 0.0)
                out[b, h, rows] = (p @ v[b, h]) / p.sum(axis=1, keepdims=True)
    return out


# --------------------------------------------------------------------------
# Plan: frame-aligned active-block list [vi:Mask, Fig. 3], [uk:Mask]
# --------------------------------------------------------------------------
def aligned_block_sizes(tokens_per_frame: int) -> list[int]:
    """Multiples of 16 that divide the frame's token count."""
    return [b for b in range(TILE, tokens_per_frame + 1, TILE) if tokens_per_frame % b == 0]


def auto_block_sizes(tokens_per_frame: int) -> tuple[int, int]:
    """Reading: largest aligned size <= 256 for queries, <= 128 for keys."""
    sizes = aligned_block_sizes(tokens_per_frame)
    bq = max(b for b in sizes if b <= AUTO_BQ_CAP)
    bk = max(b for b in sizes if b <= AUTO_BK_CAP)
    return bq, bk


def block_classes(frames: int, tokens_per_frame: int, window: int, ref_frame: int,
                  block_q: int, block_k: int) -> np.ndarray:
    """Brute-force classification of every (query block, key block) pair from the
    token-level mask: 0 = fully outside, 1 = fully inside, 2 = partial. Any block
    sizes >= 1 are accepted; when a size does not divide N the grid is padded at
    the end and a block holding padding counts as partial unless it is empty of
    mask entries (the generic tiling the pages start from)."""
    n = frames * tokens_per_frame
    n_qb = -(-n // block_q)
    n_kb = -(-n // block_k)
    out = np.zeros((n_qb, n_kb), dtype=np.int8)
    for qb in range(n_qb):
        rows = np.arange(qb * block_q, (qb + 1) * block_q)
        valid = rows < n
        m = np.zeros((block_q, n_kb * block_k), dtype=bool)
        m[valid, :n] = token_mask_rows(rows[valid], frames, tokens_per_frame, window, ref_frame)
        m = m.reshape(block_q, n_kb, block_k)
        any_on = m.any(axis=(0, 2))
        all_on = m.all(axis=(0, 2))
        out[qb] = np.where(all_on, 1, np.where(any_on, 2, 0))
    return out


def check_plan_args(frames, tokens_per_frame, window, ref_frame, block_q, block_k):
    if frames < 1:
        raise ValueError("frames must be >= 1")
    if tokens_per_frame < TILE or tokens_per_frame % TILE:
        raise ValueError("tokens per frame must be a positive multiple of 16")
    if window < 0:
        raise ValueError("window must be >= 0")
    if not 0 <= ref_frame < frames:
        raise ValueError("reference frame out of range")
    for bs in (block_q, block_k):
        if bs % TILE or bs <= 0 or tokens_per_frame % bs:
            raise ValueError("block sizes must be multiples of 16 dividing T")


def plan(frames: int, tokens_per_frame: int, window: int, ref_frame: int,
         block_q: int = 0, block_k: int = 0):
    """Active-block list in CSR form, by brute force from the token mask.

    Returns (info, row_ptr, col_idx): ``info`` is a dict with frames,
    tokens_per_frame, window, ref_frame, seq_len, block_q, block_k, n_qblocks,
    n_kblocks and nnz; row_ptr is int32 [n_qb + 1]; col_idx is int32 [nnz], key
    blocks ascending within each query block. Raises if any block is partial,
    which the frame alignment rules out [vi:Mask]."""
    abq, abk = auto_block_sizes(tokens_per_frame) if tokens_per_frame >= TILE else (0, 0)
    block_q = block_q or abq
    block_k = block_k or abk
    check_plan_args(frames, tokens_per_frame, window, ref_frame, block_q, block_k)
    cls = block_classes(frames, tokens_per_frame, window, ref_frame, block_q, block_k)
    if (cls == 2).any():
        raise AssertionError("partial block in a frame-aligned grid")
    n = frames * tokens_per_frame
    row_ptr = np.zeros(cls.shape[0] + 1, dtype=np.int32)
    cols = []
    for qb in range(cls.shape[0]):
        active = np.nonzero(cls[qb] == 1)[0]
        cols.extend(active.tolist())
        row_ptr[qb + 1] = len(cols)
    col_idx = np.asarray(cols, dtype=np.int32)
    info = dict(frames=frames, tokens_per_frame=tokens_per_frame, window=window,
                ref_frame=ref_frame, seq_len=n, block_q=block_q, block_k=block_k,
                n_qblocks=cls.shape[0], n_kblocks=cls.shape[1], nnz=len(cols))
    return info, row_ptr, col_idx


# --------------------------------------------------------------------------
# Bounds [vi:Softmax], [uk:Softmax]
# --------------------------------------------------------------------------
def effective_bound_limit(bound_limit: float) -> float:
    """Reading: a limit <= 0 or NaN selects the default of 32."""
    if not (bound_limit > 0):
        return DEFAULT_BOUND_LIMIT
    return float(bound_limit)


def bounds(q, k, frames: int, tokens_per_frame: int, window: int, ref_frame: int,
           scale: float, block_q: int = 0, block_k: int = 0,
           bound_limit: float = DEFAULT_BOUND_LIMIT, center: bool = False):
    """Norm array and per-head eligibility, fp64.

    qnorm[b,h,i] = ||q_i||_2; kmax[b,h,kb] = max over the block's keys of ||k_j||_2;
    row bound B_i = scale * qnorm_i * max of kmax over the key blocks active for
    the query block holding i (Cauchy-Schwarz: s_ij <= B_i on every active pair);
    bmax[b,h] = max_i B_i; eligible[b,h] = bmax <= bound_limit.

    With ``center`` the keys are mean-centred first [vi:Softmax]: the pages
    note that keys share a large common component, that removing the mean key
    tightens the bound, and that the softmax does not change. Reading: the mean
    is taken over all N keys of the (b, h) head, kmean[b,h] = (1/N) sum_j k_j,
    and kmax becomes max ||k_j - kmean|| per key block. Since
    s_ij = scale q_i.kmean + scale q_i.(k_j - kmean), the per-row shift
    C_i = scale q_i.kmean + B_i bounds s_ij on every active pair, while
    s_ij - C_i stays >= -2 B_i; B_i (the centred bound) is what eligibility
    checks. The term scale q_i.kmean is the same for every key of row i, so
    the softmax is unchanged. Without ``center`` kmean is zero and C_i = B_i.

    Returns dict(qnorm, kmax, kmean, row_bound, row_shift, bmax, eligible, info):
    row_bound is B_i, row_shift is C_i (the value each row's exponent is
    shifted by on the bound path).
    """
    q, k = _f64(q), _f64(k)
    info, row_ptr, col_idx = plan(frames, tokens_per_frame, window, ref_frame, block_q, block_k)
    bq, bk = info["block_q"], info["block_k"]
    n_qb, n_kb = info["n_qblocks"], info["n_kblocks"]
    if center:
        kmean = k.mean(axis=2)                                   # [B, H, D]
    else:
        kmean = np.zeros(k.shape[:2] + k.shape[3:])
    kc = k - kmean[:, :, None, :]
    qnorm = np.sqrt((q * q).sum(axis=-1))
    knorm = np.sqrt((kc * kc).sum(axis=-1))
    bsz, heads, n = qnorm.shape
    kmax = knorm.reshape(bsz, heads, n_kb, bk).max(axis=-1)
    row_bound = np.empty_like(qnorm)
    for qb in range(n_qb):
        kbs = col_idx[row_ptr[qb]:row_ptr[qb + 1]]
        mk = kmax[:, :, kbs].max(axis=-1)                         # [B, H]
        sl = slice(qb * bq, (qb + 1) * bq)
        row_bound[:, :, sl] = scale * qnorm[:, :, sl] * mk[:, :, None]
    row_shift = row_bound + scale * (q @ kmean[:, :, :, None])[..., 0]
    bmax = row_bound.max(axis=-1)
    eligible = (bmax <= effective_bound_limit(bound_limit)).astype(np.int32)
    return dict(qnorm=qnorm, kmax=kmax, kmean=kmean, row_bound=row_bound, row_shift=row_shift,
                bmax=bmax, eligible=eligible, info=info)


def row_bound_by_frames(q, k, frames: int, tokens_per_frame: int, window: int,
                        ref_frame: int, scale: float) -> np.ndarray:
    """The row bound written over frames instead of blocks:
    B_i = scale * ||q_i|| * max{||k_j|| : frame(j) in V(frame(i))}.
    Because blocks tile frames exactly, this equals the block form for every
    aligned (bq, bk)."""
    q, k = _f64(q), _f64(k)
    t = tokens_per_frame
    qnorm = np.sqrt((q * q).sum(axis=-1))
    knorm = np.sqrt((k * k).sum(axis=-1))
    bsz, heads, n = qnorm.shape
    frame_kmax = knorm.reshape(bsz, heads, frames, t).max(axis=-1)   # [B, H, F]
    out = np.empty_like(qnorm)
    for f in range(frames):
        vis = visible_frames(f, frames, window, ref_frame)
        mk = frame_kmax[:, :, vis].max(axis=-1)
        out[:, :, f * t:(f + 1) * t] = scale * qnorm[:, :, f * t:(f + 1) * t] * mk[:, :, None]
    return out


# --------------------------------------------------------------------------
# Fused pre-attention [vi:Layout]
# --------------------------------------------------------------------------
DEFAULT_RMS_EPS = 1e-6
DEFAULT_ROPE_BASE = 10000.0


def rms_norm(x, gain, eps: float = DEFAULT_RMS_EPS) -> np.ndarray:
    """x / sqrt(mean over channels of x^2 + eps) * gain, fp64. x: [..., C], gain: [C]."""
    x = _f64(x)
    r = 1.0 / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)
    return x * r * _f64(gain)


def rope_frequencies(head_dim: int, base: float = DEFAULT_ROPE_BASE) -> np.ndarray:
    """Angular frequency of rotation pair j (j < D/2): base^(-2j/D)."""
    j = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * j / head_dim)


def rope(t, base: float = DEFAULT_ROPE_BASE, positions=None) -> np.ndarray:
    """Rotary position embedding of t: [B, H, N, D], position = token index n
    (or ``positions[n]`` when given, for a subset of a sequence's tokens).

    Pair j couples features j and j + D/2 and turns them by the angle p * w_j:
    out_j = t_j cos - t_{j+D/2} sin, out_{j+D/2} = t_{j+D/2} cos + t_j sin."""
    t = _f64(t)
    n, d = t.shape[-2], t.shape[-1]
    pos = np.arange(n, dtype=np.float64) if positions is None else _f64(positions)
    ang = pos[:, None] * rope_frequencies(d, base)[None, :]                          # [N, D/2]
    c, s = np.cos(ang), np.sin(ang)
    lo, hi = t[..., : d // 2], t[..., d // 2:]
    return np.concatenate([lo * c - hi * s, hi * c + lo * s], axis=-1)


def pre_attention(x, gain, w_qkv, heads: int, head_dim: int, eps: float = DEFAULT_RMS_EPS,
                  rope_base: float = DEFAULT_ROPE_BASE, positions=None):
    """The chain that produces the attention inputs, as one function [vi:Layout]:
    normalisation, projection, rotary embedding and head packing.

    x: [B, N, C] token activations (frame-major tokens); gain: [C];
    w_qkv: [3 H D, C], a linear layer's weight (output features by input
    channels): rows 0 .. HD-1 make q, then k, then v; within each, head h owns
    rows h D .. h D + D - 1. Readings (the page lists the four steps only):
    RMS normalisation with a per-channel gain, no projection bias, rotary
    embedding on q and k (not v) at position n = the token's index in its
    sequence, pairs (j, j + D/2), base 10000.

    ``positions`` (optional, [N]) gives each token's index in its sequence when
    x holds only some of the sequence's tokens.

    Returns q, k, v, each fp64 [B, H, N, D] (the layout the attention reads).
    """
    xn = rms_norm(x, gain, eps)                                   # [B, N, C]
    y = xn @ _f64(w_qkv).T                                        # [B, N, 3 H D]
    bsz, n, _ = y.shape
    y = y.reshape(bsz, n, 3, heads, head_dim).transpose(2, 0, 3, 1, 4)   # [3, B, H, N, D]
    return rope(y[0], rope_base, positions), rope(y[1], rope_base, positions), y[2].copy()


def pre_attention_flops(batch: int, seq_len: int, channels: int, heads: int, head_dim: int) -> int:
    """Algorithmic FLOPs of the projection: 2 C per output feature."""
    return 2 * batch * seq_len * channels * 3 * heads * head_dim


# --------------------------------------------------------------------------
# Work counts (used for throughput figures)
# --------------------------------------------------------------------------
def active_pairs(frames: int, tokens_per_frame: int, window: int, ref_frame: int) -> int:
    """Number of (query, key) pairs on the mask, per (batch, head)."""
    pairs = sum(len(visible_frames(f, frames, window, ref_frame)) for f in range(frames))
    return pairs * tokens_per_frame * tokens_per_frame


def active_flops(batch: int, heads: int, head_dim: int, frames: int, tokens_per_frame: int,
                 window: int, ref_frame: int) -> int:
    """Algorithmic FLOPs on active blocks: 2D for q.k plus 2D for p.v per pair."""
    return 4 * head_dim * batch * heads * active_pairs(frames, tokens_per_frame, window, ref_frame)


MAX_ABS_BAR = 1e-2
REL_L2_BAR = 5e-3


def bf16_ulp(x) -> np.ndarray:
    """Spacing of bf16 numbers (8 significant bits) at |x| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(_f64(x)), 2.0 ** -126)))
    return 2.0 ** (e - 7)


def _gamma(n) -> np.ndarray:
    """Classic bound n u / (1 - n u) on the relative error of n fp32 roundings."""
    nu = _f64(n) * 2.0 ** -24
    return nu / (1.0 - nu)


def element_bar(ref, m2, score_bound, n_keys, head_dim: int) -> np.ndarray:
    """Per-element max-abs bar for a bf16 output against the fp64 result ``ref``.

    The target bar is 1e-2. An element may exceed it only where correct bf16 /
    fp32 arithmetic itself can: the bar is max(1e-2, ulp(|ref| + e) / 2 + e),
    with e the worst-case error of the fp32 value before the final rounding
    to bf16 (half a bf16 spacing):

    * weights rounded to bf16 (relative 2^-8 each) and perturbed by the fp32
      score error (at most gamma_D * scale ||q_i|| ||k_j|| <= gamma_D * B_i with
      B_i = ``score_bound``, the row's Cauchy-Schwarz bound over its visible
      keys, plus 2^-20 (1 + B_i) for the exponent's own roundings): each
      weight p_j becomes p_j (1 + eps_j), |eps_j| <= rho = (1 + 2^-8) exp(eta) - 1.
      The row sum adds the same weights, so the result is
      o + sum_j p_j eps_j (v_j - o) / sum_j p_j (1 + eps_j) (the terms
      p_j (v_j - o) alone sum to zero); with 1 + eps_j >= (1 - 2^-8) exp(-eta)
      that is at most rho exp(eta) / (1 - 2^-8) times
      sum_j w_j |v_j - o| <= sigma = sqrt(m2 - o^2) (Jensen) away from o;
    * fp32 accumulation of the weighted values in 16-key products (depth
      n/16 + 16 for n = ``n_keys``) and of the row sum per lane in pairs
      (depth n/4 + 4): (gamma_{n/16+16} + gamma_{n/4+4}) sqrt(m2).

    ref, m2: [..., D]; score_bound, n_keys: [...] (broadcast over D)."""
    ref, m2 = _f64(ref), _f64(m2)
    b = _f64(score_bound)[..., None]
    n = _f64(n_keys)[..., None]
    eta = _gamma(head_dim) * b + 2.0 ** -20 * (1.0 + b)
    rho = (1.0 + 2.0 ** -8) * np.exp(eta) - 1.0
    sigma = np.sqrt(np.maximum(m2 - ref * ref, 0.0))
    e = rho * np.exp(eta) / (1.0 - 2.0 ** -8) * sigma
    e = e + (_gamma(n / 16.0 + 16.0) + _gamma(n / 4.0 + 4.0)) * np.sqrt(np.maximum(m2, 0.0))
    return np.maximum(MAX_ABS_BAR, 0.5 * bf16_ulp(np.abs(ref) + e) + e)


def max_abs_and_rel_l2(got, ref) -> tuple[float, float]:
    """The two comparison metrics: max |got - ref| and ||got - ref||_2 / ||ref||_2."""
    got, ref = _f64(got), _f64(ref)
    diff = got - ref
    max_abs = float(np.abs(diff).max()) if diff.size else 0.0
    den = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff)) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


__all__ = [
    "DEFAULT_BOUND_LIMIT", "visible_frames", "frame_visibility", "token_mask_rows",
    "token_mask", "attention", "attention_visible", "attention_rows", "attention_weights",
    "attention_bound_shift", "aligned_block_sizes", "auto_block_sizes", "block_classes",
    "check_plan_args", "plan", "effective_bound_limit", "bounds", "row_bound_by_frames",
    "active_pairs", "active_flops", "max_abs_and_rel_l2", "MAX_ABS_BAR", "REL_L2_BAR", "bf16_ulp",
    "element_bar",
    "DEFAULT_RMS_EPS", "DEFAULT_ROPE_BASE", "rms_norm", "rope_frequencies", "rope", "pre_attention",
    "pre_attention_flops",
]
