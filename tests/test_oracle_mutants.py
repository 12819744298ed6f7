"""Planted mistakes in the CPU oracle must be caught by its pins.

Each mutant is a copy of the oracle with one plausible mistake (a dropped
term, a wrong sign or index, a transposed operand, a wrong reduction). The
test runs the pin checks of ``oracle_pins`` against the mutant and requires at
least one of them to fail. Mistakes are planted on the CPU, in the oracle only.
"""
import types

import numpy as np
import pytest

import oracle
from oracle import fsa_oracle as fo
from tests import oracle_pins

fo.ROPE_ORIG = fo.rope


def _namespace(**overrides):
    ns = types.SimpleNamespace(**{name: getattr(oracle, name) for name in oracle.__all__})
    for key, val in overrides.items():
        setattr(ns, key, val)
    return ns


def _vis_no_ref(f, frames, window, ref_frame):
    return sorted(set(range(max(0, f - window), min(frames - 1, f + window) + 1)))


def _vis_wrap(f, frames, window, ref_frame):
    return sorted({(f + d) % frames for d in range(-window, window + 1)} | {ref_frame})


def _vis_short(f, frames, window, ref_frame):
    return sorted(set(range(max(0, f - window), min(frames - 1, f + window - 1) + 1)) | {ref_frame})


def _vis_ref_query_global(f, frames, window, ref_frame):
    if f == ref_frame:
        return list(range(frames))
    return sorted(set(range(max(0, f - window), min(frames - 1, f + window) + 1)) | {ref_frame})


def _attention_wrong_axis(q, k, v, frames, t, window, ref_frame, scale):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    vis = fo.frame_visibility(frames, window, ref_frame)
    key_frame = np.arange(q.shape[2]) // t
    out = np.empty_like(q)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            for f in range(frames):
                rows = slice(f * t, (f + 1) * t)
                s = scale * (q[b, h, rows] @ k[b, h].T)
                s = np.where(vis[f][key_frame][None, :], s, -np.inf)
                p = np.exp(s - s.max(axis=1, keepdims=True))
                out[b, h, rows] = (p @ v[b, h]) / p.sum(axis=0).sum()
    return out


def _bounds_kmin(q, k, frames, t, window, ref_frame, scale, block_q=0, block_k=0,
                 bound_limit=32.0, center=False):
    res = oracle.bounds(q, k, frames, t, window, ref_frame, scale, block_q, block_k, bound_limit,
                        center)
    info = res["info"]
    kn = np.sqrt((np.asarray(k, dtype=np.float64) ** 2).sum(-1))
    res["kmax"] = kn.reshape(*kn.shape[:2], info["n_kblocks"], info["block_k"]).min(-1)
    return res


def _bounds_global(q, k, frames, t, window, ref_frame, scale, block_q=0, block_k=0,
                   bound_limit=32.0, center=False):
    res = oracle.bounds(q, k, frames, t, window, ref_frame, scale, block_q, block_k, bound_limit,
                        center)
    qn = res["qnorm"]
    kn = np.sqrt((np.asarray(k, dtype=np.float64) ** 2).sum(-1)).max(-1)
    res["row_bound"] = scale * qn * kn[..., None]
    return res


def _bounds_no_sqrt(q, k, frames, t, window, ref_frame, scale, block_q=0, block_k=0,
                    bound_limit=32.0, center=False):
    res = oracle.bounds(q, k, frames, t, window, ref_frame, scale, block_q, block_k, bound_limit,
                        center)
    res["row_bound"] = res["row_bound"] * res["qnorm"]
    return res


def _centred(fn):
    """A bounds variant that applies ``fn(res, q, k, scale, mask_args)`` to centred results only."""
    def bounds(q, k, frames, t, window, ref_frame, scale, block_q=0, block_k=0,
               bound_limit=32.0, center=False):
        res = oracle.bounds(q, k, frames, t, window, ref_frame, scale, block_q, block_k,
                            bound_limit, center)
        if center:
            fn(res, np.asarray(q, dtype=np.float64), np.asarray(k, dtype=np.float64), scale,
               (frames, t, window, ref_frame))
        return res
    return bounds


def _shift_sign(res, q, k, scale, mask_args):
    res["row_shift"] = res["row_bound"] - scale * np.einsum("bhnd,bhd->bhn", q, res["kmean"])


def _shift_dropped(res, q, k, scale, mask_args):
    res["row_shift"] = res["row_bound"].copy()


def _uncentred_norms(res, q, k, scale, mask_args):
    plain = oracle.bounds(q, k, *mask_args, scale, res["info"]["block_q"], res["info"]["block_k"])
    res["kmax"] = plain["kmax"]
    res["row_bound"] = plain["row_bound"]
    res["row_shift"] = plain["row_bound"] + scale * np.einsum("bhnd,bhd->bhn", q, res["kmean"])


def _block_mean(res, q, k, scale, mask_args):
    bsz, heads, n, d = k.shape
    bk = res["info"]["block_k"]
    kb = k.reshape(bsz, heads, n // bk, bk, d)
    res["kmax"] = np.sqrt(((kb - kb.mean(axis=3, keepdims=True)) ** 2).sum(-1)).max(-1)


def _query_mean(res, q, k, scale, mask_args):
    res["kmean"] = q.mean(axis=2)


def _rope_interleaved(t, base=10000.0, positions=None):
    t = np.asarray(t, dtype=np.float64)
    n, d = t.shape[-2], t.shape[-1]
    pos = np.arange(n) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = pos[:, None] * fo.rope_frequencies(d, base)[None, :]
    c, s_ = np.cos(ang), np.sin(ang)
    out = t.copy()
    out[..., 0::2] = t[..., 0::2] * c - t[..., 1::2] * s_
    out[..., 1::2] = t[..., 1::2] * c + t[..., 0::2] * s_
    return out


def _rope_sign(t, base=10000.0, positions=None):
    t = np.asarray(t, dtype=np.float64)
    d = t.shape[-1]
    flip = np.ones(d)
    flip[d // 2:] = -1.0
    return fo.ROPE_ORIG(t * flip, base, positions) * flip


def _rope_from_one(t, base=10000.0, positions=None):
    t = np.asarray(t, dtype=np.float64)
    n, d = t.shape[-2], t.shape[-1]
    pos = np.arange(n) if positions is None else np.asarray(positions, dtype=np.float64)
    ang = (1.0 + pos)[:, None] * fo.rope_frequencies(d, base)[None, :]
    c, s_ = np.cos(ang), np.sin(ang)
    lo, hi = t[..., : d // 2], t[..., d // 2:]
    return np.concatenate([lo * c - hi * s_, hi * c + lo * s_], axis=-1)


def _pre_rope_v(x, gain, w, heads, d, eps=1e-6, base=10000.0, positions=None):
    q, k, v = oracle.pre_attention(x, gain, w, heads, d, eps, base, positions)
    return q, k, fo.rope(v, base, positions)


def _pre_heads_swapped(x, gain, w, heads, d, eps=1e-6, base=10000.0, positions=None):
    xn = fo.rms_norm(x, gain, eps)
    y = xn @ np.asarray(w, dtype=np.float64).T
    bsz, n, _ = y.shape
    y = y.reshape(bsz, n, 3, d, heads).transpose(2, 0, 4, 1, 3)
    return fo.rope(y[0], base, positions), fo.rope(y[1], base, positions), y[2].copy()


def _pre_qk_swapped(x, gain, w, heads, d, eps=1e-6, base=10000.0, positions=None):
    q, k, v = oracle.pre_attention(x, gain, w, heads, d, eps, base, positions)
    return k, q, v


def _rms_over_tokens(x, gain, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-2, keepdims=True) + eps) * np.asarray(gain)


def _rms_no_gain(x, gain, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + eps)


def _rms_no_sqrt(x, gain, eps=1e-6):
    x = np.asarray(x, dtype=np.float64)
    return x / ((x * x).mean(axis=-1, keepdims=True) + eps) * np.asarray(gain)


def _plan_descending(*args, **kw):
    info, row_ptr, col_idx = oracle.plan(*args, **kw)
    col = col_idx.copy()
    for qb in range(info["n_qblocks"]):
        col[row_ptr[qb]:row_ptr[qb + 1]] = col[row_ptr[qb]:row_ptr[qb + 1]][::-1]
    return info, row_ptr, col


def _plan_swapped_sizes(frames, t, window, ref_frame, block_q=0, block_k=0):
    return oracle.plan(frames, t, window, ref_frame, block_k, block_q)


def _visible_window_only(q, k, v, frames, t, window, ref_frame, scale, moments=False):
    q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
    out, m2 = np.empty_like(q), np.empty_like(v)
    for f in range(frames):
        rows = slice(f * t, (f + 1) * t)
        keys = np.arange(max(0, f - window) * t, (min(frames - 1, f + window) + 1) * t)
        s = scale * (q[:, :, rows] @ np.swapaxes(k[:, :, keys], -1, -2))
        p = np.exp(s - s.max(-1, keepdims=True))
        z = p.sum(-1, keepdims=True)
        out[:, :, rows] = (p @ v[:, :, keys]) / z
        m2[:, :, rows] = (p @ v[:, :, keys] ** 2) / z
    return (out, m2) if moments else out


def _moment_of_mean(fn):
    def wrapped(q, k, v, frames, t, window, ref_frame, scale, moments=False):
        if not moments:
            return fn(q, k, v, frames, t, window, ref_frame, scale)
        o = fn(q, k, v, frames, t, window, ref_frame, scale)
        return o, o * o
    return wrapped


def _bar_no_half_spacing(ref, m2, score_bound, n_keys, head_dim):
    return np.minimum(oracle.element_bar(ref, m2, score_bound, n_keys, head_dim),
                      np.maximum(1e-2, oracle.element_bar(ref, m2, score_bound, n_keys, head_dim)
                                 - 0.5 * oracle.bf16_ulp(ref)))


def _bar_full_spacing(ref, m2, score_bound, n_keys, head_dim):
    return np.maximum(1e-2, oracle.bf16_ulp(ref))


MUTANTS = {
    "reference frame dropped": dict(module={"visible_frames": _vis_no_ref}),
    "window wraps around": dict(module={"visible_frames": _vis_wrap}),
    "window one frame short": dict(module={"visible_frames": _vis_short}),
    "reference frame global as query": dict(module={"visible_frames": _vis_ref_query_global}),
    "scale dropped": dict(ns={"attention": lambda q, k, v, F, T, w, r, s: oracle.attention(
        q, k, v, F, T, w, r, 1.0)}),
    "keys used as values": dict(ns={"attention": lambda q, k, v, F, T, w, r, s: oracle.attention(
        q, k, k, F, T, w, r, s)}),
    "q and k swapped": dict(ns={"attention": lambda q, k, v, F, T, w, r, s: oracle.attention(
        k, q, v, F, T, w, r, s)}),
    "softmax normalised over the wrong axis": dict(ns={"attention": _attention_wrong_axis}),
    "key-block max taken as min": dict(ns={"bounds": _bounds_kmin}),
    "row bound over all keys": dict(ns={"bounds": _bounds_global}),
    "row bound with a squared query norm": dict(ns={"bounds": _bounds_no_sqrt}),
    "centring shift with the wrong sign": dict(ns={"bounds": _centred(_shift_sign)}),
    "centring shift dropped": dict(ns={"bounds": _centred(_shift_dropped)}),
    "centred shift over uncentred key norms": dict(ns={"bounds": _centred(_uncentred_norms)}),
    "key mean taken per key block": dict(ns={"bounds": _centred(_block_mean)}),
    "query mean used as the key mean": dict(ns={"bounds": _centred(_query_mean)}),
    "rotary pairs interleaved": dict(module={"rope": _rope_interleaved}),
    "rotary sine with the wrong sign": dict(module={"rope": _rope_sign}),
    "rotary positions counted from one": dict(module={"rope": _rope_from_one}),
    "rotary embedding applied to v": dict(ns={"pre_attention": _pre_rope_v}),
    "head and feature axes swapped in packing": dict(ns={"pre_attention": _pre_heads_swapped}),
    "q and k outputs swapped": dict(ns={"pre_attention": _pre_qk_swapped}),
    "rms taken over tokens": dict(module={"rms_norm": _rms_over_tokens}),
    "norm gain dropped": dict(module={"rms_norm": _rms_no_gain}),
    "rms without the square root": dict(module={"rms_norm": _rms_no_sqrt}),
    "visible-key attention without the reference frame": dict(ns={"attention_visible": _visible_window_only}),
    "second moment taken as the squared mean": dict(ns={"attention_visible": _moment_of_mean(
        oracle.attention_visible)}),
    "element bar without the half bf16 spacing": dict(ns={"element_bar": _bar_no_half_spacing}),
    "element bar widened to one bf16 spacing": dict(ns={"element_bar": _bar_full_spacing}),
    "key blocks listed descending": dict(ns={"plan": _plan_descending}),
    "query and key block sizes swapped": dict(ns={"plan": _plan_swapped_sizes}),
}

FAST_CHECKS = [c for c in oracle_pins.ALL_CHECKS if c is not oracle_pins.check_plan_closed_form]


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    spec = MUTANTS[name]
    for attr, fn in spec.get("module", {}).items():
        monkeypatch.setattr(fo, attr, fn)
    ns = _namespace(**spec.get("ns", {}))
    failures = []
    for check in FAST_CHECKS + [oracle_pins.check_plan_closed_form]:
        try:
            check(ns)
        except Exception as exc:           # noqa: BLE001 - any failure counts
            failures.append((check.__name__, type(exc).__name__))
            break
    assert failures, f"no pin caught the planted mistake: {name}"
