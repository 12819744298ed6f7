"""The C-ABI library on the CPU: it loads, exports what include/fsa.h
declares, and rejects invalid arguments on the host before any launch."""
import ctypes

import pytest

import frame_windowed_block_amd as fsa
from frame_windowed_block_amd import _abi


def test_exports_every_declared_symbol():
    L = fsa.lib()
    names = fsa.header_symbols()
    assert {"fsa_plan", "fsa_bounds", "fsa_attention", "fsa_status_string",
            "fsa_last_error", "fsa_version"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_strings():
    assert fsa.version() == 10100
    L = fsa.lib()
    for code in range(6):
        assert L.fsa_status_string(code)
    assert L.fsa_status_string(99) == b"unknown status"


def _plan_info(frames=5, t=80, w=1, r=0):
    info, _, _ = fsa.plan(frames, t, w, r)
    return info


FAKE = 0x10000          # a 64 KiB-aligned address that is never dereferenced


def _bounds(info, **kw):
    args = dict(row_ptr=FAKE, col_idx=FAKE, q=FAKE, k=FAKE, batch=1, heads=2, head_dim=64,
                head_offset=0, head_count=0, scale=0.125, bound_limit=0.0, qnorm=FAKE,
                kmax=FAKE, eligible=FAKE, bmax=FAKE, kmean=0)
    args.update(kw)
    L = fsa.lib()
    st = L.fsa_bounds(ctypes.byref(info) if info is not None else None,
                      args["row_ptr"], args["col_idx"], args["q"], args["k"], args["batch"],
                      args["heads"], args["head_dim"], args["head_offset"], args["head_count"],
                      args["scale"], args["bound_limit"], args["qnorm"], args["kmax"],
                      args["eligible"], args["bmax"], args["kmean"], None)
    return st, L.fsa_last_error().decode()


def _attn(info, **kw):
    args = dict(row_ptr=FAKE, col_idx=FAKE, q=FAKE, k=FAKE * 4096, v=FAKE * 8192, o=FAKE * 16384,
                qnorm=FAKE, kmax=FAKE, eligible=FAKE, kmean=0, batch=1, heads=2, head_dim=64,
                scale=0.125, head_offset=0, head_count=0)
    args.update(kw)
    L = fsa.lib()
    st = L.fsa_attention(ctypes.byref(info) if info is not None else None,
                         args["row_ptr"], args["col_idx"], args["q"], args["k"], args["v"],
                         args["o"], args["qnorm"], args["kmax"], args["eligible"], args["kmean"],
                         args["batch"],
                         args["heads"], args["head_dim"], args["scale"], args["head_offset"],
                         args["head_count"], None)
    return st, L.fsa_last_error().decode()


BAD_COMMON = [
    (dict(batch=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(heads=-2), fsa.FSA_ERR_INVALID_ARG),
    (dict(head_offset=3), fsa.FSA_ERR_INVALID_ARG),
    (dict(head_offset=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(head_count=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(head_offset=1, head_count=2), fsa.FSA_ERR_INVALID_ARG),
    (dict(head_dim=96), fsa.FSA_ERR_UNSUPPORTED),
    (dict(head_dim=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(scale=0.0), fsa.FSA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fsa.FSA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fsa.FSA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fsa.FSA_ERR_INVALID_ARG),
    (dict(q=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(q=FAKE + 8), fsa.FSA_ERR_INVALID_ARG),
    (dict(k=FAKE + 2), fsa.FSA_ERR_INVALID_ARG),
    (dict(row_ptr=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(col_idx=FAKE + 2), fsa.FSA_ERR_INVALID_ARG),
    (dict(qnorm=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(kmax=FAKE + 1), fsa.FSA_ERR_INVALID_ARG),
    (dict(eligible=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(kmean=FAKE + 2), fsa.FSA_ERR_INVALID_ARG),     # kmean is optional, but aligned if given
]


@pytest.mark.parametrize("kw,want", BAD_COMMON)
def test_bounds_rejects(kw, want):
    st, msg = _bounds(_plan_info(), **kw)
    assert st == want and msg


@pytest.mark.parametrize("kw,want", BAD_COMMON + [
    (dict(v=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(o=FAKE * 16384 + 4), fsa.FSA_ERR_INVALID_ARG),
    (dict(o=FAKE), fsa.FSA_ERR_INVALID_ARG),                 # overlaps q
])
def test_attention_rejects(kw, want):
    st, msg = _attn(_plan_info(), **kw)
    assert st == want and msg


@pytest.mark.parametrize("kw", [dict(bmax=0), dict(bmax=FAKE + 2)])
def test_bounds_requires_bmax(kw):
    st, _ = _bounds(_plan_info(), **kw)
    assert st == fsa.FSA_ERR_INVALID_ARG


def test_plan_info_must_be_consistent():
    info = _plan_info()
    assert _bounds(None)[0] == fsa.FSA_ERR_INVALID_ARG
    for field, val in (("nnz", 15), ("n_qblocks", 4), ("seq_len", 401), ("block_q", 0),
                       ("block_k", 48), ("tokens_per_frame", 72), ("ref_frame", 5)):
        bad = _abi.PlanInfo.from_buffer_copy(info)
        setattr(bad, field, val)
        st, msg = _bounds(bad)
        assert st in (fsa.FSA_ERR_INVALID_ARG, fsa.FSA_ERR_UNALIGNED), field
        st, msg = _attn(bad)
        assert st in (fsa.FSA_ERR_INVALID_ARG, fsa.FSA_ERR_UNALIGNED), field


def test_empty_work_is_a_noop():
    # no device work, so null pointers are fine and nothing is launched
    info = _plan_info()
    assert _bounds(info, batch=0, q=0, k=0, qnorm=0)[0] == fsa.FSA_OK
    assert _attn(info, batch=0, q=0, o=0)[0] == fsa.FSA_OK
    assert _bounds(info, head_offset=2, head_count=0, q=0)[0] == fsa.FSA_OK
    assert _attn(info, heads=0, q=0)[0] == fsa.FSA_OK


def test_error_text_is_per_call():
    L = fsa.lib()
    _bounds(_plan_info(), head_dim=96)
    assert "head_dim" in L.fsa_last_error().decode()
    fsa.plan(5, 80, 1, 0)
    assert L.fsa_last_error().decode() == ""


def test_binding_raises():
    with pytest.raises(fsa.FsaError) as ei:
        fsa.plan(5, 72, 1, 0)
    assert ei.value.status == fsa.FSA_ERR_UNALIGNED


def _pre(**kw):
    args = dict(x=FAKE, w=FAKE * 3, batch=1, seq_len=16, channels=64, heads=2,
                head_dim=64, eps=1e-6, base=10000.0, q=FAKE * 4096, k=FAKE * 8192, v=FAKE * 16384)
    args.update(kw)
    L = fsa.lib()
    st = L.fsa_pre_attention(args["x"], args["w"], args["batch"], args["seq_len"],
                             args["channels"], args["heads"], args["head_dim"], args["eps"],
                             args["base"], args["q"], args["k"], args["v"], None)
    return st, L.fsa_last_error().decode()


@pytest.mark.parametrize("kw,want", [
    (dict(batch=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(seq_len=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(heads=-1), fsa.FSA_ERR_INVALID_ARG),
    (dict(channels=48), fsa.FSA_ERR_UNSUPPORTED),
    (dict(channels=0), fsa.FSA_ERR_UNSUPPORTED),
    (dict(channels=(1 << 20) + 32), fsa.FSA_ERR_UNSUPPORTED),
    (dict(head_dim=96), fsa.FSA_ERR_UNSUPPORTED),
    (dict(head_dim=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(eps=-1.0), fsa.FSA_ERR_INVALID_ARG),
    (dict(eps=float("nan")), fsa.FSA_ERR_INVALID_ARG),
    (dict(base=0.0), fsa.FSA_ERR_INVALID_ARG),
    (dict(base=float("inf")), fsa.FSA_ERR_INVALID_ARG),
    (dict(x=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(x=FAKE + 8), fsa.FSA_ERR_INVALID_ARG),
    (dict(w=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(q=FAKE * 4096 + 2), fsa.FSA_ERR_INVALID_ARG),
    (dict(v=0), fsa.FSA_ERR_INVALID_ARG),
    (dict(q=FAKE), fsa.FSA_ERR_INVALID_ARG),                    # overlaps x
    (dict(k=FAKE * 4096 + 16), fsa.FSA_ERR_INVALID_ARG),        # overlaps q
])
def test_pre_attention_rejects(kw, want):
    st, msg = _pre(**kw)
    assert st == want and msg


def test_pre_attention_empty_is_noop():
    assert _pre(batch=0, x=0, q=0)[0] == fsa.FSA_OK
    assert _pre(seq_len=0, x=0)[0] == fsa.FSA_OK
    assert _pre(heads=0, w=0)[0] == fsa.FSA_OK


def test_head_slab_limit():
    """One head's K / V slab is addressed with 32-bit byte offsets: N * D * 2
    must stay below 2 GiB (rejected before anything is launched)."""
    info, _, _ = fsa.plan(8192, 1024, 0, 0)          # N = 2^23 tokens
    assert info.seq_len == 1 << 23
    st, msg = _bounds(info, head_dim=128)
    assert st == fsa.FSA_ERR_UNSUPPORTED and "2 GiB" in msg
    st, msg = _attn(info, head_dim=128)
    assert st == fsa.FSA_ERR_UNSUPPORTED and "2 GiB" in msg


def test_block_list_limit():
    """fsa_attention reads the plan's block list with 32-bit byte offsets:
    nnz * 4 must stay below 2 GiB (rejected before anything is launched)."""
    f = 23171                                   # dense: f^2 = 536,895,241 >= 2^29 blocks
    info = _abi.PlanInfo(frames=f, tokens_per_frame=16, window=f - 1, ref_frame=0, seq_len=16 * f,
                         block_q=16, block_k=16, n_qblocks=f, n_kblocks=f, nnz=f * f)
    st, msg = _attn(info, head_dim=128)
    assert st == fsa.FSA_ERR_UNSUPPORTED and "block list" in msg
