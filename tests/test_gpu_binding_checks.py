"""The Python binding rejects mismatched buffers before anything is enqueued
(needs an MI355X for the device tensors).

The C ABI takes plain device pointers and indexes every buffer by the plan's
sequence length and key-block count, so a buffer of the wrong size, dtype or
device would be read or written out of bounds; the binding checks each one and
raises ValueError, leaving every output untouched.
"""
import pytest
import torch

import synthetic

pytestmark = pytest.mark.gpu


def _setup():
    import frame_windowed_block_amd as fsa
    fsa.lib()
    wl = synthetic.Workload("chk", 1, 2, 128, 3, 240, 1, 0, seed=5)
    q, k, v = (x.cuda() for x in synthetic.make_inputs(wl))
    dplan = fsa.DevicePlan(wl.frames, wl.tokens_per_frame, wl.window, wl.ref_frame)
    info = dplan.info
    bufs = dict(
        qnorm=torch.full((1, 2, wl.seq_len), -1.0, device="cuda"),
        kmax=torch.full((1, 2, info.n_kblocks), -1.0, device="cuda"),
        eligible=torch.full((1, 2), -3, dtype=torch.int32, device="cuda"),
        bmax=torch.full((1, 2), -1.0, device="cuda"),
        kmean=torch.full((1, 2, 128), -5.0, device="cuda"),
    )
    return fsa, wl, q, k, v, dplan, bufs


def _untouched(bufs, out=None):
    torch.cuda.synchronize()
    assert torch.all(bufs["qnorm"] == -1.0) and torch.all(bufs["kmax"] == -1.0)
    assert torch.all(bufs["eligible"] == -3) and torch.all(bufs["bmax"] == -1.0)
    assert torch.all(bufs["kmean"] == -5.0)
    if out is not None:
        assert torch.all(out == 7.0)


BAD_BOUNDS = {
    "kmax one key block short": lambda b: b.update(kmax=b["kmax"][..., :-1].contiguous()),
    "qnorm as fp16": lambda b: b.update(qnorm=b["qnorm"].half()),
    "eligible as int64": lambda b: b.update(eligible=b["eligible"].long()),
    "bmax of the wrong shape": lambda b: b.update(bmax=b["bmax"].reshape(2, 1)),
    "kmean of the wrong head dim": lambda b: b.update(kmean=b["kmean"][..., :64].contiguous()),
    "qnorm on the host": lambda b: b.update(qnorm=b["qnorm"].cpu()),
    "kmax not contiguous": lambda b: b.update(kmax=torch.full((1, 2, 2 * b["kmax"].shape[-1]), -1.0,
                                                              device="cuda")[..., ::2]),
}


@pytest.mark.parametrize("name", list(BAD_BOUNDS))
def test_bounds_rejects(name):
    fsa, wl, q, k, v, dplan, bufs = _setup()
    bad = dict(bufs)
    BAD_BOUNDS[name](bad)
    with pytest.raises(ValueError):
        fsa.bounds(dplan, q, k, wl.scale, 0.0, 0, 0, bad["qnorm"], bad["kmax"], bad["eligible"],
                   bad["bmax"], kmean=bad["kmean"])
    _untouched(bufs)


# fsa_attention does not take bmax
@pytest.mark.parametrize("name", [n for n in BAD_BOUNDS if not n.startswith("bmax")])
def test_attention_rejects(name):
    fsa, wl, q, k, v, dplan, bufs = _setup()
    bad = dict(bufs)
    BAD_BOUNDS[name](bad)
    out = torch.full_like(q, 7.0)
    with pytest.raises(ValueError):
        fsa.attention(dplan, q, k, v, bad["qnorm"], bad["kmax"], bad["eligible"], wl.scale, 0, 0,
                      out=out, kmean=bad["kmean"])
    _untouched(bufs, out)


def test_plan_of_another_sequence_rejected():
    fsa, wl, q, k, v, dplan, bufs = _setup()
    other = fsa.DevicePlan(wl.frames + 1, wl.tokens_per_frame, wl.window, wl.ref_frame)
    out = torch.full_like(q, 7.0)
    with pytest.raises(ValueError):
        fsa.bounds(other, q, k, wl.scale, 0.0, 0, 0, bufs["qnorm"], bufs["kmax"], bufs["eligible"],
                   bufs["bmax"])
    with pytest.raises(ValueError):
        fsa.attention(other, q, k, v, bufs["qnorm"], bufs["kmax"], bufs["eligible"], wl.scale, 0, 0,
                      out=out)
    _untouched(bufs, out)


def test_plan_arrays_on_the_host_rejected():
    fsa, wl, q, k, v, dplan, bufs = _setup()
    dplan.row_ptr = dplan.row_ptr.cpu()
    out = torch.full_like(q, 7.0)
    with pytest.raises(ValueError):
        fsa.attention(dplan, q, k, v, bufs["qnorm"], bufs["kmax"], bufs["eligible"], wl.scale, 0, 0,
                      out=out)
    _untouched(bufs, out)


def test_output_on_the_host_rejected():
    fsa, wl, q, k, v, dplan, bufs = _setup()
    fsa.bounds(dplan, q, k, wl.scale, 0.0, 0, 0, bufs["qnorm"], bufs["kmax"], bufs["eligible"],
               bufs["bmax"])
    out = torch.full_like(q, 7.0).cpu()
    with pytest.raises(ValueError):
        fsa.attention(dplan, q, k, v, bufs["qnorm"], bufs["kmax"], bufs["eligible"], wl.scale, 0, 0,
                      out=out)
    torch.cuda.synchronize()
    assert torch.all(out == 7.0)


def test_pre_attention_outputs_checked():
    import frame_windowed_block_amd as fsa
    fsa.lib()
    x = torch.zeros((1, 32, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((3 * 64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fsa.pre_attention(x, w.cpu(), 1, 64)
    q = torch.full((1, 1, 32, 64), 7.0, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fsa.pre_attention(x, w, 1, 64, q=q[:, :, :16])
    torch.cuda.synchronize()
    assert torch.all(q == 7.0)
