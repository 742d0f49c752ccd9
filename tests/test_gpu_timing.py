"""Kernel timestamps of a decode call (pkv_time_next_decode), on the GPU."""

import pytest
import torch

import paged_attention_amd as pkv
import workloads
from tests import paged_case as pc

pytestmark = pytest.mark.gpu


def test_time_next_decode_records_the_call():
    wl = workloads.custom([1, 17, 130, 300, 64, 257, 9, 200], num_heads=8, head_dim=128, dtype="f16", seed=11)
    case = pc.build(wl, "cuda")
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    w0.record(stream)
    pkv.pkv_time_next_decode(e0, e1)
    out = pc.run_gpu(case).clone()
    w1.record(stream)
    torch.cuda.synchronize()
    kern = e0.elapsed_time(e1)
    wall = w0.elapsed_time(w1)
    assert 0.0 < kern <= wall
    # the request is consumed: a second call leaves both events where they were
    out2 = pc.run_gpu(case)
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == kern
    assert torch.equal(out, out2)


def test_time_next_decode_consumed_by_a_failed_call():
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    before = e0.elapsed_time(e1)
    pkv.pkv_time_next_decode(e0, e1)
    # head_dim 100 is refused before any pointer is used; the C entry point is
    # called directly so that the request reaches the library.
    st = pkv._lib.pkv_attention_decode(None, None, None, None, None, 1, None, 1, 1, 4, 100, 16, 4, 1.0,
                                       pkv.PKV_F16, 0, None, 0, None)
    assert st == pkv.PKV_ERR_INVALID
    torch.cuda.synchronize()
    assert e0.elapsed_time(e1) == before
