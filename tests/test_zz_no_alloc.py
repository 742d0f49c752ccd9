"""pkv_attention_decode_scratch: decode attention with the library's own device
scratch, for callers that cannot allocate.

Two calls in a row through the C interface, the second on a smaller input,
each checked against pkv_attention_decode with a caller workspace (the same
kernels and work split: identical bits) and against the oracle (2e-3, fp16).
Also: a request whose workspace would exceed the scratch is refused before
anything runs, and repeated calls allocate no device memory.
"""

import numpy as np
import pytest
import torch

import paged_attention_amd as pkv
import workloads
from tests import paged_case as pc

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()


def _both(c, work_groups=0):
    got = torch.full_like(c.q, float("nan"))
    pkv.pkv_attention_decode_scratch(got, c.q, c.k_cache, c.v_cache, c.tables, c.lens, c.wl.max_seq_len,
                                     scale=c.wl.scale, work_groups=work_groups)
    torch.cuda.synchronize()
    want = pc.run_gpu(c, work_groups=work_groups, out=torch.empty_like(c.q))
    return got, want


def test_scratch_decode_two_calls_then_smaller():
    rng = np.random.default_rng(71)
    big = workloads.custom(rng.integers(128, 2049, size=32), num_heads=32, head_dim=128, dtype="f16",
                           block_size=16, seed=72)
    small = workloads.custom([1, 9, 300, 77, 16], num_heads=32, head_dim=128, dtype="f16", block_size=16, seed=73)
    cb, cs = pc.build(big, DEV), pc.build(small, DEV)
    ref_b, ref_s = pc.oracle_out(cb), pc.oracle_out(cs)
    got, want = _both(cb)                       # first call on the device looks the scratch up
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    pc.compare(cb, got, ref_b, record="scratch decode (no allocation), 7B-shaped")
    free0, _ = torch.cuda.mem_get_info()
    got, want = _both(cs)                       # the smaller input reuses the same scratch
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    pc.compare(cs, got, ref_s, record="scratch decode (no allocation), small")
    got, want = _both(cb, work_groups=100)      # and a larger one again, another work split
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    pc.compare(cb, got, ref_b)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert free1 == free0


def test_scratch_decode_refuses_what_does_not_fit():
    wl = workloads.custom([40, 3], num_heads=32, head_dim=128, dtype="f16", block_size=16, seed=74)
    c = pc.build(wl, DEV)
    # 4096 work-groups x 32 heads x (128 + 2) floats x 2 pieces is far above 32 MiB
    assert pkv.pkv_decode_workspace_bytes(wl.batch, 32, 128, "f16", 4096) > pkv.DECODE_SCRATCH_BYTES
    out = torch.full_like(c.q, float("nan"))
    with pytest.raises(pkv.InvalidArgument, match="scratch"):
        pkv.pkv_attention_decode_scratch(out, c.q, c.k_cache, c.v_cache, c.tables, c.lens, wl.max_seq_len,
                                         work_groups=4096)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    # an empty batch is not an error; a bad shape is reported as by pkv_attention_decode
    empty = torch.empty((0, 32, 128), dtype=torch.float16, device=DEV)
    pkv.pkv_attention_decode_scratch(empty, empty, c.k_cache, c.v_cache, c.tables[:0], c.lens[:0], 8)
    with pytest.raises(pkv.InvalidArgument):
        pkv.pkv_attention_decode_scratch(out, c.q, c.k_cache, c.v_cache, c.tables, c.lens, wl.max_seq_len,
                                         work_groups=-1)
