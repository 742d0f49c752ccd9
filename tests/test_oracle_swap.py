"""Pins of the swap oracle (oracle.pool.swap_blocks): a swap is a bit copy
between two pools, so a round trip out and back in at other ids restores
every byte, and attention read through the remapped table is unchanged."""

import numpy as np
import pytest

import workloads
from oracle import attention as oat
from oracle import pool as opool


def test_round_trip_restores_bytes_and_attention():
    rng = np.random.default_rng(3)
    nb, bs, h, d = 10, 4, 2, 8
    kp = workloads.to_storage(rng.standard_normal((nb, bs, h, d), dtype=np.float32), "f16")
    vp = workloads.to_storage(rng.standard_normal((nb, bs, h, d), dtype=np.float32), "f16")
    tables = np.array([[3, 7, 1], [5, 0, 9]], dtype=np.int32)
    lens = [11, 9]
    q = workloads.to_storage(rng.standard_normal((2, h, d), dtype=np.float32), "f16")
    ref = oat.decode_attention(q, kp, vp, tables, lens, "f16")
    # out: blocks of sequence 0 to host blocks 2, 0, 5 of a 6-block swap space
    hk = np.zeros((6, bs, h, d), dtype=np.float16)
    hv = np.zeros_like(hk)
    out_pairs = [(3, 2), (7, 0), (1, 5)]
    opool.swap_blocks([hk, hv], [kp, vp], out_pairs)
    for s, dd in out_pairs:
        assert np.array_equal(hk[dd], kp[s]) and np.array_equal(hv[dd], vp[s])
    # the device blocks are reused by someone else (poisoned), then swapped back in at 4, 6, 8
    kp2, vp2 = kp.copy(), vp.copy()
    for b in (3, 7, 1):
        kp2[b] = workloads.nan_storage("f16")
        vp2[b] = workloads.nan_storage("f16")
    in_pairs = [(2, 4), (0, 6), (5, 8)]
    opool.swap_blocks([kp2, vp2], [hk, hv], in_pairs)
    tables2 = tables.copy()
    tables2[0] = [4, 6, 8]
    got = oat.decode_attention(q, kp2, vp2, tables2, lens, "f16")
    assert np.array_equal(got, ref)


def test_repeated_destinations_rejected():
    a = np.zeros((4, 2))
    b = np.zeros((4, 2))
    with pytest.raises(ValueError):
        opool.swap_blocks([a], [b], [(0, 1), (2, 1)])
