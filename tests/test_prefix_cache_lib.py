"""The prefix cache in libpkv against the prefix-cache oracle: bit-exact.

Keys (the library's own SHA-256 against hashlib through the oracle), hits,
block ids, free queue, LRU order, counts and error codes must match on the
hand-derived trace and on random request traces.
"""

import random

import numpy as np
import pytest

import paged_attention_amd as pkv
from oracle import prefix_cache as opc
from oracle.allocator import ERR_INVALID, ERR_NO_BLOCKS, ERR_REFCOUNT, AllocatorError
from tests import prefix_trace
from tests.test_oracle_prefix_cache import _random_trace

CODES = {pkv.PKV_ERR_NO_BLOCKS: ERR_NO_BLOCKS, pkv.PKV_ERR_INVALID: ERR_INVALID, pkv.PKV_ERR_REFCOUNT: ERR_REFCOUNT}


class LibCache:
    """The oracle's interface over pkv.BlockAllocator with the prefix cache on."""

    def __init__(self, n, bs, order):
        self.a = pkv.BlockAllocator(n, bs, order)
        self.a.enable_prefix_cache()
        self.block_size = bs
        self.num_blocks = n

    def _call(self, fn, *args):
        try:
            return fn(*args)
        except pkv.PkvError as e:
            raise AllocatorError(CODES.get(e.status, e.status), str(e)) from None

    def match(self, tokens, cap):
        return self._call(self.a.prefix_match, tokens, cap)

    def register(self, tokens, row, n, first_block=0):
        return self._call(self.a.prefix_register, tokens, row, n, first_block)

    def reserve(self, row, cur_len, n_new):
        return self._call(self.a.reserve, row, cur_len, n_new)

    def release(self, row, n=None):
        return self._call(self.a.release, row)

    def free_list(self):
        return self.a.free_list()

    def lru_order(self):
        return self.a.prefix_lru()

    def cached(self):
        return self.a.prefix_cached()

    def refcount(self, b):
        return self.a.refcount(b)

    @property
    def ref(self):
        return [self.a.refcount(b) for b in range(self.num_blocks)]


def test_golden_trace_on_library():
    assert prefix_trace.run(LibCache) == []


@pytest.mark.parametrize("bs", [1, 2, 3, 4, 5, 6, 7, 8, 13, 16, 32])
def test_keys_match_hashlib(bs):
    rng = np.random.default_rng(bs)
    for n in (0, bs - 1, bs, 3 * bs + 1, 10 * bs):
        toks = rng.integers(-2**31, 2**31 - 1, size=max(n, 0), dtype=np.int64).astype(np.int32)
        assert pkv.prefix_block_keys(toks, bs) == opc.block_keys(toks, bs)


@pytest.mark.parametrize("seed", range(60))
def test_random_traces_match_oracle(seed):
    lo, _ = _random_trace(seed, lambda n, bs, order: opc.OracleCachingAllocator(n, bs, order))
    ll, _ = _random_trace(seed, LibCache)
    assert ll == lo


def test_cache_off_and_argument_errors():
    a = pkv.BlockAllocator(4, 2)
    with pytest.raises(pkv.InvalidArgument):
        a.prefix_match([1, 2], 4)
    with pytest.raises(pkv.InvalidArgument):
        a.prefix_register([1, 2], [0], 1)
    assert a.prefix_lru() == []
    a.enable_prefix_cache()
    a.enable_prefix_cache()                     # idempotent
    with pytest.raises(pkv.PkvError) as ei:
        a.prefix_register([1, 2], [0], 1)       # block 0 is not held
    assert ei.value.status == pkv.PKV_ERR_REFCOUNT
    with pytest.raises(pkv.PkvError) as ei:
        a.prefix_register([1, 2], [9], 1)
    assert ei.value.status == pkv.PKV_ERR_BAD_BLOCK


def test_shared_prompt_reuses_blocks():
    # 64 requests with one 520-token prompt and private suffixes (the shape of
    # the prefix workload): after the first, each reuses the 32 full prompt
    # blocks; the pool holds 32 + the private blocks only.
    bs, n_req = 16, 64
    rng = random.Random(3)
    prompt = [rng.randrange(32000) for _ in range(520)]
    a = pkv.BlockAllocator(4096, bs)
    a.enable_prefix_cache()
    rows, private = [], 0
    for r in range(n_req):
        toks = prompt + [rng.randrange(32000) for _ in range(rng.randint(1, 40))]
        row = a.prefix_match(toks, 1 << 20)
        assert len(row) == (0 if r == 0 else 32)
        a.reserve(row, len(row) * bs, len(toks) - len(row) * bs)
        a.prefix_register(toks, row, len(row))
        private += len(row) - 32
        rows.append(row)
    assert 4096 - a.num_free() == 32 + private
    for row in rows:
        a.release(row)
    assert a.num_free() + len(a.prefix_lru()) == 4096


def _prefix_driver_expected(ops, nb, bs, order):
    a = opc.OracleCachingAllocator(nb, bs, order)
    rows, lines = {}, ["0"]
    for op in ops:
        try:
            if op[0] == "match":
                rows[op[1]] = a.match(op[3], op[2])
                lines.append(" ".join(["ok"] + [str(b) for b in rows[op[1]]]))
            elif op[0] == "register":
                lines.append(f"ok {a.register(op[3], rows.get(op[1], []), len(rows.get(op[1], [])), op[2])}")
            elif op[0] == "reserve":
                row = rows.setdefault(op[1], [])
                trial = list(row)
                slots, _ = a.reserve(trial, op[2], op[3])
                row[:] = trial
                lines.append(" ".join(["ok"] + [str(s) for s in slots]))
            elif op[0] == "release":
                a.release(rows.get(op[1], []), len(rows.get(op[1], [])))
                rows.pop(op[1], None)
                lines.append("ok")
        except AllocatorError as e:
            lines.append(f"err {e.code}")
        lines.append("free" + "".join(f" {b}" for b in a.free_list()) + " | lru" +
                     "".join(f" {b}" for b in a.lru_order()) + f" | cached {a.cached()} | ref" +
                     "".join(f" {r}" for r in a.ref))
    return lines


def test_prefix_cache_under_sanitizers(tmp_path):
    import os
    import shutil
    import subprocess
    if shutil.which("g++") is None:
        pytest.skip("needs g++")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    csrc = os.path.join(root, "paged_attention_amd", "csrc")
    exe = tmp_path / "prefix_driver"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-D__HIP_PLATFORM_AMD__", f"-I{root}/include", f"-I{csrc}", "-I/opt/rocm/include",
           os.path.join(root, "tests", "native", "prefix_driver.cpp"), os.path.join(csrc, "allocator.cpp"),
           os.path.join(csrc, "status.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True)
    rng = random.Random(7)
    for trial in range(25):
        nb, bs = rng.randint(2, 16), rng.choice([1, 2, 4])
        order = list(range(nb))
        rng.shuffle(order)
        stems = [[rng.randint(1, 3) for _ in range(rng.randint(0, 10))] for _ in range(3)]
        ops, live, nxt = [], {}, 0
        for _ in range(rng.randint(5, 40)):
            k = rng.random()
            if live and k < 0.3:
                sid = rng.choice(sorted(live))
                ops.append(("release", sid))
                del live[sid]
                continue
            toks = list(rng.choice(stems)) + [rng.randint(1, 3) for _ in range(rng.randint(0, 5))]
            sid, nxt = nxt, nxt + 1
            ops.append(("match", sid, rng.randint(0, 6), toks))
            ops.append(("reserve", sid, -1, len(toks)))       # cur_len filled in below
            ops.append(("register", sid, 0, toks))
            live[sid] = toks
        # resolve reserve lengths from the oracle's matches (cur_len = hit blocks x bs)
        a = opc.OracleCachingAllocator(nb, bs, order)
        hits, matched = {}, {}
        fixed = []
        for op in ops:
            if op[0] == "match":
                hits[op[1]] = a.match(op[3], op[2])
                matched[op[1]] = len(hits[op[1]])
                fixed.append(op)
            elif op[0] == "reserve":
                cur = len(hits[op[1]]) * bs
                fixed.append(("reserve", op[1], cur, op[3] - cur))
                try:
                    row = list(hits[op[1]])
                    a.reserve(row, cur, op[3] - cur)
                    hits[op[1]] = row
                except AllocatorError:
                    pass
            elif op[0] == "register":
                first = matched[op[1]] if len(hits[op[1]]) >= matched[op[1]] else 0
                try:
                    a.register(op[3], hits[op[1]], len(hits[op[1]]), first)
                except AllocatorError:
                    pass
                fixed.append(("register", op[1], first, op[3]))
            else:
                try:
                    a.release(hits.get(op[1], []), len(hits.get(op[1], [])))
                    hits.pop(op[1], None)
                except AllocatorError:
                    pass
                fixed.append(op)
        script = [f"create {nb} {bs} " + " ".join(map(str, order))]
        for op in fixed:
            if op[0] in ("match", "register"):
                script.append(f"{op[0]} {op[1]} {op[2]} {len(op[3])} " + " ".join(map(str, op[3])))
            else:
                script.append(" ".join(map(str, op)))
        res = subprocess.run([str(exe)], input="\n".join(script) + "\n", capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        assert res.stdout.splitlines() == _prefix_driver_expected(fixed, nb, bs, order), f"trial {trial}"
