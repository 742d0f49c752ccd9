"""libpkv loads, exports every symbol include/pkv.h declares, and validates
arguments on the host (no kernel is launched by these tests)."""

import ctypes
import os
import re
import subprocess

import pytest

import paged_attention_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"PKV_API\s+[^;(]*?\b(pkv_\w+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared()
    for must in ("pkv_append", "pkv_attention_decode", "pkv_copy_blocks", "pkv_allocator_create",
                 "pkv_block_alloc", "pkv_block_decref", "pkv_seq_reserve", "pkv_seq_release"):
        assert must in names
    assert len(names) >= 20


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", pkv.LIB_PATH], capture_output=True, text=True, check=True)
    exported = {line.split()[-1] for line in out.stdout.splitlines() if " T " in line}
    missing = [n for n in _declared() if n not in exported]
    assert not missing, missing
    # Nothing else leaks out of the library's C interface.
    extra = [n for n in exported if n.startswith("pkv_") and n not in _declared()]
    assert not extra, extra
    lib = ctypes.CDLL(pkv.LIB_PATH)
    for n in _declared():
        getattr(lib, n)


def _c_kind(decl: str):
    """Kind of a C parameter or return type: ptr, i32, i64, size, f32 or void."""
    d = " ".join(decl.replace("const ", "").split())
    if "*" in d or d.split()[0] in ("hipStream_t", "hipEvent_t"):
        return "ptr"
    t = d.split()[0]
    return {"int32_t": "i32", "int": "i32", "pkv_dtype": "i32", "int64_t": "i64", "size_t": "size",
            "float": "f32", "void": "void"}[t]


def _ctypes_kind(t):
    if t is None:
        return "void"
    if t in (ctypes.c_void_p, ctypes.c_char_p) or (isinstance(t, type) and issubclass(t, ctypes._Pointer)):
        return "ptr"
    return {ctypes.c_int32: "i32", ctypes.c_int64: "i64", ctypes.c_size_t: "size", ctypes.c_float: "f32"}[t]


def test_binding_signatures_match_the_header():
    with open(os.path.join(ROOT, "include", "pkv.h")) as f:
        text = re.sub(r"/\*.*?\*/", "", f.read(), flags=re.S)
    decls = re.findall(r"PKV_API\s+([^;(]*?)\b(pkv_\w+)\s*\(([^)]*)\)\s*;", text, flags=re.S)
    assert len(decls) == len(_declared())
    for ret, name, params in decls:
        params = [q for q in (x.strip() for x in params.split(",")) if q and q != "void"]
        fn = getattr(pkv._lib, name)
        assert fn.argtypes is not None, name
        want = [_c_kind(q.rsplit(" ", 1)[0] if "*" not in q.rsplit(" ", 1)[-1] else q) for q in params]
        got = [_ctypes_kind(t) for t in fn.argtypes]
        assert got == want, (name, got, want)
        assert _ctypes_kind(fn.restype) == _c_kind(ret.strip()), (name, fn.restype, ret)


def test_status_strings_and_version():
    lib = pkv._lib
    assert pkv.version() >= 100
    for code in (0, -1, -2, -3, -4, -5):
        assert lib.pkv_strerror(code)
    assert lib.pkv_strerror(-99) == b"unknown status"


def test_device_calls_reject_bad_shapes_before_launch():
    lib = pkv._lib
    null = ctypes.c_void_p(0)
    # Unsupported head_dim / block size / dtype: rejected on the host.
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 1, 4, 96, 16, 8, 1.0, 1, 0, null, 0,
                                  null)
    assert st == pkv.PKV_ERR_INVALID
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 1, 4, 128, 12, 8, 1.0, 1, 0, null, 0,
                                  null)
    assert st == pkv.PKV_ERR_INVALID
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 1, 4, 128, 16, 8, 1.0, 7, 0, null, 0,
                                  null)
    assert st == pkv.PKV_ERR_INVALID
    # The work-group count must be 0 (automatic) or a positive count.
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 1, 4, 128, 16, 8, 1.0, 1, -3, null, 0,
                                  null)
    assert st == pkv.PKV_ERR_INVALID
    # Null pointers with a non-empty batch.
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 1, 4, 128, 16, 8, 1.0, 1, 0, null, 0,
                                  null)
    assert st == pkv.PKV_ERR_INVALID
    # Empty batch: nothing to do.
    st = lib.pkv_attention_decode(null, null, null, null, null, 4, null, 64, 0, 4, 128, 16, 8, 1.0, 1, 0, null, 0,
                                  null)
    assert st == pkv.PKV_OK
    assert lib.pkv_append(null, null, 0, null, null, null, 8, 16, 4, 128, 1, null) == pkv.PKV_OK
    assert lib.pkv_append(null, null, 3, null, null, null, 8, 16, 4, 128, 1, null) == pkv.PKV_ERR_INVALID
    assert lib.pkv_append(null, null, 3, null, null, null, 8, 16, 4, 100, 1, null) == pkv.PKV_ERR_INVALID
    assert lib.pkv_copy_blocks(None, None, 1, null, 1, 8, 100, null) == pkv.PKV_ERR_INVALID
    assert lib.pkv_copy_blocks(None, None, 1, null, 0, 8, 4096, null) == pkv.PKV_OK


def test_misaligned_rows_and_pools_are_refused_before_launch():
    # Kernels move 16 bytes per lane; odd addresses (never dereferenced)
    # must be refused on the host.
    lib = pkv._lib
    null = ctypes.c_void_p(0)
    odd, even = ctypes.c_void_p(0x1008), ctypes.c_void_p(0x1000)
    f16 = pkv.PKV_F16

    def decode(q=even, pool=even):
        return lib.pkv_attention_decode(even, q, pool, pool, even, 4, even, 64, 1, 4, 128, 16, 8, 1.0, f16, 8, null,
                                        0, null)

    assert decode(q=odd) == pkv.PKV_ERR_INVALID
    assert b"16-byte aligned" in lib.pkv_last_error()
    assert decode(pool=odd) == pkv.PKV_ERR_INVALID
    assert b"16-byte aligned" in lib.pkv_last_error()
    assert decode() == pkv.PKV_ERR_INVALID                  # aligned, but no workspace
    assert b"workspace" in lib.pkv_last_error()
    assert lib.pkv_append(odd, even, 3, even, even, even, 8, 16, 4, 128, f16, null) == pkv.PKV_ERR_INVALID
    assert lib.pkv_append(even, even, 3, even, odd, even, 8, 16, 4, 128, f16, null) == pkv.PKV_ERR_INVALID
    pools_ok = (ctypes.c_void_p * 2)(0x1000, 0x2000)
    pools_odd = (ctypes.c_void_p * 2)(0x1000, 0x2008)
    st = lib.pkv_copy_blocks(pools_ok, pools_odd, 2, even, 1, 8, 4096, null)
    assert st == pkv.PKV_ERR_INVALID and b"layer 1" in lib.pkv_last_error()


def test_fused_grouped_calls_reject_bad_arguments_before_launch():
    lib = pkv._lib
    null = ctypes.c_void_p(0)
    odd = ctypes.c_void_p(0x1008)   # never dereferenced: rejected first
    f16, f32, fp8 = pkv.PKV_F16, pkv.PKV_F32, pkv.PKV_FP8_E4M3

    def dense(batch=1, dt=f16, rows=null):
        return lib.pkv_append_attention_decode_grouped(odd, odd, rows, rows, odd, odd, odd, 4, odd, 64, batch, 4, 128,
                                                       16, 8, 1.0, dt, odd, null, 0, 0, null, 0, null)

    assert dense() == pkv.PKV_ERR_INVALID                   # null new rows
    assert dense(rows=odd, dt=f32) == pkv.PKV_ERR_INVALID   # grouped decode runs on f16 / bf16 caches
    assert dense(batch=0) == pkv.PKV_OK

    def quant(batch=1, qdt=f16, rows=null):
        return lib.pkv_append_attention_decode_grouped_quant(odd, odd, rows, rows, odd, odd, odd, odd, odd, 4, odd, 64,
                                                             batch, 4, 128, 16, 8, 1.0, qdt, fp8, odd, null, 0, 0,
                                                             null, 0, null)

    assert quant() == pkv.PKV_ERR_INVALID                   # null new rows
    assert quant(rows=odd) == pkv.PKV_ERR_INVALID           # misaligned new rows
    assert quant(batch=0) == pkv.PKV_OK


def test_quant_calls_reject_bad_arguments_before_launch():
    lib = pkv._lib
    null = ctypes.c_void_p(0)
    odd = ctypes.c_void_p(0x1008)   # never dereferenced: rejected as misaligned first
    f16, i8, fp8 = pkv.PKV_F16, pkv.PKV_I8, pkv.PKV_FP8_E4M3

    def decode(batch=1, hd=128, bs=16, qdt=f16, cdt=fp8, wg=0, ptr=null, scales=null):
        return lib.pkv_attention_decode_quant(ptr, ptr, ptr, ptr, scales, scales, ptr, 4, ptr, 64, batch, 4, hd, bs,
                                              8, 1.0, qdt, cdt, wg, null, 0, null)

    assert decode(hd=96) == pkv.PKV_ERR_INVALID
    assert decode(cdt=f16) == pkv.PKV_ERR_INVALID           # not an 8-bit cache
    assert decode(qdt=i8) == pkv.PKV_ERR_INVALID            # queries are never 8-bit
    assert decode(wg=-1) == pkv.PKV_ERR_INVALID
    assert decode() == pkv.PKV_ERR_INVALID                  # null scale pools
    assert decode(ptr=odd, scales=odd) == pkv.PKV_ERR_INVALID
    assert decode(batch=0) == pkv.PKV_OK

    def append(T=3, hd=128, sdt=f16, cdt=i8, ptr=null):
        return lib.pkv_append_quant(ptr, ptr, T, ptr, ptr, ptr, ptr, ptr, 8, 16, 4, hd, sdt, cdt, null)

    assert append(T=0) == pkv.PKV_OK
    assert append() == pkv.PKV_ERR_INVALID                  # null pointers
    assert append(ptr=odd) == pkv.PKV_ERR_INVALID           # misaligned
    assert append(cdt=pkv.PKV_BF16) == pkv.PKV_ERR_INVALID
    assert append(sdt=fp8) == pkv.PKV_ERR_INVALID
    assert append(hd=80) == pkv.PKV_ERR_INVALID


def test_time_next_decode_takes_null_events():
    assert pkv._lib.pkv_time_next_decode(None, None) == pkv.PKV_OK
    # consumed by the next decode call, here one refused before any launch
    st = pkv._lib.pkv_attention_decode(None, None, None, None, None, 1, None, 1, 1, 4, 100, 16, 4, 1.0,
                                       pkv.PKV_F16, 0, None, 0, None)
    assert st == pkv.PKV_ERR_INVALID


def test_grouped_call_rejects_bad_arguments_before_launch():
    lib = pkv._lib

    def grouped(batch=1, dtype=pkv.PKV_F16, hd=128, n_tiles=0, spb=None):
        return lib.pkv_attention_decode_grouped(None, None, None, None, None, 4, None, 64, batch, 4, hd, 16, 8, 1.0,
                                                dtype, spb, None, n_tiles, 0, None, 0, None)

    assert grouped(dtype=pkv.PKV_F32) == pkv.PKV_ERR_INVALID   # the matrix-core path is f16 / bf16 only
    assert grouped(hd=96) == pkv.PKV_ERR_INVALID
    assert grouped(n_tiles=-1) == pkv.PKV_ERR_INVALID
    assert grouped(n_tiles=(1 << 22) + 1) == pkv.PKV_ERR_INVALID  # beyond the prefix grid's cap
    assert grouped() == pkv.PKV_ERR_INVALID                    # null prefix lengths with a non-empty batch
    assert grouped(batch=0, n_tiles=1 << 22) == pkv.PKV_OK      # empty batch: nothing to do


def test_workspace_queries():
    up = lambda x: -(-x // 256) * 256  # noqa: E731
    b, h, d, wg = 32, 32, 128, 512
    # plan (2 int32 per sequence) + 2*wg partial pieces of h*(d floats + (m, l))
    want = up(b * 8) + up(2 * wg * h * d * 4) + up(2 * wg * h * 8)
    assert pkv.pkv_decode_workspace_bytes(b, h, d, "f16", wg) == want
    # 160 heads at fp16 x 128: 40 wavefronts -> 3 head slices of <= 16 wavefronts
    want = up(b * 3 * 8) + up(2 * wg * 160 * d * 4) + up(2 * wg * 160 * 8)
    assert pkv.pkv_decode_workspace_bytes(b, 160, d, "bf16", wg) == want
    # The plan holds at most one launch's worth of sequences (5460 per head slice).
    big = pkv.pkv_decode_workspace_bytes(20000, 4, 64, "f32", 8)
    assert big == up(5460 * 8) + up(2 * 8 * 4 * 64 * 4) + up(2 * 8 * 4 * 8)
    assert pkv.pkv_decode_workspace_bytes(b, h, 96, "f16", wg) == 0
    # 8-bit caches: 16 elements per lane -> 8 heads per wavefront at 128, at
    # most 8 wavefronts per work-group.
    assert pkv.pkv_decode_workspace_bytes(b, h, d, "fp8", wg) == (
        up(b * 8) + up(2 * wg * h * d * 4) + up(2 * wg * h * 8))
    assert pkv.pkv_decode_workspace_bytes(b, 160, d, "i8", wg) == (
        up(b * 3 * 8) + up(2 * wg * 160 * d * 4) + up(2 * wg * 160 * 8))
    assert pkv.pkv_decode_workspace_bytes(b, 256, 64, "i8", wg) == (
        up(b * 2 * 8) + up(2 * wg * 256 * 64 * 4) + up(2 * wg * 256 * 8))
    assert pkv.pkv_decode_workspace_bytes(b, h, d, "f16", -1) == 0
    # grouped: one more piece slot per sequence, then 16 parts of prefix states
    for dt in ("f16", "bf16", "fp8", "i8"):
        want = up(b * 8) + up((2 * wg + b) * h * d * 4) + up((2 * wg + b) * h * 8) + up(16 * b * h * (d + 4) * 4)
        assert pkv.pkv_decode_grouped_workspace_bytes(b, h, d, dt, wg) == want
    assert pkv.pkv_decode_grouped_workspace_bytes(b, h, d, "f32", wg) == 0


def test_one_hip_runtime_per_process():
    # Importing the binding first must not load a second HIP runtime beside
    # the one torch brings: the library has to share torch's streams.
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "import paged_attention_amd\n"
        "import torch\n"
        "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}\n"
        "print(len(paths), sorted(paths))\n"
    ) % ROOT
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, check=True).stdout
    assert out.startswith("1 "), out
