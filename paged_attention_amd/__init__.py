"""Python binding of libpkv: paged-KV decode attention for MI355X (gfx950).

A thin ctypes layer over the C interface in ``include/pkv.h``: every function
here checks tensor shapes and dtypes, passes raw pointers and the current
HIP stream, and turns status codes into exceptions.  All computation happens
in the library (HIP kernels and the C++ allocator); there is no Python or CPU
fallback, and importing this package fails loudly if ``libpkv.so`` has not
been built (``python paged_attention_amd/build.py``).

Entry points keep the C names:

* :class:`BlockAllocator` — ``pkv_allocator_*``, ``pkv_block_*``, ``pkv_seq_*``
* :func:`pkv_append`, :func:`pkv_copy_blocks`, :func:`pkv_attention_decode`,
  :func:`pkv_decode_workspace_bytes`, :func:`pkv_decode_work_groups`
* 8-bit caches: :func:`pkv_append_quant`, :func:`pkv_attention_decode_quant`
  (code pools of one-byte elements plus float32 scale pools ``[NB][H][bs]``)
"""

from __future__ import annotations

import ctypes
import math
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpkv.so")

PKV_OK = 0
PKV_ERR_INVALID = -1
PKV_ERR_NO_BLOCKS = -2
PKV_ERR_BAD_BLOCK = -3
PKV_ERR_REFCOUNT = -4
PKV_ERR_HIP = -5

PKV_F32, PKV_F16, PKV_BF16, PKV_I8, PKV_FP8_E4M3 = 0, 1, 2, 3, 4
DTYPE_CODES = {"f32": PKV_F32, "f16": PKV_F16, "bf16": PKV_BF16, "i8": PKV_I8, "fp8": PKV_FP8_E4M3}
CACHE_FORMATS = ("i8", "fp8")   # 8-bit cache formats: int8 codes, OCP FP8 E4M3 codes


class PkvError(RuntimeError):
    """A libpkv call returned an error status."""

    def __init__(self, status: int, detail: str):
        super().__init__(f"{detail} (status {status})")
        self.status = status


class OutOfBlocks(PkvError):
    """The block pool cannot satisfy a request; nothing was taken."""


class InvalidArgument(PkvError, ValueError):
    pass


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python paged_attention_amd/build.py`")
    # torch opens its own HIP runtime by path.  Loading it first lets the
    # library's libamdhip64.so.7 dependency resolve to that same runtime;
    # otherwise the process holds two runtimes and torch's streams and
    # device state are unknown to the library's.
    import torch  # noqa: F401

    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    p32 = p64 = vp  # host arrays are passed as raw addresses
    sig = {
        "pkv_strerror": (ctypes.c_char_p, [ctypes.c_int]),
        "pkv_last_error": (ctypes.c_char_p, []),
        "pkv_version": (ctypes.c_int, []),
        "pkv_time_next_decode": (ctypes.c_int, [vp, vp]),
        "pkv_prefix_tiles": (ctypes.c_int, [p32, i32, p32, i32, i32, i32, p32, p32, i32, vp]),
        "pkv_decode_grouped_workspace_bytes": (sz, [i32, i32, i32, ctypes.c_int, i32]),
        "pkv_attention_decode_grouped": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                                        ctypes.c_float, ctypes.c_int, vp, vp, i32, i32, vp, sz, vp]),
        "pkv_attention_decode_grouped_quant": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                                              i32, i32, i32, ctypes.c_float, ctypes.c_int,
                                                              ctypes.c_int, vp, vp, i32, i32, vp, sz, vp]),
        "pkv_allocator_create": (ctypes.c_int, [i32, i32, p32, ctypes.POINTER(vp)]),
        "pkv_allocator_destroy": (None, [vp]),
        "pkv_block_alloc": (ctypes.c_int, [vp, p32]),
        "pkv_blocks_alloc": (ctypes.c_int, [vp, i32, p32]),
        "pkv_block_incref": (ctypes.c_int, [vp, i32]),
        "pkv_block_decref": (ctypes.c_int, [vp, i32]),
        "pkv_block_refcount": (ctypes.c_int, [vp, i32]),
        "pkv_num_free": (i32, [vp]),
        "pkv_num_blocks": (i32, [vp]),
        "pkv_block_size": (i32, [vp]),
        "pkv_free_list": (ctypes.c_int, [vp, p32, i32]),
        "pkv_seq_fork": (ctypes.c_int, [vp, p32, i32, p32]),
        "pkv_seq_reserve": (ctypes.c_int, [vp, p32, i32, p32, i32, i32, p64, p32, p32]),
        "pkv_seq_reserve_batch": (ctypes.c_int, [vp, p32, i32, p32, p32, p32, i32, p64, p32, i32, p32]),
        "pkv_seq_release": (ctypes.c_int, [vp, p32, i32]),
        "pkv_prefix_cache_enable": (ctypes.c_int, [vp]),
        "pkv_prefix_block_keys": (ctypes.c_int, [p32, i32, i32, vp, i32]),
        "pkv_prefix_match": (ctypes.c_int, [vp, p32, i32, p32, i32, p32]),
        "pkv_prefix_register": (ctypes.c_int, [vp, p32, i32, p32, i32, i32, p32]),
        "pkv_prefix_cached_blocks": (i32, [vp]),
        "pkv_prefix_lru": (ctypes.c_int, [vp, p32, i32]),
        "pkv_append": (ctypes.c_int, [vp, vp, i32, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int, vp]),
        "pkv_copy_blocks": (ctypes.c_int, [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32, i32, sz, vp]),
        "pkv_decode_work_groups": (i32, [ctypes.c_int]),
        "pkv_swap_blocks": (ctypes.c_int, [ctypes.POINTER(vp), ctypes.POINTER(vp), i32, vp, i32, i32, i32, sz, vp]),
        "pkv_decode_workspace_bytes": (sz, [i32, i32, i32, ctypes.c_int, i32]),
        "pkv_attention_decode_scratch": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                                        ctypes.c_float, ctypes.c_int, i32, vp]),
        "pkv_attention_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                                ctypes.c_float, ctypes.c_int, i32, vp, sz, vp]),
        "pkv_append_quant": (ctypes.c_int, [vp, vp, i32, vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_int,
                                            ctypes.c_int, vp]),
        "pkv_attention_decode_quant": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                                      i32, ctypes.c_float, ctypes.c_int, ctypes.c_int, i32, vp, sz,
                                                      vp]),
        "pkv_decode_scores_workspace_bytes": (sz, [i32, i32, i32]),
        "pkv_attention_decode_scores": (ctypes.c_int, [vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32, i32,
                                                       ctypes.c_float, ctypes.c_int, i32, vp, sz, vp, i32,
                                                       ctypes.c_float, vp, sz, vp]),
        "pkv_attention_decode_quant_scores": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                                             i32, i32, i32, ctypes.c_float, ctypes.c_int,
                                                             ctypes.c_int, i32, vp, sz, vp, i32, ctypes.c_float,
                                                             vp, sz, vp]),
        "pkv_append_attention_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32, i32, i32,
                                                       i32, ctypes.c_float, ctypes.c_int, i32, vp, sz, vp]),
        "pkv_append_attention_decode_quant": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32,
                                                             i32, i32, i32, i32, ctypes.c_float, ctypes.c_int,
                                                             ctypes.c_int, i32, vp, sz, vp]),
        "pkv_append_attention_decode_grouped": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, i32, vp, i32, i32, i32,
                                                               i32, i32, i32, ctypes.c_float, ctypes.c_int, vp, vp,
                                                               i32, i32, vp, sz, vp]),
        "pkv_append_attention_decode_grouped_quant": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i32, vp, i32,
                                                                     i32, i32, i32, i32, i32, ctypes.c_float,
                                                                     ctypes.c_int, ctypes.c_int, vp, vp, i32, i32, vp,
                                                                     sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _check(status: int) -> int:
    if status >= 0:
        return status
    detail = _lib.pkv_last_error().decode() or _lib.pkv_strerror(status).decode()
    if status == PKV_ERR_NO_BLOCKS:
        raise OutOfBlocks(status, detail)
    if status == PKV_ERR_INVALID:
        raise InvalidArgument(status, detail)
    raise PkvError(status, detail)


def version() -> int:
    return _lib.pkv_version()


def _ptr(arr: np.ndarray):
    # The array interface is far cheaper than numpy's .ctypes attribute.
    return ctypes.c_void_p(arr.__array_interface__["data"][0])


_i32p = _ptr
_i64p = _ptr


def _host_array(arr, dtype, name, ndim=None, size=None, size_at_least=None) -> None:
    """Checks a host array handed to the library as a raw pointer."""
    if not isinstance(arr, np.ndarray) or arr.dtype != dtype or not arr.flags.c_contiguous:
        raise ValueError(f"{name} must be a C-contiguous numpy array of {np.dtype(dtype).name}")
    if ndim is not None and arr.ndim != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, not {arr.ndim}")
    if size is not None and arr.size != size:
        raise ValueError(f"{name} must hold {size} elements, not {arr.size}")
    if size_at_least is not None and arr.size < size_at_least:
        raise ValueError(f"{name} must hold at least {size_at_least} elements, not {arr.size}")


class BlockAllocator:
    """Host block allocator (FIFO free queue + reference counts), backed by libpkv."""

    def __init__(self, num_blocks: int, block_size: int, free_order=None):
        handle = ctypes.c_void_p()
        order = None
        if free_order is not None:
            order = np.ascontiguousarray(free_order, dtype=np.int32)
            if order.shape != (num_blocks,):
                raise InvalidArgument(PKV_ERR_INVALID, "free_order must hold num_blocks ids")
        _check(_lib.pkv_allocator_create(num_blocks, block_size, _i32p(order) if order is not None else None,
                                         ctypes.byref(handle)))
        self._h = handle
        self.num_blocks = num_blocks
        self.block_size = block_size

    def close(self):
        if getattr(self, "_h", None) and _lib is not None:
            _lib.pkv_allocator_destroy(self._h)
        self._h = None

    def __del__(self):
        self.close()

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    # single blocks
    def alloc(self) -> int:
        out = ctypes.c_int32()
        _check(_lib.pkv_block_alloc(self._h, ctypes.byref(out)))
        return out.value

    def alloc_n(self, n: int, out: np.ndarray | None = None) -> np.ndarray:
        """Take ``n`` blocks at once (all or nothing); returns their ids (int32), in ``out`` if given."""
        if out is None:
            out = np.zeros(max(1, n), dtype=np.int32)
        _host_array(out, np.int32, "out", size_at_least=n)
        _check(_lib.pkv_blocks_alloc(self._h, n, _i32p(out)))
        return out[:n]

    def incref(self, block: int) -> None:
        _check(_lib.pkv_block_incref(self._h, block))

    def decref(self, block: int) -> None:
        _check(_lib.pkv_block_decref(self._h, block))

    def refcount(self, block: int) -> int:
        return _check(_lib.pkv_block_refcount(self._h, block))

    def num_free(self) -> int:
        return _lib.pkv_num_free(self._h)

    def free_list(self) -> list:
        buf = np.zeros(max(1, self.num_blocks), dtype=np.int32)
        n = _check(_lib.pkv_free_list(self._h, _i32p(buf), self.num_blocks))
        return buf[:n].tolist()

    # sequences over Python lists (convenience) ---------------------------
    def fork(self, row) -> list:
        src = np.ascontiguousarray(row, dtype=np.int32)
        dst = np.zeros(max(1, len(src)), dtype=np.int32)
        _check(_lib.pkv_seq_fork(self._h, _i32p(src), len(src), _i32p(dst)))
        return dst[: len(src)].tolist()

    def reserve(self, row: list, cur_len: int, n_new: int, capacity: int | None = None):
        """Grow ``row`` (a list, updated in place) by n_new positions; returns (slots, pairs)."""
        bs = self.block_size
        cap = capacity if capacity is not None else -(-(cur_len + n_new) // bs) + 1
        buf = np.zeros(max(cap, len(row), 1), dtype=np.int32)
        buf[: len(row)] = row
        nb = ctypes.c_int32(len(row))
        slots = np.zeros(max(1, n_new), dtype=np.int64)
        pair = np.zeros(2, dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.pkv_seq_reserve(self._h, _i32p(buf), len(buf), ctypes.byref(nb), cur_len, n_new, _i64p(slots),
                                    _i32p(pair), ctypes.byref(ncow)))
        row[:] = buf[: nb.value].tolist()
        pairs = [(int(pair[0]), int(pair[1]))] if ncow.value else []
        return slots[:n_new].tolist(), pairs

    def release(self, row) -> None:
        arr = np.ascontiguousarray(row, dtype=np.int32)
        _check(_lib.pkv_seq_release(self._h, _i32p(arr) if len(arr) else None, len(arr)))

    # sequences over numpy tables (batched, no per-sequence Python work) ---
    def reserve_batch(self, tables: np.ndarray, n_blocks: np.ndarray, cur_lens, n_new):
        """Reserve for every row of ``tables`` ([B][stride] int32, updated in place).

        ``n_blocks`` (int32 [B]) is updated in place.  Returns (slots int64
        [sum n_new], pairs int32 [k][2]).
        """
        _host_array(tables, np.int32, "tables", ndim=2)
        _host_array(n_blocks, np.int32, "n_blocks", size=tables.shape[0])
        lens = np.ascontiguousarray(cur_lens, dtype=np.int32)
        new = np.ascontiguousarray(n_new, dtype=np.int32)
        batch = tables.shape[0]
        slots = np.zeros(max(1, int(new.sum())), dtype=np.int64)
        pairs = np.zeros((max(1, batch), 2), dtype=np.int32)
        ncow = ctypes.c_int32(0)
        _check(_lib.pkv_seq_reserve_batch(self._h, _i32p(tables), tables.shape[1], _i32p(n_blocks), _i32p(lens),
                                          _i32p(new), batch, _i64p(slots), _i32p(pairs), max(1, batch),
                                          ctypes.byref(ncow)))
        return slots[: int(new.sum())], pairs[: ncow.value]

    def reserve_batch_into(self, tables: np.ndarray, n_blocks: np.ndarray, cur_lens: np.ndarray, n_new: np.ndarray,
                           slots_out: np.ndarray, pairs_out: np.ndarray) -> int:
        """As :meth:`reserve_batch`, writing into caller arrays (e.g. pinned staging
        memory); every array must already be C-contiguous of the right dtype
        (int32, slots int64).  Returns the number of copy pairs written."""
        batch = tables.shape[0] if isinstance(tables, np.ndarray) else 0
        _host_array(tables, np.int32, "tables", ndim=2)
        for arr, name in ((n_blocks, "n_blocks"), (cur_lens, "cur_lens"), (n_new, "n_new")):
            _host_array(arr, np.int32, name, size=batch)
        _host_array(slots_out, np.int64, "slots_out", size_at_least=int(np.asarray(n_new).sum()))
        _host_array(pairs_out, np.int32, "pairs_out", ndim=2)
        if pairs_out.shape[1] != 2:
            raise ValueError("pairs_out must have shape [k][2]")
        ncow = ctypes.c_int32(0)
        _check(_lib.pkv_seq_reserve_batch(self._h, _i32p(tables), tables.shape[1], _i32p(n_blocks), _i32p(cur_lens),
                                          _i32p(n_new), tables.shape[0], _i64p(slots_out), _i32p(pairs_out),
                                          pairs_out.shape[0], ctypes.byref(ncow)))
        return ncow.value

    def release_table_row(self, tables: np.ndarray, i: int, n_blocks: int) -> None:
        row = np.ascontiguousarray(tables[i, :n_blocks])
        self.release(row)

    # -- prefix cache --------------------------------------------------
    def enable_prefix_cache(self) -> None:
        _check(_lib.pkv_prefix_cache_enable(self._h))

    def prefix_match(self, tokens, capacity: int) -> list:
        """Blocks of the longest cached prefix of ``tokens`` (at most ``capacity``); each is incremented."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        capacity = max(0, min(capacity, len(toks) // self.block_size))   # only full blocks can match
        out = np.empty(max(1, capacity), dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(_lib.pkv_prefix_match(self._h, _i32p(toks) if len(toks) else None, len(toks), _i32p(out),
                                     capacity, ctypes.byref(n)))
        return out[:n.value].tolist()

    def prefix_register(self, tokens, row, n_blocks: int, first_block: int = 0) -> int:
        """Record the full blocks of a sequence under their prefix keys; returns how many were new.
        ``first_block`` = blocks ``prefix_match`` returned for these tokens (not hashed again)."""
        toks = np.ascontiguousarray(tokens, dtype=np.int32)
        arr = np.ascontiguousarray(row, dtype=np.int32)
        n = ctypes.c_int32(0)
        _check(_lib.pkv_prefix_register(self._h, _i32p(toks) if len(toks) else None, len(toks),
                                        _i32p(arr) if len(arr) else None, n_blocks, first_block, ctypes.byref(n)))
        return n.value

    def prefix_cached(self) -> int:
        return _check(_lib.pkv_prefix_cached_blocks(self._h))

    def prefix_lru(self) -> list:
        buf = np.zeros(max(1, self.num_blocks), dtype=np.int32)
        n = _check(_lib.pkv_prefix_lru(self._h, _i32p(buf), self.num_blocks))
        return buf[:n].tolist()


def prefix_block_keys(tokens, block_size: int) -> list:
    """Chained SHA-256 keys (32 bytes each) of the full blocks of ``tokens``."""
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    n = len(toks) // block_size if block_size > 0 else 0
    out = np.zeros(max(1, 32 * n), dtype=np.uint8)
    got = _check(_lib.pkv_prefix_block_keys(_i32p(toks) if len(toks) else None, len(toks), block_size, _ptr(out), n))
    return [out[32 * i:32 * (i + 1)].tobytes() for i in range(got)]


# ---------------------------------------------------------------------------
# device operations
# ---------------------------------------------------------------------------

def _torch():
    import torch

    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    codes = {torch.float32: PKV_F32, torch.float16: PKV_F16, torch.bfloat16: PKV_BF16}
    if t.dtype not in codes:
        raise InvalidArgument(PKV_ERR_INVALID, f"unsupported dtype {t.dtype}")
    return codes[t.dtype]


def _dev(t, name, dtype=None, ndim=None, pinned_ok=False):
    # Small per-step metadata may live in pinned host memory, which the GPU
    # reads directly; everything else must be device memory.
    if not (t.is_cuda or (pinned_ok and t.is_pinned())):
        kind = "a device tensor or pinned host tensor" if pinned_ok else "a device tensor"
        raise InvalidArgument(PKV_ERR_INVALID, f"{name} must be {kind}")
    if not t.is_contiguous():
        raise InvalidArgument(PKV_ERR_INVALID, f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise InvalidArgument(PKV_ERR_INVALID, f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise InvalidArgument(PKV_ERR_INVALID, f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _append_args(k_new, v_new, slot_mapping, k_cache, v_cache, stream):
    torch = _torch()
    nb, bs, h, d = k_cache.shape
    if k_new.shape[1:] != (h, d) or v_new.shape != k_new.shape or v_cache.shape != k_cache.shape:
        raise InvalidArgument(PKV_ERR_INVALID, "append: shape mismatch")
    if k_new.dtype != k_cache.dtype or v_new.dtype != k_cache.dtype or v_cache.dtype != k_cache.dtype:
        raise InvalidArgument(PKV_ERR_INVALID, "append: dtype mismatch")
    if slot_mapping.shape != (k_new.shape[0],):
        raise InvalidArgument(PKV_ERR_INVALID, "append: slot_mapping must be [T]")
    return [_dev(k_new, "k_new"), _dev(v_new, "v_new"), k_new.shape[0],
            _dev(slot_mapping, "slot_mapping", torch.int64, pinned_ok=True),
            _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4), nb, bs, h, d, _dtype_code(k_cache),
            _stream(stream)]


def pkv_append(k_new, v_new, slot_mapping, k_cache, v_cache, stream=None) -> None:
    """Scatter rows ``k_new[t]``/``v_new[t]`` ([T][H][D]) to flat slot ``slot_mapping[t]``."""
    _check(_lib.pkv_append(*_append_args(k_new, v_new, slot_mapping, k_cache, v_cache, stream)))


def pkv_copy_blocks(k_caches, v_caches, pairs, stream=None) -> None:
    """Copy blocks ``pairs[i, 0] -> pairs[i, 1]`` in every layer's K and V pool.

    A pool is any tensor whose first dimension is the block id: K/V pools
    ``[NB][bs][H][D]`` and also the ``[NB][H][bs]`` scale pools of 8-bit caches
    (copy those with a second call).
    """
    torch = _torch()
    if len(k_caches) != len(v_caches) or not k_caches:
        raise InvalidArgument(PKV_ERR_INVALID, "copy_blocks: need matching non-empty layer lists")
    nb = k_caches[0].shape[0]
    for t in list(k_caches) + list(v_caches):
        if t.shape != k_caches[0].shape or t.dtype != k_caches[0].dtype:
            raise InvalidArgument(PKV_ERR_INVALID, "copy_blocks: layer pools differ in shape or dtype")
        if t.dim() < 2:
            raise InvalidArgument(PKV_ERR_INVALID, "copy_blocks: a pool is [num_blocks][...]")
        _dev(t, "pool")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise InvalidArgument(PKV_ERR_INVALID, "copy_blocks: pairs must be [n][2]")
    nl = len(k_caches)
    karr = (ctypes.c_void_p * nl)(*[t.data_ptr() for t in k_caches])
    varr = (ctypes.c_void_p * nl)(*[t.data_ptr() for t in v_caches])
    bytes_per_block = k_caches[0][0].numel() * k_caches[0].element_size()
    _check(_lib.pkv_copy_blocks(karr, varr, nl, _dev(pairs, "pairs", torch.int32, pinned_ok=True), pairs.shape[0], nb,
                                bytes_per_block, _stream(stream)))


def pkv_swap_blocks(dst_pools, src_pools, pairs, stream=None) -> None:
    """Copy blocks ``pairs[i, 0]`` of every source pool to ``pairs[i, 1]`` of the matching destination
    pool; one side is device memory, the other device or pinned host memory (preemption swap)."""
    torch = _torch()
    if len(dst_pools) != len(src_pools) or not dst_pools:
        raise InvalidArgument(PKV_ERR_INVALID, "swap_blocks: need matching non-empty pool lists")
    per_block = src_pools[0][0].numel() * src_pools[0].element_size()
    for t in list(dst_pools) + list(src_pools):
        if t.dim() < 2 or t[0].numel() * t.element_size() != per_block or not t.is_contiguous():
            raise InvalidArgument(PKV_ERR_INVALID, "swap_blocks: pools must be contiguous [num_blocks][...] alike")
        if not (t.is_cuda or t.is_pinned()):
            raise InvalidArgument(PKV_ERR_INVALID, "swap_blocks: pools must be device or pinned host tensors")
    if pairs.dim() != 2 or pairs.shape[1] != 2:
        raise InvalidArgument(PKV_ERR_INVALID, "swap_blocks: pairs must be [n][2]")
    n = len(dst_pools)
    darr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in dst_pools])
    sarr = (ctypes.c_void_p * n)(*[t.data_ptr() for t in src_pools])
    _check(_lib.pkv_swap_blocks(darr, sarr, n, _dev(pairs, "pairs", torch.int32, pinned_ok=True), pairs.shape[0],
                                src_pools[0].shape[0], dst_pools[0].shape[0], per_block, _stream(stream)))


def _event_handle(ev):
    if ev is None:
        return None
    if isinstance(ev, int):
        return ev
    h = ev.cuda_event   # torch.cuda.Event: the HIP event exists once it has been recorded
    if not h:
        raise InvalidArgument(PKV_ERR_INVALID, "time_next_decode: record the event once before passing it")
    return h


def pkv_time_next_decode(start=None, stop=None) -> None:
    """Kernel timestamps of this thread's next decode-attention call.

    ``start`` / ``stop`` are ``torch.cuda.Event(enable_timing=True)`` objects
    that have been recorded at least once (or raw HIP event handles); the next
    decode call records ``start`` at the start of its first kernel and
    ``stop`` at the end of its last, with no extra packet on the queue.
    """
    _check(_lib.pkv_time_next_decode(_event_handle(start), _event_handle(stop)))


def pkv_decode_work_groups(cache_dtype: str = "f16") -> int:
    """Work-groups decode attention launches by default on the current device for this cache type."""
    if cache_dtype not in DTYPE_CODES:
        raise InvalidArgument(PKV_ERR_INVALID, f"unknown dtype {cache_dtype!r}")
    return _check(_lib.pkv_decode_work_groups(DTYPE_CODES[cache_dtype]))


def pkv_decode_workspace_bytes(batch, num_heads, head_dim, dtype, work_groups=0) -> int:
    return int(_lib.pkv_decode_workspace_bytes(batch, num_heads, head_dim, DTYPE_CODES[dtype], work_groups))


_DT_NAMES = {PKV_F32: "f32", PKV_F16: "f16", PKV_BF16: "bf16", PKV_I8: "i8", PKV_FP8_E4M3: "fp8"}


def _bytes_on(nbytes, device, stream):
    """A uint8 tensor allocated for use on ``stream`` (the current stream when None).

    torch's caching allocator hands a freed block back only to later work on
    the stream it was allocated on, so a workspace the wrappers drop right
    after enqueueing a call on ``stream`` cannot be reused by work on another
    stream while that call's kernels still write it.
    """
    torch = _torch()
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def decode_workspace(batch, num_heads, head_dim, dtype, work_groups=0, device="cuda", stream=None):
    """Allocate a workspace for these decode sizes (a uint8 tensor) for use on ``stream``."""
    need = pkv_decode_workspace_bytes(batch, num_heads, head_dim, dtype, work_groups)
    if need == 0:
        detail = _lib.pkv_last_error().decode()
        raise InvalidArgument(PKV_ERR_INVALID, f"decode_workspace: unsupported sizes ({detail})")
    return _bytes_on(need, device, stream)


def _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, work_groups, workspace,
                 stream):
    torch = _torch()
    nb, bs, h, d = k_cache.shape
    batch = q.shape[0]
    if q.shape != (batch, h, d) or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode: shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode: dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or seq_lens.shape != (batch,):
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode: tables must be [B][max_blocks], lens [B]")
    code = _dtype_code(q)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(max(batch, 1), h, d, _DT_NAMES[code], work_groups, q.device, stream)
    args = [_dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
            _dev(block_tables, "block_tables", torch.int32, pinned_ok=True), block_tables.shape[1],
            _dev(seq_lens, "seq_lens", torch.int32, pinned_ok=True), int(max_seq_len), batch, h, d, bs, nb,
            float(scale), code,
            int(work_groups), _dev(workspace, "workspace"), workspace.numel() * workspace.element_size(),
            _stream(stream)]
    return args, workspace


def pkv_attention_decode(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale=None,
                         work_groups=0, workspace=None, stream=None) -> None:
    """Decode attention of ``q`` ([B][H][D]) over each sequence's paged K/V; writes ``out``."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, work_groups,
                           workspace, stream)
    _check(_lib.pkv_attention_decode(*args))


DECODE_SCRATCH_BYTES = 32 << 20   # PKV_DECODE_SCRATCH_BYTES


def pkv_attention_decode_scratch(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale=None,
                                 work_groups=0, stream=None) -> None:
    """pkv_attention_decode with the library's own device scratch as workspace: allocates nothing.

    Calls on one device share that scratch; they must not overlap (one stream, in order).
    """
    torch = _torch()
    nb, bs, h, d = k_cache.shape
    batch = q.shape[0]
    if q.shape != (batch, h, d) or out.shape != q.shape or v_cache.shape != k_cache.shape:
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_scratch: shape mismatch")
    if not (q.dtype == out.dtype == k_cache.dtype == v_cache.dtype):
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_scratch: dtype mismatch")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or seq_lens.shape != (batch,):
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_scratch: tables must be [B][max_blocks], lens [B]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    _check(_lib.pkv_attention_decode_scratch(
        _dev(out, "out"), _dev(q, "q"), _dev(k_cache, "k_cache", ndim=4), _dev(v_cache, "v_cache", ndim=4),
        _dev(block_tables, "block_tables", torch.int32, pinned_ok=True), block_tables.shape[1],
        _dev(seq_lens, "seq_lens", torch.int32, pinned_ok=True), int(max_seq_len), batch, h, d, bs, nb,
        float(scale), _dtype_code(q), int(work_groups), _stream(stream)))


PREFIX_TILE_SEQS, PREFIX_TILE_INTS, PREFIX_MAX_BLOCKS = 16, 18, 1024


def prefix_tiles(tables, seq_lens, block_size: int, min_sharers: int = 2):
    """Groups of sequences sharing leading blocks (pkv_prefix_tiles), on the host.

    ``tables`` [B][max_blocks] and ``seq_lens`` [B] are host int32 arrays (this
    step's); returns ``(seq_prefix_blocks [B], tiles [n][PREFIX_TILE_INTS])``,
    both int32 numpy arrays.
    """
    tables = np.ascontiguousarray(tables, dtype=np.int32)
    lens = np.ascontiguousarray(seq_lens, dtype=np.int32)
    if tables.ndim != 2 or lens.shape != (tables.shape[0],):
        raise InvalidArgument(PKV_ERR_INVALID, "prefix_tiles: tables must be [B][max_blocks], lens [B]")
    batch, maxb = tables.shape
    cap = max(1, (batch + 1) // 2)
    spb = np.zeros(max(batch, 1), dtype=np.int32)
    tiles = np.full((cap, PREFIX_TILE_INTS), -1, dtype=np.int32)
    n = ctypes.c_int32(0)
    _check(_lib.pkv_prefix_tiles(_ptr(tables), maxb, _ptr(lens), batch, int(block_size), int(min_sharers), _ptr(spb),
                                 _ptr(tiles), cap, ctypes.byref(n)))
    return spb[:batch].copy(), tiles[: n.value].copy()


def pkv_decode_grouped_workspace_bytes(batch, num_heads, head_dim, dtype, work_groups=0) -> int:
    return int(_lib.pkv_decode_grouped_workspace_bytes(batch, num_heads, head_dim, DTYPE_CODES[dtype], work_groups))


def _grouped_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, seq_prefix_blocks, tiles, scale,
                  work_groups, workspace, stream):
    torch = _torch()
    batch, h, d = q.shape
    if workspace is None:
        need = pkv_decode_grouped_workspace_bytes(max(batch, 1), h, d, _DT_NAMES[_dtype_code(q)], work_groups)
        if need == 0:
            raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_grouped: unsupported sizes")
        workspace = _bytes_on(need, q.device, stream)
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, work_groups,
                           workspace, stream)
    if seq_prefix_blocks.shape != (batch,) or tiles.dim() != 2 or tiles.shape[1] != PREFIX_TILE_INTS:
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_grouped: seq_prefix_blocks [B], tiles [n][18]")
    grouped = [_dev(seq_prefix_blocks, "seq_prefix_blocks", torch.int32, pinned_ok=True),
               _dev(tiles, "tiles", torch.int32, pinned_ok=True) if tiles.shape[0] else None, tiles.shape[0]]
    # the plain argument list with the prefix arrays before the work-group count
    return args[:15] + grouped + args[15:], workspace


def pkv_attention_decode_grouped(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, seq_prefix_blocks,
                                 tiles, scale=None, work_groups=0, workspace=None, stream=None) -> None:
    """pkv_attention_decode with shared prefixes read once per tile.

    ``seq_prefix_blocks`` [B] and ``tiles`` [n][PREFIX_TILE_INTS] are int32
    tensors (device or pinned host) as prefix_tiles returns them for the same
    tables and lengths; f16 or bf16 caches.
    """
    if q.shape[0] == 0:
        return
    args, _ = _grouped_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, seq_prefix_blocks, tiles,
                            scale, work_groups, workspace, stream)
    _check(_lib.pkv_attention_decode_grouped(*args))


class PreparedDecode:
    """A pkv_attention_decode call whose arguments are checked once.

    ``launch(q, out)`` only swaps the query/output pointers (tensors of the
    same shape and dtype as at preparation) and enqueues the kernels; it is
    meant for decode loops where Python overhead would otherwise dominate.
    ``set_metadata`` repoints the tables and lengths (same shapes).  The
    tensors given at preparation must stay alive and in place.
    """

    def __init__(self, out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale=None, work_groups=0,
                 workspace=None, stream=None, scores=None, decay=0.995, scores_ws=None, prefix=None):
        if prefix is not None:   # grouped call: prefix = (seq_prefix_blocks, tiles)
            if scores is not None:
                raise InvalidArgument(PKV_ERR_INVALID, "prepared decode: scores and prefix groups do not combine")
            self._args, ws = _grouped_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, prefix[0],
                                           prefix[1], scale, work_groups, workspace, stream)
            self._keep = (k_cache, v_cache, block_tables, seq_lens, ws, prefix)
            self._shape, self._dtype = tuple(q.shape), q.dtype
            self._fn = _lib.pkv_attention_decode_grouped
            self._ti = 4
            return
        self._args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale,
                                      work_groups, workspace, stream)
        self._keep = (k_cache, v_cache, block_tables, seq_lens, ws)
        self._shape, self._dtype = tuple(q.shape), q.dtype
        self._fn = _lib.pkv_attention_decode
        if scores is not None:   # also update cumulative attention scores
            extra, sws = _score_args(scores, q, max_seq_len, decay, scores_ws, stream)
            self._args = self._args[:-1] + extra + self._args[-1:]
            self._keep = self._keep + (scores, sws)
            self._fn = _lib.pkv_attention_decode_scores
        self._ti = 4   # argument index of block_tables (max_blocks and seq_lens follow)

    def _swap(self, i, t, what):
        if tuple(t.shape) != self._shape or t.dtype != self._dtype or not t.is_contiguous() or not t.is_cuda:
            raise InvalidArgument(PKV_ERR_INVALID, f"prepared call: {what} differs from the prepared tensor")
        self._args[i] = ctypes.c_void_p(t.data_ptr())

    def set_metadata(self, block_tables, seq_lens) -> None:
        """Point the call at other tables/lengths of the prepared shapes (device or pinned host)."""
        torch = _torch()
        ti = self._ti
        if tuple(block_tables.shape) != (self._shape[0], self._args[ti + 1]) or \
                tuple(seq_lens.shape) != (self._shape[0],):
            raise InvalidArgument(PKV_ERR_INVALID, "prepared decode: metadata shapes differ")
        self._args[ti] = _dev(block_tables, "block_tables", torch.int32, pinned_ok=True)
        self._args[ti + 2] = _dev(seq_lens, "seq_lens", torch.int32, pinned_ok=True)
        self._meta = (block_tables, seq_lens)   # kept alive while the call points at them

    def launch(self, q=None, out=None) -> None:
        if q is not None:
            self._swap(1, q, "q")
        if out is not None:
            self._swap(0, out, "out")
        _check(self._fn(*self._args))


class PreparedAppend(PreparedDecode):
    """A pkv_append call checked once; ``launch(k_new, v_new)`` swaps the new rows."""

    def __init__(self, k_new, v_new, slot_mapping, k_cache, v_cache, stream=None):  # noqa: D107
        self._args = _append_args(k_new, v_new, slot_mapping, k_cache, v_cache, stream)
        self._keep = (slot_mapping, k_cache, v_cache)
        self._shape, self._dtype = tuple(k_new.shape), k_new.dtype

    def set_slots(self, slot_mapping) -> None:
        """Point the call at another slot array of the prepared length (device or pinned host)."""
        torch = _torch()
        if tuple(slot_mapping.shape) != (self._shape[0],):
            raise InvalidArgument(PKV_ERR_INVALID, "prepared append: slot_mapping shape differs")
        self._args[3] = _dev(slot_mapping, "slot_mapping", torch.int64, pinned_ok=True)
        self._meta = (slot_mapping,)

    def launch(self, k_new=None, v_new=None) -> None:
        if k_new is not None:
            self._swap(0, k_new, "k_new")
        if v_new is not None:
            self._swap(1, v_new, "v_new")
        _check(_lib.pkv_append(*self._args))



# ---------------------------------------------------------------------------
# 8-bit caches
# ---------------------------------------------------------------------------

def _fmt_code(cache_dtype: str) -> int:
    if cache_dtype not in CACHE_FORMATS:
        raise InvalidArgument(PKV_ERR_INVALID, f"cache_dtype must be one of {CACHE_FORMATS}, got {cache_dtype!r}")
    return DTYPE_CODES[cache_dtype]


def _q8_pools(k_cache, v_cache, k_scales, v_scales, what):
    torch = _torch()
    if k_cache.dim() != 4 or v_cache.shape != k_cache.shape:
        raise InvalidArgument(PKV_ERR_INVALID, f"{what}: code pools must be [NB][bs][H][D] and alike")
    if k_cache.element_size() != 1 or v_cache.element_size() != 1:
        raise InvalidArgument(PKV_ERR_INVALID, f"{what}: code pools hold one-byte elements")
    nb, bs, h, d = k_cache.shape
    if k_scales.shape != (nb, h, bs) or v_scales.shape != (nb, h, bs):
        raise InvalidArgument(PKV_ERR_INVALID, f"{what}: scale pools must be [NB][H][bs] = {(nb, h, bs)}")
    return [_dev(k_cache, "k_cache"), _dev(v_cache, "v_cache"), _dev(k_scales, "k_scales", torch.float32),
            _dev(v_scales, "v_scales", torch.float32)], (nb, bs, h, d)


def _append_quant_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales, cache_dtype, stream):
    torch = _torch()
    pools, (nb, bs, h, d) = _q8_pools(k_cache, v_cache, k_scales, v_scales, "append_quant")
    if k_new.shape[1:] != (h, d) or v_new.shape != k_new.shape or v_new.dtype != k_new.dtype:
        raise InvalidArgument(PKV_ERR_INVALID, "append_quant: new rows must be [T][H][D], K and V alike")
    if slot_mapping.shape != (k_new.shape[0],):
        raise InvalidArgument(PKV_ERR_INVALID, "append_quant: slot_mapping must be [T]")
    return [_dev(k_new, "k_new"), _dev(v_new, "v_new"), k_new.shape[0],
            _dev(slot_mapping, "slot_mapping", torch.int64, pinned_ok=True), *pools, nb, bs, h, d,
            _dtype_code(k_new), _fmt_code(cache_dtype), _stream(stream)]


def pkv_append_quant(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales, cache_dtype,
                     stream=None) -> None:
    """Quantise rows ``k_new[t]``/``v_new[t]`` ([T][H][D], f32/f16/bf16) into 8-bit codes
    and per-(token, head) scales at flat slot ``slot_mapping[t]``."""
    _check(_lib.pkv_append_quant(*_append_quant_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales,
                                                     v_scales, cache_dtype, stream)))


def _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                       cache_dtype, scale, work_groups, workspace, stream):
    torch = _torch()
    pools, (nb, bs, h, d) = _q8_pools(k_cache, v_cache, k_scales, v_scales, "attention_decode_quant")
    batch = q.shape[0]
    if q.shape != (batch, h, d) or out.shape != q.shape or out.dtype != q.dtype:
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_quant: q and out must be [B][H][D], one dtype")
    if block_tables.dim() != 2 or block_tables.shape[0] != batch or seq_lens.shape != (batch,):
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_quant: tables must be [B][max_blocks], lens [B]")
    code = _fmt_code(cache_dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if workspace is None:
        workspace = decode_workspace(max(batch, 1), h, d, cache_dtype, work_groups, q.device, stream)
    args = [_dev(out, "out"), _dev(q, "q"), *pools,
            _dev(block_tables, "block_tables", torch.int32, pinned_ok=True), block_tables.shape[1],
            _dev(seq_lens, "seq_lens", torch.int32, pinned_ok=True), int(max_seq_len), batch, h, d, bs, nb,
            float(scale), _dtype_code(q), code, int(work_groups), _dev(workspace, "workspace"),
            workspace.numel() * workspace.element_size(), _stream(stream)]
    return args, workspace


def pkv_attention_decode_quant(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                               cache_dtype, scale=None, work_groups=0, workspace=None, stream=None) -> None:
    """Decode attention of ``q`` over an 8-bit paged cache (dequantised in the kernel); writes ``out``."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                 max_seq_len, cache_dtype, scale, work_groups, workspace, stream)
    _check(_lib.pkv_attention_decode_quant(*args))


def _grouped_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                        seq_prefix_blocks, tiles, cache_dtype, scale, work_groups, workspace, stream):
    torch = _torch()
    batch, h, d = q.shape
    if workspace is None:
        need = pkv_decode_grouped_workspace_bytes(max(batch, 1), h, d, cache_dtype, work_groups)
        if need == 0:
            raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_grouped_quant: unsupported sizes")
        workspace = _bytes_on(need, q.device, stream)
    args, _ = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                                 cache_dtype, scale, work_groups, workspace, stream)
    if seq_prefix_blocks.shape != (batch,) or tiles.dim() != 2 or tiles.shape[1] != PREFIX_TILE_INTS:
        raise InvalidArgument(PKV_ERR_INVALID, "attention_decode_grouped_quant: seq_prefix_blocks [B], tiles [n][18]")
    grouped = [_dev(seq_prefix_blocks, "seq_prefix_blocks", torch.int32, pinned_ok=True),
               _dev(tiles, "tiles", torch.int32, pinned_ok=True) if tiles.shape[0] else None, tiles.shape[0]]
    # the quant argument list with the prefix arrays before the work-group count
    return args[:18] + grouped + args[18:], workspace


def pkv_attention_decode_grouped_quant(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                       max_seq_len, seq_prefix_blocks, tiles, cache_dtype, scale=None,
                                       work_groups=0, workspace=None, stream=None) -> None:
    """pkv_attention_decode_quant with shared prefixes read once per tile (f16 or bf16 queries)."""
    if q.shape[0] == 0:
        return
    args, _ = _grouped_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                  max_seq_len, seq_prefix_blocks, tiles, cache_dtype, scale, work_groups, workspace,
                                  stream)
    _check(_lib.pkv_attention_decode_grouped_quant(*args))


class PreparedDecodeQuant(PreparedDecode):
    """A pkv_attention_decode_quant call checked once; ``launch(q, out)`` swaps q/out.

    With ``prefix = (seq_prefix_blocks, tiles)`` the call is
    pkv_attention_decode_grouped_quant.
    """

    def __init__(self, out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                 cache_dtype, scale=None, work_groups=0, workspace=None, stream=None, prefix=None):  # noqa: D107
        if prefix is not None:
            self._args, ws = _grouped_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables,
                                                 seq_lens, max_seq_len, prefix[0], prefix[1], cache_dtype, scale,
                                                 work_groups, workspace, stream)
            self._fn = _lib.pkv_attention_decode_grouped_quant
        else:
            self._args, ws = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables,
                                                seq_lens, max_seq_len, cache_dtype, scale, work_groups, workspace,
                                                stream)
            self._fn = _lib.pkv_attention_decode_quant
        self._keep = (k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, ws, prefix)
        self._shape, self._dtype = tuple(q.shape), q.dtype
        self._ti = 6


class PreparedAppendQuant(PreparedDecode):
    """A pkv_append_quant call checked once; ``launch(k_new, v_new)`` swaps the new rows."""

    def __init__(self, k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales, cache_dtype,
                 stream=None):  # noqa: D107
        self._args = _append_quant_args(k_new, v_new, slot_mapping, k_cache, v_cache, k_scales, v_scales,
                                        cache_dtype, stream)
        self._keep = (slot_mapping, k_cache, v_cache, k_scales, v_scales)
        self._shape, self._dtype = tuple(k_new.shape), k_new.dtype
        self._fn = _lib.pkv_append_quant

    def launch(self, k_new=None, v_new=None) -> None:
        if k_new is not None:
            self._swap(0, k_new, "k_new")
        if v_new is not None:
            self._swap(1, v_new, "v_new")
        _check(self._fn(*self._args))



# ---------------------------------------------------------------------------
# cumulative attention scores
# ---------------------------------------------------------------------------

def pkv_decode_scores_workspace_bytes(batch, num_heads, max_seq_len) -> int:
    return int(_lib.pkv_decode_scores_workspace_bytes(batch, num_heads, max_seq_len))


def scores_workspace(batch, num_heads, max_seq_len, device="cuda", stream=None):
    """Allocate the workspace a score-updating decode call needs (a uint8 tensor) for use on ``stream``."""
    need = pkv_decode_scores_workspace_bytes(batch, num_heads, max_seq_len)
    return _bytes_on(max(need, 1), device, stream)


def _score_args(scores, q, max_seq_len, decay, scores_ws, stream):
    torch = _torch()
    batch = q.shape[0]
    if scores.dim() != 2 or scores.shape[0] != batch or scores.shape[1] < max_seq_len:
        raise InvalidArgument(PKV_ERR_INVALID, "scores must be float32 [batch][>= max_seq_len]")
    if scores_ws is None:
        scores_ws = scores_workspace(batch, q.shape[1], int(max_seq_len), q.device, stream)
    return [_dev(scores, "scores", torch.float32), scores.shape[1], float(decay), _dev(scores_ws, "scores_ws"),
            scores_ws.numel() * scores_ws.element_size()], scores_ws


def pkv_attention_decode_scores(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scores, decay,
                                scale=None, work_groups=0, workspace=None, scores_ws=None, stream=None) -> None:
    """Decode attention that also updates ``scores[b][t] = decay * scores[b][t] + mean_h p_{b,h}(t)``."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, work_groups,
                           workspace, stream)
    extra, _ = _score_args(scores, q, max_seq_len, decay, scores_ws, stream)
    _check(_lib.pkv_attention_decode_scores(*(args[:-1] + extra + args[-1:])))


def pkv_attention_decode_quant_scores(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                      max_seq_len, cache_dtype, scores, decay, scale=None, work_groups=0,
                                      workspace=None, scores_ws=None, stream=None) -> None:
    """pkv_attention_decode_scores for an 8-bit cache."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                                 cache_dtype, scale, work_groups, workspace, stream)
    extra, _ = _score_args(scores, q, max_seq_len, decay, scores_ws, stream)
    _check(_lib.pkv_attention_decode_quant_scores(*(args[:-1] + extra + args[-1:])))


# ---------------------------------------------------------------------------
# scatter + decode in one launch
# ---------------------------------------------------------------------------

def _check_new_rows(k_new, v_new, q):
    if tuple(k_new.shape) != tuple(q.shape) or v_new.shape != k_new.shape or k_new.dtype != q.dtype or \
            v_new.dtype != q.dtype:
        raise InvalidArgument(PKV_ERR_INVALID, "append_attention_decode: k_new/v_new must match q ([B][H][D])")
    return [_dev(k_new, "k_new"), _dev(v_new, "v_new")]


def pkv_append_attention_decode(out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, max_seq_len,
                                scale=None, work_groups=0, workspace=None, stream=None) -> None:
    """Store each sequence's new K/V row at its position ``seq_lens[b] - 1`` (through the
    table) and run decode attention over all positions, in one launch."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale, work_groups,
                           workspace, stream)
    _check(_lib.pkv_append_attention_decode(*(args[:2] + _check_new_rows(k_new, v_new, q) + args[2:])))


def pkv_append_attention_decode_quant(out, q, k_new, v_new, k_cache, v_cache, k_scales, v_scales, block_tables,
                                      seq_lens, max_seq_len, cache_dtype, scale=None, work_groups=0, workspace=None,
                                      stream=None) -> None:
    """pkv_append_attention_decode for an 8-bit cache (the new rows are quantised on the way in)."""
    if q.shape[0] == 0:
        return
    args, _ = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, max_seq_len,
                                 cache_dtype, scale, work_groups, workspace, stream)
    _check(_lib.pkv_append_attention_decode_quant(*(args[:2] + _check_new_rows(k_new, v_new, q) + args[2:])))


def pkv_append_attention_decode_grouped(out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens,
                                        max_seq_len, seq_prefix_blocks, tiles, scale=None, work_groups=0,
                                        workspace=None, stream=None) -> None:
    """pkv_append_attention_decode with shared prefixes read once per tile (f16 or bf16 caches)."""
    if q.shape[0] == 0:
        return
    args, _ = _grouped_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, seq_prefix_blocks, tiles,
                            scale, work_groups, workspace, stream)
    _check(_lib.pkv_append_attention_decode_grouped(*(args[:2] + _check_new_rows(k_new, v_new, q) + args[2:])))


def pkv_append_attention_decode_grouped_quant(out, q, k_new, v_new, k_cache, v_cache, k_scales, v_scales,
                                              block_tables, seq_lens, max_seq_len, seq_prefix_blocks, tiles,
                                              cache_dtype, scale=None, work_groups=0, workspace=None,
                                              stream=None) -> None:
    """pkv_append_attention_decode_grouped for an 8-bit cache (the new rows are quantised on the way in)."""
    if q.shape[0] == 0:
        return
    args, _ = _grouped_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                  max_seq_len, seq_prefix_blocks, tiles, cache_dtype, scale, work_groups, workspace,
                                  stream)
    _check(_lib.pkv_append_attention_decode_grouped_quant(*(args[:2] + _check_new_rows(k_new, v_new, q) +
                                                            args[2:])))


class PreparedAppendDecode(PreparedDecode):
    """A pkv_append_attention_decode[_quant] call checked once.

    ``launch(q, k_new, v_new, out)`` swaps the per-step row pointers (same
    shapes and dtype as at preparation); ``set_metadata`` repoints the tables
    and lengths.  Pass ``k_scales``, ``v_scales`` and ``cache_dtype`` for an
    8-bit cache, and ``prefix = (seq_prefix_blocks, tiles)`` for the grouped
    call (pkv_append_attention_decode_grouped[_quant]).
    """

    def __init__(self, out, q, k_new, v_new, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale=None,
                 work_groups=0, workspace=None, stream=None, k_scales=None, v_scales=None,
                 cache_dtype=None, prefix=None):  # noqa: D107
        if cache_dtype is None:
            if prefix is None:
                args, ws = _decode_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, scale,
                                        work_groups, workspace, stream)
                self._fn = _lib.pkv_append_attention_decode
            else:
                args, ws = _grouped_args(out, q, k_cache, v_cache, block_tables, seq_lens, max_seq_len, prefix[0],
                                         prefix[1], scale, work_groups, workspace, stream)
                self._fn = _lib.pkv_append_attention_decode_grouped
            self._ti = 6
        else:
            if prefix is None:
                args, ws = _decode_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                              max_seq_len, cache_dtype, scale, work_groups, workspace, stream)
                self._fn = _lib.pkv_append_attention_decode_quant
            else:
                args, ws = _grouped_quant_args(out, q, k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens,
                                               max_seq_len, prefix[0], prefix[1], cache_dtype, scale, work_groups,
                                               workspace, stream)
                self._fn = _lib.pkv_append_attention_decode_grouped_quant
            self._ti = 8
        self._args = args[:2] + _check_new_rows(k_new, v_new, q) + args[2:]
        self._keep = (k_cache, v_cache, k_scales, v_scales, block_tables, seq_lens, ws, prefix)
        self._shape, self._dtype = tuple(q.shape), q.dtype

    def launch(self, q=None, k_new=None, v_new=None, out=None) -> None:
        if q is not None:
            self._swap(1, q, "q")
        if k_new is not None:
            self._swap(2, k_new, "k_new")
        if v_new is not None:
            self._swap(3, v_new, "v_new")
        if out is not None:
            self._swap(0, out, "out")
        _check(self._fn(*self._args))


__all__ = [
    "BlockAllocator", "PkvError", "OutOfBlocks", "InvalidArgument", "pkv_append", "pkv_copy_blocks",
    "pkv_attention_decode", "pkv_decode_workspace_bytes", "pkv_decode_work_groups",
    "pkv_attention_decode_scratch", "DECODE_SCRATCH_BYTES",
    "decode_workspace", "PreparedDecode", "PreparedAppend", "version", "LIB_PATH",
    "pkv_append_quant", "pkv_attention_decode_quant", "PreparedDecodeQuant", "PreparedAppendQuant",
    "CACHE_FORMATS", "prefix_block_keys", "pkv_swap_blocks", "pkv_attention_decode_scores",
    "pkv_attention_decode_quant_scores", "pkv_decode_scores_workspace_bytes", "scores_workspace",
    "prefix_tiles", "pkv_attention_decode_grouped", "pkv_decode_grouped_workspace_bytes", "PREFIX_TILE_SEQS",
    "pkv_attention_decode_grouped_quant", "pkv_append_attention_decode_grouped",
    "pkv_append_attention_decode_grouped_quant",
    "PREFIX_TILE_INTS", "pkv_append_attention_decode", "pkv_append_attention_decode_quant", "PreparedAppendDecode",
]
