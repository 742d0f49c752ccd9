"""Reference oracle for paged-KV decode attention — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct CPU implementation of what the
paged-KV decode path computes.  It exists to check the HIP library, never to
stand in for it: only the test-suite, the smoke check in ``__graft_entry__`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product package
(``paged_attention_amd``) never imports, links or calls anything here, and this
package imports nothing from the product package.

Floating point is carried in float64 on inputs upcast from their stored dtype;
integer and byte work (allocator, slot mapping, scatter, block copy) is exact.

Sources (the pages are cited by address and section; none carries a title line;
``zskr.cn/news/1363082.html`` — windowed KV eviction with recomputation — is
cited for the cumulative score only):

* ``hnwysp.cn/news/103996`` — KV-cache sizing, shared pool, paging, block table
  with refcounts and copy-on-write, ``alloc_block``/``free_block``.
* ``icman.com.cn/news/78786`` — PagedAttention and prefix caching: byte formula,
  block-size table, pool arithmetic, kernel notes.
* ``m.lqnn.cn/news/240480`` — "kvcache sharemem": page pool, page table,
  index redirection ``[page, slot, head, dim]``, ``PagePool.allocate_pages``.

Modules:

* :mod:`oracle.sizes` — closed forms (bytes per token, blocks, fragmentation,
  pool capacity).
* :mod:`oracle.allocator` — FIFO free list + refcounts + sequence helpers
  (fork, reserve with copy-on-write, release).
* :mod:`oracle.pool` — K/V scatter into blocks and whole-block copies.
* :mod:`oracle.attention` — decode attention by its plain definition.
* :mod:`oracle.quant` — 8-bit (int8 / FP8 E4M3) K/V rows: per-row absmax
  quantisation on write, exact dequantisation and attention on read.
* :mod:`oracle.prefix_cache` — block-level prefix cache over the allocator
  (chained SHA-256 keys, match to the first miss, LRU of zero-count blocks).
* :mod:`oracle.scores` — cumulative attention score per cached token
  (decayed running sum of the head-mean softmax weight).

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
closed forms printed on the pages, hand-derived traces, library routines
(``torch.nn.functional.scaled_dot_product_attention`` in float64, torch's
``float8_e4m3fn`` type) and invariants; none is "parity unpinned".
"""

from . import allocator, attention, pool, prefix_cache, quant, scores, sizes  # noqa: F401
