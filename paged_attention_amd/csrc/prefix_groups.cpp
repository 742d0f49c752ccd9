// Groups of sequences whose block-table rows begin with the same physical
// blocks: the shared prefix that fork and prefix caching create
// (hnwysp.cn/news/103996 §3.3; icman.com.cn/news/78786 §3.1).  Grouped
// decode attention (pkv_attention_decode_grouped) reads such a prefix once
// for all sequences of a tile instead of once per sequence.  Host code only.
#include <algorithm>
#include <cstdint>
#include <cstring>
#include <vector>

#include "status.h"

extern "C" {

PKV_API int pkv_prefix_tiles(const int32_t* tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                             int32_t batch, int32_t block_size, int32_t min_sharers, int32_t* seq_prefix_blocks,
                             int32_t* tiles, int32_t max_tiles, int32_t* num_tiles) {
  if (batch < 0 || max_blocks_per_seq <= 0 || block_size <= 0 || max_tiles < 0 || !num_tiles ||
      (batch > 0 && (!tables || !seq_lens || !seq_prefix_blocks)) || (max_tiles > 0 && !tiles))
    return pkv::fail(PKV_ERR_INVALID, "prefix_tiles: bad arguments");
  const int32_t need_members = std::max<int32_t>(2, min_sharers);
  // Candidates: sequences with at least one full block before their last
  // position, keyed by their first block id; equal keys in ascending order.
  std::vector<int32_t> order;
  order.reserve(batch);
  std::vector<int32_t> full(batch, 0);  // whole blocks strictly before position L - 1
  for (int32_t b = 0; b < batch; ++b) {
    const int64_t L = seq_lens[b];
    if (L < 2) continue;
    full[b] = static_cast<int32_t>(
        std::min<int64_t>(std::min<int64_t>((L - 1) / block_size, max_blocks_per_seq), PKV_PREFIX_MAX_BLOCKS));
    if (full[b] >= 1) order.push_back(b);
  }
  std::stable_sort(order.begin(), order.end(), [&](int32_t x, int32_t y) {
    return tables[static_cast<int64_t>(x) * max_blocks_per_seq] < tables[static_cast<int64_t>(y) * max_blocks_per_seq];
  });
  std::vector<int32_t> prefix(batch, 0);
  std::vector<int32_t> out_tiles;
  for (size_t i = 0; i < order.size();) {
    const int32_t* lead = tables + static_cast<int64_t>(order[i]) * max_blocks_per_seq;
    size_t j = i + 1;
    while (j < order.size() && tables[static_cast<int64_t>(order[j]) * max_blocks_per_seq] == lead[0]) ++j;
    const size_t n = j - i;
    if (n >= static_cast<size_t>(need_members)) {
      // the leading run all members share, limited to each member's whole blocks
      int32_t p = full[order[i]];
      for (size_t k = i + 1; k < j; ++k) {
        const int32_t* row = tables + static_cast<int64_t>(order[k]) * max_blocks_per_seq;
        int32_t lcp = 0;
        const int32_t lim = std::min(p, full[order[k]]);
        while (lcp < lim && row[lcp] == lead[lcp]) ++lcp;
        p = lcp;
      }
      if (p >= 1) {
        for (size_t k = i; k < j; k += PKV_PREFIX_TILE_SEQS) {
          const size_t m = std::min<size_t>(PKV_PREFIX_TILE_SEQS, j - k);
          const size_t at = out_tiles.size();
          out_tiles.resize(at + PKV_PREFIX_TILE_INTS, -1);
          out_tiles[at] = p;
          out_tiles[at + 1] = static_cast<int32_t>(m);
          for (size_t u = 0; u < m; ++u) {
            out_tiles[at + 2 + u] = order[k + u];
            prefix[order[k + u]] = p;
          }
        }
      }
    }
    i = j;
  }
  const int32_t n_tiles = static_cast<int32_t>(out_tiles.size() / PKV_PREFIX_TILE_INTS);
  if (n_tiles > max_tiles)
    return pkv::fail(PKV_ERR_INVALID, "prefix_tiles: %d tiles needed, room for %d", n_tiles, max_tiles);
  if (batch > 0) std::memcpy(seq_prefix_blocks, prefix.data(), sizeof(int32_t) * batch);
  if (n_tiles > 0) std::memcpy(tiles, out_tiles.data(), sizeof(int32_t) * out_tiles.size());
  *num_tiles = n_tiles;
  return PKV_OK;
}

}  // extern "C"
