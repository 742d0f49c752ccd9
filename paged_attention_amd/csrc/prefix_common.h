// Shared-prefix attention for grouped decode, generic over the cache format:
// the prefix kernel (matrix cores), its load policies' interface, and the
// host side of a grouped call (workspace, parts, launches).
//
// A group is a set of sequences whose block-table rows begin with the same
// physical blocks: forks and prefix-cache hits share their prompt that way
// (hnwysp.cn/news/103996 §3.3; icman.com.cn/news/78786 §3.1).  Plain decode
// reads such a prefix once per sequence; here it is read once per tile of up
// to 16 sequences and head.
//
// One work-group per (prefix tile, head, part): up to 16 sequences whose
// first P blocks are the same physical blocks.  The parts of a (tile, head)
// and their kPrefixWaves wavefronts take the prefix in steps of 16
// positions.  A step runs on the matrix cores, v_mfma_f32_16x16x16 (f16 or
// bf16 inputs, float32 accumulation), whose lane l holds A[l % 16][4 (l / 16)
// + j] and B[4 (l / 16) + j][l % 16] (j < 4) and receives D[4 (l / 16) +
// r][l % 16] (r < 4):
//   S^T (16 positions x 16 sequences) = K (16 x D) Q^T (D x 16), D / 16
//   products; the products' k-slots 4 (l / 16) + j stand for elements
//   (l / 16) D/4 + 4 s + j of product s, so that a lane's K and q operands
//   for all products are one contiguous run of D/4 elements;
//   online softmax per sequence, i.e. per column, whose four lane groups
//   hold four positions each (two cross-group shuffles per reduction);
//   O^T (D x 16) += V^T (D x 16 positions) P^T (16 x 16): the softmax weights
//   are already in the B layout, split as P = P_hi + P_lo into two 16-bit
//   parts so that they keep float32 precision.
// K reaches the A layout straight from the pool; V goes through LDS
// transposed, so that a lane reads four consecutive positions of one
// element.  The wavefronts' states are merged in LDS and stored per
// (sequence, head) as acc[D], max, sum in the decode kernel's units (log2 of
// the scaled logits, unnormalised sums); the merge kernel of the same call
// combines them with the pieces of each sequence's own positions.
//
// A load policy PF supplies:
//   MT                       the matrix-core input type (the query's dtype,
//                            PKV_F16 or PKV_BF16);
//   KB                       cache bytes per element;
//   kScaled                  the cache stores one float32 scale per (token,
//                            head) row that multiplies its elements;
//   widen<N>(raw, w)         N cache elements (raw 32-bit words) as N / 2
//                            words of two MT values, exactly;
//   k_scales(a), v_scales(a) the scale pools (kScaled).
// With scales, a position's K scale multiplies its scores and its V scale
// its softmax weight in the second product (the sum of weights stays
// unscaled), so the codes enter the matrix cores unchanged.
#pragma once

#include <algorithm>
#include <type_traits>

#include "decode_common.h"

namespace {

constexpr int kPrefixWaves = 4;
constexpr int kPrefixStep = 16;     // positions per step (the MFMA's M and K)
constexpr int kPrefixIdsLds = PKV_PREFIX_MAX_BLOCKS;  // a tile's block ids, all staged in LDS
// The prefix grid's x size is tiles × parts work-groups of 256 lanes and the
// dispatch counts lanes in 32 bits; parts is 1 from 512 tiles on, so this cap
// keeps every launch far inside it.
constexpr int32_t kPrefixMaxTiles = 1 << 22;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

template <int DT>
struct PrefixMma;

template <>
struct PrefixMma<PKV_F16> {
  __device__ static f32x4 mma(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a), __builtin_bit_cast(f16x4, b), c, 0, 0,
                                                 0);
  }
  __device__ static uint32_t bits(float x) { return f16_bits(x); }
  __device__ static float value(uint32_t b) {
    return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(b)));
  }
};

template <>
struct PrefixMma<PKV_BF16> {
  __device__ static f32x4 mma(uint2 a, uint2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), __builtin_bit_cast(i16x4, b), c,
                                                     0, 0, 0);
  }
  __device__ static uint32_t bits(float x) { return bf16_rne(x); }
  __device__ static float value(uint32_t b) { return __uint_as_float(b << 16); }
};

// Load policy of 16-bit caches (the cache and the query share the dtype).
template <int DT>
struct PrefixDense {
  static_assert(DT == PKV_F16 || DT == PKV_BF16, "matrix-core input types");
  static constexpr int MT = DT;
  static constexpr int KB = 2;
  static constexpr bool kScaled = false;
  template <int N>
  __device__ static void widen(const uint32_t* raw, uint32_t* w) {
#pragma unroll
    for (int i = 0; i < N / 2; ++i) w[i] = raw[i];
  }
  __device__ static const float* k_scales(const DecodeArgs&) { return nullptr; }
  __device__ static const float* v_scales(const DecodeArgs&) { return nullptr; }
};

// Sequence of column j of a tile, or -1: an index inside the batch whose
// length is valid and longer than the prefix (the decode kernel attends the
// others from position 0 itself).
template <int BS>
__device__ __forceinline__ int tile_member(const int32_t* tp, int j, int n, int prefix_tokens, const DecodeArgs& a) {
  if (j >= n) return -1;
  const int b = tp[2 + j];
  if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(a.batch)) return -1;
  const int L = a.lens[b];
  return length_ok<BS>(L, a) && prefix_tokens < L ? b : -1;
}

// One unit of prefix work: tile x / prefix_parts, its part x % prefix_parts
// and head h, taken by the kPrefixWaves wavefronts of sub-group `sub` of the
// work-group (local thread index tid < kPrefixWaves * 64).  A work-group of
// NSUB sub-groups runs NSUB units side by side; all its threads reach the
// same barriers, so a sub-group with no unit (live = false) or a malformed
// tile takes no step and writes nothing, but does not leave early.
template <class PF, int D, int BS, int NSUB>
__device__ __forceinline__ void prefix_unit(const DecodeArgs& a, const int32_t* tiles, const int x, const int h,
                                            const int sub, const int tid, const bool live) {
  using M = PrefixMma<PF::MT>;
  constexpr int KS = D / 16;   // products per S^T step; 16-element tiles of O^T
  constexpr int RUN = D / 4;   // elements of a lane's K (and V) run
  constexpr int RW = RUN * PF::KB / 4;  // 32-bit words of a run in the cache
  constexpr int EPT = D / (kPrefixWaves * 4);  // elements per thread in the final merge (16 threads a column)
  constexpr int NS = PKV_PREFIX_TILE_SEQS;
  constexpr int kUnitThreads = kPrefixWaves * 64;
  static_assert(NS == 16, "one MFMA column per sequence");
  static_assert(RW % 4 == 0, "whole 16-byte loads");
  // LDS per sub-group: the V^T of each wavefront's step, and after the steps
  // (in the same bytes) the wavefronts' weighted values for the merge; 37 KB
  // at D = 128, so that four one-unit work-groups share a compute unit.
  __shared__ __align__(16) float s_buf_all[NSUB][kPrefixWaves * D * NS];
  __shared__ float s_m_all[NSUB][kPrefixWaves][NS];
  __shared__ float s_l_all[NSUB][kPrefixWaves][NS];
  __shared__ int32_t s_bad[NSUB];
  auto s_v = reinterpret_cast<uint16_t(*)[D][kPrefixStep]>(s_buf_all[sub]);
  auto s_acc = reinterpret_cast<float(*)[D][NS]>(s_buf_all[sub]);
  auto s_m = s_m_all[sub];
  auto s_l = s_l_all[sub];

  const int part = x % a.prefix_parts;  // which share of the tile's steps
  const int32_t* tp = tiles + static_cast<int64_t>(x / a.prefix_parts) * PKV_PREFIX_TILE_INTS;
  const int P = tp[0], n = tp[1], lead = tp[2];
  // a malformed tile (uniform over the sub-group) is taken as no unit
  const bool ok = live && P > 0 && P <= a.max_blocks && n >= 1 && n <= NS &&
                  static_cast<uint32_t>(lead) < static_cast<uint32_t>(a.batch);
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: the step loop does not diverge
  const int lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int prefix_tokens = ok ? P * BS : 0;
  const uint8_t* kpool = static_cast<const uint8_t*>(a.k);
  const uint8_t* vpool = static_cast<const uint8_t*>(a.v);
  const int64_t row_bytes = static_cast<int64_t>(a.num_heads) * D * PF::KB;  // one token's cache row
  const int32_t* trow = a.tables + static_cast<int64_t>(ok ? lead : 0) * a.max_blocks;

  // Prologue: after the tile header, one round of independent loads.  The
  // tables and lengths may be pinned host memory, where every read is a PCIe
  // round trip, so nothing waits on one of them before the barrier:
  //   - the tile's block ids into LDS (a read of global memory inside the
  //     step loop would also make the compiler wait for the prefetched rows;
  //     a tile longer than kPrefixIdsLds blocks is refused, its members NaN);
  //   - the members' validity (their lengths) into LDS, for this and the merge;
  //   - this lane's Q^T operand (its column's sequence, elements grp D/4 ..
  //     grp D/4 + D/4 - 1), loaded for the header's index clamped into the
  //     batch and zeroed after the barrier when the member is not valid.
  __shared__ int32_t s_ids_all[NSUB][kPrefixIdsLds];
  __shared__ int32_t s_member_all[NSUB][NS];
  int32_t* s_ids = s_ids_all[sub];
  int32_t* s_member = s_member_all[sub];
  const bool too_long = P > kPrefixIdsLds;
  const int nids = ok ? min(P, kPrefixIdsLds) : 0;
  for (int i = tid; i < nids; i += kUnitThreads) s_ids[i] = trow[i];
  if (tid < NS) s_member[tid] = ok ? tile_member<BS>(tp, tid, n, prefix_tokens, a) : -1;
  if (tid == 0) s_bad[sub] = 0;
  uint2 qb[KS];
  {
    const int bh = col < n ? tp[2 + col] : 0;
    const int bc = static_cast<uint32_t>(bh) < static_cast<uint32_t>(a.batch) ? bh : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(bc) * a.num_heads + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = *reinterpret_cast<const uint2*>(qrow + grp * RUN + 4 * s);
  }
  __syncthreads();
  {
    const uint32_t keep = s_member[col] >= 0 ? ~0u : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = make_uint2(qb[s].x & keep, qb[s].y & keep);
  }
  int bad = too_long ? 1 : 0;
  auto block_at = [&](int t) -> int32_t {  // checked block id of prefix position t, or -1 (no branch)
    const int32_t blk = s_ids[min(t, prefix_tokens - 1) / BS];
    const bool in_pool = static_cast<uint32_t>(blk) < static_cast<uint32_t>(a.num_blocks);
    bad |= in_pool ? 0 : 1;
    return t < prefix_tokens && in_pool ? blk : -1;
  };
  struct StepRows {
    uint32_t k[RW];  // K: position t0 + col, elements grp D/4 ..
    uint32_t v[RW];  // V: position t0 + lane / 4, elements (lane % 4) D/4 ..
    float4 ks, vs;   // scales of positions t0 + 4 grp .. + 3 (0 where not attended)
  };
  // Every load is issued (from block 0 where the position is past the prefix
  // or its id is bad) and the rows it must not contribute are masked to zero
  // afterwards: a load under a lane condition would leave the compiler unable
  // to count the loads in flight, and it would wait for all of them.
  auto load_run = [&](uint32_t* dst, const uint8_t* pool, int t, int e0) {
    const int32_t blk = block_at(t);
    const uint32_t keep = blk >= 0 ? ~0u : 0u;
    const uint8_t* p = pool + (static_cast<int64_t>(blk < 0 ? 0 : blk) * BS + t % BS) * row_bytes +
                       (static_cast<int64_t>(h) * D + e0) * PF::KB;
#pragma unroll
    for (int i = 0; i < RW / 4; ++i) {
      const Vec16 w = reinterpret_cast<const Vec16*>(p)[i];
#pragma unroll
      for (int k = 0; k < 4; ++k) dst[4 * i + k] = w.w[k] & keep;
    }
  };
  auto load_scales = [&](const float* pool, int t) -> float4 {  // positions t .. t + 3 (one block)
    const int32_t blk = block_at(t);
    const float4 s = *reinterpret_cast<const float4*>(
        pool + (static_cast<int64_t>(blk < 0 ? 0 : blk) * a.num_heads + h) * BS + t % BS);
    auto kept = [&](float x, int j) { return blk >= 0 && t + j < prefix_tokens ? x : 0.f; };
    return make_float4(kept(s.x, 0), kept(s.y, 1), kept(s.z, 2), kept(s.w, 3));
  };
  auto load_step = [&](StepRows& r, int st) {
    const int t0 = st * kPrefixStep;
    load_run(r.k, kpool, t0 + col, grp * RUN);
    load_run(r.v, vpool, t0 + (lane >> 2), (lane & 3) * RUN);
    if constexpr (PF::kScaled) {
      r.ks = load_scales(PF::k_scales(a), t0 + 4 * grp);
      r.vs = load_scales(PF::v_scales(a), t0 + 4 * grp);
    } else {
      r.ks = r.vs = make_float4(1.f, 1.f, 1.f, 1.f);  // unused
    }
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 acc[KS];
#pragma unroll
  for (int c = 0; c < KS; ++c) acc[c] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto fold_step = [&](const StepRows& r, int st) {
    const int t0 = st * kPrefixStep;
    // V rows into LDS, transposed (element-major)
    {
      uint32_t vw[RUN / 2];
      PF::template widen<RUN>(r.v, vw);
      const int e0 = (lane & 3) * RUN;
#pragma unroll
      for (int k = 0; k < RUN; ++k) s_v[wave][e0 + k][lane >> 2] = static_cast<uint16_t>(vw[k >> 1] >> (16 * (k & 1)));
    }
    // S^T and the online softmax per column
    uint32_t kw[RUN / 2];
    PF::template widen<RUN>(r.k, kw);
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sc = M::mma(make_uint2(kw[2 * s], kw[2 * s + 1]), qb[s], sc);
    const float ks[4] = {r.ks.x, r.ks.y, r.ks.z, r.ks.w};
    const float vs[4] = {r.vs.x, r.vs.y, r.vs.z, r.vs.w};
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float x = PF::kScaled ? sc[q] * ks[q] : sc[q];
      sv[q] = t0 + 4 * grp + q < prefix_tokens ? x * a.scale_log2 : -INFINITY;
      mx = fmaxf(mx, sv[q]);
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float mn = fmaxf(m, mx);
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    lsum *= alpha;
#pragma unroll
    for (int c = 0; c < KS; ++c) acc[c] *= alpha;
    uint32_t hi[4], lo[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float p = __builtin_amdgcn_exp2f(sv[q] - mn);
      lsum += p;
      const float pw = PF::kScaled ? p * vs[q] : p;  // the weight the V codes take
      hi[q] = M::bits(pw);
      lo[q] = M::bits(pw - M::value(hi[q]));
    }
    m = mn;
    const uint2 phi = make_uint2(hi[0] | (hi[1] << 16), hi[2] | (hi[3] << 16));
    const uint2 plo = make_uint2(lo[0] | (lo[1] << 16), lo[2] | (lo[3] << 16));
    // O^T += V^T P^T, V^T operand from LDS: element 16 c + col, positions 4 grp + (0..3)
#pragma unroll
    for (int c = 0; c < KS; ++c) {
      const uint2 va = *reinterpret_cast<const uint2*>(&s_v[wave][16 * c + col][4 * grp]);
      acc[c] = M::mma(va, phi, acc[c]);
      acc[c] = M::mma(va, plo, acc[c]);
    }
  };

  // The tile's steps are dealt over its prefix_parts work-groups and their
  // wavefronts: wavefront w of part p takes steps p * kPrefixWaves + w +
  // i * kPrefixWaves * prefix_parts.  Two register sets: the wavefront's next
  // step is loaded before its current one is folded.  The loads are
  // unconditional (the last step is read again at the end) so that the
  // compiler's waits stay partial.
  const int nsteps = too_long || !ok ? 0 : (prefix_tokens + kPrefixStep - 1) / kPrefixStep;
  const int stride = kPrefixWaves * a.prefix_parts;
  int st = part * kPrefixWaves + wave;
  if (st < nsteps) {
    StepRows ra, rb;
    load_step(ra, st);
    for (;;) {
      load_step(rb, min(st + stride, nsteps - 1));
      fold_step(ra, st);
      st += stride;
      if (st >= nsteps) break;
      load_step(ra, min(st + stride, nsteps - 1));
      fold_step(rb, st);
      st += stride;
      if (st >= nsteps) break;
    }
  }
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  __syncthreads();  // every wavefront is done with its V^T before the buffer takes the values
  if (grp == 0) {
    s_m[wave][col] = m;
    s_l[wave][col] = lsum;
  }
#pragma unroll
  for (int c = 0; c < KS; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) s_acc[wave][16 * c + 4 * grp + r][col] = acc[c][r];
  if (__any(bad) && lane == 0) s_bad[sub] = 1;  // the sub-group's bad-block flag (same value from any wavefront)
  __syncthreads();
  bad = s_bad[sub];

  // merge the wavefronts' states; thread t: column t % 16, elements EPT * (t / 16) + (0 .. EPT)
  static_assert(EPT % 2 == 0 && EPT * kPrefixWaves * 4 == D, "the merge covers every element");
  const int j = tid & 15;
  const int e0 = EPT * (tid >> 4);
  const int bj = s_member[j];
  if (bj < 0) return;
  float mmax = -INFINITY;
#pragma unroll
  for (int w = 0; w < kPrefixWaves; ++w) mmax = fmaxf(mmax, s_m[w][j]);
  float total = 0.f;
  float out[EPT];
#pragma unroll
  for (int e = 0; e < EPT; ++e) out[e] = 0.f;
#pragma unroll
  for (int w = 0; w < kPrefixWaves; ++w) {
    const float wt = s_m[w][j] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(s_m[w][j] - mmax);
    total = fmaf(s_l[w][j], wt, total);
#pragma unroll
    for (int e = 0; e < EPT; ++e) out[e] = fmaf(s_acc[w][e0 + e][j], wt, out[e]);
  }
  // this part's state: (max, sum) = (-inf, 0) and zero values when it had no step
  float* ps = a.prefix_state + ((static_cast<int64_t>(part) * a.prefix_batch + bj) * a.num_heads + h) * a.prefix_row;
#pragma unroll
  for (int e = 0; e < EPT; e += 2) *reinterpret_cast<float2*>(ps + e0 + e) = make_float2(out[e], out[e + 1]);
  if (e0 == 0) {
    ps[D] = mmax;
    ps[D + 1] = bad ? __builtin_nanf("") : total;
  }
}

// Grid (tiles x parts, heads): one unit per work-group.
template <class PF, int D, int BS>
__global__ void __launch_bounds__(kPrefixWaves * 64) prefix_kernel(DecodeArgs a, const int32_t* tiles) {
  prefix_unit<PF, D, BS, 1>(a, tiles, static_cast<int>(blockIdx.x), static_cast<int>(blockIdx.y), 0,
                            static_cast<int>(threadIdx.x), true);
}

// A grouped call's decode and prefix work in one grid.  Work-groups
// [0, a.grid_decode) take the stream-K ranges of the sequences' own
// positions, as decode_kernel; the ones after them take the prefix units,
// NSUB units each (unit u: tile part u / H, head u % H; NSUB * kPrefixWaves
// wavefronts are the decode work-group's, and the host launches only such
// shapes), into the same partial prefix states as prefix_kernel.  Neither
// half reads what the other writes: the merge kernel, launched after,
// combines them.  Work-groups start in index order, so the ranges are
// resident first, and the fused kernel's register count (the prefix body's)
// lets a compute unit hold one work-group of 8 wavefronts: with fewer ranges
// than compute units, prefix units run on the units the ranges leave free
// instead of sharing a compute unit's issue slots with a range.  (8-bit
// caches get there with both chunk streams of a range in one work-group of
// 8 wavefronts: 224 ranges for the automatic 448 streams.)
// DUAL: the ranges run two chunk streams (decode_body), as the plain launch
// of the same shape does.
template <class KV, class PF, int D, int BS, int MODE, int NSUB, bool DUAL>
__global__ void __launch_bounds__(NSUB * kPrefixWaves * 64)
    grouped_decode_kernel(DecodeArgs a, const int32_t* tiles, int32_t prefix_units) {
  const int g = static_cast<int>(blockIdx.x);
  if (g < a.grid_decode) {
    decode_body<KV, D, BS, MODE, true, DUAL>(a, a.grid_decode, g);
    return;
  }
  constexpr int kUnitThreads = kPrefixWaves * 64;
  const int sub = static_cast<int>(threadIdx.x) / kUnitThreads;
  const int64_t u = static_cast<int64_t>(g - a.grid_decode) * NSUB + sub;
  const bool live = u < prefix_units;
  const int uu = live ? static_cast<int>(u) : 0;
  prefix_unit<PF, D, BS, NSUB>(a, tiles, uu / a.num_heads, uu % a.num_heads, sub,
                               static_cast<int>(threadIdx.x) % kUnitThreads, live);
}

// ---- host side of a grouped call ---------------------------------------------

// Workspace of a grouped call: the decode workspace (with a piece slot per
// sequence more), then the partial prefix states of up to kPrefixPartsMax
// parts.
inline size_t grouped_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype cache_dtype,
                                      int32_t wg) {
  const size_t base = workspace_layout(batch, num_heads, head_dim, cache_dtype, wg, true).total;
  return base + (static_cast<size_t>(kPrefixPartsMax) * batch * num_heads * (head_dim + 4) * sizeof(float) + 255) /
                    256 * 256;
}

template <class PF, int D>
void launch_prefix(const DecodeArgs& a, int32_t bs, const int32_t* tiles, int32_t num_tiles, hipStream_t stream,
                   hipEvent_t start) {
  const dim3 grid(num_tiles * a.prefix_parts, a.num_heads), block(kPrefixWaves * 64);
  switch (bs) {
    case 8: hipExtLaunchKernelGGL((prefix_kernel<PF, D, 8>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
    case 16: hipExtLaunchKernelGGL((prefix_kernel<PF, D, 16>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
    default: hipExtLaunchKernelGGL((prefix_kernel<PF, D, 32>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
  }
}

// A grouped call's decode and prefix work in one launch (grouped_decode_kernel,
// `units` prefix units after the a.grid_decode ranges), then the merge.
template <class KV, class PF, int D, int BS, int MODE, int NSUB, bool DUAL>
void launch_fused_k(const DecodeArgs& a, const int32_t* tiles, int32_t units, hipStream_t stream, hipEvent_t start) {
  hipExtLaunchKernelGGL((grouped_decode_kernel<KV, PF, D, BS, MODE, NSUB, DUAL>),
                        dim3(a.grid_decode + (units + NSUB - 1) / NSUB), dim3(NSUB * kPrefixWaves * 64),
                        decode_lds_bytes(a, true), stream, start, nullptr, 0, a, tiles, units);
}

// The work-group holds the ranges' wavefronts: waves_per_group per stream,
// two streams where the plain launch of the shape runs two (launch_decode_g's
// rule).  Only totals of 4 or 8 wavefronts (one or two prefix units) are
// launched; run_grouped offers no other shape (fusable_shape).
template <class KV, class PF, int D, int BS, int MODE>
int launch_fused_g(const DecodeArgs& a, const int32_t* tiles, int32_t units, hipStream_t stream,
                   const pkv::CallEvents& tm) {
  const bool dual = KV::kDual && 2 * a.waves_per_group <= KV::kMaxWaves;
  const int waves = a.waves_per_group * (dual ? 2 : 1);
  if (waves != kPrefixWaves && waves != 2 * kPrefixWaves)
    return pkv::fail(PKV_ERR_INVALID, "grouped decode: %d wavefronts per work-group in one launch", waves);
  if (dual) {
    if constexpr (KV::kDual) {
      if (waves == 2 * kPrefixWaves) launch_fused_k<KV, PF, D, BS, MODE, 2, true>(a, tiles, units, stream, tm.start);
      else launch_fused_k<KV, PF, D, BS, MODE, 1, true>(a, tiles, units, stream, tm.start);
    }
  } else {
    if (waves == 2 * kPrefixWaves) launch_fused_k<KV, PF, D, BS, MODE, 2, false>(a, tiles, units, stream, tm.start);
    else launch_fused_k<KV, PF, D, BS, MODE, 1, false>(a, tiles, units, stream, tm.start);
  }
  launch_merge<KV, D, MODE, true>(a, stream, tm.stop);
  return PKV_OK;
}

template <class KV, class PF, int MODE>
int launch_fused(const DecodeArgs& a, int32_t bs, int32_t d, const int32_t* tiles, int32_t units, hipStream_t stream,
                 const pkv::CallEvents& tm) {
  if (d == 64) {
    switch (bs) {
      case 8: return launch_fused_g<KV, PF, 64, 8, MODE>(a, tiles, units, stream, tm);
      case 16: return launch_fused_g<KV, PF, 64, 16, MODE>(a, tiles, units, stream, tm);
      default: return launch_fused_g<KV, PF, 64, 32, MODE>(a, tiles, units, stream, tm);
    }
  }
  switch (bs) {
    case 8: return launch_fused_g<KV, PF, 128, 8, MODE>(a, tiles, units, stream, tm);
    case 16: return launch_fused_g<KV, PF, 128, 16, MODE>(a, tiles, units, stream, tm);
    default: return launch_fused_g<KV, PF, 128, 32, MODE>(a, tiles, units, stream, tm);
  }
}

// Batches (times head slices) up to this run fused: the decode half's LDS
// arrays then stay small beside the prefix half's.
constexpr int32_t kFusedMaxVirtual = 1024;
// Prefix units of one fused launch at most (the grid stays far from any limit).
constexpr int64_t kFusedMaxUnits = int64_t{1} << 24;
constexpr int kFusedMaxWaves = 2 * kPrefixWaves;  // work-groups of one or two prefix units

// Whether a grouped call of this shape and batch can run its prefix units in
// the decode launch: work-groups (both chunk streams) of whole prefix units,
// one launch.
inline bool fusable_shape(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype cache_dtype) {
  const Shape sh = decode_shape(num_heads, head_dim, cache_dtype);
  const int waves = sh.wpg * chunk_streams(cache_dtype, sh.wpg);
  return waves % kPrefixWaves == 0 && waves <= kFusedMaxWaves &&
         static_cast<int64_t>(batch) * sh.groups_y <= kFusedMaxVirtual;
}

inline int check_grouped_sizes(const char* what, int32_t batch, int32_t num_heads, int32_t head_dim,
                               int32_t block_size, int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t max_seq_len, int32_t num_tiles) {
  if (batch < 0 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 ||
      !supported_geometry(head_dim, block_size) || num_tiles < 0 || num_tiles > kPrefixMaxTiles || num_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID, "%s: unsupported sizes (batch %d, heads %d, head_dim %d, block %d, blocks %d, "
                                      "max_blocks %d, max_len %d, tiles %d)", what, batch, num_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_seq_len, num_tiles);
  return PKV_OK;
}

// The rest of a grouped call once `a` is prepared (prepare_decode with
// grouped = true): prefix arrays, parts, then either one fused launch
// (launch_fused_fn(args, events, units); nullptr where the format has none)
// or the prefix launch (launch_prefix_fn(pa, start event)) followed by the
// decode and merge launches over slices of the batch (launch_decode_fn(slice
// args, events)).
//
// Fused when the ranges leave compute units free (fewer decode work-groups,
// i.e. streams over chunk_streams, than compute units), the whole batch
// fits one launch and every work-group holds whole prefix units: the prefix
// then costs no time of its own where
// it fits beside the ranges.  Its parts per (tile, head) are then chosen so
// that the units cover the free compute units' slots (at least one part);
// otherwise they give the separate prefix launch two work-groups per compute
// unit.
template <class LaunchPrefix, class LaunchDecode, class LaunchFused>
int run_grouped(DecodeArgs& a, int wg, void* out, const void* q, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, int32_t num_heads,
                int32_t head_dim, pkv_dtype cache_dtype, int64_t q_row_bytes, const int32_t* seq_prefix_blocks,
                int32_t num_tiles, void* workspace, size_t workspace_bytes, const pkv::CallEvents& timing,
                const char* what, LaunchPrefix launch_prefix_fn, LaunchDecode launch_decode_fn,
                LaunchFused launch_fused_fn) {
  const size_t need = grouped_workspace_bytes(batch, num_heads, head_dim, cache_dtype, wg);
  if (workspace_bytes < need)
    return pkv::fail(PKV_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", what, need, workspace_bytes);
  // no tiles: exactly the plain call's kernels
  a.prefix_blocks = num_tiles > 0 ? seq_prefix_blocks : nullptr;
  a.prefix_state = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            workspace_layout(batch, num_heads, head_dim, cache_dtype, wg, true).total);
  a.prefix_row = head_dim + 4;
  a.prefix_batch = batch;
  a.grid_decode = wg;
  const int64_t units = static_cast<int64_t>(num_tiles) * num_heads;  // (tile, head) pairs
  const int32_t cus = device_compute_units();
  auto parts_for = [&](int64_t slots) {
    return units <= 0 ? 1 : static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(
                                kPrefixPartsMax, (slots + units - 1) / units)));
  };
  if constexpr (!std::is_same_v<LaunchFused, std::nullptr_t>) {
    const int streams = chunk_streams(cache_dtype, a.waves_per_group);
    const int ranges = (wg + streams - 1) / streams;                 // decode work-groups
    const int64_t free_slots = static_cast<int64_t>(cus) - ranges;  // compute units no range takes
    if (num_tiles > 0 && free_slots > 0 && fusable_shape(batch, num_heads, head_dim, cache_dtype)) {
      a.grid_decode = ranges;
      a.prefix_parts = parts_for(free_slots * (streams * a.waves_per_group / kPrefixWaves));
      const int64_t prefix_units = units * a.prefix_parts;
      if (prefix_units <= kFusedMaxUnits) {
        a.batch = batch;
        a.out = out;
        a.q = q;
        a.tables = block_tables;
        a.lens = seq_lens;
        const int fst = launch_fused_fn(static_cast<const DecodeArgs&>(a), timing, static_cast<int32_t>(prefix_units));
        if (fst != PKV_OK) return fst;
        return check_launch(what);
      }
    }
  }
  // Parts per (tile, head): enough work-groups for two per compute unit.
  a.prefix_parts = parts_for(2 * static_cast<int64_t>(cus));
  pkv::CallEvents rest = timing;
  if (num_tiles > 0) {  // the shared prefixes first, over the whole batch
    DecodeArgs pa = a;
    pa.batch = batch;
    pa.q = q;
    pa.out = out;
    pa.tables = block_tables;
    pa.lens = seq_lens;
    launch_prefix_fn(pa, timing.start);
    const int lst = check_launch(what);
    if (lst != PKV_OK) return lst;
    rest.start = nullptr;
  }
  return run_sliced(a, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, q_row_bytes, rest,
                    launch_decode_fn);
}

}  // namespace
