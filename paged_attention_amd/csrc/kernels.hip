// Decode attention for 16/32-bit caches (fp32, fp16, bf16) and its C entry
// points.  The decode kernel and its launch geometry are shared with the
// 8-bit path (decode_common.h); this file supplies the format policy that
// loads and scores 16-bit or 32-bit rows.
#include "decode_common.h"

namespace {

// ---- decode attention (16/32-bit caches) ------------------------------------

// One online-softmax step over a chunk of kChunk tokens whose K/V rows are
// already in registers.  `valid` = tokens of the chunk inside the segment.
template <int DT, int EPL, int LPH, bool SCORES>
__device__ __forceinline__ void softmax_chunk(const Vec16& qv, const Vec16* kr, const Vec16* vr, int valid,
                                              float scale_log2, float& m, float& l, float* acc, float* logit_slot,
                                              int lane_c) {
  float s[kChunk];
  float mc = m;
#pragma unroll
  for (int u = 0; u < kChunk; ++u) {
    s[u] = group_sum<LPH>(dot16<DT>(qv, kr[u], 0.f)) * scale_log2;
    if (u < valid) mc = fmaxf(mc, s[u]);
  }
  if constexpr (SCORES) stage_logits(logit_slot, s, lane_c);
  const float alpha = __builtin_amdgcn_exp2f(m - mc);
  l *= alpha;
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] *= alpha;
#pragma unroll
  for (int u = 0; u < kChunk; ++u) {
    const float pu = u < valid ? __builtin_amdgcn_exp2f(s[u] - mc) : 0.f;
    l += pu;
    float vf[EPL];
    unpack16<DT>(vr[u], vf);
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = fmaf(pu, vf[e], acc[e]);
  }
  m = mc;
}

// Format policy of 16/32-bit caches: q, K, V and out share one dtype; a lane
// holds 16 bytes of a row (8 fp16/bf16 or 4 fp32 elements) and q stays packed
// for the dot-product instructions.
template <int DT>
struct DenseKV {
  static constexpr int QT = DT;
  static constexpr int KB = dtype_bytes(DT);
  static constexpr int EPL = 16 / KB;
  static constexpr int kMaxWaves = ::kMaxWaves;
  static constexpr bool kGrouped = true;  // pkv_attention_decode_grouped uses this policy
  using QReg = Vec16;

  __device__ static Vec16 load_q(const uint8_t* p) { return *reinterpret_cast<const Vec16*>(p); }

  template <int D, int BS, int LPH, bool SCORES>
  __device__ static void chunk(const Vec16& qv, const DecodeArgs& a, const uint8_t* kp, const uint8_t* vp, int32_t blk,
                               int pos0, int /*head*/, int64_t row_bytes, int lastu, int valid, float& m, float& l,
                               float* acc, float* logit_slot, int lane_c) {
    const int64_t base = (static_cast<int64_t>(blk) * BS + pos0) * row_bytes;
    Vec16 kr[kChunk], vr[kChunk];
    // K rows take ordinary loads, V rows non-temporal ones.  Measured on
    // MI355X, fp16, us per call (ordinary / V non-temporal / both):
    //   7B-shaped layer, the caches of six layers read in turn so that no
    //   call finds the previous one's rows cached: 115 / 104.6 / 103.6;
    //   64 sequences sharing a 520-token prefix: 133 / 134 / 152 (with both
    //   streams non-temporal the sharers' repeated reads of the prefix
    //   blocks stop hitting in the caches).
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int64_t ro = base + static_cast<int64_t>(u < lastu ? u : lastu) * row_bytes;
      kr[u] = *reinterpret_cast<const Vec16*>(kp + ro);
      vr[u] = stream_load(vp + ro);
    }
    softmax_chunk<DT, EPL, LPH, SCORES>(qv, kr, vr, valid, a.scale_log2, m, l, acc, logit_slot, lane_c);
  }

  // The new row is already in the cache's dtype: a 16-byte copy per lane.
  template <int D, int BS, int LPH>
  __device__ static void store_new(const DecodeArgs& a, int b, int /*head*/, int e0, int32_t blk, int pos,
                                   int64_t row_bytes) {
    const int64_t src = (static_cast<int64_t>(b) * a.num_heads * D + e0) * KB;
    const int64_t dst = (static_cast<int64_t>(blk) * BS + pos) * row_bytes + e0 * KB;
    *reinterpret_cast<Vec16*>(static_cast<uint8_t*>(a.k) + dst) =
        *reinterpret_cast<const Vec16*>(static_cast<const uint8_t*>(a.k_new) + src);
    *reinterpret_cast<Vec16*>(static_cast<uint8_t*>(a.v) + dst) =
        *reinterpret_cast<const Vec16*>(static_cast<const uint8_t*>(a.v_new) + src);
  }
};

// ---- shared-prefix attention (grouped decode) --------------------------------
//
// One work-group per (prefix tile, head): up to 16 sequences whose first P
// blocks are the same physical blocks.  Its kPrefixWaves wavefronts take the
// prefix in steps of 16 positions (wavefront w: steps w, w + kPrefixWaves,
// ...).  A step runs on the matrix cores, v_mfma_f32_16x16x16 (f16 or bf16
// inputs, float32 accumulation), whose lane l holds A[l % 16][4 (l / 16) + j]
// and B[4 (l / 16) + j][l % 16] (j < 4) and receives D[4 (l / 16) + r][l % 16]
// (r < 4):
//   S^T (16 positions x 16 sequences) = K (16 x D) Q^T (D x 16), D / 16 products;
//   online softmax per sequence, i.e. per column, whose four lane groups
//   hold four positions each (two cross-group shuffles per reduction);
//   O^T (D x 16) += V^T (D x 16 positions) P^T (16 x 16): the softmax weights
//   are already in the B layout, split as P = P_hi + P_lo into two 16-bit
//   parts so that they keep float32 precision.
// K reaches the A layout straight from the pool (four consecutive elements of
// one position per lane); V goes through LDS transposed, so that a lane reads
// four consecutive positions of one element.  The wavefronts' states are
// merged in LDS and stored per (sequence, head) as acc[D], max, sum in the
// decode kernel's units (log2 of the scaled logits, unnormalised sums).
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

template <int DT, int D, int BS>
__global__ void __launch_bounds__(kPrefixWaves * 64) prefix_kernel(DecodeArgs a, const int32_t* tiles) {
  using M = PrefixMma<DT>;
  constexpr int KS = D / 16;   // products per S^T step; 16-element tiles of O^T
  constexpr int VL = D / 32;   // 16-byte V loads per lane per step
  constexpr int EPT = D / (kPrefixWaves * 4);  // elements per thread in the final merge (16 threads a column)
  constexpr int NS = PKV_PREFIX_TILE_SEQS;
  static_assert(NS == 16, "one MFMA column per sequence");
  // LDS: the V^T of each wavefront's step, and after the steps (in the same
  // bytes) the wavefronts' weighted values for the merge; 37 KB at D = 128,
  // so that four work-groups share a compute unit.
  __shared__ __align__(16) float s_buf[kPrefixWaves * D * NS];
  auto s_v = reinterpret_cast<uint16_t(*)[D][kPrefixStep]>(s_buf);
  auto s_acc = reinterpret_cast<float(*)[D][NS]>(s_buf);
  __shared__ float s_m[kPrefixWaves][NS];
  __shared__ float s_l[kPrefixWaves][NS];

  const int part = blockIdx.x % a.prefix_parts;  // which share of the tile's steps
  const int32_t* tp = tiles + static_cast<int64_t>(blockIdx.x / a.prefix_parts) * PKV_PREFIX_TILE_INTS;
  const int h = blockIdx.y;
  const int P = tp[0], n = tp[1], lead = tp[2];
  if (P <= 0 || P > a.max_blocks || n < 1 || n > NS || static_cast<uint32_t>(lead) >= static_cast<uint32_t>(a.batch))
    return;  // a malformed tile (uniform over the work-group)
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform: the step loop does not diverge
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int prefix_tokens = P * BS;
  const uint16_t* kpool = static_cast<const uint16_t*>(a.k);
  const uint16_t* vpool = static_cast<const uint16_t*>(a.v);
  const int32_t* trow = a.tables + static_cast<int64_t>(lead) * a.max_blocks;

  // Prologue: after the tile header, one round of independent loads.  The
  // tables and lengths may be pinned host memory, where every read is a PCIe
  // round trip, so nothing waits on one of them before the barrier:
  //   - the tile's block ids into LDS (a read of global memory inside the
  //     step loop would also make the compiler wait for the prefetched rows;
  //     a tile longer than kPrefixIdsLds blocks is refused, its members NaN);
  //   - the members' validity (their lengths) into LDS, for this and the merge;
  //   - this lane's Q^T operand (its column's sequence, elements 16 s + 4 grp
  //     + (0..3)), loaded for the header's index clamped into the batch and
  //     zeroed after the barrier when the member is not valid.
  __shared__ int32_t s_ids[kPrefixIdsLds];
  __shared__ int32_t s_member[NS];
  const bool too_long = P > kPrefixIdsLds;
  for (int i = threadIdx.x; i < P && i < kPrefixIdsLds; i += blockDim.x) s_ids[i] = trow[i];
  if (threadIdx.x < NS) s_member[threadIdx.x] = tile_member<BS>(tp, threadIdx.x, n, prefix_tokens, a);
  uint2 qb[KS];
  {
    const int bh = col < n ? tp[2 + col] : 0;
    const int bc = static_cast<uint32_t>(bh) < static_cast<uint32_t>(a.batch) ? bh : 0;
    const uint16_t* qrow = static_cast<const uint16_t*>(a.q) + (static_cast<int64_t>(bc) * a.num_heads + h) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) qb[s] = *reinterpret_cast<const uint2*>(qrow + 16 * s + 4 * grp);
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
    uint2 k[KS];  // K operand: position t0 + col, elements 16 s + 4 grp + (0..3)
    uint4 v[VL];  // V: position t0 + lane / 4, elements (lane % 4) * D / 4 + 8 i + (0..7)
  };
  // Every load is issued (from block 0 where the position is past the prefix
  // or its id is bad) and the rows it must not contribute are masked to zero
  // afterwards: a load under a lane condition would leave the compiler unable
  // to count the loads in flight, and it would wait for all of them.
  auto load_step = [&](StepRows& r, int st) {
    const int t0 = st * kPrefixStep;
    {
      const int t = t0 + col;
      const int32_t blk = block_at(t);
      const uint32_t keep = blk >= 0 ? ~0u : 0u;
      const uint16_t* kr = kpool + ((static_cast<int64_t>(blk < 0 ? 0 : blk) * BS + t % BS) * a.num_heads + h) * D;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const uint2 w = *reinterpret_cast<const uint2*>(kr + 16 * s + 4 * grp);
        r.k[s] = make_uint2(w.x & keep, w.y & keep);
      }
    }
    {
      const int t = t0 + (lane >> 2);
      const int32_t blk = block_at(t);
      const uint32_t keep = blk >= 0 ? ~0u : 0u;
      const uint16_t* vr = vpool + ((static_cast<int64_t>(blk < 0 ? 0 : blk) * BS + t % BS) * a.num_heads + h) * D +
                           (lane & 3) * (D / 4);
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const uint4 w = *reinterpret_cast<const uint4*>(vr + 8 * i);
        r.v[i] = make_uint4(w.x & keep, w.y & keep, w.z & keep, w.w & keep);
      }
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
      const int e0 = (lane & 3) * (D / 4);
#pragma unroll
      for (int i = 0; i < VL; ++i) {
        const uint32_t ww[4] = {r.v[i].x, r.v[i].y, r.v[i].z, r.v[i].w};
#pragma unroll
        for (int k = 0; k < 8; ++k)
          s_v[wave][e0 + 8 * i + k][lane >> 2] = static_cast<uint16_t>(ww[k >> 1] >> (16 * (k & 1)));
      }
    }
    // S^T and the online softmax per column
    f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) sc = M::mma(r.k[s], qb[s], sc);
    float sv[4];
    float mx = -INFINITY;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      sv[q] = t0 + 4 * grp + q < prefix_tokens ? sc[q] * a.scale_log2 : -INFINITY;
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
      hi[q] = M::bits(p);
      lo[q] = M::bits(p - M::value(hi[q]));
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
  const int nsteps = too_long ? 0 : (prefix_tokens + kPrefixStep - 1) / kPrefixStep;
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
  bad = __syncthreads_or(bad);

  // merge the wavefronts' states; thread t: column t % 16, elements EPT * (t / 16) + (0 .. EPT)
  static_assert(EPT % 2 == 0 && EPT * kPrefixWaves * 4 == D, "the merge covers every element");
  const int j = threadIdx.x & 15;
  const int e0 = EPT * (threadIdx.x >> 4);
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

bool supported(int32_t head_dim, int32_t block_size, pkv_dtype dtype) {
  return supported_geometry(head_dim, block_size) && is_16_32(dtype);
}

// Both 16/32-bit decode entry points; k_new != nullptr selects the variant
// that first stores each sequence's new row at its position L - 1.
int decode_dense(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                 const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                 const int32_t* seq_lens, int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim,
                 int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype, int32_t num_work_groups,
                 void* workspace, size_t workspace_bytes, hipStream_t stream, const char* what,
                 const ScoreRequest* sc = nullptr) {
  const pkv::CallEvents timing = pkv::take_call_events();  // consumed by this call, whatever its outcome
  if (batch < 0 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 ||
      !supported(head_dim, block_size, dtype))
    return pkv::fail(PKV_ERR_INVALID, "%s: unsupported sizes (batch %d, heads %d, head_dim %d, block %d, blocks %d, "
                                      "max_blocks %d, max_len %d, dtype %d)", what, batch, num_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_seq_len, static_cast<int>(dtype));
  const int st = check_decode_scalars(scale, num_work_groups);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  DecodeArgs a;
  const int wg = prepare_decode(a, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                                workspace, workspace_bytes, out);
  if (wg <= 0) return wg;
  a.k_new = k_new;
  a.v_new = v_new;
  const int sst = attach_scores(a, sc, batch, num_heads, max_seq_len, what);
  if (sst != PKV_OK) return sst;
  const int64_t row = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(dtype);
  return run_sliced(a, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, row, timing,
                    [&](const DecodeArgs& s, const pkv::CallEvents& tm) {
                      switch (dtype) {
                        case PKV_F32: launch_decode_d<DenseKV<PKV_F32>>(s, wg, block_size, head_dim, stream, tm); break;
                        case PKV_F16: launch_decode_d<DenseKV<PKV_F16>>(s, wg, block_size, head_dim, stream, tm); break;
                        default: launch_decode_d<DenseKV<PKV_BF16>>(s, wg, block_size, head_dim, stream, tm); break;
                      }
                    });
}

// Workspace of a grouped call: the decode workspace, then the partial prefix
// states of up to kPrefixPartsMax parts.
inline size_t grouped_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                      int32_t wg) {
  const size_t base = workspace_layout(batch, num_heads, head_dim, dtype, wg, true).total;
  return base + (static_cast<size_t>(kPrefixPartsMax) * batch * num_heads * (head_dim + 4) * sizeof(float) + 255) /
                    256 * 256;
}

template <int DT, int D>
void launch_prefix_d(const DecodeArgs& a, int32_t bs, const int32_t* tiles, int32_t num_tiles, hipStream_t stream,
                     hipEvent_t start) {
  const dim3 grid(num_tiles * a.prefix_parts, a.num_heads), block(kPrefixWaves * 64);
  switch (bs) {
    case 8: hipExtLaunchKernelGGL((prefix_kernel<DT, D, 8>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
    case 16: hipExtLaunchKernelGGL((prefix_kernel<DT, D, 16>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
    default: hipExtLaunchKernelGGL((prefix_kernel<DT, D, 32>), grid, block, 0, stream, start, nullptr, 0, a, tiles); break;
  }
}

int decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                   int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                   int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                   pkv_dtype dtype, const int32_t* seq_prefix_blocks, const int32_t* tiles, int32_t num_tiles,
                   int32_t num_work_groups, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const pkv::CallEvents timing = pkv::take_call_events();  // consumed by this call, whatever its outcome
  const char* what = "attention_decode_grouped";
  if (batch < 0 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 ||
      !supported_geometry(head_dim, block_size) || (dtype != PKV_F16 && dtype != PKV_BF16) || num_tiles < 0 ||
      num_tiles > kPrefixMaxTiles || num_heads > 65535)
    return pkv::fail(PKV_ERR_INVALID, "%s: unsupported sizes (batch %d, heads %d, head_dim %d, block %d, blocks %d, "
                                      "max_blocks %d, max_len %d, dtype %d, tiles %d)", what, batch, num_heads,
                     head_dim, block_size, num_blocks, max_blocks_per_seq, max_seq_len, static_cast<int>(dtype),
                     num_tiles);
  const int st = check_decode_scalars(scale, num_work_groups);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  if (!seq_prefix_blocks || (num_tiles > 0 && !tiles))
    return pkv::fail(PKV_ERR_INVALID, "%s: null prefix arrays", what);
  DecodeArgs a;
  const int wg = prepare_decode(a, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                                workspace, workspace_bytes, out, /*grouped=*/true);
  if (wg <= 0) return wg;
  const size_t need = grouped_workspace_bytes(batch, num_heads, head_dim, dtype, wg);
  if (workspace_bytes < need)
    return pkv::fail(PKV_ERR_INVALID, "%s: workspace of %zu bytes needed, %zu given", what, need, workspace_bytes);
  a.prefix_blocks = seq_prefix_blocks;
  a.prefix_state = reinterpret_cast<float*>(static_cast<char*>(workspace) +
                                            workspace_layout(batch, num_heads, head_dim, dtype, wg, true).total);
  a.prefix_row = head_dim + 4;
  a.prefix_batch = batch;
  // Parts per (tile, head): enough work-groups for two per compute unit.
  {
    const int64_t units = static_cast<int64_t>(num_tiles) * num_heads;
    const int64_t want = 2 * static_cast<int64_t>(auto_work_groups(dtype));
    a.prefix_parts = units <= 0 ? 1 : static_cast<int32_t>(std::max<int64_t>(1, std::min<int64_t>(
                                                                kPrefixPartsMax, (want + units - 1) / units)));
  }
  pkv::CallEvents rest = timing;
  if (num_tiles > 0) {  // the shared prefixes first, over the whole batch
    DecodeArgs pa = a;
    pa.batch = batch;
    pa.q = q;
    pa.out = out;
    pa.tables = block_tables;
    pa.lens = seq_lens;
    if (dtype == PKV_F16) {
      if (head_dim == 64) launch_prefix_d<PKV_F16, 64>(pa, block_size, tiles, num_tiles, stream, timing.start);
      else launch_prefix_d<PKV_F16, 128>(pa, block_size, tiles, num_tiles, stream, timing.start);
    } else {
      if (head_dim == 64) launch_prefix_d<PKV_BF16, 64>(pa, block_size, tiles, num_tiles, stream, timing.start);
      else launch_prefix_d<PKV_BF16, 128>(pa, block_size, tiles, num_tiles, stream, timing.start);
    }
    const int lst = check_launch(what);
    if (lst != PKV_OK) return lst;
    rest.start = nullptr;
  }
  const int64_t row = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(dtype);
  return run_sliced(a, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, row, rest,
                    [&](const DecodeArgs& s, const pkv::CallEvents& tm) {
                      if (dtype == PKV_F16) launch_decode_m<DenseKV<PKV_F16>, kPlain>(s, wg, block_size, head_dim,
                                                                                      stream, tm);
                      else launch_decode_m<DenseKV<PKV_BF16>, kPlain>(s, wg, block_size, head_dim, stream, tm);
                    });
}

}  // namespace

// ---- decode with the library's own device scratch ----------------------------
//
// pkv_attention_decode_scratch runs pkv_attention_decode with its workspace
// (the per-sequence plan and the split pieces' partial states) in this
// file-scope array instead of caller memory, for callers that cannot
// allocate.  Each device holds its own copy from module load until the
// process ends.  In host code `scratch` names a host-side stand-in, never the
// device memory: its device address is looked up once per device, with that
// device current, and only that address is handed to kernels.  Every call on
// a device shares the device's copy, so calls that overlap on one device
// (several streams or threads) race.  Nothing in it has to start at zero: the
// decode kernel writes the plan and the pieces before any of them is read.
constexpr size_t kScratchBytes = PKV_DECODE_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kScratchDevices = 64;

// Device address of `scratch` on the current device (looked up on the first
// call per device), or nullptr after recording the error.
void* scratch_on_current_device() {
  static std::atomic<void*> addr[kScratchDevices];  // zero-initialised; racing look-ups store the same value
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    pkv::fail(PKV_ERR_HIP, "attention_decode_scratch: no usable current HIP device (%d)", dev);
    return nullptr;
  }
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) {
      pkv::fail(PKV_ERR_HIP, "attention_decode_scratch: device address of the scratch array on device %d: %s", dev,
                hipGetErrorString(e));
      return nullptr;
    }
    addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

PKV_API int pkv_attention_decode_scratch(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, pkv_dtype dtype, int32_t num_work_groups, hipStream_t stream) {
  if (batch > 0 && num_heads > 0 && num_work_groups >= 0 && num_work_groups <= (1 << 20) &&
      supported(head_dim, block_size, dtype)) {
    const int32_t wg = num_work_groups > 0 ? num_work_groups : auto_work_groups(dtype);
    if (wg <= 0) {
      pkv::take_call_events();  // a pending timing request belongs to this call
      return wg;
    }
    const size_t need = workspace_layout(batch, num_heads, head_dim, dtype, wg).total;
    if (need > kScratchBytes) {
      pkv::take_call_events();
      return pkv::fail(PKV_ERR_INVALID, "attention_decode_scratch: these sizes need %zu bytes of scratch, the library "
                                        "holds %zu (fewer work-groups or heads, or pkv_attention_decode with a "
                                        "workspace)", need, kScratchBytes);
    }
    void* ws = scratch_on_current_device();
    if (ws == nullptr) {
      pkv::take_call_events();
      return PKV_ERR_HIP;
    }
    return decode_dense(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                        max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, wg, ws,
                        kScratchBytes, stream, "attention_decode_scratch");
  }
  // invalid or empty requests: decode_dense reports them exactly as pkv_attention_decode does
  return decode_dense(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                      max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                      nullptr, 0, stream, "attention_decode_scratch");
}

PKV_API size_t pkv_decode_grouped_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                                  int32_t num_work_groups) {
  if (batch < 0 || num_heads <= 0 || num_work_groups < 0 || !supported_geometry(head_dim, 8) ||
      (dtype != PKV_F16 && dtype != PKV_BF16))
    return 0;
  const int32_t wg = num_work_groups > 0 ? num_work_groups : auto_work_groups(dtype);
  if (wg <= 0) return 0;
  return grouped_workspace_bytes(batch, num_heads, head_dim, dtype, wg);
}

PKV_API int pkv_attention_decode_grouped(void* out, const void* q, const void* k_cache, const void* v_cache,
                                         const int32_t* block_tables, int32_t max_blocks_per_seq,
                                         const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                         int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                         float scale, pkv_dtype dtype, const int32_t* seq_prefix_blocks,
                                         const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                         void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_grouped(out, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len, batch,
                        num_heads, head_dim, block_size, num_blocks, scale, dtype, seq_prefix_blocks, tiles, num_tiles,
                        num_work_groups, workspace, workspace_bytes, stream);
}

PKV_API int32_t pkv_decode_work_groups(pkv_dtype cache_dtype) {
  if (!is_16_32(cache_dtype) && !is_8bit(cache_dtype))
    return pkv::fail(PKV_ERR_INVALID, "decode_work_groups: unknown dtype %d", static_cast<int>(cache_dtype));
  return auto_work_groups(cache_dtype);
}

PKV_API size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                          int32_t num_work_groups) {
  if (batch < 0 || num_heads <= 0 || num_work_groups < 0 || !supported_geometry(head_dim, 8) ||
      !(is_16_32(dtype) || is_8bit(dtype)))
    return 0;
  const int32_t wg = num_work_groups > 0 ? num_work_groups : auto_work_groups(dtype);
  if (wg <= 0) return 0;
  return workspace_layout(batch, num_heads, head_dim, dtype, wg).total;
}

PKV_API int pkv_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
                                 int32_t num_work_groups, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  return decode_dense(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                      max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                      workspace, workspace_bytes, stream, "attention_decode");
}

PKV_API size_t pkv_decode_scores_workspace_bytes(int32_t batch, int32_t num_heads, int32_t max_seq_len) {
  if (batch < 0 || num_heads <= 0 || max_seq_len < 0) return 0;
  return scores_workspace_bytes(batch, num_heads, max_seq_len);
}

PKV_API int pkv_attention_decode_scores(void* out, const void* q, const void* k_cache, const void* v_cache,
                                        const int32_t* block_tables, int32_t max_blocks_per_seq,
                                        const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                        int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                        float scale, pkv_dtype dtype, int32_t num_work_groups, void* workspace,
                                        size_t workspace_bytes, float* scores, int32_t score_stride, float decay,
                                        void* scores_workspace, size_t scores_workspace_bytes,
                                        hipStream_t stream) {
  const ScoreRequest sc{scores, score_stride, decay, scores_workspace, scores_workspace_bytes};
  return decode_dense(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                      max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                      workspace, workspace_bytes, stream, "attention_decode_scores", &sc);
}

PKV_API int pkv_append_attention_decode(void* out, const void* q, const void* k_new, const void* v_new,
                                        void* k_cache, void* v_cache, const int32_t* block_tables,
                                        int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                        int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                        int32_t num_blocks, float scale, pkv_dtype dtype, int32_t num_work_groups,
                                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch > 0 && (!k_new || !v_new)) return pkv::fail(PKV_ERR_INVALID, "append_attention_decode: null new rows");
  return decode_dense(out, q, k_new, v_new, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                      max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                      workspace, workspace_bytes, stream, "append_attention_decode");
}

}  // extern "C"
