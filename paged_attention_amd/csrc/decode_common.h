// Device code shared by the 16/32-bit and the 8-bit K/V paths of libpkv
// (gfx950, CDNA4): element helpers, lane reductions, the stream-K decode
// attention kernel (generic over how a chunk of K/V rows is loaded and
// scored), the merge kernel for sequences split across work-groups, and the
// host-side launch geometry.
//
// Pool layout (K and V alike): [num_blocks][block_size][num_heads][head_dim].
// One token's row for all heads is contiguous, so the rows a wavefront needs
// for a group of adjacent heads at one token form one contiguous 1 KiB run.
//
// Decode attention is a memory-bound matrix-vector product: per (token, head)
// it reads 2 * head_dim * element bytes and does about 4 * head_dim flops,
// far below the FP32 vector ridge point, so it runs on the vector ALUs, not
// MFMA.  Work split:
//   - each wavefront takes HPW adjacent heads, and each head's row is spread
//     over LPH lanes holding 16 bytes each (one global_load_dwordx4 per lane
//     per token fetches K, one fetches V);
//   - q.k is reduced across the LPH lanes with DPP row permutes;
//   - the softmax runs online over chunks of 8 tokens (running max m, sum l,
//     weighted value accumulator) in base 2 with log2(e) folded into the
//     scale;
//   - work-groups take equal ranges of all sequences' chunks (stream-K); a
//     sequence cut by range boundaries leaves one (m, l, acc) piece per range
//     in the workspace and the merge kernel combines them.
// Block-table entries are wavefront-uniform; every id is range-checked before
// it forms an address.
//
// Everything here has internal linkage: each source that includes this file
// gets its own copy of the templates it instantiates.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "status.h"

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

struct alignas(16) Vec16 {
  uint32_t w[4];
};

constexpr int kChunk = 8;        // tokens per online-softmax step
constexpr int kMaxWaves = 16;    // wavefronts per work-group at most (any format)

__host__ __device__ constexpr int dtype_bytes(int dt) {
  return dt == PKV_F32 ? 4 : (dt == PKV_F16 || dt == PKV_BF16) ? 2 : 1;
}

__host__ __device__ constexpr bool is_8bit(int dt) { return dt == PKV_I8 || dt == PKV_FP8_E4M3; }

// ---- element helpers -------------------------------------------------------

template <int DT>
__device__ __forceinline__ float dot16(const Vec16& q, const Vec16& k, float acc) {
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) acc = fmaf(__uint_as_float(q.w[i]), __uint_as_float(k.w[i]), acc);
  } else if constexpr (DT == PKV_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, q.w[i]), __builtin_bit_cast(half2v, k.w[i]), acc, false);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, q.w[i]), __builtin_bit_cast(bf162v, k.w[i]),
                                            acc, false);
  }
  return acc;
}

template <int DT>
__device__ __forceinline__ void unpack16(const Vec16& v, float* out) {
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v.w[i]);
  } else if constexpr (DT == PKV_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      half2v h = __builtin_bit_cast(half2v, v.w[i]);
      out[2 * i] = static_cast<float>(h.x);
      out[2 * i + 1] = static_cast<float>(h.y);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(v.w[i] << 16);
      out[2 * i + 1] = __uint_as_float(v.w[i] & 0xffff0000u);
    }
  }
}

// float -> bfloat16 bits, round to nearest even (quiet NaN kept quiet).
__device__ __forceinline__ uint32_t bf16_rne(float x) {
  uint32_t u = __float_as_uint(x);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f16_bits(float x) {
  _Float16 h = static_cast<_Float16>(x);  // v_cvt_f16_f32: round to nearest even
  return static_cast<uint32_t>(__builtin_bit_cast(uint16_t, h));
}

// Packs N floats (N = 16 / dtype bytes) into 16 bytes of storage.
template <int DT>
__device__ __forceinline__ Vec16 pack16(const float* in) {
  Vec16 r;
  if constexpr (DT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = __float_as_uint(in[i]);
  } else if constexpr (DT == PKV_F16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = f16_bits(in[2 * i]) | (f16_bits(in[2 * i + 1]) << 16);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) r.w[i] = bf16_rne(in[2 * i]) | (bf16_rne(in[2 * i + 1]) << 16);
  }
  return r;
}

// Stores N floats as N elements of DT at p (16-byte aligned; N * bytes a
// multiple of 16).
template <int DT, int N>
__device__ __forceinline__ void store_row(uint8_t* p, const float* in) {
  constexpr int per = 16 / dtype_bytes(DT);
  static_assert(N % per == 0, "whole 16-byte stores only");
#pragma unroll
  for (int k = 0; k < N / per; ++k) reinterpret_cast<Vec16*>(p)[k] = pack16<DT>(in + k * per);
}

// A 16-byte load marked non-temporal (`nt`): for rows a call reads once,
// so that the stream does not displace other lines in the caches.
__device__ __forceinline__ Vec16 stream_load(const uint8_t* p) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(Vec16, __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p)));
}

// DPP lane permutes inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over each aligned group of N lanes (N = 4, 8, 16 or 32); every lane of
// the group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// Maximum over each aligned group of N lanes (N = 4, 8 or 16).
template <int N>
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, dpp<kDppXor1>(x));
  x = fmaxf(x, dpp<kDppXor2>(x));
  if constexpr (N >= 8) x = fmaxf(x, dpp<kDppHalfMirror>(x));
  if constexpr (N >= 16) x = fmaxf(x, dpp<kDppMirror>(x));
  static_assert(N <= 16, "groups within one DPP row");
  return x;
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off, 64));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off, 64);
  return x;
}

// ---- decode attention ------------------------------------------------------
//
// Stream-K schedule.  Every (sequence, head slice) is cut into chunks of
// kChunk logical tokens (the last chunk of a sequence may be short); the
// chunks of all sequences are laid end to end and the G work-groups of the
// launch take equal contiguous ranges of them.  Each work-group therefore
// reads the same number of K/V bytes (to within one chunk) and pays its
// start-up latency once, however ragged the lengths are.  A range that holds
// a whole sequence writes the output directly; a sequence cut by range
// boundaries leaves one partial softmax state (m, l, acc) per piece, and a
// small merge kernel combines the pieces.  Cut points depend only on logical
// positions, so the result does not depend on where blocks sit physically.

constexpr int kMaxVirtual = 5460;   // sequences x head slices per launch (the LDS arrays: 3 x (5460 + 1) int32 <= 64 KiB)
constexpr int kMaxVirtualGrouped = 4095;  // the same for a grouped launch, which also stages the prefix blocks in LDS
constexpr int kTableWindow = 64;    // block ids held in registers at a time (one per lane)
constexpr int kMergeWaves = 4;      // heads per merge work-group
constexpr int32_t kPlanPrefix = 1 << 30;  // plan flag: the sequence has a shared prefix's partial states
constexpr int32_t kPlanCount = kPlanPrefix - 1;
constexpr int kPrefixPartsMax = 16;  // work-groups per (prefix tile, head) at most: partial states per sequence

struct DecodeArgs {
  void* out;
  const void* q;
  void* k;                // pools (written only by the appending variant)
  void* v;
  float* k_scales;        // 8-bit caches: [num_blocks][H][block_size] per-row scales (else unused)
  float* v_scales;
  const void* k_new;      // appending variant: [batch][H][D] new rows in q's dtype (else unused)
  const void* v_new;
  float* logits;          // score variant: [batch][H][logit_stride] scaled logits (log2 units), else null
  float2* final_ml;       // score variant: [batch][H] final (max, sum) of each sequence the decode kernel
                          // attends whole (cut ones are formed from their pieces)
  float* scores;          // score variant: [batch][score_stride] cumulative scores, updated in place
  int32_t logit_stride;   // max_seq_len rounded up to kLogitGroup
  int32_t score_stride;
  float decay;
  const int32_t* prefix_blocks;  // grouped call: [batch] shared-prefix blocks per sequence (else null)
  float* prefix_state;           // grouped call: [prefix_parts][prefix_batch][H][prefix_row] partial
                                 // prefix states acc[D], max, sum
  int32_t prefix_row;            // = D + 4 (rows stay 16-byte aligned)
  int32_t prefix_parts;          // work-groups per prefix tile and head (partial states per sequence)
  int32_t prefix_batch;          // the whole call's batch (stride of the parts)
  int32_t grid_decode;           // work-groups sharing the chunks (a fused grouped grid runs prefix units after them)
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;      // [partial slot][H][D]
  float2* ws_ml;      // [partial slot][H]: running max (log2 units), running sum
  int32_t* ws_plan;   // [virtual sequence][2]: first partial slot, number of pieces (0 = written directly)
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t batch;
  int32_t num_heads;
  int32_t num_blocks;
  int32_t groups_y;         // head slices (work-groups per sequence piece)
  int32_t waves_per_group;  // head groups (wavefronts) per work-group
  int32_t heads_per_wave;
  int32_t block_size;
  float scale_log2;         // softmax scale * log2(e)
};

// Exclusive prefix sums of f(0..n-1) into out[0..n] (out[n] = total), over
// the whole work-group; every thread must call it.  Up to 64 * kScanRun
// terms (batches of up to 1024 sequences per launch and head slice) one
// wavefront scans alone: each lane sums a contiguous run (up to 64 terms:
// one term, evaluated once), the runs are scanned across lanes, and a single
// barrier publishes the result.  Longer inputs are spread over all threads,
// scanned across lanes and then across wavefronts.
constexpr int kScanRun = 16;
template <typename F>
__device__ void block_exclusive_scan(F f, int n, int32_t* out, int32_t* s_waves) {
  if (n <= 64) {  // one term per lane, each evaluated once
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int32_t local = lane < n ? f(lane) : 0;
      int32_t x = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      if (lane < n) out[lane] = x - local;
      if (lane == 63) out[n] = x;
    }
    __syncthreads();
    return;
  }
  if (n <= 64 * kScanRun) {
    if (threadIdx.x < 64) {
      const int lane = threadIdx.x;
      const int run = (n + 63) / 64;
      const int i0 = min(n, lane * run);
      const int i1 = min(n, i0 + run);
      int32_t local = 0;
      for (int i = i0; i < i1; ++i) local += f(i);
      int32_t x = local;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int32_t y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      int32_t pre = x - local;
      for (int i = i0; i < i1; ++i) {
        out[i] = pre;
        pre += f(i);
      }
      if (lane == 63) out[n] = x;
    }
    __syncthreads();
    return;
  }
  const int nt = blockDim.x;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int run = (n + nt - 1) / nt;
  const int i0 = min(n, t * run);
  const int i1 = min(n, i0 + run);
  int32_t local = 0;
  for (int i = i0; i < i1; ++i) local += f(i);
  int32_t x = local;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int32_t y = __shfl_up(x, off, 64);
    if (lane >= off) x += y;
  }
  if (lane == 63) s_waves[t >> 6] = x;
  __syncthreads();
  if (t == 0) {
    int32_t acc = 0;
    for (int w = 0; w < nt / 64; ++w) {
      const int32_t v = s_waves[w];
      s_waves[w] = acc;
      acc += v;
    }
    s_waves[kMaxWaves] = acc;
  }
  __syncthreads();
  int32_t pre = x - local + s_waves[t >> 6];
  for (int i = i0; i < i1; ++i) {
    out[i] = pre;
    pre += f(i);
  }
  if (t == 0) out[n] = s_waves[kMaxWaves];
  __syncthreads();
}

// floor(x / d) for 0 <= x, 0 < d: 32-bit division where both fit (the usual
// case; a 64-bit division is a long instruction sequence on the GPU).
__device__ __forceinline__ int64_t div_nonneg(int64_t x, int64_t d) {
  if (((x | d) >> 32) == 0) return static_cast<uint32_t>(x) / static_cast<uint32_t>(d);
  return x / d;
}

// Index of the work-group whose chunk range [g*total/nwg, (g+1)*total/nwg)
// holds chunk c.
__device__ __forceinline__ int range_owner(int64_t c, int64_t nwg, int64_t total) {
  return static_cast<int>(div_nonneg((c + 1) * nwg - 1, total));
}

template <int BS>
__device__ __forceinline__ bool length_ok(int L, const DecodeArgs& a) {
  return L >= 0 && L <= a.max_seq_len && static_cast<int64_t>(L) <= static_cast<int64_t>(a.max_blocks) * BS;
}

// First logical position the decode kernel attends for a sequence of valid
// length L in a grouped call: the end of a shared prefix of prefix_blocks
// blocks if it is shorter than L (the prefix itself is attended by
// prefix_kernel, whose partial states the merge kernel folds in); else 0.
template <int BS>
__device__ __forceinline__ int suffix_start(int64_t prefix_blocks, int L) {
  return prefix_blocks > 0 && prefix_blocks * BS < L ? static_cast<int>(prefix_blocks * BS) : 0;
}

// Scaled logits (score variant) leave the decode kernel in whole 128-byte
// lines: a head's logits for kLogitGroup consecutive positions (four chunks)
// are collected in LDS and then stored by the head's lanes 16 bytes each.
// Storing each chunk's 32 bytes as it was scored left partly written lines,
// which the read stream evicted from L2 before the next chunk completed them
// (on MI355X a line lives ~5 us in L2 under this stream); the partial writes
// cost 10 us of a 120 us call on the 7B-shaped layer.  Logit rows are padded
// to a multiple of kLogitGroup positions so that the groups are aligned.
constexpr int kLogitGroup = 32;

inline int32_t padded_logit_stride(int32_t max_seq_len) {
  return static_cast<int32_t>((static_cast<int64_t>(max_seq_len) + kLogitGroup - 1) / kLogitGroup * kLogitGroup);
}

// The chunk's 8 logits into the head's LDS slot at the chunk's offset in its
// group; every lane of the head holds all of them after the DPP sum, and the
// head's first lane writes them.
__device__ __forceinline__ void stage_logits(float* slot, const float (&s)[kChunk], int c) {
  if (c == 0) {
    reinterpret_cast<float4*>(slot)[0] = make_float4(s[0], s[1], s[2], s[3]);
    reinterpret_cast<float4*>(slot)[1] = make_float4(s[4], s[5], s[6], s[7]);
  }
}

// Stores a head's staged group starting at position g0 into its logit row,
// only positions in [t_begin, t_end) (the segment this work-group owns; the
// rest of the group belongs to other work-groups or lies past the length).
template <int LPH>
__device__ __forceinline__ void flush_logits(const float* slot, float* row, int g0, int t_begin, int t_end, int c) {
#pragma unroll
  for (int qd = c; qd < kLogitGroup / 4; qd += LPH) {
    const int t = g0 + 4 * qd;
    const float4 v = reinterpret_cast<const float4*>(slot)[qd];
    if (t >= t_begin && t + 4 <= t_end) {
      *reinterpret_cast<float4*>(row + t) = v;
    } else {
      const float w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (t + j >= t_begin && t + j < t_end) row[t + j] = w[j];
    }
  }
}

// Kernel variants: plain decode, decode that first stores each sequence's new
// row (APPEND), decode that also records logits and final softmax states for
// the cumulative scores (SCORES).
enum DecodeMode { kPlain = 0, kAppend = 1, kScores = 2 };

// The decode kernel.  KV (a format policy) supplies:
//   QT, KB, EPL, kMaxWaves       q/out dtype, cache bytes per element, cache
//                                elements per lane (16 / KB), launch bound;
//   QReg load_q(const uint8_t*)  this lane's EPL query elements;
//   chunk<D, BS, LPH>(...)       load kChunk rows of K/V from block `blk`
//                                starting at in-block position pos0 and fold
//                                them into the online softmax state (and,
//                                given a logit row, store the scaled logits);
//   store_new<D, BS, LPH>(...)   (APPEND) store this lane's part of the
//                                sequence's new K/V row at a pool position.
// With APPEND the launch first stores each sequence's new row (k_new[b],
// v_new[b]) at its position L - 1, then attends over all L positions.  The
// work-group whose range holds a sequence's last chunk is the only one that
// reads position L - 1, and it stores the row itself, lane by lane, before
// reading it back with the same lanes: no other work-group is involved.
// decode_body is the work of one of the `grid` work-groups that share the
// chunks (work-group g); decode_kernel runs it over its whole grid.
//
// With DUAL the work-group holds two chunk streams of waves_per_group
// wavefronts each: stream s takes the chunks s, s + 2, s + 4, ... of every
// segment of its range, and at the segment's end stream 1 hands its state to
// stream 0 through LDS, which folds it in and writes the piece or the row.
// So one work-group of 8 wavefronts does what two of 4 did, with one range
// (and at most one piece per segment) instead of two.
template <class KV, int D, int BS, int MODE, bool GROUPED, bool DUAL = false>
__device__ __forceinline__ void decode_body(const DecodeArgs& a, const int grid, const int g) {
  constexpr bool APPEND = MODE == kAppend;
  constexpr bool SCORES = MODE == kScores;
  static_assert(!(DUAL && SCORES), "the score variant stages logits per chunk group: one stream");
  constexpr int NSTREAM = DUAL ? 2 : 1;
  constexpr int EPL = KV::EPL;
  constexpr int LPH = D / EPL;   // lanes holding one head's row
  constexpr int HPW = 64 / LPH;  // heads per wavefront
  constexpr int KB = KV::KB;
  constexpr int QB = dtype_bytes(KV::QT);
  static_assert(BS % kChunk == 0, "a chunk of tokens must sit inside one block");
  static_assert(KV::kMaxWaves <= kMaxWaves, "wave count bound");
  using Elem = uint8_t;          // addresses are formed in bytes

  extern __shared__ int32_t s_dyn[];
  __shared__ int32_t s_waves[kMaxWaves + 1];
  // score variant: one staged logit group per head slot of every wavefront
  __shared__ __align__(16) float s_logits[SCORES ? KV::kMaxWaves * HPW * kLogitGroup : 4];
  // DUAL: stream 1's (acc[EPL], m, l) per lane of each of its wavefronts, element-major
  constexpr int kDualWaves = KV::kMaxWaves / 2;
  __shared__ float s_dual[DUAL ? (EPL + 2) * kDualWaves * 64 : 1];
  const int nv = a.batch * a.groups_y;
  int32_t* s_pref = s_dyn;           // [nv + 1]: first chunk of each virtual sequence
  int32_t* s_part = s_dyn + nv + 1;  // [nv + 1]: first partial slot of each virtual sequence
  int32_t* s_len = s_part + nv + 1;  // [batch]: the lengths, read once (they may be host memory)
  int32_t* s_pblk = s_len + a.batch;  // GROUPED, [batch]: shared-prefix blocks, read with the lengths

  // 1. chunk counts of every (head slice, sequence); bad lengths count zero.
  for (int b = threadIdx.x; b < a.batch; b += blockDim.x) {
    s_len[b] = a.lens[b];
    if constexpr (GROUPED) s_pblk[b] = a.prefix_blocks[b];
  }
  __syncthreads();
  auto start_of = [&](int b, int L) -> int {  // first attended position (L valid)
    if constexpr (GROUPED) return suffix_start<BS>(s_pblk[b], L);
    return 0;
  };
  auto chunks = [&](int v) -> int32_t {
    const int b = v % a.batch;
    const int L = s_len[b];
    return length_ok<BS>(L, a) ? (L - start_of(b, L) + kChunk - 1) / kChunk : 0;
  };
  // 2. pieces of every sequence the ranges cut; slots for their partials.
  // Ranges are dealt over min(grid, chunks) work-groups so none is empty.
  // A sequence with a shared prefix (grouped call) always leaves pieces: the
  // merge kernel folds the prefix's partial states in with them.
  auto prefixed = [&](int v) -> bool {
    const int b = v % a.batch;
    const int L = s_len[b];
    return length_ok<BS>(L, a) && start_of(b, L) > 0;
  };
  auto pieces_of = [&](int v, int64_t c0, int64_t c1, int64_t nwg, int64_t total) -> int32_t {
    if (c1 == c0) return 0;
    const int k = range_owner(c1 - 1, nwg, total) - range_owner(c0, nwg, total) + 1;
    return k > 1 || prefixed(v) ? k : 0;
  };
  block_exclusive_scan(chunks, nv, s_pref, s_waves);
  {
    const int64_t tot = s_pref[nv];
    const int64_t nw = tot < grid ? tot : static_cast<int64_t>(grid);
    block_exclusive_scan([&](int v) { return pieces_of(v, s_pref[v], s_pref[v + 1], nw, tot); }, nv, s_part,
                         s_waves);
  }
  const int64_t total = s_pref[nv];
  const int64_t nwg = total < grid ? total : static_cast<int64_t>(grid);
  if (g == 0) {
    for (int v = threadIdx.x; v < nv; v += blockDim.x) {
      a.ws_plan[2 * v] = s_part[v];
      a.ws_plan[2 * v + 1] = (s_part[v + 1] - s_part[v]) | (prefixed(v) ? kPlanPrefix : 0);
    }
  }

  // DUAL: the stream index is made uniform for the compiler (it bounds the
  // chunk loop; a loop it took for divergent would wait for every load in
  // flight at each turn)
  const int wave_all = DUAL ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6))
                            : static_cast<int>(threadIdx.x >> 6);
  const int stream = DUAL ? wave_all / a.waves_per_group : 0;
  const int wave = wave_all - stream * a.waves_per_group;  // head group in the slice
  const int lane = threadIdx.x & 63;
  const int r = lane / LPH;
  const int c = lane % LPH;
  const int64_t row_bytes = static_cast<int64_t>(a.num_heads) * D * KB;    // one token's cache row
  const int64_t q_row_bytes = static_cast<int64_t>(a.num_heads) * D * QB;  // one sequence's q / out row

  // 3. sequences with no chunks (length 0, or a length the table cannot
  // hold) are written here: zero rows, or NaN rows for an invalid length.
  for (int v = g; v < nv && stream == 0; v += grid) {
    if (s_pref[v + 1] != s_pref[v]) continue;
    const int b = v % a.batch, y = v / a.batch;
    const int h = (y * a.waves_per_group + wave) * HPW + r;
    if ((y * a.waves_per_group + wave) * HPW >= a.num_heads || h >= a.num_heads) continue;
    const float fill = s_len[b] == 0 ? 0.f : __builtin_nanf("");
    float f[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) f[e] = fill;
    store_row<KV::QT, EPL>(static_cast<Elem*>(a.out) + b * q_row_bytes + (h * D + c * EPL) * QB, f);
  }
  if (total == 0) return;

  // 4. this work-group's chunks [first, last)
  if (g >= nwg) return;
  const int64_t first = div_nonneg(g * total, nwg);
  const int64_t last = div_nonneg((g + 1) * total, nwg);
  if (first >= last) return;
  int v;
  {  // virtual sequence holding chunk `first`: the last v < nv with s_pref[v] <= first
    if (nv <= 64) {  // one LDS read per lane and a ballot (s_pref is non-decreasing)
      const bool le = lane < nv && s_pref[lane] <= first;
      v = __popcll(__ballot(le)) - 1;
    } else {
      int lo = 0, hi = nv;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (s_pref[mid] <= first) lo = mid; else hi = mid;
      }
      v = lo;
    }
    while (s_pref[v + 1] == s_pref[v]) ++v;
  }

  for (int64_t cur = first; cur < last;) {
    const int64_t seq0 = s_pref[v], seq1 = s_pref[v + 1];
    const int64_t seg_end = last < seq1 ? last : seq1;
    const int b = v % a.batch, y = v / a.batch;
    const int hg = y * a.waves_per_group + wave;
    const int h = hg * HPW + r;
    const bool active = hg * HPW < a.num_heads;  // uniform per wavefront (and equal in both streams)
    const bool head_ok = h < a.num_heads;
    const int hl = head_ok ? h : a.num_heads - 1;  // clamped head for loads
    const int e0 = hl * D + c * EPL;                // this lane's first element of the row
    const int L = s_len[b];
    const int start = start_of(b, L);
    const int t_begin = start + static_cast<int>(cur - seq0) * kChunk;
    const int t_end = min(L, start + static_cast<int>(seg_end - seq0) * kChunk);
    // a piece of a sequence with a shared prefix never writes the output:
    // the merge kernel adds the prefix's partial states
    const bool whole = cur == seq0 && seg_end == seq1 && start == 0;
    float m = -INFINITY, l = 0.f;
    float acc[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
    // the output row (whole sequence) or the piece's partial state
    auto finish = [&]() {
      if (!head_ok) return;
      if (SCORES && whole && c == 0) a.final_ml[static_cast<int64_t>(b) * a.num_heads + h] = make_float2(m, l);
      if (whole) {
        const float inv = 1.f / l;
        float o[EPL];
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
        store_row<KV::QT, EPL>(static_cast<Elem*>(a.out) + b * q_row_bytes + e0 * QB, o);
      } else {
        const int piece = g - range_owner(seq0, nwg, total);
        const int64_t slot = static_cast<int64_t>(s_part[v] + piece) * a.num_heads + h;
        float* dst = a.ws_acc + slot * D + c * EPL;
#pragma unroll
        for (int e = 0; e < EPL; e += 4)
          *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
        if (c == 0) a.ws_ml[slot] = make_float2(m, l);
      }
    };
    if (active) {
      const Elem* kp = static_cast<const Elem*>(a.k) + e0 * KB;
      const Elem* vp = static_cast<const Elem*>(a.v) + e0 * KB;
      const int32_t* trow = a.tables + static_cast<int64_t>(b) * a.max_blocks;
      const typename KV::QReg qv = KV::load_q(static_cast<const Elem*>(a.q) + b * q_row_bytes + e0 * QB);
      if constexpr (APPEND) {
        // stored by the stream that reads position L - 1 back
        const bool mine = !DUAL || (((L - 1 - t_begin) / kChunk) & 1) == stream;
        if (head_ok && seg_end == seq1 && L >= 1 && mine) {
          const int pos = L - 1;
          const int32_t id = trow[pos / BS];
          if (static_cast<uint32_t>(id) < static_cast<uint32_t>(a.num_blocks))
            KV::template store_new<D, BS, LPH>(a, b, hl, e0, id, pos % BS, row_bytes);
        }
      }

      bool bad_block = false;
      float* lrow = SCORES && head_ok ? a.logits + (static_cast<int64_t>(b) * a.num_heads + h) * a.logit_stride
                                      : nullptr;
      float* lslot = SCORES ? s_logits + (wave * HPW + r) * kLogitGroup : nullptr;
      int win = -kTableWindow;  // first block index held in `tbl`
      int32_t tbl = 0;
      for (int t0 = t_begin + stream * kChunk; t0 < t_end; t0 += NSTREAM * kChunk) {
        const int j = t0 / BS;
        if (j - win >= kTableWindow) {  // next window of block ids, one per lane, each checked once
          win = j;
          const int nb = min(kTableWindow, (t_end - 1) / BS + 1 - win);
          tbl = lane < nb ? trow[win + lane] : 0;
          const bool bad = lane < nb && static_cast<uint32_t>(tbl) >= static_cast<uint32_t>(a.num_blocks);
          bad_block |= __any(bad);
          if (bad) tbl = 0;
        }
        const int32_t blk = __builtin_amdgcn_readlane(tbl, j - win);
        // rows past the segment repeat its last row (masked)
        KV::template chunk<D, BS, LPH, SCORES>(qv, a, kp, vp, blk, t0 % BS, hl, row_bytes, t_end - 1 - t0,
                                               t_end - t0, m, l, acc,
                                               SCORES ? lslot + (t0 & (kLogitGroup - 1)) : nullptr, c);
        if constexpr (SCORES) {
          const int next = t0 + kChunk;
          if (lrow != nullptr && ((next & (kLogitGroup - 1)) == 0 || next >= t_end))
            flush_logits<LPH>(lslot, lrow, t0 & ~(kLogitGroup - 1), t_begin, t_end, c);
        }
      }
      if (bad_block) l = __builtin_nanf("");
      if constexpr (!DUAL) finish();
    }
    if constexpr (DUAL) {
      // stream 1's state to stream 0 (element-major, so that lanes store
      // and load consecutive words), which folds it in:
      //   M = max(m0, m1), l = l0 2^(m0 - M) + l1 2^(m1 - M), acc likewise;
      // a stream with no chunk of the segment holds (-inf, 0, 0) and weighs 0
      // (a NaN sum, from a bad block id, stays NaN).
      float* s_x = s_dual + wave * 64 + lane;
      constexpr int kStride = kDualWaves * 64;
      if (active && stream == 1) {
#pragma unroll
        for (int e = 0; e < EPL; ++e) s_x[e * kStride] = acc[e];
        s_x[EPL * kStride] = m;
        s_x[(EPL + 1) * kStride] = l;
      }
      __syncthreads();
      if (active && stream == 0) {
        const float m1 = s_x[EPL * kStride], l1 = s_x[(EPL + 1) * kStride];
        const float mn = fmaxf(m, m1);
        const float w0 = m == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m - mn);
        const float w1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mn);
        const bool nan = l != l || l1 != l1;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[e] = acc[e] * w0 + s_x[e * kStride] * w1;
        l = nan ? __builtin_nanf("") : l * w0 + l1 * w1;
        m = mn;
        finish();
      }
      __syncthreads();  // the next segment's hand-over reuses the buffer
    }
    cur = seg_end;
    if (cur < last) {
      ++v;
      while (s_pref[v + 1] == s_pref[v]) ++v;
    }
  }
}

template <class KV, int D, int BS, int MODE, bool GROUPED, bool DUAL>
__global__ void __launch_bounds__(KV::kMaxWaves * 64) decode_kernel(DecodeArgs a) {
  decode_body<KV, D, BS, MODE, GROUPED, DUAL>(a, static_cast<int>(gridDim.x), static_cast<int>(blockIdx.x));
}

// Merges the pieces of every cut sequence, after the partial states of its
// shared prefix when it has one (grouped call):
//   M = max_i m_i,  S = sum_i l_i 2^(m_i - M),  out = sum_i acc_i 2^(m_i - M) / S,
// over the prefix's parts and then the pieces, in that order.
// One wavefront per (sequence, head).  Lane i holds piece i's (m, l); the
// lanes also split into groups of D/4 lanes that hold whole piece rows as
// float4, kMergeRows rows per group.  Every load of a batch of pieces is
// issued before any of them is used, so a batch costs one memory round trip;
// the weights reach the row holders by lane shuffles.
constexpr int kMergeRows = 8;

// Work-group (bx, v) of the merge: heads bx*kMergeWaves.. of virtual sequence v.
template <int DT, int D, bool GROUPED>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int bx, int v) {
  constexpr int LPR = D / 4;     // lanes per piece row (float4 each)
  constexpr int RPW = 64 / LPR;  // rows per wavefront instruction
  constexpr int BATCH = RPW * kMergeRows;
  static_assert(BATCH <= 64, "a batch of pieces must fit one (m, l) per lane");
  static_assert(BATCH >= kPrefixPartsMax, "a shared prefix's parts fit one batch");
  const int b = v % a.batch, y = v / a.batch;
  const int slice_lo = y * a.waves_per_group * a.heads_per_wave;
  const int slice_hi = min(a.num_heads, slice_lo + a.waves_per_group * a.heads_per_wave);
  const int h = slice_lo + __builtin_amdgcn_readfirstlane(bx * kMergeWaves + (threadIdx.x >> 6));
  if (h >= slice_hi) return;
  const int lane = threadIdx.x & 63;
  const int grp = lane / LPR;
  const int sub = lane % LPR;

  // A batch of states 0 .. n-1 (n <= BATCH): lane i holds state i's (m, l),
  // the lane groups hold float4s of the weighted values.
  struct Batch {
    float2 mine;
    float4 rows[kMergeRows];
  };
  auto load_batch = [&](int n, auto ml_at, auto row_at) {
    Batch bt;
    bt.mine = lane < n ? ml_at(lane) : make_float2(-INFINITY, 0.f);
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      const int i = grp + k * RPW;
      bt.rows[k] = i < n ? row_at(i) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    return bt;
  };
  // GROUPED: the prefix parts' loads go out with the plan's (their addresses
  // do not depend on it); they are used only if the plan marks a prefix.
  const float* ps = a.prefix_state + (static_cast<int64_t>(b) * a.num_heads + h) * a.prefix_row;
  const int64_t part_stride = static_cast<int64_t>(a.prefix_batch) * a.num_heads * a.prefix_row;
  Batch pre_batch{};
  if constexpr (GROUPED) {
    pre_batch = load_batch(
        a.prefix_parts,
        [&](int i) {
          const float* p = ps + i * part_stride + D;
          return make_float2(p[0], p[1]);
        },
        [&](int i) { return *reinterpret_cast<const float4*>(ps + i * part_stride + sub * 4); });
  }
  const int first = a.ws_plan[2 * v];
  const int word = a.ws_plan[2 * v + 1];
  const int count = word & kPlanCount;
  const bool pre = GROUPED && (word & kPlanPrefix) != 0;
  if (count == 0 && !pre) return;

  float mx = -INFINITY;   // running max over batches (wave-uniform)
  float sum = 0.f;        // running sum, scaled to mx
  float4 o = make_float4(0.f, 0.f, 0.f, 0.f);
  auto fold = [&](int n, const Batch& bt) {
    const float bmx = wave_max(bt.mine.x);
    const float nmx = fmaxf(mx, bmx);
    const float rescale = __builtin_amdgcn_exp2f(mx - nmx);  // 0 on the first batch
    const float w = lane < n ? __builtin_amdgcn_exp2f(bt.mine.x - nmx) : 0.f;
    sum = sum * rescale + wave_sum(bt.mine.y * w);
    o.x *= rescale;
    o.y *= rescale;
    o.z *= rescale;
    o.w *= rescale;
#pragma unroll
    for (int k = 0; k < kMergeRows; ++k) {
      const float wk = __shfl(w, grp + k * RPW, 64);
      o.x = fmaf(bt.rows[k].x, wk, o.x);
      o.y = fmaf(bt.rows[k].y, wk, o.y);
      o.z = fmaf(bt.rows[k].z, wk, o.z);
      o.w = fmaf(bt.rows[k].w, wk, o.w);
    }
    mx = nmx;
  };
  if (pre) fold(a.prefix_parts, pre_batch);  // the shared prefix's parts first
  const float2* ml = a.ws_ml + static_cast<int64_t>(first) * a.num_heads + h;  // stride num_heads
  const float* accp = a.ws_acc + (static_cast<int64_t>(first) * a.num_heads + h) * D + sub * 4;
  const int64_t row_stride = static_cast<int64_t>(a.num_heads) * D;
  for (int i0 = 0; i0 < count; i0 += BATCH) {
    const int n = min(BATCH, count - i0);
    fold(n, load_batch(
                n, [&](int i) { return ml[static_cast<int64_t>(i0 + i) * a.num_heads]; },
                [&](int i) { return *reinterpret_cast<const float4*>(accp + static_cast<int64_t>(i0 + i) * row_stride); }));
  }
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
    o.x += __shfl_xor(o.x, off, 64);
    o.y += __shfl_xor(o.y, off, 64);
    o.z += __shfl_xor(o.z, off, 64);
    o.w += __shfl_xor(o.w, off, 64);
  }
  if (grp != 0) return;
  const float inv = 1.f / sum;
  const int64_t out_idx = (static_cast<int64_t>(b) * a.num_heads + h) * D + sub * 4;
  if constexpr (DT == PKV_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + out_idx) =
        make_float4(o.x * inv, o.y * inv, o.z * inv, o.w * inv);
  } else {
    uint32_t lo, hi;
    if constexpr (DT == PKV_F16) {
      lo = f16_bits(o.x * inv) | (f16_bits(o.y * inv) << 16);
      hi = f16_bits(o.z * inv) | (f16_bits(o.w * inv) << 16);
    } else {
      lo = bf16_rne(o.x * inv) | (bf16_rne(o.y * inv) << 16);
      hi = bf16_rne(o.z * inv) | (bf16_rne(o.w * inv) << 16);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + out_idx) = make_uint2(lo, hi);
  }
}

template <int DT, int D, bool GROUPED>
__global__ void __launch_bounds__(kMergeWaves * 64) decode_merge_kernel(DecodeArgs a) {
  merge_pieces<DT, D, GROUPED>(a, blockIdx.x, blockIdx.y);
}

// Cumulative attention scores: one thread per (sequence, position t < L):
//   scores[b][t] = decay * scores[b][t] + (1/H) sum_h 2^(logit[b][h][t] - M[b][h]) / S[b][h]
// with (M, S) each head's final softmax max and sum.  These work-groups run
// in the merge kernel's launch, so they do not wait for its work-groups:
// for a sequence the decode kernel wrote whole, (M, S) is what it stored;
// for a cut one, (M, S) is formed here from its pieces' (m, l):
//   M = max_i m_i,  S = sum_i l_i 2^(m_i - M).
// Lane k works out head h0 + k's (M, S) and 1/S; the heads' values then
// reach every lane by v_readlane.  A wavefront reads 64 consecutive
// positions of one head per load.  Two memory round trips: each head's plan
// entry, then together the logits of up to 32 (or 64) heads, the stored
// (M, S), a cut sequence's first pieces' (m, l), the old score and, last,
// the length (loads complete in order, and the length may be a host read).
// Loads at one address across the wavefront would become scalar loads,
// whose waits the compiler places before the vector loads, so the length is
// read through a per-lane index.  Threads past the longest
// sequence load the last position's entries (inside every row) and store
// nothing.  Sequences whose length the decode kernel refused (it attended to
// nothing) are left untouched.
constexpr int kScoreHeads = 64;
constexpr int kScorePieces = 16;  // pieces' (m, l) loaded per batch

__device__ __forceinline__ float lane_value(float x, int k) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), k));
}

// Positions bx*256.. of sequence b.
__device__ __forceinline__ void score_positions(const DecodeArgs& a, int bx, int b) {
  const int t = bx * 256 + static_cast<int>(threadIdx.x);
  const int lane = threadIdx.x & 63;
  const int tc = min(t, a.max_seq_len - 1);  // launched only for max_seq_len >= 1
  // mbcnt of an empty mask is 0 in every lane, but not provably uniform
  const int* lp = a.lens + b + static_cast<int>(__builtin_amdgcn_mbcnt_lo(0u, 0u));
  float* sp = a.scores + static_cast<int64_t>(b) * a.score_stride + tc;
  int L = 0;
  float old = 0.f;
  const float* lg = a.logits + static_cast<int64_t>(b) * a.num_heads * a.logit_stride + tc;
  const int slice_heads = a.waves_per_group * a.heads_per_wave;
  float acc = 0.f;
  // A batch of up to NH heads (32, or 64 when there are more than 32).  The
  // first batch also loads the length and the old score, after its own
  // loads: loads complete in order, so the length (host memory when the
  // tables are pinned) must not come first.
  auto heads = [&](int h0, auto first_batch, auto width) {
    constexpr int NH = decltype(width)::value;
    const int hk = min(h0 + lane, a.num_heads - 1);  // this lane's head
    const int v = (hk / slice_heads) * a.batch + b;   // its virtual sequence
    const int first = a.ws_plan[2 * v];
    const int count = a.ws_plan[2 * v + 1] & kPlanCount;
    float2 fm = a.final_ml[static_cast<int64_t>(b) * a.num_heads + hk];
    float x[NH];
#pragma unroll
    for (int k = 0; k < NH; ++k) x[k] = lg[static_cast<int64_t>(min(h0 + k, a.num_heads - 1)) * a.logit_stride];
    if constexpr (decltype(first_batch)::value) {
      L = *lp;
      old = *sp;
    }
    // A cut sequence combines its pieces' (m, l).  The first kScorePieces
    // are read by every lane, at slots clamped into the sequence's range (a
    // lane-masked load would make the compiler wait for every load in
    // flight, the length's host read included); more pieces take a loop.
    const float2* ml = a.ws_ml + static_cast<int64_t>(first) * a.num_heads + hk;
    float2 p[kScorePieces];
#pragma unroll
    for (int k = 0; k < kScorePieces; ++k)
      p[k] = ml[static_cast<int64_t>(max(0, min(k, count - 1))) * a.num_heads];
    float mx = -INFINITY, sum = 0.f;
    auto fold = [&](int i0) {
      float nmx = mx;
#pragma unroll
      for (int k = 0; k < kScorePieces; ++k)
        if (i0 + k < count) nmx = fmaxf(nmx, p[k].x);
      sum *= __builtin_amdgcn_exp2f(mx - nmx);  // 0 on the first batch
#pragma unroll
      for (int k = 0; k < kScorePieces; ++k)
        if (i0 + k < count) sum = fmaf(p[k].y, __builtin_amdgcn_exp2f(p[k].x - nmx), sum);
      mx = nmx;
    };
    fold(0);
    for (int i0 = kScorePieces; i0 < count; i0 += kScorePieces) {
#pragma unroll
      for (int k = 0; k < kScorePieces; ++k)
        p[k] = ml[static_cast<int64_t>(min(i0 + k, count - 1)) * a.num_heads];
      fold(i0);
    }
    if (count > 0) fm = make_float2(mx, sum);
    const float inv = 1.f / fm.y;
#pragma unroll
    for (int k = 0; k < NH; ++k)
      if (h0 + k < a.num_heads) acc += __builtin_amdgcn_exp2f(x[k] - lane_value(fm.x, k)) * lane_value(inv, k);
  };
  // Up to 32 heads in straight-line code; more in a loop (at whose head the
  // compiler waits for every load in flight, the length's included).
  using Narrow = std::integral_constant<int, kScoreHeads / 2>;
  using Wide = std::integral_constant<int, kScoreHeads>;
  if (a.num_heads <= Narrow::value) {
    heads(0, std::true_type{}, Narrow{});
  } else {
    L = *lp;
    old = *sp;
    for (int h0 = 0; h0 < a.num_heads; h0 += kScoreHeads) heads(h0, std::false_type{}, Wide{});
  }
  const bool ok = L >= 0 && L <= a.max_seq_len &&
                  static_cast<int64_t>(L) <= static_cast<int64_t>(a.max_blocks) * a.block_size;
  if (ok && t < L) *sp = a.decay * old + acc / static_cast<float>(a.num_heads);
}

// The score variant's second launch: work-groups (x < merge_x, v) merge the
// pieces of virtual sequence v; work-groups (merge_x + bx, b < batch) score
// positions bx*256.. of sequence b.  Neither waits for the other.
template <int DT, int D>
__global__ void __launch_bounds__(kMergeWaves * 64) merge_score_kernel(DecodeArgs a, int merge_x) {
  static_assert(kMergeWaves * 64 == 256, "merge and score work-groups share the launch's shape");
  const int x = blockIdx.x;
  if (x < merge_x) merge_pieces<DT, D, false>(a, x, blockIdx.y);
  else if (static_cast<int>(blockIdx.y) < a.batch) score_positions(a, x - merge_x, blockIdx.y);
}

// ---- host helpers ----------------------------------------------------------

inline int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

inline bool supported_geometry(int32_t head_dim, int32_t block_size) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 8 || block_size == 16 || block_size == 32);
}

inline bool is_16_32(pkv_dtype dt) { return dt == PKV_F32 || dt == PKV_F16 || dt == PKV_BF16; }

// Wavefronts a work-group may hold for a cache format: the 8-bit kernels keep
// more registers per lane (16 elements per 16-byte load), so they launch at
// most 8 wavefronts per work-group.
inline int max_waves_for(pkv_dtype cache_dtype) { return is_8bit(cache_dtype) ? 8 : kMaxWaves; }

inline int heads_per_wave(int32_t head_dim, pkv_dtype cache_dtype) {
  const int epl = 16 / dtype_bytes(cache_dtype);
  return 64 / (head_dim / epl);
}

// Compute units of the current device (cached per device); PKV_ERR_HIP
// (negative) when no device is current or the query fails.
inline int32_t device_compute_units() {
  static std::atomic<int32_t> cus_cached[64];  // zero-initialised; calls from several threads may fill it
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return pkv::fail(PKV_ERR_HIP, "no current HIP device");
  int cus = dev < 64 ? cus_cached[dev].load(std::memory_order_relaxed) : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return pkv::fail(PKV_ERR_HIP, "cannot query the compute-unit count");
    if (dev < 64) cus_cached[dev].store(cus, std::memory_order_relaxed);
  }
  return cus;
}

// Chunk streams of the automatic choice on the current device (a stream is
// one work-group's set of wavefronts over the heads; see chunk_streams for
// 8-bit caches).  Measured on MI355X with 16-bit caches (µs per call, 160 /
// 192 / 208 / 224 / 240 / 256 work-groups of 8 wavefronts): 7B-shaped layer
// 104.9 / 99.8 / 99.5 / 98.7 / 99.8 / 99.8, 13B long context 229.7 / 216.6 /
// 215.5 / 214.4 / 214.8 / 216.0; 512 read 5 % slower than 256.  Fewer,
// longer streams keep more DRAM pages open per request until too few remain
// to cover the latency: seven eighths of the compute units (28 of the 32 of
// each XCD, as the dispatcher deals work-groups to the XCDs in turn) is the
// best of the sweep.  8-bit caches carry twice the elements per byte and
// run 4 wavefronts per stream for 32 heads, so they take two streams per
// compute unit to keep the same wavefronts resident.
inline int32_t auto_work_groups(pkv_dtype cache_dtype) {
  const int32_t cus = device_compute_units();
  if (cus <= 0) return cus;
  const int32_t per_cu = is_8bit(cache_dtype) ? 2 : 1;
  return std::max<int32_t>(1, per_cu * (cus - cus / 8));
}

// Chunk streams per decode work-group outside the score variant: 8-bit
// caches run two streams of 4 wavefronts in one work-group of 8 when both
// fit (decode_body's DUAL), so the automatic 448 streams take 224 work-groups
// and leave the same compute units free as 16-bit caches do.
inline int chunk_streams(pkv_dtype cache_dtype, int waves_per_group) {
  return is_8bit(cache_dtype) && 2 * waves_per_group <= max_waves_for(cache_dtype) ? 2 : 1;
}

inline int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

// Work-group shape: head groups (one wavefront each) are split into
// groups_y slices of at most max_waves wavefronts.
struct Shape {
  int groups;    // head groups = ceil(H / heads per wavefront)
  int groups_y;  // head slices
  int wpg;       // wavefronts per work-group
  int hpw;       // heads per wavefront
};

inline Shape decode_shape(int32_t num_heads, int32_t head_dim, pkv_dtype cache_dtype) {
  Shape sh;
  sh.hpw = heads_per_wave(head_dim, cache_dtype);
  sh.groups = ceil_div(num_heads, sh.hpw);
  sh.groups_y = ceil_div(sh.groups, max_waves_for(cache_dtype));
  sh.wpg = ceil_div(sh.groups, sh.groups_y);
  return sh;
}

// Workspace: [plan: virtual sequences x 2 int32][acc: P slots x H x D f32][(m, l): P slots x H].
// A cut at each of the G-1 range boundaries adds at most one piece and one
// cut sequence, so the pieces of all cut sequences number at most 2(G-1);
// in a grouped call a sequence with a shared prefix leaves a piece even
// when it is not cut, at most one more per virtual sequence.  P = 2G, plus
// the virtual sequences of a launch for a grouped call.
struct Layout {
  size_t plan, acc, ml, total;
};

inline Layout workspace_layout(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype cache_dtype,
                               int32_t wg, bool grouped = false) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  const Shape sh = decode_shape(num_heads, head_dim, cache_dtype);
  const int64_t per_launch = kMaxVirtual / sh.groups_y;
  const size_t nv = static_cast<size_t>(batch < per_launch ? batch : per_launch) * sh.groups_y;
  const size_t slots = (2 * static_cast<size_t>(wg) + (grouped ? nv : 0)) * num_heads;
  Layout w{};
  w.plan = 0;
  w.acc = up(nv * 2 * sizeof(int32_t));
  w.ml = w.acc + up(slots * head_dim * sizeof(float));
  w.total = w.ml + up(slots * sizeof(float2));
  return w;
}

// Kernels of one launch_decode: the decode kernel, then the merge kernel (for
// a score request, the merge and score kernel).  `tm.start` goes with the
// first and `tm.stop` with the second (kernel timestamps, no extra queue
// packets).
// GROUPED: a grouped call (shared prefixes attended by the prefix kernel).
// Dynamic LDS of a decode work-group: the two prefix-sum arrays and the
// lengths (and, grouped, the shared-prefix blocks).
inline size_t decode_lds_bytes(const DecodeArgs& a, bool grouped) {
  return (2 * (static_cast<size_t>(a.batch) * a.groups_y + 1) + a.batch * (grouped ? 2 : 1)) * sizeof(int32_t);
}

// The merge (or merge-and-score) launch after a decode launch.
template <class KV, int D, int MODE, bool GROUPED>
void launch_merge(const DecodeArgs& a, hipStream_t stream, hipEvent_t stop) {
  const bool scores = MODE == kScores && a.max_seq_len > 0;
  const int slice_heads = a.waves_per_group * a.heads_per_wave;
  const int merge_x = ceil_div(slice_heads, kMergeWaves);
  if (scores)
    hipExtLaunchKernelGGL((merge_score_kernel<KV::QT, D>),
                          dim3(merge_x + ceil_div(a.max_seq_len, 256), a.batch * a.groups_y), dim3(kMergeWaves * 64),
                          0, stream, nullptr, stop, 0, a, merge_x);
  else
    hipExtLaunchKernelGGL((decode_merge_kernel<KV::QT, D, GROUPED>), dim3(merge_x, a.batch * a.groups_y),
                          dim3(kMergeWaves * 64), 0, stream, nullptr, stop, 0, a);
}

// `wg` counts chunk streams; a format with two streams per work-group
// (KV::kDual, outside the score variant, when both fit a work-group) runs
// them in ceil(wg / 2) work-groups of twice the wavefronts.
template <class KV, int D, int BS, int MODE, bool GROUPED>
void launch_decode_g(const DecodeArgs& a, int wg, hipStream_t stream, const pkv::CallEvents& tm) {
  const size_t lds = decode_lds_bytes(a, GROUPED);
  if constexpr (KV::kDual && MODE != kScores) {
    if (2 * a.waves_per_group <= KV::kMaxWaves) {
      hipExtLaunchKernelGGL((decode_kernel<KV, D, BS, MODE, GROUPED, true>), dim3((wg + 1) / 2),
                            dim3(2 * a.waves_per_group * 64), lds, stream, tm.start, nullptr, 0, a);
      launch_merge<KV, D, MODE, GROUPED>(a, stream, tm.stop);
      return;
    }
  }
  hipExtLaunchKernelGGL((decode_kernel<KV, D, BS, MODE, GROUPED, false>), dim3(wg), dim3(a.waves_per_group * 64),
                        lds, stream, tm.start, nullptr, 0, a);
  launch_merge<KV, D, MODE, GROUPED>(a, stream, tm.stop);
}

template <class KV, int D, int BS, int MODE>
void launch_decode(const DecodeArgs& a, int wg, hipStream_t stream, const pkv::CallEvents& tm) {
  if constexpr ((MODE == kPlain || MODE == kAppend) && KV::kGrouped) {
    if (a.prefix_blocks != nullptr) {
      launch_decode_g<KV, D, BS, MODE, true>(a, wg, stream, tm);
      return;
    }
  }
  launch_decode_g<KV, D, BS, MODE, false>(a, wg, stream, tm);
}

template <class KV, int D, int MODE>
void launch_decode_bs(const DecodeArgs& a, int wg, int32_t bs, hipStream_t stream, const pkv::CallEvents& tm) {
  switch (bs) {
    case 8: launch_decode<KV, D, 8, MODE>(a, wg, stream, tm); break;
    case 16: launch_decode<KV, D, 16, MODE>(a, wg, stream, tm); break;
    default: launch_decode<KV, D, 32, MODE>(a, wg, stream, tm); break;
  }
}

template <class KV, int MODE>
void launch_decode_m(const DecodeArgs& a, int wg, int32_t bs, int32_t d, hipStream_t stream,
                     const pkv::CallEvents& tm) {
  if (d == 64) launch_decode_bs<KV, 64, MODE>(a, wg, bs, stream, tm);
  else launch_decode_bs<KV, 128, MODE>(a, wg, bs, stream, tm);
}

// The mode follows from the arguments: new rows given -> APPEND, a score
// request -> SCORES (the entry points never ask for both).
template <class KV>
void launch_decode_d(const DecodeArgs& a, int wg, int32_t bs, int32_t d, hipStream_t stream,
                     const pkv::CallEvents& tm) {
  if (a.k_new != nullptr) launch_decode_m<KV, kAppend>(a, wg, bs, d, stream, tm);
  else if (a.logits != nullptr) launch_decode_m<KV, kScores>(a, wg, bs, d, stream, tm);
  else launch_decode_m<KV, kPlain>(a, wg, bs, d, stream, tm);
}

// Cumulative-score workspace: logits [batch][H][padded_logit_stride] float32,
// then the final (max, sum) [batch][H] float2, each region 256-byte aligned.
inline size_t scores_workspace_bytes(int32_t batch, int32_t num_heads, int32_t max_seq_len) {
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  return up(static_cast<size_t>(batch) * num_heads * padded_logit_stride(max_seq_len) * sizeof(float)) +
         up(static_cast<size_t>(batch) * num_heads * sizeof(float2));
}

// The optional cumulative-score request of a decode call.
struct ScoreRequest {
  float* scores;
  int32_t score_stride;
  float decay;
  void* workspace;
  size_t workspace_bytes;
};

inline int attach_scores(DecodeArgs& a, const ScoreRequest* sc, int32_t batch, int32_t num_heads,
                         int32_t max_seq_len, const char* what) {
  if (sc == nullptr) return PKV_OK;
  if (sc->scores == nullptr || sc->workspace == nullptr)
    return pkv::fail(PKV_ERR_INVALID, "%s: null score buffer or score workspace", what);
  if (sc->score_stride < max_seq_len)
    return pkv::fail(PKV_ERR_INVALID, "%s: score_stride %d below max_seq_len %d", what, sc->score_stride,
                     max_seq_len);
  if (!std::isfinite(sc->decay)) return pkv::fail(PKV_ERR_INVALID, "%s: decay must be finite", what);
  const size_t need = scores_workspace_bytes(batch, num_heads, max_seq_len);
  const int32_t stride = padded_logit_stride(max_seq_len);
  if (sc->workspace_bytes < need)
    return pkv::fail(PKV_ERR_INVALID, "%s: score workspace of %zu bytes needed, %zu given", what, need,
                     sc->workspace_bytes);
  auto up = [](size_t x) { return (x + 255) / 256 * 256; };
  char* base = static_cast<char*>(sc->workspace);
  a.logits = reinterpret_cast<float*>(base);
  a.final_ml = reinterpret_cast<float2*>(base + up(static_cast<size_t>(batch) * num_heads * stride * 4));
  a.scores = sc->scores;
  a.logit_stride = stride;
  a.score_stride = sc->score_stride;
  a.decay = sc->decay;
  return PKV_OK;
}

// Checks of the scalar arguments of a decode call (made before anything else
// so that an empty batch still reports them).
inline int check_decode_scalars(float scale, int32_t num_work_groups) {
  if (!(std::isfinite(scale))) return pkv::fail(PKV_ERR_INVALID, "attention_decode: scale must be finite");
  if (num_work_groups < 0 || num_work_groups > (1 << 20))
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: num_work_groups %d out of range", num_work_groups);
  return PKV_OK;
}

// Host-side checks and set-up shared by both decode entry points; fills
// everything in `a` except the per-slice pointers and batch.  Returns the
// work-group count (> 0) or a negative status.
inline int prepare_decode(DecodeArgs& a, const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                          int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size,
                          int32_t num_blocks, float scale, pkv_dtype cache_dtype, int32_t num_work_groups,
                          void* workspace, size_t workspace_bytes, const void* out, bool grouped = false) {
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: null pointer");
  const int32_t wg = num_work_groups > 0 ? num_work_groups : auto_work_groups(cache_dtype);
  if (wg <= 0) return wg;
  const Layout ws = workspace_layout(batch, num_heads, head_dim, cache_dtype, wg, grouped);
  if (workspace == nullptr || workspace_bytes < ws.total)
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: workspace of %zu bytes needed, %zu given", ws.total,
                     workspace_bytes);
  const Shape sh = decode_shape(num_heads, head_dim, cache_dtype);
  char* base = static_cast<char*>(workspace);
  a.k = const_cast<void*>(k_cache);
  a.v = const_cast<void*>(v_cache);
  a.k_scales = nullptr;
  a.v_scales = nullptr;
  a.k_new = nullptr;
  a.v_new = nullptr;
  a.logits = nullptr;
  a.final_ml = nullptr;
  a.scores = nullptr;
  a.logit_stride = 0;
  a.score_stride = 0;
  a.decay = 0.f;
  a.prefix_blocks = nullptr;
  a.prefix_state = nullptr;
  a.prefix_row = 0;
  a.prefix_parts = 0;
  a.prefix_batch = 0;
  a.grid_decode = wg;
  a.ws_plan = reinterpret_cast<int32_t*>(base + ws.plan);
  a.ws_acc = reinterpret_cast<float*>(base + ws.acc);
  a.ws_ml = reinterpret_cast<float2*>(base + ws.ml);
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.num_heads = num_heads;
  a.num_blocks = num_blocks;
  a.groups_y = sh.groups_y;
  a.waves_per_group = sh.wpg;
  a.heads_per_wave = sh.hpw;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  return wg;
}

// Runs `launch(a, tm)` over slices of the batch small enough for the on-chip
// prefix arrays; the slices run one after another on the stream and share the
// workspace.  The timing events go to the first slice's first kernel and the
// last slice's last kernel.
template <class Launch>
int run_sliced(const DecodeArgs& base, void* out, const void* q, const int32_t* block_tables,
               int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t batch, int64_t q_row_bytes,
               const pkv::CallEvents& timing, Launch launch) {
  DecodeArgs a = base;
  const int32_t per_launch = (base.prefix_blocks != nullptr ? kMaxVirtualGrouped : kMaxVirtual) / a.groups_y;
  for (int32_t b0 = 0; b0 < batch; b0 += per_launch) {
    const pkv::CallEvents tm{b0 == 0 ? timing.start : nullptr,
                             b0 + per_launch >= batch ? timing.stop : nullptr};
    a.batch = batch - b0 < per_launch ? batch - b0 : per_launch;
    a.out = static_cast<char*>(out) + b0 * q_row_bytes;
    a.q = static_cast<const char*>(q) + b0 * q_row_bytes;
    if (base.k_new) {
      a.k_new = static_cast<const char*>(base.k_new) + b0 * q_row_bytes;
      a.v_new = static_cast<const char*>(base.v_new) + b0 * q_row_bytes;
    }
    if (base.logits) {
      a.logits = base.logits + static_cast<int64_t>(b0) * base.num_heads * base.logit_stride;
      a.final_ml = base.final_ml + static_cast<int64_t>(b0) * base.num_heads;
      a.scores = base.scores + static_cast<int64_t>(b0) * base.score_stride;
    }
    a.tables = block_tables + static_cast<int64_t>(b0) * max_blocks_per_seq;
    a.lens = seq_lens + b0;
    if (base.prefix_blocks) {
      a.prefix_blocks = base.prefix_blocks + b0;
      a.prefix_state = base.prefix_state + static_cast<int64_t>(b0) * base.num_heads * base.prefix_row;
    }
    launch(a, tm);
    const int st = check_launch("attention_decode");
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // namespace
