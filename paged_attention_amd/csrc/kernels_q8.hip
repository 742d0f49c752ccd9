// 8-bit K/V cache (int8 or OCP FP8 E4M3): quantising scatter and decode
// attention that dequantises inside the kernel, plus their C entry points.
//
// An 8-bit cache halves the bytes per token against fp16, and it changes
// nothing else of the paging: block tables, slots and block copies are the
// same (hnwysp.cn/news/103996 §5.4; icman.com.cn/news/78786 §1.3;
// m.lqnn.cn/news/240480 §6.2).
//
// Format.  Every (token, head) row of head_dim values is stored as head_dim
// code bytes plus one float32 scale:
//   scale = max |x| / QMAX            (QMAX = 127 for int8, 448 for FP8 E4M3)
//   r     = x / scale                 (IEEE float32 division)
//   int8: code = clamp(rint(r), -127, 127)
//   fp8:  code = E4M3 value nearest to clamp(r, -448, 448), ties to even
// and a row of zeros stores scale 0 and zero codes.  Reading gives
// code * scale.  Codes sit in the usual pool layout
// [num_blocks][block_size][H][D] (one byte each); scales sit in
// [num_blocks][H][block_size] so that a head's scales for the 8 tokens of a
// chunk are 32 contiguous bytes.
//
// Decode reuses the stream-K kernel of decode_common.h with a policy whose
// lanes hold 16 codes (one 16-byte load per lane per token for K and for V),
// fold the K scale into the score and the V scale into the softmax weight.
// For q.k over FP8 codes, fp16 and bf16 queries meet the codes as 16-bit
// pairs in dot2 instructions; otherwise the codes become floats
// (v_cvt_pk_f32_fp8 for E4M3, signed byte conversion for int8).
#include "decode_common.h"
#include "prefix_common.h"

namespace {

typedef float float2v __attribute__((ext_vector_type(2)));

// ---- quantising scatter ----------------------------------------------------

constexpr int kQuantElems = 8;   // row elements per thread

template <int KT>
__device__ __forceinline__ float qmax() {
  return KT == PKV_I8 ? 127.f : 448.f;
}

// E4M3 code of r (finite, |r| <= 448), nearest value with ties to the even
// code, from the float32 bit pattern: normal values keep 3 mantissa bits
// (rounding may carry into the exponent), values below 2^-6 land on the
// subnormal grid of 2^-9.
__device__ __forceinline__ uint32_t e4m3_code(float r) {
  const uint32_t sign = (__float_as_uint(r) >> 24) & 0x80u;
  const float a = fabsf(r);
  uint32_t mag;
  if (a < 0.015625f) {
    mag = static_cast<uint32_t>(rintf(a * 512.f));     // 0..8; 8 is the smallest normal
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7ffffu + ((b >> 20) & 1u);                  // round the mantissa to 3 bits, ties to even
    mag = (b >> 20) - (120u << 3);                     // rebias the exponent: 127 -> 7
  }
  return sign | mag;
}

template <int KT>
__device__ __forceinline__ uint32_t quant_code(float r) {
  if constexpr (KT == PKV_I8) {
    const int c = min(127, max(-127, static_cast<int>(rintf(r))));
    return static_cast<uint32_t>(c) & 0xffu;
  } else {
    return e4m3_code(fminf(fmaxf(r, -448.f), 448.f));
  }
}

// One thread per 8 elements of one (token, head) row of K (blockIdx.y = 0)
// or V (1); the D / 8 threads of a row are adjacent lanes and find the row's
// largest magnitude with DPP.  A row whose slot is negative or out of range
// is skipped as a whole, so the lanes of a row are active together.
template <int ST, int KT, int D>
__global__ void __launch_bounds__(256) append_q8_kernel(const uint8_t* __restrict__ k_new,
                                                        const uint8_t* __restrict__ v_new,
                                                        const int64_t* __restrict__ slots,
                                                        uint8_t* __restrict__ k_cache, uint8_t* __restrict__ v_cache,
                                                        float* __restrict__ k_scales, float* __restrict__ v_scales,
                                                        int32_t num_tokens, int32_t num_heads, int32_t block_size,
                                                        int64_t total_slots) {
  constexpr int R = D / kQuantElems;   // threads per row
  constexpr int SB = dtype_bytes(ST);
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t row = i / R;
  const int part = static_cast<int>(i % R);
  if (row >= static_cast<int64_t>(num_tokens) * num_heads) return;
  const int64_t t = row / num_heads;
  const int h = static_cast<int>(row % num_heads);
  const int64_t s = slots[t];
  if (s < 0 || s >= total_slots) return;
  const bool is_v = blockIdx.y == 1;
  const uint8_t* src = (is_v ? v_new : k_new) + (row * D + part * kQuantElems) * SB;
  float x[kQuantElems];
#pragma unroll
  for (int k = 0; k < kQuantElems * SB / 16; ++k)
    unpack16<ST>(reinterpret_cast<const Vec16*>(src)[k], x + k * (16 / SB));
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < kQuantElems; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = group_max<R>(amax);
  const float scale = amax / qmax<KT>();
  uint32_t w0 = 0, w1 = 0;
  if (scale > 0.f) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      w0 |= quant_code<KT>(x[e] / scale) << (8 * e);
      w1 |= quant_code<KT>(x[e + 4] / scale) << (8 * e);
    }
  }
  uint8_t* dst = (is_v ? v_cache : k_cache) + (s * num_heads + h) * D + part * kQuantElems;
  *reinterpret_cast<uint2*>(dst) = make_uint2(w0, w1);
  if (part == 0) {
    float* sc = is_v ? v_scales : k_scales;
    sc[((s / block_size) * num_heads + h) * block_size + s % block_size] = scale;
  }
}

// ---- decode attention (8-bit caches) ---------------------------------------

// Format policy of 8-bit caches: a lane holds 16 codes of a row; q (fp32,
// fp16 or bf16) is widened to 16 floats once per sequence.
template <int Q, int K>
struct Q8KV {
  static constexpr int QT = Q;
  static constexpr int KB = 1;
  static constexpr int EPL = 16;
  static constexpr int kMaxWaves = 8;
  static constexpr bool kGrouped = true;   // pkv_attention_decode_grouped_quant uses this policy
  static constexpr bool kDual = true;      // two chunk streams of 4 wavefronts per work-group where they fit
  // q.k on 16-bit pairs (see qk16).
  static constexpr bool kPairQK = K == PKV_FP8_E4M3 && (Q == PKV_F16 || Q == PKV_BF16);
  struct QReg {
    float f[16];     // the lane's 16 query elements as floats
    uint32_t p[8];   // the same elements as raw 16-bit pairs (fp16 / bf16 queries)
  };

  __device__ static QReg load_q(const uint8_t* p) {
    constexpr int per = 16 / dtype_bytes(Q);
    QReg r;
#pragma unroll
    for (int k = 0; k < 16 / per; ++k) {
      const Vec16 v = reinterpret_cast<const Vec16*>(p)[k];
      unpack16<Q>(v, r.f + k * per);
      if constexpr (Q != PKV_F32) {
#pragma unroll
        for (int i = 0; i < 4; ++i) r.p[4 * k + i] = v.w[i];
      }
    }
    return r;
  }

  // q.k over one 16-byte load of K codes (this lane's 16 elements), float32
  // accumulation.  With kPairQK two FP8 codes at a time become an f16 or bf16
  // pair (v_cvt_scalef32_pk_*_fp8 with scale 1: every E4M3 value is exact in
  // both) that a dot2 instruction multiplies with the matching pair of q.
  // Otherwise the codes are widened to floats.  (An int8 form, the f16 value
  // 1152 + c built by a byte permute with 1152 * sum(q) taken off afterwards,
  // measured no faster and loses bits of q.k for large queries.)
  __device__ static float qk16(const QReg& q, const Vec16& w) {
    if constexpr (kPairQK) {
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if constexpr (Q == PKV_F16) {
          const half2v lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.w[i], 1.f, false);
          const half2v hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w.w[i], 1.f, true);
          d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, q.p[2 * i]), lo, d, false);
          d = __builtin_amdgcn_fdot2(__builtin_bit_cast(half2v, q.p[2 * i + 1]), hi, d, false);
        } else {
          const auto lo = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w[i], 1.f, false);
          const auto hi = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w.w[i], 1.f, true);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, q.p[2 * i]), __builtin_bit_cast(bf162v, lo),
                                              d, false);
          d = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf162v, q.p[2 * i + 1]),
                                              __builtin_bit_cast(bf162v, hi), d, false);
        }
      }
      return d;
    } else {
      float c[16];
      codes16(w, c);
      float d = 0.f;
#pragma unroll
      for (int e = 0; e < 16; ++e) d = fmaf(q.f[e], c[e], d);
      return d;
    }
  }

  // The 16 code values of one 16-byte load, in byte order (unscaled).
  __device__ static void codes16(const Vec16& w, float* o) {
    if constexpr (K == PKV_FP8_E4M3) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float2v lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.w[i]), false);
        const float2v hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w.w[i]), true);
        o[4 * i] = lo.x;
        o[4 * i + 1] = lo.y;
        o[4 * i + 2] = hi.x;
        o[4 * i + 3] = hi.y;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) o[4 * i + j] = static_cast<float>(static_cast<int8_t>(w.w[i] >> (8 * j)));
    }
  }

  template <int D, int BS, int LPH, bool SCORES>
  __device__ static void chunk(const QReg& q, const DecodeArgs& a, const uint8_t* kp, const uint8_t* vp, int32_t blk,
                               int pos0, int head, int64_t row_bytes, int lastu, int valid, float& m, float& l,
                               float* acc, float* logit_slot, int lane_c) {
    const int64_t base = (static_cast<int64_t>(blk) * BS + pos0) * row_bytes;
    Vec16 kr[kChunk], vr[kChunk];
    // As in the 16/32-bit path, K codes take ordinary loads and V codes
    // non-temporal ones.  Measured on MI355X, us per call (ordinary / V
    // non-temporal / both): FP8 7B-shaped layer 65.7 / 63.0 / 68.3; int8
    // 13B-shaped long context 151.0 / 128.7 / -; FP8 with 64 sequences
    // sharing a 520-token prefix 75.4 / 82.6 / - (the one workload here that
    // loses: sharers re-read V prefix blocks that are no longer cached).
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int64_t ro = base + static_cast<int64_t>(u < lastu ? u : lastu) * row_bytes;
      kr[u] = *reinterpret_cast<const Vec16*>(kp + ro);
      vr[u] = stream_load(vp + ro);
    }
    // Scales of the chunk's 8 positions (positions past the segment are
    // read but never used: their weights are selected to zero).
    const int64_t so = (static_cast<int64_t>(blk) * a.num_heads + head) * BS + pos0;
    const float4 k0 = *reinterpret_cast<const float4*>(a.k_scales + so);
    const float4 k1 = *reinterpret_cast<const float4*>(a.k_scales + so + 4);
    const float4 v0 = *reinterpret_cast<const float4*>(a.v_scales + so);
    const float4 v1 = *reinterpret_cast<const float4*>(a.v_scales + so + 4);
    const float ks[kChunk] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
    const float vs[kChunk] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};

    float s[kChunk];
    float mc = m;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      s[u] = group_sum<LPH>(qk16(q, kr[u])) * (ks[u] * a.scale_log2);
      if (u < valid) mc = fmaxf(mc, s[u]);
    }
    if constexpr (SCORES) stage_logits(logit_slot, s, lane_c);
    const float alpha = __builtin_amdgcn_exp2f(m - mc);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[e] *= alpha;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float pu = u < valid ? __builtin_amdgcn_exp2f(s[u] - mc) : 0.f;
      const float pv = u < valid ? pu * vs[u] : 0.f;
      l += pu;
      float c[16];
      codes16(vr[u], c);
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = fmaf(pv, c[e], acc[e]);
    }
    m = mc;
  }

  // Quantises one row part of 16 elements held by this lane; the LPH lanes of
  // the head agree on the scale through a DPP maximum.  Every lane of the
  // head stores the (same) scale, so each reads back its own store.
  template <int LPH>
  __device__ static void quant_store(const uint8_t* src, uint8_t* dst, float* scale_dst) {
    const QReg x = load_q(src);
    float amax = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x.f[e]));
    amax = group_max<LPH>(amax);
    const float scale = amax / qmax<K>();
    Vec16 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w.w[i] = 0;
      if (scale > 0.f) {
#pragma unroll
        for (int j = 0; j < 4; ++j) w.w[i] |= quant_code<K>(x.f[4 * i + j] / scale) << (8 * j);
      }
    }
    *reinterpret_cast<Vec16*>(dst) = w;
    *scale_dst = scale;
  }

  template <int D, int BS, int LPH>
  __device__ static void store_new(const DecodeArgs& a, int b, int head, int e0, int32_t blk, int pos,
                                   int64_t row_bytes) {
    constexpr int QB = dtype_bytes(Q);
    const int64_t src = (static_cast<int64_t>(b) * a.num_heads * D + e0) * QB;
    const int64_t dst = (static_cast<int64_t>(blk) * BS + pos) * row_bytes + e0;
    const int64_t so = (static_cast<int64_t>(blk) * a.num_heads + head) * BS + pos;
    quant_store<LPH>(static_cast<const uint8_t*>(a.k_new) + src, static_cast<uint8_t*>(a.k) + dst, a.k_scales + so);
    quant_store<LPH>(static_cast<const uint8_t*>(a.v_new) + src, static_cast<uint8_t*>(a.v) + dst, a.v_scales + so);
  }
};

// Prefix-kernel load policy of 8-bit caches with f16 or bf16 queries: the
// codes enter the matrix cores as the query's type (every E4M3 value and
// every int8 value in [-127, 127] is exact in f16 and in bf16), the scales
// act on scores and weights.
template <int Q, int K>
struct PrefixQ8 {
  static_assert(Q == PKV_F16 || Q == PKV_BF16, "matrix-core input types");
  static constexpr int MT = Q;
  static constexpr int KB = 1;
  static constexpr bool kScaled = true;
  __device__ static uint32_t bits16(float x) { return Q == PKV_F16 ? f16_bits(x) : bf16_rne(x); }
  template <int N>
  __device__ static void widen(const uint32_t* raw, uint32_t* w) {
#pragma unroll
    for (int i = 0; i < N / 4; ++i) {
      if constexpr (K == PKV_FP8_E4M3) {
        if constexpr (Q == PKV_F16) {
          w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i], 1.f, false));
          w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(raw[i], 1.f, true));
        } else {
          w[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], 1.f, false));
          w[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(raw[i], 1.f, true));
        }
      } else {
        float c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = static_cast<float>(static_cast<int8_t>(raw[i] >> (8 * j)));
        w[2 * i] = bits16(c[0]) | (bits16(c[1]) << 16);
        w[2 * i + 1] = bits16(c[2]) | (bits16(c[3]) << 16);
      }
    }
  }
  __device__ static const float* k_scales(const DecodeArgs& a) { return a.k_scales; }
  __device__ static const float* v_scales(const DecodeArgs& a) { return a.v_scales; }
};

using pkv::aligned16;

template <int ST, int KT>
void launch_append_q8(int32_t head_dim, dim3 grid, hipStream_t stream, const void* k_new, const void* v_new,
                      const int64_t* slots, void* kc, void* vc, float* ks, float* vs, int32_t num_tokens,
                      int32_t num_heads, int32_t block_size, int64_t total_slots) {
  auto run = [&](auto kernel) {
    hipLaunchKernelGGL(kernel, grid, dim3(256), 0, stream, static_cast<const uint8_t*>(k_new),
                       static_cast<const uint8_t*>(v_new), slots, static_cast<uint8_t*>(kc),
                       static_cast<uint8_t*>(vc), ks, vs, num_tokens, num_heads, block_size, total_slots);
  };
  if (head_dim == 64)
    run(append_q8_kernel<ST, KT, 64>);
  else
    run(append_q8_kernel<ST, KT, 128>);
}

template <int KT>
void launch_decode_q8(const DecodeArgs& a, int wg, int32_t bs, int32_t d, pkv_dtype q_dtype, hipStream_t stream,
                      const pkv::CallEvents& tm) {
  switch (q_dtype) {
    case PKV_F32: launch_decode_d<Q8KV<PKV_F32, KT>>(a, wg, bs, d, stream, tm); break;
    case PKV_F16: launch_decode_d<Q8KV<PKV_F16, KT>>(a, wg, bs, d, stream, tm); break;
    default: launch_decode_d<Q8KV<PKV_BF16, KT>>(a, wg, bs, d, stream, tm); break;
  }
}

// Both 8-bit decode entry points; k_new != nullptr selects the variant that
// first quantises and stores each sequence's new row at its position L - 1.
int decode_q8(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
              const void* v_cache, const float* k_scales, const float* v_scales, const int32_t* block_tables,
              int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
              int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
              pkv_dtype q_dtype, pkv_dtype cache_dtype, int32_t num_work_groups, void* workspace,
              size_t workspace_bytes, hipStream_t stream, const char* what, const ScoreRequest* sc = nullptr) {
  const pkv::CallEvents timing = pkv::take_call_events();  // consumed by this call, whatever its outcome
  if (batch < 0 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 || max_seq_len < 0 ||
      !supported_geometry(head_dim, block_size) || !is_16_32(q_dtype) || !is_8bit(cache_dtype))
    return pkv::fail(PKV_ERR_INVALID, "%s: unsupported sizes (batch %d, heads %d, head_dim %d, block %d, blocks %d, "
                                      "max_blocks %d, max_len %d, q dtype %d, cache dtype %d)", what, batch,
                     num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq, max_seq_len,
                     static_cast<int>(q_dtype), static_cast<int>(cache_dtype));
  const int st = check_decode_scalars(scale, num_work_groups);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  if (!k_scales || !v_scales) return pkv::fail(PKV_ERR_INVALID, "%s: null scale pool", what);
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_scales) ||
      !aligned16(v_scales))
    return pkv::fail(PKV_ERR_INVALID, "%s: q, out, pools and scales must be 16-byte aligned", what);
  DecodeArgs a;
  const int wg = prepare_decode(a, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                batch, num_heads, head_dim, block_size, num_blocks, scale, cache_dtype,
                                num_work_groups, workspace, workspace_bytes, out);
  if (wg <= 0) return wg;
  a.k_scales = const_cast<float*>(k_scales);
  a.v_scales = const_cast<float*>(v_scales);
  a.k_new = k_new;
  a.v_new = v_new;
  const int sst = attach_scores(a, sc, batch, num_heads, max_seq_len, what);
  if (sst != PKV_OK) return sst;
  const int64_t row = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(q_dtype);
  return run_sliced(a, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, row, timing,
                    [&](const DecodeArgs& s, const pkv::CallEvents& tm) {
                      if (cache_dtype == PKV_I8)
                        launch_decode_q8<PKV_I8>(s, wg, block_size, head_dim, q_dtype, stream, tm);
                      else
                        launch_decode_q8<PKV_FP8_E4M3>(s, wg, block_size, head_dim, q_dtype, stream, tm);
                    });
}

template <int Q, int K>
void launch_prefix_q8(const DecodeArgs& pa, int32_t bs, int32_t d, const int32_t* tiles, int32_t num_tiles,
                      hipStream_t stream, hipEvent_t start) {
  if (d == 64) launch_prefix<PrefixQ8<Q, K>, 64>(pa, bs, tiles, num_tiles, stream, start);
  else launch_prefix<PrefixQ8<Q, K>, 128>(pa, bs, tiles, num_tiles, stream, start);
}

// Both 8-bit grouped entry points; k_new != nullptr selects the variant that
// first quantises and stores each sequence's new row at its position L - 1.
int decode_grouped_q8(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                      const void* v_cache, const float* k_scales, const float* v_scales, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                      int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                      pkv_dtype q_dtype, pkv_dtype cache_dtype, const int32_t* seq_prefix_blocks,
                      const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups, void* workspace,
                      size_t workspace_bytes, hipStream_t stream, const char* what) {
  const pkv::CallEvents timing = pkv::take_call_events();  // consumed by this call, whatever its outcome
  const int sz = check_grouped_sizes(what, batch, num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                     max_seq_len, num_tiles);
  if (sz != PKV_OK) return sz;
  if ((q_dtype != PKV_F16 && q_dtype != PKV_BF16) || !is_8bit(cache_dtype))
    return pkv::fail(PKV_ERR_INVALID, "%s: queries must be f16 or bf16 and the cache 8-bit (q dtype %d, cache %d)",
                     what, static_cast<int>(q_dtype), static_cast<int>(cache_dtype));
  const int st = check_decode_scalars(scale, num_work_groups);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  if (!seq_prefix_blocks || (num_tiles > 0 && !tiles))
    return pkv::fail(PKV_ERR_INVALID, "%s: null prefix arrays", what);
  if (!k_scales || !v_scales) return pkv::fail(PKV_ERR_INVALID, "%s: null scale pool", what);
  if (!aligned16(q) || !aligned16(out) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(k_scales) ||
      !aligned16(v_scales))
    return pkv::fail(PKV_ERR_INVALID, "%s: q, out, pools and scales must be 16-byte aligned", what);
  DecodeArgs a;
  const int wg = prepare_decode(a, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                batch, num_heads, head_dim, block_size, num_blocks, scale, cache_dtype,
                                num_work_groups, workspace, workspace_bytes, out, /*grouped=*/true);
  if (wg <= 0) return wg;
  a.k_scales = const_cast<float*>(k_scales);
  a.v_scales = const_cast<float*>(v_scales);
  a.k_new = k_new;
  a.v_new = v_new;
  const int64_t row = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(q_dtype);
  const bool fp8 = cache_dtype == PKV_FP8_E4M3;
  return run_grouped(
      a, wg, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, num_heads, head_dim, cache_dtype, row,
      seq_prefix_blocks, num_tiles, workspace, workspace_bytes, timing, what,
      [&](const DecodeArgs& pa, hipEvent_t start) {
        if (q_dtype == PKV_F16) {
          if (fp8) launch_prefix_q8<PKV_F16, PKV_FP8_E4M3>(pa, block_size, head_dim, tiles, num_tiles, stream, start);
          else launch_prefix_q8<PKV_F16, PKV_I8>(pa, block_size, head_dim, tiles, num_tiles, stream, start);
        } else {
          if (fp8) launch_prefix_q8<PKV_BF16, PKV_FP8_E4M3>(pa, block_size, head_dim, tiles, num_tiles, stream, start);
          else launch_prefix_q8<PKV_BF16, PKV_I8>(pa, block_size, head_dim, tiles, num_tiles, stream, start);
        }
      },
      [&](const DecodeArgs& s, const pkv::CallEvents& tm) {
        if (k_new != nullptr) {
          if (q_dtype == PKV_F16) {
            if (fp8) launch_decode_m<Q8KV<PKV_F16, PKV_FP8_E4M3>, kAppend>(s, wg, block_size, head_dim, stream, tm);
            else launch_decode_m<Q8KV<PKV_F16, PKV_I8>, kAppend>(s, wg, block_size, head_dim, stream, tm);
          } else {
            if (fp8) launch_decode_m<Q8KV<PKV_BF16, PKV_FP8_E4M3>, kAppend>(s, wg, block_size, head_dim, stream, tm);
            else launch_decode_m<Q8KV<PKV_BF16, PKV_I8>, kAppend>(s, wg, block_size, head_dim, stream, tm);
          }
        } else {
          if (q_dtype == PKV_F16) {
            if (fp8) launch_decode_m<Q8KV<PKV_F16, PKV_FP8_E4M3>, kPlain>(s, wg, block_size, head_dim, stream, tm);
            else launch_decode_m<Q8KV<PKV_F16, PKV_I8>, kPlain>(s, wg, block_size, head_dim, stream, tm);
          } else {
            if (fp8) launch_decode_m<Q8KV<PKV_BF16, PKV_FP8_E4M3>, kPlain>(s, wg, block_size, head_dim, stream, tm);
            else launch_decode_m<Q8KV<PKV_BF16, PKV_I8>, kPlain>(s, wg, block_size, head_dim, stream, tm);
          }
        }
      },
      [&](const DecodeArgs& s, const pkv::CallEvents& tm, int32_t units) {
        const int32_t bs = block_size, d = head_dim;
        if (k_new != nullptr) {
          if (q_dtype == PKV_F16) {
            if (fp8) return launch_fused<Q8KV<PKV_F16, PKV_FP8_E4M3>, PrefixQ8<PKV_F16, PKV_FP8_E4M3>, kAppend>(
                         s, bs, d, tiles, units, stream, tm);
            else return launch_fused<Q8KV<PKV_F16, PKV_I8>, PrefixQ8<PKV_F16, PKV_I8>, kAppend>(s, bs, d, tiles, units,
                                                                                         stream, tm);
          } else {
            if (fp8) return launch_fused<Q8KV<PKV_BF16, PKV_FP8_E4M3>, PrefixQ8<PKV_BF16, PKV_FP8_E4M3>, kAppend>(
                         s, bs, d, tiles, units, stream, tm);
            else return launch_fused<Q8KV<PKV_BF16, PKV_I8>, PrefixQ8<PKV_BF16, PKV_I8>, kAppend>(s, bs, d, tiles, units,
                                                                                           stream, tm);
          }
        } else {
          if (q_dtype == PKV_F16) {
            if (fp8) return launch_fused<Q8KV<PKV_F16, PKV_FP8_E4M3>, PrefixQ8<PKV_F16, PKV_FP8_E4M3>, kPlain>(
                         s, bs, d, tiles, units, stream, tm);
            else return launch_fused<Q8KV<PKV_F16, PKV_I8>, PrefixQ8<PKV_F16, PKV_I8>, kPlain>(s, bs, d, tiles, units,
                                                                                        stream, tm);
          } else {
            if (fp8) return launch_fused<Q8KV<PKV_BF16, PKV_FP8_E4M3>, PrefixQ8<PKV_BF16, PKV_FP8_E4M3>, kPlain>(
                         s, bs, d, tiles, units, stream, tm);
            else return launch_fused<Q8KV<PKV_BF16, PKV_I8>, PrefixQ8<PKV_BF16, PKV_I8>, kPlain>(s, bs, d, tiles, units,
                                                                                          stream, tm);
          }
        }
      });
}

}  // namespace

extern "C" {

PKV_API int pkv_attention_decode_grouped_quant(void* out, const void* q, const void* k_cache, const void* v_cache,
                                               const float* k_scales, const float* v_scales,
                                               const int32_t* block_tables, int32_t max_blocks_per_seq,
                                               const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                                               int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                               pkv_dtype cache_dtype, const int32_t* seq_prefix_blocks,
                                               const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_grouped_q8(out, q, nullptr, nullptr, k_cache, v_cache, k_scales, v_scales, block_tables,
                           max_blocks_per_seq, seq_lens, max_seq_len, batch, num_heads, head_dim, block_size,
                           num_blocks, scale, q_dtype, cache_dtype, seq_prefix_blocks, tiles, num_tiles,
                           num_work_groups, workspace, workspace_bytes, stream, "attention_decode_grouped_quant");
}

PKV_API int pkv_append_attention_decode_grouped_quant(
    void* out, const void* q, const void* k_new, const void* v_new, void* k_cache, void* v_cache, float* k_scales,
    float* v_scales, const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
    int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
    float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype, const int32_t* seq_prefix_blocks, const int32_t* tiles,
    int32_t num_tiles, int32_t num_work_groups, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  const char* what = "append_attention_decode_grouped_quant";
  if (batch > 0 && (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))) {
    pkv::take_call_events();  // a pending timing request belongs to this call
    return pkv::fail(PKV_ERR_INVALID, "%s: new rows must be non-null and 16-byte aligned", what);
  }
  return decode_grouped_q8(out, q, k_new, v_new, k_cache, v_cache, k_scales, v_scales, block_tables,
                           max_blocks_per_seq, seq_lens, max_seq_len, batch, num_heads, head_dim, block_size,
                           num_blocks, scale, q_dtype, cache_dtype, seq_prefix_blocks, tiles, num_tiles,
                           num_work_groups, workspace, workspace_bytes, stream, what);
}

PKV_API int pkv_append_quant(const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                             void* k_cache, void* v_cache, float* k_scales, float* v_scales, int32_t num_blocks,
                             int32_t block_size, int32_t num_heads, int32_t head_dim, pkv_dtype src_dtype,
                             pkv_dtype cache_dtype, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_heads <= 0 || !supported_geometry(head_dim, block_size) ||
      !is_16_32(src_dtype) || !is_8bit(cache_dtype))
    return pkv::fail(PKV_ERR_INVALID, "append_quant: unsupported sizes (tokens %d, blocks %d, heads %d, head_dim %d, "
                                      "block %d, src dtype %d, cache dtype %d)", num_tokens, num_blocks, num_heads,
                     head_dim, block_size, static_cast<int>(src_dtype), static_cast<int>(cache_dtype));
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache || !k_scales || !v_scales)
    return pkv::fail(PKV_ERR_INVALID, "append_quant: null pointer");
  if (!aligned16(k_new) || !aligned16(v_new) || !aligned16(k_cache) || !aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID, "append_quant: rows and pools must be 16-byte aligned");
  const int64_t threads = static_cast<int64_t>(num_tokens) * num_heads * (head_dim / kQuantElems);
  const int64_t blocks = (threads + 255) / 256;
  if (blocks > 0x7fffffff) return pkv::fail(PKV_ERR_INVALID, "append_quant: too many tokens");
  const dim3 grid(static_cast<uint32_t>(blocks), 2);
  const int64_t total = static_cast<int64_t>(num_blocks) * block_size;
#define PKV_APPEND_Q8(ST, KT)                                                                                  \
  launch_append_q8<ST, KT>(head_dim, grid, stream, k_new, v_new, slot_mapping, k_cache, v_cache, k_scales,  \
                           v_scales, num_tokens, num_heads, block_size, total)
  if (cache_dtype == PKV_I8) {
    switch (src_dtype) {
      case PKV_F32: PKV_APPEND_Q8(PKV_F32, PKV_I8); break;
      case PKV_F16: PKV_APPEND_Q8(PKV_F16, PKV_I8); break;
      default: PKV_APPEND_Q8(PKV_BF16, PKV_I8); break;
    }
  } else {
    switch (src_dtype) {
      case PKV_F32: PKV_APPEND_Q8(PKV_F32, PKV_FP8_E4M3); break;
      case PKV_F16: PKV_APPEND_Q8(PKV_F16, PKV_FP8_E4M3); break;
      default: PKV_APPEND_Q8(PKV_BF16, PKV_FP8_E4M3); break;
    }
  }
#undef PKV_APPEND_Q8
  return check_launch("append_quant");
}

PKV_API int pkv_attention_decode_quant(void* out, const void* q, const void* k_cache, const void* v_cache,
                                       const float* k_scales, const float* v_scales, const int32_t* block_tables,
                                       int32_t max_blocks_per_seq, const int32_t* seq_lens, int32_t max_seq_len,
                                       int32_t batch, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                       int32_t num_blocks, float scale, pkv_dtype q_dtype, pkv_dtype cache_dtype,
                                       int32_t num_work_groups, void* workspace, size_t workspace_bytes,
                                       hipStream_t stream) {
  return decode_q8(out, q, nullptr, nullptr, k_cache, v_cache, k_scales, v_scales, block_tables, max_blocks_per_seq,
                   seq_lens, max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, q_dtype,
                   cache_dtype, num_work_groups, workspace, workspace_bytes, stream, "attention_decode_quant");
}

PKV_API int pkv_attention_decode_quant_scores(void* out, const void* q, const void* k_cache, const void* v_cache,
                                              const float* k_scales, const float* v_scales,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                              pkv_dtype cache_dtype, int32_t num_work_groups, void* workspace,
                                              size_t workspace_bytes, float* scores, int32_t score_stride,
                                              float decay, void* scores_workspace, size_t scores_workspace_bytes,
                                              hipStream_t stream) {
  const ScoreRequest sc{scores, score_stride, decay, scores_workspace, scores_workspace_bytes};
  return decode_q8(out, q, nullptr, nullptr, k_cache, v_cache, k_scales, v_scales, block_tables, max_blocks_per_seq,
                   seq_lens, max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, q_dtype,
                   cache_dtype, num_work_groups, workspace, workspace_bytes, stream, "attention_decode_quant_scores",
                   &sc);
}

PKV_API int pkv_append_attention_decode_quant(void* out, const void* q, const void* k_new, const void* v_new,
                                              void* k_cache, void* v_cache, float* k_scales, float* v_scales,
                                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                                              const int32_t* seq_lens, int32_t max_seq_len, int32_t batch,
                                              int32_t num_heads, int32_t head_dim, int32_t block_size,
                                              int32_t num_blocks, float scale, pkv_dtype q_dtype,
                                              pkv_dtype cache_dtype, int32_t num_work_groups, void* workspace,
                                              size_t workspace_bytes, hipStream_t stream) {
  if (batch > 0 && (!k_new || !v_new))
    return pkv::fail(PKV_ERR_INVALID, "append_attention_decode_quant: null new rows");
  if (batch > 0 && (!aligned16(k_new) || !aligned16(v_new)))
    return pkv::fail(PKV_ERR_INVALID, "append_attention_decode_quant: new rows must be 16-byte aligned");
  return decode_q8(out, q, k_new, v_new, k_cache, v_cache, k_scales, v_scales, block_tables, max_blocks_per_seq,
                   seq_lens, max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, q_dtype,
                   cache_dtype, num_work_groups, workspace, workspace_bytes, stream, "append_attention_decode_quant");
}

}  // extern "C"
