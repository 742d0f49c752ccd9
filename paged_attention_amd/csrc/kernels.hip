// Device side of libpkv for gfx950 (CDNA4): K/V scatter, whole-block copy and
// decode attention over a paged cache, plus their C entry points.
//
// Pool layout (K and V alike): [num_blocks][block_size][num_heads][head_dim].
// One token's row for all heads is contiguous, so the rows a wavefront needs
// for a group of adjacent heads at one token form one contiguous 1 KiB run.
//
// Decode attention is a memory-bound matrix-vector product: per (token, head)
// it reads 2 * head_dim * dtype bytes and does about 4 * head_dim flops, far
// below the FP32 vector ridge point, so it runs on the vector ALUs, not MFMA.
// Work split:
//   - a work-group owns one (sequence, partition of P logical tokens) and
//     all heads: each wavefront takes HPW adjacent heads, and each head's row
//     is spread over LPH lanes holding 16 bytes each (one global_load_dwordx4
//     per lane per token fetches K, one fetches V);
//   - q.k is reduced across the LPH lanes with DPP row permutes;
//   - the softmax runs online over chunks of 8 tokens (running max m, sum l,
//     weighted value accumulator) in base 2 with log2(e) folded into the
//     scale;
//   - a sequence longer than one partition writes (m, l, acc) per head to the
//     workspace and a combine kernel merges the partitions.
// Block-table entries are wavefront-uniform, so they are read with scalar
// loads into SGPRs; every id is range-checked before it forms an address.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

#include "status.h"

namespace {

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

struct alignas(16) Vec16 {
  uint32_t w[4];
};

constexpr int kChunk = 8;        // tokens per online-softmax step
constexpr int kMaxWaves = 16;    // wavefronts per work-group at most
constexpr int kXcds = 8;         // accelerator dies; work-groups are dealt round-robin

__host__ __device__ constexpr int dtype_bytes(int dt) { return dt == PKV_F32 ? 4 : 2; }

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

// DPP lane permutes inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <- lane 15-i within 16

// Sum over each aligned group of N lanes (N = 8, 16 or 32); every lane of the
// group receives the total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<kDppXor1>(x);
  x += dpp<kDppXor2>(x);
  x += dpp<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp<kDppMirror>(x);
  if constexpr (N >= 32) x += __shfl_xor(x, 16, 64);
  return x;
}

// ---- append ----------------------------------------------------------------

__global__ void __launch_bounds__(256) append_kernel(const Vec16* __restrict__ k_new, const Vec16* __restrict__ v_new,
                                                     const int64_t* __restrict__ slots, Vec16* __restrict__ k_cache,
                                                     Vec16* __restrict__ v_cache, int32_t num_tokens, int32_t row_vec,
                                                     int64_t total_slots) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t t = i / row_vec;
  if (t >= num_tokens) return;
  const int64_t j = i - t * row_vec;
  const int64_t s = slots[t];
  if (s < 0 || s >= total_slots) return;
  k_cache[s * row_vec + j] = k_new[t * row_vec + j];
  v_cache[s * row_vec + j] = v_new[t * row_vec + j];
}

// ---- block copy ------------------------------------------------------------

constexpr int kCopyLayers = 32;  // layer pointers carried per launch

struct LayerPtrs {
  Vec16* k[kCopyLayers];
  Vec16* v[kCopyLayers];
};

__global__ void __launch_bounds__(256) copy_blocks_kernel(LayerPtrs ptrs, const int32_t* __restrict__ pairs,
                                                          int32_t num_blocks, int64_t vec_per_block) {
  const int pair = blockIdx.x;
  const int layer = blockIdx.y;
  const int32_t src = pairs[2 * pair];
  const int32_t dst = pairs[2 * pair + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks || src == dst) return;
  Vec16* base = blockIdx.z == 0 ? ptrs.k[layer] : ptrs.v[layer];
  const Vec16* from = base + static_cast<int64_t>(src) * vec_per_block;
  Vec16* to = base + static_cast<int64_t>(dst) * vec_per_block;
  for (int64_t i = threadIdx.x; i < vec_per_block; i += blockDim.x) to[i] = from[i];
}

// ---- decode attention ------------------------------------------------------

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k;
  const void* v;
  const int32_t* tables;
  const int32_t* lens;
  float* ws_acc;    // [batch][max_parts][H][D]
  float2* ws_ml;    // [batch][max_parts][H]  (running max in log2 units, sum)
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t num_heads;
  int32_t num_blocks;
  int32_t part;       // tokens per partition
  int32_t max_parts;  // stride of the partition axis in the workspace
  int32_t waves_per_group;
  int32_t block_size;
  float scale_log2;   // softmax scale * log2(e)
};

// One online-softmax step over a chunk of kChunk tokens whose K/V rows are
// already in registers.  `valid` = tokens of the chunk inside the partition.
template <int DT, int EPL, int LPH>
__device__ __forceinline__ void softmax_chunk(const Vec16& qv, const Vec16* kr, const Vec16* vr, int valid,
                                              float scale_log2, float& m, float& l, float* acc) {
  float s[kChunk];
  float mc = m;
#pragma unroll
  for (int u = 0; u < kChunk; ++u) {
    s[u] = group_sum<LPH>(dot16<DT>(qv, kr[u], 0.f)) * scale_log2;
    if (u < valid) mc = fmaxf(mc, s[u]);
  }
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

template <int DT, int D, int BS>
__global__ void __launch_bounds__(kMaxWaves * 64) decode_partition_kernel(DecodeArgs a) {
  constexpr int EPL = 16 / dtype_bytes(DT);  // elements per lane per 16-byte load
  constexpr int LPH = D / EPL;                // lanes holding one head's row
  constexpr int HPW = 64 / LPH;               // heads per wavefront
  static_assert(BS % kChunk == 0, "a chunk of tokens must sit inside one block");
  using Elem = uint8_t;                       // addresses are formed in bytes

  const int p = blockIdx.x;
  const int b = blockIdx.z;
  const int L = a.lens[b];
  const bool bad_len =
      L < 0 || L > a.max_seq_len || static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * BS;
  const int nparts = (bad_len || L == 0) ? 1 : (L + a.part - 1) / a.part;
  if (p >= nparts) return;

  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int hg = blockIdx.y * a.waves_per_group + wave;
  if (hg * HPW >= a.num_heads) return;  // this wavefront has no heads (no barriers follow)
  const int r = lane / LPH;
  const int c = lane % LPH;
  const int h = hg * HPW + r;
  const bool head_ok = h < a.num_heads;
  const int hl = head_ok ? h : a.num_heads - 1;  // clamped head for loads
  const int64_t row_bytes = static_cast<int64_t>(a.num_heads) * D * dtype_bytes(DT);
  // Per-lane byte offset inside a token row (32-bit: the uniform part of each
  // address stays in SGPRs).
  const uint32_t lane_off = static_cast<uint32_t>((hl * D + c * EPL) * dtype_bytes(DT));
  const int64_t out_off = static_cast<int64_t>(b) * row_bytes + lane_off;

  if (bad_len || L == 0) {
    if (head_ok) {
      float fill[EPL];
#pragma unroll
      for (int e = 0; e < EPL; ++e) fill[e] = bad_len ? __builtin_nanf("") : 0.f;
      *reinterpret_cast<Vec16*>(static_cast<Elem*>(a.out) + out_off) = pack16<DT>(fill);
    }
    return;
  }

  const int t_begin = p * a.part;
  const int n = min(a.part, L - t_begin);
  const int32_t* trow = a.tables + static_cast<int64_t>(b) * a.max_blocks + t_begin / BS;
  const Elem* kpool = static_cast<const Elem*>(a.k);
  const Elem* vpool = static_cast<const Elem*>(a.v);
  const Vec16 qv = *reinterpret_cast<const Vec16*>(static_cast<const Elem*>(a.q) + out_off);

  float m = -INFINITY;
  float l = 0.f;
  float acc[EPL];
#pragma unroll
  for (int e = 0; e < EPL; ++e) acc[e] = 0.f;
  bool bad_block = false;

  // Byte offset of the first row of the chunk starting at partition token t0.
  // The chunk never crosses a block (t_begin and t0 are multiples of kChunk
  // and kChunk divides BS).
  auto chunk_base = [&](int t0) -> int64_t {
    int32_t blk = trow[t0 / BS];
    if (static_cast<uint32_t>(blk) >= static_cast<uint32_t>(a.num_blocks)) {
      bad_block = true;
      blk = 0;
    }
    return (static_cast<int64_t>(blk) * BS + (t_begin + t0) % BS) * row_bytes;
  };
  auto load_chunk = [&](int t0, Vec16* kr, Vec16* vr) {
    const int64_t base = chunk_base(t0);
    const int last = n - 1 - t0;  // rows past the partition repeat its last row
    const Elem* kc = kpool + base;
    const Elem* vc = vpool + base;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const int64_t ro = static_cast<int64_t>(u < last ? u : last) * row_bytes;
      kr[u] = *reinterpret_cast<const Vec16*>(kc + ro + lane_off);
      vr[u] = *reinterpret_cast<const Vec16*>(vc + ro + lane_off);
    }
  };

  Vec16 kr[kChunk], vr[kChunk];
  for (int t0 = 0; t0 < n; t0 += kChunk) {
    load_chunk(t0, kr, vr);
    softmax_chunk<DT, EPL, LPH>(qv, kr, vr, n - t0, a.scale_log2, m, l, acc);
  }
  if (bad_block) l = __builtin_nanf("");
  if (!head_ok) return;

  if (nparts == 1) {
    const float inv = 1.f / l;
    float o[EPL];
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[e] = acc[e] * inv;
    *reinterpret_cast<Vec16*>(static_cast<Elem*>(a.out) + out_off) = pack16<DT>(o);
  } else {
    const int64_t slot = (static_cast<int64_t>(b) * a.max_parts + p) * a.num_heads + h;
    float* dst = a.ws_acc + slot * D + c * EPL;
#pragma unroll
    for (int e = 0; e < EPL; e += 4)
      *reinterpret_cast<float4*>(dst + e) = make_float4(acc[e], acc[e + 1], acc[e + 2], acc[e + 3]);
    if (c == 0) a.ws_ml[slot] = make_float2(m, l);
  }
}

// Merges the partitions of every sequence that has more than one:
//   M = max_i m_i,  S = sum_i l_i 2^(m_i - M),  out = sum_i acc_i 2^(m_i - M) / S.
template <int DT, int D>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a) {
  constexpr int kPer = 4;  // output elements per thread
  const int b = blockIdx.y;
  const int e0 = (blockIdx.x * blockDim.x + threadIdx.x) * kPer;
  if (e0 >= a.num_heads * D) return;
  const int L = a.lens[b];
  if (L <= 0 || L > a.max_seq_len || static_cast<int64_t>(L) > static_cast<int64_t>(a.max_blocks) * a.block_size) return;
  const int nparts = (L + a.part - 1) / a.part;
  if (nparts <= 1) return;
  const int h = e0 / D;
  const int64_t row = static_cast<int64_t>(b) * a.max_parts;
  float mx = -INFINITY;
  for (int p = 0; p < nparts; ++p) mx = fmaxf(mx, a.ws_ml[(row + p) * a.num_heads + h].x);
  float sum = 0.f;
  float o[kPer] = {0.f, 0.f, 0.f, 0.f};
  for (int p = 0; p < nparts; ++p) {
    const float2 ml = a.ws_ml[(row + p) * a.num_heads + h];
    const float w = __builtin_amdgcn_exp2f(ml.x - mx);
    sum += ml.y * w;
    const float4 av = *reinterpret_cast<const float4*>(a.ws_acc + ((row + p) * a.num_heads + h) * D + (e0 % D));
    o[0] = fmaf(av.x, w, o[0]);
    o[1] = fmaf(av.y, w, o[1]);
    o[2] = fmaf(av.z, w, o[2]);
    o[3] = fmaf(av.w, w, o[3]);
  }
  const float inv = 1.f / sum;
  const int64_t out_idx = static_cast<int64_t>(b) * a.num_heads * D + e0;
  if constexpr (DT == PKV_F32) {
    *reinterpret_cast<float4*>(static_cast<float*>(a.out) + out_idx) =
        make_float4(o[0] * inv, o[1] * inv, o[2] * inv, o[3] * inv);
  } else {
    uint32_t lo, hi;
    if constexpr (DT == PKV_F16) {
      lo = f16_bits(o[0] * inv) | (f16_bits(o[1] * inv) << 16);
      hi = f16_bits(o[2] * inv) | (f16_bits(o[3] * inv) << 16);
    } else {
      lo = bf16_rne(o[0] * inv) | (bf16_rne(o[1] * inv) << 16);
      hi = bf16_rne(o[2] * inv) | (bf16_rne(o[3] * inv) << 16);
    }
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out) + out_idx) = make_uint2(lo, hi);
  }
}

// ---- host helpers ----------------------------------------------------------

bool supported(int32_t head_dim, int32_t block_size, pkv_dtype dtype) {
  return (head_dim == 64 || head_dim == 128) && (block_size == 8 || block_size == 16 || block_size == 32) &&
         (dtype == PKV_F32 || dtype == PKV_F16 || dtype == PKV_BF16);
}

int heads_per_wave(int32_t head_dim, pkv_dtype dtype) {
  const int epl = 16 / dtype_bytes(dtype);
  return 64 / (head_dim / epl);
}

int32_t ceil_div(int64_t a, int64_t b) { return static_cast<int32_t>((a + b - 1) / b); }

int32_t auto_partition(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype, int32_t max_seq_len) {
  // Aim for enough wavefronts to keep every CU's memory pipeline full,
  // estimating the mean length as half the bound.
  const int64_t groups = ceil_div(num_heads, heads_per_wave(head_dim, dtype));
  const int64_t target = 256 * 16;
  const int64_t mean = max_seq_len / 2 + 1;
  for (int32_t part : {512, 256, 128}) {
    if (static_cast<int64_t>(batch) * ceil_div(mean, part) * groups >= target) return part;
  }
  return 64;
}

int check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return pkv::fail(PKV_ERR_HIP, "%s: launch failed: %s", what, hipGetErrorString(e));
  return PKV_OK;
}

template <int DT, int D, int BS>
void launch_decode(const DecodeArgs& a, int32_t batch, int groups, hipStream_t stream) {
  const int wpg = a.waves_per_group;
  dim3 grid(ceil_div(a.max_parts, kXcds) * kXcds, ceil_div(groups, wpg), batch);
  hipLaunchKernelGGL((decode_partition_kernel<DT, D, BS>), grid, dim3(wpg * 64), 0, stream, a);
  if (a.max_parts > 1) {
    dim3 cgrid(ceil_div(static_cast<int64_t>(a.num_heads) * D / 4, 256), batch);
    hipLaunchKernelGGL((decode_combine_kernel<DT, D>), cgrid, dim3(256), 0, stream, a);
  }
}

template <int DT, int D>
void launch_decode_bs(const DecodeArgs& a, int32_t batch, int groups, int32_t bs, hipStream_t stream) {
  switch (bs) {
    case 8: launch_decode<DT, D, 8>(a, batch, groups, stream); break;
    case 16: launch_decode<DT, D, 16>(a, batch, groups, stream); break;
    default: launch_decode<DT, D, 32>(a, batch, groups, stream); break;
  }
}

template <int DT>
void launch_decode_d(const DecodeArgs& a, int32_t batch, int groups, int32_t bs, int32_t d, hipStream_t stream) {
  if (d == 64)
    launch_decode_bs<DT, 64>(a, batch, groups, bs, stream);
  else
    launch_decode_bs<DT, 128>(a, batch, groups, bs, stream);
}

size_t workspace_for(int32_t batch, int32_t num_heads, int32_t head_dim, int32_t max_parts) {
  if (max_parts <= 1) return 0;
  const size_t slots = static_cast<size_t>(batch) * max_parts * num_heads;
  const size_t acc = (slots * head_dim * sizeof(float) + 255) / 256 * 256;
  return acc + (slots * sizeof(float2) + 255) / 256 * 256;
}

}  // namespace

extern "C" {

PKV_API int pkv_append(const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                       int32_t head_dim, pkv_dtype dtype, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_heads <= 0 || !supported(head_dim, block_size, dtype))
    return pkv::fail(PKV_ERR_INVALID, "append: unsupported sizes (tokens %d, blocks %d, heads %d, head_dim %d, "
                                      "block %d, dtype %d)", num_tokens, num_blocks, num_heads, head_dim, block_size,
                     static_cast<int>(dtype));
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return pkv::fail(PKV_ERR_INVALID, "append: null pointer");
  const int64_t row_vec = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(dtype) / 16;
  const int64_t total = static_cast<int64_t>(num_tokens) * row_vec;
  const int64_t blocks = (total + 255) / 256;
  if (blocks > 0x7fffffff) return pkv::fail(PKV_ERR_INVALID, "append: too many tokens");
  hipLaunchKernelGGL(append_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, stream,
                     static_cast<const Vec16*>(k_new), static_cast<const Vec16*>(v_new), slot_mapping,
                     static_cast<Vec16*>(k_cache), static_cast<Vec16*>(v_cache), num_tokens,
                     static_cast<int32_t>(row_vec), static_cast<int64_t>(num_blocks) * block_size);
  return check_launch("append");
}

PKV_API int pkv_copy_blocks(void* const* k_caches, void* const* v_caches, int32_t num_layers, const int32_t* pairs,
                            int32_t n_pairs, int32_t num_blocks, size_t bytes_per_block, hipStream_t stream) {
  if (num_layers < 0 || n_pairs < 0 || num_blocks <= 0 || bytes_per_block == 0 || bytes_per_block % 16 != 0)
    return pkv::fail(PKV_ERR_INVALID, "copy_blocks: bad sizes (layers %d, pairs %d, blocks %d, bytes %zu)", num_layers,
                     n_pairs, num_blocks, bytes_per_block);
  if (n_pairs == 0 || num_layers == 0) return PKV_OK;
  if (!k_caches || !v_caches || !pairs) return pkv::fail(PKV_ERR_INVALID, "copy_blocks: null pointer");
  if (n_pairs > 0x7fffffff / 2) return pkv::fail(PKV_ERR_INVALID, "copy_blocks: too many pairs");
  for (int32_t l0 = 0; l0 < num_layers; l0 += kCopyLayers) {
    const int32_t nl = num_layers - l0 < kCopyLayers ? num_layers - l0 : kCopyLayers;
    LayerPtrs ptrs{};
    for (int32_t i = 0; i < nl; ++i) {
      if (!k_caches[l0 + i] || !v_caches[l0 + i]) return pkv::fail(PKV_ERR_INVALID, "copy_blocks: null layer pool");
      ptrs.k[i] = static_cast<Vec16*>(k_caches[l0 + i]);
      ptrs.v[i] = static_cast<Vec16*>(v_caches[l0 + i]);
    }
    hipLaunchKernelGGL(copy_blocks_kernel, dim3(n_pairs, nl, 2), dim3(256), 0, stream, ptrs, pairs, num_blocks,
                       static_cast<int64_t>(bytes_per_block / 16));
    int st = check_launch("copy_blocks");
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

PKV_API int32_t pkv_decode_partition_tokens(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                            int32_t block_size, int32_t max_seq_len) {
  if (batch < 0 || num_heads <= 0 || max_seq_len < 0 || !supported(head_dim, block_size, dtype))
    return pkv::fail(PKV_ERR_INVALID, "decode_partition_tokens: unsupported sizes");
  return auto_partition(batch, num_heads, head_dim, dtype, max_seq_len);
}

PKV_API size_t pkv_decode_workspace_bytes(int32_t batch, int32_t num_heads, int32_t head_dim, pkv_dtype dtype,
                                          int32_t block_size, int32_t max_seq_len, int32_t partition_tokens) {
  if (batch < 0 || num_heads <= 0 || max_seq_len < 0 || !supported(head_dim, block_size, dtype)) return 0;
  const int32_t part =
      partition_tokens > 0 ? partition_tokens : auto_partition(batch, num_heads, head_dim, dtype, max_seq_len);
  if (part % 32 != 0) return 0;
  return workspace_for(batch, num_heads, head_dim, ceil_div(max_seq_len > 0 ? max_seq_len : 1, part));
}

PKV_API int pkv_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                 int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
                                 int32_t partition_tokens, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream) {
  if (batch < 0 || batch > 65535 || num_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_seq_len < 0 || !supported(head_dim, block_size, dtype))
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: unsupported sizes (batch %d, heads %d, head_dim %d, block %d, "
                                      "blocks %d, max_blocks %d, max_len %d, dtype %d)", batch, num_heads, head_dim,
                     block_size, num_blocks, max_blocks_per_seq, max_seq_len, static_cast<int>(dtype));
  if (!(std::isfinite(scale))) return pkv::fail(PKV_ERR_INVALID, "attention_decode: scale must be finite");
  if (partition_tokens < 0 || (partition_tokens > 0 && partition_tokens % 32 != 0))
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: partition_tokens %d is not a positive multiple of 32",
                     partition_tokens);
  if (batch == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !block_tables || !seq_lens)
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: null pointer");
  const int32_t part =
      partition_tokens > 0 ? partition_tokens : auto_partition(batch, num_heads, head_dim, dtype, max_seq_len);
  const int32_t max_parts = ceil_div(max_seq_len > 0 ? max_seq_len : 1, part);
  const size_t need = workspace_for(batch, num_heads, head_dim, max_parts);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need))
    return pkv::fail(PKV_ERR_INVALID, "attention_decode: workspace of %zu bytes needed, %zu given", need,
                     workspace_bytes);
  const int groups = ceil_div(num_heads, heads_per_wave(head_dim, dtype));
  DecodeArgs a;
  a.out = out;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.tables = block_tables;
  a.lens = seq_lens;
  const size_t slots = static_cast<size_t>(batch) * max_parts * num_heads;
  a.ws_acc = static_cast<float*>(workspace);
  a.ws_ml = need ? reinterpret_cast<float2*>(static_cast<char*>(workspace) +
                                             (slots * head_dim * sizeof(float) + 255) / 256 * 256)
                 : nullptr;
  a.max_blocks = max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.num_heads = num_heads;
  a.num_blocks = num_blocks;
  a.part = part;
  a.max_parts = max_parts;
  a.waves_per_group = groups < kMaxWaves ? groups : kMaxWaves;
  a.block_size = block_size;
  a.scale_log2 = scale * 1.4426950408889634f;
  switch (dtype) {
    case PKV_F32: launch_decode_d<PKV_F32>(a, batch, groups, block_size, head_dim, stream); break;
    case PKV_F16: launch_decode_d<PKV_F16>(a, batch, groups, block_size, head_dim, stream); break;
    default: launch_decode_d<PKV_BF16>(a, batch, groups, block_size, head_dim, stream); break;
  }
  return check_launch("attention_decode");
}

}  // extern "C"
