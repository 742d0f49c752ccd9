// Decode attention for 16/32-bit caches (fp32, fp16, bf16) and its C entry
// points.  The decode kernel and its launch geometry are shared with the
// 8-bit path (decode_common.h); this file supplies the format policy that
// loads and scores 16-bit or 32-bit rows.
#include "decode_common.h"
#include "prefix_common.h"

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
  static constexpr bool kDual = false;    // one chunk stream per work-group
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
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) ||
      !pkv::aligned16(k_new) || !pkv::aligned16(v_new))
    return pkv::fail(PKV_ERR_INVALID, "%s: q, out, pools and new rows must be 16-byte aligned", what);
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

// Both grouped entry points; k_new != nullptr selects the variant that first
// stores each sequence's new row at its position L - 1 (never a prefix
// position: a tile's prefix ends before every member's last block).
int decode_grouped(void* out, const void* q, const void* k_new, const void* v_new, const void* k_cache,
                   const void* v_cache, const int32_t* block_tables, int32_t max_blocks_per_seq,
                   const int32_t* seq_lens, int32_t max_seq_len, int32_t batch, int32_t num_heads, int32_t head_dim,
                   int32_t block_size, int32_t num_blocks, float scale, pkv_dtype dtype,
                   const int32_t* seq_prefix_blocks, const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                   void* workspace, size_t workspace_bytes, hipStream_t stream, const char* what) {
  const pkv::CallEvents timing = pkv::take_call_events();  // consumed by this call, whatever its outcome
  const int sz = check_grouped_sizes(what, batch, num_heads, head_dim, block_size, num_blocks, max_blocks_per_seq,
                                     max_seq_len, num_tiles);
  if (sz != PKV_OK) return sz;
  if (dtype != PKV_F16 && dtype != PKV_BF16)
    return pkv::fail(PKV_ERR_INVALID, "%s: the cache must be f16 or bf16 (dtype %d)", what, static_cast<int>(dtype));
  const int st = check_decode_scalars(scale, num_work_groups);
  if (st != PKV_OK) return st;
  if (batch == 0) return PKV_OK;
  if (!seq_prefix_blocks || (num_tiles > 0 && !tiles))
    return pkv::fail(PKV_ERR_INVALID, "%s: null prefix arrays", what);
  if (!pkv::aligned16(q) || !pkv::aligned16(out) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache) ||
      !pkv::aligned16(k_new) || !pkv::aligned16(v_new))
    return pkv::fail(PKV_ERR_INVALID, "%s: q, out, pools and new rows must be 16-byte aligned", what);
  DecodeArgs a;
  const int wg = prepare_decode(a, q, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens, max_seq_len,
                                batch, num_heads, head_dim, block_size, num_blocks, scale, dtype, num_work_groups,
                                workspace, workspace_bytes, out, /*grouped=*/true);
  if (wg <= 0) return wg;
  a.k_new = k_new;
  a.v_new = v_new;
  const int64_t row = static_cast<int64_t>(num_heads) * head_dim * dtype_bytes(dtype);
  return run_grouped(
      a, wg, out, q, block_tables, max_blocks_per_seq, seq_lens, batch, num_heads, head_dim, dtype, row,
      seq_prefix_blocks, num_tiles, workspace, workspace_bytes, timing, what,
      [&](const DecodeArgs& pa, hipEvent_t start) {
        if (dtype == PKV_F16) {
          if (head_dim == 64) launch_prefix<PrefixDense<PKV_F16>, 64>(pa, block_size, tiles, num_tiles, stream, start);
          else launch_prefix<PrefixDense<PKV_F16>, 128>(pa, block_size, tiles, num_tiles, stream, start);
        } else {
          if (head_dim == 64) launch_prefix<PrefixDense<PKV_BF16>, 64>(pa, block_size, tiles, num_tiles, stream, start);
          else launch_prefix<PrefixDense<PKV_BF16>, 128>(pa, block_size, tiles, num_tiles, stream, start);
        }
      },
      [&](const DecodeArgs& s, const pkv::CallEvents& tm) {
        if (k_new != nullptr) {
          if (dtype == PKV_F16) launch_decode_m<DenseKV<PKV_F16>, kAppend>(s, wg, block_size, head_dim, stream, tm);
          else launch_decode_m<DenseKV<PKV_BF16>, kAppend>(s, wg, block_size, head_dim, stream, tm);
        } else {
          if (dtype == PKV_F16) launch_decode_m<DenseKV<PKV_F16>, kPlain>(s, wg, block_size, head_dim, stream, tm);
          else launch_decode_m<DenseKV<PKV_BF16>, kPlain>(s, wg, block_size, head_dim, stream, tm);
        }
      },
      [&](const DecodeArgs& s, const pkv::CallEvents& tm, int32_t units) {
        using F16 = DenseKV<PKV_F16>;
        using B16 = DenseKV<PKV_BF16>;
        if (k_new != nullptr) {
          if (dtype == PKV_F16)
            return launch_fused<F16, PrefixDense<PKV_F16>, kAppend>(s, block_size, head_dim, tiles, units, stream, tm);
          else
            return launch_fused<B16, PrefixDense<PKV_BF16>, kAppend>(s, block_size, head_dim, tiles, units, stream, tm);
        } else {
          if (dtype == PKV_F16)
            return launch_fused<F16, PrefixDense<PKV_F16>, kPlain>(s, block_size, head_dim, tiles, units, stream, tm);
          else
            return launch_fused<B16, PrefixDense<PKV_BF16>, kPlain>(s, block_size, head_dim, tiles, units, stream, tm);
        }
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
      (dtype != PKV_F16 && dtype != PKV_BF16 && !is_8bit(dtype)))
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
  return decode_grouped(out, q, nullptr, nullptr, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                        max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                        seq_prefix_blocks, tiles, num_tiles, num_work_groups, workspace, workspace_bytes, stream,
                        "attention_decode_grouped");
}

PKV_API int pkv_append_attention_decode_grouped(void* out, const void* q, const void* k_new, const void* v_new,
                                                void* k_cache, void* v_cache, const int32_t* block_tables,
                                                int32_t max_blocks_per_seq, const int32_t* seq_lens,
                                                int32_t max_seq_len, int32_t batch, int32_t num_heads,
                                                int32_t head_dim, int32_t block_size, int32_t num_blocks, float scale,
                                                pkv_dtype dtype, const int32_t* seq_prefix_blocks,
                                                const int32_t* tiles, int32_t num_tiles, int32_t num_work_groups,
                                                void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (batch > 0 && (!k_new || !v_new)) {
    pkv::take_call_events();  // a pending timing request belongs to this call
    return pkv::fail(PKV_ERR_INVALID, "append_attention_decode_grouped: null new rows");
  }
  return decode_grouped(out, q, k_new, v_new, k_cache, v_cache, block_tables, max_blocks_per_seq, seq_lens,
                        max_seq_len, batch, num_heads, head_dim, block_size, num_blocks, scale, dtype,
                        seq_prefix_blocks, tiles, num_tiles, num_work_groups, workspace, workspace_bytes, stream,
                        "append_attention_decode_grouped");
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
