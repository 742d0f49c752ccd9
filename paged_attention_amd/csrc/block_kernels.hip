// Bit-copy kernels over K/V pools and their C entry points: scatter of new
// rows into their slots (pkv_append), whole-block copies inside a pool for
// copy-on-write (pkv_copy_blocks), and whole-block swaps between a device pool
// and a pinned host pool for preemption (pkv_swap_blocks).
#include "decode_common.h"

namespace {

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

// ---- block swap between two pools (device <-> pinned host) ----------------

constexpr int kSwapPools = 64;  // pool pointers carried per launch (K and V of 32 layers)
constexpr int kSwapUnroll = 4;  // 16-byte moves in flight per thread

struct SwapPtrs {
  const Vec16* src[kSwapPools];
  Vec16* dst[kSwapPools];
};

// One work-group per (pair, pool): block `src` of pool y of the source side
// is copied to block `dst` of pool y of the destination side.  Either side
// may be pinned host memory, which the GPU reads or writes over the host
// link; each thread keeps kSwapUnroll 16-byte moves in flight to cover its
// latency.  Ids outside a side's pool are skipped.
__global__ void __launch_bounds__(256) swap_blocks_kernel(SwapPtrs p, const int32_t* __restrict__ pairs,
                                                          int32_t src_blocks, int32_t dst_blocks,
                                                          int64_t vec_per_block) {
  const int32_t src = pairs[2 * blockIdx.x];
  const int32_t dst = pairs[2 * blockIdx.x + 1];
  if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
  const Vec16* from = p.src[blockIdx.y] + static_cast<int64_t>(src) * vec_per_block;
  Vec16* to = p.dst[blockIdx.y] + static_cast<int64_t>(dst) * vec_per_block;
  const int64_t step = static_cast<int64_t>(blockDim.x) * kSwapUnroll;
  for (int64_t i0 = threadIdx.x; i0 < vec_per_block; i0 += step) {
    Vec16 v[kSwapUnroll];
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < vec_per_block) v[u] = from[i];
    }
#pragma unroll
    for (int u = 0; u < kSwapUnroll; ++u) {
      const int64_t i = i0 + static_cast<int64_t>(u) * blockDim.x;
      if (i < vec_per_block) to[i] = v[u];
    }
  }
}

// A pool pointer the GPU may use: device memory, or host memory pinned with
// hipHostMalloc (mapped into the device's address space).  Pageable host
// memory is refused here, before any launch, instead of faulting the GPU.
bool gpu_accessible(const void* p) {
  hipPointerAttribute_t attr;
  if (hipPointerGetAttributes(&attr, p) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error the query leaves for unknown pointers
    return false;
  }
  return attr.type == hipMemoryTypeDevice || (attr.type == hipMemoryTypeHost && attr.devicePointer != nullptr) ||
         attr.type == hipMemoryTypeManaged;
}

bool supported_dense(int32_t head_dim, int32_t block_size, pkv_dtype dtype) {
  return supported_geometry(head_dim, block_size) && is_16_32(dtype);
}

}  // namespace

extern "C" {

PKV_API int pkv_append(const void* k_new, const void* v_new, int32_t num_tokens, const int64_t* slot_mapping,
                       void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t num_heads,
                       int32_t head_dim, pkv_dtype dtype, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_heads <= 0 || !supported_dense(head_dim, block_size, dtype))
    return pkv::fail(PKV_ERR_INVALID, "append: unsupported sizes (tokens %d, blocks %d, heads %d, head_dim %d, "
                                      "block %d, dtype %d)", num_tokens, num_blocks, num_heads, head_dim, block_size,
                     static_cast<int>(dtype));
  if (num_tokens == 0) return PKV_OK;
  if (!k_new || !v_new || !slot_mapping || !k_cache || !v_cache) return pkv::fail(PKV_ERR_INVALID, "append: null pointer");
  if (!pkv::aligned16(k_new) || !pkv::aligned16(v_new) || !pkv::aligned16(k_cache) || !pkv::aligned16(v_cache))
    return pkv::fail(PKV_ERR_INVALID, "append: rows and pools must be 16-byte aligned");
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
  for (int32_t l = 0; l < num_layers; ++l)  // every pool before any launch: nothing is copied on an error
    if (!k_caches[l] || !v_caches[l] || !pkv::aligned16(k_caches[l]) || !pkv::aligned16(v_caches[l]))
      return pkv::fail(PKV_ERR_INVALID, "copy_blocks: layer %d's pools must be non-null and 16-byte aligned", l);
  for (int32_t l0 = 0; l0 < num_layers; l0 += kCopyLayers) {
    const int32_t nl = num_layers - l0 < kCopyLayers ? num_layers - l0 : kCopyLayers;
    LayerPtrs ptrs{};
    for (int32_t i = 0; i < nl; ++i) {
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

PKV_API int pkv_swap_blocks(void* const* dst_pools, const void* const* src_pools, int32_t num_pools,
                            const int32_t* pairs, int32_t n_pairs, int32_t src_num_blocks, int32_t dst_num_blocks,
                            size_t bytes_per_block, hipStream_t stream) {
  if (num_pools < 0 || n_pairs < 0 || src_num_blocks <= 0 || dst_num_blocks <= 0 || bytes_per_block == 0 ||
      bytes_per_block % 16 != 0)
    return pkv::fail(PKV_ERR_INVALID, "swap_blocks: bad sizes (pools %d, pairs %d, blocks %d/%d, bytes %zu)",
                     num_pools, n_pairs, src_num_blocks, dst_num_blocks, bytes_per_block);
  if (n_pairs == 0 || num_pools == 0) return PKV_OK;
  if (!dst_pools || !src_pools || !pairs) return pkv::fail(PKV_ERR_INVALID, "swap_blocks: null pointer");
  if (n_pairs > 0x7fffffff / 2) return pkv::fail(PKV_ERR_INVALID, "swap_blocks: too many pairs");
  if (!gpu_accessible(pairs))
    return pkv::fail(PKV_ERR_INVALID, "swap_blocks: pairs must be device or pinned host memory");
  for (int32_t i = 0; i < num_pools; ++i) {
    if (!dst_pools[i] || !src_pools[i]) return pkv::fail(PKV_ERR_INVALID, "swap_blocks: null pool %d", i);
    if (reinterpret_cast<uintptr_t>(dst_pools[i]) % 16 || reinterpret_cast<uintptr_t>(src_pools[i]) % 16)
      return pkv::fail(PKV_ERR_INVALID, "swap_blocks: pool %d is not 16-byte aligned", i);
    if (!gpu_accessible(dst_pools[i]) || !gpu_accessible(src_pools[i]))
      return pkv::fail(PKV_ERR_INVALID, "swap_blocks: pool %d is neither device nor pinned host memory", i);
  }
  for (int32_t p0 = 0; p0 < num_pools; p0 += kSwapPools) {
    const int32_t np = num_pools - p0 < kSwapPools ? num_pools - p0 : kSwapPools;
    SwapPtrs ptrs{};
    for (int32_t i = 0; i < np; ++i) {
      ptrs.src[i] = static_cast<const Vec16*>(src_pools[p0 + i]);
      ptrs.dst[i] = static_cast<Vec16*>(dst_pools[p0 + i]);
    }
    hipLaunchKernelGGL(swap_blocks_kernel, dim3(n_pairs, np), dim3(256), 0, stream, ptrs, pairs, src_num_blocks,
                       dst_num_blocks, static_cast<int64_t>(bytes_per_block / 16));
    const int st = check_launch("swap_blocks");
    if (st != PKV_OK) return st;
  }
  return PKV_OK;
}

}  // extern "C"
