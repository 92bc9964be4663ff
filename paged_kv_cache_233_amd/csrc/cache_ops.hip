// Writes into the paged KV pools: the slot-mapped scatter of new tokens and
// whole-block copies for copy-on-write.
//
// Pool layout [num_blocks][num_kv_heads][16][head_dim]; slot = block*16 +
// offset ("vLLM: what PagedAttention turned into", section "The problem
// PagedAttention was actually solving", on the int64 slot mapping the worker
// keeps per scheduled token). Both kernels move 16-byte vectors: one token's
// row for one head is head_dim*elem bytes (128, 256 or 512), so every thread
// reads and writes aligned 16-byte pieces and a wave covers 1 KiB of
// consecutive bytes on both sides.
#include <algorithm>

#include "internal.h"

namespace {

// One thread per (token, tensor, head, 16-byte piece). `pieces` is the
// number of 16-byte pieces in one head row.
__global__ void __launch_bounds__(256)
reshape_and_cache_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                         const uint4* __restrict__ k_new, const uint4* __restrict__ v_new,
                         int64_t token_stride_vec, const int64_t* __restrict__ slots,
                         int64_t num_tokens, int64_t num_slots, int32_t num_kv_heads,
                         int32_t pieces) {
  // (32-bit index arithmetic: the grid holds fewer than 2^31 threads)
  const uint32_t per_tensor = (uint32_t)num_kv_heads * pieces;
  const uint32_t per_token = 2 * per_tensor;
  const uint32_t idx = blockIdx.x * blockDim.x + threadIdx.x;
  if ((int64_t)idx >= num_tokens * per_token) return;
  const uint32_t t = idx / per_token;
  uint32_t r = idx - t * per_token;
  const bool is_v = r >= per_tensor;
  if (is_v) r -= per_tensor;
  const int32_t h = (int32_t)(r / (uint32_t)pieces);
  const int32_t piece = (int32_t)(r - (uint32_t)h * pieces);
  // The source row is read before the slot is checked (it is in bounds
  // whatever the slot), so both loads take one memory round trip; the empty
  // asm keeps the compiler from sinking the row's load past the branch.
  const uint4 val =
      (is_v ? v_new : k_new)[t * token_stride_vec + (int64_t)h * pieces + piece];
  const int64_t slot = slots[t];
  __asm__ volatile("" ::"v"(val.x), "v"(val.y), "v"(val.z), "v"(val.w), "v"(slot));
  if (slot < 0 || slot >= num_slots) return;  // padding or out-of-range: no write
  const int64_t blk = slot >> 4;
  const int64_t off = slot & 15;
  uint4* dst = (is_v ? v_cache : k_cache) +
               ((blk * num_kv_heads + h) * 16 + off) * pieces + piece;
  *dst = val;
}

// One workgroup per copy pair; the block's K and V bytes are copied in
// 16-byte pieces.
__global__ void __launch_bounds__(256)
copy_blocks_kernel(uint4* __restrict__ k_cache, uint4* __restrict__ v_cache,
                   const int64_t* __restrict__ pairs, int32_t num_blocks, int32_t block_vecs) {
  const int64_t src = pairs[2 * (int64_t)blockIdx.x];
  const int64_t dst = pairs[2 * (int64_t)blockIdx.x + 1];
  if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
  const uint4* ks = k_cache + src * block_vecs;
  const uint4* vs = v_cache + src * block_vecs;
  uint4* kd = k_cache + dst * block_vecs;
  uint4* vd = v_cache + dst * block_vecs;
  for (int32_t i = threadIdx.x; i < block_vecs; i += blockDim.x) {
    uint4 a = ks[i];
    uint4 b = vs[i];
    kd[i] = a;
    vd[i] = b;
  }
}

// Plain copy of the per-step index arrays (slot mapping, lengths, block
// table) from pinned host memory into device memory: 16-byte pieces on a
// grid-stride loop, then the bytes of a ragged tail.
__global__ void __launch_bounds__(256)
stage_copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t vecs,
                  char* __restrict__ dst_tail, const char* __restrict__ src_tail, int32_t tail) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < vecs; i += stride)
    dst[i] = src[i];
  if (blockIdx.x == 0 && (int32_t)threadIdx.x < tail) dst_tail[threadIdx.x] = src_tail[threadIdx.x];
}

// Streaming read: workgroup b reads the b-th of gridDim.x equal contiguous
// slices with 16-byte non-temporal loads (as the decode reads its K/V tiles),
// four in flight per thread, and writes one word folded from what it read
// (so that the loads stay live).
__global__ void __launch_bounds__(256)
stream_read_kernel(const uint4* __restrict__ src, int64_t vecs, uint32_t* __restrict__ out) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const u32x4* v = reinterpret_cast<const u32x4*>(src);
  const int64_t per = (vecs + gridDim.x - 1) / gridDim.x;
  const int64_t b = per * blockIdx.x;
  const int64_t e = min(b + per, vecs);
  uint32_t acc = 0;
  for (int64_t i = b + threadIdx.x; i < e; i += 4 * 256) {
    u32x4 x[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t j = i + u * 256;
      x[u] = j < e ? __builtin_nontemporal_load(v + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) acc ^= x[u][0] ^ x[u][1] ^ x[u][2] ^ x[u][3];
  }
  // one word per workgroup: lane 0 of wave 0 keeps its own fold
  if (threadIdx.x == 0) out[blockIdx.x] = acc;
}

}  // namespace

namespace pkv {

hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t workgroups,
                              hipStream_t stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)workgroups), dim3(256), 0, stream,
                     (const uint4*)src, (int64_t)(bytes / 16), out);
  return hipGetLastError();
}

hipError_t launch_stage_copy(void* dst, const void* src, size_t bytes, hipStream_t stream) {
  const int64_t vecs = (int64_t)(bytes / 16);
  const int32_t tail = (int32_t)(bytes % 16);
  const int64_t grid = std::min<int64_t>(std::max<int64_t>((vecs + 255) / 256, 1), 1024);
  hipLaunchKernelGGL(stage_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream, (uint4*)dst,
                     (const uint4*)src, vecs, (char*)dst + vecs * 16,
                     (const char*)src + vecs * 16, tail);
  return hipGetLastError();
}


hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new,
                                    const void* v_new, int64_t token_stride,
                                    const int64_t* slots, int64_t num_tokens, int32_t num_blocks,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    hipStream_t stream) {
  const int elem = dtype == PKV_F32 ? 4 : 2;
  const int32_t pieces = head_dim * elem / 16;
  const int64_t total = num_tokens * 2 * num_kv_heads * pieces;
  const int64_t grid = (total + 255) / 256;
  hipLaunchKernelGGL(reshape_and_cache_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                     (uint4*)k_cache, (uint4*)v_cache, (const uint4*)k_new, (const uint4*)v_new,
                     token_stride * elem / 16, slots, num_tokens, (int64_t)num_blocks * 16,
                     num_kv_heads, pieces);
  return hipGetLastError();
}

hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n,
                              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                              int32_t dtype, hipStream_t stream) {
  const int elem = dtype == PKV_F32 ? 4 : 2;
  const int32_t block_vecs = num_kv_heads * 16 * head_dim * elem / 16;
  hipLaunchKernelGGL(copy_blocks_kernel, dim3(n), dim3(256), 0, stream, (uint4*)k_cache,
                     (uint4*)v_cache, pairs, num_blocks, block_vecs);
  return hipGetLastError();
}

}  // namespace pkv
