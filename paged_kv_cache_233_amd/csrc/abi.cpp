// C entry points of the device kernels: argument checks on the host, then an
// asynchronous launch on the caller's stream.
#include <cstdio>
#include <cstring>
#include <vector>

#include "internal.h"

namespace pkv {

int hip_fail(hipError_t e, const char* what) {
  return fail(PKV_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

}  // namespace pkv

namespace {

using pkv::fail;

int check_shape(int32_t num_kv_heads, int32_t head_dim, int32_t dtype) {
  if (dtype != PKV_F32 && dtype != PKV_BF16) return fail(PKV_ERR_UNSUPPORTED, "dtype %d not supported", dtype);
  if (head_dim != 64 && head_dim != 128)
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", head_dim);
  if (num_kv_heads <= 0) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads must be > 0");
  return PKV_OK;
}

int check_heads(int32_t num_q_heads, int32_t num_kv_heads) {
  if (num_q_heads <= 0 || num_kv_heads <= 0 || num_q_heads % num_kv_heads != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads %d must be a positive multiple of num_kv_heads %d",
                num_q_heads, num_kv_heads);
  if (num_q_heads / num_kv_heads > 16)
    return fail(PKV_ERR_UNSUPPORTED, "at most 16 query heads per KV head (got %d)",
                num_q_heads / num_kv_heads);
  return PKV_OK;
}

// Debug mode of pkv_reshape_and_cache: waits for the stream, reads the slot
// mapping back (device or pinned host memory) and checks it on the host
// before launching. Not for graph capture.
int debug_check_slots(const int64_t* slot_mapping, int64_t num_tokens, int32_t num_blocks,
                      hipStream_t stream) {
  std::vector<int64_t> host((size_t)num_tokens);
  hipError_t err = hipStreamSynchronize(stream);
  if (err == hipSuccess)
    err = hipMemcpy(host.data(), slot_mapping, (size_t)num_tokens * sizeof(int64_t), hipMemcpyDefault);
  if (err != hipSuccess) return pkv::hip_fail(err, "reshape_and_cache debug check (reading the slots)");
  return pkv::check_slot_mapping(host.data(), num_tokens, num_blocks);
}

}  // namespace

extern "C" {

int pkv_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new, const void* v_new,
                          int64_t new_token_stride, const int64_t* slot_mapping,
                          int64_t num_tokens, int32_t num_blocks, int32_t num_kv_heads,
                          int32_t head_dim, int32_t dtype, void* stream) {
  pkv::clear_error();
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (num_tokens < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_tokens == 0) return PKV_OK;
  if (!k_cache || !v_cache || !k_new || !v_new || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (new_token_stride < (int64_t)num_kv_heads * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "new_token_stride %lld < num_kv_heads*head_dim",
                (long long)new_token_stride);
  const int64_t elem = dtype == PKV_F32 ? 4 : 2;
  // one thread per 16-byte piece of K and V: the grid must stay below 2^31 threads
  if (num_tokens * 2 * num_kv_heads * (head_dim * elem / 16) > INT32_MAX - 255)
    return fail(PKV_ERR_INVALID_ARG, "too many tokens for one launch");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache | (uintptr_t)k_new | (uintptr_t)v_new) % 16 != 0 ||
      (new_token_stride * elem) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pools, new K/V and the token stride must be 16-byte aligned");
  if (pkv::debug_checks()) {
    if (int e = debug_check_slots(slot_mapping, num_tokens, num_blocks, (hipStream_t)stream)) return e;
  }
  hipError_t err = pkv::launch_reshape_and_cache(k_cache, v_cache, k_new, v_new, new_token_stride,
                                                 slot_mapping, num_tokens, num_blocks, num_kv_heads,
                                                 head_dim, dtype, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "reshape_and_cache launch");
}

int pkv_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n,
                    int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                    void* stream) {
  pkv::clear_error();
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (n < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (n == 0) return PKV_OK;
  if (!k_cache || !v_cache || !pairs) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (((uintptr_t)k_cache | (uintptr_t)v_cache) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "pools must be 16-byte aligned");
  hipError_t err = pkv::launch_copy_blocks(k_cache, v_cache, pairs, n, num_blocks, num_kv_heads,
                                           head_dim, dtype, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "copy_blocks launch");
}

int pkv_stage_copy(void* dst, const void* src, size_t bytes, void* stream) {
  pkv::clear_error();
  if (bytes == 0) return PKV_OK;
  if (!dst || !src) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if (((uintptr_t)dst | (uintptr_t)src) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "dst and src must be 16-byte aligned");
  if ((uintptr_t)dst < (uintptr_t)src + bytes && (uintptr_t)src < (uintptr_t)dst + bytes)
    return fail(PKV_ERR_INVALID_ARG, "dst and src overlap");
  hipError_t err = pkv::launch_stage_copy(dst, src, bytes, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "stage_copy launch");
}

int pkv_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t workgroups, void* stream) {
  pkv::clear_error();
  if (bytes == 0) return PKV_OK;
  if (!src || !out) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((uintptr_t)src % 16 != 0 || bytes % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "src and bytes must be multiples of 16");
  if (workgroups < 1 || workgroups > (1 << 20))
    return fail(PKV_ERR_INVALID_ARG, "workgroups %d outside [1, 2^20]", workgroups);
  hipError_t err = pkv::launch_stream_read(src, bytes, out, workgroups, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "stream_read launch");
}

int pkv_decode_workspace_size(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim, size_t* out) {
  pkv::clear_error();
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "num_seqs < 0");
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (pkv::decode_num_waves() <= 0) return fail(PKV_ERR_HIP, "no HIP device");
  *out = pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
  return PKV_OK;
}

int pkv_decode_set_waves_per_cu(int32_t per_cu) {
  pkv::clear_error();
  if (per_cu < 0 || per_cu > 32) return fail(PKV_ERR_INVALID_ARG, "waves per CU %d outside [0, 32]", per_cu);
  pkv::decode_set_waves_per_cu(per_cu);
  return PKV_OK;
}

namespace {

// The current token's K/V for the append mode of the decode (nullptr: none).
struct NewTokens {
  const void* k_new;
  const void* v_new;
  int64_t stride;
};

int decode_entry(void* out, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* block_table, const int32_t* context_lens, int32_t num_seqs,
                 int32_t num_blocks, int32_t max_blocks_per_seq, int32_t num_q_heads,
                 int32_t num_kv_heads, int32_t head_dim, float scale, int32_t dtype,
                 void* workspace, size_t workspace_bytes, void* stream, int phases,
                 const NewTokens* append = nullptr) {
  pkv::clear_error();
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (num_seqs < 0 || num_blocks <= 0 || max_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || (!block_table && max_blocks_per_seq > 0))
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  // (the decode partitions blocks plus a few units per sequence in int32)
  if ((int64_t)num_seqs * num_kv_heads * ((int64_t)max_blocks_per_seq + 16) > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs*num_kv_heads*max_blocks_per_seq too large");
  if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache |
       (uintptr_t)workspace) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "q, out, pools and workspace must be 16-byte aligned");
  if (pkv::decode_num_waves() <= 0) return fail(PKV_ERR_HIP, "no HIP device");
  size_t need = pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
  if (!workspace || workspace_bytes < need)
    return fail(PKV_ERR_WORKSPACE, "decode needs %zu workspace bytes, got %zu", need,
                workspace ? workspace_bytes : (size_t)0);
  pkv::DecodeArgs a{out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                    max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                    workspace};
  if (append != nullptr) {
    if (!append->k_new || !append->v_new) return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
    if (append->stride < (int64_t)num_kv_heads * head_dim)
      return fail(PKV_ERR_INVALID_ARG, "new_token_stride %lld < num_kv_heads*head_dim",
                  (long long)append->stride);
    const int64_t elem = dtype == PKV_F32 ? 4 : 2;
    if (((uintptr_t)append->k_new | (uintptr_t)append->v_new) % 16 != 0 ||
        (append->stride * elem) % 16 != 0)
      return fail(PKV_ERR_INVALID_ARG, "new K/V and the token stride must be 16-byte aligned");
    a.k_new = append->k_new;
    a.v_new = append->v_new;
    a.new_token_stride = append->stride;
  }
  hipError_t err = pkv::launch_decode(a, phases, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "decode launch");
}

}  // namespace

int pkv_paged_attention_decode(void* out, const void* q, const void* k_cache, const void* v_cache,
                               const int32_t* block_table, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_blocks, int32_t max_blocks_per_seq,
                               int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                               float scale, int32_t dtype, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      workspace, workspace_bytes, stream, 3);
}

int pkv_paged_attention_decode_split(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float scale, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      workspace, workspace_bytes, stream, 1);
}

int pkv_paged_attention_decode_merge(void* out, const void* q, const void* k_cache,
                                     const void* v_cache, const int32_t* block_table,
                                     const int32_t* context_lens, int32_t num_seqs,
                                     int32_t num_blocks, int32_t max_blocks_per_seq,
                                     int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                     float scale, int32_t dtype, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      workspace, workspace_bytes, stream, 2);
}

int pkv_paged_attention_decode_append(void* out, const void* q, const void* k_new,
                                      const void* v_new, int64_t new_token_stride, void* k_cache,
                                      void* v_cache, const int32_t* block_table,
                                      const int32_t* context_lens, int32_t num_seqs,
                                      int32_t num_blocks, int32_t max_blocks_per_seq,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float scale, int32_t dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  const NewTokens nt{k_new, v_new, new_token_stride};
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      workspace, workspace_bytes, stream, 3, &nt);
}

int pkv_paged_attention_decode_append_split(void* out, const void* q, const void* k_new,
                                            const void* v_new, int64_t new_token_stride,
                                            void* k_cache, void* v_cache,
                                            const int32_t* block_table,
                                            const int32_t* context_lens, int32_t num_seqs,
                                            int32_t num_blocks, int32_t max_blocks_per_seq,
                                            int32_t num_q_heads, int32_t num_kv_heads,
                                            int32_t head_dim, float scale, int32_t dtype,
                                            void* workspace, size_t workspace_bytes,
                                            void* stream) {
  const NewTokens nt{k_new, v_new, new_token_stride};
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      workspace, workspace_bytes, stream, 1, &nt);
}

int pkv_paged_attention_decode_noalloc(void* out, const void* q, const void* k_cache,
                                       const void* v_cache, const int32_t* block_table,
                                       const int32_t* context_lens, int32_t num_seqs,
                                       int32_t num_blocks, int32_t max_blocks_per_seq,
                                       int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                       float scale, int32_t dtype, void* stream) {
  pkv::clear_error();
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (num_seqs < 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs == 0) return PKV_OK;
  if (pkv::decode_num_waves() <= 0) return fail(PKV_ERR_HIP, "no HIP device");
  const size_t need = pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim);
  if (need > (size_t)PKV_DECODE_SCRATCH_BYTES)
    return fail(PKV_ERR_WORKSPACE,
                "the no-alloc decode's scratch holds %zu bytes; these sizes need %zu (use "
                "pkv_paged_attention_decode with a workspace)",
                (size_t)PKV_DECODE_SCRATCH_BYTES, need);
  void* scratch = nullptr;
  hipError_t err = pkv::decode_scratch(&scratch);
  if (err != hipSuccess) return pkv::hip_fail(err, "no-alloc decode scratch lookup");
  return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                      max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                      scratch, (size_t)PKV_DECODE_SCRATCH_BYTES, stream, 3);
}

// Workspace of the shared-prefix decode: the decode workspace; the states
// of the sequences one wave holds whole (num_seqs x num_kv_heads x G x
// (head_dim + 4) floats); then the prefix states (parts x num_seqs x
// num_q_heads x (head_dim + 4) floats), which the merge folds first.
struct SharedLayout {
  size_t decode, whole, state, total;
  int32_t parts;
};
static SharedLayout shared_prefix_layout(int32_t num_seqs, int32_t num_q_heads,
                                         int32_t num_kv_heads, int32_t head_dim,
                                         int32_t prefix_blocks) {
  SharedLayout l;
  l.decode = (pkv::decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim) + 255) /
             256 * 256;
  l.whole = ((size_t)num_seqs * num_q_heads * (head_dim + 4) * 4 + 255) / 256 * 256;
  l.parts = pkv::decode_prefix_parts(num_seqs, num_q_heads, num_kv_heads, prefix_blocks);
  l.state = (size_t)l.parts * num_seqs * num_q_heads * (head_dim + 4) * 4;
  l.total = l.decode + l.whole + l.state;
  return l;
}

int pkv_decode_shared_prefix_workspace_size(int32_t num_seqs, int32_t num_q_heads,
                                            int32_t num_kv_heads, int32_t head_dim,
                                            int32_t prefix_blocks, size_t* out) {
  pkv::clear_error();
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  if (num_seqs < 0 || prefix_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  if (pkv::decode_num_waves() <= 0) return fail(PKV_ERR_HIP, "no HIP device");
  *out = shared_prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim, prefix_blocks).total;
  return PKV_OK;
}

int pkv_paged_attention_decode_shared_prefix(void* out, const void* q, const void* k_cache,
                                             const void* v_cache, const int32_t* block_table,
                                             const int32_t* context_lens, int32_t num_seqs,
                                             int32_t num_blocks, int32_t max_blocks_per_seq,
                                             int32_t prefix_blocks, int32_t num_q_heads,
                                             int32_t num_kv_heads, int32_t head_dim, float scale,
                                             int32_t dtype, void* workspace,
                                             size_t workspace_bytes, void* stream) {
  pkv::clear_error();
  if (prefix_blocks < 0 || prefix_blocks > max_blocks_per_seq)
    return fail(PKV_ERR_INVALID_ARG, "prefix_blocks %d outside [0, max_blocks_per_seq %d]",
                prefix_blocks, max_blocks_per_seq);
  // fp32 (no bf16 MFMA prefix phase) and an empty prefix: the ordinary decode
  if (prefix_blocks == 0 || dtype == PKV_F32)
    return decode_entry(out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                        max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                        workspace, workspace_bytes, stream, 3);
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (num_seqs < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_seqs == 0) return PKV_OK;
  if (!out || !q || !k_cache || !v_cache || !context_lens || !block_table)
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  // (the decode partitions blocks plus a few units per sequence in int32)
  if ((int64_t)num_seqs * num_kv_heads * ((int64_t)max_blocks_per_seq + 16) > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "num_seqs*num_kv_heads*max_blocks_per_seq too large");
  if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache |
       (uintptr_t)workspace) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "q, out, pools and workspace must be 16-byte aligned");
  if (pkv::decode_num_waves() <= 0) return fail(PKV_ERR_HIP, "no HIP device");
  const SharedLayout l = shared_prefix_layout(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                              prefix_blocks);
  if (!workspace || workspace_bytes < l.total)
    return fail(PKV_ERR_WORKSPACE, "shared-prefix decode needs %zu workspace bytes, got %zu",
                l.total, workspace ? workspace_bytes : (size_t)0);
  char* ws = reinterpret_cast<char*>(workspace);
  float* whole = reinterpret_cast<float*>(ws + l.decode);
  float* state = reinterpret_cast<float*>(ws + l.decode + l.whole);
  pkv::DecodeArgs a{out, q, k_cache, v_cache, block_table, context_lens, num_seqs, num_blocks,
                    max_blocks_per_seq, num_q_heads, num_kv_heads, head_dim, scale, dtype,
                    workspace};
  const hipError_t err = pkv::launch_decode_shared_prefix(a, prefix_blocks, state, l.parts,
                                                          (hipStream_t)stream, whole);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "shared-prefix decode launch");
}

int pkv_prefill_workspace_size(int32_t num_chunks, int32_t total_q, int32_t num_q_heads,
                               int32_t num_kv_heads, int32_t head_dim, int32_t max_q_len,
                               int32_t max_context_len, size_t* out) {
  pkv::clear_error();
  if (!out) return fail(PKV_ERR_INVALID_ARG, "out is NULL");
  if (num_chunks < 0 || total_q < 0 || max_q_len < 0 || max_context_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (head_dim != 64 && head_dim != 128) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d", head_dim);
  (void)total_q;
  (void)max_context_len;
  *out = pkv::prefill_workspace_bytes(num_chunks, num_q_heads, num_kv_heads, head_dim, max_q_len);
  return PKV_OK;
}

int pkv_paged_attention_prefill_chunk(void* out, const void* q, const int32_t* cu_q_lens,
                                      const int32_t* context_lens, const int32_t* block_table,
                                      const void* k_cache, const void* v_cache,
                                      int32_t num_chunks, int32_t total_q, int32_t num_blocks,
                                      int32_t max_blocks_per_seq, int32_t max_q_len,
                                      int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                      float scale, int32_t dtype, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  pkv::clear_error();
  if (int e = check_shape(num_kv_heads, head_dim, dtype)) return e;
  if (int e = check_heads(num_q_heads, num_kv_heads)) return e;
  if (num_chunks < 0 || total_q < 0 || num_blocks <= 0 || max_blocks_per_seq < 0 || max_q_len < 0)
    return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (num_chunks == 0 || max_q_len == 0 || total_q == 0) return PKV_OK;
  if (((uintptr_t)out | (uintptr_t)q | (uintptr_t)k_cache | (uintptr_t)v_cache) % 16 != 0)
    return fail(PKV_ERR_INVALID_ARG, "q, out and pools must be 16-byte aligned");
  if (!out || !q || !cu_q_lens || !context_lens || !k_cache || !v_cache ||
      (!block_table && max_blocks_per_seq > 0))
    return fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  if ((int64_t)num_chunks * num_kv_heads * ((max_q_len + 15) / 16) > INT32_MAX)
    return fail(PKV_ERR_INVALID_ARG, "grid too large");
  if (workspace != nullptr && dtype == PKV_BF16) {
    const size_t need =
        pkv::prefill_workspace_bytes(num_chunks, num_q_heads, num_kv_heads, head_dim, max_q_len);
    if (workspace_bytes < need)
      return fail(PKV_ERR_WORKSPACE, "prefill workspace %zu bytes, need %zu", workspace_bytes, need);
    if ((uintptr_t)workspace % 16 != 0)
      return fail(PKV_ERR_INVALID_ARG, "prefill workspace must be 16-byte aligned");
  }
  pkv::PrefillArgs a{out, q, cu_q_lens, context_lens, block_table, k_cache, v_cache, num_chunks,
                     total_q, num_blocks, max_blocks_per_seq, max_q_len, num_q_heads,
                     num_kv_heads, head_dim, scale, dtype, workspace, workspace_bytes};
  hipError_t err = pkv::launch_prefill(a, (hipStream_t)stream);
  return err == hipSuccess ? PKV_OK : pkv::hip_fail(err, "prefill launch");
}

}  // extern "C"
