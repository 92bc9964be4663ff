// Internal declarations of the translation units of libpkv that launch
// kernels (the host-only ones include host.h alone).
#pragma once

#include <hip/hip_runtime.h>

#include <string>

#include "host.h"

namespace pkv {

// Maps a HIP error from a launch to PKV_ERR_HIP with a message.
int hip_fail(hipError_t e, const char* what);

// ---------------------------------------------------------------- launchers
// Each returns hipSuccess or the launch error; arguments were validated by
// the caller.
hipError_t launch_reshape_and_cache(void* k_cache, void* v_cache, const void* k_new,
                                    const void* v_new, int64_t token_stride,
                                    const int64_t* slots, int64_t num_tokens, int32_t num_blocks,
                                    int32_t num_kv_heads, int32_t head_dim, int32_t dtype,
                                    hipStream_t stream);

hipError_t launch_stage_copy(void* dst, const void* src, size_t bytes, hipStream_t stream);
// Plain streaming read of `bytes` (a multiple of 16) by `workgroups`
// workgroups; one folded word per workgroup to out[workgroups].
hipError_t launch_stream_read(const void* src, size_t bytes, uint32_t* out, int32_t workgroups,
                              hipStream_t stream);
hipError_t launch_copy_blocks(void* k_cache, void* v_cache, const int64_t* pairs, int32_t n,
                              int32_t num_blocks, int32_t num_kv_heads, int32_t head_dim,
                              int32_t dtype, hipStream_t stream);

struct DecodeArgs {
  void* out;
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;
  int32_t dtype;
  void* workspace;
  // Append mode: each sequence's current token (k_new/v_new rows, tokens
  // new_token_stride elements apart) is written into the cache by the
  // split-KV kernel itself before it attends; nullptr = plain decode.
  const void* k_new = nullptr;
  const void* v_new = nullptr;
  int64_t new_token_stride = 0;
};

// Number of waves the split-KV decode kernel is launched with on the current
// device (a multiple of 8), and the workspace it needs.
int decode_num_waves();
// Waves per CU of the split-KV decode (0 = the default); takes effect on the
// next call that sizes or launches a decode.
void decode_set_waves_per_cu(int per_cu);
size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim);
// Device address of the current device's copy of the no-alloc decode's
// scratch array (PKV_DECODE_SCRATCH_BYTES bytes), looked up once per device.
hipError_t decode_scratch(void** out);
// phases: 1 = split-KV kernel, 2 = merge kernel, 3 = both.
hipError_t launch_decode(const DecodeArgs& a, int phases, hipStream_t stream);
// Shared-prefix decode (bf16): one split-KV launch whose extra workgroups
// attend the first `skip_blocks` blocks of table row 0 (common to every
// sequence) in `parts` position ranges for all sequences at once, leaving
// prefix_state[part][row][head_dim + 4] (unnormalised O, max in log2 units,
// sum, two floats of padding; row = sequence * num_q_heads + head), while
// its decode waves attend each sequence's blocks from skip_blocks on; then
// the merge kernel folds the prefix states and the sequence's own states.
// whole_states: num_seqs x num_kv_heads states of G x (head_dim + 4)
// floats, where the split kernel leaves the state of a sequence whose
// blocks one wave holds whole. 1 <= parts <= skip_blocks.
int decode_prefix_parts(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t prefix_blocks);
hipError_t launch_decode_shared_prefix(const DecodeArgs& a, int32_t skip_blocks,
                                       float* prefix_state, int32_t parts, hipStream_t stream,
                                       float* whole_states);

struct PrefillArgs {
  void* out;
  const void* q;
  const int32_t* cu_q_lens;
  const int32_t* context_lens;
  const int32_t* block_table;
  const void* k_cache;
  const void* v_cache;
  int32_t num_chunks;
  int32_t total_q;
  int32_t num_blocks;
  int32_t max_blocks_per_seq;
  int32_t max_q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  float scale;
  int32_t dtype;
  void* workspace;          // optional: the position parts' softmax states
  size_t workspace_bytes;
};

// Workspace bytes the bf16 prefill uses to cut row blocks into position
// parts on the current device (0: this shape runs without).
size_t prefill_workspace_bytes(int32_t num_chunks, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_q_len);
hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream);

}  // namespace pkv
