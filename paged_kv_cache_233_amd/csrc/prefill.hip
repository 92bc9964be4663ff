// Chunked-prefill attention over paged KV for gfx950: a chunk of consecutive
// query tokens of one sequence attends causally to the sequence's cached
// tokens plus the chunk's own ("(2) vLLM Internals: From PagedAttention to
// Removing PagedAttention", section "2. Continuous Batching"; "vLLM: what
// PagedAttention turned into", section "The scheduler, and what it has to
// balance now"). Keys and values are gathered through the block table inside
// the kernel.
//
// Work split: one workgroup of 4 waves per (chunk, KV head, block of query
// tokens). A wave owns NG groups of 16 MFMA columns; a group is 16/G
// consecutive query tokens x the G query heads of the KV head (grouped
// query attention), so every K/V tile a wave loads serves 16*NG query rows.
// The wave walks the K/V blocks from position 0 up to its last query's
// causal limit, running the MFMA tile step of tile_attn.h with a per-column
// limit (query position p sees positions 0..p); only blocks that reach past
// the wave's first query position need masking.
#include <cstdlib>

#include "internal.h"
#include "tile_attn.h"

namespace {

using namespace pkv::tile;

constexpr int kWaves = 4;       // waves per workgroup
constexpr int kIds = 256;       // block ids staged in LDS per wave and round

struct PrefillParams {
  void* out;
  const void* q;
  const int32_t* cu_q_lens;
  const int32_t* context_lens;
  const int32_t* block_table;
  const char* k_cache;
  const char* v_cache;
  int32_t num_chunks;
  int32_t total_q;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t max_q_len;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // query heads per KV head
  int32_t tokens_per_group;  // query tokens per 16-column group = 16 / group
  float scale_log2;
};

template <int DT, int D, int NG, int DEPTH>
__global__ void __launch_bounds__(64 * kWaves)
prefill_kernel(PrefillParams p) {
  using Sh = Shape<DT, D>;
  __shared__ int32_t s_ids[kWaves][kIds];
  const int wv = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t c = blockIdx.z;
  const int32_t g = blockIdx.y;
  const int32_t G = p.group;
  const int32_t tpg = p.tokens_per_group;
  const int32_t wave_tokens = NG * tpg;

  // Rows outside [0, total_q) are never touched, whatever cu_q_lens holds.
  const int32_t q_begin = max(0, __builtin_amdgcn_readfirstlane(p.cu_q_lens[c]));
  const int32_t q_end = min(p.total_q, __builtin_amdgcn_readfirstlane(p.cu_q_lens[c + 1]));
  const int32_t qlen = max(0, min(q_end - q_begin, p.max_q_len));
  int32_t ctx = __builtin_amdgcn_readfirstlane(p.context_lens[c]);
  ctx = max(0, min(ctx, p.max_blocks * 16));
  const int32_t p0 = max(ctx - qlen, 0);  // position of the chunk's first query
  const int32_t tok0 = (blockIdx.x * kWaves + wv) * wave_tokens;
  if (tok0 >= qlen) return;
  const int32_t tok_last = min(tok0 + wave_tokens, qlen) - 1;
  const int32_t lim_max = min(p0 + tok_last, ctx - 1);
  const int32_t lim_min = min(p0 + tok0, ctx - 1);

  // Columns of group gi: token tok0 + gi*tpg + n/G, head g*G + n%G.
  QOp<DT, D> qv[NG];
  int lim[NG];
  bool valid[NG];
  int64_t row[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int32_t tok = tok0 + gi * tpg + n / G;
    valid[gi] = n < tpg * G && tok < qlen;
    row[gi] = ((int64_t)(q_begin + tok)) * p.num_q_heads + (int64_t)g * G + n % G;
    // Padding columns get a zero query and the wave's widest limit, so their
    // softmax state stays finite; they are never stored.
    lim[gi] = valid[gi] ? min(p0 + tok, ctx - 1) : lim_max;
    load_query<DT, D>(qv[gi], reinterpret_cast<const char*>(p.q) + (valid[gi] ? row[gi] : 0) * Sh::kRow,
                      valid[gi], kg);
  }
  State<DT, D> st[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) st[gi].reset();

  if (lim_max >= 0) {
    const int32_t nblk = lim_max / 16 + 1;
    const int32_t* trow = p.block_table + (int64_t)c * p.max_blocks;
    const uint32_t k_off = k_lane_offset<DT, D>(n, kg);
    const uint32_t v_off = v_lane_offset<DT, D>(n, kg);
    const int64_t block_stride = (int64_t)p.num_kv_heads * Sh::kTileBytes;
    const char* kbase = p.k_cache + (int64_t)g * Sh::kTileBytes;
    const char* vbase = p.v_cache + (int64_t)g * Sh::kTileBytes;
    int32_t* ids = s_ids[wv];
    for (int32_t c0 = 0; c0 < nblk; c0 += kIds) {
      const int32_t c1 = min(c0 + kIds, nblk);
      // This wave's own LDS row: in-order LDS access within the wave needs
      // no barrier.
      for (int32_t i = lane; i < c1 - c0; i += 64) {
        const int32_t b = trow[c0 + i];
        ids[i] = (uint32_t)b < (uint32_t)p.num_blocks ? b : 0;
      }
      __builtin_amdgcn_wave_barrier();
      auto block_of = [&](int32_t j) -> int64_t {
        return __builtin_amdgcn_readfirstlane(ids[min(j, c1 - 1) - c0]);
      };
      Tile<DT, D> buf[DEPTH];
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        const int64_t b = block_of(c0 + u);
        load_tile<DT, D>(buf[u], kbase + b * block_stride, vbase + b * block_stride, k_off, v_off);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int32_t jb = c0; jb < c1; jb += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
          const int32_t j = jb + u;
          const int32_t t0 = 16 * j;
          // Past the end of the round (at most DEPTH-1 tiles) everything is
          // masked, which leaves the state unchanged; the body stays free of
          // branches so the load wait counts stay exact.
          const bool live = j < c1;
          int lj[NG];
#pragma unroll
          for (int gi = 0; gi < NG; ++gi) lj[gi] = live ? lim[gi] : t0 - 1;
          attend_tile<DT, D, NG>(st, buf[u], qv, p.scale_log2, t0, lj, live ? ctx : t0,
                                 !live || t0 + 15 > lim_min, kg);
          const int64_t b = block_of(j + DEPTH);
          load_tile<DT, D>(buf[u], kbase + b * block_stride, vbase + b * block_stride, k_off, v_off);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_wave_barrier();
    }
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) store_row<DT, D>(p.out, row[gi], st[gi], kg, valid[gi]);
  } else {
    // Empty context: nothing to attend to, zero output.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (!valid[gi]) continue;
      char* dst = reinterpret_cast<char*>(p.out) + row[gi] * Sh::kRow;
      for (int b = 16 * kg; b < Sh::kRow; b += 64) *reinterpret_cast<uint4*>(dst + b) = uint4{0u, 0u, 0u, 0u};
    }
  }
}

int g_ng = 0;

int prefill_groups() {
  if (g_ng == 0) {
    int v = 2;
    if (const char* env = getenv("PKV_PREFILL_GROUPS")) {
      int e = atoi(env);
      if (e == 1 || e == 2 || e == 4) v = e;
    }
    g_ng = v;
  }
  return g_ng;
}

template <int DT, int D, int NG>
hipError_t launch_ng(const PrefillParams& prm, hipStream_t stream) {
  const int32_t wg_tokens = kWaves * NG * prm.tokens_per_group;
  const dim3 grid((prm.max_q_len + wg_tokens - 1) / wg_tokens, prm.num_kv_heads, prm.num_chunks);
  hipLaunchKernelGGL((prefill_kernel<DT, D, NG, 2>), grid, dim3(64 * kWaves), 0, stream, prm);
  return hipGetLastError();
}

template <int DT, int D>
hipError_t launch(const PrefillParams& prm, hipStream_t stream) {
  // fp32 head_dim 128 keeps one column group (register budget).
  if constexpr (Shape<DT, D>::kRow > 256) {
    return launch_ng<DT, D, 1>(prm, stream);
  } else {
    const int ng = prefill_groups();
    if (ng == 1) return launch_ng<DT, D, 1>(prm, stream);
    if (ng == 4) return launch_ng<DT, D, 4>(prm, stream);
    return launch_ng<DT, D, 2>(prm, stream);
  }
}

}  // namespace

namespace pkv {

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t stream) {
  PrefillParams p;
  p.out = a.out;
  p.q = a.q;
  p.cu_q_lens = a.cu_q_lens;
  p.context_lens = a.context_lens;
  p.block_table = a.block_table;
  p.k_cache = reinterpret_cast<const char*>(a.k_cache);
  p.v_cache = reinterpret_cast<const char*>(a.v_cache);
  p.num_chunks = a.num_chunks;
  p.total_q = a.total_q;
  p.num_blocks = a.num_blocks;
  p.max_blocks = a.max_blocks_per_seq;
  p.max_q_len = a.max_q_len;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.tokens_per_group = 16 / p.group;
  p.scale_log2 = a.scale * kLog2e;
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch<PKV_BF16, 128>(p, stream) : launch<PKV_BF16, 64>(p, stream);
  return a.head_dim == 128 ? launch<PKV_F32, 128>(p, stream) : launch<PKV_F32, 64>(p, stream);
}

}  // namespace pkv
