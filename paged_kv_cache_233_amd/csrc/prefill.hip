// Chunked-prefill attention over paged KV for gfx950: a chunk of consecutive
// query tokens of one sequence attends causally to the sequence's cached
// tokens plus the chunk's own ("(2) vLLM Internals: From PagedAttention to
// Removing PagedAttention", section "2. Continuous Batching"; "vLLM: what
// PagedAttention turned into", section "The scheduler, and what it has to
// balance now"). Keys and values are gathered through the block table inside
// the kernel.
//
// Rows: a "column group" is 16 MFMA columns = 16/G consecutive query tokens x
// the G query heads of one KV head (grouped-query attention), so every K/V
// tile serves all G heads at once. Query position p sees positions 0..p.
//
// bf16 (prefill_lds_kernel): a workgroup of 4 waves owns 4*NG column groups
// of one (chunk, KV head) and walks that sequence's K/V in tiles of 32
// positions (two pool blocks). The four waves load each tile once, together,
// into LDS (three buffers: one being filled while one is scored and one is
// multiplied), and every wave reads its MFMA operands from there, so the
// tile crosses from L2 once per workgroup instead of once per wave. Both
// products run on the 16x16x32 bf16 MFMA. The softmax keeps a lazily
// updated running max: a row's reference max moves only when a score
// exceeds it by more than 2^8, so the rescale of the accumulators (which
// would otherwise follow almost every tile) is skipped; the result is the
// same softmax, since any reference value cancels in the normalisation.
// Workgroups of one (chunk, KV head) are placed on the same XCD so that its
// K/V stays in that XCD's L2.
//
// f32 (prefill_kernel): each wave loads its own K/V tiles in MFMA register
// layout and runs the 16-token tile step shared with decode.
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

// ------------------------------------------------------------ bf16, LDS
constexpr int kKeys = 32;          // positions per LDS tile (two pool blocks)
constexpr int kBufs = 3;           // LDS tile buffers
constexpr int kRoundIds = 2048;    // block ids staged in LDS per round
constexpr float kLazyMax = 8.0f;   // log2 of the largest weight before a rescale

template <int D>
struct Lds {
  static constexpr int kRow = 2 * D;                  // bytes of one position of one head
  static constexpr int kPitch = kRow + 16;            // padded LDS row: no bank conflicts on
                                                      // the column-wise K operand reads
  static constexpr int kPieces = kRow / 16;           // 16-byte pieces per row
  static constexpr int kPerThread = kKeys * kPieces / (64 * kWaves);
  static constexpr int kHalf = kKeys * kPitch;        // K (or V) part of one buffer
  static constexpr int kBuf = 2 * kHalf;
  static constexpr int kVBytes = kRow / 16;           // V bytes per lane per row
  static_assert(kPerThread >= 1, "tile smaller than the workgroup");
};

template <int D>
struct Staged {
  uint4 k[Lds<D>::kPerThread];
  uint4 v[Lds<D>::kPerThread];
};

// Global -> registers: this thread's pieces of tile `j` (ids of the tile's
// blocks at s_ids[2*jl], [2*jl+1]).
template <int D>
__device__ __forceinline__ void tile_fetch(Staged<D>& st, const char* kbase, const char* vbase,
                                           int64_t block_stride, const int32_t* s_ids, int jl,
                                           int tid) {
  using L = Lds<D>;
#pragma unroll
  for (int u = 0; u < L::kPerThread; ++u) {
    const int q = tid + 64 * kWaves * u;
    const int r = q / L::kPieces;               // position in the tile
    const int col = q % L::kPieces;
    const int64_t b = s_ids[2 * jl + (r >> 4)];
    const int64_t off = b * block_stride + (r & 15) * L::kRow + 16 * col;
    st.k[u] = *reinterpret_cast<const uint4*>(kbase + off);
    st.v[u] = *reinterpret_cast<const uint4*>(vbase + off);
  }
}

// Registers -> LDS buffer. V rows past `vlim` (no query of this workgroup
// sees them; the pool may hold anything there) are stored as zeros, so that
// their zero weights cannot meet a NaN.
template <int D>
__device__ __forceinline__ void tile_store(const Staged<D>& st, char* buf, int t0, int vlim,
                                           int tid) {
  using L = Lds<D>;
#pragma unroll
  for (int u = 0; u < L::kPerThread; ++u) {
    const int q = tid + 64 * kWaves * u;
    const int r = q / L::kPieces;
    const int col = q % L::kPieces;
    char* dst = buf + r * L::kPitch + 16 * col;
    const uint32_t keep = t0 + r <= vlim ? ~0u : 0u;
    *reinterpret_cast<uint4*>(dst) = st.k[u];
    *reinterpret_cast<uint4*>(dst + L::kHalf) =
        uint4{st.v[u].x & keep, st.v[u].y & keep, st.v[u].z & keep, st.v[u].w & keep};
  }
}

// Scores of one LDS tile against NG column groups: s[gi][h] holds, in lane
// (n, kg), S[16h + 4kg + i][n] (position offset within the tile, column n).
template <int D, int NG>
__device__ __forceinline__ void tile_scores(f32x4 (&s)[NG][2], const char* buf,
                                            const QOp<PKV_BF16, D> (&qv)[NG], int n, int kg) {
  using L = Lds<D>;
  constexpr int kC = L::kRow / 64;
  uint4 kf[2][kC];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < kC; ++c)
      kf[h][c] = *reinterpret_cast<const uint4*>(buf + (16 * h + n) * L::kPitch + 64 * c + 16 * kg);
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < kC; ++c)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kf[h][c]),
                                                      __builtin_bit_cast(bf16x8, qv[gi].c[c]), acc,
                                                      0, 0, 0);
      s[gi][h] = acc;
    }
}

// Softmax weights of one tile and their product with its V rows.
// Lane (n, kg) owns positions {4kg + i, 16 + 4kg + i} of the tile for column
// n; those eight are also the reduction slots 8kg..8kg+7 of the PV MFMA, in
// the same order on both operands.
template <int D, int NG>
__device__ __forceinline__ void tile_softmax_pv(const f32x4 (&s)[NG][2], const char* buf,
                                                float (&m)[NG], float (&lsum)[NG],
                                                f32x4 (&o)[NG][D / 16], const int (&lim)[NG],
                                                int t0, bool mask, float c, int n, int kg) {
  using L = Lds<D>;
  constexpr int kE = D / 16;
  float x[NG][8];
  bool grow = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float v = s[gi][h][i];
        if (mask && t0 + 16 * h + 4 * kg + i > lim[gi]) v = -INFINITY;
        x[gi][4 * h + i] = v;
      }
    const float lmax = fmaxf(fmaxf(fmaxf(x[gi][0], x[gi][1]), fmaxf(x[gi][2], x[gi][3])),
                             fmaxf(fmaxf(x[gi][4], x[gi][5]), fmaxf(x[gi][6], x[gi][7])));
    grow |= lmax * c > m[gi] + kLazyMax;
  }
  if (__ballot(grow) != 0) {
    // Some row's scores passed its reference max by more than 2^kLazyMax:
    // those rows move their reference to the row max (the same value in the
    // row's four lanes) and rescale; every other row keeps alpha = 1.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float lmax = x[gi][0];
#pragma unroll
      for (int i = 1; i < 8; ++i) lmax = fmaxf(lmax, x[gi][i]);
      const float rmax = wave_max_kg(lmax) * c;
      const float m_new = rmax > m[gi] + kLazyMax ? rmax : m[gi];
      const float alpha = __builtin_amdgcn_exp2f(m[gi] - m_new);
      m[gi] = m_new;
      lsum[gi] *= alpha;
#pragma unroll
      for (int e = 0; e < kE; ++e) o[gi][e] *= alpha;
    }
  }
  uint4 pb[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[gi][i], c, -m[gi]));
    lsum[gi] += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bf16x2 pr = {(__bf16)p[2 * k], (__bf16)p[2 * k + 1]};
      w[k] = __builtin_bit_cast(uint32_t, pr);
    }
    pb[gi] = uint4{w[0], w[1], w[2], w[3]};
  }
  // V rows of this lane's eight positions, dims [n*D/16, (n+1)*D/16).
  constexpr int kW = L::kVBytes / 4;
  uint32_t vr[8][kW];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int row = 16 * (k >> 2) + 4 * kg + (k & 3);
    const char* src = buf + L::kHalf + row * L::kPitch + n * L::kVBytes;
    if constexpr (kW == 4) {
      const uint4 t = *reinterpret_cast<const uint4*>(src);
      vr[k][0] = t.x; vr[k][1] = t.y; vr[k][2] = t.z; vr[k][3] = t.w;
    } else {
      const uint2 t = *reinterpret_cast<const uint2*>(src);
      vr[k][0] = t.x; vr[k][1] = t.y;
    }
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const int w = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint4 a;
    a.x = __builtin_amdgcn_perm(vr[1][w], vr[0][w], sel);
    a.y = __builtin_amdgcn_perm(vr[3][w], vr[2][w], sel);
    a.z = __builtin_amdgcn_perm(vr[5][w], vr[4][w], sel);
    a.w = __builtin_amdgcn_perm(vr[7][w], vr[6][w], sel);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      o[gi][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                         __builtin_bit_cast(bf16x8, pb[gi]),
                                                         o[gi][e], 0, 0, 0);
  }
}

struct LdsParams {
  PrefillParams p;
  int32_t row_blocks;     // workgroups per (chunk, KV head)
  int32_t per_xcd;        // workgroups per XCD slot range
  int32_t num_wg;         // real workgroups (the grid may hold a few more)
};

template <int D, int NG>
__global__ void __launch_bounds__(64 * kWaves)
prefill_lds_kernel(LdsParams lp) {
  using L = Lds<D>;
  constexpr int kE = D / 16;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int32_t* s_ids = reinterpret_cast<int32_t*>(smem);
  char* bufs = smem + kRoundIds * 4;
  const PrefillParams& p = lp.p;

  // XCD-aware placement: hardware workgroup b runs on XCD b % 8; the
  // workgroups of one (chunk, KV head) take consecutive logical ids, which
  // land on one XCD.
  const int32_t hw = blockIdx.x;
  const int32_t wg = (hw & 7) * lp.per_xcd + (hw >> 3);
  if (wg >= lp.num_wg) return;
  const int32_t rb = wg % lp.row_blocks;
  const int32_t pair = wg / lp.row_blocks;
  const int32_t g = pair % p.num_kv_heads;
  const int32_t ch = pair / p.num_kv_heads;

  const int tid = threadIdx.x;
  const int wv = tid >> 6;
  const int lane = tid & 63;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t G = p.group;
  const int32_t tpg = p.tokens_per_group;

  const int32_t q_begin = max(0, __builtin_amdgcn_readfirstlane(p.cu_q_lens[ch]));
  const int32_t q_end = min(p.total_q, __builtin_amdgcn_readfirstlane(p.cu_q_lens[ch + 1]));
  const int32_t qlen = max(0, min(q_end - q_begin, p.max_q_len));
  int32_t ctx = __builtin_amdgcn_readfirstlane(p.context_lens[ch]);
  ctx = max(0, min(ctx, p.max_blocks * 16));
  const int32_t p0 = max(ctx - qlen, 0);
  const int32_t wg_tok0 = rb * (kWaves * NG * tpg);
  if (wg_tok0 >= qlen) return;  // whole workgroup idle: before any barrier
  const int32_t wg_tok_last = min(wg_tok0 + kWaves * NG * tpg, qlen) - 1;
  const int32_t lim_wg = min(p0 + wg_tok_last, ctx - 1);  // furthest position any row sees

  // This wave's columns (waves past the chunk's end keep padding columns and
  // still take part in the loads and barriers).
  const int32_t tok0 = wg_tok0 + wv * NG * tpg;
  const int32_t lim_min = min(p0 + min(tok0, qlen - 1), ctx - 1);
  QOp<PKV_BF16, D> qv[NG];
  int lim[NG];
  bool valid[NG];
  int64_t row[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int32_t tok = tok0 + gi * tpg + n / G;
    valid[gi] = n < tpg * G && tok < qlen;
    row[gi] = ((int64_t)(q_begin + tok)) * p.num_q_heads + (int64_t)g * G + n % G;
    lim[gi] = valid[gi] ? min(p0 + tok, ctx - 1) : lim_wg;
    load_query<PKV_BF16, D>(qv[gi], reinterpret_cast<const char*>(p.q) + (valid[gi] ? row[gi] : 0) * L::kRow,
                            valid[gi], kg);
  }

  if (lim_wg < 0) {
    // Empty context: nothing to attend to, zero output.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (!valid[gi]) continue;
      char* dst = reinterpret_cast<char*>(p.out) + row[gi] * L::kRow;
      for (int b = 16 * kg; b < L::kRow; b += 64) *reinterpret_cast<uint4*>(dst + b) = uint4{0u, 0u, 0u, 0u};
    }
    return;
  }

  float m[NG], lsum[NG];
  f32x4 o[NG][kE];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    m[gi] = -INFINITY;
    lsum[gi] = 0.f;
#pragma unroll
    for (int e = 0; e < kE; ++e) o[gi][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float c = p.scale_log2;
  const int32_t nblk = lim_wg / 16 + 1;        // blocks any row of this workgroup sees
  const int32_t ntiles = lim_wg / kKeys + 1;
  const int32_t* trow = p.block_table + (int64_t)ch * p.max_blocks;
  const int64_t block_stride = (int64_t)p.num_kv_heads * L::kRow * 16;
  const char* kbase = p.k_cache + (int64_t)g * L::kRow * 16;
  const char* vbase = p.v_cache + (int64_t)g * L::kRow * 16;

  for (int32_t j0 = 0; j0 < ntiles; j0 += kRoundIds / 2) {
    const int32_t nt = min(kRoundIds / 2, ntiles - j0);
    __syncthreads();  // the previous round is done with the ids and buffers
    for (int32_t i = tid; i < 2 * nt; i += 64 * kWaves) {
      const int32_t bi = 2 * j0 + i;
      const int32_t b = bi < nblk ? trow[bi] : 0;
      s_ids[i] = (uint32_t)b < (uint32_t)p.num_blocks ? b : 0;
    }
    __syncthreads();
    Staged<D> st;
    tile_fetch<D>(st, kbase, vbase, block_stride, s_ids, 0, tid);
    tile_store<D>(st, bufs, kKeys * j0, lim_wg, tid);
    if (nt > 1) {
      tile_fetch<D>(st, kbase, vbase, block_stride, s_ids, 1, tid);
      tile_store<D>(st, bufs + L::kBuf, kKeys * (j0 + 1), lim_wg, tid);
    }
    __syncthreads();
    f32x4 scur[NG][2];
    tile_scores<D, NG>(scur, bufs, qv, n, kg);
    for (int32_t i = 0; i < nt; ++i) {
      // The body has no branches: near the round's end it fetches the last
      // tile again and stores it into the buffer no later step reads.
      tile_fetch<D>(st, kbase, vbase, block_stride, s_ids, min(i + 2, nt - 1), tid);
      // scores of the next tile (its buffer is ready) ahead of this tile's
      // softmax, so the two overlap; past the round's end they are unused
      f32x4 snext[NG][2];
      tile_scores<D, NG>(snext, bufs + ((i + 1) % kBufs) * L::kBuf, qv, n, kg);
      const int32_t t0 = kKeys * (j0 + i);
      tile_softmax_pv<D, NG>(scur, bufs + (i % kBufs) * L::kBuf, m, lsum, o, lim, t0,
                             t0 + kKeys - 1 > lim_min, c, n, kg);
      tile_store<D>(st, bufs + ((i + 2) % kBufs) * L::kBuf, kKeys * (j0 + min(i + 2, nt - 1)), lim_wg, tid);
      __syncthreads();
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        scur[gi][0] = snext[gi][0];
        scur[gi][1] = snext[gi][1];
      }
    }
  }

#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l = wave_sum_kg(lsum[gi]);
    if (!valid[gi]) continue;
    const float inv = 1.0f / l;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * kg + i) * kE;
      uint32_t w[kE / 2];
#pragma unroll
      for (int e = 0; e < kE; e += 2) {
        bf16x2 v = {(__bf16)(o[gi][e][i] * inv), (__bf16)(o[gi][e + 1][i] * inv)};
        w[e / 2] = __builtin_bit_cast(uint32_t, v);
      }
      char* dst = reinterpret_cast<char*>(p.out) + (row[gi] * D + d0) * 2;
      if constexpr (kE == 8) {
        *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
      } else {
        *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
      }
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

template <int D, int NG>
hipError_t launch_lds(const PrefillParams& prm, hipStream_t stream) {
  LdsParams lp;
  lp.p = prm;
  const int32_t wg_tokens = kWaves * NG * prm.tokens_per_group;
  lp.row_blocks = (prm.max_q_len + wg_tokens - 1) / wg_tokens;
  const int64_t nwg = (int64_t)lp.row_blocks * prm.num_kv_heads * prm.num_chunks;
  if (nwg * 64 * kWaves > INT32_MAX) return hipErrorInvalidConfiguration;
  lp.num_wg = (int32_t)nwg;
  lp.per_xcd = (lp.num_wg + 7) / 8;
  const size_t lds = kRoundIds * 4 + kBufs * Lds<D>::kBuf;
  hipLaunchKernelGGL((prefill_lds_kernel<D, NG>), dim3(8 * lp.per_xcd), dim3(64 * kWaves), lds,
                     stream, lp);
  return hipGetLastError();
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
  if constexpr (DT == PKV_BF16) {
    const int ng = prefill_groups();
    if (ng == 1) return launch_lds<D, 1>(prm, stream);
    if (ng == 4) return launch_lds<D, 4>(prm, stream);
    return launch_lds<D, 2>(prm, stream);
  } else if constexpr (Shape<DT, D>::kRow > 256) {
    // fp32 head_dim 128 keeps one column group (register budget).
    return launch_ng<DT, D, 1>(prm, stream);
  } else {
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
