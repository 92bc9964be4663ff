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
// straight from global memory into LDS (two buffers: the next tile lands in
// one while the other is read), and every wave reads its MFMA operands from
// there, so the tile crosses from L2 once per workgroup instead of once per
// wave. Both products run on the 16x16x32 bf16 MFMA. The softmax keeps a
// lazily updated running max: a row's reference max moves only when a score
// exceeds it by more than 2^8, so the rescale of the accumulators (which
// would otherwise follow almost every tile) is skipped; the result is the
// same softmax, since any reference value cancels in the normalisation.
// Workgroups of one (chunk, KV head) are placed on the same XCD so that its
// K/V stays in that XCD's L2.
//
// f32 (prefill_kernel): each wave loads its own K/V tiles in MFMA register
// layout and runs the 16-token tile step shared with decode.
#include <atomic>
#include <cstdlib>
#include <utility>

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
constexpr int kRoundIds = 2048;    // block ids staged in LDS per round
constexpr float kLazyMax = 8.0f;   // log2 of the largest weight before a rescale
constexpr float kNoMax = -1e30f;   // reference max of a row that has seen nothing

typedef __attribute__((address_space(3))) char lds_char;
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

// LDS tile layout. A tile's K rows (32 positions of one head, 2*D bytes
// each) and then its V rows, unpadded; the 16-byte chunks of row r sit at
// chunk index c ^ swz(r). The swizzle spreads both operand reads over the
// 64 banks: the K operand read (16 rows x 64 bytes per instruction) finds
// four rows in each 64-byte bank window, the transposing V read (16 rows x
// 32 bytes) two rows in each 32-byte window.
template <int D>
struct Lds {
  static constexpr int kRow = 2 * D;                  // bytes of one position of one head
  static constexpr int kChunks = kRow / 16;           // 16-byte chunks per row
  static constexpr int kTile = kKeys * kRow;          // one tensor's tile
  static constexpr int kBuf = 2 * kTile;              // K tile, then V tile
  static constexpr int kThreads = 64 * kWaves;        // threads of one tile pipeline
  static constexpr int kRowsPerLoad = 1024 / kRow;    // rows one wave's 64 x 16-byte load fills
  static constexpr int kLoads = kTile / (1024 * kWaves);  // loads per wave and tensor
  static_assert(kLoads >= 1 && 16 % kRowsPerLoad == 0, "a load's rows must lie in one block");
};

template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + 2 * ((r >> 2) & 1);
  else return 2 * ((r >> 1) & 3);
}

// Calls f(std::integral_constant<int, 0>) ... f(<N-1>): the per-load values
// are then indexed by constants, which keeps them in registers.
template <typename F, int... I>
__device__ __forceinline__ void unroll_seq(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void unroll(F&& f) {
  unroll_seq(f, std::make_integer_sequence<int, N>{});
}

// Native 4 x 32-bit vector: loads and copies stay plain vector operations.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// Sixteen bytes of zeros per lane: the source of V rows past the
// workgroup's last visible position (so that their zero weights cannot
// meet a NaN in the pool).
static __device__ __align__(16) const char kZeroRows[1024] = {};

// Loop-invariant offsets of one thread. Load u of the thread's wave fills
// LDS bytes [1024 * (wq * kLoads + u), +1024) of a tensor's tile, lane l the
// 16 bytes at +16 l: row srow[u], chunk l % kChunks, which holds the
// source chunk (l % kChunks) ^ swz(row). All rows of one load lie in one
// pool block (blk[u], wave-uniform), so the block's address is scalar and
// the load takes it plus this 32-bit offset.
template <int D>
struct Lanes {
  static constexpr int kC = Lds<D>::kRow / 64;  // 64-byte K operand reads per 16 rows
  static constexpr int kE = D / 16;             // 16-dim V tiles
  uint32_t gofs[Lds<D>::kLoads];  // source byte offset inside the (block, head) tile
  uint32_t lofs[Lds<D>::kLoads];  // LDS byte offset of the load in a tensor tile (uniform)
  int32_t srow[Lds<D>::kLoads];   // tile position of the lane's piece
  int32_t blk[Lds<D>::kLoads];    // which of the tile's two blocks (uniform)
  uint32_t kofs[kC];              // K operand read offsets (lane (n, kg), rows 0..15)
  uint32_t vofs[kE];              // V operand read offsets (lane (n, kg), rows 4kg + n / 4)

  __device__ __forceinline__ void init(int wq, int lane, int n, int kg) {
    using L = Lds<D>;
    unroll<L::kLoads>([&](auto uc) {
      constexpr int u = decltype(uc)::value;
      const int r = (wq * L::kLoads + u) * L::kRowsPerLoad + lane / L::kChunks;
      const int c = lane % L::kChunks;
      gofs[u] = (uint32_t)((r % 16) * L::kRow + 16 * (c ^ swz<D>(r)));
      lofs[u] = (uint32_t)((wq * L::kLoads + u) * 1024);
      srow[u] = r;
      blk[u] = (wq * L::kLoads + u) * L::kRowsPerLoad / 16;
    });
    // K operand: lane (n, kg) reads 16 bytes (dims 8kg..8kg+7 of 64c..64c+31)
    // of row n: chunk kg + 4c.
#pragma unroll
    for (int c = 0; c < kC; ++c) kofs[c] = (uint32_t)(n * L::kRow + 16 * ((kg + 4 * c) ^ swz<D>(n)));
    // Transposing V read: lane 4j + q of a 16-lane group reads 8 bytes (dims
    // 4q..4q+3 of dim tile e) of row 4kg + j; lane n then receives dim n of
    // rows 4kg + 0..3.
    const int row = 4 * kg + n / 4, q = n % 4;
#pragma unroll
    for (int e = 0; e < kE; ++e)
      vofs[e] = (uint32_t)(L::kTile + row * L::kRow + 16 * ((2 * e + (q >> 1)) ^ swz<D>(row)) +
                           8 * (q & 1));
  }
};

// Global -> LDS, directly: this wave's loads of tile `jl` of the round (ids
// of its two blocks at s_ids[2*jl], [2*jl+1]) into buffer `buf`. V rows
// past `vlim` load zeros. Completion is tracked by the wave's vector memory
// counter; the buffer is read only after a wait and a barrier.
template <int D>
__device__ __forceinline__ void stage_tile(const Lanes<D>& ln, lds_char* buf, const char* kbase,
                                          const char* vbase, uint32_t block_stride,
                                          const lds_char* s_ids, int jl, int t0, int vlim,
                                          int lane) {
  using L = Lds<D>;
#pragma unroll
  for (int u = 0; u < L::kLoads; ++u) {
    const int32_t id = *reinterpret_cast<const __attribute__((address_space(3))) int32_t*>(
        s_ids + 4 * (2 * jl + ln.blk[u]));
    // 32 x 32 -> 64-bit product in scalar registers (block_stride < 2^32)
    const uint32_t b = (uint32_t)__builtin_amdgcn_readfirstlane(id);
    const uint64_t off = ((uint64_t)__umulhi(b, block_stride) << 32) | (uint32_t)(b * block_stride);
    const uint32_t lofs = (uint32_t)__builtin_amdgcn_readfirstlane(ln.lofs[u]);
    const char* vsrc = t0 + ln.srow[u] <= vlim ? vbase + off + ln.gofs[u] : kZeroRows + 16 * lane;
    // (the builtin exists only for the device target: the host pass, which
    // never runs this, does not see it)
#if defined(__HIP_DEVICE_COMPILE__)
    __builtin_amdgcn_global_load_lds(kbase + off + ln.gofs[u], (lds_void*)(buf + lofs), 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vsrc, (lds_void*)(buf + L::kTile + lofs), 16, 0, 0);
#endif
  }
}

// Scores of one LDS tile against NG column groups: s[gi][h] holds, in lane
// (n, kg), S[16h + 4kg + i][n] (position offset within the tile, column n).
template <int D, int NG>
__device__ __forceinline__ void tile_scores(f32x4 (&s)[NG][2], const lds_char* buf,
                                            const Lanes<D>& ln, const QOp<PKV_BF16, D> (&qv)[NG]) {
  using L = Lds<D>;
  typedef const __attribute__((address_space(3))) u32x4 lds_u32x4;
  constexpr int kC = L::kRow / 64;
  u32x4 kf[2][kC];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int c = 0; c < kC; ++c)
      kf[h][c] = *reinterpret_cast<lds_u32x4*>(buf + ln.kofs[c] + 16 * h * L::kRow);
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

// Running softmax state of one lane for NG column groups. The reference max
// mc (log2 units) moves only when a score passes thr, the raw score that
// stands 2^kLazyMax above it. o[gi][e] holds O^T rows 4kg + i of dim tile e
// (dims 16e + 4kg + i) of column n; l[gi] holds the column's weight sum in
// all four entries (a product with a row of ones).
template <int D, int NG>
struct Acc {
  float mc[NG];
  float thr[NG];
  f32x4 l[NG];
  f32x4 o[NG][D / 16];
};

__device__ __forceinline__ float max8(const float (&x)[8]) {
  const float a = fmaxf(fmaxf(x[0], x[1]), x[2]);
  const float b = fmaxf(fmaxf(x[3], x[4]), x[5]);
  return fmaxf(fmaxf(x[6], x[7]), fmaxf(a, b));
}

// Softmax weights of one tile and their product with its V rows.
// Lane (n, kg) owns positions {4kg + i, 16 + 4kg + i} of the tile for column
// n; those eight are also the reduction slots 8kg..8kg+7 of the PV MFMA, in
// the same order on both operands. `mask` (wave-uniform) applies the
// per-column causal limit (tiles that reach past the wave's smallest limit).
template <int D, int NG>
__device__ __forceinline__ void tile_softmax_pv(const f32x4 (&s)[NG][2], const lds_char* buf,
                                                const Lanes<D>& ln, Acc<D, NG>& a,
                                                const int (&lim)[NG], int t0, bool mask, float c,
                                                float tau_raw, int kg) {
  using L = Lds<D>;
  constexpr int kE = D / 16;
  // V operands first: their LDS latency then overlaps the softmax. (Rows
  // 16.. of the tile have the same swizzle as rows 0..15.)
  bf16x8 av[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + ln.vofs[e]));
    const i16x4_t hi =
        __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(buf + ln.vofs[e] + 16 * L::kRow));
    av[e] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
  }
  float x[NG][8];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi)
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[gi][4 * h + i] = s[gi][h][i];
  if (mask) {
    // (a scalar branch: only tiles that reach past the wave's smallest limit)
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
#pragma unroll
      for (int k = 0; k < 8; ++k)
        if (t0 + 16 * (k >> 2) + 4 * kg + (k & 3) > lim[gi]) x[gi][k] = -INFINITY;
  }
  bool grow = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) grow |= max8(x[gi]) > a.thr[gi];
  if (__ballot(grow) != 0) {
    // Some row passed its threshold: those rows move their reference to the
    // row max (the same value in the row's four lanes) and rescale; every
    // other row keeps alpha = 1.
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float rmax = wave_max_kg(max8(x[gi]));
      const bool upd = rmax > a.thr[gi];
      const float m_new = upd ? rmax * c : a.mc[gi];
      const float alpha = __builtin_amdgcn_exp2f(a.mc[gi] - m_new);
      a.mc[gi] = m_new;
      a.thr[gi] = upd ? rmax + tau_raw : a.thr[gi];
      a.l[gi] *= alpha;
#pragma unroll
      for (int e = 0; e < kE; ++e) a.o[gi][e] *= alpha;
    }
  }
  const u32x4 ones = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};  // bf16 1.0
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[gi][i], c, -a.mc[gi]));
    u32x4 pw;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bf16x2 pr = {(__bf16)p[2 * k], (__bf16)p[2 * k + 1]};
      pw[k] = __builtin_bit_cast(uint32_t, pr);
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
    // the weights as the MFMA sees them, summed by the MFMA itself
    a.l[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ones), pb, a.l[gi],
                                                      0, 0, 0);
#pragma unroll
    for (int e = 0; e < kE; ++e)
      a.o[gi][e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[e], pb, a.o[gi][e], 0, 0, 0);
  }
}

// Workgroup barrier for the LDS tile pipeline: waits for this wave's LDS
// writes only; global loads in flight stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

struct LdsParams {
  PrefillParams p;
  int32_t row_blocks;     // row blocks per (chunk, KV head)
  int32_t per_xcd;        // workgroups per XCD slot range
  int32_t num_wg;         // real workgroups (the grid may hold a few more)
  // Position parts: each row block's tiles are cut into `parts` equal runs,
  // one workgroup each. With parts > 1 a workgroup leaves its rows' softmax
  // state in `states` (slot = its logical index: NG x (2 + 4 D/16) x 256
  // floats, value v of group gi and thread t at (gi * kPer + v) * 256 + t)
  // and prefill_fold_kernel writes the output.
  int32_t parts;
  float* states;
};

// Most position parts per row block.
constexpr int kMaxParts = 16;

// SPLIT = 1: four waves, each with its own rows, walk all of the
// workgroup's tiles. SPLIT = 2: eight waves; waves 4..7 take the same rows as
// waves 0..3 but the second half of the tiles, through a second LDS pipeline,
// and hand their softmax state to waves 0..3 through LDS at the end. Either
// way a SIMD runs two waves (the second workgroup on the CU, or the other
// half), so one wave's MFMA work hides the other's softmax and waits.
template <int D, int NG, int SPLIT>
__global__ void __launch_bounds__(64 * kWaves * SPLIT, SPLIT == 1 ? 2 : 1)
prefill_lds_kernel(LdsParams lp) {
  using L = Lds<D>;
  constexpr int kE = D / 16;
  constexpr int kIds = kRoundIds / SPLIT;     // block ids per half and round
  constexpr int kBigPos = 1 << 30;            // position of a tile past every limit
  constexpr int kPer = 2 + 4 * kE;            // floats of a lane's softmax state per group
  // Two tile buffers per pipeline, as separate arrays: the compiler then
  // sees that the loads filling one never touch the other, and lets this
  // wave read one while its loads into the other are in flight.
  __shared__ __attribute__((aligned(16))) char s_bufa[SPLIT][L::kBuf];
  __shared__ __attribute__((aligned(16))) char s_bufb[SPLIT][L::kBuf];
  __shared__ __attribute__((aligned(16))) int32_t s_idarr[kRoundIds];
  __shared__ __attribute__((aligned(16))) float s_xs[SPLIT == 2 ? NG * kPer * 256 : 1];
  const PrefillParams& p = lp.p;

  // XCD-aware placement: hardware workgroup b runs on XCD b % 8; the
  // workgroups of one (chunk, KV head) take consecutive logical ids, which
  // land on one XCD.
  const int32_t hw = blockIdx.x;
  const int32_t wg = (hw & 7) * lp.per_xcd + (hw >> 3);
  if (wg >= lp.num_wg) return;
  const int32_t part = wg % lp.parts;   // the parts of a row block are consecutive
  const int32_t rbw = wg / lp.parts;
  const int32_t rb = rbw % lp.row_blocks;
  const int32_t pair = rbw / lp.row_blocks;
  const int32_t g = pair % p.num_kv_heads;
  const int32_t ch = pair / p.num_kv_heads;
  float* const state = lp.parts > 1 ? lp.states + (int64_t)wg * NG * kPer * 256 : nullptr;

  const int tid = threadIdx.x;
  // (wave-uniform values are made visibly uniform, so that the decisions
  // taken on them are scalar branches)
  const int half = __builtin_amdgcn_readfirstlane(tid >> 8);   // tile half (0 when SPLIT = 1)
  const int htid = tid & 255;                                   // thread index within the half
  const int wq = __builtin_amdgcn_readfirstlane(htid >> 6);    // row quarter of the workgroup
  const int lane = tid & 63;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t G = p.group;
  const int32_t tpg = p.tokens_per_group;
  lds_char* s_ids = (lds_char*)s_idarr + half * kIds * 4;
  lds_char* const bufa = (lds_char*)s_bufa[half];
  lds_char* const bufb = (lds_char*)s_bufb[half];

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
  const int32_t tok0 = wg_tok0 + wq * NG * tpg;
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

  const int32_t ntiles = lim_wg / kKeys + 1;
  if (lim_wg < 0) {
    // Empty context: nothing to attend to, zero output (with parts, an
    // empty state, which the fold turns into zeros).
    if (half != 0) return;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      if (lp.parts > 1) {
        float* d = state + gi * kPer * 256 + htid;
        for (int v = 0; v < kPer; ++v) d[v * 256] = v == 0 ? kNoMax : 0.f;
        continue;
      }
      if (!valid[gi]) continue;
      char* dst = reinterpret_cast<char*>(p.out) + row[gi] * L::kRow;
      for (int b = 16 * kg; b < L::kRow; b += 64) *reinterpret_cast<uint4*>(dst + b) = uint4{0u, 0u, 0u, 0u};
    }
    return;
  }

  // The reference max starts finite but below any score: a row that has
  // seen no position yet (possible in the second tile half) keeps weights
  // exp2(-inf) = 0 instead of exp2(-inf + inf); its first visible score
  // passes the -inf threshold and sets the reference.
  Acc<D, NG> acc;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    acc.mc[gi] = kNoMax;
    acc.thr[gi] = -INFINITY;
    acc.l[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int e = 0; e < kE; ++e) acc.o[gi][e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const float c = p.scale_log2;
  const float tau_raw = kLazyMax / c;
  const int32_t nblk = lim_wg / 16 + 1;        // blocks any row of this workgroup sees
  // Tiles of this part: [t_lo, t_hi) of [0, ntiles) (possibly none); of
  // this half: [tbeg, tbeg + tcnt). The first half has the most tiles; both
  // halves take the same number of steps, the second one's surplus steps
  // being fully masked.
  const int32_t span = (ntiles + lp.parts - 1) / lp.parts;
  const int32_t t_lo = min(ntiles, part * span);
  const int32_t t_hi = min(ntiles, t_lo + span);
  const int32_t steps = (t_hi - t_lo + SPLIT - 1) / SPLIT;
  const int32_t tbeg = t_lo + half * steps;
  const int32_t tcnt = max(0, min(steps, t_hi - tbeg));
  const int32_t* trow = p.block_table + (int64_t)ch * p.max_blocks;
  const uint32_t block_stride = (uint32_t)p.num_kv_heads * L::kRow * 16;
  const char* kbase = p.k_cache + (int64_t)g * L::kRow * 16;
  const char* vbase = p.v_cache + (int64_t)g * L::kRow * 16;
  Lanes<D> ln;
  ln.init(wq, lane, n, kg);

  for (int32_t j0 = 0; j0 < steps; j0 += kIds / 2) {
    const int32_t nt = min(kIds / 2, steps - j0);    // steps of this round
    const int32_t nv = max(0, min(nt, tcnt - j0));   // real tiles of this half in it
    __syncthreads();  // the previous round is done with the ids and buffers
    for (int32_t i = htid; i < 2 * nt; i += L::kThreads) {
      const int32_t bi = 2 * (tbeg + j0) + i;
      const int32_t b = i < 2 * nv && bi < nblk ? trow[bi] : 0;
      *reinterpret_cast<__attribute__((address_space(3))) int32_t*>(s_ids + 4 * i) =
          (uint32_t)b < (uint32_t)p.num_blocks ? b : 0;
    }
    __syncthreads();
    // Position of tile i of the round; a step with no tile of this half
    // gets a position past every limit (its K/V rows are block 0's, masked,
    // and its V rows load as zeros).
    auto pos = [&](int32_t i) -> int32_t {
      return i < nv ? kKeys * (tbeg + j0 + i) : kBigPos;
    };
    // Step i: the loads of tile i+1 go into the other buffer (which tile
    // i-1 used) while this wave scores tile i and takes its softmax and PV
    // product; then each wave waits for its own loads and the barrier makes
    // every wave's visible. Tiles alternate between the two buffers, which
    // the loop names directly (a buffer chosen at run time would hide from
    // the compiler that the in-flight loads never touch the buffer read).
#define PKV_TILE_LOAD(buf, i)                                                              \
  stage_tile<D>(ln, buf, kbase, vbase, block_stride, s_ids, i, pos(i), lim_wg, lane)
#define PKV_TILE_ATTEND(buf, i)                                                            \
  do {                                                                                     \
    f32x4 sc[NG][2];                                                                       \
    tile_scores<D, NG>(sc, buf, ln, qv);                                                   \
    const int32_t t0 = pos(i);                                                             \
    tile_softmax_pv<D, NG>(sc, buf, ln, acc, lim, t0, t0 + kKeys - 1 > lim_min, c, tau_raw, \
                           kg);                                                            \
  } while (0)
    PKV_TILE_LOAD(bufa, 0);
    __builtin_amdgcn_s_waitcnt(0);
    lds_barrier();
    int32_t i = 0;
    for (; i + 2 <= nt; i += 2) {
      PKV_TILE_LOAD(bufb, i + 1);
      PKV_TILE_ATTEND(bufa, i);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
      if (i + 2 < nt) PKV_TILE_LOAD(bufa, i + 2);
      PKV_TILE_ATTEND(bufb, i + 1);
      __builtin_amdgcn_s_waitcnt(0);
      lds_barrier();
    }
    if (i < nt) PKV_TILE_ATTEND(bufa, i);
#undef PKV_TILE_LOAD
#undef PKV_TILE_ATTEND
  }

  if constexpr (SPLIT == 2) {
    // Waves 4..7 hand (reference max, sum, accumulators) to the waves 0..3
    // that own the same rows, lane for lane; value v of lane t sits at float
    // v * 256 + t.
    typedef __attribute__((address_space(3))) float lds_float;
    lds_float* xs = (lds_float*)s_xs;
    __syncthreads();
    if (half == 1) {
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        lds_float* d = xs + gi * kPer * 256 + htid;
        d[0] = acc.mc[gi];
        d[256] = acc.l[gi][0];
#pragma unroll
        for (int e = 0; e < kE; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) d[(2 + 4 * e + i) * 256] = acc.o[gi][e][i];
      }
    }
    __syncthreads();
    if (half == 1) return;
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const lds_float* d = xs + gi * kPer * 256 + htid;
      const float mb = d[0];
      // A half that saw nothing visible still has max kNoMax, which gives it
      // weight 0 (and a row that saw nothing in either keeps sum 0; the
      // first half of part 0 always holds position 0).
      const float m = fmaxf(acc.mc[gi], mb);
      const float sa_ = __builtin_amdgcn_exp2f(acc.mc[gi] - m);
      const float sb_ = __builtin_amdgcn_exp2f(mb - m);
      acc.mc[gi] = m;   // the merged sum and accumulators are relative to m
      acc.l[gi][0] = acc.l[gi][0] * sa_ + d[256] * sb_;
#pragma unroll
      for (int e = 0; e < kE; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          acc.o[gi][e][i] = acc.o[gi][e][i] * sa_ + d[(2 + 4 * e + i) * 256] * sb_;
    }
  }

  if (lp.parts > 1) {
    // a part: the rows' state, for the fold
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      float* d = state + gi * kPer * 256 + htid;
      d[0] = acc.mc[gi];
      d[256] = acc.l[gi][0];
#pragma unroll
      for (int e = 0; e < kE; ++e)
#pragma unroll
        for (int i = 0; i < 4; ++i) d[(2 + 4 * e + i) * 256] = acc.o[gi][e][i];
    }
    return;
  }
  // Lane (n, kg) writes dims 16e + 4kg + 0..3 of its column's row.
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    if (!valid[gi]) continue;
    const float inv = 1.0f / acc.l[gi][0];
    char* dst = reinterpret_cast<char*>(p.out) + (row[gi] * D + 4 * kg) * 2;
#pragma unroll
    for (int e = 0; e < kE; ++e) {
      bf16x2 v01 = {(__bf16)(acc.o[gi][e][0] * inv), (__bf16)(acc.o[gi][e][1] * inv)};
      bf16x2 v23 = {(__bf16)(acc.o[gi][e][2] * inv), (__bf16)(acc.o[gi][e][3] * inv)};
      *reinterpret_cast<uint2*>(dst + 32 * e) =
          uint2{__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
    }
  }
}

// Parts whose states one fold thread loads together.
constexpr int kFoldBatch = 4;

// The fold of a launch with position parts: one workgroup of four waves per
// (row block, column group), each lane the same rows as in
// prefill_lds_kernel. The parts' states are folded in part order with the
// online-softmax rescale (to the larger of the two reference maxima), the
// loads of kFoldBatch parts issued together; then the normalised output
// (zeros for a row with no visible position: an empty context).
template <int D, int NG>
__global__ void __launch_bounds__(64 * kWaves)
prefill_fold_kernel(LdsParams lp) {
  constexpr int kE = D / 16;
  constexpr int kPer = 2 + 4 * kE;
  const PrefillParams& p = lp.p;
  const int32_t gi = blockIdx.x % NG;
  const int32_t rbw = blockIdx.x / NG;
  const int32_t rb = rbw % lp.row_blocks;
  const int32_t pair = rbw / lp.row_blocks;
  const int32_t g = pair % p.num_kv_heads;
  const int32_t ch = pair / p.num_kv_heads;
  const int htid = threadIdx.x;
  const int wq = __builtin_amdgcn_readfirstlane(htid >> 6);
  const int lane = htid & 63;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t G = p.group;
  const int32_t tpg = p.tokens_per_group;
  const int32_t q_begin = max(0, __builtin_amdgcn_readfirstlane(p.cu_q_lens[ch]));
  const int32_t q_end = min(p.total_q, __builtin_amdgcn_readfirstlane(p.cu_q_lens[ch + 1]));
  const int32_t qlen = max(0, min(q_end - q_begin, p.max_q_len));
  const int32_t wg_tok0 = rb * (kWaves * NG * tpg);
  if (wg_tok0 >= qlen) return;   // the main kernel left nothing here either
  const int32_t tok = wg_tok0 + wq * NG * tpg + gi * tpg + n / G;
  if (!(n < tpg * G && tok < qlen)) return;
  const int64_t row = ((int64_t)(q_begin + tok)) * p.num_q_heads + (int64_t)g * G + n % G;
  const int64_t part_stride = (int64_t)NG * kPer * 256;
  const float* d0 = lp.states + (int64_t)rbw * lp.parts * part_stride + gi * kPer * 256 + htid;
  float m = kNoMax, l = 0.f;
  f32x4 o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int32_t k0 = 0; k0 < lp.parts; k0 += kFoldBatch) {
    float v[kFoldBatch][kPer];
#pragma unroll
    for (int b = 0; b < kFoldBatch; ++b)
      if (k0 + b < lp.parts) {
        const float* d = d0 + (k0 + b) * part_stride;
#pragma unroll
        for (int j = 0; j < kPer; ++j) v[b][j] = d[j * 256];
      }
#pragma unroll
    for (int b = 0; b < kFoldBatch; ++b)
      if (k0 + b < lp.parts) {
        // (an empty part has reference kNoMax and sum 0: weight 0, or a
        // factor 1 on another empty state)
        const float mn = fmaxf(m, v[b][0]);
        const float so = __builtin_amdgcn_exp2f(m - mn);
        const float sk = __builtin_amdgcn_exp2f(v[b][0] - mn);
        l = l * so + v[b][1] * sk;
#pragma unroll
        for (int e = 0; e < kE; ++e)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[e][i] = o[e][i] * so + v[b][2 + 4 * e + i] * sk;
        m = mn;
      }
  }
  const float inv = l > 0.f ? 1.0f / l : 0.f;
  char* dst = reinterpret_cast<char*>(p.out) + (row * D + 4 * kg) * 2;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    bf16x2 v01 = {(__bf16)(o[e][0] * inv), (__bf16)(o[e][1] * inv)};
    bf16x2 v23 = {(__bf16)(o[e][2] * inv), (__bf16)(o[e][3] * inv)};
    *reinterpret_cast<uint2*>(dst + 32 * e) =
        uint2{__builtin_bit_cast(uint32_t, v01), __builtin_bit_cast(uint32_t, v23)};
  }
}

// Launch settings read by every call, possibly from several host threads:
// atomics; the CU count is cached per device (0 = not known yet).
std::atomic<int> g_ng{0};

int prefill_groups() {
  int v = g_ng.load(std::memory_order_relaxed);
  if (v == 0) {
    v = 2;
    if (const char* env = getenv("PKV_PREFILL_GROUPS")) {
      int e = atoi(env);
      if (e == 1 || e == 2) v = e;
    }
    g_ng.store(v, std::memory_order_relaxed);
  }
  return v;
}

constexpr int kMaxDevices = 64;
std::atomic<int> g_num_cus[kMaxDevices];

int num_cus() {
  int dev = 0, v = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < kMaxDevices && (v = g_num_cus[dev].load(std::memory_order_relaxed)) > 0) return v;
  if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || v <= 0)
    v = 256;
  if (dev < kMaxDevices) g_num_cus[dev].store(v, std::memory_order_relaxed);
  return v;
}

template <int D, int NG, int SPLIT>
hipError_t launch_lds_split(const LdsParams& lp, hipStream_t stream) {
  // (LDS: static arrays of the kernel)
  hipLaunchKernelGGL((prefill_lds_kernel<D, NG, SPLIT>), dim3(8 * lp.per_xcd),
                     dim3(64 * kWaves * SPLIT), 0, stream, lp);
  return hipGetLastError();
}

// Position parts of a launch of `nwg` row blocks. With fewer row blocks
// than CUs, as many parts as keep one eight-wave workgroup per CU; if that
// still leaves a quarter of the CUs idle, enough for two four-wave
// workgroups per CU instead; at most kMaxParts. 1 with a row block per CU
// or more (more parts there measured slower).
int position_parts(int64_t nwg) {
  if (const char* env = getenv("PKV_PREFILL_PARTS")) {   // tuning override
    const int v = atoi(env);
    if (v >= 1 && v <= kMaxParts) return v;
  }
  const int64_t cus = num_cus();
  if (nwg <= 0 || nwg >= cus) return 1;
  int64_t parts = cus / nwg;
  if (4 * parts * nwg < 3 * cus) parts = (2 * cus + nwg - 1) / nwg;
  return (int)std::min<int64_t>(kMaxParts, parts);
}

template <int D, int NG>
hipError_t launch_lds(const PrefillParams& prm, hipStream_t stream, float* states) {
  LdsParams lp;
  lp.p = prm;
  const int32_t wg_tokens = kWaves * NG * prm.tokens_per_group;
  lp.row_blocks = (prm.max_q_len + wg_tokens - 1) / wg_tokens;
  const int64_t nwg = (int64_t)lp.row_blocks * prm.num_kv_heads * prm.num_chunks;
  if (nwg * kMaxParts * 64 * kWaves * 2 > INT32_MAX) return hipErrorInvalidConfiguration;
  lp.parts = states != nullptr ? position_parts(nwg) : 1;
  lp.states = states;
  lp.num_wg = (int32_t)(nwg * lp.parts);
  lp.per_xcd = (lp.num_wg + 7) / 8;
  // Two waves per SIMD either way: with fewer than two workgroups per CU,
  // each workgroup splits its tiles over two sets of waves.
  hipError_t e = lp.num_wg >= 2 * (int64_t)num_cus() ? launch_lds_split<D, NG, 1>(lp, stream)
                                                      : launch_lds_split<D, NG, 2>(lp, stream);
  if (e != hipSuccess || lp.parts == 1) return e;
  hipLaunchKernelGGL((prefill_fold_kernel<D, NG>), dim3((uint32_t)(nwg * NG)), dim3(64 * kWaves), 0,
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
hipError_t launch(const PrefillParams& prm, hipStream_t stream, float* states) {
  if constexpr (DT == PKV_BF16) {
    if (prefill_groups() == 1) return launch_lds<D, 1>(prm, stream, states);
    return launch_lds<D, 2>(prm, stream, states);
  } else if constexpr (Shape<DT, D>::kRow > 256) {
    // fp32 head_dim 128 keeps one column group (register budget).
    return launch_ng<DT, D, 1>(prm, stream);
  } else {
    return launch_ng<DT, D, 2>(prm, stream);
  }
}

}  // namespace

namespace pkv {

size_t prefill_workspace_bytes(int32_t num_chunks, int32_t num_q_heads, int32_t num_kv_heads,
                               int32_t head_dim, int32_t max_q_len) {
  if (num_chunks <= 0 || max_q_len <= 0 || num_kv_heads <= 0 || num_q_heads < num_kv_heads)
    return 0;
  const int64_t ng = prefill_groups();
  const int64_t rows = kWaves * ng * (16 / (num_q_heads / num_kv_heads));
  const int64_t nwg = (int64_t)num_chunks * num_kv_heads * ((max_q_len + rows - 1) / rows);
  const int parts = position_parts(nwg);
  if (parts == 1) return 0;
  return (size_t)(nwg * parts * ng * (2 + 4 * (head_dim / 16)) * 256 * 4);
}

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
  // position parts only with a workspace that holds their states
  float* states = nullptr;
  if (a.dtype == PKV_BF16 && a.workspace != nullptr) {
    const size_t need = prefill_workspace_bytes(a.num_chunks, a.num_q_heads, a.num_kv_heads,
                                                a.head_dim, a.max_q_len);
    if (need > 0 && a.workspace_bytes >= need) states = reinterpret_cast<float*>(a.workspace);
  }
  if (a.dtype == PKV_BF16)
    return a.head_dim == 128 ? launch<PKV_BF16, 128>(p, stream, states)
                             : launch<PKV_BF16, 64>(p, stream, states);
  return a.head_dim == 128 ? launch<PKV_F32, 128>(p, stream, nullptr)
                           : launch<PKV_F32, 64>(p, stream, nullptr);
}

}  // namespace pkv
