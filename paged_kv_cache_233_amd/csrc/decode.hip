// Paged decode attention for gfx950: one query token per sequence, grouped
// query heads, keys and values gathered through the block table inside the
// kernel ("(2) vLLM Internals: From PagedAttention to Removing
// PagedAttention", section 4.1 "Why It Could Go"; "My Understanding of vLLM
// and PagedAttention", sections "3. PagedAttention CUDA Kernel" and "Step 4 --
// Attention Computation").
//
// Work split (split-KV, balanced): all (KV head g, sequence s, block j) tiles
// form one index space ordered by g, then s, then j, in which every sequence
// also counts a few units before its first block for the fixed cost of a
// piece (below). The grid is a fixed number W of single-wave workgroups;
// logical wave w takes the contiguous unit range [w*T/W, (w+1)*T/W), T the
// total unit count, so every wave reads about the same number of K/V bytes
// whatever the length mix. Hardware workgroup b
// runs on XCD b % 8; logical waves are numbered so that each XCD owns one
// contiguous eighth of the index space (one KV head when there are 8), which
// keeps blocks shared between sequences (a common prefix) in one XCD's L2.
//
// A wave's range splits into pieces, one per (g, s) it touches. A piece that
// covers a whole sequence writes the final output; any other piece writes
// its partial softmax state (running max, sum, unnormalised output) to one of
// the wave's two workspace slots. A second kernel merges the partial states
// of each split sequence in wave order, which is token order: the result is
// deterministic and needs no atomics. (Merging in the last-arriving wave
// instead would need a device-scope release per partial state, which writes
// back the whole L2 of an XCD and costs far more than the second launch.)
//
// Per 16-token block and KV head the wave loads the K tile and the V tile
// straight into registers and runs the MFMA tile step of tile_attn.h; the G
// query heads of the group fill G of the 16 MFMA columns, the other columns
// carry zero queries and are never stored.
//
// Append mode folds the cache write of the step's new token into the same
// pass: the wave holding a sequence's last block writes the token's K and V
// rows into it while staging its round, before it loads that block.
#include <atomic>
#include <cstdlib>
#include <mutex>

#include "internal.h"
#include "tile_attn.h"

// (the scratch array of the no-alloc decode; see decode_scratch below)
static __device__ __align__(256) char scratch[PKV_DECODE_SCRATCH_BYTES];

namespace {

using namespace pkv::tile;

constexpr int kXcds = 8;        // workgroups are dealt round-robin over 8 XCDs

struct DecodeParams {
  void* out;
  const void* q;
  const char* k_cache;
  const char* v_cache;
  const int32_t* block_table;
  const int32_t* context_lens;
  int32_t* ws_prefix;     // [num_seqs + 1] block-count prefix sums (written by wave 0)
  float* ws_partial;      // [2 * W][G * (D + 4)] partial states: O[G][D], m[G], l[G]
  int32_t num_seqs;
  int32_t num_blocks;
  int32_t max_blocks;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t num_waves;
  int32_t pieces_per_round;  // pieces whose query rows fit the LDS budget
  int32_t piece_cost;        // partition units a sequence costs besides its blocks
  float scale_log2;
  // Shared-prefix mode: every sequence's first `skip` blocks (the same
  // blocks in every row of the table) are attended once for all sequences,
  // by `pwaves` extra workgroups after the decode waves (see prefix_wave).
  // They leave `pparts` softmax states per query row
  // (pstate[part * pstride + row * (D + 4)]: O[D], max (log2 units), sum, two
  // floats of padding that keep every row 16-byte aligned), which the merge
  // kernel folds before the sequence's own states. The decode waves then
  // write no output: they leave the state of a sequence one wave holds whole
  // in ws_whole[s * num_kv_heads + g] (G x (D + 4) floats), and the merge
  // kernel writes every output. skip = 0, pwaves = 0 and pstate = nullptr
  // otherwise.
  int32_t skip;
  int32_t pparts;
  float* pstate;
  int64_t pstride;
  float* ws_whole;
  int32_t pwaves;    // prefix workgroups (a multiple of 8)
  int32_t pcols;     // prefix column blocks per KV head
  int32_t punits;    // num_kv_heads * pcols * pparts
  // Append mode (k_new != nullptr): before attending, the wave holding the
  // block of a sequence's last position writes that position's key and
  // value (k_new/v_new rows new_stride bytes apart, [num_kv_heads][D] each)
  // into it, and its own later loads of the block read them back.
  const char* k_new;
  const char* v_new;
  int64_t new_stride;
};

// Length of sequence s after clamping to [0, table width in tokens]; s may
// differ per lane.
__device__ __forceinline__ int32_t seq_len_clamped(const DecodeParams& p, int32_t s) {
  int32_t n = p.context_lens[s];
  n = n < 0 ? 0 : n;
  const int32_t cap = p.max_blocks * 16;
  n = n > cap ? cap : n;
  n -= 16 * p.skip;                      // positions left after the shared prefix
  return n < 0 ? 0 : n;
}

// The same for a wave-uniform s, kept in a scalar register.
__device__ __forceinline__ int32_t seq_len_uniform(const DecodeParams& p, int32_t s) {
  return __builtin_amdgcn_readfirstlane(seq_len_clamped(p, s));
}

// Inclusive prefix sum across the wave.
__device__ __forceinline__ int32_t wave_incl_scan(int32_t x) {
  const int lane = threadIdx.x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int32_t y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

template <int DT, int D>
__device__ __forceinline__ void write_state(const DecodeParams& p, const State<DT, D>& st,
                                            float* base, int n, int kg) {
  using Sh = Shape<DT, D>;
  if (n >= p.group) return;
  float* o = base + n * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d0 = (4 * kg + i) * Sh::kTiles;
#pragma unroll
    for (int e = 0; e < Sh::kTiles; e += 4)
      *reinterpret_cast<float4*>(o + d0 + e) = float4{st.o[e][i], st.o[e + 1][i], st.o[e + 2][i], st.o[e + 3][i]};
  }
  if (kg == 0) {
    base[p.group * D + n] = st.m;
    base[p.group * D + p.group + n] = st.l;
  }
}

template <int DT, int D>
__device__ __forceinline__ void write_partial(const DecodeParams& p, const State<DT, D>& st,
                                              int32_t slot, int n, int kg) {
  write_state<DT, D>(p, st, p.ws_partial + (int64_t)slot * p.group * (D + 4), n, kg);
}

// The waves' flat tile ranges: wave w takes [begin(w), begin(w + 1)) with
// begin(w) = floor(total * w / W). total < 2^31 (the host bounds sequences x
// heads x table width) and W < 2^15, so with total = q W + r,
// begin(w) = q w + (r w) / W stays in 32-bit arithmetic (64-bit divisions
// are long software sequences on the GPU).
struct WaveRanges {
  int32_t q, r, W;
  float w_per_tile;
  __device__ __forceinline__ WaveRanges(int32_t total, int32_t W_) : W(W_) {
    q = total / W;
    r = total - q * W;
    w_per_tile = (float)W / (float)max(total, 1);
  }
  __device__ __forceinline__ int32_t begin(int32_t w) const { return q * w + (r * w) / W; }
  __device__ __forceinline__ bool empty(int32_t w) const { return begin(w) == begin(w + 1); }
  // The wave whose range holds tile i: the largest w with begin(w) <= i
  // (an estimate in float, then exact steps).
  __device__ __forceinline__ int32_t owner(int32_t i) const {
    int32_t w = min(max((int32_t)(((float)i + 0.5f) * w_per_tile), 0), W - 1);
    while (w > 0 && begin(w) > i) --w;
    while (w + 1 < W && begin(w + 1) <= i) ++w;
    return w;
  }
};

// Zero output of an empty sequence (all query heads).
template <int DT, int D>
__device__ __forceinline__ void zero_rows(const DecodeParams& p, int32_t s) {
  const int64_t elems = (int64_t)p.num_q_heads * D;
  const int per = 16 / Shape<DT, D>::kElem;
  char* row = reinterpret_cast<char*>(p.out) + (int64_t)s * elems * Shape<DT, D>::kElem;
  for (int64_t e = (int64_t)threadIdx.x * per; e < elems; e += 64 * per)
    *reinterpret_cast<uint4*>(row + e * Shape<DT, D>::kElem) = uint4{0u, 0u, 0u, 0u};
}

// Partial states whose loads one merge thread issues together.
constexpr int kMergeBatch = 4;
// Waves of the merge workgroup: each folds a contiguous quarter of a split
// sequence's partial states, then the first folds the four results in order.
constexpr int kMergeWaves = 4;

// Running fold of partial softmax states for 8 consecutive output values of
// one query head.
struct Fold {
  float mx, den;
  float num[8];
  __device__ __forceinline__ void reset() {
    mx = -INFINITY;
    den = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) num[i] = 0.f;
  }
  // Add a state (max m, sum l, unnormalised values o) to the fold: the
  // online-softmax rescale to the larger of the two maxima.
  __device__ __forceinline__ void add(float m, float l, const float (&o)[8]) {
    const float m_new = fmaxf(mx, m);
    const float so = __builtin_amdgcn_exp2f(mx - m_new);
    const float sk = __builtin_amdgcn_exp2f(m - m_new);
    den = den * so + l * sk;
#pragma unroll
    for (int i = 0; i < 8; ++i) num[i] = num[i] * so + o[i] * sk;
    mx = m_new;
  }
};

// Fold, in order, the partial states that the non-empty waves of [wa, wb)
// hold for the sequence whose units start at `start`: lane values e .. e+7
// (query head h of the group). A wave whose range starts before the
// sequence's units finished a piece of an earlier sequence first and holds
// its state in its second slot, every other wave in its first. The loads of
// kMergeBatch states are issued together.
template <int D>
__device__ __forceinline__ void fold_owners(const DecodeParams& p, const WaveRanges& R, int32_t wa,
                                            int32_t wb, int32_t start, int32_t e, int32_t h,
                                            Fold& f) {
  const int32_t G = p.group;
  const int32_t stride = G * (D + 4);
  int32_t wv = wa;
  while (wv < wb) {
    int32_t slot[kMergeBatch];
    int cnt = 0;
    for (; wv < wb && cnt < kMergeBatch; ++wv) {
      if (R.empty(wv)) continue;
      slot[cnt++] = 2 * wv + (R.begin(wv) < start ? 1 : 0);
    }
    float4 o0[kMergeBatch], o1[kMergeBatch];
    float mk[kMergeBatch], lk[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (k < cnt) {
        const float* base = p.ws_partial + (int64_t)slot[k] * stride;
        o0[k] = *reinterpret_cast<const float4*>(base + e);
        o1[k] = *reinterpret_cast<const float4*>(base + e + 4);
        mk[k] = base[G * D + h];
        lk[k] = base[G * D + G + h];
      }
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (k < cnt) {
        const float ov[8] = {o0[k].x, o0[k].y, o0[k].z, o0[k].w, o1[k].x, o1[k].y, o1[k].z, o1[k].w};
        f.add(mk[k], lk[k], ov);
      }
    }
  }
}

// Normalised values e .. e+7 of the output rows starting at out_row.
template <int DT, int D>
__device__ __forceinline__ void store_folded(const DecodeParams& p, const Fold& f, int64_t out_row,
                                             int32_t e) {
  const float inv = 1.0f / f.den;
  if constexpr (DT == PKV_BF16) {
    uint32_t wd[4];
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
      bf16x2 v = {(__bf16)(f.num[i] * inv), (__bf16)(f.num[i + 1] * inv)};
      wd[i / 2] = __builtin_bit_cast(uint32_t, v);
    }
    *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(p.out) + out_row + e) =
        uint4{wd[0], wd[1], wd[2], wd[3]};
  } else {
    float* o = reinterpret_cast<float*>(p.out) + out_row + e;
    *reinterpret_cast<float4*>(o) = float4{f.num[0] * inv, f.num[1] * inv, f.num[2] * inv, f.num[3] * inv};
    *reinterpret_cast<float4*>(o + 4) = float4{f.num[4] * inv, f.num[5] * inv, f.num[6] * inv, f.num[7] * inv};
  }
}

// Fold the partial states of sequence s, KV head g (units start..last, its
// tiles first..last) and write the normalised output. The owners of the
// sequence's tiles are waves w0..w1 (in token order); merge wave k folds the
// contiguous quarter [w0 + k*n/4, w0 + (k+1)*n/4) of them in order, each lane
// owning 8 consecutive output values of one query head and issuing the loads
// of kMergeBatch states together; merge wave 0 then folds the four results
// in order through LDS. The order is fixed, so the result is deterministic.
template <int DT, int D>
__device__ void merge_sequence(const DecodeParams& p, int32_t s, int32_t g, int32_t start,
                               int32_t first, int32_t last, const WaveRanges& R) {
  __shared__ float xs[kMergeWaves - 1][10][64];
  const int lane = threadIdx.x & 63;
  const int mw = threadIdx.x >> 6;
  const int32_t G = p.group;
  const int64_t out_row = ((int64_t)s * p.num_q_heads + (int64_t)g * G) * D;
  const int32_t w0 = R.owner(first), w1 = R.owner(last);
  const int32_t nw = w1 - w0 + 1;
  const int32_t wa = w0 + (mw * nw) / kMergeWaves;
  const int32_t wb = w0 + ((mw + 1) * nw) / kMergeWaves;
  for (int32_t e0 = 0; e0 < G * D; e0 += 512) {
    const int32_t e = e0 + 8 * lane;
    const bool act = e < G * D;
    const int32_t h = act ? e / D : 0;
    Fold f;
    f.reset();
    if (act) fold_owners<D>(p, R, wa, wb, start, e, h, f);
    if (mw > 0) {
      xs[mw - 1][0][lane] = f.mx;
      xs[mw - 1][1][lane] = f.den;
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[mw - 1][2 + i][lane] = f.num[i];
    }
    __syncthreads();
    if (mw == 0 && act) {
#pragma unroll
      for (int k = 0; k < kMergeWaves - 1; ++k) {
        float ov[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] = xs[k][2 + i][lane];
        // (an empty quarter has max -inf and sum 0: weight 0)
        if (xs[k][0][lane] != -INFINITY) f.add(xs[k][0][lane], xs[k][1][lane], ov);
      }
      store_folded<DT, D>(p, f, out_row, e);
    }
    __syncthreads();   // the LDS slots are reused by the next chunk of values
  }
}

// Merge of sequence s, KV head g in shared-prefix mode: the prefix parts in
// position order, then the suffix's
// states in token order (units a..b of the head; none when a == b): the state
// in ws_whole when one wave held the whole suffix, else the owners' partial
// states, a contiguous quarter per merge wave as in merge_sequence. Merge wave
// 0 folds the prefix before its quarter; the order is fixed.
template <int DT, int D>
__device__ void merge_with_prefix(const DecodeParams& p, int32_t s, int32_t g, int32_t a,
                                  int32_t b, int32_t per_head, const WaveRanges& R) {
  __shared__ float xs[kMergeWaves - 1][10][64];
  const int lane = threadIdx.x & 63;
  const int mw = threadIdx.x >> 6;
  const int32_t G = p.group;
  const int64_t out_row = ((int64_t)s * p.num_q_heads + (int64_t)g * G) * D;
  int32_t start = 0, w0 = 0, nw = 0;
  bool whole = false;
  if (a < b) {
    start = g * per_head + a;
    w0 = R.owner(start + p.piece_cost);
    const int32_t w1 = R.owner(g * per_head + b - 1);
    whole = w0 == w1;
    nw = whole ? 0 : w1 - w0 + 1;
  }
  const int32_t wa = w0 + (mw * nw) / kMergeWaves;
  const int32_t wb = w0 + ((mw + 1) * nw) / kMergeWaves;
  for (int32_t e0 = 0; e0 < G * D; e0 += 512) {
    const int32_t e = e0 + 8 * lane;
    const bool act = e < G * D;
    const int32_t h = act ? e / D : 0;
    Fold f;
    f.reset();
    if (act && mw == 0) {
      const float* row = p.pstate + ((int64_t)s * p.num_q_heads + g * G + h) * (D + 4);
      for (int32_t k = 0; k < p.pparts; ++k) {
        const float* src = row + k * p.pstride;
        const float4 o0 = *reinterpret_cast<const float4*>(src + (e - h * D));
        const float4 o1 = *reinterpret_cast<const float4*>(src + (e - h * D) + 4);
        const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        f.add(src[D], src[D + 1], ov);
      }
      if (whole) {
        const float* base = p.ws_whole + ((int64_t)s * p.num_kv_heads + g) * G * (D + 4);
        const float4 o0 = *reinterpret_cast<const float4*>(base + e);
        const float4 o1 = *reinterpret_cast<const float4*>(base + e + 4);
        const float ov[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        f.add(base[G * D + h], base[G * D + G + h], ov);
      }
    }
    if (act && nw > 0) fold_owners<D>(p, R, wa, wb, start, e, h, f);
    if (mw > 0) {
      xs[mw - 1][0][lane] = f.mx;
      xs[mw - 1][1][lane] = f.den;
#pragma unroll
      for (int i = 0; i < 8; ++i) xs[mw - 1][2 + i][lane] = f.num[i];
    }
    __syncthreads();
    if (mw == 0 && act) {
#pragma unroll
      for (int k = 0; k < kMergeWaves - 1; ++k) {
        float ov[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) ov[i] = xs[k][2 + i][lane];
        // (an empty quarter has max -inf and sum 0: weight 0)
        if (xs[k][0][lane] != -INFINITY) f.add(xs[k][0][lane], xs[k][1][lane], ov);
      }
      store_folded<DT, D>(p, f, out_row, e);
    }
    __syncthreads();   // the LDS slots are reused by the next chunk of values
  }
}

// Query column blocks of a prefix wave: kPrefixNG groups of 16 MFMA columns
// (16 / G sequences x the G query heads of one KV head each).
constexpr int kPrefixNG = 2;
// Bytes between K rows in a prefix wave's LDS tiles: 32 bytes of padding
// keep the operand reads of 16 rows off shared banks.
constexpr int kPrefixPad = 32;

// LDS of a prefix wave: the K rows of two pairs of tiles.
template <int D>
constexpr size_t prefix_lds_bytes() {
  return (size_t)4 * 16 * (D * 2 + kPrefixPad);
}

// A pair of prefix tiles (32 positions) in registers, K and V alike in the
// row-major layout of the V operand of tile_attn.h: lane (n, kg) holds
// bytes [n*R/16, (n+1)*R/16) of rows 4kg .. 4kg+3 of each tile, so each
// load instruction reads 4 whole rows. (The K operand layout, 16 rows x 64
// bytes per instruction, takes the vector memory pipeline about four times
// as long per byte, so the K rows go to the MFMA layout through LDS.)
template <int D>
struct PrefixPair {
  static constexpr int W = Shape<PKV_BF16, D>::kVWords;
  uint32_t k[2][4][W];
  uint32_t v[2][4][W];
};

template <int D>
__device__ __forceinline__ void prefix_load(PrefixPair<D>& t, int h, const char* kb,
                                            const char* vb, uint32_t off) {
  constexpr int R = Shape<PKV_BF16, D>::kRow;
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<PrefixPair<D>::W, false>(t.k[h][j], kb + off + j * R);
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<PrefixPair<D>::W, false>(t.v[h][j], vb + off + j * R);
}

// K rows of a pair into LDS (row r of tile h at (16h + r) * pitch).
template <int D>
__device__ __forceinline__ void prefix_store_k(char* kl, const PrefixPair<D>& t, int n, int kg) {
  constexpr int R = Shape<PKV_BF16, D>::kRow;
  constexpr int pitch = R + kPrefixPad;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      char* dst = kl + (16 * h + 4 * kg + j) * pitch + n * (R / 16);
      if constexpr (PrefixPair<D>::W == 4)
        *reinterpret_cast<uint4*>(dst) = uint4{t.k[h][j][0], t.k[h][j][1], t.k[h][j][2], t.k[h][j][3]};
      else
        *reinterpret_cast<uint2*>(dst) = uint2{t.k[h][j][0], t.k[h][j][1]};
    }
}

// One step of a prefix wave over a pair of tiles (32 positions; the second
// tile's positions are dropped when `both` is false) for NG column groups:
//   scores S = K Q^T (16x16x32 MFMAs, the K operand read from the LDS rows);
//   weights against a reference max per column that moves only when a score
//     passes it by more than 2^8 (log2 units: 8), so the common step needs
//     no cross-lane reduction: each lane keeps its own partial sum (st.l),
//     reduced over the column's four lanes at the end, and the weights stay
//     below 2^8 (any reference gives the same softmax once the sum divides
//     it out);
//   O^T += V^T P^T over all 32 positions in one 16x16x32 MFMA per output
//     tile: lane (n, kg) holds the weights of rows 4kg..4kg+3 of both tiles
//     (the C layout of the score MFMAs), which is the B layout when the
//     contraction index runs over tile 0's four rows, then tile 1's, in each
//     group of eight; the V operand packs the same rows' values.
template <int D, int NG>
__device__ __forceinline__ void prefix_step(State<PKV_BF16, D> (&st)[NG], const char* kl,
                                            const PrefixPair<D>& t, const QOp<PKV_BF16, D> (&qv)[NG],
                                            float scale_log2, bool both, int n, int kg) {
  using Sh = Shape<PKV_BF16, D>;
  constexpr int pitch = Sh::kRow + kPrefixPad;
  f32x4 s[2][NG];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint4 ka[Sh::kKLoads];
#pragma unroll
    for (int c = 0; c < Sh::kKLoads; ++c)
      ka[c] = *reinterpret_cast<const uint4*>(kl + (16 * h + n) * pitch + 64 * c + 16 * kg);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      s[h][gi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < Sh::kKLoads; ++c)
        s[h][gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, ka[c]),
                                                           __builtin_bit_cast(bf16x8, qv[gi].c[c]),
                                                           s[h][gi], 0, 0, 0);
    }
  }
  float x[NG][8], lmax[NG];
  bool move = false;
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[gi][i] = s[0][gi][i] * scale_log2;
      x[gi][4 + i] = both ? s[1][gi][i] * scale_log2 : -INFINITY;
    }
    lmax[gi] = fmaxf(fmaxf(fmaxf(x[gi][0], x[gi][1]), fmaxf(x[gi][2], x[gi][3])),
                     fmaxf(fmaxf(x[gi][4], x[gi][5]), fmaxf(x[gi][6], x[gi][7])));
    move = move || lmax[gi] > st[gi].m + 8.0f;
  }
  if (__ballot(move) != 0) {
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      const float m_new = fmaxf(st[gi].m, wave_max_kg(lmax[gi]));
      const float alpha = __builtin_amdgcn_exp2f(st[gi].m - m_new);
      st[gi].l *= alpha;
#pragma unroll
      for (int e = 0; e < Sh::kTiles; ++e) st[gi].o[e] *= alpha;
      st[gi].m = m_new;
    }
  }
  bf16x8 b[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float p[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) p[i] = bf16_round(__builtin_amdgcn_exp2f(x[gi][i] - st[gi].m));
    st[gi].l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
#pragma unroll
    for (int i = 0; i < 8; ++i) b[gi][i] = (__bf16)p[i];
  }
#pragma unroll
  for (int e = 0; e < Sh::kTiles; ++e) {
    // element e of each of the 4 rows this lane holds of each tile
    const int w = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    uint4 a;
    a.x = __builtin_amdgcn_perm(t.v[0][1][w], t.v[0][0][w], sel);
    a.y = __builtin_amdgcn_perm(t.v[0][3][w], t.v[0][2][w], sel);
    a.z = __builtin_amdgcn_perm(t.v[1][1][w], t.v[1][0][w], sel);
    a.w = __builtin_amdgcn_perm(t.v[1][3][w], t.v[1][2][w], sel);
    const bf16x8 av = __builtin_bit_cast(bf16x8, a);
#pragma unroll
    for (int gi = 0; gi < NG; ++gi)
      st[gi].o[e] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, b[gi], st[gi].o[e], 0, 0, 0);
  }
}

// Shared-prefix mode: the prefix attention of one work unit (KV head g,
// column block c, part k of the prefix blocks), run by workgroup
// num_waves + pj of the split kernel beside the decode waves. The prefix
// blocks are the first `skip` entries of row 0 of the table (every row holds
// the same ones); part k covers blocks [k * skip / pparts, (k + 1) * skip /
// pparts), at least one. The wave attends them for all its columns at once,
// a pair of tiles per step, and writes each query row's softmax state to the
// part's slice of pstate. The K rows of a pair, loaded a step earlier, go
// through LDS into the MFMA layout; two pairs are in flight. Units are
// numbered head first and dealt to the XCDs in contiguous eighths, like the
// decode waves, so one XCD's L2 serves the prefix blocks of its heads;
// prefix tiles are read by many waves: cached loads.
template <int D>
__device__ __forceinline__ void prefix_wave(const DecodeParams& p, int32_t pj, char* lds) {
  using Sh = Shape<PKV_BF16, D>;
  constexpr int NG = kPrefixNG;
  constexpr int pitch = Sh::kRow + kPrefixPad;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t per_xcd = p.pwaves / kXcds;
  const int32_t unit = (pj % kXcds) * per_xcd + pj / kXcds;
  if (unit >= p.punits) return;
  const int32_t part = unit % p.pparts;
  const int32_t gc = unit / p.pparts;
  const int32_t c = gc % p.pcols;
  const int32_t g = gc / p.pcols;
  const int32_t G = p.group;
  const int32_t tpg = 16 / G;                       // sequences per 16 columns
  const int32_t b0 = (int32_t)((int64_t)part * p.skip / p.pparts);
  const int32_t nt = (int32_t)((int64_t)(part + 1) * p.skip / p.pparts) - b0;
  // column n of group gi: sequence (c * NG + gi) * tpg + n / G, head n % G
  const int32_t ts = n / G;
  const int32_t h = n - ts * G;
  QOp<PKV_BF16, D> qv[NG];
  State<PKV_BF16, D> st[NG];
  int64_t row[NG];
  bool valid[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const int32_t sq = (c * NG + gi) * tpg + ts;
    valid[gi] = ts < tpg && sq < p.num_seqs;
    row[gi] = (int64_t)sq * p.num_q_heads + (int64_t)g * G + h;
    load_query<PKV_BF16, D>(qv[gi], reinterpret_cast<const char*>(p.q) + row[gi] * Sh::kRow,
                            valid[gi], kg);
    st[gi].reset();
  }
  const uint32_t off = v_lane_offset<PKV_BF16, D>(n, kg);
  char* kl[2] = {lds, lds + 32 * pitch};
  // The part's tiles in chunks of up to 64: the chunk's block ids in a
  // register (lane t: tile t of the chunk), read out per tile; tiles past
  // the chunk's end repeat its last tile (loaded, never used). The tile
  // loads are the only memory loads of the loop, so the compiler's wait
  // counts stay exact.
  for (int32_t cb = 0; cb < nt; cb += 64) {
    const int32_t cn = min(64, nt - cb);
    const int32_t np = (cn + 1) >> 1;               // pairs of the chunk
    const int32_t ids = lane < cn ? p.block_table[b0 + cb + lane] : 0;
    auto load = [&](PrefixPair<D>& t, int32_t q) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        int32_t id = __builtin_amdgcn_readlane(ids, min(2 * q + hh, cn - 1));
        id = (uint32_t)id < (uint32_t)p.num_blocks ? id : 0;
        const int64_t tb = ((int64_t)id * p.num_kv_heads + g) * Sh::kTileBytes;
        prefix_load<D>(t, hh, p.k_cache + tb, p.v_cache + tb, off);
      }
    };
    PrefixPair<D> buf[2];
    load(buf[0], 0);
    __builtin_amdgcn_sched_barrier(0);
    load(buf[1], 1);
    __builtin_amdgcn_sched_barrier(0);
    prefix_store_k<D>(kl[0], buf[0], n, kg);
    int32_t q = 0;
    for (; q + 2 <= np; q += 2) {
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        // pair q + u: K rows in kl[u], V rows in buf[u]
        prefix_step<D, NG>(st, kl[u], buf[u], qv, p.scale_log2, 2 * (q + u) + 1 < cn, n, kg);
        prefix_store_k<D>(kl[1 - u], buf[1 - u], n, kg);
        load(buf[u], q + u + 2);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (q < np) prefix_step<D, NG>(st, kl[0], buf[0], qv, p.scale_log2, 2 * q + 1 < cn, n, kg);
  }
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    const float l = wave_sum_kg(st[gi].l);
    if (!valid[gi]) continue;
    float* o = p.pstate + part * p.pstride + row[gi] * (D + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = (4 * kg + i) * Sh::kTiles;
#pragma unroll
      for (int e = 0; e < Sh::kTiles; e += 4)
        *reinterpret_cast<float4*>(o + d0 + e) =
            float4{st[gi].o[e][i], st[gi].o[e + 1][i], st[gi].o[e + 2][i], st[gi].o[e + 3][i]};
    }
    if (kg == 0) {
      o[D] = st[gi].m;
      o[D + 1] = l;
    }
  }
}

// Piece of a wave's range: the tiles of one (sequence, KV head) it covers in
// one round. Kept in LDS while the round streams.
struct Piece {
  int32_t s, g;        // sequence and KV head
  int32_t j0;          // first block (of the sequence) in the piece
  int32_t kstart;      // first flat tile index of the piece in the round
  int32_t kend;        // one past its last flat tile index
  int32_t len;         // clamped sequence length (tokens)
  int32_t flags;       // kFinal | kWhole | kFirst | kCont
  int32_t pad;
};
constexpr int32_t kFinal = 1;  // the wave's work on this sequence ends here
constexpr int32_t kWhole = 2;  // the wave holds the whole sequence: store the output
constexpr int32_t kFirst = 4;  // the sequence is the wave's first: partial state in slot 2w
constexpr int32_t kCont = 8;   // continues the previous round's last piece: keep the state
constexpr int32_t kTail = 16;  // holds the sequence's last block

constexpr int kTilesPerRound = 512;
constexpr int kPiecesPerRound = 16;

// Split-KV decode. Each wave streams the tiles of its range as one flat list
// (staged in LDS per round with the block ids resolved to pool tiles), so
// the K/V load pipeline runs across sequence boundaries without draining;
// the query rows of the round's pieces are staged in LDS too. The loop body
// keeps the loads in issue order (the compiler's wait counts stay exact);
// the last DEPTH-1 tiles of a round are computed in an epilogue without
// further loads.
template <int DT, int D, int DEPTH>
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(DEPTH <= 4 ? 2 : 1)))
decode_split_kernel(DecodeParams p) {
  using Sh = Shape<DT, D>;
  extern __shared__ __align__(16) char lds[];
  int32_t* tiles = reinterpret_cast<int32_t*>(lds);                       // [kTilesPerRound]
  int32_t* tile_head = tiles + kTilesPerRound;                            // [kTilesPerRound]
  Piece* pieces = reinterpret_cast<Piece*>(tile_head + kTilesPerRound);   // [kPiecesPerRound]
  int32_t* tails = reinterpret_cast<int32_t*>(pieces + kPiecesPerRound);  // [kPiecesPerRound]
  char* qlds = reinterpret_cast<char*>(tails + kPiecesPerRound);          // [kq][G * kRow]
  const int32_t hw = blockIdx.x;
  if (hw >= p.num_waves) {   // shared-prefix mode: a prefix workgroup
    if constexpr (DT == PKV_BF16) prefix_wave<D>(p, hw - p.num_waves, lds);
    return;
  }
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t per_xcd = p.num_waves / kXcds;
  const int32_t w = (hw % kXcds) * per_xcd + hw / kXcds;
  const int32_t G = p.group;
  const int32_t qbytes = G * Sh::kRow;       // one piece's query rows

  // Total tiles per head: scan the block counts in chunks of 64 sequences.
  // The first chunk's scan is kept: with up to 64 sequences it also serves
  // to locate the wave's first tile without reading the lengths again.
  // The partition is over units, not tiles: a sequence with blocks counts
  // piece_cost units before its blocks, the time a wave spends opening and
  // closing a piece (staging its query rows, writing its state) measured in
  // tiles streamed. A wave whose units are the cost units of a sequence takes
  // no tile for them.
  int32_t per_head = 0;
  int32_t nv0 = 0, incl0 = 0, len0 = 0;
  for (int32_t base = 0; base < p.num_seqs; base += 64) {
    const int32_t sq = base + lane;
    const int32_t len = sq < p.num_seqs ? seq_len_clamped(p, sq) : 0;
    const int32_t nb = (len + 15) >> 4;
    const int32_t nv = nb > 0 ? nb + p.piece_cost : 0;
    const int32_t incl = wave_incl_scan(nv);
    if (base == 0) {
      nv0 = nv;
      incl0 = incl;
      len0 = len;
    }
    if (hw == 0) {
      if (sq < p.num_seqs) p.ws_prefix[sq + 1] = per_head + incl;
      if (base == 0 && lane == 0) p.ws_prefix[0] = 0;
      // Empty sequences own no tile: this wave writes their zero output
      // (the merge writes it in shared-prefix mode).
      uint64_t empty = p.pstate != nullptr ? 0 : __ballot(sq < p.num_seqs && len == 0);
      while (empty) {
        const int li = __builtin_ctzll(empty);
        empty &= empty - 1;
        zero_rows<DT, D>(p, base + li);
      }
    }
    per_head += __builtin_amdgcn_readlane(incl, 63);
  }
  const WaveRanges R(per_head * p.num_kv_heads, p.num_waves);
  const int32_t i0 = R.begin(w);
  const int32_t i1 = R.begin(w + 1);
  if (i0 >= i1) return;

  // Locate the (head, sequence) holding unit i0.
  int32_t g = i0 / per_head;
  const int32_t r = i0 - g * per_head;
  int32_t s = 0, seq_start = 0, len_s = 0;
  {
    int32_t start = 0;
    for (int32_t base = 0; base < p.num_seqs; base += 64) {
      int32_t nv = nv0, incl = incl0, len = len0;
      if (base > 0) {
        const int32_t sq = base + lane;
        len = sq < p.num_seqs ? seq_len_clamped(p, sq) : 0;
        const int32_t nb = (len + 15) >> 4;
        nv = nb > 0 ? nb + p.piece_cost : 0;
        incl = wave_incl_scan(nv);
      }
      const uint64_t hit = __ballot(start + incl > r);
      if (hit) {
        const int li = __builtin_ctzll(hit);
        s = base + li;
        seq_start = start + __builtin_amdgcn_readlane(incl - nv, li);
        len_s = __builtin_amdgcn_readlane(len, li);
        break;
      }
      start += __builtin_amdgcn_readlane(incl, 63);
    }
  }
  // next unit of sequence s to take: its cost units, then block u - piece_cost
  int32_t u = r - seq_start;

  const uint32_t k_off = k_lane_offset<DT, D>(n, kg);
  const uint32_t v_off = v_lane_offset<DT, D>(n, kg);
  const char* kpool = p.k_cache;
  const char* vpool = p.v_cache;

  QOp<DT, D> qv[1];
  State<DT, D> st[1];
  int64_t i = i0;
  bool first = true;                     // no piece finished yet: partial goes to slot 2w
  bool cont = false;                     // the next round continues an open piece
  int32_t open_j0 = 0;                   // first block the wave took of the open sequence
  while (i < i1) {
    // ---- build a round: pieces, their tiles and their query rows -------
    int32_t nt = 0, np = 0, ntail = 0;
    __syncthreads();
    while (i < i1 && nt < kTilesPerRound && np < p.pieces_per_round) {
      const int32_t nb_s = (len_s + 15) >> 4;
      const int32_t nv_s = nb_s > 0 ? nb_s + p.piece_cost : 0;
      if (u < p.piece_cost && nv_s > 0) {     // the sequence's cost units: no tile
        const int32_t c = (int32_t)min((int64_t)(p.piece_cost - u), i1 - i);
        u += c;
        i += c;
      }
      const int32_t j = u - p.piece_cost;     // next block of sequence s
      const int32_t cnt = u < p.piece_cost ? 0
          : (int32_t)min((int64_t)min(nb_s - j, kTilesPerRound - nt), i1 - i);
      if (cnt > 0) {
        const bool fin = j + cnt == nb_s || i + cnt == i1;
        const bool tail = j + cnt == nb_s;
        if (!(cont && np == 0)) open_j0 = j;
        if (lane == 0) {
          Piece pc;
          pc.s = s;
          pc.g = g;
          pc.j0 = j;
          pc.kstart = nt;
          pc.kend = nt + cnt;
          pc.len = len_s;
          pc.flags = (fin ? kFinal : 0) | (open_j0 == 0 && tail ? kWhole : 0) |
                     (first ? kFirst : 0) | (cont && np == 0 ? kCont : 0) | (tail ? kTail : 0);
          pc.pad = 0;
          pieces[np] = pc;
          if (tail) tails[ntail] = np;
        }
        ntail += tail ? 1 : 0;
        // For now each tile holds its index in the block table (and its KV
        // head); the ids are read below, for all pieces at once.
        const int32_t tbase = s * p.max_blocks + p.skip + j;
        for (int32_t t = lane; t < cnt; t += 64) {
          tiles[nt + t] = tbase + t;
          tile_head[nt + t] = g;
        }
        ++np;
        nt += cnt;
        i += cnt;
        u += cnt;
        cont = !fin;
        if (fin) first = false;
      }
      if (u >= nv_s) {  // next sequence, wrapping to the next head
        u = 0;
        if (++s == p.num_seqs) {
          s = 0;
          ++g;
        }
        if (i < i1) {
          // lengths of the first 64 sequences are still in the scan registers
          len_s = s < 64 ? __builtin_amdgcn_readlane(len0, s) : seq_len_uniform(p, s);
        }
      }
    }
    // (the range ended inside a sequence's cost units: nothing left to stream)
    if (nt == 0) break;
    __syncthreads();
    // Staging, in batches: (a) read from LDS what the batch's loads need,
    // (b) issue all its global loads -- in the first batch the block ids of
    // every tile of the round, and in every batch up to 64*kQ chunks of the
    // pieces' query rows (heads g*G .. g*G+G-1 of the sequence, contiguous)
    // and, in append mode, up to 64*kN chunks of the new K/V rows -- (c) wait
    // once, (d) write LDS and store the new rows. One memory round trip per
    // batch; a round needs one batch unless it holds more than 64*kQ query
    // chunks or 64*kN new-row chunks.
    {
      constexpr int kB = kTilesPerRound / 64;     // block ids per lane
      constexpr int kQ = Sh::kRow > 256 ? 2 : 4;  // query chunks per lane and batch
      constexpr int kCpr = Sh::kRow / 16;         // 16-byte chunks per K or V row
      constexpr int kN = 4;                       // new-row chunks per lane and batch
      // (a native vector type: the HIP uint4 class copies through memcpy,
      // which would put these registers in scratch memory)
      typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
      const int32_t cpp = qbytes / 16;            // query chunks per piece
      const int32_t nq = np * cpp;
      // new-row chunk c: chunk o of row kv (0 = K, 1 = V) of tail piece c / (2 kCpr)
      const int32_t nn = p.k_new != nullptr ? ntail * 2 * kCpr : 0;
      for (int32_t c0 = 0, n0 = 0; c0 == 0 || c0 < nq || n0 < nn; c0 += 64 * kQ, n0 += 64 * kN) {
        const bool first_batch = c0 == 0;
        // (a) addresses
        int32_t tix[kB];
        if (first_batch) {
#pragma unroll
          for (int m = 0; m < kB; ++m) {
            const int32_t k = lane + 64 * m;
            tix[m] = k < nt ? tiles[k] : 0;
          }
        }
        const char* qsrc[kQ];
        int32_t qdst[kQ];
#pragma unroll
        for (int m = 0; m < kQ; ++m) {
          const int32_t c = c0 + lane + 64 * m;
          const int32_t pi = c < nq ? c / cpp : 0;
          const int32_t o = c - pi * cpp;
          const Piece& P = pieces[pi];
          qsrc[m] = reinterpret_cast<const char*>(p.q) +
                    ((int64_t)P.s * p.num_q_heads + (int64_t)P.g * G) * Sh::kRow + 16 * o;
          qdst[m] = pi * qbytes + 16 * o;
        }
        const char* nsrc[kN];
        int32_t nlast[kN], nrow[kN];   // tile index of the row's block; byte offset in the tile
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          const int32_t c = n0 + lane + 64 * m;
          const int32_t ti = c < nn ? c / (2 * kCpr) : 0;
          const int32_t r = c - ti * 2 * kCpr;
          const int32_t kv = r >= kCpr ? 1 : 0;
          const int32_t o = r - kv * kCpr;
          const Piece& P = pieces[c < nn ? tails[ti] : 0];
          nsrc[m] = (kv ? p.v_new : p.k_new) + (int64_t)P.s * p.new_stride +
                    (int64_t)P.g * Sh::kRow + 16 * o;
          nlast[m] = P.kend - 1;
          // bit 30 marks a V row (the offset itself is below 2^13)
          nrow[m] = (((P.len - 1) & 15) * Sh::kRow + 16 * o) | (kv << 30);
        }
        __builtin_amdgcn_sched_barrier(0);
        // (b) loads
        int32_t bid[kB];
        if (first_batch) {
#pragma unroll
          for (int m = 0; m < kB; ++m)
            bid[m] = lane + 64 * m < nt ? p.block_table[tix[m]] : 0;
        }
        u32x4 qc[kQ], nc[kN];
#pragma unroll
        for (int m = 0; m < kQ; ++m)
          if (c0 + lane + 64 * m < nq) qc[m] = *reinterpret_cast<const u32x4*>(qsrc[m]);
#pragma unroll
        for (int m = 0; m < kN; ++m)
          if (n0 + lane + 64 * m < nn) nc[m] = *reinterpret_cast<const u32x4*>(nsrc[m]);
        __builtin_amdgcn_sched_barrier(0);
        // (d) LDS writes: pool tile of every tile of the round, query rows
        if (first_batch) {
#pragma unroll
          for (int m = 0; m < kB; ++m) {
            const int32_t k = lane + 64 * m;
            if (k < nt)
              tiles[k] = ((uint32_t)bid[m] < (uint32_t)p.num_blocks ? bid[m] : 0) * p.num_kv_heads +
                         tile_head[k];
          }
        }
#pragma unroll
        for (int m = 0; m < kQ; ++m)
          if (c0 + lane + 64 * m < nq) *reinterpret_cast<u32x4*>(qlds + qdst[m]) = qc[m];
        // The new rows go to position len - 1 of their sequence: row
        // (len - 1) % 16 of the tail piece's last tile, unless that tile is
        // in block 0 (an id outside the pool, or the null block, which is
        // never written). The tile loads of the round come after these
        // stores in this wave's program order and read the same addresses,
        // so they return the new rows; no other wave reads this
        // (block, KV head).
        char* ndst[kN];
#pragma unroll
        for (int m = 0; m < kN; ++m) {
          ndst[m] = nullptr;
          if (n0 + lane + 64 * m < nn) {
            const int32_t t = tiles[nlast[m]];
            if (t >= p.num_kv_heads)
              ndst[m] = const_cast<char*>((nrow[m] >> 30) ? p.v_cache : p.k_cache) +
                        (int64_t)t * Sh::kTileBytes + (nrow[m] & ((1 << 30) - 1));
          }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < kN; ++m)
          if (ndst[m] != nullptr) *reinterpret_cast<u32x4*>(ndst[m]) = nc[m];
      }
    }
    __syncthreads();

    // ---- stream the round's tiles ---------------------------------------
    int32_t pc = -1, kend = 0, j0 = 0, kstart = 0, plen = 0, pflags = 0, ps = 0, pg = 0;
    auto tile_ptr = [&](int32_t k) -> int64_t {
      return (int64_t)__builtin_amdgcn_readfirstlane(tiles[min(k, nt - 1)]) * Sh::kTileBytes;
    };
    // One tile: open the next piece at its first tile, attend, close the
    // piece at its last tile.
    auto step = [&](Tile<DT, D>& tl, int32_t k) {
      if (k == kend) {
        ++pc;
        const Piece& P = pieces[pc];
        ps = __builtin_amdgcn_readfirstlane(P.s);
        pg = __builtin_amdgcn_readfirstlane(P.g);
        j0 = __builtin_amdgcn_readfirstlane(P.j0);
        kstart = __builtin_amdgcn_readfirstlane(P.kstart);
        kend = __builtin_amdgcn_readfirstlane(P.kend);
        plen = __builtin_amdgcn_readfirstlane(P.len);
        pflags = __builtin_amdgcn_readfirstlane(P.flags);
        if (!(pflags & kCont)) {
          const char* qrow = qlds + pc * qbytes + n * Sh::kRow;
#pragma unroll
          for (int c = 0; c < Sh::kKLoads; ++c)
            qv[0].c[c] = n < G ? *reinterpret_cast<const uint4*>(qrow + 64 * c + 16 * kg)
                               : uint4{0u, 0u, 0u, 0u};
          st[0].reset();
        }
      }
      const int32_t t0 = 16 * (j0 + k - kstart);
      const int32_t end = min(t0 + 16, plen);   // valid positions [t0, end)
      const int lim[1] = {end - 1};
      attend_tile<DT, D, 1>(st, tl, qv, p.scale_log2, t0, lim, end, end < t0 + 16, kg);
      if (k == kend - 1 && (pflags & kFinal)) {
        if ((pflags & kWhole) && p.pstate != nullptr)
          write_state<DT, D>(p, st[0], p.ws_whole + ((int64_t)ps * p.num_kv_heads + pg) * G * (D + 4),
                             n, kg);
        else if (pflags & kWhole)
          store_row<DT, D>(p.out, (int64_t)ps * p.num_q_heads + pg * G + n, st[0], kg, n < G);
        else
          write_partial<DT, D>(p, st[0], 2 * w + ((pflags & kFirst) ? 0 : 1), n, kg);
      }
    };
    Tile<DT, D> buf[DEPTH];
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) {
      const int64_t t = tile_ptr(u);
      load_tile<DT, D, true>(buf[u], kpool + t, vpool + t, k_off, v_off);
      __builtin_amdgcn_sched_barrier(0);
    }
    int32_t kb = 0;
    for (; kb + DEPTH <= nt; kb += DEPTH) {
#pragma unroll
      for (int u = 0; u < DEPTH; ++u) {
        step(buf[u], kb + u);
        // the next load is always issued (the last tile again past the end)
        const int64_t t = tile_ptr(kb + u + DEPTH);
        load_tile<DT, D, true>(buf[u], kpool + t, vpool + t, k_off, v_off);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
#pragma unroll
    for (int u = 0; u < DEPTH; ++u)
      if (kb + u < nt) step(buf[u], kb + u);
  }
}

// Merge the partial states of every sequence whose tiles were split across
// waves. One workgroup per (sequence, KV head); sequences held by a single wave
// (written directly) and empty sequences (zeroed by the split kernel) are
// skipped.
template <int DT, int D>
__global__ void __launch_bounds__(64 * kMergeWaves)
decode_merge_kernel(DecodeParams p) {
  const int32_t s = blockIdx.x / p.num_kv_heads;
  const int32_t g = blockIdx.x - s * p.num_kv_heads;
  const int32_t per_head = p.ws_prefix[p.num_seqs];
  const int32_t a = p.ws_prefix[s];
  const int32_t b = p.ws_prefix[s + 1];
  if (p.pstate != nullptr) {
    const WaveRanges R(max(per_head, 1) * p.num_kv_heads, p.num_waves);
    merge_with_prefix<DT, D>(p, s, g, a, b, per_head, R);
    return;
  }
  if (a == b) return;
  const WaveRanges R(per_head * p.num_kv_heads, p.num_waves);
  const int32_t start = g * per_head + a;          // the sequence's first (cost) unit
  const int32_t first = start + p.piece_cost;      // its first tile
  const int32_t last = g * per_head + b - 1;       // its last tile
  if (R.owner(first) == R.owner(last)) return;
  merge_sequence<DT, D>(p, s, g, start, first, last, R);
}

// Launch settings, read by every decode call and possibly from several host
// threads: atomics. The wave count is cached per device (0 = not known yet).
constexpr int kMaxDevices = 64;
std::atomic<int> g_waves[kMaxDevices];
std::atomic<int> g_waves_per_cu{0};   // set by decode_set_waves_per_cu; 0 = default
std::atomic<int> g_depth{0};

// Partition units a sequence costs besides its blocks (see the split
// kernel); PKV_DECODE_PIECE_COST overrides it (0..8) for tuning.
std::atomic<int> g_piece_cost{-1};

int decode_piece_cost() {
  int c = g_piece_cost.load(std::memory_order_relaxed);
  if (c < 0) {
    c = 2;
    if (const char* env = getenv("PKV_DECODE_PIECE_COST")) {
      int v = atoi(env);
      if (v >= 0 && v <= 8) c = v;
    }
    g_piece_cost.store(c, std::memory_order_relaxed);
  }
  return c;
}

int decode_depth() {
  int d = g_depth.load(std::memory_order_relaxed);
  if (d == 0) {
    d = 2;
    if (const char* env = getenv("PKV_DECODE_DEPTH")) {
      int v = atoi(env);
      if (v == 2 || v == 4 || v == 8) d = v;
    }
    g_depth.store(d, std::memory_order_relaxed);
  }
  return d;
}

// Dynamic LDS of the split kernel: tile list, pieces, query rows.
template <int DT, int D>
size_t split_lds_bytes(const DecodeParams& prm) {
  return (size_t)kTilesPerRound * 8 + kPiecesPerRound * (sizeof(Piece) + 4) +
         (size_t)prm.pieces_per_round * prm.group * Shape<DT, D>::kRow;
}

template <int DT, int D>
hipError_t launch(const DecodeParams& prm, int phases, hipStream_t stream) {
  size_t lds = split_lds_bytes<DT, D>(prm);
  if (prm.pwaves > 0) lds = std::max(lds, prefix_lds_bytes<D>());   // the prefix waves' query rows
  if (phases & 1) {
  // 512-byte rows (fp32, head_dim 128) only fit two tiles in flight.
  const int depth = Shape<DT, D>::kRow > 256 ? 2 : decode_depth();
  const dim3 grid(prm.num_waves + prm.pwaves);
  if constexpr (Shape<DT, D>::kRow > 256) {
    hipLaunchKernelGGL((decode_split_kernel<DT, D, 2>), grid, dim3(64), lds, stream, prm);
  } else if (depth == 2)
    hipLaunchKernelGGL((decode_split_kernel<DT, D, 2>), grid, dim3(64), lds, stream, prm);
  else if (depth == 8)
    hipLaunchKernelGGL((decode_split_kernel<DT, D, 8>), grid, dim3(64), lds, stream, prm);
  else
    hipLaunchKernelGGL((decode_split_kernel<DT, D, 4>), grid, dim3(64), lds, stream, prm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (phases & 2) {
    hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3(prm.num_seqs * prm.num_kv_heads), dim3(64 * kMergeWaves),
                       0, stream, prm);
    return hipGetLastError();
  }
  return hipSuccess;
}


// Scratch of the no-alloc decode (pkv_paged_attention_decode_noalloc): the
// same bookkeeping and partial states the decode keeps in a caller's
// workspace, in a file-scope device array instead. Every GPU the library runs
// on holds its own copy for the life of the process. In host code `scratch`
// names a host-side stand-in, not device memory: the device address of each
// GPU's copy comes from hipGetSymbolAddress and is the only one ever passed
// to a kernel.
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address per device (nullptr: not looked up yet)

}  // namespace

namespace pkv {

hipError_t decode_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    // with this device current: its own copy of the array
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (ptr == nullptr || (uintptr_t)ptr % 256 != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

void decode_set_waves_per_cu(int per_cu) {
  g_waves_per_cu.store(per_cu, std::memory_order_relaxed);
  for (auto& w : g_waves) w.store(0, std::memory_order_relaxed);   // recomputed on the next call
}

int decode_num_waves() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return -1;
  const int cached = dev < kMaxDevices ? g_waves[dev].load(std::memory_order_relaxed) : 0;
  if (cached > 0) return cached;
  {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    // Three single-wave workgroups per CU: with non-temporal tile loads the
    // llama-shaped batch runs as fast as with two (88.3 vs 88.7 us) and a
    // batch sharing a long prefix runs faster (127 vs 140 us).
    int per_cu = 3;
    if (const char* env = getenv("PKV_DECODE_WAVES_PER_CU")) {
      int v = atoi(env);
      if (v >= 1 && v <= 32) per_cu = v;
    }
    const int set = g_waves_per_cu.load(std::memory_order_relaxed);
    if (set > 0) per_cu = set;
    int w = prop.multiProcessorCount * per_cu;
    w = (w + kXcds - 1) / kXcds * kXcds;
    if (dev < kMaxDevices) g_waves[dev].store(w, std::memory_order_relaxed);
    return w;
  }
}

// Workspace: [block-count prefix sums, num_seqs + 1 int32, padded to 256 B]
// [partial states, 2 per wave].
static size_t prefix_bytes(int32_t num_seqs) {
  return ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim) {
  const size_t prefix = prefix_bytes(num_seqs);
  const size_t group = (size_t)(num_q_heads / num_kv_heads);
  const size_t partial = 2 * (size_t)decode_num_waves() * group * (head_dim + 4) * 4;
  return prefix + partial;
}

// Sequences of one prefix work unit: kPrefixNG groups of 16 / G.
static int32_t prefix_unit_seqs(int32_t group) { return kPrefixNG * (16 / group); }

static hipError_t launch_decode_impl(const DecodeArgs& a, int32_t skip, float* pstate,
                                     int32_t pparts, int phases, hipStream_t stream,
                                     float* whole_states = nullptr) {
  DecodeParams p;
  p.skip = skip;
  p.pstate = pstate;
  p.pparts = pparts;
  p.ws_whole = whole_states;
  p.pstride = (int64_t)a.num_seqs * a.num_q_heads * (a.head_dim + 4);
  p.pwaves = 0;
  p.pcols = 0;
  p.punits = 0;
  if (pstate != nullptr) {
    const int32_t us = prefix_unit_seqs(a.num_q_heads / a.num_kv_heads);
    p.pcols = (a.num_seqs + us - 1) / us;
    p.punits = a.num_kv_heads * p.pcols * pparts;
    p.pwaves = (p.punits + kXcds - 1) / kXcds * kXcds;
  }
  p.k_new = reinterpret_cast<const char*>(a.k_new);
  p.v_new = reinterpret_cast<const char*>(a.v_new);
  p.new_stride = a.new_token_stride * (a.dtype == PKV_F32 ? 4 : 2);
  p.out = a.out;
  p.q = a.q;
  p.k_cache = reinterpret_cast<const char*>(a.k_cache);
  p.v_cache = reinterpret_cast<const char*>(a.v_cache);
  p.block_table = a.block_table;
  p.context_lens = a.context_lens;
  p.ws_prefix = reinterpret_cast<int32_t*>(a.workspace);
  const size_t prefix = prefix_bytes(a.num_seqs);
  p.ws_partial = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + prefix);
  p.num_seqs = a.num_seqs;
  p.num_blocks = a.num_blocks;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.num_waves = decode_num_waves();
  p.piece_cost = decode_piece_cost();
  p.scale_log2 = a.scale * kLog2e;
  {
    // query rows of up to 16 pieces per round, within 16 KiB of LDS
    const int32_t qb = p.group * a.head_dim * (a.dtype == PKV_F32 ? 4 : 2);
    int32_t k = 16384 / qb;
    p.pieces_per_round = k < 2 ? 2 : (k > kPiecesPerRound ? kPiecesPerRound : k);
  }
  if (a.dtype == PKV_BF16) {
    return a.head_dim == 128 ? launch<PKV_BF16, 128>(p, phases, stream)
                             : launch<PKV_BF16, 64>(p, phases, stream);
  }
  return a.head_dim == 128 ? launch<PKV_F32, 128>(p, phases, stream)
                           : launch<PKV_F32, 64>(p, phases, stream);
}

hipError_t launch_decode(const DecodeArgs& a, int phases, hipStream_t stream) {
  return launch_decode_impl(a, 0, nullptr, 0, phases, stream);
}

constexpr int kMaxPrefixParts = 16;

int decode_prefix_parts(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                        int32_t prefix_blocks) {
  // About one prefix wave for every three decode waves (one per CU beside
  // the decode's three), each part at least one block. Every part is one
  // more state for the merge to fold per query row. (The prefix waves' L2
  // reads slow the decode waves beside them, whatever their number: on 128
  // sequences sharing a 2048-token prefix the whole call takes 44.5 us with
  // 2 parts, 45.2 with 4, 51.2 with 8.)
  const int32_t us = prefix_unit_seqs(num_q_heads / num_kv_heads);
  const int64_t base = std::max<int64_t>((int64_t)((num_seqs + us - 1) / us) * num_kv_heads, 1);
  const int64_t target = std::max((int64_t)decode_num_waves() / 3, (int64_t)1);
  int64_t parts = (target + base - 1) / base;
  if (const char* env = getenv("PKV_PREFIX_PARTS")) {  // tuning override
    const int v = atoi(env);
    if (v >= 1 && v <= kMaxPrefixParts) parts = v;
  }
  parts = std::min<int64_t>(parts, std::max(prefix_blocks, 1));
  return (int)std::max<int64_t>(1, std::min<int64_t>(parts, kMaxPrefixParts));
}

hipError_t launch_decode_shared_prefix(const DecodeArgs& a, int32_t skip_blocks,
                                       float* prefix_state, int32_t parts, hipStream_t stream,
                                       float* whole_states) {
  if (skip_blocks < 1 || parts < 1 || parts > skip_blocks || a.dtype != PKV_BF16)
    return hipErrorInvalidValue;
  return launch_decode_impl(a, skip_blocks, prefix_state, parts, 3, stream, whole_states);
}

}  // namespace pkv
