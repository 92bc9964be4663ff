// Paged decode attention for gfx950: one query token per sequence, grouped
// query heads, keys and values gathered through the block table inside the
// kernel ("(2) vLLM Internals: From PagedAttention to Removing
// PagedAttention", section 4.1 "Why It Could Go"; "My Understanding of vLLM
// and PagedAttention", sections "3. PagedAttention CUDA Kernel" and "Step 4 --
// Attention Computation").
//
// Work split (split-KV, balanced): all (KV head g, sequence s, block j) tiles
// form one index space ordered by g, then s, then j. The grid is a fixed
// number W of single-wave workgroups; logical wave w takes the contiguous
// tile range [w*T/W, (w+1)*T/W), T the total tile count, so every wave reads
// the same number of K/V bytes whatever the length mix. Hardware workgroup b
// runs on XCD b % 8; logical waves are numbered so that each XCD owns one
// contiguous eighth of the index space (one KV head when there are 8), which
// keeps blocks shared between sequences (a common prefix) in one XCD's L2.
//
// A wave's range splits into pieces, one per (g, s) it touches. A piece that
// covers a whole sequence writes the final output; any other piece writes
// its partial softmax state (running max, sum, unnormalised output) to one of
// the wave's two workspace slots, and a second kernel merges the partial
// states of each split sequence in token order (deterministic, no atomics).
//
// Per 16-token block and KV head the wave loads the K tile and the V tile
// ([16][head_dim] each, contiguous) straight into registers and runs:
//   S[t][n] = sum_d K[t][d] Q[n][d]           (MFMA, tokens x query heads)
//   online softmax over t per head n         (exp2, cross-lane max/sum)
//   O^T[d][n] += sum_t V[t][d] P[n][t]        (MFMA, head_dim x query heads)
// The G query heads of the group fill G of the 16 MFMA columns; the other
// columns carry zero queries and are never stored. Register layouts (lane l,
// n = l % 16, kg = l / 16):
//   K operand: row t = n of the tile, a 64-byte piece per load (kg picks the
//              16-byte quarter), so each load instruction reads 16 rows x 64 B.
//   S result : lane (n, kg) holds S[4kg + i][n], i = 0..3.
//   V operand: lane reads row 4kg + j (j = 0..3), bytes [n*R/16, (n+1)*R/16)
//              of the R-byte row, so each load instruction reads 4 whole rows.
//   O result : lane (n, kg) holds head n, dims (4kg + i) * (D/16) + e.
#include <cstdlib>

#include "internal.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kXcds = 8;        // workgroups are dealt round-robin over 8 XCDs

template <int DT, int D>
struct Shape {
  static constexpr int kElem = DT == PKV_F32 ? 4 : 2;
  static constexpr int kRow = D * kElem;       // bytes of one token row of one head
  static constexpr int kKLoads = kRow / 64;    // 16-byte K loads per lane per tile
  static constexpr int kVWords = kRow / 64;    // 32-bit V words per lane per row
  static constexpr int kTiles = D / 16;        // 16-row MFMA tiles of head_dim
  static constexpr int kTileBytes = 16 * kRow; // one (block, head) tile
  static constexpr int kDepth = kRow <= 256 ? 4 : 2;  // K/V tiles in flight per wave
};

template <int DT, int D>
struct Tile {
  uint4 k[Shape<DT, D>::kKLoads];
  uint32_t v[4][Shape<DT, D>::kVWords];
};

template <int W>
__device__ __forceinline__ void load_words(uint32_t* dst, const char* p) {
  if constexpr (W == 2) {
    uint2 x = *reinterpret_cast<const uint2*>(p);
    dst[0] = x.x;
    dst[1] = x.y;
  } else {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      uint4 x = *reinterpret_cast<const uint4*>(p + 4 * i);
      dst[i] = x.x;
      dst[i + 1] = x.y;
      dst[i + 2] = x.z;
      dst[i + 3] = x.w;
    }
  }
}

template <int DT, int D>
__device__ __forceinline__ void load_tile(Tile<DT, D>& tl, const char* kb, const char* vb,
                                          uint32_t k_off, uint32_t v_off) {
  using Sh = Shape<DT, D>;
#pragma unroll
  for (int c = 0; c < Sh::kKLoads; ++c)
    tl.k[c] = *reinterpret_cast<const uint4*>(kb + k_off + 64 * c);
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<Sh::kVWords>(tl.v[j], vb + v_off + j * Sh::kRow);
}

__device__ __forceinline__ float wave_max_kg(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  return fmaxf(x, __shfl_xor(x, 32));
}

__device__ __forceinline__ float wave_sum_kg(float x) {
  x += __shfl_xor(x, 16);
  return x + __shfl_xor(x, 32);
}

__device__ __forceinline__ float bf16_round(float x) {
  bf16x2 p = {(__bf16)x, (__bf16)0.0f};
  return (float)p[0];
}

// Running softmax state of one lane: head n = lane % 16.
template <int DT, int D>
struct State {
  float m;                                  // running max of scaled scores (log2 units)
  float l;                                  // running sum of weights
  f32x4 o[Shape<DT, D>::kTiles];            // unnormalised output, see layout above
};

// One 16-token block. `valid` = number of tokens of the block inside the
// context (1..16).
template <int DT, int D>
__device__ __forceinline__ void attend_block(State<DT, D>& st, Tile<DT, D>& tl,
                                             const uint4* qv, float scale_log2, int valid,
                                             int kg) {
  using Sh = Shape<DT, D>;
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if constexpr (DT == PKV_BF16) {
#pragma unroll
    for (int c = 0; c < Sh::kKLoads; ++c)
      s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, tl.k[c]),
                                                  __builtin_bit_cast(bf16x8, qv[c]), s, 0, 0, 0);
  } else {
#pragma unroll
    for (int c = 0; c < Sh::kKLoads; ++c) {
      const float* kf = reinterpret_cast<const float*>(&tl.k[c]);
      const float* qf = reinterpret_cast<const float*>(&qv[c]);
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qf[e], s, 0, 0, 0);
    }
  }
  float x[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) x[i] = s[i] * scale_log2;
  if (valid < 16) {  // wave-uniform: only the last block of a sequence
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (4 * kg + i >= valid) x[i] = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (4 * kg + j >= valid) {
#pragma unroll
        for (int w = 0; w < Sh::kVWords; ++w) tl.v[j][w] = 0u;
      }
  }
  const float bmax = wave_max_kg(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
  const float m_new = fmaxf(st.m, bmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);
  float p[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
  if constexpr (DT == PKV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p[i] = bf16_round(p[i]);  // the weights the MFMA sees
  }
  const float rsum = wave_sum_kg((p[0] + p[1]) + (p[2] + p[3]));
  st.l = st.l * alpha + rsum;
  st.m = m_new;
  if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
    for (int e = 0; e < Sh::kTiles; ++e) st.o[e] *= alpha;
  }
  if constexpr (DT == PKV_BF16) {
    bf16x2 p01 = {(__bf16)p[0], (__bf16)p[1]};
    bf16x2 p23 = {(__bf16)p[2], (__bf16)p[3]};
    uint2 pb = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
    const i16x4 b = __builtin_bit_cast(i16x4, pb);
#pragma unroll
    for (int e = 0; e < Sh::kTiles; ++e) {
      // element e of each of the 4 rows this lane loaded, packed as 4 bf16
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 a;
      a.x = __builtin_amdgcn_perm(tl.v[1][w], tl.v[0][w], sel);
      a.y = __builtin_amdgcn_perm(tl.v[3][w], tl.v[2][w], sel);
      st.o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(i16x4, a), b,
                                                          st.o[e], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < Sh::kTiles; ++e)
        st.o[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(__builtin_bit_cast(float, tl.v[j][e]), p[j],
                                                       st.o[e], 0, 0, 0);
    }
  }
}

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
  float scale_log2;
};

// Blocks of sequence s after clamping its length to the table width.
__device__ __forceinline__ int32_t seq_len_clamped(const DecodeParams& p, int32_t s) {
  int32_t n = p.context_lens[s];
  n = n < 0 ? 0 : n;
  const int32_t cap = p.max_blocks * 16;
  return n > cap ? cap : n;
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
__device__ __forceinline__ void write_output(const DecodeParams& p, const State<DT, D>& st,
                                             int32_t s, int32_t g, int n, int kg) {
  using Sh = Shape<DT, D>;
  if (n >= p.group) return;
  const float inv = 1.0f / st.l;
  const int64_t row = ((int64_t)s * p.num_q_heads + g * p.group + n) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int d0 = (4 * kg + i) * Sh::kTiles;
    if constexpr (DT == PKV_BF16) {
      uint32_t w[Sh::kTiles / 2];
#pragma unroll
      for (int e = 0; e < Sh::kTiles; e += 2) {
        bf16x2 v = {(__bf16)(st.o[e][i] * inv), (__bf16)(st.o[e + 1][i] * inv)};
        w[e / 2] = __builtin_bit_cast(uint32_t, v);
      }
      char* dst = reinterpret_cast<char*>(p.out) + (row + d0) * 2;
      if constexpr (Sh::kTiles == 8) {
        *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
      } else {
        *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
      }
    } else {
      float* dst = reinterpret_cast<float*>(p.out) + row + d0;
#pragma unroll
      for (int e = 0; e < Sh::kTiles; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            float4{st.o[e][i] * inv, st.o[e + 1][i] * inv, st.o[e + 2][i] * inv, st.o[e + 3][i] * inv};
    }
  }
}

template <int DT, int D>
__device__ __forceinline__ void write_partial(const DecodeParams& p, const State<DT, D>& st,
                                              int32_t slot, int n, int kg) {
  using Sh = Shape<DT, D>;
  if (n >= p.group) return;
  float* base = p.ws_partial + (int64_t)slot * p.group * (D + 4);
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
__global__ void __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2)))
decode_split_kernel(DecodeParams p) {
  using Sh = Shape<DT, D>;
  const int lane = threadIdx.x;
  const int n = lane & 15;
  const int kg = lane >> 4;
  const int32_t hw = blockIdx.x;
  const int32_t per_xcd = p.num_waves / kXcds;
  const int32_t w = (hw % kXcds) * per_xcd + hw / kXcds;

  // Total tiles per head: scan the block counts in chunks of 64 sequences.
  int32_t per_head = 0;
  for (int32_t base = 0; base < p.num_seqs; base += 64) {
    const int32_t s = base + lane;
    const int32_t nb = s < p.num_seqs ? (seq_len_clamped(p, s) + 15) >> 4 : 0;
    const int32_t incl = wave_incl_scan(nb);
    if (hw == 0) {
      if (s < p.num_seqs) p.ws_prefix[s + 1] = per_head + incl;
      if (base == 0 && lane == 0) p.ws_prefix[0] = 0;
    }
    per_head += __shfl(incl, 63);
  }
  const int64_t total = (int64_t)per_head * p.num_kv_heads;
  const int64_t i0 = total * w / p.num_waves;
  const int64_t i1 = total * (w + 1) / p.num_waves;
  if (i0 >= i1) return;

  // Locate the (head, sequence) holding tile i0.
  int32_t g = (int32_t)(i0 / per_head);
  const int32_t r = (int32_t)(i0 - (int64_t)g * per_head);
  int32_t s = 0, seq_start = 0;
  {
    int32_t start = 0;
    for (int32_t base = 0; base < p.num_seqs; base += 64) {
      const int32_t sq = base + lane;
      const int32_t nb = sq < p.num_seqs ? (seq_len_clamped(p, sq) + 15) >> 4 : 0;
      const int32_t incl = wave_incl_scan(nb);
      const uint64_t hit = __ballot(start + incl > r);
      if (hit) {
        const int li = __builtin_ctzll(hit);
        s = base + li;
        seq_start = start + __shfl(incl - nb, li);
        break;
      }
      start += __shfl(incl, 63);
    }
  }
  int32_t j0 = r - seq_start;
  int32_t len_s = seq_len_clamped(p, s);
  int32_t nb_s = (len_s + 15) >> 4;

  const uint32_t k_off = (uint32_t)(n * Sh::kRow + kg * 16);
  const uint32_t v_off = (uint32_t)((4 * kg) * Sh::kRow + n * (Sh::kRow / 16));
  const int64_t head_stride = Sh::kTileBytes;
  const int64_t block_stride = (int64_t)p.num_kv_heads * Sh::kTileBytes;

  int64_t i = i0;
  bool first_piece = true;
  while (i < i1) {
    const int32_t j1 = (int32_t)min((int64_t)nb_s, (int64_t)j0 + (i1 - i));
    if (j1 > j0) {
      // Query operand: head g*G + n for n < G, zero otherwise.
      uint4 qv[Sh::kKLoads];
      if (n < p.group) {
        const char* qrow = reinterpret_cast<const char*>(p.q) +
                           ((int64_t)s * p.num_q_heads + g * p.group + n) * Sh::kRow;
#pragma unroll
        for (int c = 0; c < Sh::kKLoads; ++c)
          qv[c] = *reinterpret_cast<const uint4*>(qrow + 64 * c + 16 * kg);
      } else {
#pragma unroll
        for (int c = 0; c < Sh::kKLoads; ++c) qv[c] = uint4{0u, 0u, 0u, 0u};
      }
      State<DT, D> st;
      st.m = -INFINITY;
      st.l = 0.f;
#pragma unroll
      for (int e = 0; e < Sh::kTiles; ++e) st.o[e] = f32x4{0.f, 0.f, 0.f, 0.f};

      const int32_t* trow = p.block_table + (int64_t)s * p.max_blocks;
      const char* kbase = p.k_cache + (int64_t)g * head_stride;
      const char* vbase = p.v_cache + (int64_t)g * head_stride;
      // Block ids of the piece, 64 at a time: lane i holds block j0c + i.
      int32_t idc = j0;
      int32_t ids = 0;
      {
        const int32_t jj = min(idc + lane, j1 - 1);
        ids = trow[jj];
      }
      auto block_of = [&](int32_t j) -> int32_t {
        if (j >= idc + 64) {
          idc = j;
          const int32_t jj = min(idc + lane, j1 - 1);
          ids = trow[jj];
        }
        int32_t b = __builtin_amdgcn_readlane(ids, j - idc);
        return (uint32_t)b < (uint32_t)p.num_blocks ? b : 0;
      };

      Tile<DT, D> buf[Sh::kDepth];
#pragma unroll
      for (int u = 0; u < Sh::kDepth; ++u) {
        const int32_t b = block_of(min(j0 + u, j1 - 1));
        load_tile<DT, D>(buf[u], kbase + (int64_t)b * block_stride, vbase + (int64_t)b * block_stride,
                         k_off, v_off);
      }
      for (int32_t jb = j0; jb < j1; jb += Sh::kDepth) {
#pragma unroll
        for (int u = 0; u < Sh::kDepth; ++u) {
          const int32_t j = jb + u;
          if (j < j1) {
            const int32_t valid = min(16, len_s - 16 * j);
            attend_block<DT, D>(st, buf[u], qv, p.scale_log2, valid, kg);
          }
          const int32_t b = block_of(min(j + Sh::kDepth, j1 - 1));
          load_tile<DT, D>(buf[u], kbase + (int64_t)b * block_stride,
                           vbase + (int64_t)b * block_stride, k_off, v_off);
        }
      }
      if (j0 == 0 && j1 == nb_s) {
        write_output<DT, D>(p, st, s, g, n, kg);
      } else {
        write_partial<DT, D>(p, st, 2 * w + (first_piece ? 0 : 1), n, kg);
      }
      i += j1 - j0;
      first_piece = false;
    }
    // Next sequence (wrapping to the next head).
    if (i >= i1) break;
    ++s;
    if (s == p.num_seqs) {
      s = 0;
      ++g;
    }
    len_s = seq_len_clamped(p, s);
    nb_s = (len_s + 15) >> 4;
    j0 = 0;
  }
}

// Merge the partial states of sequences whose tiles were split across
// waves, and zero the output of empty sequences. One workgroup per
// (sequence, KV head).
template <int DT, int D>
__global__ void __launch_bounds__(64)
decode_merge_kernel(DecodeParams p) {
  const int32_t s = blockIdx.x / p.num_kv_heads;
  const int32_t g = blockIdx.x - s * p.num_kv_heads;
  const int32_t per_head = p.ws_prefix[p.num_seqs];
  const int32_t a = p.ws_prefix[s];
  const int32_t b = p.ws_prefix[s + 1];
  const int lane = threadIdx.x;
  const int32_t G = p.group;
  const int64_t out_row = ((int64_t)s * p.num_q_heads + (int64_t)g * G) * D;
  if (a == b) {  // empty sequence: zero output
    for (int32_t e = lane; e < G * D; e += 64) {
      if constexpr (DT == PKV_BF16)
        reinterpret_cast<uint16_t*>(p.out)[out_row + e] = 0;
      else
        reinterpret_cast<float*>(p.out)[out_row + e] = 0.f;
    }
    return;
  }
  const int64_t total = (int64_t)per_head * p.num_kv_heads;
  const int64_t first = (int64_t)g * per_head + a;
  const int64_t last = (int64_t)g * per_head + b - 1;
  // wave covering tile i: largest w with floor(w*total/W) <= i
  const int32_t W = p.num_waves;
  const int32_t w0 = (int32_t)(((first + 1) * W + total - 1) / total - 1);
  const int32_t w1 = (int32_t)(((last + 1) * W + total - 1) / total - 1);
  if (w0 == w1) return;  // written directly by its wave
  const int32_t stride = G * (D + 4);
  // Waves w0..w1 overlap the sequence; those with an empty range (possible
  // when there are fewer tiles than waves) wrote nothing and are skipped.
  // A wave whose range starts before the sequence holds it in its second
  // slot, every other one in its first.
  for (int32_t e = lane; e < G * D; e += 64) {
    const int32_t h = e / D;
    float mmax = -INFINITY;
    for (int32_t w = w0; w <= w1; ++w) {
      const int64_t st = total * w / W;
      if (st == total * (w + 1) / W) continue;
      const int32_t slot = 2 * w + (st < first ? 1 : 0);
      mmax = fmaxf(mmax, p.ws_partial[(int64_t)slot * stride + G * D + h]);
    }
    float num = 0.f, den = 0.f;
    for (int32_t w = w0; w <= w1; ++w) {
      const int64_t st = total * w / W;
      if (st == total * (w + 1) / W) continue;
      const int32_t slot = 2 * w + (st < first ? 1 : 0);
      const float* base = p.ws_partial + (int64_t)slot * stride;
      const float sc = __builtin_amdgcn_exp2f(base[G * D + h] - mmax);
      num += sc * base[e];
      den += sc * base[G * D + G + h];
    }
    const float o = num / den;
    if constexpr (DT == PKV_BF16) {
      bf16x2 v = {(__bf16)o, (__bf16)0.0f};
      reinterpret_cast<uint16_t*>(p.out)[out_row + e] =
          (uint16_t)(__builtin_bit_cast(uint32_t, v) & 0xFFFFu);
    } else {
      reinterpret_cast<float*>(p.out)[out_row + e] = o;
    }
  }
}

int g_waves_device = -1;
int g_waves = 0;

template <int DT, int D>
hipError_t launch(const DecodeParams& prm, int32_t seqs_heads, hipStream_t stream) {
  hipLaunchKernelGGL((decode_split_kernel<DT, D>), dim3(prm.num_waves), dim3(64), 0, stream, prm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((decode_merge_kernel<DT, D>), dim3(seqs_heads), dim3(64), 0, stream, prm);
  return hipGetLastError();
}

}  // namespace

namespace pkv {

int decode_num_waves() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (dev != g_waves_device) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    int per_cu = 8;
    if (const char* env = getenv("PKV_DECODE_WAVES_PER_CU")) {
      int v = atoi(env);
      if (v >= 1 && v <= 32) per_cu = v;
    }
    int w = prop.multiProcessorCount * per_cu;
    w = (w + kXcds - 1) / kXcds * kXcds;
    g_waves = w;
    g_waves_device = dev;
  }
  return g_waves;
}

size_t decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                              int32_t head_dim) {
  const size_t prefix = ((size_t)(num_seqs + 1) * 4 + 255) / 256 * 256;
  const size_t group = (size_t)(num_q_heads / num_kv_heads);
  const size_t partial = 2 * (size_t)decode_num_waves() * group * (head_dim + 4) * 4;
  return prefix + partial;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  DecodeParams p;
  p.out = a.out;
  p.q = a.q;
  p.k_cache = reinterpret_cast<const char*>(a.k_cache);
  p.v_cache = reinterpret_cast<const char*>(a.v_cache);
  p.block_table = a.block_table;
  p.context_lens = a.context_lens;
  p.ws_prefix = reinterpret_cast<int32_t*>(a.workspace);
  const size_t prefix = ((size_t)(a.num_seqs + 1) * 4 + 255) / 256 * 256;
  p.ws_partial = reinterpret_cast<float*>(reinterpret_cast<char*>(a.workspace) + prefix);
  p.num_seqs = a.num_seqs;
  p.num_blocks = a.num_blocks;
  p.max_blocks = a.max_blocks_per_seq;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.group = a.num_q_heads / a.num_kv_heads;
  p.num_waves = decode_num_waves();
  p.scale_log2 = a.scale * kLog2e;
  const int32_t sh = a.num_seqs * a.num_kv_heads;
  if (a.dtype == PKV_BF16) {
    return a.head_dim == 128 ? launch<PKV_BF16, 128>(p, sh, stream) : launch<PKV_BF16, 64>(p, sh, stream);
  }
  return a.head_dim == 128 ? launch<PKV_F32, 128>(p, sh, stream) : launch<PKV_F32, 64>(p, sh, stream);
}

}  // namespace pkv
