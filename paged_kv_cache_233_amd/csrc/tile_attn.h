// One 16-token block of paged attention on gfx950 MFMA tiles: the register
// layouts and the online-softmax step shared by the decode and the
// chunked-prefill kernels.
//
// A wave holds one K tile and one V tile ([16 tokens][head_dim] each, one
// (block, KV head) of the pool, contiguous) and NG groups of 16 query rows
// ("columns"). For each group it computes
//   S[t][n] = sum_d K[t][d] Q[n][d]           (MFMA 16x16x32 bf16 / 16x16x4 f32)
//   online softmax over t for each column n  (exp2, cross-lane max/sum)
//   O^T[d][n] += sum_t V[t][d] P[n][t]        (MFMA 16x16x16 bf16 / 16x16x4 f32)
// Register layouts (lane l, n = l % 16, kg = l / 16):
//   K operand: row t = n of the tile; load c reads bytes [64c + 16kg, +16), so
//              each load instruction reads 16 rows x 64 contiguous bytes.
//   S result : lane (n, kg) holds S[4kg + i][n], i = 0..3 (the C layout of
//              the 16x16 MFMAs), which is also the B-operand layout P^T needs.
//   V operand: lane reads row 4kg + j (j = 0..3), bytes [n*R/16, (n+1)*R/16)
//              of the R-byte row, so each load instruction reads 4 whole rows;
//              element e of those four rows, packed, is the A operand of
//              output tile e (dims d = m*(D/16) + e for MFMA row m).
//   O result : lane (n, kg) holds column n, dims (4kg + i) * (D/16) + e.
// The running max m and sum l of column n live in the four lanes (n, kg),
// kept bit-identical by commutative cross-lane combines.
#pragma once

#include "internal.h"

namespace pkv {
namespace tile {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

template <int DT, int D>
struct Shape {
  static constexpr int kElem = DT == PKV_F32 ? 4 : 2;
  static constexpr int kRow = D * kElem;       // bytes of one token row of one head
  static constexpr int kKLoads = kRow / 64;    // 16-byte K loads per lane per tile
  static constexpr int kVWords = kRow / 64;    // 32-bit V words per lane per row
  static constexpr int kTiles = D / 16;        // 16-row MFMA tiles of head_dim
  static constexpr int kTileBytes = 16 * kRow; // one (block, head) tile
};

template <int DT, int D>
struct Tile {
  uint4 k[Shape<DT, D>::kKLoads];
  uint32_t v[4][Shape<DT, D>::kVWords];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// A load of N 32-bit words; STREAM marks it non-temporal (data read once:
// on gfx950 the decode's K/V tiles stream ≈ 10% faster this way).
template <bool STREAM, typename T>
__device__ __forceinline__ T load_vec(const char* p) {
  if constexpr (STREAM)
    return __builtin_nontemporal_load(reinterpret_cast<const T*>(p));
  else
    return *reinterpret_cast<const T*>(p);
}

template <int W, bool STREAM>
__device__ __forceinline__ void load_words(uint32_t* dst, const char* p) {
  if constexpr (W == 2) {
    const u32x2 x = load_vec<STREAM, u32x2>(p);
    dst[0] = x[0];
    dst[1] = x[1];
  } else {
#pragma unroll
    for (int i = 0; i < W; i += 4) {
      const u32x4 x = load_vec<STREAM, u32x4>(p + 4 * i);
      dst[i] = x[0];
      dst[i + 1] = x[1];
      dst[i + 2] = x[2];
      dst[i + 3] = x[3];
    }
  }
}

// Lane (n, kg) offsets of its K and V pieces within a (block, head) tile.
template <int DT, int D>
__device__ __forceinline__ uint32_t k_lane_offset(int n, int kg) {
  return (uint32_t)(n * Shape<DT, D>::kRow + kg * 16);
}
template <int DT, int D>
__device__ __forceinline__ uint32_t v_lane_offset(int n, int kg) {
  return (uint32_t)((4 * kg) * Shape<DT, D>::kRow + n * (Shape<DT, D>::kRow / 16));
}

// One (block, head) tile into registers; STREAM: non-temporal loads (for
// tiles read once, as in decode).
template <int DT, int D, bool STREAM = false>
__device__ __forceinline__ void load_tile(Tile<DT, D>& tl, const char* kb, const char* vb,
                                          uint32_t k_off, uint32_t v_off) {
  using Sh = Shape<DT, D>;
#pragma unroll
  for (int c = 0; c < Sh::kKLoads; ++c) {
    const u32x4 x = load_vec<STREAM, u32x4>(kb + k_off + 64 * c);
    tl.k[c] = uint4{x[0], x[1], x[2], x[3]};
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) load_words<Sh::kVWords, STREAM>(tl.v[j], vb + v_off + j * Sh::kRow);
}

// Query operand of one column group (B operand of the score MFMAs): the
// same byte pieces of the query row as the K operand takes of a key row.
template <int DT, int D>
struct QOp {
  uint4 c[Shape<DT, D>::kKLoads];
};

// Load it from a query row at `qrow` (the head's D values), or zero.
template <int DT, int D>
__device__ __forceinline__ void load_query(QOp<DT, D>& qv, const char* qrow, bool valid, int kg) {
#pragma unroll
  for (int c = 0; c < Shape<DT, D>::kKLoads; ++c)
    qv.c[c] = valid ? *reinterpret_cast<const uint4*>(qrow + 64 * c + 16 * kg) : uint4{0u, 0u, 0u, 0u};
}

// Reductions over the four lanes l, l^16, l^32, l^48 (the four token groups
// of one column). The gfx950 row-swap instructions hand each lane the value
// of its partner 16 (then 32) lanes away in a VALU operation, so the loop has
// no LDS traffic and no LDS wait. The combine is commutative, so all four
// lanes end with the same bits.
__device__ __forceinline__ float wave_max_kg(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ float wave_sum_kg(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

__device__ __forceinline__ float bf16_round(float x) {
  bf16x2 p = {(__bf16)x, (__bf16)0.0f};
  return (float)p[0];
}

// Running softmax state of one lane for one column group.
template <int DT, int D>
struct State {
  float m;                                  // running max of scaled scores (log2 units)
  float l;                                  // running sum of weights
  f32x4 o[Shape<DT, D>::kTiles];            // unnormalised output, layout above

  __device__ __forceinline__ void reset() {
    m = -INFINITY;
    l = 0.f;
#pragma unroll
    for (int e = 0; e < Shape<DT, D>::kTiles; ++e) o[e] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
};

// One 16-token block starting at sequence position t0 against NG column
// groups. lim[g] is the last position column group g's lane may attend to
// (its causal limit; per lane); positions at or beyond `ctx` are outside the
// sequence and their V rows are zeroed (the pool may hold anything there).
// `mask` (wave-uniform) must be true whenever the block reaches past the
// smallest limit or past ctx; otherwise masking is skipped. Every column must
// see at least one position in the first block it processes.
template <int DT, int D, int NG>
__device__ __forceinline__ void attend_tile(State<DT, D> (&st)[NG], Tile<DT, D>& tl,
                                            const QOp<DT, D> (&qv)[NG],
                                            float scale_log2, int t0, const int (&lim)[NG],
                                            int ctx, bool mask, int kg) {
  using Sh = Shape<DT, D>;
  f32x4 s[NG];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    s[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (DT == PKV_BF16) {
#pragma unroll
      for (int c = 0; c < Sh::kKLoads; ++c)
        s[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, tl.k[c]),
                                                        __builtin_bit_cast(bf16x8, qv[gi].c[c]), s[gi],
                                                        0, 0, 0);
    } else {
#pragma unroll
      for (int c = 0; c < Sh::kKLoads; ++c) {
        const float* kf = reinterpret_cast<const float*>(&tl.k[c]);
        const float* qf = reinterpret_cast<const float*>(&qv[gi].c[c]);
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[gi] = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[e], qf[e], s[gi], 0, 0, 0);
      }
    }
  }
  const int tk = t0 + 4 * kg;  // position of this lane's first score row
  if (mask) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (tk + j >= ctx) {
#pragma unroll
        for (int w = 0; w < Sh::kVWords; ++w) tl.v[j][w] = 0u;
      }
  }
  float p[NG][4];
#pragma unroll
  for (int gi = 0; gi < NG; ++gi) {
    float x[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = s[gi][i] * scale_log2;
    if (mask) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (tk + i > lim[gi]) x[i] = -INFINITY;
    }
    const float bmax = wave_max_kg(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])));
    const float m_new = fmaxf(st[gi].m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(st[gi].m - m_new);
#pragma unroll
    for (int i = 0; i < 4; ++i) p[gi][i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    if constexpr (DT == PKV_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) p[gi][i] = bf16_round(p[gi][i]);  // the weights the MFMA sees
    }
    const float rsum = wave_sum_kg((p[gi][0] + p[gi][1]) + (p[gi][2] + p[gi][3]));
    st[gi].l = st[gi].l * alpha + rsum;
    st[gi].m = m_new;
    // alpha is exactly 1 unless the running max grew: skipping is exact.
    if (__ballot(alpha != 1.0f) != 0) {
#pragma unroll
      for (int e = 0; e < Sh::kTiles; ++e) st[gi].o[e] *= alpha;
    }
  }
  if constexpr (DT == PKV_BF16) {
    i16x4 b[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
      bf16x2 p01 = {(__bf16)p[gi][0], (__bf16)p[gi][1]};
      bf16x2 p23 = {(__bf16)p[gi][2], (__bf16)p[gi][3]};
      uint2 pb = {__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
      b[gi] = __builtin_bit_cast(i16x4, pb);
    }
#pragma unroll
    for (int e = 0; e < Sh::kTiles; ++e) {
      // element e of each of the 4 rows this lane loaded, packed as 4 bf16
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      uint2 a;
      a.x = __builtin_amdgcn_perm(tl.v[1][w], tl.v[0][w], sel);
      a.y = __builtin_amdgcn_perm(tl.v[3][w], tl.v[2][w], sel);
      const i16x4 av = __builtin_bit_cast(i16x4, a);
#pragma unroll
      for (int gi = 0; gi < NG; ++gi)
        st[gi].o[e] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(av, b[gi], st[gi].o[e], 0, 0, 0);
    }
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int e = 0; e < Sh::kTiles; ++e) {
        const float av = __builtin_bit_cast(float, tl.v[j][e]);
#pragma unroll
        for (int gi = 0; gi < NG; ++gi)
          st[gi].o[e] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, p[gi][j], st[gi].o[e], 0, 0, 0);
      }
    }
  }
}

// Normalised output of one column group: lane (n, kg) writes its dims of
// the output row `row` (D elements), if `valid`.
template <int DT, int D>
__device__ __forceinline__ void store_row(void* out, int64_t row, const State<DT, D>& st, int kg,
                                          bool valid) {
  using Sh = Shape<DT, D>;
  if (!valid) return;
  const float inv = 1.0f / st.l;
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
      char* dst = reinterpret_cast<char*>(out) + (row * D + d0) * 2;
      if constexpr (Sh::kTiles == 8) {
        *reinterpret_cast<uint4*>(dst) = uint4{w[0], w[1], w[2], w[3]};
      } else {
        *reinterpret_cast<uint2*>(dst) = uint2{w[0], w[1]};
      }
    } else {
      float* dst = reinterpret_cast<float*>(out) + row * D + d0;
#pragma unroll
      for (int e = 0; e < Sh::kTiles; e += 4)
        *reinterpret_cast<float4*>(dst + e) =
            float4{st.o[e][i] * inv, st.o[e + 1][i] * inv, st.o[e + 2][i] * inv, st.o[e + 3][i] * inv};
    }
  }
}

}  // namespace tile
}  // namespace pkv
