// SHA-256 (FIPS 180-4) and the chained content hash of a KV block.
//
// A block's hash covers its parent block's hash, its own token ids and an
// extra key, so it names a prefix ending at the block boundary, not sixteen
// tokens ("vLLM: what PagedAttention turned into", section "What a block hash
// actually is"). The message is fixed here as
//   parent hash (32 bytes; the seed hash for a first block)
//   || the 16 token ids as little-endian int32 || extra key as little-endian
//   uint64,
// hashed with SHA-256. The seed hash is SHA-256 of a fixed string, so a hash
// means the same thing in every process (the same section's point about
// pinning the seed).
//
// The round constants and initial state are derived at first use from their
// definition (the first 32 fractional bits of the cube roots of the first 64
// primes, and of the square roots of the first 8 primes), with exact integer
// roots.
#include <cstring>

#include "host.h"

namespace pkv {
namespace {

struct Sha256Consts {
  uint32_t k[64];
  uint32_t h0[8];
};

typedef unsigned __int128 u128;

// floor(cbrt(v)) for v < 2^110.
uint64_t icbrt(u128 v) {
  uint64_t lo = 0, hi = (uint64_t)1 << 37;
  while (hi - lo > 1) {
    uint64_t mid = lo + (hi - lo) / 2;
    if ((u128)mid * mid * mid <= v) lo = mid; else hi = mid;
  }
  return lo;
}

// floor(sqrt(v)) for v < 2^72.
uint64_t isqrt(u128 v) {
  uint64_t lo = 0, hi = (uint64_t)1 << 37;
  while (hi - lo > 1) {
    uint64_t mid = lo + (hi - lo) / 2;
    if ((u128)mid * mid <= v) lo = mid; else hi = mid;
  }
  return lo;
}

Sha256Consts make_consts() {
  Sha256Consts c;
  int found = 0;
  for (uint32_t p = 2; found < 64; ++p) {
    bool prime = true;
    for (uint32_t d = 2; d * d <= p; ++d)
      if (p % d == 0) { prime = false; break; }
    if (!prime) continue;
    // floor(cbrt(p) * 2^32) = floor(cbrt(p * 2^96)); keep the fraction bits
    c.k[found] = (uint32_t)icbrt((u128)p << 96);
    if (found < 8) c.h0[found] = (uint32_t)isqrt((u128)p << 64);
    ++found;
  }
  return c;
}

const Sha256Consts& consts() {
  static const Sha256Consts c = make_consts();
  return c;
}

inline uint32_t rotr(uint32_t x, int n) { return (x >> n) | (x << (32 - n)); }

void compress(uint32_t h[8], const uint8_t* blk, const uint32_t* k) {
  // Message schedule kept as a 16-word window, extended as the rounds go.
  uint32_t w[16];
  for (int i = 0; i < 16; ++i) {
    uint32_t x;
    std::memcpy(&x, blk + 4 * i, 4);
    w[i] = __builtin_bswap32(x);
  }
  uint32_t a = h[0], b = h[1], c = h[2], d = h[3], e = h[4], f = h[5], g = h[6], hh = h[7];
#pragma unroll 16
  for (int i = 0; i < 64; ++i) {
    uint32_t wi;
    if (i < 16) {
      wi = w[i];
    } else {
      const uint32_t w15 = w[(i - 15) & 15], w2 = w[(i - 2) & 15];
      const uint32_t s0 = rotr(w15, 7) ^ rotr(w15, 18) ^ (w15 >> 3);
      const uint32_t s1 = rotr(w2, 17) ^ rotr(w2, 19) ^ (w2 >> 10);
      wi = w[i & 15] = w[i & 15] + s0 + w[(i - 7) & 15] + s1;
    }
    const uint32_t S1 = rotr(e, 6) ^ rotr(e, 11) ^ rotr(e, 25);
    const uint32_t ch = (e & f) ^ (~e & g);
    const uint32_t t1 = hh + S1 + ch + k[i] + wi;
    const uint32_t S0 = rotr(a, 2) ^ rotr(a, 13) ^ rotr(a, 22);
    const uint32_t maj = (a & b) ^ (a & c) ^ (b & c);
    const uint32_t t2 = S0 + maj;
    hh = g; g = f; f = e; e = d + t1; d = c; c = b; b = a; a = t1 + t2;
  }
  h[0] += a; h[1] += b; h[2] += c; h[3] += d; h[4] += e; h[5] += f; h[6] += g; h[7] += hh;
}

}  // namespace

void sha256(const void* data, size_t n, uint8_t out[32]) {
  const Sha256Consts& c = consts();
  uint32_t h[8];
  std::memcpy(h, c.h0, sizeof(h));
  const uint8_t* p = static_cast<const uint8_t*>(data);
  size_t full = n / 64;
  for (size_t i = 0; i < full; ++i) compress(h, p + 64 * i, c.k);
  // Last one or two blocks: the remaining bytes, 0x80, zeros, bit length.
  uint8_t tail[128] = {0};
  size_t rem = n - 64 * full;
  if (rem) std::memcpy(tail, p + 64 * full, rem);
  tail[rem] = 0x80;
  size_t tlen = rem + 1 + 8 <= 64 ? 64 : 128;
  uint64_t bits = (uint64_t)n * 8;
  for (int i = 0; i < 8; ++i) tail[tlen - 1 - i] = (uint8_t)(bits >> (8 * i));
  compress(h, tail, c.k);
  if (tlen == 128) compress(h, tail + 64, c.k);
  for (int i = 0; i < 8; ++i) {
    out[4 * i] = (uint8_t)(h[i] >> 24);
    out[4 * i + 1] = (uint8_t)(h[i] >> 16);
    out[4 * i + 2] = (uint8_t)(h[i] >> 8);
    out[4 * i + 3] = (uint8_t)h[i];
  }
}

const uint8_t* none_hash() {
  static uint8_t h[32];
  static const bool done = [] {
    static const char seed[] = "pkv none hash";
    sha256(seed, sizeof(seed) - 1, h);
    return true;
  }();
  (void)done;
  return h;
}

void block_hash(const uint8_t* parent, const int32_t* tokens, uint64_t extra, uint8_t out[32]) {
  uint8_t msg[32 + 4 * kBlock + 8];
  std::memcpy(msg, parent ? parent : none_hash(), 32);
  for (int i = 0; i < kBlock; ++i) {
    uint32_t t = (uint32_t)tokens[i];
    for (int j = 0; j < 4; ++j) msg[32 + 4 * i + j] = (uint8_t)(t >> (8 * j));
  }
  for (int j = 0; j < 8; ++j) msg[32 + 4 * kBlock + j] = (uint8_t)(extra >> (8 * j));
  sha256(msg, sizeof(msg), out);
}

}  // namespace pkv

extern "C" {

int pkv_sha256(const void* data, size_t n, uint8_t* out) {
  pkv::clear_error();
  if (!out || (!data && n > 0)) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  pkv::sha256(data, n, out);
  return PKV_OK;
}

int pkv_hash_block_tokens(const uint8_t* parent_hash, const int32_t* tokens, uint64_t extra_key,
                          uint8_t* out) {
  pkv::clear_error();
  if (!tokens || !out) return pkv::fail(PKV_ERR_INVALID_ARG, "NULL pointer argument");
  pkv::block_hash(parent_hash, tokens, extra_key, out);
  return PKV_OK;
}

}  // extern "C"
