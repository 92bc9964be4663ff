// Internal declarations of the host-only translation units of libpkv (the
// allocator, the scheduler, SHA-256 and the error plumbing). Nothing here
// needs the HIP runtime, so these files also build with a plain host compiler
// (the sanitizer build of the host code does exactly that).
#pragma once

#include <cstdarg>
#include <cstddef>
#include <cstdint>

#include "pkv.h"

namespace pkv {

// Records a message for pkv_last_error() and returns `code`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clears the per-thread message.
void clear_error();

constexpr int kBlock = PKV_BLOCK_SIZE;

// SHA-256 of n bytes; the seed hash of a first block; the chained content
// hash of one full block (parent may be NULL for the first block).
void sha256(const void* data, size_t n, uint8_t out[32]);
const uint8_t* none_hash();
void block_hash(const uint8_t* parent, const int32_t* tokens, uint64_t extra, uint8_t out[32]);

// Host check of one reshape_and_cache call's slot mapping (host memory):
// PKV_OK, or PKV_ERR_INVALID_ARG with a message naming the first offending
// entry (a slot outside the pool, a slot in the null block, or a
// non-negative slot that an earlier token of the call also has).
int check_slot_mapping(const int64_t* slots, int64_t n, int32_t num_blocks);
// Whether the device entry points run their debug checks (pkv_set_debug_checks
// or PKV_DEBUG_CHECKS=1 in the environment at load).
bool debug_checks();

}  // namespace pkv
