// Status plumbing of the C ABI (per-thread messages, status strings) and the
// host-side debug checks. Host only: no HIP runtime calls here.
#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <unordered_set>

#include "host.h"

namespace pkv {

namespace {
thread_local char g_msg[512] = "";

// Debug checks: off unless PKV_DEBUG_CHECKS=1 was set when the library was
// loaded, or switched with pkv_set_debug_checks.
std::atomic<int> g_debug{-1};
}  // namespace

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return code;
}

void clear_error() { g_msg[0] = '\0'; }

bool debug_checks() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* env = getenv("PKV_DEBUG_CHECKS");
    v = env && env[0] == '1' ? 1 : 0;
    int expected = -1;
    g_debug.compare_exchange_strong(expected, v, std::memory_order_relaxed);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

// One token per slot: the worker's slot mapping names one destination per
// scheduled token ("vLLM: what PagedAttention turned into", section "The
// problem PagedAttention was actually solving"), so two tokens of one call
// with the same slot would race in the scatter, and the null block is never a
// write target ("The block pool, and the two tricks in it"). Negative slots
// are padding.
int check_slot_mapping(const int64_t* slots, int64_t n, int32_t num_blocks) {
  if (n < 0 || num_blocks <= 0) return fail(PKV_ERR_INVALID_ARG, "bad sizes");
  if (n > 0 && !slots) return fail(PKV_ERR_INVALID_ARG, "slot mapping is NULL");
  const int64_t limit = (int64_t)num_blocks * kBlock;
  std::unordered_set<int64_t> seen;
  seen.reserve((size_t)n);
  for (int64_t t = 0; t < n; ++t) {
    const int64_t s = slots[t];
    if (s < 0) continue;
    if (s >= limit)
      return fail(PKV_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld lies outside the pool (%lld slots)",
                  (long long)t, (long long)s, (long long)limit);
    if (s < kBlock)
      return fail(PKV_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld lies in the null block",
                  (long long)t, (long long)s);
    if (!seen.insert(s).second)
      return fail(PKV_ERR_INVALID_ARG, "slot_mapping[%lld] = %lld repeats an earlier token's slot",
                  (long long)t, (long long)s);
  }
  return PKV_OK;
}

}  // namespace pkv

extern "C" {

const char* pkv_last_error(void) { return pkv::g_msg; }

const char* pkv_strerror(int code) {
  switch (code) {
    case PKV_OK: return "ok";
    case PKV_ERR_INVALID_ARG: return "invalid argument";
    case PKV_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKV_ERR_OUT_OF_BLOCKS: return "out of KV blocks";
    case PKV_ERR_NO_SUCH_SEQ: return "no such sequence";
    case PKV_ERR_SEQ_EXISTS: return "sequence exists";
    case PKV_ERR_WORKSPACE: return "workspace too small";
    case PKV_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int pkv_version(void) { return 200; }

int pkv_set_debug_checks(int32_t enabled) {
  pkv::clear_error();
  pkv::g_debug.store(enabled ? 1 : 0, std::memory_order_relaxed);
  return PKV_OK;
}

int pkv_check_slot_mapping(const int64_t* slot_mapping, int64_t num_tokens, int32_t num_blocks) {
  pkv::clear_error();
  return pkv::check_slot_mapping(slot_mapping, num_tokens, num_blocks);
}

}  // extern "C"
