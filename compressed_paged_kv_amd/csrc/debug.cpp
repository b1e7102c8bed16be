// Debug and tracing switches of the library (host C++).
//
//   ZP_TRACE=1         roctx ranges around the host side of every call
//                      (planning, each kernel launch), for rocprofv3's
//                      marker trace; the roctx library is loaded on first
//                      use and tracing stays off if it is not there;
//   ZP_DEBUG_POISON=1  after every compression, NaN into the blocks the call
//                      freed and into every slot of each request's reserved
//                      block (all past the new length), in every layer, so a
//                      later read of stale rows shows up in the outputs;
//   ZP_VALIDATE=1      a compression given a device copy of the block tables
//                      first reads it back and rejects the call when it
//                      differs from the host tables (one host synchronisation).
// The environment sets the flags when the library first needs them;
// zp_set_debug_flags() replaces them at run time.
#include <dlfcn.h>

#include <atomic>
#include <cstdlib>
#include <mutex>

#include "zp_internal.h"

namespace zp {
namespace {

std::once_flag g_env_once;
std::atomic<uint32_t> g_flags{0};

bool env_on(const char* name) {
  const char* v = std::getenv(name);
  return v && *v && !(v[0] == '0' && v[1] == '\0');
}

void read_env() {
  uint32_t f = 0;
  if (env_on("ZP_TRACE")) f |= ZP_DEBUG_TRACE;
  if (env_on("ZP_DEBUG_POISON")) f |= ZP_DEBUG_POISON;
  if (env_on("ZP_VALIDATE")) f |= ZP_DEBUG_VALIDATE;
  g_flags.store(f);
}

typedef int (*range_push_fn)(const char*);
typedef int (*range_pop_fn)(void);
std::once_flag g_roctx_once;
range_push_fn g_push = nullptr;
range_pop_fn g_pop = nullptr;

void load_roctx() {
  for (const char* name : {"librocprofiler-sdk-roctx.so.1", "librocprofiler-sdk-roctx.so",
                           "libroctx64.so.4", "libroctx64.so"}) {
    void* h = dlopen(name, RTLD_NOW | RTLD_LOCAL);
    if (!h) continue;
    auto push = reinterpret_cast<range_push_fn>(dlsym(h, "roctxRangePushA"));
    auto pop = reinterpret_cast<range_pop_fn>(dlsym(h, "roctxRangePop"));
    if (push && pop) {
      g_push = push;
      g_pop = pop;
      return;
    }
  }
}

}  // namespace

uint32_t debug_flags() {
  std::call_once(g_env_once, read_env);
  return g_flags.load(std::memory_order_relaxed);
}

bool trace_available() {
  std::call_once(g_roctx_once, load_roctx);
  return g_push != nullptr;
}

TraceRange::TraceRange(const char* name) {
  if (!(debug_flags() & ZP_DEBUG_TRACE) || !trace_available()) return;
  g_push(name);
  active_ = true;
}

TraceRange::~TraceRange() {
  if (active_) g_pop();
}

}  // namespace zp

extern "C" {

uint32_t zp_debug_flags(void) { return zp::debug_flags(); }

zp_status zp_set_debug_flags(uint32_t flags) {
  zp::clear_error();
  if (flags & ~(ZP_DEBUG_TRACE | ZP_DEBUG_POISON | ZP_DEBUG_VALIDATE)) {
    zp::set_error("unknown debug flags 0x%x", flags);
    return ZP_ERR_INVALID;
  }
  (void)zp::debug_flags();  // the environment is read first, then replaced
  zp::g_flags.store(flags);
  return ZP_OK;
}

int32_t zp_trace_available(void) { return zp::trace_available() ? 1 : 0; }

}  // extern "C"
