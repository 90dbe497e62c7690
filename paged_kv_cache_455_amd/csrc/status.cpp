// Status codes and the per-thread text of the last failure (pa_status_string,
// pa_last_error).  Host code only, with no HIP calls, so the host modules that
// use it (the block manager) also build on their own, e.g. under sanitizers.
#include "status.h"

#include <stdio.h>

namespace {
thread_local char g_last_error[512] = "";
}  // namespace

namespace pa {

pa_status_t set_errorv(pa_status_t st, const char *fmt, va_list ap) {
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  return st;
}

pa_status_t set_error(pa_status_t st, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  set_errorv(st, fmt, ap);
  va_end(ap);
  return st;
}

}  // namespace pa

extern "C" {

const char *pa_version(void) { return "paged_kv_cache_455_amd 0.2 (gfx950)"; }

const char *pa_status_string(pa_status_t s) {
  switch (s) {
    case PA_OK: return "ok";
    case PA_E_ARG: return "invalid argument";
    case PA_E_UNSUPPORTED: return "unsupported shape or dtype";
    case PA_E_WORKSPACE: return "workspace too small";
    case PA_E_HIP: return "HIP error";
    case PA_E_NO_BLOCKS: return "no free block";
  }
  return "unknown status";
}

const char *pa_last_error(void) { return g_last_error; }

}  // extern "C"
