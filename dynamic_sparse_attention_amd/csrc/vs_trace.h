// vs_trace.h — optional per-kernel timing: when enabled (vs_trace_enable),
// every kernel launch of the library is bracketed by HIP events on its stream.
#pragma once

#include <hip/hip_runtime.h>

namespace vs {
void trace_begin(hipStream_t st, const char* name);
void trace_end(hipStream_t st);
}  // namespace vs

#define VS_TRACED(st, name, ...)  \
  do {                            \
    vs::trace_begin(st, name);    \
    __VA_ARGS__;                  \
    vs::trace_end(st);            \
  } while (0)
