// Host-side helpers shared by the launch code (never compiled into kernels):
// the per-device CU count used to size persistent grids, and the optional
// launch log.
//
// Launch log: with ATTN_LOG=1 in the environment (read once, at the first
// call), every entry point prints one line to stderr with its arguments and
// status, and the launchers print each kernel's grid; otherwise nothing is
// printed.  This is the library's counterpart of the debug logging the
// vllm_mlx.attention backend does through its module logger.
#pragma once

namespace attn {

// Compute units of the current device, looked up once per device (thread-safe);
// 0 if the runtime cannot say.
int device_cu_count();

bool log_enabled();
void log_line(const char* fmt, ...) __attribute__((format(printf, 1, 2)));

}  // namespace attn
