// Optional diagnostics of the host library, switched by environment variables
// read at every call:
//   HA_LOG=1          one line per entry-point call (sizes, path, workspace) and
//                     per kernel launch (grid, block, tiling) on stderr;
//   HA_CHECK_FINITE=1 after every state write, a scan of the state for
//                     non-finite values; the call then synchronises its stream
//                     and returns HA_ERR_NONFINITE if it finds one.
// Any value other than empty or "0" switches a flag on.
#pragma once

namespace ha {
bool env_flag(const char* name);
void log_line(const char* fmt, ...) __attribute__((format(printf, 1, 2)));
}  // namespace ha

#define HA_LOG(...)                                              \
  do {                                                           \
    if (::ha::env_flag("HA_LOG")) ::ha::log_line(__VA_ARGS__);   \
  } while (0)
