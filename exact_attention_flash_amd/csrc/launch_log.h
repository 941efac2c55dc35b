// Launch log: with FLASH_ATTN_LOG set to anything but "0" in the environment (read
// once per process), every launcher prints one line per kernel it enqueues to stderr:
// the kernel instance, its grid and the schedule choices made on the host.
#pragma once
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

namespace fa {

inline bool launch_log_enabled() {
  static const bool on = [] {
    const char* e = std::getenv("FLASH_ATTN_LOG");
    return e != nullptr && *e != '\0' && std::strcmp(e, "0") != 0;
  }();
  return on;
}

inline void launch_log(const char* fmt, ...) {
  if (!launch_log_enabled()) return;
  std::va_list ap;
  va_start(ap, fmt);
  std::fputs("flash_attn: ", stderr);
  std::vfprintf(stderr, fmt, ap);
  std::fputc('\n', stderr);
  va_end(ap);
}

inline const char* dtype_name(bool fp16) { return fp16 ? "fp16" : "bf16"; }

}  // namespace fa
