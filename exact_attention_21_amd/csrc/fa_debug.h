// Debug mode of the C ABI (environment variable FA_DEBUG or
// FLASH_ATTENTION_DEBUG set to anything but "0"); implemented in fa_debug.hip.
// Host code only; no torch types.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace fa {

struct DebugTensor {
  const char *name;
  const void *ptr;
  size_t n;   // elements
  int kind;   // 0 fp16, 1 bf16 (the dtype codes of the C ABI), 2 fp32
};
bool debug_enabled();
void debug_print(const char *fmt, ...) __attribute__((format(printf, 1, 2)));
// Waits for the stream, then prints the NaN / +inf / -inf counts of each tensor.
void debug_scan(const char *fn, hipStream_t st, const DebugTensor *t, int count);
// Waits for the stream, then prints the per-batch valid lengths (device
// arrays, either may be null) and whether any lies outside [0, N].
void debug_lengths(const char *fn, hipStream_t st, const int *lq, const int *lk, int B, int Nq, int Nk);

}  // namespace fa
