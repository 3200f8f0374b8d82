// Debug mode of the C ABI (environment variable FA_DEBUG, or the name the
// FA1-vs-FA2 page gives, FLASH_ATTENTION_DEBUG, set to anything but "0"):
// each entry point prints its launch plan to stderr and, after its kernels,
// waits for the stream and counts the non-finite values (NaN, +inf, -inf) in
// each of its inputs and outputs; an LSE of -inf marks a row that sees no
// key.  This is the troubleshooting advice of the FA1-vs-FA2 page (section
// 6.2, numerical problems): turn on a debug mode to look for NaN values.  Off
// by default; it changes timing (a stream synchronisation per call) but not
// results.  It allocates nothing: the counters are a static device array, so
// debug-mode calls that overlap on one GPU share them.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <vector>

#include "fa_debug.h"

namespace {

// counts of NaN, +inf and -inf of the tensor being scanned
static __device__ unsigned long long debug_counts[3];

// Non-finite values among n elements: kind 0 = fp16, 1 = bf16 (16-bit
// patterns), 2 = fp32.
__global__ __launch_bounds__(256) void count_nonfinite_kernel(const void *data, size_t n, int kind,
                                                              unsigned long long *counts) {
  unsigned long long nan = 0, pinf = 0, ninf = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
    if (kind == 2) {
      const uint32_t u = reinterpret_cast<const uint32_t *>(data)[i];
      if ((u & 0x7F800000u) == 0x7F800000u) {
        if (u & 0x007FFFFFu) ++nan;
        else if (u >> 31) ++ninf;
        else ++pinf;
      }
    } else {
      const uint16_t u = reinterpret_cast<const uint16_t *>(data)[i];
      const uint16_t em = kind == 0 ? 0x7C00u : 0x7F80u;  // exponent field
      if ((u & em) == em) {
        if (u & (uint16_t)~(em | 0x8000u)) ++nan;
        else if (u >> 15) ++ninf;
        else ++pinf;
      }
    }
  }
  // one atomic per wave and counter
  for (int off = 32; off > 0; off >>= 1) {
    nan += __shfl_xor(nan, off, 64);
    pinf += __shfl_xor(pinf, off, 64);
    ninf += __shfl_xor(ninf, off, 64);
  }
  if ((threadIdx.x & 63) == 0) {
    if (nan) atomicAdd(counts, nan);
    if (pinf) atomicAdd(counts + 1, pinf);
    if (ninf) atomicAdd(counts + 2, ninf);
  }
}

__global__ void zero_counts_kernel(unsigned long long *counts) {
  if (threadIdx.x < 3) counts[threadIdx.x] = 0;
}

constexpr int kMaxDev = 64;
std::atomic<unsigned long long *> g_counts[kMaxDev];
std::mutex g_counts_mu;

unsigned long long *counts_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return nullptr;
  unsigned long long *p = g_counts[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_counts_mu);
  p = g_counts[dev].load(std::memory_order_relaxed);
  if (!p) {
    void *addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(debug_counts)) != hipSuccess || !addr) {
      (void)hipGetLastError();
      return nullptr;
    }
    p = static_cast<unsigned long long *>(addr);
    g_counts[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

namespace fa {

bool debug_enabled() {
  for (const char *name : {"FA_DEBUG", "FLASH_ATTENTION_DEBUG"}) {
    const char *v = std::getenv(name);
    if (v && *v && std::strcmp(v, "0") != 0) return true;
  }
  return false;
}

void debug_print(const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::fputs("[FA_DEBUG] ", stderr);
  std::vfprintf(stderr, fmt, ap);
  std::fputc('\n', stderr);
  std::fflush(stderr);
  va_end(ap);
}

void debug_scan(const char *fn, hipStream_t st, const DebugTensor *tensors, int count) {
  unsigned long long *counts = counts_ptr();
  if (!counts) {
    debug_print("%s: cannot address the counters on this device; no scan", fn);
    return;
  }
  for (int i = 0; i < count; ++i) {
    const DebugTensor &t = tensors[i];
    unsigned long long h[3] = {0, 0, 0};
    hipLaunchKernelGGL(zero_counts_kernel, dim3(1), dim3(64), 0, st, counts);
    if (t.n > 0) {
      const size_t blocks = (t.n + 255) / 256;
      const int grid = (int)(blocks < 4096 ? blocks : 4096);
      hipLaunchKernelGGL(count_nonfinite_kernel, dim3(grid), dim3(256), 0, st, t.ptr, t.n, t.kind, counts);
    }
    if (hipMemcpyAsync(h, counts, sizeof h, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
      debug_print("%s: %s: scan failed: %s", fn, t.name, hipGetErrorString(hipGetLastError()));
      continue;
    }
    debug_print("%s: %s: %llu NaN, %llu +inf, %llu -inf of %zu values%s", fn, t.name, h[0], h[1], h[2], t.n,
                t.kind == 2 ? " (an LSE of -inf marks a row that sees no key)" : "");
  }
}

void debug_lengths(const char *fn, hipStream_t st, const int *lq, const int *lk, int B, int Nq, int Nk) {
  for (int side = 0; side < 2; ++side) {
    const int *dev = side ? lk : lq;
    if (!dev || B < 1) continue;
    const int N = side ? Nk : Nq;
    std::vector<int> h((size_t)B);
    if (hipMemcpyAsync(h.data(), dev, sizeof(int) * (size_t)B, hipMemcpyDeviceToHost, st) != hipSuccess ||
        hipStreamSynchronize(st) != hipSuccess) {
      debug_print("%s: seqlens_%c: copy failed: %s", fn, side ? 'k' : 'q', hipGetErrorString(hipGetLastError()));
      continue;
    }
    std::string list;
    int bad = 0;
    for (int b = 0; b < B; ++b) {
      if (h[(size_t)b] < 0 || h[(size_t)b] > N) ++bad;
      if (b < 16) list += (b ? ", " : "") + std::to_string(h[(size_t)b]);
    }
    if (B > 16) list += ", ...";
    debug_print("%s: seqlens_%c (B=%d, N=%d): [%s]%s", fn, side ? 'k' : 'q', B, N, list.c_str(),
                bad ? "; outside [0, N], clamped on the device" : "");
  }
}

}  // namespace fa
