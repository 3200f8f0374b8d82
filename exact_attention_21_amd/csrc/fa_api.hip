// C-ABI layer: argument validation, launch planning, device gating and kernel
// launches for the fused attention library.  No allocation; global mutable
// state is limited to per-device caches (the "is gfx950" check and the device
// address of the no-allocation backward's static scratch array).  In debug
// mode (FA_DEBUG) each computing entry point prints its plan once its
// arguments have passed the host checks, before the device check, and after
// its launches the counts of non-finite values in its inputs and outputs.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstring>
#include <initializer_list>

#include "fa.h"
#include "fa_debug.h"
#include "fa_kernels.h"

// Scratch of fa_bwd_noalloc: the backward workspace (-D and LSE * log2(e), fp32,
// one 256-byte aligned block each) for up to FA_BWD_NOALLOC_MAX_ROWS query
// rows.  Each GPU the library runs on holds its own copy until the process
// ends.  In host code `scratch` is only a handle for the runtime: its device
// address (per device) comes from hipGetSymbolAddress, and only that address
// is ever handed to a kernel.
constexpr size_t kScratchBytes = 2 * (size_t)FA_BWD_NOALLOC_MAX_ROWS * sizeof(float);
static __device__ __align__(256) char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::atomic<int> g_arch_ok[kMaxDevices];  // 0 unknown, 1 gfx950, 2 other

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return FA_ERR_DEVICE;
  if (dev < kMaxDevices) {
    const int c = g_arch_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return FA_OK;
    if (c == 2) return FA_ERR_DEVICE;
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return FA_ERR_DEVICE;
  const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < kMaxDevices) g_arch_ok[dev].store(ok ? 1 : 2, std::memory_order_relaxed);
  return ok ? FA_OK : FA_ERR_DEVICE;
}

std::atomic<void *> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// Device address of `scratch` on device `dev` (which must be current), looked
// up once per device; nullptr if the runtime cannot resolve it.
void *scratch_ptr(int dev) {
  if (dev < 0 || dev >= kMaxDevices) return nullptr;
  void *p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
      (void)hipGetLastError();  // do not leave the error for the caller's next HIP call
      return nullptr;
    }
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Dropout probability -> 8-bit threshold p8 = round(256 p) in [0, 255]; the
// kernels keep a pair iff its random byte is >= p8 and scale kept weights by
// 256 / (256 - p8).  Returns false for p outside [0, 255.5/256).
bool dropout_spec(float p, uint64_t seed, uint32_t offset, fa::DropoutSpec *d) {
  // range first: lrint of a value past the range of long is unspecified
  const double x = (double)p * 256.0;
  if (!(x >= 0.0 && x < 255.5)) return false;  // NaN fails both
  const long p8 = std::lrint(x);  // round half to even: 255.5 would give 256
  if (p8 > 255) return false;
  d->p8 = (uint32_t)p8;
  d->k0 = (uint32_t)seed;
  d->k1 = (uint32_t)(seed >> 32);
  d->offset = offset;
  d->scale = (float)(256.0 / (256.0 - (double)p8));
  return true;
}

fa::SeqShape seq_shape(int H, int Nq, int Nk, const int *lq, const int *lk) {
  fa::SeqShape s;
  s.Nq = Nq;
  s.Nk = Nk;
  s.H = H;
  s.lq = lq;
  s.lk = lk;
  return s;
}

int check_common(int B, int H, int N, int d, int causal, int dtype) {
  if (B < 1 || H < 1 || N < 1) return FA_ERR_SHAPE;
  const long double elems = (long double)B * H * N * (d > 0 ? d : 1);
  if (elems > 4.0e18L) return FA_ERR_SHAPE;
  // one head is addressed through a 32-bit buffer resource
  if ((long double)N * (d > 0 ? d : 1) * 2 >= 4294967296.0L) return FA_ERR_SHAPE;
  if (d != 64 && d != 128) return FA_ERR_HEAD_DIM;
  if (dtype != FA_F16 && dtype != FA_BF16) return FA_ERR_DTYPE;
  if (causal != 0 && causal != 1) return FA_ERR_ARG;
  return FA_OK;
}

// Query rows per forward workgroup = 128 * qb (32 * qb rows per wave): one
// block per wave at d = 128 (register budget) and, by default, at d = 64 too
// (FWD_QB_D64; two blocks at occupancy 2 measured slower than one at 4).
int fwd_qb(int N, int d) { return d == 128 ? 1 : (N > 128 ? FWD_QB_D64 : 1); }

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// heads per dispatch group of a causal grid (see fa_kernels.h)
int causal_group(const int *lq, const int *lk, int Nk, int d) {
  const bool small = (long)Nk * d <= fa::CAUSAL_GROUP_SMALL_MAX_ND;
  return !lq && !lk && small ? fa::CAUSAL_GROUP_SMALL : fa::CAUSAL_GROUP_PAIR;
}

// Debug mode, after the launches of one call: the launch error, or the
// non-finite counts of the listed tensors (not while the stream is being
// captured: the scan waits for the stream).
// With per-batch lengths (lq, lk) it prints those first.
void debug_after(const char *fn, hipError_t e, hipStream_t st,
                 std::initializer_list<fa::DebugTensor> ts, const int *lq = nullptr,
                 const int *lk = nullptr, int B = 0, int Nq = 0, int Nk = 0) {
  if (e != hipSuccess) {
    fa::debug_print("%s: launch failed: %s", fn, hipGetErrorString(e));
    return;
  }
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) == hipSuccess && cs != hipStreamCaptureStatusNone) {
    fa::debug_print("%s: stream is being captured; no scan", fn);
    return;
  }
  if (lq || lk) fa::debug_lengths(fn, st, lq, lk, B, Nq, Nk);
  fa::debug_scan(fn, st, ts.begin(), (int)ts.size());
}

// Key chunks of the split forward.  Its workgroups all carry about the same
// work, and the GPU holds 768 of them at once (256 CUs x 3), so the chunk count
// is chosen by how well the grid fills whole rounds of 768: the smallest count
// whose rounds are >= 95 % full (else the fullest), with at least 256 keys
// per chunk and chunks a multiple of two key tiles.
struct SplitPlan {
  int bm, n_qtiles, nsplit, chunk;
};
SplitPlan split_plan(int B, int H, int Nq, int Nk, int d) {
  constexpr long long kResident = 256 * 3;
  SplitPlan sp;
  sp.bm = 128;
  sp.n_qtiles = (Nq + sp.bm - 1) / sp.bm;
  const long long units = (long long)B * H * sp.n_qtiles;
  const long long most = ((long long)Nk + 255) / 256;
  const long long tiles2 = 2LL * fa::FWD_BN;
  double best_fill = -1.0;
  for (long long want = 1; want <= most && want <= 4 * kResident; ++want) {
    const long long chunk = ((long long)Nk + want - 1) / want;
    const long long c = (chunk + tiles2 - 1) / tiles2 * tiles2;
    const long long n = ((long long)Nk + c - 1) / c;
    const long long wgs = units * n;
    const double fill = (double)wgs / (double)(((wgs + kResident - 1) / kResident) * kResident);
    if (fill > best_fill + 1e-9) {
      best_fill = fill;
      sp.chunk = (int)c;
      sp.nsplit = (int)n;
    }
    if (fill >= 0.95) break;
  }
  return sp;
}

// Decode (Nq = 1): partials per head = 4 waves x workgroups per head, sized so
// that B*H heads give about 4096 waves (one per SIMD slot at occupancy 4), each
// over at least 256 keys; chunks are whole tiles.
SplitPlan decode_plan(int B, int H, int Nk, int d) {
  constexpr long long kWaves = 4096, kMinKeys = 256;
  const long long heads = (long long)B * H;
  const long long tk = fa::fwd_decode_tile(d);
  long long wg = (kWaves + 4 * heads - 1) / (4 * heads);
  wg = std::min(wg, ((long long)Nk + 4 * kMinKeys - 1) / (4 * kMinKeys));
  wg = std::max(wg, 1LL);
  const long long per = ((long long)Nk + 4 * wg - 1) / (4 * wg);
  SplitPlan sp;
  sp.bm = 1;
  sp.n_qtiles = 1;
  sp.nsplit = (int)(4 * wg);
  sp.chunk = (int)std::max(tk, (per + tk - 1) / tk * tk);
  return sp;
}

size_t split_workspace_bytes(int B, int H, int Nq, int d, const SplitPlan &sp) {
  const size_t rows = (size_t)B * H * sp.nsplit * Nq;
  return align256(rows * d * sizeof(float)) + align256(rows * sizeof(float));
}

}  // namespace

extern "C" {

const char *fa_status_str(int s) {
  switch (s) {
    case FA_OK: return "ok";
    case FA_ERR_NULL: return "null pointer argument";
    case FA_ERR_SHAPE: return "invalid shape (B, H, N must be >= 1; a head or the element count is too large)";
    case FA_ERR_HEAD_DIM: return "head dim must be 64 or 128";
    case FA_ERR_DTYPE: return "dtype must be FA_F16 (0) or FA_BF16 (1)";
    case FA_ERR_ALIGN: return "tensor pointer not 16-byte aligned, or length array not 4-byte aligned";
    case FA_ERR_WORKSPACE: return "backward workspace too small";
    case FA_ERR_DEVICE: return "current device is not a gfx950 GPU";
    case FA_ERR_LAUNCH: return "kernel launch failed";
    case FA_ERR_ARG: return "scale must be finite; causal must be 0 or 1; dropout_p in [0, 255.5/256)";
    case FA_ERR_SCRATCH: return "fa_bwd_noalloc: B*H*N exceeds FA_BWD_NOALLOC_MAX_ROWS (4194304 rows)";
    default: return "unknown status";
  }
}

int fa_fwd_plan(int B, int H, int N, int d, int causal, int dtype, fa_plan_t *plan) {
  if (!plan) return FA_ERR_NULL;
  const int rc = check_common(B, H, N, d, causal, dtype);
  if (rc) return rc;
  const int qb = fwd_qb(N, d);
  const int bm = 128 * qb;
  const int bn = fa::FWD_BN;
  const long long nq = (N + bm - 1) / bm;
  const long long grid = nq * B * H;
  if (grid > 0x7fffffffLL) return FA_ERR_SHAPE;
  plan->block_m = bm;
  plan->block_n = bn;
  plan->threads = 256;
  plan->grid = (int)grid;
  plan->lds_bytes = (d == 128 ? FWD_NSLOT_D128 : 2) * 2 * bn * d * 2;  // K and V rings (no dropout)
  plan->xcd_grouped = ((long long)B * H) % 8 == 0;
  return FA_OK;
}

}  // extern "C"

namespace {

int fwd_impl(const char *fn, const void *q, const void *k, const void *v, void *o, float *lse,
             const int *lq, const int *lk, int B, int H, int Nq, int Nk, int d, float scale,
             int causal, float dropout_p, uint64_t seed, uint32_t offset, int dtype, void *stream) {
  if (!q || !k || !v || !o || !lse) return FA_ERR_NULL;
  fa_plan_t plan;
  int rc = fa_fwd_plan(B, H, Nq, d, causal, dtype, &plan);
  if (rc) return rc;
  rc = check_common(B, H, Nk, d, causal, dtype);
  if (rc) return rc;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  fa::FwdParams p;
  std::memset(&p, 0, sizeof p);
  if (!dropout_spec(dropout_p, seed, offset, &p.drop)) return FA_ERR_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
    return FA_ERR_ALIGN;
  if (!aligned4(lq) || !aligned4(lk)) return FA_ERR_ALIGN;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    fa::debug_print("%s: B=%d H=%d Nq=%d Nk=%d d=%d dtype=%s causal=%d scale=%g dropout_p=%g "
                    "seqlens=%s; grid %d x %d threads, %d query rows and %d-key tiles per "
                    "workgroup, %d bytes of LDS, xcd_grouped=%d",
                    fn, B, H, Nq, Nk, d, dtype == FA_BF16 ? "bf16" : "f16", causal, scale,
                    dropout_p, lq || lk ? "per sequence" : "full", plan.grid, plan.threads,
                    plan.block_m, plan.block_n, plan.lds_bytes, plan.xcd_grouped);
  rc = check_device();
  if (rc) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.seq = seq_shape(H, Nq, Nk, lq, lk);
  p.n_qtiles = (Nq + plan.block_m - 1) / plan.block_m;
  p.xcd_grouped = plan.xcd_grouped;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal_group = causal_group(lq, lk, Nk, d);
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_fwd(p, dtype, d, causal, plan.block_m / 128, plan.grid, st);
  if (dbg) {
    const size_t nq = (size_t)B * H * Nq, nk = (size_t)B * H * Nk;
    debug_after(fn, e, st, {{"q", q, nq * d, dtype}, {"k", k, nk * d, dtype}, {"v", v, nk * d, dtype},
                            {"o", o, nq * d, dtype}, {"lse", lse, nq, 2}}, lq, lk, B, Nq, Nk);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse, int B, int H,
           int N, int d, float scale, int causal, int dtype, void *stream) {
  return fwd_impl("fa_fwd", q, k, v, o, lse, nullptr, nullptr, B, H, N, N, d, scale, causal, 0.f, 0,
                  0, dtype, stream);
}

int fa_fwd_padded(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, int dtype, void *stream) {
  return fwd_impl("fa_fwd_padded", q, k, v, o, lse, seqlens_q, seqlens_k, B, H, Nq, Nk, d, scale,
                  causal, 0.f, 0, 0, dtype, stream);
}

int fa_fwd_dropout(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, float dropout_p, uint64_t seed,
                   uint32_t offset, int dtype, void *stream) {
  return fwd_impl("fa_fwd_dropout", q, k, v, o, lse, seqlens_q, seqlens_k, B, H, Nq, Nk, d, scale,
                  causal, dropout_p, seed, offset, dtype, stream);
}

size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d) {
  if (check_common(B, H, Nq, d, 0, FA_BF16) != FA_OK || check_common(B, H, Nk, d, 0, FA_BF16) != FA_OK)
    return 0;
  return split_workspace_bytes(B, H, Nq, d, Nq == 1 ? decode_plan(B, H, Nk, d) : split_plan(B, H, Nq, Nk, d));
}

int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, int dtype, void *workspace,
                   size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !lse || !workspace) return FA_ERR_NULL;
  int rc = check_common(B, H, Nq, d, causal, dtype);
  if (rc) return rc;
  rc = check_common(B, H, Nk, d, causal, dtype);
  if (rc) return rc;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  const bool decode = Nq == 1;
  const SplitPlan sp = decode ? decode_plan(B, H, Nk, d) : split_plan(B, H, Nq, Nk, d);
  const long long grid = decode ? (long long)B * H * (sp.nsplit / 4) : (long long)sp.n_qtiles * sp.nsplit * B * H;
  if (grid > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(workspace))
    return FA_ERR_ALIGN;
  if (!aligned4(seqlens_q) || !aligned4(seqlens_k)) return FA_ERR_ALIGN;
  if (workspace_bytes < split_workspace_bytes(B, H, Nq, d, sp)) return FA_ERR_WORKSPACE;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    fa::debug_print("fa_fwd_splitkv: B=%d H=%d Nq=%d Nk=%d d=%d dtype=%s causal=%d scale=%g "
                    "seqlens=%s; %s: %d partials per query block of %d rows, %d keys each; "
                    "grid %lld x 256 threads, then the merge (one wave per row)",
                    B, H, Nq, Nk, d, dtype == FA_BF16 ? "bf16" : "f16", causal, scale,
                    seqlens_q || seqlens_k ? "per sequence" : "full",
                    decode ? "decode (one partial per wave)" : "split forward", sp.nsplit, sp.bm,
                    sp.chunk, grid);
  rc = check_device();
  if (rc) return rc;
  fa::FwdParams p;
  std::memset(&p, 0, sizeof p);
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.lse = lse;
  p.seq = seq_shape(H, Nq, Nk, seqlens_q, seqlens_k);
  p.n_qtiles = sp.n_qtiles;
  p.xcd_grouped = 0;
  p.scale_log2 = scale * 1.4426950408889634f;
  p.causal_group = causal_group(seqlens_q, seqlens_k, Nk, d);
  p.nsplit = sp.nsplit;
  p.chunk = sp.chunk;
  char *ws = static_cast<char *>(workspace);
  const size_t prows = (size_t)B * H * sp.nsplit * Nq;
  p.opart = reinterpret_cast<float *>(ws);
  p.lpart = reinterpret_cast<float *>(ws + align256(prows * d * sizeof(float)));
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  hipError_t e = decode ? fa::launch_fwd_decode(p, dtype, d, (int)grid, st)
                        : fa::launch_fwd_split(p, dtype, d, causal, (int)grid, st);
  if (e == hipSuccess) e = fa::launch_fwd_combine(p, dtype, d, (long)B * H * Nq, st);
  if (dbg) {
    const size_t nq = (size_t)B * H * Nq, nk = (size_t)B * H * Nk;
    debug_after("fa_fwd_splitkv", e, st,
                {{"q", q, nq * d, dtype}, {"k", k, nk * d, dtype}, {"v", v, nk * d, dtype},
                 {"o", o, nq * d, dtype}, {"lse", lse, nq, 2}},
                seqlens_q, seqlens_k, B, Nq, Nk);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

size_t fa_bwd_workspace_size(int B, int H, int N, int d) {
  if (check_common(B, H, N, d, 0, FA_BF16) != FA_OK) return 0;
  const size_t rows = (size_t)B * H * N;
  return 2 * align256(rows * sizeof(float));
}

int fa_bwd_plan(int B, int H, int N, int d, int causal, int dtype, fa_plan_t *plan) {
  if (!plan) return FA_ERR_NULL;
  const int rc = check_common(B, H, N, d, causal, dtype);
  if (rc) return rc;
  const long long nk = (N + fa::BWD_DKDV_BN - 1) / fa::BWD_DKDV_BN;
  const long long nq = (N + fa::BWD_DQ_BM - 1) / fa::BWD_DQ_BM;
  const long long grid = (nk > nq ? nk : nq) * B * H;
  if (grid > 0x7fffffffLL) return FA_ERR_SHAPE;
  plan->block_m = fa::BWD_DKDV_BM;
  plan->block_n = fa::BWD_DKDV_BN;
  plan->threads = 256;
  plan->grid = (int)(nk * B * H);
  plan->lds_bytes = BWD_DKDV_NSLOT * (2 * fa::BWD_DKDV_BM * d * 2 + fa::BWD_DKDV_STAT);
  plan->xcd_grouped = ((long long)B * H) % 8 == 0;
  return FA_OK;
}

}  // extern "C"

namespace {

// Shared checks of the backward entry points; fills the parameter block's
// shape fields and workspace pointers.  Q-side tensors have Nq rows, K-side Nk.
int bwd_setup(int B, int H, int Nq, int Nk, const int *lq, const int *lk, int d, float scale,
              int causal, int dtype, void *workspace, size_t workspace_bytes, fa::BwdParams *p,
              fa_plan_t *plan) {
  int rc = fa_bwd_plan(B, H, Nk, d, causal, dtype, plan);
  if (rc) return rc;
  rc = check_common(B, H, Nq, d, causal, dtype);
  if (rc) return rc;
  if ((long long)(Nq + fa::BWD_DQ_BM - 1) / fa::BWD_DQ_BM * B * H > 0x7fffffffLL) return FA_ERR_SHAPE;
  if (!std::isfinite(scale)) return FA_ERR_ARG;
  if (!workspace) return FA_ERR_NULL;
  if (!aligned16(workspace)) return FA_ERR_ALIGN;
  if (!aligned4(lq) || !aligned4(lk)) return FA_ERR_ALIGN;
  if (workspace_bytes < fa_bwd_workspace_size(B, H, Nq, d)) return FA_ERR_WORKSPACE;
  const size_t rows = (size_t)B * H * Nq;
  char *ws = static_cast<char *>(workspace);
  std::memset(p, 0, sizeof *p);
  p->dws = reinterpret_cast<float *>(ws);
  p->lse2 = reinterpret_cast<float *>(ws + align256(rows * sizeof(float)));
  p->seq = seq_shape(H, Nq, Nk, lq, lk);
  p->n_qtiles = (Nq + fa::BWD_DQ_BM - 1) / fa::BWD_DQ_BM;
  p->n_ktiles = (Nk + fa::BWD_DKDV_BN - 1) / fa::BWD_DKDV_BN;
  p->xcd_grouped = plan->xcd_grouped;
  p->scale = scale;
  p->scale_log2 = scale * 1.4426950408889634f;
  p->causal_group = causal_group(lq, lk, Nk, d);
  return FA_OK;
}

bool all_aligned(std::initializer_list<const void *> ptrs) {
  for (const void *ptr : ptrs)
    if (!aligned16(ptr)) return false;
  return true;
}

// Debug mode: the plan of a backward call (its passes and their grids).
void debug_bwd_plan(const char *fn, const char *passes, int B, int H, int Nq, int Nk, int d,
                    int dtype, int causal, float scale, float dropout_p, bool per_seq,
                    const fa::BwdParams &p, const fa_plan_t &plan) {
  fa::debug_print("%s: B=%d H=%d Nq=%d Nk=%d d=%d dtype=%s causal=%d scale=%g dropout_p=%g "
                  "seqlens=%s; %s; dQ grid %lld (%d query rows per workgroup), dK/dV grid %lld "
                  "(%d keys per workgroup, %d-row query blocks, %d bytes of LDS), xcd_grouped=%d",
                  fn, B, H, Nq, Nk, d, dtype == FA_BF16 ? "bf16" : "f16", causal, scale, dropout_p,
                  per_seq ? "per sequence" : "full", passes, (long long)p.n_qtiles * B * H,
                  fa::BWD_DQ_BM, (long long)p.n_ktiles * B * H, plan.block_n, plan.block_m,
                  plan.lds_bytes, plan.xcd_grouped);
}

// the two fp32 arrays of the backward workspace, for the debug scan
fa::DebugTensor ws_neg_d(const fa::BwdParams &p, size_t rows) { return {"workspace -D", p.dws, rows, 2}; }
fa::DebugTensor ws_lse2(const fa::BwdParams &p, size_t rows) {
  return {"workspace LSE*log2(e)", p.lse2, rows, 2};
}

}  // namespace

extern "C" {

int fa_bwd_preprocess(const void *o, const void *dout, const float *lse, int B, int H, int N,
                      int d, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
  if (!o || !dout || !lse || !workspace) return FA_ERR_NULL;
  fa::BwdParams p;
  fa_plan_t plan;
  int rc = bwd_setup(B, H, N, N, nullptr, nullptr, d, 1.f, 0, dtype, workspace, workspace_bytes,
                     &p, &plan);
  if (rc) return rc;
  if (!all_aligned({o, dout, lse})) return FA_ERR_ALIGN;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    fa::debug_print("fa_bwd_preprocess: B=%d H=%d N=%d d=%d dtype=%s; one wave per row",
                    B, H, N, d, dtype == FA_BF16 ? "bf16" : "f16");
  rc = check_device();
  if (rc) return rc;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_bwd_pre(p, dtype, d, (long)B * H * N, st);
  if (dbg) {
    const size_t rows = (size_t)B * H * N;
    debug_after("fa_bwd_preprocess", e, st,
                {{"o", o, rows * d, dtype}, {"dout", dout, rows * d, dtype}, {"lse", lse, rows, 2},
                 ws_neg_d(p, rows), ws_lse2(p, rows)});
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

int fa_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout, void *dk,
                void *dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                void *workspace, size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !dout || !dk || !dv || !workspace) return FA_ERR_NULL;
  fa::BwdParams p;
  fa_plan_t plan;
  int rc = bwd_setup(B, H, N, N, nullptr, nullptr, d, scale, causal, dtype, workspace,
                     workspace_bytes, &p, &plan);
  if (rc) return rc;
  if (!all_aligned({q, k, v, dout, dk, dv})) return FA_ERR_ALIGN;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    debug_bwd_plan("fa_bwd_dkdv", "dK/dV pass only", B, H, N, N, d, dtype, causal, scale, 0.f, false,
                   p, plan);
  rc = check_device();
  if (rc) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.dout = dout;
  p.dk = dk;
  p.dv = dv;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_bwd_dkdv(p, dtype, d, causal, p.n_ktiles * B * H, st);
  if (dbg) {
    const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    debug_after("fa_bwd_dkdv", e, st,
                {{"q", q, n, dtype}, {"k", k, n, dtype}, {"v", v, n, dtype}, {"dout", dout, n, dtype},
                 ws_neg_d(p, rows), ws_lse2(p, rows), {"dk", dk, n, dtype}, {"dv", dv, n, dtype}});
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // extern "C"

namespace {

// dQ pass of the staged backward; with o and lse it also computes the row
// statistics (the preprocessing step) instead of reading them
int dq_stage(const char *fn, const void *q, const void *k, const void *v, const void *o,
             const void *dout, const float *lse, void *dq, int B, int H, int N, int d, float scale,
             int causal, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
  fa::BwdParams p;
  fa_plan_t plan;
  int rc = bwd_setup(B, H, N, N, nullptr, nullptr, d, scale, causal, dtype, workspace,
                     workspace_bytes, &p, &plan);
  if (rc) return rc;
  const int pre = o != nullptr;
  if (!all_aligned({q, k, v, dout, dq}) || (pre && !all_aligned({o, lse}))) return FA_ERR_ALIGN;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    debug_bwd_plan(fn, pre ? "dQ pass with the row statistics" : "dQ pass only", B, H, N, N, d, dtype,
                   causal, scale, 0.f, false, p, plan);
  rc = check_device();
  if (rc) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const hipError_t e = fa::launch_bwd_dq(p, dtype, d, causal, pre, p.n_qtiles * B * H, st);
  if (dbg) {
    const size_t n = (size_t)B * H * N * d, rows = (size_t)B * H * N;
    if (pre)
      debug_after(fn, e, st,
                  {{"q", q, n, dtype}, {"k", k, n, dtype}, {"v", v, n, dtype}, {"o", o, n, dtype},
                   {"dout", dout, n, dtype}, {"lse", lse, rows, 2}, ws_neg_d(p, rows),
                   ws_lse2(p, rows), {"dq", dq, n, dtype}});
    else
      debug_after(fn, e, st,
                  {{"q", q, n, dtype}, {"k", k, n, dtype}, {"v", v, n, dtype}, {"dout", dout, n, dtype},
                   ws_neg_d(p, rows), ws_lse2(p, rows), {"dq", dq, n, dtype}});
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_bwd_dq(const void *q, const void *k, const void *v, const void *dout, void *dq, int B,
              int H, int N, int d, float scale, int causal, int dtype, void *workspace,
              size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !dout || !dq || !workspace) return FA_ERR_NULL;
  return dq_stage("fa_bwd_dq", q, k, v, nullptr, dout, nullptr, dq, B, H, N, d, scale, causal, dtype,
                  workspace, workspace_bytes, stream);
}

int fa_bwd_dq_preprocess(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, int B, int H, int N, int d,
                         float scale, int causal, int dtype, void *workspace,
                         size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !workspace) return FA_ERR_NULL;
  return dq_stage("fa_bwd_dq_preprocess", q, k, v, o, dout, lse, dq, B, H, N, d, scale, causal, dtype,
                  workspace, workspace_bytes, stream);
}

}  // extern "C"

namespace {

int bwd_impl(const char *fn, const void *q, const void *k, const void *v, const void *o,
             const void *dout, const float *lse, void *dq, void *dk, void *dv, const int *lq,
             const int *lk, int B, int H, int Nq, int Nk, int d, float scale, int causal,
             float dropout_p, uint64_t seed, uint32_t offset, int dtype, void *workspace,
             size_t workspace_bytes, void *stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv || !workspace) return FA_ERR_NULL;
  fa::BwdParams p;
  fa_plan_t plan;
  int rc = bwd_setup(B, H, Nq, Nk, lq, lk, d, scale, causal, dtype, workspace, workspace_bytes,
                     &p, &plan);
  if (rc) return rc;
  if (!dropout_spec(dropout_p, seed, offset, &p.drop)) return FA_ERR_ARG;
  if (!all_aligned({q, k, v, o, dout, lse, dq, dk, dv})) return FA_ERR_ALIGN;
  const bool dbg = fa::debug_enabled();
  if (dbg)
    debug_bwd_plan(fn, "dQ pass with the row statistics, then the dK/dV pass", B, H, Nq, Nk, d, dtype,
                   causal, scale, dropout_p, lq || lk, p, plan);
  rc = check_device();
  if (rc) return rc;
  p.q = q;
  p.k = k;
  p.v = v;
  p.o = o;
  p.dout = dout;
  p.lse = lse;
  p.dq = dq;
  p.dk = dk;
  p.dv = dv;
  const hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  // the dQ pass computes the row statistics the dK/dV pass then reads
  hipError_t e = fa::launch_bwd_dq(p, dtype, d, causal, 1, p.n_qtiles * B * H, st);
  if (e == hipSuccess) e = fa::launch_bwd_dkdv(p, dtype, d, causal, p.n_ktiles * B * H, st);
  if (dbg) {
    const size_t nq = (size_t)B * H * Nq, nk = (size_t)B * H * Nk;
    debug_after(fn, e, st,
                {{"q", q, nq * d, dtype}, {"k", k, nk * d, dtype}, {"v", v, nk * d, dtype},
                 {"o", o, nq * d, dtype}, {"dout", dout, nq * d, dtype}, {"lse", lse, nq, 2},
                 {"dq", dq, nq * d, dtype}, {"dk", dk, nk * d, dtype}, {"dv", dv, nk * d, dtype}},
                lq, lk, B, Nq, Nk);
  }
  return e == hipSuccess ? FA_OK : FA_ERR_LAUNCH;
}

}  // namespace

extern "C" {

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const void *dout,
           const float *lse, void *dq, void *dk, void *dv, int B, int H, int N, int d,
           float scale, int causal, int dtype, void *workspace, size_t workspace_bytes,
           void *stream) {
  return bwd_impl("fa_bwd", q, k, v, o, dout, lse, dq, dk, dv, nullptr, nullptr, B, H, N, N, d, scale,
                  causal, 0.f, 0, 0, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, void *dq, void *dk, void *dv, int B, int H, int N, int d,
                   float scale, int causal, int dtype, void *stream) {
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return FA_ERR_NULL;
  int rc = check_common(B, H, N, d, causal, dtype);
  if (rc) return rc;
  if ((long double)B * H * N > (long double)FA_BWD_NOALLOC_MAX_ROWS) return FA_ERR_SCRATCH;
  const size_t need = fa_bwd_workspace_size(B, H, N, d);
  if (need == 0 || need > kScratchBytes) return FA_ERR_SCRATCH;
  rc = check_device();
  if (rc) return rc;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return FA_ERR_DEVICE;
  void *ws = scratch_ptr(dev);
  if (!ws) return FA_ERR_DEVICE;
  return bwd_impl("fa_bwd_noalloc", q, k, v, o, dout, lse, dq, dk, dv, nullptr, nullptr, B, H, N, N,
                  d, scale, causal, 0.f, 0, 0, dtype, ws, kScratchBytes, stream);
}

int fa_bwd_padded(const void *q, const void *k, const void *v, const void *o, const void *dout,
                  const float *lse, void *dq, void *dk, void *dv, const int *seqlens_q,
                  const int *seqlens_k, int B, int H, int Nq, int Nk, int d, float scale,
                  int causal, int dtype, void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl("fa_bwd_padded", q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k, B, H, Nq,
                  Nk, d, scale, causal, 0.f, 0, 0, dtype, workspace, workspace_bytes, stream);
}

int fa_bwd_dropout(const void *q, const void *k, const void *v, const void *o, const void *dout,
                   const float *lse, void *dq, void *dk, void *dv, const int *seqlens_q,
                   const int *seqlens_k, int B, int H, int Nq, int Nk, int d, float scale,
                   int causal, float dropout_p, uint64_t seed, uint32_t offset, int dtype,
                   void *workspace, size_t workspace_bytes, void *stream) {
  return bwd_impl("fa_bwd_dropout", q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k, B, H, Nq,
                  Nk, d, scale, causal, dropout_p, seed, offset, dtype, workspace, workspace_bytes,
                  stream);
}

}  // extern "C"
