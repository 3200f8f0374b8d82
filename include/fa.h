/*
 * Fused exact softmax attention for AMD Instinct MI355X (gfx950) -- C ABI.
 *
 * The operation (llmtrend.com page "FlashAttention", section on the bottleneck
 * of self-attention, and its four listed steps):
 *     O = softmax(Q K^T * scale [+ causal mask]) V
 * computed as one fused, tiled kernel: each workgroup keeps a block of query
 * rows on chip, streams K/V tiles through LDS and runs an online softmax (a
 * running row max and running row sum, rescaling the partial output; MHA tuning
 * handbook ch.3, sections "core idea" and "engineering implementation"), so the
 * N x N score matrix never reaches HBM.  The forward also writes the per-row
 * log-sum-exp (the same section's `lse` statistic), and the backward recomputes
 * the probabilities from it instead of storing them ("Flash Attention
 * application", section "Recomputation").
 *
 * Conventions shared by every entry point:
 *   - Tensors are device pointers to contiguous row-major [B][H][N][d] arrays of
 *     the 16-bit element type `dtype` (handbook ch.3 pseudocode layout
 *     [batch, num_heads, seq_len, head_dim]; inputs must be contiguous as the
 *     FA1-vs-FA2 page's troubleshooting section requires).  LSE and D are fp32
 *     [B][H][N].  Every pointer must be 16-byte aligned.
 *   - The caller owns all memory.  The library allocates nothing; the backward
 *     takes a caller-provided workspace of fa_bwd_workspace_size() bytes.
 *   - Only fp16 and bf16 are accepted ("Flash Attention application",
 *     recommended configuration: FP16/BF16 only), accumulation is fp32.
 *   - head_dim d must be 64 or 128.  Any N >= 1 is accepted; ragged tails are
 *     masked inside the kernels.
 *   - scale is any finite float (the pages use 1/sqrt(d_k) for it; 0 gives the
 *     plain mean of the visible V rows, a negative scale favours the smallest
 *     scores).  The mask is applied to the scaled scores, so it holds for every
 *     finite scale.
 *   - causal = 1 applies the lower-triangular mask of a square attention
 *     matrix: query i sees key j iff j <= i (handbook ch.3, notes on the causal
 *     mask: future positions are skipped); fully masked tiles are never loaded.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*, NULL =
 *     the null stream).  The return value reports argument and launch errors
 *     only; execution errors surface at the caller's next synchronisation.  No
 *     exception or abort crosses the ABI.  Global mutable state is limited to
 *     per-device caches and the static device arrays of fa_bwd_noalloc and of
 *     debug mode, so concurrent calls on different streams are safe (except
 *     overlapping fa_bwd_noalloc calls on one GPU, and debug mode's scans).
 *   - The device current at the call must be a gfx950 GPU, else FA_ERR_DEVICE
 *     (there is no fallback path).
 *   - Debug mode: with the environment variable FA_DEBUG (or
 *     FLASH_ATTENTION_DEBUG, the name the FA1-vs-FA2 page uses) set to anything
 *     but "0" (read at every call), each entry point that launches kernels prints
 *     its launch plan to stderr once its arguments have passed the host
 *     checks (before the device check), and after its launches waits for
 *     `stream` and prints, for each input and output, how many of its values
 *     are NaN, +inf and -inf (in an LSE, -inf marks a row that sees no key),
 *     after the per-batch lengths if the call takes them (values outside
 *     [0, N] are flagged: the kernels clamp them).
 *     This follows the advice to run a debug mode that looks for NaN values
 *     (FA1-vs-FA2 page, section 6.2, troubleshooting).  Results are
 *     unchanged; the call becomes synchronous.  While `stream` is being
 *     captured into a graph the scan is skipped.  Off by default.
 */
#ifndef FA_H_
#define FA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { FA_F16 = 0, FA_BF16 = 1 } fa_dtype_t;

typedef enum {
  FA_OK = 0,
  FA_ERR_NULL = 1,      /* a required pointer is NULL */
  FA_ERR_SHAPE = 2,     /* B, H or N < 1, or a head or the element count is too large */
  FA_ERR_HEAD_DIM = 3,  /* d not in {64, 128} */
  FA_ERR_DTYPE = 4,     /* dtype not FA_F16 / FA_BF16 */
  FA_ERR_ALIGN = 5,     /* a pointer is not 16-byte aligned */
  FA_ERR_WORKSPACE = 6, /* backward workspace too small */
  FA_ERR_DEVICE = 7,    /* current device is not gfx950, or no device */
  FA_ERR_LAUNCH = 8,    /* the HIP runtime rejected a kernel launch */
  FA_ERR_ARG = 9,       /* scale not finite, causal not 0/1, or dropout_p out of range */
  FA_ERR_SCRATCH = 10   /* fa_bwd_noalloc: B*H*N exceeds FA_BWD_NOALLOC_MAX_ROWS */
} fa_status_t;

/*
 * Forward.  Inputs q, k, v: [B][H][N][d] in `dtype`.  Outputs: o [B][H][N][d] in
 * `dtype` (rounded to nearest even from fp32), lse [B][H][N] fp32, the natural
 * log of the sum over visible keys of exp(scale * q_i . k_j).
 * Nothing is written when the call returns an error.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void *stream);

/*
 * Bytes of device workspace fa_bwd needs: -D = -rowsum(dO * O) and LSE * log2(e),
 * each fp32 [B][H][N] and 256-byte aligned.  Returns 0 for invalid shapes.
 */
size_t fa_bwd_workspace_size(int B, int H, int N, int d);

/*
 * Backward with recomputation ("Flash Attention application", section
 * "Recomputation"; its v2 section on re-parallelising the backward kernel).
 * Inputs: q, k, v, o (the forward's output), dout = dL/dO, all [B][H][N][d] in
 * `dtype`; lse [B][H][N] fp32 from fa_fwd with the same scale and causal flag.
 * Outputs: dq, dk, dv [B][H][N][d] in `dtype`.  The gradients are those of the
 * definition above:
 *   P = softmax(scale Q K^T [mask]), dV = P^T dO, dP = dO V^T,
 *   D_i = rowsum(dO_i * O_i), dS = P * (dP - D), dQ = scale dS K, dK = scale dS^T Q.
 * No atomics are used: dq, dk and dv are bitwise reproducible run to run.
 * `workspace` must hold fa_bwd_workspace_size(B,H,N,d) bytes (16-byte aligned);
 * its contents on entry do not matter and are clobbered.
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o,
           const void *dout, const float *lse, void *dq, void *dk, void *dv,
           int B, int H, int N, int d, float scale, int causal, int dtype,
           void *workspace, size_t workspace_bytes, void *stream);

/*
 * fa_bwd for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * arguments without the workspace, the same kernels and bitwise the same
 * results as fa_bwd.  The backward's row statistics (-D and LSE * log2(e),
 * 8 bytes per query row) live in a static device array of the library, one per
 * GPU, held until the process ends; the call allocates nothing (no hipMalloc,
 * hipFree or allocating library routine).  The array's device address is
 * looked up once per device, on the first call with that device current.
 * Limit: B*H*N <= FA_BWD_NOALLOC_MAX_ROWS (32 MiB of scratch), else
 * FA_ERR_SCRATCH.  Nothing in the array needs to start at zero: each call
 * writes every row statistic before reading it.  All calls on one GPU share
 * the array, so calls that overlap on one GPU (concurrent streams, threads, or
 * a captured graph replayed concurrently with another call) race and give
 * wrong results; calls on different GPUs are independent.
 */
#define FA_BWD_NOALLOC_MAX_ROWS 4194304
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse, void *dq, void *dk, void *dv,
                   int B, int H, int N, int d, float scale, int causal, int dtype,
                   void *stream);

/*
 * The stages of the backward, exposed so that a caller can schedule or time
 * them separately.  They share fa_bwd's argument rules and workspace layout.
 * Two orders give results bitwise equal to fa_bwd's (which runs the second):
 *   fa_bwd_preprocess -> fa_bwd_dkdv and fa_bwd_dq (these two in either order)
 *   fa_bwd_dq_preprocess -> fa_bwd_dkdv
 *
 * fa_bwd_preprocess: reads o, dout and lse; writes -D_i = -sum_c dO_ic O_ic and
 *   lse * log2(e) (fp32) into the workspace.
 * fa_bwd_dkdv: recomputes P and dS key-block by key-block; writes dk and dv.
 *   Reads the workspace written by either preprocessing stage.
 * fa_bwd_dq: recomputes P and dS query-block by query-block; writes dq.  Reads
 *   the workspace written by fa_bwd_preprocess.
 * fa_bwd_dq_preprocess: fa_bwd_dq that computes the row statistics itself from
 *   o, dout and lse (it needs no preprocessed workspace) and stores them in the
 *   workspace, as fa_bwd_preprocess does, for fa_bwd_dkdv.
 */
int fa_bwd_preprocess(const void *o, const void *dout, const float *lse, int B, int H,
                      int N, int d, int dtype, void *workspace, size_t workspace_bytes,
                      void *stream);
int fa_bwd_dkdv(const void *q, const void *k, const void *v, const void *dout, void *dk,
                void *dv, int B, int H, int N, int d, float scale, int causal, int dtype,
                void *workspace, size_t workspace_bytes, void *stream);
int fa_bwd_dq(const void *q, const void *k, const void *v, const void *dout, void *dq,
              int B, int H, int N, int d, float scale, int causal, int dtype,
              void *workspace, size_t workspace_bytes, void *stream);
int fa_bwd_dq_preprocess(const void *q, const void *k, const void *v, const void *o,
                         const void *dout, const float *lse, void *dq, int B, int H, int N,
                         int d, float scale, int causal, int dtype, void *workspace,
                         size_t workspace_bytes, void *stream);

/*
 * Padded batches and cross-attention.  "Flash Attention application"
 * (jsqmd.com), section "Notes", recommends the standard causal mask or a
 * padding mask; llmtrend.com's "Limitations" section notes that cross-attention
 * (queries and keys from different sequences) needs its own implementation.
 *
 * q, o, dout, dq: [B][H][Nq][d]; k, v, dk, dv: [B][H][Nk][d]; lse: [B][H][Nq]
 * fp32 (all contiguous, 16-byte aligned, in `dtype`).  seqlens_q / seqlens_k
 * are device int32 arrays [B] (4-byte aligned) giving the valid queries Lq[b]
 * and valid keys Lk[b] of each batch entry, or NULL for "all valid" (Nq, Nk).
 * Values are clamped to [0, Nq] and [0, Nk]; they are read on the device, so
 * they may be produced by earlier work on the same stream.
 *
 * For valid query i (< Lq) and valid key j (< Lk) the pair is visible iff
 * causal == 0 or j <= i + Lk - Lq, i.e. the causal diagonal ends at the last
 * query and the last key (for Lq == Lk this is the square rule of fa_fwd).
 * Outputs:
 *   - valid rows as in fa_fwd over their visible keys;
 *   - rows with no visible key (Lk == 0, or causal with i < Lq - Lk) and
 *     padding rows (i >= Lq): O = 0, LSE = -inf;
 *   - backward: dQ = 0 for those rows, dK = dV = 0 for padding keys (j >= Lk).
 * Padding entries of the inputs are never read as data.
 * fa_bwd_padded takes the forward's o and lse and a workspace of
 * fa_bwd_workspace_size(B, H, Nq, d) bytes; it has fa_bwd's other properties
 * (no atomics, bitwise reproducible).  Errors as for fa_fwd / fa_bwd, plus
 * FA_ERR_ALIGN for misaligned length arrays.
 */
int fa_fwd_padded(const void *q, const void *k, const void *v, void *o, float *lse,
                  const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, int dtype, void *stream);
int fa_bwd_padded(const void *q, const void *k, const void *v, const void *o,
                  const void *dout, const float *lse, void *dq, void *dk, void *dv,
                  const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                  int d, float scale, int causal, int dtype, void *workspace,
                  size_t workspace_bytes, void *stream);

/*
 * Dropout on the attention weights ("MHA tuning, part 1", section "notes in
 * practice": the dropout mask is generated block by block inside the fused
 * computation, and the backward regenerates the same mask instead of storing
 * it).  Arguments as for fa_fwd_padded / fa_bwd_padded, plus:
 *   dropout_p  drop probability in [0, 1), quantised to p8 = round(256 p),
 *              which must be <= 255 (else FA_ERR_ARG); p8 = 0 is no dropout;
 *   seed       64-bit key of the generator; offset: 32-bit stream offset, so
 *              successive calls (layers, steps) can use independent masks.
 * Pair (i, j) of head bh = b*H + h (i, j indices within the head) is kept iff
 * byte (j mod 4) of word (i mod 4) of Philox4x32-10 (Salmon, Moraes, Dror,
 * Shaw, SC'11) at counter (j/4, i/4, bh, offset) with key (seed low, seed high
 * 32 bits) is >= p8; kept weights are scaled by 256 / (256 - p8):
 *   O_i = sum_j P_ij Z_ij V_j,  Z_ij = keep_ij * 256 / (256 - p8),
 * with P (and LSE) the softmax before dropout.  The backward must be called
 * with the same dropout_p, seed and offset as the forward; its gradients are
 * those of this O (dV = (P Z)^T dO, dS = P (Z (dO V^T) - D)).  Deterministic:
 * the same arguments give the same mask and bitwise the same outputs.
 */
int fa_fwd_dropout(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, float dropout_p, uint64_t seed,
                   uint32_t offset, int dtype, void *stream);
int fa_bwd_dropout(const void *q, const void *k, const void *v, const void *o,
                   const void *dout, const float *lse, void *dq, void *dk, void *dv,
                   const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, float dropout_p, uint64_t seed,
                   uint32_t offset, int dtype, void *workspace, size_t workspace_bytes,
                   void *stream);

/*
 * Forward split over key blocks, for few queries over a long K/V (decoding
 * against a key/value cache; the xformers page's decoding benchmark and the
 * first-token latency scenario of "Flash Attention application").  The keys
 * of each (batch, head, query tile) are cut into chunks that run as separate
 * workgroups (with Nq = 1: separate waves of a streaming kernel on the vector
 * ALUs), so that B*H*ceil(Nq/128) small does not leave the GPU idle; each
 * chunk writes its normalised partial output and log-sum-exp, and a second
 * kernel merges the chunks with the LSE merge rule of the handbook's
 * engineering-implementation pseudocode:
 *   LSE = log sum_c exp(L_c),  O = sum_c exp(L_c - LSE) O_c.
 * Arguments and results as for fa_fwd_padded (the same function: padded
 * lengths, N_q != N_k, causal aligned to the last query and key); the
 * workspace must hold fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d) bytes
 * (16-byte aligned; fp32 partials), its contents on entry do not matter.
 * Results are deterministic but not bitwise equal to fa_fwd_padded's (the
 * additions happen in another order).  Forward only.
 */
size_t fa_fwd_splitkv_workspace_size(int B, int H, int Nq, int Nk, int d);
int fa_fwd_splitkv(const void *q, const void *k, const void *v, void *o, float *lse,
                   const int *seqlens_q, const int *seqlens_k, int B, int H, int Nq, int Nk,
                   int d, float scale, int causal, int dtype, void *workspace,
                   size_t workspace_bytes, void *stream);

/* Launch plan of a forward call (host-only, no GPU needed). */
typedef struct {
  int block_m;          /* query rows per workgroup */
  int block_n;          /* keys per K/V tile */
  int threads;          /* threads per workgroup */
  int grid;             /* workgroups (1-D grid) */
  int lds_bytes;        /* LDS per workgroup */
  int xcd_grouped;      /* 1 if heads are grouped per XCD */
} fa_plan_t;

/* Fills *plan for a forward with these arguments; returns a status code
 * (argument checks only, no device check). */
int fa_fwd_plan(int B, int H, int N, int d, int causal, int dtype,
                fa_plan_t *plan);

/* Fills *plan for the dK/dV pass of the backward (block_m = query rows per
 * inner step, block_n = keys per workgroup). */
int fa_bwd_plan(int B, int H, int N, int d, int causal, int dtype,
                fa_plan_t *plan);

/* Static description of a status code. */
const char *fa_status_str(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H_ */
