/*
 * fa.h -- C ABI of libfa, a FlashAttention forward pass for AMD MI355X (gfx950).
 *
 * Operation (one call):
 *
 *     O   = softmax(scale * Q K^T) V        row-wise softmax over the keys
 *     LSE = ln sum_j exp(scale * q_i . k_j)  natural-log log-sum-exp per row
 *
 * as defined on "Flash Attention 4" (mlc.ai), section "algorithm structure"
 * (O_i = o_i / l_i with the online row state r_i, l_i, o_i) and on
 * "FlashAttention：一次前向计算" (qingsen), sections "what attention computes"
 * and "general update" (explicit scale s, L_i = s m_i + log l_i).  K/V are
 * visited block by block with the online-softmax row state; the score matrix
 * never reaches memory.  The exponent is base 2 with the scale folded in
 * (scale_log2 = scale * log2 e), and the reference of a row is only moved when
 * the new block maximum exceeds it by more than the rescale threshold tau
 * (FA4 page, "algorithm structure": keep the old reference while
 * delta >= -tau; tau = 8 by default, tau = 0 rescales whenever the maximum
 * grows).
 *
 * Causal masking is aligned to the bottom-right corner (FA4 page, section
 * "Causal Mask"): query i may use keys j <= i + Nk - Nq.  A row with no usable
 * key gets O = 0 and LSE = -inf.
 *
 * Grouped K/V heads (fa_fwd_ex, opts.kv_heads = Hkv; FA4 page, section "GQA
 * support"): Hkv divides H and the G = H / Hkv consecutive query heads
 * kv*G .. kv*G+G-1 share K/V head kv (Hkv = 1 is multi-query attention).
 * fa_fwd, and kv_heads = 0, mean Hkv = H.
 *
 * Conventions shared by every entry point:
 *   - q, k, v, o, lse and varlen_offsets are DEVICE pointers on the current
 *     HIP device; the caller owns them; libfa keeps no pointer after return.
 *   - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream).  A return of FA_OK means the kernel was enqueued.
 *   - Arguments are checked before any HIP call; a bad argument returns an
 *     error status and enqueues nothing.  No call aborts or prints.
 *   - Inputs are bf16 (raw 16-bit patterns).  O is bf16 by default (fp32 via
 *     fa_fwd_ex); LSE is fp32.
 *
 * Layouts (row-major, contiguous, head dimension fastest; Hkv = H unless
 * opts.kv_heads says otherwise):
 *   fixed length (varlen_offsets == NULL):
 *     q [B, Nq, H, d], k and v [B, Nk, Hkv, d], o [B, Nq, H, d], lse [B, H, Nq]
 *   packed variable length (varlen_offsets != NULL):
 *     varlen_offsets: int32 [B + 1], offsets[0] = 0, non-decreasing; sequence
 *     b holds tokens offsets[b] .. offsets[b+1]-1 and attends to itself
 *     (self attention, Nq = Nk = its length).  With T = offsets[B]:
 *     q, o [T, H, d], k, v [T, Hkv, d], lse [H, T].  Nq and Nk must both equal an upper
 *     bound of every sequence length (normally the maximum).  The device reads
 *     the offsets; they are not validated -- offsets that decrease, exceed T
 *     or a length above Nq are undefined behaviour.
 *
 * Supported: d in {64, 128}; B, H, Nq, Nk >= 1; any Nq, Nk (tails masked);
 * pointers 16-byte aligned; B*H*ceil(Nq/256) below 2^31; H*d below 2^23;
 * B*Nq and B*Nk below 2^31.
 */
#ifndef LIBFA_FA_H
#define LIBFA_FA_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
typedef enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = -1,   /* null/misaligned pointer, size <= 0, bad option value */
    FA_ERR_UNSUPPORTED = -2,   /* well-formed but not implemented: d not 64/128, dtype */
    FA_ERR_HIP = -3,           /* the HIP runtime reported an error at launch */
    FA_ERR_TOO_LARGE = -4      /* fa_bwd_noalloc: the problem exceeds its static scratch array */
} fa_status;

/* Element type of O. */
typedef enum fa_dtype {
    FA_DTYPE_BF16 = 0,
    FA_DTYPE_F32 = 1
} fa_dtype;

/* Tile order. AUTO = longest-first (LPT) for causal or varlen, linear otherwise. */
typedef enum fa_schedule {
    FA_SCHEDULE_AUTO = 0,
    FA_SCHEDULE_LINEAR = 1,
    FA_SCHEDULE_LPT = 2
} fa_schedule;

/*
 * Options of fa_fwd_ex.
 *   o_dtype           : fa_dtype of O (default FA_DTYPE_BF16).
 *   rescale_threshold : tau in base-2 exponent units, finite, 0 <= tau <= 64
 *                       (default 8).  0 = always rescale when the row maximum
 *                       grows.  The upper bound keeps P <= 2^tau and the row
 *                       sum finite in fp32.
 *   schedule          : fa_schedule (default FA_SCHEDULE_AUTO).
 *   kv_heads          : number of K/V heads Hkv; 0 (the default) means H,
 *                       otherwise 1 <= Hkv <= H and Hkv divides H.
 *   rescale_counts    : NULL (the default), or device memory, 4-byte aligned,
 *                       of one uint32 per query row laid out like lse
 *                       ([B, H, Nq], or [H, T] for varlen), owned by the caller.
 *                       When given, each row's count of rescale events is
 *                       written: the K/V blocks after the row's first one with a
 *                       valid key at which its exponent reference moved
 *                       ("Flash Attention 4", section "algorithm structure":
 *                       delta < -tau).  Diagnostics: the computation and the
 *                       other outputs are the same; without it the kernels
 *                       carry no counting code.
 *   trace, trace_workgroups : NULL / 0 (the defaults).  Only the timeline
 *                       build of the library (libfa_trace.so, compiled with
 *                       FA_TRACE) accepts a trace buffer: device memory,
 *                       8-byte aligned, of trace_workgroups * 8 * 1024 uint64,
 *                       owned by the caller.  Lane 0 of every wave w (0..7;
 *                       0..3 at d = 64) of each of the first trace_workgroups
 *                       workgroups writes up to 1024 stamps (event << 56 |
 *                       shader clock) at the phase boundaries of the block loop
 *                       into slots [(wg * 8 + w) * 1024, +1024); unused slots
 *                       keep their contents.  The default library returns
 *                       FA_ERR_UNSUPPORTED for a non-NULL trace.
 *   exp2_poly         : 0 (the default), 4, 8 or 16: the split exp2 of
 *                       "Flash Attention 4" (section "algorithm structure"),
 *                       where part of the exponentials P = 2^x runs on the
 *                       FMA pipes as 2^floor(x) * p(x - floor(x)), p a cubic
 *                       of relative error below 7.5e-5 on [0, 1).  The value
 *                       is how many of each 16 use the polynomial (evenly
 *                       spread), the rest the hardware exp2.  Supported with
 *                       bf16 O, rescale_threshold <= 15 and no
 *                       rescale_counts (FA_ERR_UNSUPPORTED otherwise).  Off
 *                       by default: on gfx950 the transcendental unit is
 *                       faster per element than the polynomial's eight VALU
 *                       instructions.
 */
typedef struct fa_fwd_opts {
    int32_t o_dtype;
    float rescale_threshold;
    int32_t schedule;
    int32_t kv_heads;
    uint32_t *rescale_counts;
    uint64_t *trace;
    int32_t trace_workgroups;
    int32_t exp2_poly;
} fa_fwd_opts;

/* Fill *opts with the defaults (bf16 O, tau = 8, automatic schedule, Hkv = H,
 * no rescale counts, no trace). */
void fa_fwd_opts_default(fa_fwd_opts *opts);

/*
 * Attention forward with the default options.  scale is explicit (there is
 * no default; 1/sqrt(d) is the usual choice); it may be any finite value.
 * causal: 0 = full attention, 1 = bottom-right causal mask.
 * Returns a fa_status.
 */
int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           const int32_t *varlen_offsets, void *stream);

/* As fa_fwd, with options (opts == NULL means the defaults). */
int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              const int32_t *varlen_offsets, void *stream, const fa_fwd_opts *opts);

/*
 * The argument checks of fa_fwd_ex alone: returns the status fa_fwd_ex would
 * return before launching, and makes no HIP call (usable without a GPU).
 */
int fa_fwd_check(const void *q, const void *k, const void *v, const void *o,
                 const float *lse, int B, int H, int Nq, int Nk, int d, float scale,
                 int causal, const int32_t *varlen_offsets, const fa_fwd_opts *opts);

/*
 * Backward pass: the gradients dQ, dK, dV of the forward's O for an upstream
 * gradient dO ("FlashAttention-4（下）", argus-lessons, section 1: recompute S
 * and P, then dP = dO V^T, dV = P^T dO, dS = P (dP - rowsum(dO O)),
 * dQ = scale dS K, dK = scale dS^T Q).
 *
 *   q, k, v      : the forward's inputs (bf16), layouts as for fa_fwd_ex
 *   o, lse       : the forward's outputs for these inputs (o bf16, lse fp32)
 *   dout         : dO, bf16, laid out like o
 *   dq           : bf16, like q; dk, dv: bf16, like k and v
 *   workspace    : device memory of fa_bwd_workspace_size(B, H, Nq) bytes,
 *                  owned by the caller, 4-byte aligned; its contents are
 *                  scratch (no state is kept across calls)
 *   kv_heads     : K/V heads Hkv (0 = H), as opts.kv_heads of fa_fwd_ex;
 *                  dk and dv sum over the query heads of each K/V head
 *   scale, causal, varlen_offsets, B, H, Nq, Nk, d, stream: as for fa_fwd_ex
 *
 * The result is deterministic: no atomics; dQ and dK/dV are reduced by two
 * kernels in a fixed order.  Checks and errors as for fa_fwd_ex (plus null
 * or misaligned o, dout, dq, dk, dv, workspace).
 */
int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, void *workspace,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           const int32_t *varlen_offsets, int kv_heads, void *stream);

/* Bytes of workspace fa_bwd needs (4 * B * H * Nq; for varlen B * Nq bounds
 * the packed token count). */
int64_t fa_bwd_workspace_size(int B, int H, int Nq);

/* The argument checks of fa_bwd alone (no HIP call). */
int fa_bwd_check(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, const void *dq, const void *dk, const void *dv,
                 const void *workspace, int B, int H, int Nq, int Nk, int d, float scale,
                 int causal, const int32_t *varlen_offsets, int kv_heads);

/*
 * fa_bwd without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, layouts, checks and results as fa_bwd, bit for
 * bit (the same kernels), except that the row terms D live in a static device
 * array of the library, fa_bwd_noalloc_max_bytes() bytes (32 MiB) per GPU,
 * held from the library's first use on that GPU until the process ends.
 *   - The call allocates nothing (no hipMalloc/hipFree); on a GPU's first
 *     call it looks up the array's address there (hipGetSymbolAddress).
 *   - It returns FA_ERR_TOO_LARGE, launching nothing, when
 *     fa_bwd_workspace_size(B, H, Nq) exceeds that size (B*H*Nq above 2^23).
 *   - Every call on one GPU uses that GPU's one array: calls that overlap in
 *     time on one GPU (several streams, several host threads) race and give
 *     undefined results.  Calls in one stream order are safe; the array keeps
 *     the last call's values, and each call writes every entry it reads.
 */
int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   const int32_t *varlen_offsets, int kv_heads, void *stream);

/* The argument checks of fa_bwd_noalloc alone (no HIP call). */
int fa_bwd_noalloc_check(const void *q, const void *k, const void *v, const void *o,
                         const float *lse, const void *dout, const void *dq, const void *dk,
                         const void *dv, int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, const int32_t *varlen_offsets, int kv_heads);

/* Size in bytes of fa_bwd_noalloc's static array (the bound on 4*B*H*Nq). */
int64_t fa_bwd_noalloc_max_bytes(void);

/*
 * Diagnostics, no part of the attention computation: measure the compute-unit
 * (shader) clock, against which matrix-core throughput is priced.  One
 * wavefront is launched on `stream` and records n pairs of 64-bit counts,
 * samples[2*i] = shader-clock cycles and samples[2*i+1] = ticks of the
 * device's constant-rate clock, interval_us microseconds apart on the latter.
 * The clock over a window is (shader delta) / (constant delta) * *ref_hz.
 * Launch it on a second stream beside the work being measured; it sleeps
 * between samples.
 *   samples   : device memory of 2*n uint64, 8-byte aligned, caller-owned
 *   n         : 2 .. 1000000;  interval_us: 1 .. 100000
 *   ref_hz    : host pointer; receives the constant-rate clock's frequency
 * Returns FA_ERR_INVALID_ARG for bad arguments (nothing launched), FA_ERR_HIP
 * if the device query or the launch fails.
 */
int fa_clock_probe(uint64_t *samples, int n, int interval_us, double *ref_hz, void *stream);

/* A static, NUL-terminated description of a status code. */
const char *fa_status_string(int status);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int fa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFA_FA_H */
