// fa_api.cpp -- the C ABI of libfa: argument checks, tile-count set-up, launch.
//
// Every argument check runs before the first HIP call, so a rejected call
// enqueues nothing and fa_fwd_check can run on a machine without a GPU.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/fa.h"
#include "fa_internal.h"

namespace {

constexpr int kVersion = 500;   // 0.5.0: fp16 P, fa_bwd_noalloc, the trace fields of fa_fwd_opts

bool aligned16(const void *ptr) { return ((uintptr_t)ptr & 15u) == 0; }

int check_args(const void *q, const void *k, const void *v, const void *o, const float *lse,
               int B, int H, int Nq, int Nk, int d, float scale, int causal,
               const int32_t *offsets, const fa_fwd_opts &opts) {
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse))
        return FA_ERR_INVALID_ARG;
    if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return FA_ERR_INVALID_ARG;
    if (causal != 0 && causal != 1) return FA_ERR_INVALID_ARG;
    if (!isfinite(scale)) return FA_ERR_INVALID_ARG;
    if (!isfinite(opts.rescale_threshold) || opts.rescale_threshold < 0.f ||
        opts.rescale_threshold > 64.f)
        return FA_ERR_INVALID_ARG;
    if (opts.schedule < FA_SCHEDULE_AUTO || opts.schedule > FA_SCHEDULE_LPT) return FA_ERR_INVALID_ARG;
    if (opts.kv_heads < 0 || opts.kv_heads > H || (opts.kv_heads > 0 && H % opts.kv_heads != 0))
        return FA_ERR_INVALID_ARG;
    if ((uintptr_t)opts.rescale_counts & 3u) return FA_ERR_INVALID_ARG;
    if (opts.trace) {
#ifdef FA_TRACE
        if (((uintptr_t)opts.trace & 7u) || opts.trace_workgroups < 1) return FA_ERR_INVALID_ARG;
#else
        return FA_ERR_UNSUPPORTED;   // only the timeline build records
#endif
    }
    if (opts.o_dtype != FA_DTYPE_BF16 && opts.o_dtype != FA_DTYPE_F32) return FA_ERR_UNSUPPORTED;
    if (opts.exp2_poly != 0) {
        if (opts.exp2_poly != 4 && opts.exp2_poly != 8 && opts.exp2_poly != 16) return FA_ERR_UNSUPPORTED;
        if (opts.rescale_threshold > fa::kMaxTauF16 || opts.rescale_counts ||
            opts.o_dtype != FA_DTYPE_BF16)
            return FA_ERR_UNSUPPORTED;
    }
    if (d != 64 && d != 128) return FA_ERR_UNSUPPORTED;
    if (offsets) {
        if ((uintptr_t)offsets & 3u) return FA_ERR_INVALID_ARG;
        if (Nq != Nk) return FA_ERR_INVALID_ARG;   // packed sequences attend to themselves
    }
    // Tile count and element offsets must fit the kernel's integer arithmetic.
    const int64_t num_m = ((int64_t)Nq + fa::fwd_block_m(d) - 1) / fa::fwd_block_m(d);
    if ((int64_t)B * H * num_m >= (int64_t)1 << 31) return FA_ERR_INVALID_ARG;
    // Byte offsets inside a tile's buffer descriptors are 32-bit: a 256-row
    // Q/O tile spans 256 * H * d * 2 bytes (the same bound for every head size).
    if ((int64_t)fa::kBlockMMax * H * d * 2 >= (int64_t)1 << 32) return FA_ERR_INVALID_ARG;
    if ((int64_t)B * Nq >= (int64_t)1 << 31 || (int64_t)B * Nk >= (int64_t)1 << 31)
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

int check_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
              const void *dout, const void *dq, const void *dk, const void *dv, const void *ws,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              const int32_t *offsets, int kv_heads) {
    fa_fwd_opts opts;
    fa_fwd_opts_default(&opts);
    opts.kv_heads = kv_heads;
    const int st = check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, offsets, opts);
    if (st != FA_OK) return st;
    if (!dout || !dq || !dk || !dv || !ws) return FA_ERR_INVALID_ARG;
    if (!aligned16(dout) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) ||
        ((uintptr_t)ws & 3u))
        return FA_ERR_INVALID_ARG;
    return FA_OK;
}

// Launch the backward with D in `dsum` (already checked arguments).
int run_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
            const void *dout, void *dq, void *dk, void *dv, float *dsum,
            int B, int H, int Nq, int Nk, int d, float scale, int causal,
            const int32_t *varlen_offsets, int kv_heads, void *stream) {
    fa::BwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.dout = dout;
    p.lse = lse;
    p.dq = dq;
    p.dk = dk;
    p.dv = dv;
    p.dsum = dsum;
    p.offsets = varlen_offsets;
    p.B = B;
    p.H = H;
    p.group = kv_heads > 0 ? H / kv_heads : 1;
    p.Hkv = H / p.group;
    p.Nq = Nq;
    p.Nk = Nk;
    p.scale = scale;
    // P = exp2(S * scale * log2 e - LSE * log2 e); scale_log2 computed in
    // double and rounded once, with its sign (LSE is given, no maximum kept).
    p.scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
    (void)hipGetLastError();
    const int err = fa::launch_bwd(p, d, causal != 0, stream);
    return err == 0 ? FA_OK : FA_ERR_HIP;
}

}  // namespace

extern "C" {

int64_t fa_bwd_workspace_size(int B, int H, int Nq) {
    if (B < 1 || H < 1 || Nq < 1) return 0;
    return (int64_t)4 * B * H * Nq;
}

int fa_bwd_check(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 const void *dout, const void *dq, const void *dk, const void *dv,
                 const void *workspace, int B, int H, int Nq, int Nk, int d, float scale,
                 int causal, const int32_t *varlen_offsets, int kv_heads) {
    return check_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale, causal,
                     varlen_offsets, kv_heads);
}

int fa_bwd(const void *q, const void *k, const void *v, const void *o, const float *lse,
           const void *dout, void *dq, void *dk, void *dv, void *workspace,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           const int32_t *varlen_offsets, int kv_heads, void *stream) {
    const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, B, H, Nq, Nk, d, scale,
                             causal, varlen_offsets, kv_heads);
    if (st != FA_OK) return st;
    return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, (float *)workspace, B, H, Nq, Nk, d, scale,
                   causal, varlen_offsets, kv_heads, stream);
}

int fa_bwd_noalloc_check(const void *q, const void *k, const void *v, const void *o,
                         const float *lse, const void *dout, const void *dq, const void *dk,
                         const void *dv, int B, int H, int Nq, int Nk, int d, float scale,
                         int causal, const int32_t *varlen_offsets, int kv_heads) {
    // The workspace check of fa_bwd is passed a stand-in: D goes to the
    // library's own array, whose size bounds the problem instead.
    const int st = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, (const void *)16, B, H, Nq, Nk, d,
                             scale, causal, varlen_offsets, kv_heads);
    if (st != FA_OK) return st;
    if (fa_bwd_workspace_size(B, H, Nq) > fa_bwd_noalloc_max_bytes()) return FA_ERR_TOO_LARGE;
    return FA_OK;
}

int fa_bwd_noalloc(const void *q, const void *k, const void *v, const void *o, const float *lse,
                   const void *dout, void *dq, void *dk, void *dv,
                   int B, int H, int Nq, int Nk, int d, float scale, int causal,
                   const int32_t *varlen_offsets, int kv_heads, void *stream) {
    const int st = fa_bwd_noalloc_check(q, k, v, o, lse, dout, dq, dk, dv, B, H, Nq, Nk, d, scale,
                                        causal, varlen_offsets, kv_heads);
    if (st != FA_OK) return st;
    void *dsum = nullptr;
    if (fa::bwd_scratch(&dsum) != 0) return FA_ERR_HIP;
    return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, (float *)dsum, B, H, Nq, Nk, d, scale,
                   causal, varlen_offsets, kv_heads, stream);
}

int64_t fa_bwd_noalloc_max_bytes(void) { return fa::kBwdScratchBytes; }

void fa_fwd_opts_default(fa_fwd_opts *opts) {
    if (!opts) return;
    opts->o_dtype = FA_DTYPE_BF16;
    opts->rescale_threshold = 8.0f;
    opts->schedule = FA_SCHEDULE_AUTO;
    opts->kv_heads = 0;
    opts->rescale_counts = nullptr;
    opts->trace = nullptr;
    opts->trace_workgroups = 0;
    opts->exp2_poly = 0;
}

int fa_fwd_check(const void *q, const void *k, const void *v, const void *o, const float *lse,
                 int B, int H, int Nq, int Nk, int d, float scale, int causal,
                 const int32_t *varlen_offsets, const fa_fwd_opts *opts) {
    fa_fwd_opts def;
    fa_fwd_opts_default(&def);
    return check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets,
                      opts ? *opts : def);
}

int fa_fwd_ex(const void *q, const void *k, const void *v, void *o, float *lse,
              int B, int H, int Nq, int Nk, int d, float scale, int causal,
              const int32_t *varlen_offsets, void *stream, const fa_fwd_opts *opts) {
    fa_fwd_opts op;
    fa_fwd_opts_default(&op);
    if (opts) op = *opts;
    const int st = check_args(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets, op);
    if (st != FA_OK) return st;

    fa::FwdParams p;
    p.q = q;
    p.k = k;
    p.v = v;
    p.o = o;
    p.lse = lse;
    p.offsets = varlen_offsets;
    p.B = B;
    p.H = H;
    p.group = op.kv_heads > 0 ? H / op.kv_heads : 1;   // query heads per K/V head
    p.Hkv = H / p.group;
    p.Nq = Nq;
    p.Nk = Nk;
    p.num_m = (Nq + fa::fwd_block_m(d) - 1) / fa::fwd_block_m(d);
    p.num_tiles = B * H * p.num_m;
    // Tiles of unequal work (causal rows, sequences of different lengths) run
    // longest first; with packed sequences that order is also the XCD-aware one.
    const bool lpt_default = causal != 0 || varlen_offsets != nullptr;
    p.lpt = op.schedule == FA_SCHEDULE_LPT ? 1 : op.schedule == FA_SCHEDULE_LINEAR ? 0 : lpt_default;
    // The kernel tracks the maximum of the unscaled scores, which is the
    // maximum of the scaled ones only for scale > 0.  A negative scale is
    // applied as softmax(|s| * (-Q) K^T) (negating bf16 Q is exact); scale 0
    // as softmax(1 * 0 K^T), which keeps masked scores at -inf instead of
    // -inf * 0.
    p.q_xor = 0u;
    p.q_and = 0xFFFFFFFFu;
    if (scale < 0.f) p.q_xor = 0x80008000u;
    p.scale = fabsf(scale);
    // scale_log2 = |scale| * log2(e), computed in double and rounded once.
    p.scale_log2 = (float)((double)p.scale * 1.4426950408889634073599246810019);
    if (scale == 0.f) {
        p.q_and = 0u;
        p.scale_log2 = 1.0f;
    }
    p.threshold = op.rescale_threshold;
    p.rescale_counts = op.rescale_counts;
    p.trace = op.trace;
    p.trace_workgroups = op.trace ? op.trace_workgroups : 0;
    p.exp2_poly = op.exp2_poly;

    // Clear a stale error so the status below belongs to this launch.
    (void)hipGetLastError();
    const int err = fa::launch_fwd(p, d, causal != 0,
                                   op.o_dtype == FA_DTYPE_F32 ? fa::OutType::F32 : fa::OutType::BF16,
                                   stream);
    return err == 0 ? FA_OK : FA_ERR_HIP;
}

int fa_fwd(const void *q, const void *k, const void *v, void *o, float *lse,
           int B, int H, int Nq, int Nk, int d, float scale, int causal,
           const int32_t *varlen_offsets, void *stream) {
    return fa_fwd_ex(q, k, v, o, lse, B, H, Nq, Nk, d, scale, causal, varlen_offsets, stream,
                     nullptr);
}

int fa_clock_probe(uint64_t *samples, int n, int interval_us, double *ref_hz, void *stream) {
    if (!samples || ((uintptr_t)samples & 7u) || n < 2 || n > 1000000 || interval_us < 1 ||
        interval_us > 100000 || !ref_hz)
        return FA_ERR_INVALID_ARG;
    int khz = 0;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess || khz <= 0)
        return FA_ERR_HIP;
    *ref_hz = 1000.0 * khz;
    const double ticks = 1e-3 * khz * interval_us;
    if (ticks < 1.0 || ticks > 1e7) return FA_ERR_INVALID_ARG;
    (void)hipGetLastError();
    const int err = fa::launch_clock_probe(samples, n, (unsigned)ticks, stream);
    return err == 0 ? FA_OK : FA_ERR_HIP;
}

const char *fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_INVALID_ARG: return "invalid argument";
        case FA_ERR_UNSUPPORTED: return "unsupported configuration";
        case FA_ERR_HIP: return "HIP runtime error at launch";
        case FA_ERR_TOO_LARGE:
            return "problem exceeds the static scratch array of fa_bwd_noalloc (use fa_bwd)";
        default: return "unknown status";
    }
}

int fa_version(void) { return kVersion; }

}  // extern "C"
