// fa_internal.h -- what the C-ABI layer hands to the kernel launcher.
#pragma once

#include "fa_ns.h"

#include <stdint.h>

FA_NS_BEGIN

// Tile shape of the forward kernel: a workgroup of fwd_waves(d) wavefronts
// owns fwd_block_m(d) = 32 * fwd_waves(d) query rows (32 per wave); K/V stream
// in blocks of kBlockN keys.  d = 128: 8 waves in two ping-pong groups, one
// workgroup per CU.  d = 64: 4 waves in one group, three workgroups per CU
// (the softmax-bound head size gains from more independent waves).
constexpr int fwd_waves(int d) { return d == 64 ? 4 : 8; }
constexpr int fwd_block_m(int d) { return 32 * fwd_waves(d); }
// Waves per SIMD the forward kernel is register-budgeted for: two at d = 128
// (one 8-wave workgroup per CU), three at d = 64 (three 4-wave workgroups).
constexpr int fwd_waves_per_simd(int d) { return d == 64 ? 3 : 2; }
constexpr int kBlockMMax = 256;   // the largest fwd_block_m (sizes its 32-bit offsets)
constexpr int kBlockN = 64;
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, one L2 each
// Largest rescale threshold for which the forward rounds P to fp16: P <= 2^tau
// must stay below fp16's largest finite value (65504); above it P is bf16.
constexpr float kMaxTauF16 = 15.0f;

enum class OutType : int { BF16 = 0, F32 = 1 };

struct FwdParams {
    const void *q;
    const void *k;
    const void *v;
    void *o;
    float *lse;
    const int32_t *offsets;   // varlen: int32 [B+1]; nullptr for fixed length
    int B, H, Nq, Nk;         // varlen: Nq = Nk = upper bound of the lengths
    int Hkv;                  // K/V heads (divides H)
    int group;                // H / Hkv: query head h reads K/V head h / group
    int num_m;                // query tiles per (batch, head) (upper bound for varlen)
    int num_tiles;            // grid size
    int lpt;                  // 1: longest-first order
    unsigned q_xor;           // applied to Q's bf16 pairs on load: (q ^ q_xor) & q_and
    unsigned q_and;
    float scale;              // |s|, used for LSE
    float scale_log2;         // exponent scale: |s| * log2(e) rounded once (1 when s = 0)
    float threshold;          // tau
    uint32_t *rescale_counts; // nullptr, or per-row counts of reference moves (layout of lse)
    uint64_t *trace;          // timeline build only: event stamps, kTraceEvents per traced wave
    int trace_workgroups;     // ... of the first trace_workgroups workgroups (waves 0 and 4)
    int exp2_poly;            // exponentials per 16 by the FMA polynomial: 0, 4, 8 or 16
};

// Timeline events (the trace build): code << 56 | shader clock, kTraceEvents
// slots for each of kTraceWaves waves per traced workgroup (d = 64 uses the
// first four).
constexpr int kTraceEvents = 1024;
constexpr int kTraceWaves = 8;
enum TraceEvent : unsigned {
    kTraceStart = 1, kTraceMBegin = 2, kTraceMEnd = 3, kTraceVBegin = 4, kTraceVEnd = 7,
    kTraceLoopEnd = 8, kTraceEnd = 9
};

// Enqueue the forward kernel; returns a hipError_t value (0 = success).
int launch_fwd(const FwdParams &p, int d, bool causal, OutType out, void *stream);

struct BwdParams {
    const void *q, *k, *v, *o, *dout;   // bf16 inputs (o: the forward's output)
    const float *lse;                   // the forward's LSE
    void *dq, *dk, *dv;                 // bf16 gradients
    float *dsum;                        // workspace: D_i = dO_i . O_i, layout of LSE
    const int32_t *offsets;             // varlen: int32 [B+1]; nullptr for fixed length
    int B, H, Hkv, group, Nq, Nk;       // varlen: Nq = Nk = upper bound of the lengths
    float scale;                        // s (any finite value)
    float scale_log2;                   // s * log2(e)
};

// Enqueue the backward kernels (row sums D, then dQ, then dK and dV).
int launch_bwd(const BwdParams &p, int d, bool causal, void *stream);

// The allocation-free backward keeps D (4 bytes per query row) in a static
// device array of this size, one per GPU.
constexpr int64_t kBwdScratchBytes = (int64_t)32 << 20;
constexpr int kMaxDevices = 64;
// Device address of that array on the current device (resolved once per
// device); 0 on success, -1 if the runtime could not resolve it.
int bwd_scratch(void **ptr);

// Enqueue the clock probe: n pairs (shader clock, constant-rate clock),
// interval_ticks of the constant-rate clock apart.
int launch_clock_probe(uint64_t *samples, int n, unsigned interval_ticks, void *stream);

FA_NS_END  // namespace fa
