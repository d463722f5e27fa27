// fa_fwd_kernel.hip -- FlashAttention forward for gfx950 (MI355X).
//
// What one workgroup computes ("Flash Attention 4", mlc.ai, section "algorithm
// structure"; "FlashAttention：一次前向计算", qingsen, section "general update"):
// for a tile of fwd_block_m(d) query rows of one (batch, head) it walks the K/V blocks
// j = 0, 1, ... and keeps, per row, the exponent reference r, the running
// denominator l and the unnormalised output o:
//
//   S      = Q K_j^T                      (unscaled, fp32, MFMA)
//   S[masked] = -inf                      (causal / tail, before the maximum)
//   cand   = max(r, rowmax S)
//   delta  = (r - cand) * scale_log2      keep r while delta >= -tau,
//                                         else r = cand, alpha = exp2(delta)
//   P      = exp2(S * scale_log2 - r_safe * scale_log2)   r_safe = 0 if r = -inf
//   l      = l * alpha + rowsum fp16(P)
//   o      = o * alpha + fp16(P) V_j      (MFMA)
//
// and finally O = o / l (0 when l = 0) and LSE = ln l + r * scale ("Flash
// Attention 4", section "rescale and write-back": valid for any consistent
// reference).  The first block of a row starts from r = -inf, so delta = -inf
// switches to the candidate with alpha = 0 on a zero state, which is the
// page's first-block case (taken without evaluating delta, which would be
// -inf * 0 for scale 0).  A candidate of -inf (every key so far masked) keeps
// r = -inf with alpha = 1.
//
// P precision: the PV product takes fp16 operands, P rounded to fp16 as on the
// pages and V converted from bf16 as it is staged (exact below 2^16).  bf16 P
// (8 significant bits) is not enough for a bf16 O: with a stale reference the
// dominant weight 2^x is rounded by up to 2^-8, which on rows dominated by one
// or two keys adds up to ~4e-3 to O -- with the output's own rounding (up to
// 0.0078 for |O| in [2, 4)) more than the 1e-2 bar.  A tile whose V holds a
// finite value of 2^16 or more is computed again with V * 2^-vk (O scaled
// back exactly), and thresholds tau > 15, where P <= 2^tau can exceed fp16,
// use bf16 P and V.
//
// Two row sums: O is normalised by the sum of the same rounded P that the PV
// product uses (the pages sum P before rounding it; summing the rounded values
// keeps O a convex combination of the V rows), LSE by the fp32 sum of the
// unrounded P.
//
// Mapping onto CDNA4 (this is not the pages' Blackwell/Hopper/Ampere design):
//
// * Transposed scores.  Each wave owns 32 query rows and computes
//   S^T = K Q^T with v_mfma_f32_32x32x16_bf16: the accumulator layout puts one
//   query column in each lane (lane % 32) and 16 keys per 32-key tile in its
//   registers, keys 8*(i/4) + 4*(lane/32) + i%4.  Row max / row sum are then
//   in-lane reductions plus one exchange between the two 32-lane halves
//   (v_permlane32_swap), instead of the warp-quad shuffles of the pages.
// * P stays in registers.  The S^T accumulator of a 32-key tile, converted to
//   fp16, is directly the B operand (keys x queries) of O^T += V^T P^T for two
//   16-key steps.  The V^T operand comes from the row-major V tile by
//   ds_read_b64_tr_b16 transpose reads, two per MFMA.
// * O^T accumulates in registers with one query per lane, so the conditional
//   rescale multiplies a lane's own row by its own alpha; a wave skips the
//   multiply when no lane needs it (ballot), the CDNA analog of FA4's
//   per-warp any_sync test.
// * Ping-pong between the two waves of a SIMD (see the schedule below): one
//   wave issues its MFMAs (S_j and O += P_{j-1} V_{j-1}) while the other
//   runs its softmax on the VALU; workgroup barriers separate the phases.
//   This is the d = 128 shape (8 waves, 256 rows, one workgroup per CU).  At
//   d = 64 a workgroup is 4 waves (128 rows) with no phase offset and three
//   workgroups share a CU: there the softmax outweighs the products and more
//   independent waves issue more VALU work.
// * K and V blocks are double-buffered in LDS, staged through registers with
//   buffer loads (range-checked per block) one phase ahead.  K rows are
//   padded by 16 bytes and V rows swizzled (chunk c of row r at c ^ f(r)), so
//   the 16-byte K reads and the transpose reads meet no bank conflict.
// * Tiles are mapped XCD-aware: workgroups are dispatched round-robin over the
//   8 XCDs, so XCD x is given a contiguous set of (batch, head) pairs and its
//   L2 holds their K/V.  Causal tiles go longest first (LPT, "FlashAttention-4
//   (下)", section 6).  Packed sequences give XCD x an eighth of the heads of
//   every sequence and run each head's tiles together, longest first, so that
//   the tiles reading one head's K/V share the L2 (decode_varlen).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

FA_NS_BEGIN

template <int D_>
struct Tile {
    static constexpr int D = D_;
    static constexpr int BN = kBlockN;
    static constexpr int NW = fwd_waves(D_);
    static constexpr int BM = fwd_block_m(D_);
    static constexpr bool PINGPONG = NW == 8;   // two groups of 4 waves, one phase apart
    static constexpr int NT = 64 * NW;        // threads per workgroup
    static constexpr int KS = D + 8;          // K row stride in LDS (bf16 elements)
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = BN * D;    // V rows unpadded, 16-byte chunks swizzled
    static constexpr int LDS_BYTES = (2 * K_ELEMS + 2 * V_ELEMS) * 2;
    static constexpr int NKT = BN / 32;       // 32-key tiles of S^T per block
    static constexpr int NDS = D / 16;        // 16-wide head-dim steps of S^T
    static constexpr int NDT = D / 32;        // 32-wide head-dim tiles of O^T
    static constexpr int NKS = BN / 16;       // 16-key steps of O^T
    static constexpr int KCH = BN * D / 8;    // 16-byte chunks in a K block
    static constexpr int KPT = KCH / NT;      // ... per thread
    static_assert(KCH % NT == 0, "K block must split evenly over the threads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

// ------------------------------------------------------------------ scheduler
// Map the workgroup index to (batch, head, query tile).  Returns false when
// the index names no tile (varlen: beyond the tiles of the actual lengths).
struct TileCoord {
    int b, h, m;
    int q_tok0;   // token index of this sequence's first query (packed or b*Nq)
    int k_tok0;
    int Nq, Nk;   // this sequence's lengths
};

constexpr int kLptHeadGroup = 4;   // heads per group of the fixed-length longest-first order

__device__ __forceinline__ bool decode_fixed(int t, const FwdParams &p, TileCoord &c) {
    const int BH = p.B * p.H;
    const int nm = p.num_m;
    int bh, m;
    if (BH % kNumXcd == 0) {
        // Workgroups go round-robin over the 8 XCDs (from an XCD that depends
        // on the launches before), so the workgroups t with one value of
        // x = t % 8 share an XCD; they own heads [x*HX, (x+1)*HX).
        // Longest first, the XCD's heads in groups of kLptHeadGroup: all tiles
        // of one group (longest first across its heads) before the next
        // group's, so that the K/V of about that many heads, not of all HX,
        // is read at a time and stays in the XCD's L2; the next group's
        // longest tiles still start while the first group's short ones run.
        const int x = t % kNumXcd, u = t / kNumXcd, HX = BH / kNumXcd;
        if (p.lpt) {
            const int gs = HX % kLptHeadGroup == 0 ? kLptHeadGroup : HX;
            const int grp = u / (gs * nm), v = u % (gs * nm);
            m = nm - 1 - v / gs;
            bh = x * HX + grp * gs + v % gs;
        } else {
            bh = x * HX + u / nm;
            m = u % nm;
        }
    } else {
        if (p.lpt) { m = nm - 1 - t / BH; bh = t % BH; }
        else       { bh = t / nm; m = t % nm; }
    }
    c.b = bh / p.H;
    c.h = bh % p.H;
    c.m = m;
    c.Nq = p.Nq;
    c.Nk = p.Nk;
    c.q_tok0 = c.b * p.Nq;
    c.k_tok0 = c.b * p.Nk;
    return true;
}

// Varlen, longest first.  With H a multiple of 8, XCD-aware (below); else all
// tiles with query-tile index m = num_m-1 come first (every sequence long
// enough, in sequence order, heads innermost), then m = num_m-2, ...
// Computed per wave from the offsets, with no host sync.
template <int BM>
__device__ __forceinline__ bool decode_varlen(int t, const FwdParams &p, TileCoord &c) {
    const int lane = threadIdx.x & 63;
    const int32_t *off = p.offsets;
    int b = -1, m = -1, h = 0;
    if (p.lpt && p.H % kNumXcd == 0) {
        // The workgroups t with one value of x = t % 8 share an XCD (round-robin
        // dispatch), and they own query heads [x*HX, (x+1)*HX)
        // of every sequence (an eighth of the work for any lengths).  On an
        // XCD the tiles go sequence by sequence, head by head, each head's
        // tiles longest first, so the tiles that read one head's K/V run
        // together and share the XCD's L2.
        const int x = t % kNumXcd, HX = p.H / kNumXcd;
        const int u = t / kNumXcd;
        int base = 0;
        for (int b0 = 0; b0 < p.B && b < 0; b0 += 64) {
            const int bb = b0 + lane;
            const int nblk = bb < p.B ? (off[bb + 1] - off[bb] + BM - 1) / BM : 0;
            const int v = nblk * HX;
            int incl = v;     // inclusive prefix sum over the lanes
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const int o = __shfl_up(incl, s, 64);
                if (lane >= s) incl += o;
            }
            const int total = __builtin_amdgcn_readfirstlane(__shfl(incl, 63, 64));
            if (u < base + total) {
                const unsigned long long past = __ballot(base + incl > u);
                const int lb = __ffsll((long long)past) - 1;
                const int first = base + __builtin_amdgcn_readfirstlane(__shfl(incl - v, lb, 64));
                const int n = __builtin_amdgcn_readfirstlane(__shfl(nblk, lb, 64));
                const int r = u - first;
                b = b0 + lb;
                h = x * HX + r / n;
                m = n - 1 - r % n;
            }
            base += total;
        }
        if (b < 0) return false;
    } else if (p.lpt) {
        int rem = t;
        for (int lvl = p.num_m - 1; lvl >= 0 && b < 0; --lvl) {
            int cnt = 0;
            for (int b0 = 0; b0 < p.B; b0 += 64) {
                const int bb = b0 + lane;
                int nblk = 0;
                if (bb < p.B) nblk = (off[bb + 1] - off[bb] + BM - 1) / BM;
                cnt += __popcll(__ballot(nblk > lvl));
            }
            const int tiles = cnt * p.H;
            if (rem < tiles) {
                int target = rem / p.H;
                h = rem % p.H;
                for (int b0 = 0; b0 < p.B; b0 += 64) {
                    const int bb = b0 + lane;
                    int nblk = 0;
                    if (bb < p.B) nblk = (off[bb + 1] - off[bb] + BM - 1) / BM;
                    const unsigned long long mask = __ballot(nblk > lvl);
                    const int n = __popcll(mask);
                    if (target < n) {
                        const unsigned long long below = lane ? (mask & ((1ull << lane) - 1ull)) : 0ull;
                        const bool hit = ((mask >> lane) & 1ull) && (int)__popcll(below) == target;
                        const unsigned long long hm = __ballot(hit);
                        b = b0 + __ffsll((long long)hm) - 1;
                        m = lvl;
                        break;
                    }
                    target -= n;
                }
            }
            rem -= tiles;
        }
        if (b < 0) return false;
    } else {
        m = t % p.num_m;
        const int bh = t / p.num_m;
        b = bh / p.H;
        h = bh % p.H;
        const int L = off[b + 1] - off[b];
        if (m * BM >= L) return false;
    }
    const int start = off[b];
    const int L = off[b + 1] - start;
    c.b = b;
    c.h = h;
    c.m = m;
    c.Nq = L;
    c.Nk = L;
    c.q_tok0 = start;
    c.k_tok0 = start;
    return true;
}

// ------------------------------------------------------------------ kernel
template <int D, bool CAUSAL, bool VARLEN, typename OutT, bool COUNT, bool PV16, int EP>
__global__ __launch_bounds__(Tile<D>::NT, fwd_waves_per_simd(D)) void fa_fwd_kernel(FwdParams p) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * T::K_ELEMS + 2 * T::V_ELEMS];
    __shared__ unsigned vmax_bits;   // workgroup max of |V| (bit pattern), overflow path only
    __shared__ unsigned wave_bad[T::NW];   // per wave: a non-finite accumulator (overflow path)
    unsigned short *const Kbuf0 = smem;
    unsigned short *const Kbuf1 = smem + T::K_ELEMS;
    unsigned short *const Vbuf0 = smem + 2 * T::K_ELEMS;
    unsigned short *const Vbuf1 = smem + 2 * T::K_ELEMS + T::V_ELEMS;

    TileCoord tc;
    const bool ok = VARLEN ? decode_varlen<T::BM>(blockIdx.x, p, tc) : decode_fixed(blockIdx.x, p, tc);
    if (!ok) return;   // uniform over the workgroup

#ifdef FA_TRACE
    // Timeline build: lane 0 of every wave of the first trace_workgroups
    // workgroups records (event code << 56 | shader clock) at the phase
    // boundaries of the block loop into p.trace, kTraceEvents slots per wave
    // and kTraceWaves waves per workgroup.  Reading the clock waits for the
    // wave's outstanding LDS and scalar operations; at a phase boundary there
    // are none left to wait for (the barrier has just passed, or the phase's
    // last MFMA or exponential has been issued), so the stamps leave the
    // phases' lengths almost as they are.  A measurement tool, not the product.
    uint64_t *trace_out = nullptr;
    int trace_n = 0;
    if (p.trace && (int)blockIdx.x < p.trace_workgroups && (threadIdx.x & 63) == 0)
        trace_out = p.trace + ((int64_t)blockIdx.x * kTraceWaves + (threadIdx.x >> 6)) * kTraceEvents;
    auto mark = [&](unsigned code) {
        if (trace_out && trace_n < kTraceEvents)
            trace_out[trace_n++] = ((uint64_t)code << 56) | ((uint64_t)clock64() & 0x00FFFFFFFFFFFFFFull);
    };
#else
    auto mark = [](unsigned) {};
#endif
    mark(kTraceStart);

    const int tid = threadIdx.x;
    // Wave index, known wave-uniform (SGPR): keeps per-wave decisions and
    // the buffer descriptors that depend on it scalar.
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    const int Nq = tc.Nq, Nk = tc.Nk;
    const int m0 = tc.m * T::BM;
    const int qw0 = m0 + 32 * w;          // first query row of this wave
    const int64_t tok = (int64_t)p.H * D; // elements between consecutive Q/O tokens
    const int64_t tkv = (int64_t)p.Hkv * D;      // ... K/V tokens (grouped K/V heads)
    const unsigned tokb = (unsigned)(tok * 2);   // ... in bytes
    const unsigned tkvb = (unsigned)(tkv * 2);
    const int hkv = tc.h / p.group;       // the K/V head this query head reads
    const int causal_shift = Nk - Nq;     // bottom-right alignment
    const int wave_last_row = min(qw0 + 31, Nq - 1);

    const unsigned short *Qg = (const unsigned short *)p.q + (int64_t)tc.q_tok0 * tok + tc.h * D;
    const unsigned short *Kg = (const unsigned short *)p.k + (int64_t)tc.k_tok0 * tkv + hkv * D;
    const unsigned short *Vg = (const unsigned short *)p.v + (int64_t)tc.k_tok0 * tkv + hkv * D;

    // Number of K/V blocks this tile visits (fully masked blocks are never loaded).
    int nblocks = (Nk + T::BN - 1) / T::BN;
    if (CAUSAL) {
        const int last_row = min(m0 + T::BM, Nq) - 1;
        const int kmax = last_row + causal_shift;
        nblocks = kmax < 0 ? 0 : min(nblocks, kmax / T::BN + 1);
    }
    // Bytes of the block's valid rows: the range of its buffer descriptor.
    auto block_bytes = [&](int kb) -> unsigned {
        const int rem = Nk - kb * T::BN;
        if (kb >= nblocks || rem <= 0) return 0u;
        return (unsigned)(min(rem, T::BN) - 1) * tkvb + (unsigned)(D * 2);
    };
    auto active = [&](int kb) -> bool {   // does this wave have a live key in block kb?
        return qw0 < Nq && (!CAUSAL || kb * T::BN <= wave_last_row + causal_shift);
    };

    // Q fragments: B operand of S^T = K Q^T (query = lane % 32, 8 dims per half).
    bf16x8 qf[T::NDS];
    {
        const int rows = min(T::BM, Nq - m0);
        const __amdgpu_buffer_rsrc_t rq =
            make_rsrc(Qg + (int64_t)m0 * tok, (unsigned)(rows - 1) * tokb + (unsigned)(D * 2));
        const unsigned qoff = (unsigned)(32 * w + lq) * tokb + (unsigned)(16 * g);
#pragma unroll
        for (int ds = 0; ds < T::NDS; ++ds) {
            u32x4 x = buffer_load16(rq, qoff + 32u * ds);
            x = (x ^ p.q_xor) & p.q_and;      // sign flip (scale < 0) or zero (scale = 0)
            qf[ds] = __builtin_bit_cast(bf16x8, x);
        }
    }

    // Row state (reset by each run of the block loop below).
    f32x16 oacc[T::NDT];
    unsigned nmoves = 0;     // COUNT: reference moves after the row's first live block
    float r = -INFINITY;     // exponent reference (unscaled score units)
    float lsum = 0.f;        // this lane's half of the row sum of the rounded P (normalises O)
    float lsum32 = 0.f;      // ... of the fp32 P (gives LSE)
    const float c = p.scale_log2;
    const float tau = p.threshold;

    // ---------------------------------------------------------------------
    // Ping-pong schedule.  The 8 waves form two groups: waves 0-3 and 4-7;
    // wave w and wave w+4 share a SIMD.  Each iteration j of a wave has an
    // MFMA phase M(j) -- rescale O, S_j = Q K_j^T, O += P_{j-1} V_{j-1} --
    // and a VALU phase V(j) -- softmax of block j, LDS writes of prefetched
    // K/V, next global loads.  Group 1 runs one phase behind group 0, so on
    // every SIMD one wave issues MFMAs while the other issues VALU work.
    // Phases are separated by workgroup barriers; every wave executes the
    // same number of barriers.
    //
    //   slot 2j  : group 0 M(j)   group 1 V(j-1)
    //   slot 2j+1: group 0 V(j)   group 1 M(j)
    //
    // K_b lives in Kbuf[b % 2], V_b in Vbuf[b % 2].  Group g loads its part
    // of each block (K and V rows 32g..32g+31); in V(j) it
    // writes K_{j+1+g} and V_{j+g} (staged in registers one V phase earlier)
    // and issues the loads of K_{j+2+g} and V_{j+1+g}.  Every buffer is
    // written only after both groups' last reads of its previous block and
    // before the first read of the new one (one barrier apart).
    //
    // With 4 waves (d = 64) there is one group: M(j), V(j), barrier.  V(j)
    // writes the buffers M(j-1) read, and the barrier after V(j-1) orders
    // every wave's M(j-1) before any wave's V(j), so one barrier per block
    // suffices; the overlap of MFMA and VALU work comes from the other
    // workgroups on the CU.
    // ---------------------------------------------------------------------
    constexpr bool PP = T::PINGPONG;
    const int grp = PP ? w >> 2 : 0;
    const int gtid = PP ? tid & 255 : tid;

    // Per-thread load/store coordinates for this group's part of a block
    // (32 rows per group with the ping-pong, the whole block without).
    constexpr int GROWS = PP ? 32 : T::BN;
    constexpr int KPT2 = (GROWS * D / 8) / 256;     // 16-byte K chunks per thread
    static_assert(KPT2 >= 1 && (GROWS * D / 8) % 256 == 0, "block part must split over 256 threads");
    unsigned k_voff[KPT2];
    int k_lds[KPT2];
#pragma unroll
    for (int rr = 0; rr < KPT2; ++rr) {
        const int u = gtid + rr * 256;
        const int row = 32 * grp + u / (D / 8), cc = u % (D / 8);
        k_voff[rr] = (unsigned)row * tkvb + 16u * cc;
        k_lds[rr] = row * T::KS + 8 * cc;
    }
    int v_lds[KPT2];
#pragma unroll
    for (int rr = 0; rr < KPT2; ++rr) {
        const int u = gtid + rr * 256;
        const int row = 32 * grp + u / (D / 8);
        v_lds[rr] = row * D + (((u % (D / 8)) ^ vswz<D>(row)) << 3);
    }

    u32x4 kreg[KPT2];
    u32x4 vreg[KPT2];

    auto load_k = [&](int kb) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)kb * T::BN * tkv, block_bytes(kb));
#pragma unroll
        for (int rr = 0; rr < KPT2; ++rr) kreg[rr] = buffer_load16(rk, k_voff[rr]);
    };
    auto load_v = [&](int kb) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)kb * T::BN * tkv, block_bytes(kb));
#pragma unroll
        for (int rr = 0; rr < KPT2; ++rr) vreg[rr] = buffer_load16(rv, k_voff[rr]);
    };
    auto store_k = [&](unsigned short *Ks) {
#pragma unroll
        for (int rr = 0; rr < KPT2; ++rr) *(u32x4 *)(Ks + k_lds[rr]) = kreg[rr];
    };

    // S^T = K Q^T for the BN keys of a block.
    f32x16 s[T::NKT];
    auto qk = [&](const unsigned short *Ks) {
        constexpr int NR = T::NDS * T::NKT;       // K fragment reads, one MFMA each
        constexpr int AHEAD = NR < 8 ? NR : 8;    // reads in flight ahead of the MFMAs
        bf16x8 kf[T::NDS][T::NKT];
#pragma unroll
        for (int ds = 0; ds < T::NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
                kf[ds][kt] = *(const bf16x8 *)(Ks + (32 * kt + lq) * T::KS + 16 * ds + 8 * g);
#pragma unroll
        for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
        for (int ds = 0; ds < T::NDS; ++ds)
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
                s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[ds][kt], qf[ds], s[kt], 0, 0, 0);
        // Keep AHEAD fragment reads in flight (left alone, the scheduler
        // recycles one register pair and waits out the LDS latency for every
        // pair of MFMAs): reads first, then one MFMA per further read.
        __builtin_amdgcn_sched_group_barrier(0x100, AHEAD, 0);     // LDS reads
#pragma unroll
        for (int i = 0; i < NR - AHEAD; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
    };

    // O^T += V^T P^T, after the conditional rescale of O by alpha.  P^T is
    // held as raw 16-bit pairs (fp16 or bf16, the element type of the run).
    u32x4 pf[T::NKS];
    float alpha = 1.f;
    auto rescale = [&]() {
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        }
    };
    // V^T operand by transpose reads of the row-major V tile: source lane s
    // of each 16-lane group addresses V[row + s/4][col + 4*(s%4) .. +3], and
    // ds_read_b64_tr_b16 returns to lane i, element e, V[row + e][col + i].
    // Two reads give slots 0-3 (keys 4g..4g+3) and 4-7 (keys 8+4g..8+4g+3)
    // of the 16-key step, the key order of the P^T operand.
    // Offsets (elements) of this lane's transpose reads for each 32-wide
    // head-dim tile dt and key half h; key step ks adds 16 rows, which leaves
    // the swizzle unchanged.
    int v_off[T::NDT][2];
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int row = 4 * g + ((lane & 15) >> 2) + 8 * h;
            const int col = 32 * dt + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
            v_off[dt][h] = row * D + ((((col >> 3) ^ vswz<D>(row)) << 3) | (col & 7));
        }
    // Mask keys past the end and, for causal, after the row's last key (set
    // to -inf before the maximum).  Only blocks that cross a boundary pay.
    auto mask_block = [&](int kb) {
        const int kv0 = kb * T::BN;
        const bool need_mask = (kv0 + T::BN > Nk) ||
                               (CAUSAL && kv0 + T::BN - 1 > qw0 + causal_shift);
        if (need_mask) {
            // Lane's last usable key, relative to its first key in the block
            // (row and half from a fresh lane index: nothing lane-dependent
            // is held across the loop for the rare masked block).
            const int ln = fresh_lane();
            const int lim = (CAUSAL ? min(Nk - 1, qw0 + (ln & 31) + causal_shift) : Nk - 1) - kv0 - 4 * (ln >> 5);
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) s[kt][i] = -INFINITY;
        }
    };

    // The block loop.  With PV16 the PV product takes fp16 operands (as the
    // pages round P: 11 significant bits, so the rounding of the weights P,
    // numerator and denominator alike, stays far below that of a bf16 O),
    // with V converted from bf16 as it is staged, as V * 2^-vk (vk uniform,
    // normally 0); otherwise bf16 P and V.
    constexpr bool F16 = PV16;
    auto run = [&](int vk) {
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;
        nmoves = 0;
        r = -INFINITY;
        lsum = 0.f;
        lsum32 = 0.f;
        alpha = 1.f;

        auto store_v = [&](unsigned short *Vs) {
#pragma unroll
            for (int rr = 0; rr < KPT2; ++rr) {
                u32x4 x = vreg[rr];
                if constexpr (F16) {
                    if (vk == 0) {
                        x = u32x4{bf16x2_to_f16x2(x[0]), bf16x2_to_f16x2(x[1]), bf16x2_to_f16x2(x[2]),
                                  bf16x2_to_f16x2(x[3])};
                    } else {
                        const float sc = ldexpf(1.f, -vk);
                        const unsigned w0 = bf16x2_to_f16x2_scaled(x[0], sc), w1 = bf16x2_to_f16x2_scaled(x[1], sc);
                        const unsigned w2 = bf16x2_to_f16x2_scaled(x[2], sc), w3 = bf16x2_to_f16x2_scaled(x[3], sc);
                        x = u32x4{w0, w1, w2, w3};
                    }
                }
                *(u32x4 *)(Vs + v_lds[rr]) = x;
            }
        };

        auto pv = [&](const unsigned short *Vs) {
            // All V^T fragments read into their own registers, with AHEAD of
            // them (two transpose reads each) in flight ahead of the MFMAs:
            // left alone, the compiler recycled one register quad and waited
            // out the LDS latency before every MFMA.
            constexpr int NR = T::NKS * T::NDT;
            constexpr int AHEAD = NR < 8 ? NR : 8;
            i16x8 vf[T::NKS][T::NDT];
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks)
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) {
                    const unsigned short *a0 = Vs + 16 * ks * D;
                    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a0 + v_off[dt][0]));
                    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a0 + v_off[dt][1]));
                    vf[ks][dt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                }
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks)
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) {
                    if constexpr (F16)
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(
                            __builtin_bit_cast(f16x8, vf[ks][dt]), __builtin_bit_cast(f16x8, pf[ks]), oacc[dt], 0, 0, 0);
                    else
                        oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                            __builtin_bit_cast(bf16x8, vf[ks][dt]), __builtin_bit_cast(bf16x8, pf[ks]), oacc[dt], 0, 0, 0);
                }
            __builtin_amdgcn_sched_group_barrier(0x100, 2 * AHEAD, 0);     // LDS reads
#pragma unroll
            for (int i = 0; i < NR - AHEAD; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);         // MFMA
                __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x008, AHEAD, 0);
        };

        // Online softmax of one masked block: row max, rescale decision,
        // P = exp2, row sums, rounded P; sets alpha for the accumulator.
        auto softmax = [&]() {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
            mx = lane_pair_max(mx);
            const float cand = fmaxf(r, mx);
            // No live key so far (cand = -inf): keep r = -inf, alpha = 1.
            // First live block (r = -inf): take cand, alpha = exp2(-inf) = 0.
            // Otherwise keep r while delta = (r - cand) * c >= -tau.
            const bool live = cand != -INFINITY;
            const bool first = r == -INFINITY;
            const float delta = first ? -INFINITY : (r - cand) * c;
            const bool move = live && !(delta >= -tau);
            if constexpr (COUNT) nmoves += (move && !first) ? 1u : 0u;
            alpha = move ? __builtin_amdgcn_exp2f(delta) : 1.f;
            r = move ? cand : r;
            const float neg_rc = (r == -INFINITY) ? 0.f : -r * c;

            // P = exp2(S*c - r*c), rounded for the PV MFMA.  The row sum for O
            // is taken over the same rounded values (v_dot2 with (1, 1)), so
            // numerator and denominator see identical weights; the fp32 sum
            // feeds LSE.  (Words are kept in scalars: a bit cast of a vector
            // element reads element 0 in this compiler.)
            float fsum0 = 0.f, fsum1 = 0.f;
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    // EP of a lane's 16 exponentials per 32-key tile (every
                    // 16/EP-th) by the FMA polynomial, the rest by v_exp_f32.
                    const float xa = fmaf(s[kt][i], c, neg_rc);
                    const bool poly = EP > 0 && (i * EP) % 16 < EP;
                    const float pv_ = poly ? exp2_poly(xa) : __builtin_amdgcn_exp2f(xa);
                    s[kt][i] = pv_;
                    if (i & 1) fsum1 += pv_; else fsum0 += pv_;
                }
            float bsum0 = 0.f, bsum1 = 0.f;
            auto round_p = [&](auto f16c) {
                constexpr bool H = decltype(f16c)::value;
#pragma unroll
                for (int ks = 0; ks < T::NKS; ++ks) {
                    const f32x16 &src = s[ks >> 1];
                    const int i0 = 8 * (ks & 1);
                    unsigned w[4];
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        w[e] = H ? pack_f16x2(src[i0 + 2 * e], src[i0 + 2 * e + 1])
                                 : pack_bf16x2(src[i0 + 2 * e], src[i0 + 2 * e + 1]);
                    bsum0 = H ? add_f16x2(w[0], bsum0) : add_bf16x2(w[0], bsum0);
                    bsum1 = H ? add_f16x2(w[1], bsum1) : add_bf16x2(w[1], bsum1);
                    bsum0 = H ? add_f16x2(w[2], bsum0) : add_bf16x2(w[2], bsum0);
                    bsum1 = H ? add_f16x2(w[3], bsum1) : add_bf16x2(w[3], bsum1);
                    pf[ks] = u32x4{w[0], w[1], w[2], w[3]};
                }
            };
            round_p(std::integral_constant<bool, F16>{});
            lsum = lsum * alpha + (bsum0 + bsum1);
            lsum32 = lsum32 * alpha + (fsum0 + fsum1);
        };

        // The two phases.  j ranges: M(0..n), V(-1..n-1); out-of-range parts
        // are skipped (uniform per wave).
        const int n = nblocks;
        auto m_phase = [&](int j, const unsigned short *Kc, const unsigned short *Vp) {
            const bool do_pv = j >= 1 && j <= n && active(j - 1);
            const bool do_qk = j < n && active(j);
            mark(kTraceMBegin);
            if (do_pv) rescale();
            if (do_qk) qk(Kc);
            if (do_pv) pv(Vp);
            mark(kTraceMEnd);
        };
        auto v_phase = [&](int j, unsigned short *Kw, unsigned short *Vw) {
            mark(kTraceVBegin);
            if (j + 1 + grp < n) store_k(Kw);
            if (j + grp < n) store_v(Vw);
            load_k(j + 2 + grp);     // range 0 (reads nothing) past the last block
            load_v(j + 1 + grp);
            if (j >= 0 && j < n && active(j)) {
                mask_block(j);
                softmax();
            }
            mark(kTraceVEnd);
        };

        if (n > 0) {
            load_k(0);
            store_k(Kbuf0);
            load_k(1);
            load_v(0);
            __syncthreads();
            // Group 1 starts with V(-1) (LDS writes of K_1 and V_0, loads of the
            // next blocks) while group 0 runs M(0); from then on both groups run
            // M(j), V(j) pairs, group 1 one phase behind.  Group 0 ends with one
            // extra barrier so both groups meet the same number of barriers.
            // V(j) writes K_{j+1+grp} to Kbuf[(j+1+grp)%2] and V_{j+grp} to
            // Vbuf[(j+grp)%2].
            unsigned short *const Kw_even = grp ? Kbuf0 : Kbuf1;   // j even
            unsigned short *const Vw_even = grp ? Vbuf1 : Vbuf0;
            unsigned short *const Kw_odd = grp ? Kbuf1 : Kbuf0;    // j odd
            unsigned short *const Vw_odd = grp ? Vbuf0 : Vbuf1;
            if constexpr (PP) {
                if (grp == 1) {
                    v_phase(-1, Kw_odd, Vw_odd);
                    __syncthreads();
                }
                for (int j = 0; j <= n; j += 2) {
                    m_phase(j, Kbuf0, Vbuf1);
                    __syncthreads();
                    v_phase(j, Kw_even, Vw_even);
                    __syncthreads();
                    m_phase(j + 1, Kbuf1, Vbuf0);
                    __syncthreads();
                    v_phase(j + 1, Kw_odd, Vw_odd);
                    __syncthreads();
                }
                if (grp == 0) __syncthreads();
            } else {
                for (int j = 0; j <= n; j += 2) {
                    m_phase(j, Kbuf0, Vbuf1);
                    v_phase(j, Kw_even, Vw_even);
                    __syncthreads();
                    m_phase(j + 1, Kbuf1, Vbuf0);
                    v_phase(j + 1, Kw_odd, Vw_odd);
                    __syncthreads();
                }
            }
        }
    };

    // A finite V element of magnitude 2^16 or more has no fp16 value; it
    // becomes infinite, and since the PV product multiplies it by every row's
    // P (infinite for P > 0, NaN for P = 0), it leaves a non-finite value in
    // the accumulator of every row of the tile that visits its block -- which
    // finite inputs below 2^16 cannot (|P| <= 2^15).  Such a tile is computed
    // again with V staged as V * 2^-vk, vk from the largest |V| of its K/V
    // blocks (a separate pass over them), and O scaled back by 2^vk (exact).
    // The decision is the workgroup's (every wave takes the same branch), and
    // its barrier also orders the second run's LDS writes after the first
    // run's reads.  A V holding infinities or NaN keeps the first result: the
    // rows that see them are infinite or NaN, as with exact arithmetic.
    int vk = 0;
    for (;;) {   // one call site: the loop is inlined once
        run(vk);
        if (!PV16 || vk != 0) break;
        float t = 0.f;
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) t += oacc[dt][i];
        // Any wave with a non-finite sum?  One LDS word per wave (every lane
        // of a wave stores the same ballot result), one barrier.
        wave_bad[w] = __ballot(!(fabsf(t) <= 3.4028235e38f)) != 0 ? 1u : 0u;
        __syncthreads();
        unsigned any_bad = 0u;
#pragma unroll
        for (int i = 0; i < T::NW; ++i) any_bad |= wave_bad[i];
        if (!__builtin_amdgcn_readfirstlane(any_bad)) break;
        // Largest |V| over the tile's K/V blocks (rows past Nk read as 0).
        float vmax = 0.f;
        for (int kb = 0; kb < nblocks; ++kb) {
            const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)kb * T::BN * tkv, block_bytes(kb));
            for (int u = 64 * w + fresh_lane(); u < T::BN * D / 8; u += T::NT) {
                const u32x4 x = buffer_load16(rv, (unsigned)(u / (D / 8)) * tkvb + 16u * (u % (D / 8)));
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    vmax = fmaxf(vmax, fmaxf(fabsf(__uint_as_float(x[e] << 16)),
                                             fabsf(__uint_as_float(x[e] & 0xFFFF0000u))));
            }
        }
        if (w == 0 && fresh_lane() == 0) vmax_bits = 0u;
        __syncthreads();
        atomicMax(&vmax_bits, __float_as_uint(vmax));   // non-negative floats order as their bits
        __syncthreads();
        const float m = __uint_as_float(vmax_bits);
        if (!(m >= 65536.f && m <= 3.4028235e38f)) break;
        int e;
        (void)frexpf(m, &e);   // m < 2^e, so m * 2^-(e - 15) < 2^15
        vk = e - 15;
    }

    mark(kTraceLoopEnd);
    // Epilogue: O = o / l, LSE = ln l + r * scale.  The lane-dependent
    // values are computed again here rather than held across the loop.
    const int elane = fresh_lane(), elq = elane & 31, eg = elane >> 5;
    const int erow = qw0 + elq;
    const bool erow_ok = erow < Nq;
    const float l = lane_pair_sum(lsum);
    const float l32 = lane_pair_sum(lsum32);
    const float inv = l > 0.f ? ldexpf(1.f / l, vk) : 0.f;
    if constexpr (sizeof(OutT) == 2 && T::PINGPONG) {
        // bf16 O through LDS (d = 128): each wave puts its 32 x D tile into
        // the K/V buffers, free after the barrier below (16-byte chunks
        // XOR-swizzled by row, so the 8-byte writes of 32 rows meet at most
        // 2-way bank conflicts and the 16-byte reads none), and reads it back
        // by rows, so that each store instruction writes four whole rows of O
        // (16 lanes per row) instead of 16 bytes of each of 32 rows.  fp32 O
        // (twice the bytes) does not fit the buffers; at d = 64 the other
        // workgroups on the CU hide the direct stores, which then measure
        // faster.  Both store from the accumulator layout.
        constexpr int CPR = D / 8;                     // 16-byte chunks per row
        __syncthreads();                               // every wave is past its last K/V read
        unsigned short *Os = smem + w * 32 * D;
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int ch = 4 * dt + i4;
                const float o0 = oacc[dt][4 * i4 + 0] * inv, o1 = oacc[dt][4 * i4 + 1] * inv;
                const float o2 = oacc[dt][4 * i4 + 2] * inv, o3 = oacc[dt][4 * i4 + 3] * inv;
                *(uint2 *)(Os + elq * D + ((ch ^ (elq & (CPR - 1))) << 3) + 4 * eg) =
                    make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
            }
        unsigned short *Ob = (unsigned short *)p.o + ((int64_t)tc.q_tok0 + qw0) * tok + tc.h * D;
#pragma unroll
        for (int it = 0; it < 32 * CPR / 64; ++it) {
            const int u = 64 * it + elane, r = u / CPR, cc = u % CPR;
            const uint4 x = *(const uint4 *)(Os + r * D + ((cc ^ (r & (CPR - 1))) << 3));
            if (qw0 + r < Nq) *(uint4 *)(Ob + (int64_t)r * tok + 8 * cc) = x;
        }
    } else if (erow_ok) {
        OutT *Og = (OutT *)p.o + ((int64_t)tc.q_tok0 + erow) * tok + tc.h * D;
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = 32 * dt + 8 * i4 + 4 * eg;
                const float o0 = oacc[dt][4 * i4 + 0] * inv, o1 = oacc[dt][4 * i4 + 1] * inv;
                const float o2 = oacc[dt][4 * i4 + 2] * inv, o3 = oacc[dt][4 * i4 + 3] * inv;
                if constexpr (sizeof(OutT) == 4) {
                    float4 v4 = make_float4(o0, o1, o2, o3);
                    *(float4 *)((float *)Og + d0) = v4;
                } else {
                    uint2 v2 = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
                    *(uint2 *)((unsigned short *)Og + d0) = v2;
                }
            }
    }
    if (erow_ok) {
        if (eg == 0) {
            const float lse = l32 > 0.f ? logf(l32) + r * p.scale : -INFINITY;
            int64_t idx;
            if (VARLEN) idx = (int64_t)tc.h * p.offsets[p.B] + tc.q_tok0 + erow;
            else        idx = ((int64_t)tc.b * p.H + tc.h) * Nq + erow;
            p.lse[idx] = lse;
            if constexpr (COUNT) p.rescale_counts[idx] = nmoves;
        }
    }
    mark(kTraceEnd);
}

template <int D, bool CAUSAL, bool VARLEN, typename OutT, bool COUNT>
static void launch_pv(const FwdParams &p, hipStream_t stream) {
    // fp16 P needs P <= 2^tau below fp16's largest value 65504: tau <= 15.
    // The split exp2 is instantiated for the fp16 path with bf16 O and no
    // counts only (the C ABI refuses other combinations).
    if (p.threshold <= kMaxTauF16) {
        if constexpr (!COUNT && std::is_same<OutT, unsigned short>::value) {
            const dim3 g(p.num_tiles), b(Tile<D>::NT);
            switch (p.exp2_poly) {
                case 4: hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT, false, true, 4>), g, b, 0, stream, p); return;
                case 8: hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT, false, true, 8>), g, b, 0, stream, p); return;
                case 16: hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT, false, true, 16>), g, b, 0, stream, p); return;
                default: break;
            }
        }
        hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT, COUNT, true, 0>), dim3(p.num_tiles),
                           dim3(Tile<D>::NT), 0, stream, p);
    } else {
        hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT, COUNT, false, 0>), dim3(p.num_tiles),
                           dim3(Tile<D>::NT), 0, stream, p);
    }
}

template <int D, bool CAUSAL, bool VARLEN, typename OutT>
static int launch_one(const FwdParams &p, hipStream_t stream) {
    if (p.rescale_counts) launch_pv<D, CAUSAL, VARLEN, OutT, true>(p, stream);
    else                  launch_pv<D, CAUSAL, VARLEN, OutT, false>(p, stream);
    return (int)hipGetLastError();
}

template <int D, bool CAUSAL, bool VARLEN>
static int launch_out(const FwdParams &p, OutType out, hipStream_t s) {
    if (out == OutType::F32) return launch_one<D, CAUSAL, VARLEN, float>(p, s);
    return launch_one<D, CAUSAL, VARLEN, unsigned short>(p, s);
}

template <int D>
static int launch_d(const FwdParams &p, bool causal, OutType out, hipStream_t s) {
    const bool varlen = p.offsets != nullptr;
    if (causal) return varlen ? launch_out<D, true, true>(p, out, s) : launch_out<D, true, false>(p, out, s);
    return varlen ? launch_out<D, false, true>(p, out, s) : launch_out<D, false, false>(p, out, s);
}

int launch_fwd(const FwdParams &p, int d, bool causal, OutType out, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (p.num_tiles <= 0) return 0;
    if (d == 64) return launch_d<64>(p, causal, out, s);
    return launch_d<128>(p, causal, out, s);
}

FA_NS_END  // namespace fa

