// fa_fwd_kernel.hip -- FlashAttention forward for gfx950 (MI355X).
//
// What one workgroup computes ("Flash Attention 4", mlc.ai, section "algorithm
// structure"; "FlashAttention：一次前向计算", qingsen, section "general update"):
// for a tile of kBlockM query rows of one (batch, head) it walks the K/V blocks
// j = 0, 1, ... and keeps, per row, the exponent reference r, the running
// denominator l and the unnormalised output o:
//
//   S      = Q K_j^T                      (unscaled, fp32, MFMA)
//   S[masked] = -inf                      (causal / tail, before the maximum)
//   cand   = max(r, rowmax S)
//   delta  = (r - cand) * scale_log2      keep r while delta >= -tau,
//                                         else r = cand, alpha = exp2(delta)
//   P      = exp2(S * scale_log2 - r_safe * scale_log2)   r_safe = 0 if r = -inf
//   l      = l * alpha + rowsum bf16(P)
//   o      = o * alpha + bf16(P) V_j      (MFMA)
//
// and finally O = o / l (0 when l = 0) and LSE = ln l + r * scale ("Flash
// Attention 4", section "rescale and write-back": valid for any consistent
// reference).  O is normalised by the row sum of the bf16-rounded P that the
// PV product used, LSE by the fp32 row sum (see the softmax step).  The first block of a row starts from r = -inf, so delta = -inf
// switches to the candidate with alpha = 0 on a zero state, which is the
// page's first-block case (taken without evaluating delta, which would be
// -inf * 0 for scale 0).  A candidate of -inf (every key so far masked) keeps
// r = -inf with alpha = 1.  The row sum adds the same bf16-rounded P that the
// PV product uses (the pages sum P before rounding it): with a stale
// reference the dominant weight is 2^x rather than exactly 1, and summing the
// rounded values keeps O a convex combination of the V rows.
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
//   bf16, is directly the B operand (keys x queries) of O^T += V^T P^T for two
//   16-key steps; V^T is stored in LDS with the matching key permutation
//   (within each 16-key group, keys 4..7 and 8..11 trade places), so every
//   MFMA operand is one 16-byte LDS read.
// * O^T accumulates in registers with one query per lane, so the conditional
//   rescale multiplies a lane's own row by its own alpha; a wave skips the
//   multiply when no lane needs it (ballot), the CDNA analog of FA4's
//   per-warp any_sync test.
// * K and V^T blocks are double-buffered in LDS; the next block's global loads
//   are issued before the current block's MFMAs and written to the other
//   buffer afterwards, one barrier per block.  Row strides are padded by 16
//   bytes so the 16-byte operand reads of 16 lanes cover 64 distinct banks.
// * Tiles are mapped XCD-aware: workgroups are dispatched round-robin over the
//   8 XCDs, so XCD x is given a contiguous set of (batch, head) pairs and its
//   L2 holds their K/V.  Causal and varlen tiles go longest first (LPT,
//   "FlashAttention-4 (下)", section 6).
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "fa_internal.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int D_>
struct Tile {
    static constexpr int D = D_;
    static constexpr int BN = kBlockN;
    static constexpr int NW = kWaves;
    static constexpr int BM = kBlockM;
    static constexpr int NT = 64 * NW;        // threads per workgroup
    static constexpr int KS = D + 8;          // K row stride in LDS (bf16 elements)
    static constexpr int VS = BN + 8;         // V^T row stride in LDS
    static constexpr int K_ELEMS = BN * KS;
    static constexpr int V_ELEMS = D * VS;
    static constexpr int STAGE = K_ELEMS + V_ELEMS;
    static constexpr int LDS_BYTES = 2 * STAGE * 2;
    static constexpr int NKT = BN / 32;       // 32-key tiles of S^T per block
    static constexpr int NDS = D / 16;        // 16-wide head-dim steps of S^T
    static constexpr int NDT = D / 32;        // 32-wide head-dim tiles of O^T
    static constexpr int NKS = BN / 16;       // 16-key steps of O^T
    static constexpr int KCH = BN * D / 8;    // 16-byte chunks in a K block
    static constexpr int KPT = KCH / NT;      // ... per thread
    static constexpr int VU = (BN / 2) * (D / 8);   // (key pair, 8-dim chunk) units of a V block
    static constexpr int VPT = (VU + NT - 1) / NT;
    static_assert(KCH % NT == 0, "K block must split evenly over the threads");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
};

__device__ __forceinline__ float lane_pair_max(float x) {
    // Combine lanes l and l^32 (both halves see the maximum of the pair).
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_pair_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position of key kappa (0..15) inside its 16-key group of V^T in LDS: the
// S^T accumulator hands slot j of half g the key 8*(j/4) + 4*g + j%4, and the
// V^T operand of the same MFMA reads positions 8*g + j.
__device__ __forceinline__ int vt_pos16(int kappa) {
    return ((kappa >> 2) & 1) * 8 + (kappa & 3) + ((kappa >> 3) << 2);
}

// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
    const f32x2 f = {a, b};
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f, bf16x2));
}

// Sum of the two bf16 halves of a word, accumulated in fp32 (v_dot2 with (1, 1)).
__device__ __forceinline__ float add_bf16x2(unsigned word, float acc) {
    const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3F803F80u);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, word), ones, acc, false);
}

// ------------------------------------------------------------------ scheduler
// Map the workgroup index to (batch, head, query tile).  Returns false when
// the index names no tile (varlen: beyond the tiles of the actual lengths).
struct TileCoord {
    int b, h, m;
    int q_tok0;   // token index of this sequence's first query (packed or b*Nq)
    int k_tok0;
    int Nq, Nk;   // this sequence's lengths
};

__device__ __forceinline__ bool decode_fixed(int t, const FwdParams &p, TileCoord &c) {
    const int BH = p.B * p.H;
    const int nm = p.num_m;
    int bh, m;
    if (BH % kNumXcd == 0) {
        // Workgroup t runs on XCD t % 8; XCD x owns heads [x*HX, (x+1)*HX).
        const int x = t % kNumXcd, u = t / kNumXcd, HX = BH / kNumXcd;
        if (p.lpt) { m = nm - 1 - u / HX; bh = x * HX + u % HX; }
        else       { bh = x * HX + u / nm; m = u % nm; }
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

// Varlen, longest first: all tiles with query-tile index m = num_m-1 come
// first (every sequence long enough, in sequence order, heads innermost), then
// m = num_m-2, ...  Computed per wave from the offsets, with no host sync.
__device__ __forceinline__ bool decode_varlen(int t, const FwdParams &p, TileCoord &c) {
    const int lane = threadIdx.x & 63;
    const int32_t *off = p.offsets;
    int b = -1, m = -1, h = 0;
    if (p.lpt) {
        int rem = t;
        for (int lvl = p.num_m - 1; lvl >= 0 && b < 0; --lvl) {
            int cnt = 0;
            for (int b0 = 0; b0 < p.B; b0 += 64) {
                const int bb = b0 + lane;
                int nblk = 0;
                if (bb < p.B) nblk = (off[bb + 1] - off[bb] + kBlockM - 1) / kBlockM;
                cnt += __popcll(__ballot(nblk > lvl));
            }
            const int tiles = cnt * p.H;
            if (rem < tiles) {
                int target = rem / p.H;
                h = rem % p.H;
                for (int b0 = 0; b0 < p.B; b0 += 64) {
                    const int bb = b0 + lane;
                    int nblk = 0;
                    if (bb < p.B) nblk = (off[bb + 1] - off[bb] + kBlockM - 1) / kBlockM;
                    const unsigned long long mask = __ballot(nblk > lvl);
                    const int n = __popcll(mask);
                    if (target < n) {
                        const unsigned long long below = lane ? (mask & ((1ull << lane) - 1ull)) : 0ull;
                        const bool hit = ((mask >> lane) & 1ull) && __popcll(below) == target;
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
        if (m * kBlockM >= L) return false;
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
template <int D, bool CAUSAL, bool VARLEN, typename OutT>
__global__ __launch_bounds__(Tile<D>::NT) void fa_fwd_kernel(FwdParams p) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * T::STAGE];

    TileCoord tc;
    const bool ok = VARLEN ? decode_varlen(blockIdx.x, p, tc) : decode_fixed(blockIdx.x, p, tc);
    if (!ok) return;   // uniform over the workgroup

    const int tid = threadIdx.x;
    const int w = tid >> 6;
    const int lane = tid & 63;
    const int lq = lane & 31;
    const int g = lane >> 5;
    const int Nq = tc.Nq, Nk = tc.Nk;
    const int m0 = tc.m * T::BM;
    const int qw0 = m0 + 32 * w;          // first query row of this wave
    const int qrow = qw0 + lq;            // query row of this lane
    const bool row_ok = qrow < Nq;
    const int64_t tok = (int64_t)p.H * D; // elements between consecutive tokens
    const int causal_shift = Nk - Nq;     // bottom-right alignment

    const unsigned short *Qg = (const unsigned short *)p.q + (int64_t)tc.q_tok0 * tok + tc.h * D;
    const unsigned short *Kg = (const unsigned short *)p.k + (int64_t)tc.k_tok0 * tok + tc.h * D;
    const unsigned short *Vg = (const unsigned short *)p.v + (int64_t)tc.k_tok0 * tok + tc.h * D;

    // Number of K/V blocks this tile visits (fully masked blocks are never loaded).
    int nblocks = (Nk + T::BN - 1) / T::BN;
    if (CAUSAL) {
        const int last_row = min(m0 + T::BM, Nq) - 1;
        const int kmax = last_row + causal_shift;
        nblocks = kmax < 0 ? 0 : min(nblocks, kmax / T::BN + 1);
    }

    // Q fragments: B operand of S^T = K Q^T (query = lane % 32, 8 dims per half).
    bf16x8 qf[T::NDS];
#pragma unroll
    for (int ds = 0; ds < T::NDS; ++ds) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (row_ok) x = *(const u32x4 *)(Qg + (int64_t)qrow * tok + 16 * ds + 8 * g);
        x = (x ^ p.q_xor) & p.q_and;        // sign flip (scale < 0) or zero (scale = 0)
        qf[ds] = __builtin_bit_cast(bf16x8, x);
    }

    f32x16 oacc[T::NDT];
#pragma unroll
    for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[dt][i] = 0.f;

    float r = -INFINITY;     // exponent reference (unscaled score units)
    float lsum = 0.f;        // this lane's half of the row sum of bf16(P) (normalises O)
    float lsum32 = 0.f;      // ... of the fp32 P (gives LSE)
    const float c = p.scale_log2;
    const float tau = p.threshold;

    u32x4 kreg[T::KPT];
    u32x4 vreg[T::VPT][2];

    auto load_block = [&](int kb) {
        const int kv0 = kb * T::BN;
#pragma unroll
        for (int rr = 0; rr < T::KPT; ++rr) {
            const int u = tid + rr * T::NT;
            const int row = u / (D / 8), cc = u % (D / 8);
            const int key = kv0 + row;
            u32x4 x = {0u, 0u, 0u, 0u};
            if (key < Nk) x = *(const u32x4 *)(Kg + (int64_t)key * tok + 8 * cc);
            kreg[rr] = x;
        }
#pragma unroll
        for (int rr = 0; rr < T::VPT; ++rr) {
            const int u = tid + rr * T::NT;
            u32x4 x0 = {0u, 0u, 0u, 0u}, x1 = {0u, 0u, 0u, 0u};
            if (u < T::VU) {
                const int kp = u % (T::BN / 2), cc = u / (T::BN / 2);
                const int key = kv0 + 2 * kp;
                if (key < Nk) x0 = *(const u32x4 *)(Vg + (int64_t)key * tok + 8 * cc);
                if (key + 1 < Nk) x1 = *(const u32x4 *)(Vg + (int64_t)(key + 1) * tok + 8 * cc);
            }
            vreg[rr][0] = x0;
            vreg[rr][1] = x1;
        }
    };

    auto store_block = [&](int buf) {
        unsigned short *Ks = smem + buf * T::STAGE;
        unsigned short *Vt = Ks + T::K_ELEMS;
#pragma unroll
        for (int rr = 0; rr < T::KPT; ++rr) {
            const int u = tid + rr * T::NT;
            const int row = u / (D / 8), cc = u % (D / 8);
            *(u32x4 *)(Ks + row * T::KS + 8 * cc) = kreg[rr];
        }
#pragma unroll
        for (int rr = 0; rr < T::VPT; ++rr) {
            const int u = tid + rr * T::NT;
            if (u < T::VU) {
                const int kp = u % (T::BN / 2), cc = u / (T::BN / 2);
                const int key = 2 * kp;
                const int col = (key & ~15) + vt_pos16(key & 15);   // even; key+1 lands at col+1
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned a = vreg[rr][0][e >> 1], b = vreg[rr][1][e >> 1];
                    const unsigned word = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                                                  : ((a & 0xffffu) | (b << 16));
                    *(unsigned *)(Vt + (8 * cc + e) * T::VS + col) = word;
                }
            }
        }
    };

    if (nblocks > 0) {
        load_block(0);
        store_block(0);
        __syncthreads();
    }

    for (int kb = 0; kb < nblocks; ++kb) {
        const int buf = kb & 1;
        const bool more = kb + 1 < nblocks;
        if (more) load_block(kb + 1);

        const int kv0 = kb * T::BN;
        const int wave_last_row = min(qw0 + 31, Nq - 1);
        const bool active = qw0 < Nq && (!CAUSAL || kv0 <= wave_last_row + causal_shift);
        if (active) {
            const unsigned short *Ks = smem + buf * T::STAGE;
            const unsigned short *Vt = Ks + T::K_ELEMS;

            // S^T = K Q^T for the BN keys of the block.
            f32x16 s[T::NKT];
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
#pragma unroll
            for (int ds = 0; ds < T::NDS; ++ds) {
#pragma unroll
                for (int kt = 0; kt < T::NKT; ++kt) {
                    const bf16x8 kf = *(const bf16x8 *)(Ks + (32 * kt + lq) * T::KS + 16 * ds + 8 * g);
                    s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ds], s[kt], 0, 0, 0);
                }
            }

            // Mask keys past the end and, for causal, after the row's last key.
            const bool need_mask = (kv0 + T::BN > Nk) ||
                                   (CAUSAL && kv0 + T::BN - 1 > qw0 + causal_shift);
            if (need_mask) {
                const int lim = CAUSAL ? min(Nk - 1, qrow + causal_shift) : Nk - 1;
#pragma unroll
                for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int key = kv0 + 32 * kt + 8 * (i >> 2) + 4 * g + (i & 3);
                        if (key > lim) s[kt][i] = -INFINITY;
                    }
            }

            // Row maximum of the block and the rescale decision.
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kt][i]);
            mx = lane_pair_max(mx);
            const float cand = fmaxf(r, mx);
            float alpha = 1.f;
            if (cand != -INFINITY) {
                if (r == -INFINITY) {
                    // First block with a live key: take the candidate; the
                    // state is still zero, so alpha = 0 (exp2 of delta = -inf).
                    r = cand;
                    alpha = 0.f;
                } else {
                    const float delta = (r - cand) * c;
                    if (!(delta >= -tau)) {
                        r = cand;
                        alpha = __builtin_amdgcn_exp2f(delta);
                    }
                }
            }
            const float neg_rc = (r == -INFINITY) ? 0.f : -r * c;

            // P = exp2(S*c - r*c), rounded to bf16 for the PV MFMA.  The row
            // sum is taken over the same bf16 values (v_dot2 with (1, 1)), so
            // numerator and denominator see identical weights.
            float fsum0 = 0.f, fsum1 = 0.f;
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const float pv = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c, neg_rc));
                    s[kt][i] = pv;
                    if (i & 1) fsum1 += pv; else fsum0 += pv;
                }

            // (Words are kept in scalars: a bit cast of a vector element
            // reads element 0 in this compiler.)
            float bsum0 = 0.f, bsum1 = 0.f;
            bf16x8 pf[T::NKS];
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks) {
                const f32x16 &src = s[ks >> 1];
                const int i0 = 8 * (ks & 1);
                const unsigned w0 = pack_bf16x2(src[i0 + 0], src[i0 + 1]);
                const unsigned w1 = pack_bf16x2(src[i0 + 2], src[i0 + 3]);
                const unsigned w2 = pack_bf16x2(src[i0 + 4], src[i0 + 5]);
                const unsigned w3 = pack_bf16x2(src[i0 + 6], src[i0 + 7]);
                bsum0 = add_bf16x2(w0, bsum0);
                bsum1 = add_bf16x2(w1, bsum1);
                bsum0 = add_bf16x2(w2, bsum0);
                bsum1 = add_bf16x2(w3, bsum1);
                const u32x4 x = {w0, w1, w2, w3};
                pf[ks] = __builtin_bit_cast(bf16x8, x);
            }
            lsum = lsum * alpha + (bsum0 + bsum1);
            lsum32 = lsum32 * alpha + (fsum0 + fsum1);

            // Conditional rescale of the accumulator, skipped per wave when no
            // row of the wave moved its reference.
            if (__ballot(alpha != 1.f)) {
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
                    for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
            }

            // O^T += V^T P^T.
#pragma unroll
            for (int ks = 0; ks < T::NKS; ++ks) {
#pragma unroll
                for (int dt = 0; dt < T::NDT; ++dt) {
                    const bf16x8 vf = *(const bf16x8 *)(Vt + (32 * dt + lq) * T::VS + 16 * ks + 8 * g);
                    oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[dt], 0, 0, 0);
                }
            }
        }

        if (more) store_block(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: O = o / l, LSE = ln l + r * scale.
    const float l = lane_pair_sum(lsum);
    const float l32 = lane_pair_sum(lsum32);
    const float inv = l > 0.f ? 1.f / l : 0.f;
    if (row_ok) {
        OutT *Og = (OutT *)p.o + ((int64_t)tc.q_tok0 + qrow) * tok + tc.h * D;
#pragma unroll
        for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = 32 * dt + 8 * i4 + 4 * g;
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
        if (g == 0) {
            const float lse = l32 > 0.f ? logf(l32) + r * p.scale : -INFINITY;
            int64_t idx;
            if (VARLEN) idx = (int64_t)tc.h * p.offsets[p.B] + tc.q_tok0 + qrow;
            else        idx = ((int64_t)tc.b * p.H + tc.h) * Nq + qrow;
            p.lse[idx] = lse;
        }
    }
}

template <int D, bool CAUSAL, bool VARLEN, typename OutT>
static int launch_one(const FwdParams &p, hipStream_t stream) {
    hipLaunchKernelGGL((fa_fwd_kernel<D, CAUSAL, VARLEN, OutT>), dim3(p.num_tiles),
                       dim3(Tile<D>::NT), 0, stream, p);
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

}  // namespace fa
