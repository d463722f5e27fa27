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

#include <type_traits>

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
    static constexpr int LDS_BYTES = (2 * K_ELEMS + 2 * V_ELEMS) * 2;
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
// Global loads go through buffer resources: a descriptor per K/V block whose
// range ends at the block's last valid key, so keys past the end read as 0
// with no branch and no address arithmetic per block.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, unsigned bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, unsigned voff) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0));
}

template <int D, bool CAUSAL, bool VARLEN, typename OutT>
__global__ __launch_bounds__(Tile<D>::NT) void fa_fwd_kernel(FwdParams p) {
    using T = Tile<D>;
    __shared__ __attribute__((aligned(16))) unsigned short smem[2 * T::K_ELEMS + 2 * T::V_ELEMS];
    unsigned short *const Kbuf0 = smem;
    unsigned short *const Kbuf1 = smem + T::K_ELEMS;
    unsigned short *const Vbuf0 = smem + 2 * T::K_ELEMS;
    unsigned short *const Vbuf1 = smem + 2 * T::K_ELEMS + T::V_ELEMS;

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
    const unsigned tokb = (unsigned)(tok * 2);   // ... in bytes
    const int causal_shift = Nk - Nq;     // bottom-right alignment
    const int wave_last_row = min(qw0 + 31, Nq - 1);

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
    // Bytes of the block's valid rows: the range of its buffer descriptor.
    auto block_bytes = [&](int kb) -> unsigned {
        const int rem = Nk - kb * T::BN;
        if (kb >= nblocks || rem <= 0) return 0u;
        return (unsigned)(min(rem, T::BN) - 1) * tokb + (unsigned)(D * 2);
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

    // Per-thread load/store coordinates, fixed for the whole tile.
    unsigned k_voff[T::KPT];
    int k_lds[T::KPT];
#pragma unroll
    for (int rr = 0; rr < T::KPT; ++rr) {
        const int u = tid + rr * T::NT;
        const int row = u / (D / 8), cc = u % (D / 8);
        k_voff[rr] = (unsigned)row * tokb + 16u * cc;
        k_lds[rr] = row * T::KS + 8 * cc;
    }
    unsigned v_voff[T::VPT];
    int v_lds[T::VPT];
    bool v_mine[T::VPT];
#pragma unroll
    for (int rr = 0; rr < T::VPT; ++rr) {
        const int u = tid + rr * T::NT;
        v_mine[rr] = u < T::VU;
        const int kp = (u % (T::BN / 2)), cc = (u / (T::BN / 2)) % (D / 8);
        const int key = 2 * kp;
        v_voff[rr] = (unsigned)key * tokb + 16u * cc;
        v_lds[rr] = 8 * cc * T::VS + (key & ~15) + vt_pos16(key & 15);
    }

    u32x4 kreg[T::KPT];
    u32x4 vreg[T::VPT][2];

    auto load_k = [&](int kb) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)kb * T::BN * tok, block_bytes(kb));
#pragma unroll
        for (int rr = 0; rr < T::KPT; ++rr) kreg[rr] = buffer_load16(rk, k_voff[rr]);
    };
    auto load_v = [&](int kb) {
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)kb * T::BN * tok, block_bytes(kb));
#pragma unroll
        for (int rr = 0; rr < T::VPT; ++rr) {
            vreg[rr][0] = buffer_load16(rv, v_voff[rr]);
            vreg[rr][1] = buffer_load16(rv, v_voff[rr] + tokb);
        }
    };
    auto store_k = [&](unsigned short *Ks) {
#pragma unroll
        for (int rr = 0; rr < T::KPT; ++rr) *(u32x4 *)(Ks + k_lds[rr]) = kreg[rr];
    };
    auto store_v = [&](unsigned short *Vt) {
#pragma unroll
        for (int rr = 0; rr < T::VPT; ++rr) {
            if (v_mine[rr]) {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const unsigned a = vreg[rr][0][e >> 1], b = vreg[rr][1][e >> 1];
                    const unsigned word = (e & 1) ? ((a >> 16) | (b & 0xffff0000u))
                                                  : ((a & 0xffffu) | (b << 16));
                    *(unsigned *)(Vt + v_lds[rr] + e * T::VS) = word;
                }
            }
        }
    };

    // S^T = K Q^T for the BN keys of a block.
    auto qk = [&](const unsigned short *Ks, f32x16 (&s)[T::NKT]) {
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
    };

    // O^T += V^T P^T, after the conditional rescale of O by alpha.
    auto rescale = [&](float alpha) {
        if (__ballot(alpha != 1.f)) {
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt)
#pragma unroll
                for (int i = 0; i < 16; ++i) oacc[dt][i] *= alpha;
        }
    };
    auto pv = [&](const unsigned short *Vt, const bf16x8 (&pf)[T::NKS]) {
#pragma unroll
        for (int ks = 0; ks < T::NKS; ++ks) {
#pragma unroll
            for (int dt = 0; dt < T::NDT; ++dt) {
                const bf16x8 vf = *(const bf16x8 *)(Vt + (32 * dt + lq) * T::VS + 16 * ks + 8 * g);
                oacc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[ks], oacc[dt], 0, 0, 0);
            }
        }
    };

    // Mask keys past the end and, for causal, after the row's last key (set
    // to -inf before the maximum).  Only blocks that cross a boundary pay.
    auto mask_block = [&](int kb, f32x16 (&s)[T::NKT]) {
        const int kv0 = kb * T::BN;
        const bool need_mask = (kv0 + T::BN > Nk) ||
                               (CAUSAL && kv0 + T::BN - 1 > qw0 + causal_shift);
        if (need_mask) {
            // Lane's last usable key, relative to its first key in the block.
            const int lim = (CAUSAL ? min(Nk - 1, qrow + causal_shift) : Nk - 1) - kv0 - 4 * g;
#pragma unroll
            for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
                for (int i = 0; i < 16; ++i)
                    if (32 * kt + 8 * (i >> 2) + (i & 3) > lim) s[kt][i] = -INFINITY;
        }
    };

    // Online softmax of one (masked) block: row max, rescale decision,
    // P = exp2, row sums, bf16 P.  Branch-free, so it can interleave with the
    // MFMAs of the previous block's PV product.  Returns alpha for O.
    auto softmax = [&](f32x16 (&s)[T::NKT], bf16x8 (&pf)[T::NKS]) -> float {
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
        const float alpha = move ? __builtin_amdgcn_exp2f(delta) : 1.f;
        r = move ? cand : r;
        const float neg_rc = (r == -INFINITY) ? 0.f : -r * c;

        // P = exp2(S*c - r*c), rounded to bf16 for the PV MFMA.  The row sum
        // for O is taken over the same bf16 values (v_dot2 with (1, 1)), so
        // numerator and denominator see identical weights; the fp32 sum
        // feeds LSE.  (Words are kept in scalars: a bit cast of a vector
        // element reads element 0 in this compiler.)
        float fsum0 = 0.f, fsum1 = 0.f;
#pragma unroll
        for (int kt = 0; kt < T::NKT; ++kt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv_ = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c, neg_rc));
                s[kt][i] = pv_;
                if (i & 1) fsum1 += pv_; else fsum0 += pv_;
            }
        float bsum0 = 0.f, bsum1 = 0.f;
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
        return alpha;
    };

    // One pipelined step: S_kb = Q K_kb^T, then O += P_{kb-1} V_{kb-1} while
    // the softmax of block kb runs.  K_kb is in Kc, V_{kb-1} in Vp; the
    // prefetched K_{kb+1} and V_kb are written to Kn and Vn.  P_j lives in
    // pfA for even j and pfB for odd j.  The mask code is compiled only into
    // the steps of blocks that cross a boundary (mask_tag true).
    f32x16 s[T::NKT];
    bf16x8 pfA[T::NKS], pfB[T::NKS];
    float alphaA = 1.f, alphaB = 1.f;
    auto step = [&](auto mask_tag, int kb, const unsigned short *Kc, const unsigned short *Vp,
                    unsigned short *Kn, unsigned short *Vn,
                    const bf16x8 (&p_in)[T::NKS], float alpha_in,
                    bf16x8 (&p_out)[T::NKS], float &alpha_out) {
        constexpr bool MASK = decltype(mask_tag)::value;
        load_k(kb + 1);
        load_v(kb);
        // A wave's live blocks are a prefix 0..last of the tile's blocks, so
        // for kb >= 1 "live kb" implies "live kb-1".
        if (active(kb)) {
            qk(Kc, s);
            if constexpr (MASK) mask_block(kb, s);
            rescale(alpha_in);
            pv(Vp, p_in);
            alpha_out = softmax(s, p_out);
            // One basic block holds the PV MFMAs and the softmax VALU work:
            // interleave them so the wave issues VALU while its MFMAs run.
#pragma unroll
            for (int i = 0; i < T::NKS * T::NDT; ++i) {
                __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // LDS read
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
            }
        } else if (active(kb - 1)) {
            rescale(alpha_in);
            pv(Vp, p_in);
        }
        store_k(Kn);
        store_v(Vn);
        __syncthreads();
    };
    using NoMask = std::integral_constant<bool, false>;
    using Mask = std::integral_constant<bool, true>;

    // Blocks below n_full need no mask for any row of the tile.
    int n_full = Nk / T::BN;
    if (CAUSAL) n_full = min(n_full, max(0, (m0 + causal_shift + 1) / T::BN));

    if (nblocks > 0) {
        load_k(0);
        store_k(Kbuf0);
        __syncthreads();
        load_k(1);
        load_v(0);
        if (active(0)) {
            qk(Kbuf0, s);
            mask_block(0, s);
            alphaA = softmax(s, pfA);
        }
        store_k(Kbuf1);
        store_v(Vbuf0);
        __syncthreads();
    }
    int kb = 1;
    for (; kb + 1 < n_full; kb += 2) {
        step(NoMask{}, kb, Kbuf1, Vbuf0, Kbuf0, Vbuf1, pfA, alphaA, pfB, alphaB);
        step(NoMask{}, kb + 1, Kbuf0, Vbuf1, Kbuf1, Vbuf0, pfB, alphaB, pfA, alphaA);
    }
    // kb is odd here, so the same buffer parity as above applies.
    for (; kb < nblocks; kb += 2) {
        step(Mask{}, kb, Kbuf1, Vbuf0, Kbuf0, Vbuf1, pfA, alphaA, pfB, alphaB);
        if (kb + 1 < nblocks)
            step(Mask{}, kb + 1, Kbuf0, Vbuf1, Kbuf1, Vbuf0, pfB, alphaB, pfA, alphaA);
    }
    if (nblocks > 0 && active(nblocks - 1)) {
        // P of the last block is in pfB when its index is odd, pfA when even.
        if ((nblocks - 1) & 1) {
            rescale(alphaB);
            pv(Vbuf1, pfB);
        } else {
            rescale(alphaA);
            pv(Vbuf0, pfA);
        }
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
