// fa_bwd_kernel.hip -- FlashAttention backward for gfx950 (MI355X).
//
// What is computed ("FlashAttention-4（下）", argus-lessons, section 1: the
// backward recomputes S and P and forms the products dP, dV, dQ and dK):
// for one (batch, head), with the forward's LSE and the upstream gradient dO,
//
//   P_ij  = exp(scale * q_i.k_j - LSE_i)          (recomputed, masked -> 0)
//   D_i   = dO_i . O_i                            (one value per row, formed by
//                                                  the dQ kernel, kept for dK/dV)
//   dP_ij = dO_i . v_j,   dS_ij = P_ij (dP_ij - D_i)
//   dV_j  = sum_i P_ij dO_i,   dK_j = scale sum_i dS_ij q_i,   dQ_i = scale sum_j dS_ij k_j
//
// The exponent is base 2 with the scale folded in: P = exp2(S * c - LSE * log2 e),
// c = scale * log2 e (any sign: no running maximum is needed, LSE is given).
//
// Mapping onto CDNA4 (not the pages' Blackwell design -- no TMEM, 2-CTA MMA
// or DSMEM here):
// * Deterministic, no atomics: dQ is reduced over keys and dK, dV over queries
//   by two kernels.  The key-block kernel (dK, dV) owns 128 keys per workgroup
//   (32 per wave) and walks the query blocks; the query-block kernel (dQ) owns
//   128 queries and walks the key blocks.  Each recomputes S and dP, so the
//   pair issues 7 products per block pair instead of 5 -- the price of a fixed
//   summation order without a global atomic or a lock.
// * The query-block kernel is the forward's layout: S^T = K Q^T and
//   dP^T = V dO^T with one query per lane (Q and dO fragments in registers),
//   dS^T in bf16 as the B operand of dQ^T += K^T dS^T, K^T by transpose reads.
// * The key-block kernel is its transpose: S = Q K^T and dP = dO V^T with one
//   key per lane (K fragments in registers, the workgroup's V rows in LDS); P
//   and dS in bf16 are the B operands of dV^T += dO^T P and dK^T += Q^T dS, dO^T
//   and Q^T by transpose reads.  The per-query LSE and D come from LDS, four
//   rows per 16-byte read.
// * Tiles in LDS use the swizzled layout of fa_device.h, free of bank
//   conflicts for both the 16-byte row reads and the transpose reads.  Blocks
//   are double-buffered through registers with one barrier per block.
// * Register budget: two waves per SIMD (at most 256 VGPRs each; the library
//   is built with MFMA accumulators in ordinary VGPRs).  The dK/dV wave holds
//   128 accumulator registers, 32 of K, 32 of S and dP and the block staging;
//   hence V from LDS, the LDS read offsets kept as two registers per family
//   (LdsOffsets) and no branch around the products (a per-wave branch there
//   splits the accumulators' live ranges and costs copies every block).
// * Grouped K/V heads: the key-block kernel of K/V head kv walks the query
//   heads kv*G .. kv*G+G-1 in turn and writes dK, dV once.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "fa_device.h"
#include "fa_internal.h"

FA_NS_BEGIN

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;   // query (dQ) or key (dK/dV) rows per workgroup

// ------------------------------------------------------------------ LDS offsets
// A lane's swizzled read offsets (elements) into a row-major D-wide tile, each
// family kept as two registers instead of one per read.  With f = vswz(row):
// * row reads (16-byte chunk 2*ds + g of row lq): the chunk index XOR f splits
//   as 2*(ds ^ (f>>1)) + (g ^ (f&1)), so offset(ds) = base + ((16*ds) ^ x);
// * transpose reads (rows 4g + (lane%16)/4 + 8h, columns 32*dt + 16*((lane/16)&1)
//   + 4*(lane%4)): the chunk is 4*dt + s with s < 4, and (4*dt + s) ^ f splits as
//   4*(dt ^ (f>>2)) + (s ^ (f&3)), so offset(dt, h) = base_h + ((32*dt) ^ x_h).
struct LdsOffsets {
    int rb, rx;          // row reads
    int tb[2], tx[2];    // transpose reads, h = 0, 1
    __device__ __forceinline__ int row(int ds) const { return rb + ((16 * ds) ^ rx); }
    __device__ __forceinline__ int tr(int dt, int h) const { return tb[h] + ((32 * dt) ^ tx[h]); }
    // Make the bases opaque for one loop iteration so that the per-read sums
    // are formed next to their reads instead of being hoisted into one live
    // register per read.
    __device__ __forceinline__ void refresh() {
        asm volatile("" : "+v"(rb), "+v"(rx), "+v"(tb[0]), "+v"(tx[0]), "+v"(tb[1]), "+v"(tx[1]));
    }
};

template <int D>
__device__ __forceinline__ LdsOffsets lds_offsets(int lane) {
    const int lq = lane & 31, g = lane >> 5;
    LdsOffsets o;
    const int f = vswz<D>(lq);
    o.rb = lq * D + 8 * (g ^ (f & 1));
    o.rx = 16 * (f >> 1);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int row = 4 * g + ((lane & 15) >> 2) + 8 * h;
        const int fr = vswz<D>(row);
        const int sub = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        o.tb[h] = row * D + 8 * (sub ^ (fr & 3)) + 4 * (lane & 1);
        o.tx[h] = 32 * (fr >> 2);
    }
    return o;
}

// ------------------------------------------------------------------ tile maps
struct BwdTile {
    int b, h;            // batch (sequence) and head (query head, or K/V head)
    int m;               // tile index along the sequence
    int tok0;            // first token of the sequence
    int L_q, L_k;        // query and key lengths of the sequence
};

constexpr int kBwdHeadGroup = 4;   // (batch, head) pairs per group of the fixed-length order

// Tiles of ROWS rows along a sequence: (b, h, m) from the workgroup index t.
// heads = the head count of the owning dimension.  The order is tile-position
// major, every (b, h) at one position before the next, so that with causal
// masking the heaviest tiles start first (longest-processing-time order): the
// dQ tile m visits m + 1 key tiles' worth of blocks (reverse = true walks m
// from the top), the dK/dV tile m visits the query blocks from m to the end
// (reverse = false).  With a pair (packed: head) count that is a multiple of
// 8 the order is XCD-aware (below); otherwise it is by position only.
template <int ROWS>
__device__ __forceinline__ bool bwd_decode(int t, const BwdParams &p, int heads, int len_max,
                                           bool reverse, BwdTile &c) {
    if (p.offsets && heads % kNumXcd == 0) {
        // Varlen: the workgroups t with one value of x = t % 8 share an XCD
        // (round-robin dispatch), and they own heads
        // [x*HX, (x+1)*HX) of every sequence; on an XCD the tiles go sequence
        // by sequence, head by head, each head's tiles longest first, so the
        // tiles that read one head's K/V (or Q/dO) run together and share the
        // XCD's L2.
        const int lane = threadIdx.x & 63;
        const int32_t *off = p.offsets;
        const int x = t % kNumXcd, HX = heads / kNumXcd;
        const int u = t / kNumXcd;
        int base = 0;
        for (int b0 = 0; b0 < p.B; b0 += 64) {
            const int bb = b0 + lane;
            const int nblk = bb < p.B ? (off[bb + 1] - off[bb] + ROWS - 1) / ROWS : 0;
            const int v = nblk * HX;
            int incl = v;
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
                c.b = b0 + lb;
                c.h = x * HX + r / n;
                c.m = reverse ? n - 1 - r % n : r % n;
                c.tok0 = off[c.b];
                c.L_q = c.L_k = off[c.b + 1] - c.tok0;
                return true;
            }
            base += total;
        }
        return false;
    }
    const int nm = (len_max + ROWS - 1) / ROWS;
    const int nbh = p.B * heads;
    int bh;
    if (!p.offsets && nbh % kNumXcd == 0) {
        // Fixed length: the workgroups with t % 8 = x (one XCD) own the
        // (batch, head) pairs x + 8k; their
        // tiles go in groups of kBwdHeadGroup pairs, each group's tiles
        // position-major (heaviest first) before the next group's, so that the
        // streamed K/V (dQ) or Q/dO (dK/dV) of about that many heads, not of
        // all the XCD's, is read at a time and stays in its L2.
        const int x = t % kNumXcd, u = t / kNumXcd, HX = nbh / kNumXcd;
        const int gs = HX % kBwdHeadGroup == 0 ? kBwdHeadGroup : HX;
        const int grp = u / (gs * nm), v = u % (gs * nm);
        c.m = v / gs;
        bh = x + kNumXcd * (grp * gs + v % gs);
    } else {
        c.m = t / nbh;
        bh = t % nbh;
    }
    if (reverse) c.m = nm - 1 - c.m;
    c.b = bh / heads;
    c.h = bh % heads;
    if (p.offsets) {
        c.tok0 = p.offsets[c.b];
        c.L_q = c.L_k = p.offsets[c.b + 1] - c.tok0;
        const int len = c.L_q;
        return c.m * ROWS < len;
    }
    c.tok0 = 0;
    c.L_q = p.Nq;
    c.L_k = p.Nk;
    return true;
}

// ------------------------------------------------------------------ dQ kernel
// Workgroup: 4 waves, 128 queries of one (b, h); K/V blocks of 32 keys (64 would
// not fit two waves per SIMD: S and dP of 64 keys alone take 64 registers).
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) void fa_bwd_dq_kernel(BwdParams p) {
    constexpr int BN = 32;
    constexpr int NDS = D / 16, NDT = D / 32, NKT = BN / 32, NKS = BN / 16;
    constexpr int TILE = BN * D;                       // elements of a K or V block
    constexpr int NCHUNK = TILE / 8;                   // 16-byte chunks per block
    constexpr int CH = (NCHUNK + kBwdThreads - 1) / kBwdThreads;   // ... per thread
    constexpr bool EXACT = NCHUNK % kBwdThreads == 0;  // else the last round is partial
    __shared__ __attribute__((aligned(16))) unsigned short smem[4 * TILE];
    // K block in buffer b at smem + b * TILE, V block at smem + (2 + b) * TILE.

    BwdTile tc;
    if (!bwd_decode<kBwdRows>(blockIdx.x, p, p.H, p.Nq, CAUSAL, tc)) return;
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lq = lane & 31, g = lane >> 5;
    const int Nq = tc.L_q, Nk = tc.L_k;
    const int shift = Nk - Nq;
    const int q0 = tc.m * kBwdRows + 32 * w;           // first query of this wave
    const int qrow = q0 + lq;
    const bool row_ok = qrow < Nq;
    const int hkv = tc.h / p.group;
    const int64_t tq = (int64_t)p.H * D, tkv = (int64_t)p.Hkv * D;   // token strides
    const unsigned tqb = (unsigned)(tq * 2), tkvb = (unsigned)(tkv * 2);
    const int64_t qtok = (p.offsets ? tc.tok0 : (int64_t)tc.b * p.Nq);
    const int64_t ktok = (p.offsets ? tc.tok0 : (int64_t)tc.b * p.Nk);
    const unsigned short *Qg = (const unsigned short *)p.q + qtok * tq + tc.h * D;
    const unsigned short *dOg = (const unsigned short *)p.dout + qtok * tq + tc.h * D;
    const unsigned short *Og_in = (const unsigned short *)p.o + qtok * tq + tc.h * D;
    const unsigned short *Kg = (const unsigned short *)p.k + ktok * tkv + hkv * D;
    const unsigned short *Vg = (const unsigned short *)p.v + ktok * tkv + hkv * D;

    // Keys this tile visits.
    int nblocks = (Nk + BN - 1) / BN;
    if (CAUSAL) {
        const int last_row = min(tc.m * kBwdRows + kBwdRows, Nq) - 1;
        const int kmax = last_row + shift;
        nblocks = kmax < 0 ? 0 : min(nblocks, kmax / BN + 1);
    }

    // Q and dO fragments (B operands, one query per lane: this lane holds the
    // 16-byte chunks 2ds + g of its row) and the row terms.  D_i = dO_i . O_i is
    // formed here from the same chunks of O, the two half-waves' parts added by
    // one lane exchange, and stored for the dK/dV kernel, which runs after this
    // one on the stream.
    bf16x8 qf[NDS], of[NDS];
    float dpart = 0.f;
    {
        // Descriptor ranges are wave-uniform; read back from lane 0 so that the
        // descriptors stay scalar (the clamp compiles to a vector instruction,
        // and a descriptor in vector registers makes every load a loop).
        const int rows = max(0, min(32, Nq - q0));
        const unsigned bytes = __builtin_amdgcn_readfirstlane(
            rows > 0 ? (unsigned)(rows - 1) * tqb + (unsigned)(D * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg + (int64_t)q0 * tq, bytes);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(dOg + (int64_t)q0 * tq, bytes);
        const __amdgpu_buffer_rsrc_t rO = make_rsrc(Og_in + (int64_t)q0 * tq, bytes);
        const unsigned off = (unsigned)lq * tqb + (unsigned)(16 * g);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds) {
            qf[ds] = __builtin_bit_cast(bf16x8, buffer_load16(rq, off + 32u * ds));
            const u32x4 dov = buffer_load16(ro, off + 32u * ds);
            const u32x4 ov = buffer_load16(rO, off + 32u * ds);
            of[ds] = __builtin_bit_cast(bf16x8, dov);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                dpart = fmaf(__uint_as_float(dov[e] << 16), __uint_as_float(ov[e] << 16), dpart);
                dpart = fmaf(__uint_as_float(dov[e] & 0xFFFF0000u), __uint_as_float(ov[e] & 0xFFFF0000u), dpart);
            }
        }
    }
    const float dsum = dpart + __shfl_xor(dpart, 32, 64);
    const float c = p.scale_log2;
    float lse2 = 0.f;
    if (row_ok) {
        int64_t idx;
        if (p.offsets) idx = (int64_t)tc.h * p.offsets[p.B] + tc.tok0 + qrow;
        else           idx = ((int64_t)tc.b * p.H + tc.h) * Nq + qrow;
        lse2 = p.lse[idx] * 1.4426950408889634f;
        if (g == 0) p.dsum[idx] = dsum;
    }

    f32x16 acc[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[dt][i] = 0.f;

    // Cooperative block loads: chunk u = tid + kBwdThreads * rr of a BN x D
    // block (a chunk past the block reads out of range, is 0 and is not stored).
    unsigned ld_off[CH];
    int st_off[CH];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
        const int u = tid + kBwdThreads * rr;
        const int row = u / (D / 8), cc = u % (D / 8);
        ld_off[rr] = (EXACT || u < NCHUNK) ? (unsigned)row * tkvb + 16u * cc : 0x7FFFFFF0u;
        st_off[rr] = row * D + ((cc ^ vswz<D>(row)) << 3);
    }
    u32x4 kreg[CH], vreg[CH];
    auto block_bytes = [&](int kb) -> unsigned {
        const int rem = Nk - kb * BN;
        if (kb >= nblocks || rem <= 0) return 0u;
        return (unsigned)(min(rem, BN) - 1) * tkvb + (unsigned)(D * 2);
    };
    auto load = [&](int kb) {
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)kb * BN * tkv, block_bytes(kb));
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)kb * BN * tkv, block_bytes(kb));
#pragma unroll
        for (int rr = 0; rr < CH; ++rr) {
            kreg[rr] = buffer_load16(rk, ld_off[rr]);
            vreg[rr] = buffer_load16(rv, ld_off[rr]);
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int rr = 0; rr < CH; ++rr) {
            if (!EXACT && tid + kBwdThreads * rr >= NCHUNK) continue;
            *(u32x4 *)(smem + buf * TILE + st_off[rr]) = kreg[rr];
            *(u32x4 *)(smem + (2 + buf) * TILE + st_off[rr]) = vreg[rr];
        }
    };

    // Row reads (A operand, 32 keys x 16 dims: key lq, chunk 2ds+g) and
    // transpose reads (K^T operand, as the forward's V^T).
    LdsOffsets lo = lds_offsets<D>(lane);
    f32x16 negd;   // -D_i in every register: the start of each dP^T chain
#pragma unroll
    for (int i = 0; i < 16; ++i) negd[i] = -dsum;

    if (nblocks > 0) {
        load(0);
        store(0);
        __syncthreads();
        for (int kb = 0; kb < nblocks; ++kb) {
            const int buf = kb & 1;
            if (kb + 1 < nblocks) load(kb + 1);
            const unsigned short *Ks = smem + buf * TILE;
            const unsigned short *Vs = smem + (2 + buf) * TILE;
            lo.refresh();
            // Every wave runs every block: a wave none of whose rows sees a key of
            // this block gets dS = 0 from the mask (a branch here would split the
            // accumulators' live ranges and cost register copies every block).
            {
                // S^T = K Q^T and dP^T = V dO^T for the 64 keys (32 per tile kt;
                // 32-row tiles are 32 rows apart in the swizzled layout: the
                // swizzle depends on the row within 16, unchanged by +32).
                // The dP^T chain starts from -D_i, so it yields dP - D.
                f32x16 s[NKT], dp[NKT];
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) s[kt][i] = 0.f;
                    dp[kt] = negd;
                }
                {
                    // Each K and V fragment in its own registers, RA steps of
                    // reads in flight ahead of the MFMAs (left alone, the
                    // compiler reused one register pair and waited out the
                    // LDS latency before every pair of MFMAs).
                    constexpr int NR = NDS * NKT, RA = NR < 3 ? NR : 3;
                    bf16x8 kfr[NDS][NKT], vfr[NDS][NKT];
#pragma unroll
                    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
                        for (int kt = 0; kt < NKT; ++kt) {
                            kfr[ds][kt] = *(const bf16x8 *)(Ks + lo.row(ds) + 32 * kt * D);
                            vfr[ds][kt] = *(const bf16x8 *)(Vs + lo.row(ds) + 32 * kt * D);
                        }
#pragma unroll
                    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
                        for (int kt = 0; kt < NKT; ++kt) {
                            s[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kfr[ds][kt], qf[ds], s[kt], 0, 0, 0);
                            dp[kt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vfr[ds][kt], of[ds], dp[kt], 0, 0, 0);
                        }
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RA, 0);      // LDS reads
#pragma unroll
                    for (int i = 0; i < NR - RA; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);      // MFMAs
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 2 * RA, 0);
                }
                // dS^T = P^T (dP^T - D), masked keys -> 0; to bf16 B operands.  A
                // block every pair of which is kept skips the test (wave-uniform).
                const int kv0 = kb * BN;
                const int lim = row_ok ? (CAUSAL ? min(Nk - 1, qrow + shift) : Nk - 1) - kv0 - 4 * g
                                       : -(1 << 30);
                const bool full = q0 + 31 < Nq && kv0 + BN - 1 < Nk &&
                                  (!CAUSAL || kv0 + BN - 1 <= q0 + shift);
                bf16x8 sf[NKS];
                auto frags = [&](auto masked) {
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks) {
                        unsigned wd[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            float v2[2];
#pragma unroll
                            for (int h2 = 0; h2 < 2; ++h2) {
                                const int i = 8 * (ks & 1) + 2 * e + h2;
                                const int kt = ks >> 1;
                                const int key = 32 * kt + 8 * (i >> 2) + (i & 3);   // relative to kv0 + 4g
                                const float pr = __builtin_amdgcn_exp2f(fmaf(s[kt][i], c, -lse2));
                                const float v = pr * dp[kt][i];
                                if constexpr (decltype(masked)::value)
                                    v2[h2] = key > lim ? 0.f : v;
                                else
                                    v2[h2] = v;
                            }
                            wd[e] = pack_bf16x2(v2[0], v2[1]);
                        }
                        const u32x4 x = {wd[0], wd[1], wd[2], wd[3]};
                        sf[ks] = __builtin_bit_cast(bf16x8, x);
                    }
                };
                if (full) frags(std::false_type{});
                else      frags(std::true_type{});
                // dQ^T += K^T dS^T (K^T fragments read ahead as above).
                {
                    constexpr int NR2 = NKS * NDT, RB = NR2 < 4 ? NR2 : 4;
                    i16x8 ktf[NKS][NDT];
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt) {
                            const unsigned short *a0 = Ks + 16 * ks * D;
                            const i16x4 tlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a0 + lo.tr(dt, 0)));
                            const i16x4 thi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(a0 + lo.tr(dt, 1)));
                            ktf[ks][dt] = __builtin_shufflevector(tlo, thi, 0, 1, 2, 3, 4, 5, 6, 7);
                        }
#pragma unroll
                    for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
                        for (int dt = 0; dt < NDT; ++dt)
                            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ktf[ks][dt]),
                                                                              sf[ks], acc[dt], 0, 0, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 2 * RB, 0);
#pragma unroll
                    for (int i = 0; i < NR2 - RB; ++i) {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, RB, 0);
                }
            }
            if (kb + 1 < nblocks) store(buf ^ 1);
            __syncthreads();
        }
    }

    // dQ = scale * (dQ^T)^T, one query row per lane, bf16.
    if (row_ok) {
        unsigned short *Og = (unsigned short *)p.dq + (qtok + qrow) * tq + tc.h * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = 32 * dt + 8 * i4 + 4 * g;
                const uint2 v2 = make_uint2(pack_bf16x2(acc[dt][4 * i4] * p.scale, acc[dt][4 * i4 + 1] * p.scale),
                                            pack_bf16x2(acc[dt][4 * i4 + 2] * p.scale, acc[dt][4 * i4 + 3] * p.scale));
                *(uint2 *)(Og + d0) = v2;
            }
    }
}

// ------------------------------------------------------------------ dK, dV kernel
// Workgroup: 4 waves, 128 keys of one (b, K/V head); query blocks of 32.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads) __attribute__((amdgpu_waves_per_eu(2))) void fa_bwd_dkdv_kernel(BwdParams p) {
    constexpr int BQ = 32;
    constexpr int NDS = D / 16, NDT = D / 32, NQS = BQ / 16;
    constexpr int TILE = BQ * D;                       // elements of a Q or dO block
    constexpr int NCHUNK = TILE / 8;                   // 16-byte chunks per block
    constexpr int CH = (NCHUNK + kBwdThreads - 1) / kBwdThreads;   // ... per thread
    constexpr bool EXACT = NCHUNK % kBwdThreads == 0;  // else the last round is partial
    __shared__ __attribute__((aligned(16))) unsigned short smem[4 * TILE + kBwdRows * D];
    __shared__ __attribute__((aligned(16))) float rowt[2][2][BQ];   // [buf][lse2, -D][query]
    // Q block in buffer b at smem + b * TILE, dO block at smem + (2 + b) * TILE,
    // the workgroup's V rows at smem + 4 * TILE (read as B operands of dP).

    BwdTile tc;
    if (!bwd_decode<kBwdRows>(blockIdx.x, p, p.Hkv, p.Nk, false, tc)) return;   // tc.h is the K/V head
    const int tid = threadIdx.x;
    const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int lane = tid & 63, lq = lane & 31, g = lane >> 5;
    const int Nq = tc.L_q, Nk = tc.L_k;
    const int shift = Nk - Nq;
    const int k0w = tc.m * kBwdRows + 32 * w;          // first key of this wave
    const int key = k0w + lq;
    const int64_t tq = (int64_t)p.H * D, tkv = (int64_t)p.Hkv * D;
    const unsigned tqb = (unsigned)(tq * 2), tkvb = (unsigned)(tkv * 2);
    const int64_t qtok = (p.offsets ? tc.tok0 : (int64_t)tc.b * p.Nq);
    const int64_t ktok = (p.offsets ? tc.tok0 : (int64_t)tc.b * p.Nk);
    const unsigned short *Kg = (const unsigned short *)p.k + ktok * tkv + tc.h * D;
    const unsigned short *Vg = (const unsigned short *)p.v + ktok * tkv + tc.h * D;

    // K fragments in registers (B operands of S = Q K^T, one key per lane); the
    // V rows of the workgroup go to LDS once (B operands of dP = dO V^T are read
    // from there each block: holding them too would not fit two waves per SIMD).
    bf16x8 kf[NDS];
    unsigned short *Vs = smem + 4 * TILE;
    {
        // Wave-uniform descriptor ranges, read back from lane 0 (scalar descriptors).
        const int rows = max(0, min(32, Nk - k0w));
        const unsigned bytes = __builtin_amdgcn_readfirstlane(
            rows > 0 ? (unsigned)(rows - 1) * tkvb + (unsigned)(D * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(Kg + (int64_t)k0w * tkv, bytes);
        const unsigned off = (unsigned)lq * tkvb + (unsigned)(16 * g);
#pragma unroll
        for (int ds = 0; ds < NDS; ++ds)
            kf[ds] = __builtin_bit_cast(bf16x8, buffer_load16(rk, off + 32u * ds));
        const int vrows = max(0, min(kBwdRows, Nk - tc.m * kBwdRows));
        const unsigned vbytes = __builtin_amdgcn_readfirstlane(
            vrows > 0 ? (unsigned)(vrows - 1) * tkvb + (unsigned)(D * 2) : 0u);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(Vg + (int64_t)tc.m * kBwdRows * tkv, vbytes);
        constexpr int VCH = kBwdRows * D / 8 / kBwdThreads;
#pragma unroll
        for (int rr = 0; rr < VCH; ++rr) {
            const int u = tid + kBwdThreads * rr;
            const int row = u / (D / 8), cc = u % (D / 8);
            const u32x4 x = buffer_load16(rv, (unsigned)row * tkvb + 16u * cc);
            *(u32x4 *)(Vs + row * D + ((cc ^ vswz<D>(row)) << 3)) = x;
        }
    }
    const float c = p.scale_log2;

    f32x16 dk[NDT], dv[NDT];
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int i = 0; i < 16; ++i) { dk[dt][i] = 0.f; dv[dt][i] = 0.f; }

    // Query blocks this key tile meets: causal rows i with i + shift >= first key.
    const int kfirst = tc.m * kBwdRows;
    int qb0 = 0;
    if (CAUSAL) qb0 = max(0, kfirst - shift) / BQ;
    const int nqb = (Nq + BQ - 1) / BQ;

    unsigned ld_off[CH];
    int st_off[CH];
#pragma unroll
    for (int rr = 0; rr < CH; ++rr) {
        const int u = tid + kBwdThreads * rr;
        const int row = u / (D / 8), cc = u % (D / 8);
        ld_off[rr] = (EXACT || u < NCHUNK) ? (unsigned)row * tqb + 16u * cc : 0x7FFFFFF0u;
        st_off[rr] = row * D + ((cc ^ vswz<D>(row)) << 3);
    }
    u32x4 qreg[CH], oreg[CH];
    // One row term per lane of the first wave: LSE (lanes 0..31, scaled by
    // log2 e when stored) or D (lanes 32..63) of query qb*BQ + lane % 32.  The
    // loads are range-checked (0 past the sequence) and their values are not
    // touched until the store, so the block's loads stay in flight meanwhile.
    float tl = 0.f, td = 0.f;
    const int64_t T = p.offsets ? (int64_t)p.offsets[p.B] : 0;
    auto load = [&](int h, int qb) {
        const unsigned short *Qg = (const unsigned short *)p.q + qtok * tq + h * D;
        const unsigned short *Og = (const unsigned short *)p.dout + qtok * tq + h * D;
        const int rem = Nq - qb * BQ;
        const unsigned bytes = rem > 0 ? (unsigned)(min(rem, BQ) - 1) * tqb + (unsigned)(D * 2) : 0u;
        const __amdgpu_buffer_rsrc_t rq = make_rsrc(Qg + (int64_t)qb * BQ * tq, bytes);
        const __amdgpu_buffer_rsrc_t ro = make_rsrc(Og + (int64_t)qb * BQ * tq, bytes);
#pragma unroll
        for (int rr = 0; rr < CH; ++rr) {
            qreg[rr] = buffer_load16(rq, ld_off[rr]);
            oreg[rr] = buffer_load16(ro, ld_off[rr]);
        }
        if (w == 0) {
            const int64_t row0 = p.offsets ? (int64_t)h * T + tc.tok0
                                           : ((int64_t)tc.b * p.H + h) * Nq;
            const unsigned nb = rem > 0 ? (unsigned)min(rem, BQ) * 4u : 0u;
            const __amdgpu_buffer_rsrc_t rl = make_rsrc(p.lse + row0 + (int64_t)qb * BQ, nb);
            const __amdgpu_buffer_rsrc_t rd = make_rsrc(p.dsum + row0 + (int64_t)qb * BQ, nb);
            // Both descriptors are uniform; each half of the wave reads one of
            // them, the other load is out of range and returns 0.
            const unsigned off = (unsigned)(lane & (BQ - 1)) * 4u;
            const unsigned far = 0x7FFFFFF0u;
            tl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rl, lane < BQ ? off : far, 0, 0));
            td = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                               rd, lane < BQ ? far : off, 0, 0));
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int rr = 0; rr < CH; ++rr) {
            if (!EXACT && tid + kBwdThreads * rr >= NCHUNK) continue;
            *(u32x4 *)(smem + buf * TILE + st_off[rr]) = qreg[rr];
            *(u32x4 *)(smem + (2 + buf) * TILE + st_off[rr]) = oreg[rr];
        }
        if (w == 0)
            rowt[buf][lane / BQ][lane & (BQ - 1)] = lane < BQ ? tl * 1.4426950408889634f : -td;
    };

    LdsOffsets lo = lds_offsets<D>(lane);

    const int steps_per_head = nqb - qb0;
    const int nsteps = steps_per_head > 0 ? steps_per_head * p.group : 0;
    if (nsteps > 0) {
        load(tc.h * p.group, qb0);
        store(0);
        __syncthreads();
        for (int st = 0; st < nsteps; ++st) {
            const int buf = st & 1;
            const int h = tc.h * p.group + st / steps_per_head;
            const int qb = qb0 + st % steps_per_head;
            if (st + 1 < nsteps)
                load(tc.h * p.group + (st + 1) / steps_per_head, qb0 + (st + 1) % steps_per_head);
            (void)h;
            const unsigned short *Qs = smem + buf * TILE;
            const unsigned short *Os = smem + (2 + buf) * TILE;
            lo.refresh();
            const int qfirst = qb * BQ;
            // Every wave runs every block; pairs outside the mask get P = dS = 0.
            {
                // The dP chain starts from -D of each register's query (the
                // float4s of rowt are four consecutive queries, registers
                // i0..i0+3), so it yields dP - D.
                const float4 *lrow = (const float4 *)rowt[buf][0];
                const float4 *drow = (const float4 *)rowt[buf][1];
                f32x16 s, dp;
#pragma unroll
                for (int i4 = 0; i4 < 4; ++i4) {
                    const float4 d4 = drow[(8 * i4 + 4 * g) >> 2];
                    dp[4 * i4] = d4.x; dp[4 * i4 + 1] = d4.y; dp[4 * i4 + 2] = d4.z; dp[4 * i4 + 3] = d4.w;
                }
#pragma unroll
                for (int i = 0; i < 16; ++i) s[i] = 0.f;
#pragma unroll
                for (int ds = 0; ds < NDS; ++ds) {
                    const bf16x8 qa = *(const bf16x8 *)(Qs + lo.row(ds));
                    const bf16x8 oa = *(const bf16x8 *)(Os + lo.row(ds));
                    // V row 32w + lq: same swizzle as row lq (it depends on row % 16).
                    const bf16x8 vb = *(const bf16x8 *)(Vs + 32 * w * D + lo.row(ds));
                    s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kf[ds], s, 0, 0, 0);
                    dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(oa, vb, dp, 0, 0, 0);
                }
                // Accumulator: lane = key, register i = query qfirst + 4g + qo(i) with
                // qo(i) = 8(i/4) + i%4.  P and dS are formed for every pair and packed
                // to bf16 B operands (16 queries each); then, only in a block that the
                // mask cuts (wave-uniform test), the dropped pairs are zeroed in the
                // packed words: a pair is kept iff mlo <= qo < mhi (query in the
                // sequence, key in the sequence and, when causal, not after the query).
                // Values formed for dropped pairs may be inf or NaN; the select
                // replaces their bits without reading them as numbers.
                u32x4 pwv[NQS], swv[NQS];
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) {
#pragma unroll
                    for (int hh = 0; hh < 2; ++hh) {
                        const int i0 = 8 * qs + 4 * hh;         // registers i0..i0+3
                        const float4 l4 = lrow[(8 * (i0 >> 2) + 4 * g) >> 2];
                        const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
                        float pv[4], sv[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            pv[e] = __builtin_amdgcn_exp2f(fmaf(s[i0 + e], c, -lv[e]));
                            sv[e] = pv[e] * dp[i0 + e];
                        }
                        pwv[qs][2 * hh] = pack_bf16x2(pv[0], pv[1]);
                        pwv[qs][2 * hh + 1] = pack_bf16x2(pv[2], pv[3]);
                        swv[qs][2 * hh] = pack_bf16x2(sv[0], sv[1]);
                        swv[qs][2 * hh + 1] = pack_bf16x2(sv[2], sv[3]);
                    }
                }
                const bool full = k0w + 31 < Nk && qfirst + BQ - 1 < Nq &&
                                  (!CAUSAL || k0w + 31 <= qfirst + shift);
                if (!full) {
                    const int qbase = qfirst + 4 * g;
                    const int mhi = Nq - qbase;
                    const int mlo = key >= Nk ? (1 << 30) : (CAUSAL ? key - shift - qbase : -(1 << 30));
#pragma unroll
                    for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
                        for (int wd = 0; wd < 4; ++wd) {
                            const int r = 8 * qs + 4 * (wd >> 1) + 2 * (wd & 1);   // registers r, r + 1
                            const int qa = 8 * (r >> 2) + (r & 3), qb = qa + 1;
                            const unsigned keep = ((qa >= mlo && qa < mhi) ? 0x0000FFFFu : 0u) |
                                                  ((qb >= mlo && qb < mhi) ? 0xFFFF0000u : 0u);
                            pwv[qs][wd] &= keep;
                            swv[qs][wd] &= keep;
                        }
                }
                bf16x8 pfr[NQS], sfr[NQS];
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs) {
                    pfr[qs] = __builtin_bit_cast(bf16x8, pwv[qs]);
                    sfr[qs] = __builtin_bit_cast(bf16x8, swv[qs]);
                }
                // dV^T += dO^T P and dK^T += Q^T dS (dO^T, Q^T by transpose reads).
#pragma unroll
                for (int qs = 0; qs < NQS; ++qs)
#pragma unroll
                    for (int dt = 0; dt < NDT; ++dt) {
                        const unsigned short *o0 = Os + 16 * qs * D;
                        const unsigned short *q0p = Qs + 16 * qs * D;
                        const i16x4 olo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(o0 + lo.tr(dt, 0)));
                        const i16x4 ohi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(o0 + lo.tr(dt, 1)));
                        const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(q0p + lo.tr(dt, 0)));
                        const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4 *)(q0p + lo.tr(dt, 1)));
                        const i16x8 ob = __builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7);
                        const i16x8 qbv = __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7);
                        dv[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, ob),
                                                                         pfr[qs], dv[dt], 0, 0, 0);
                        dk[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, qbv),
                                                                         sfr[qs], dk[dt], 0, 0, 0);
                    }
            }
            if (st + 1 < nsteps) store(buf ^ 1);
            __syncthreads();
        }
    }

    // dK = scale * (dK^T)^T and dV, one key row per lane, bf16.
    if (key < Nk) {
        unsigned short *dKg = (unsigned short *)p.dk + (ktok + key) * tkv + tc.h * D;
        unsigned short *dVg = (unsigned short *)p.dv + (ktok + key) * tkv + tc.h * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
            for (int i4 = 0; i4 < 4; ++i4) {
                const int d0 = 32 * dt + 8 * i4 + 4 * g;
                const float sc = p.scale;
                *(uint2 *)(dKg + d0) = make_uint2(pack_bf16x2(dk[dt][4 * i4] * sc, dk[dt][4 * i4 + 1] * sc),
                                                  pack_bf16x2(dk[dt][4 * i4 + 2] * sc, dk[dt][4 * i4 + 3] * sc));
                *(uint2 *)(dVg + d0) = make_uint2(pack_bf16x2(dv[dt][4 * i4], dv[dt][4 * i4 + 1]),
                                                  pack_bf16x2(dv[dt][4 * i4 + 2], dv[dt][4 * i4 + 3]));
            }
    }
}

template <int D>
static int launch_bwd_d(const BwdParams &p, bool causal, hipStream_t s) {
    const unsigned gq = (unsigned)((int64_t)p.B * p.H * ((p.Nq + kBwdRows - 1) / kBwdRows));
    const unsigned gk = (unsigned)((int64_t)p.B * p.Hkv * ((p.Nk + kBwdRows - 1) / kBwdRows));
    if (causal) {
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, true>), dim3(gq), dim3(kBwdThreads), 0, s, p);
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, true>), dim3(gk), dim3(kBwdThreads), 0, s, p);
    } else {
        hipLaunchKernelGGL((fa_bwd_dq_kernel<D, false>), dim3(gq), dim3(kBwdThreads), 0, s, p);
        hipLaunchKernelGGL((fa_bwd_dkdv_kernel<D, false>), dim3(gk), dim3(kBwdThreads), 0, s, p);
    }
    return (int)hipGetLastError();
}

// The row terms D of fa_bwd_noalloc live in this device array instead of a
// caller's workspace: each GPU the library runs on holds its own copy until
// the process ends.  Host code never uses the array's name as an address (on
// the host it names a stand-in, not device memory); it uses the address
// hipGetSymbolAddress returns for the current device, resolved once per
// device and kept.
static __device__ __align__(256) float scratch[kBwdScratchBytes / sizeof(float)];

int bwd_scratch(void **ptr) {
    static std::mutex mu;
    static void *addr[kMaxDevices] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return -1;
        addr[dev] = a;
    }
    *ptr = addr[dev];
    return 0;
}

int launch_bwd(const BwdParams &p, int d, bool causal, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (d == 64) return launch_bwd_d<64>(p, causal, s);
    return launch_bwd_d<128>(p, causal, s);
}

FA_NS_END  // namespace fa
