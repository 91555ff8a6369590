// Step 4 of the scan: the outputs of one chunk ("chunk_scan").
//
// For chunk c of sequence b, head h (group g), and rows i, j of the chunk
// (cs2 = log2(e) * cumulative A*dts, h_in = state entering the chunk):
//   G[i][j]   = sum_n C[i,g,n] * B[j,g,n]            (formed by the chunk-state step)
//   M[i][j]   = G[i][j] * exp2(cs2_i - cs2_j) * dts_j     for j <= i, else 0
//   y[i][p]   = sum_j M[i][j] * x[j,h,p]                              (diagonal block)
//             + exp2(cs2_i) * sum_n C[i,g,n] * h_in[p][n]             (off-diagonal part)
//             + D[h] * x[i,h,p]                                       (skip term)
// This is the chunked form of "Mamba chunk scan with segsum" (description:
// intra-chunk attention-like block from segment sums, inter-chunk state,
// their sum); D*x is the skip term of "mamba2_ssd_scan" ("Per-token
// recurrence").  y is rounded to bf16.
//
// Work split.  One workgroup per (chunk, block of HB heads of one group),
// eight wavefronts, one 32-row block each; the two wavefronts that share a
// SIMD own row blocks k and 7-k, so each SIMD handles 9 of the 36
// lower-triangular 32x32 tiles.  The operands the heads of a group share,
// the wavefront's C rows (registers, converted here to fp16 under a
// per-wavefront power of two) and its C.B^T tiles (from the chunk-state
// step, LDS), are loaded once and stay on chip while the workgroup walks its heads; each
// head's x and h_in are loaded into registers during the previous head's
// products.  Workgroups
// are numbered so that all head blocks of a chunk land on one XCD (dispatch
// is round-robin over the 8 XCDs) and share C and the tiles in its L2.
// Row blocks that start past the chunk end skip their products.
//
// MFMA layout (v_mfma_f32_32x32x16).  Every product is formed transposed,
// y^T[p][i], so each lane ends up with 4 consecutive p of one token i (one
// 8-byte store of 4 bf16) and the per-token factors are per-lane scalars.
// C.B^T is stored transposed (rows j, columns i) in accumulator order, so a tile's 16 values per lane (all at one i, at j = 8a + 4(l/32) +
// b) are directly the B-operand layout of M^T for x^T*M^T: the 16 j of the
// first K-step are {0..3, 8..11} for lanes 0-31 and {4..7, 12..15} for lanes
// 32-63 (a permutation of 0..15), likewise 16..31 for the second; x^T is read
// from LDS in the same order.
//
// Decay without one exp2 per element.  For a tile strictly below the
// diagonal block (all j < 32*rb <= i), exp2(cs2_i - cs2_j) =
// exp2(cs2_i - cs2_r) * exp2(cs2_r - cs2_j) with r = 32*rb; both factors are
// at most 1 for A <= 0.  The second factor, times dts_j, is tabulated once
// per head in LDS as fp16 in each lane's operand order, so such a tile's M operand is the C.B^T tile times the table, eight
// packed fp16 multiplies per lane; the first factor depends only on the
// lane's row i and is applied once per head, in fp32, to a second
// accumulator that collects those tiles.  Only the diagonal tile evaluates
// exp2 per element.  The skip term D*x is folded into the diagonal of M.
//
// Precision.  M and h_in are rounded to fp16 (11-bit significand) under
// power-of-two scales that keep them far from overflow (one per head for
// the diagonal M tile and for the table, one per row for h_in); C and C.B^T
// are rounded to fp16 after power-of-two scalings (per row block, per chunk
// and group), and x after one power of two per chunk and head (none while
// its largest magnitude is in [2^-6, 2^15)), compensated inside M or the
// accumulator scale.  The product
// of a C.B^T tile and the table is rounded to fp16 once more.  All products
// accumulate in fp32.  bf16 (8 bits) for M or h_in would put the rounding
// error, which scales with the typical size of y rather than with each y,
// close to the tolerance wherever y is near zero.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kThreads = 512;
// x^T rows: 128 token pairs + pad (8-byte aligned rows).  Row p keeps token
// pair q at column q ^ (16 * ((p >> 4) & 3)): the staging stores, where the
// four lanes of a token pair write rows 16 apart (32 banks apart at this
// stride), then fall in distinct banks; the swizzle moves whole 16-pair
// groups, so reads stay contiguous.
constexpr int XT_STRIDE = 130;

template <int N>
struct __attribute__((aligned(16))) ScanSmem {
    static constexpr int H_STRIDE = N / 2 + 4;  // dwords per h_in row + pad
    uint32_t g[36 * 2 * 64 * 4];  // the chunk's fp16 C.B^T tiles: [tile][half][lane] 16-byte runs
    uint32_t h[kHeadDim * H_STRIDE];
    uint32_t xt[kHeadDim * XT_STRIDE];
    // row block r, column tile t < r: fp16 pairs of
    // exp2(cs2[32r] - cs2[j]) * dts_j * 2^-(xe_t + kw), dword
    // r*128 + t*16 + hl*8 + 2a + bh holding j = 32t + 8a + 4hl + 2bh (+1)
    uint32_t v[8 * 128];
    // per-head tables, double-buffered: head k uses buffer k & 1
    float cs2[2][kChunk];
    float dts[2][kChunk];
    float hs[2][kHeadDim];  // 2^-hexp[p]
    float dd[2];            // D of the head
    int xexp[2];            // x exponent of the chunk and head
    float dmx[2][4];        // max |dts| over each quarter of the chunk's tokens
};

// One fp16 half of a packed dword times a float plus a float, as a single
// mixed-precision FMA (v_fma_mix_f32: the fp16 operand is read directly).
__device__ __forceinline__ float hfma(uint32_t w, int hi, float f, float c) {
    const f16x2 h2 = __builtin_bit_cast(f16x2, w);
    return __builtin_fmaf((float)h2[hi], f, c);
}
// Product of two fp16 pairs (v_pk_mul_f16).
__device__ __forceinline__ uint32_t hmul2(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(f16x2, a) * __builtin_bit_cast(f16x2, b));
}

// x^T rows (32*pt + l32) of column tile t as the two A operands of a K = 32 step.
template <int N>
__device__ __forceinline__ void x_operands(const ScanSmem<N> &sm, int l32, int hl, int t, int pt, f16x8 &x0, f16x8 &x1) {
    const int sw = (2 * pt + (l32 >> 4)) & 3;  // the row's swizzle
    const uint2 *row = reinterpret_cast<const uint2 *>(sm.xt + (32 * pt + l32) * XT_STRIDE + 16 * (t ^ sw) + 2 * hl);
    const uint2 xa = row[0], xb = row[2], xc = row[4], xd = row[6];
    x0 = __builtin_bit_cast(f16x8, u32x4{xa.x, xa.y, xb.x, xb.y});
    x1 = __builtin_bit_cast(f16x8, u32x4{xc.x, xc.y, xd.x, xd.y});
}

// The tiles of row block RB strictly below its diagonal tile, for one head:
//   acc += sum_{t < RB} (2^xe x_t)^T (C.B^T_t 2^sg (.) table_t)
// one product per tile; the caller scales acc per lane (row i) afterwards.
template <int N, int RB>
__device__ __forceinline__ void below_diag(const ScanSmem<N> &sm, f32x16 (&acc)[2], int lane) {
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    const u32x4 *gbase = reinterpret_cast<const u32x4 *>(sm.g) + (RB * (RB + 1) / 2) * 128 + lane;
    // the C.B^T and table operands of tile t + 1 are read during tile t's
    // products, its x^T operands at its start
    struct Ops {
        u32x4 g0, g1, v0, v1;
    };
    auto fetch = [&](int t, Ops &o) {
        o.g0 = gbase[t * 128];
        o.g1 = gbase[t * 128 + 64];
        const u32x4 *vp = reinterpret_cast<const u32x4 *>(sm.v + RB * 128 + t * 16 + hl * 8);
        o.v0 = vp[0];
        o.v1 = vp[1];
    };
    Ops ops[2];
    fetch(0, ops[0]);
#pragma unroll
    for (int t = 0; t < RB; ++t) {
        const Ops &o = ops[t & 1];
        f16x8 x[2][2];
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) x_operands(sm, l32, hl, t, pt, x[pt][0], x[pt][1]);
        if (t + 1 < RB) fetch(t + 1, ops[(t + 1) & 1]);
        // keeps the reads ahead (the scheduler would sink them to their use)
        __builtin_amdgcn_sched_barrier(0);
        u32x4 m0, m1;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            m0[q] = hmul2(o.g0[q], o.v0[q]);
            m1[q] = hmul2(o.g1[q], o.v1[q]);
        }
        const f16x8 mf0 = __builtin_bit_cast(f16x8, m0), mf1 = __builtin_bit_cast(f16x8, m1);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            acc[pt] = mfma32_f16(x[pt][0], mf0, acc[pt]);
            acc[pt] = mfma32_f16(x[pt][1], mf1, acc[pt]);
        }
    }
}

// The diagonal tile (t = rb) of row block rb, added to acc in units of
// 2^smx (x staged as 2^xe x): M per element,
//   exp2(cs2_i - cs2_j + lmg) dts_j C.B^T_ij  with lmg = smx - sg - xe,
// plus dx = D 2^(smx - xe) on the diagonal.  ci = cs2_i + lmg.  The tile is
// zero where j > i; there the exp2 argument is capped at the chunk's total
// log2 growth (0 for A <= 0), plus lmg (capm), which leaves every j <= i
// unchanged and keeps the masked products finite.
template <int N>
__device__ __forceinline__ void diag_tile(const ScanSmem<N> &sm, const float *cs2, const float *dts, f32x16 (&acc)[2],
                                          int lane, int rb, float ci, float capm, float dx) {
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    const int dl = l32 - 4 * hl;  // the lane's diagonal element is the one with 8a + b == dl
    const u32x4 *gp = reinterpret_cast<const u32x4 *>(sm.g) + (rb * (rb + 1) / 2 + rb) * 128 + lane;
    const u32x4 gt[2] = {gp[0], gp[64]};
    float mv[16];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        const int j0 = 32 * rb + 8 * a + 4 * hl;
        const float4 c4 = *reinterpret_cast<const float4 *>(cs2 + j0);
        const float4 d4 = *reinterpret_cast<const float4 *>(dts + j0);
        const float cj[4] = {c4.x, c4.y, c4.z, c4.w};
        const float dj[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const uint32_t w = gt[a >> 1][2 * (a & 1) + (b >> 1)];
            mv[4 * a + b] = hfma(w, b & 1, fast_exp2(fminf(ci - cj[b], capm)) * dj[b], 8 * a + b == dl ? dx : 0.0f);
        }
    }
    const f16x8 mf0 = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(mv[0], mv[1]), pack_f16x2(mv[2], mv[3]),
                                                      pack_f16x2(mv[4], mv[5]), pack_f16x2(mv[6], mv[7])});
    const f16x8 mf1 = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(mv[8], mv[9]), pack_f16x2(mv[10], mv[11]),
                                                      pack_f16x2(mv[12], mv[13]), pack_f16x2(mv[14], mv[15])});
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        f16x8 x0, x1;
        x_operands(sm, l32, hl, rb, pt, x0, x1);
        acc[pt] = mfma32_f16(x0, mf0, acc[pt]);
        acc[pt] = mfma32_f16(x1, mf1, acc[pt]);
    }
}
}  // namespace

template <int N, int HB>
__global__ __launch_bounds__(kThreads) void ssd_chunk_scan_kernel(Params p) {
    constexpr int KS = N / 16;  // K-steps of the off-diagonal product
    constexpr int H_STRIDE = ScanSmem<N>::H_STRIDE;
    constexpr int HVEC = kHeadDim * (N / 8) / kThreads;  // h_in 16-byte vectors per thread
    __shared__ ScanSmem<N> sm;

    // ---- XCD-aware decode: all head blocks of chunk c share one XCD
    const int nhb = p.H / HB;
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / nhb) * 8 + xcd;
    const int cc = min(c, (int)p.nchunks_max - 1);  // a row of the chunk tables
    const int hb = slot - (slot / nhb) * nhb;
    const int h_first = hb * HB;
    const int g = h_first / (p.H / p.G);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    // row block of this wavefront: SIMD k (= wave & 3) runs blocks k and 7-k
    const int rb = (wave >> 2) ? 7 - (wave & 3) : (wave & 3);
    const int i_l = 32 * rb + l32;      // this lane's token (column of y^T)
    int64_t t0 = 0;  // the chunk's first token and length, once the chunk table is read
    int len = 1;

    // ---- per-head inputs.  Two phases per head k, each closed by a barrier:
    //   P(k): stage x^T(k), build the decay table, off-diagonal products
    //   Q(k): diagonal blocks and y(k); stage h_in and the tables of head k+1
    // so the VALU-heavy staging of one part overlaps the products of the
    // other.  Loads run one phase pair ahead: h_in and tables of head k+2 are
    // issued at the end of Q(k), x of head k+1 after staging x^T(k).  They are
    // unconditional (past the last head they repeat it), so the compiler's
    // wait counts never assume a later load is missing and wait for all.
    const int pq = tid & 3;     // x staging: quarter of p
    const int pair = tid >> 2;  // x staging: token pair
    u32x4 hreg[HVEC];
    u32x4 xr[2][2];
    float tab_cs = 0.f, tab_dt = 0.f, tab_dh = 0.f;
    int tab_hx = 0, tab_xe = 0;
    const float *dsrc = p.D ? p.D : p.A;  // a valid address either way; D = 0 when absent
    auto load_tabs = [&](int h) {
        const int64_t r = ((int64_t)cc * p.H + h) * kChunk + (tid & (kChunk - 1));
        tab_cs = p.cs2[r];
        tab_dt = p.dts[r];
        tab_hx = p.hexp[((int64_t)cc * p.H + h) * kHeadDim + (tid & (kHeadDim - 1))];
        tab_dh = dsrc[h];
        // one exponent per half of p (kNoExponent for an all-zero half): the
        // head's is the smaller, that of the larger maximum (0 if all zero)
        const int2 xe2 = *reinterpret_cast<const int2 *>(p.xexp + ((int64_t)cc * p.H + h) * 2);
        tab_xe = min(xe2.x, xe2.y);
        tab_xe = tab_xe == kNoExponent ? 0 : tab_xe;
        const uint16_t *hin_head = p.hin + ((int64_t)cc * p.H + h) * kHeadDim * N;
#pragma unroll
        for (int it = 0; it < HVEC; ++it)
            hreg[it] = *reinterpret_cast<const u32x4 *>(hin_head + (tid + it * kThreads) * 8);
    };
    auto load_x = [&](int h) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            // rows past the chunk end read the last row (len >= 1); they are
            // zeroed when staged
            const int j = min(pair * 2 + e, len - 1);
            const u32x4 *src = reinterpret_cast<const u32x4 *>(p.x + ((t0 + j) * p.H + h) * kHeadDim + pq * 16);
            xr[e][0] = src[0];
            xr[e][1] = src[1];
        }
    };
    const bool has_d = p.D != nullptr;
    auto stage_tabs = [&](int b) {
        if (tid < kChunk) {  // four whole wavefronts
            sm.cs2[b][tid] = tab_cs;
            sm.dts[b][tid] = tab_dt;
            const float m = wave_max(fabsf(tab_dt));
            if ((tid & 63) == 0) sm.dmx[b][tid >> 6] = m;
        } else if (tid < kChunk + kHeadDim) {
            sm.hs[b][tid - kChunk] = ldexpf(1.0f, -tab_hx);
        } else if (tid == kChunk + kHeadDim) {
            sm.dd[b] = has_d ? tab_dh : 0.0f;
            sm.xexp[b] = tab_xe;
        }
#pragma unroll
        for (int it = 0; it < HVEC; ++it) {
            const int idx = tid + it * kThreads;
            const int row = idx / (N / 8), v = idx - row * (N / 8);
            *reinterpret_cast<u32x4 *>(sm.h + row * H_STRIDE + v * 4) = hreg[it];
        }
    };
    const int h_last = h_first + HB - 1;
    // ---- loads that need only the chunk index go out before the chunk
    // table is read: this head's tables and h_in, the row block's C.B^T
    // tiles (all eight loads; past the row block's last tile they repeat it:
    // behind the wavefront-dependent condition each load would wait for the
    // previous one).  Workgroups past the chunk count read row cc, inside
    // the tables, and leave.  At the dstates the short path serves (64 and
    // 128) most rows can be empty (every sequence short): there the count is
    // tested first and such workgroups load nothing.
    if constexpr (N <= 128) {
        if (c >= p.meta[0]) return;
    }
    const int nchunks = p.meta[0];
    const int4 dsc = p.desc[cc];
    load_tabs(h_first);
    u32x4 ga[8], gb[8];
    {
        const uint16_t *cbt = p.cbt + (((int64_t)cc * p.G + g) * 36 + rb * (rb + 1) / 2) * 1024 + lane * 16;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            const int tt = min(t, rb);
            ga[t] = *reinterpret_cast<const u32x4 *>(cbt + tt * 1024);
            gb[t] = *reinterpret_cast<const u32x4 *>(cbt + tt * 1024 + 8);
        }
    }
    // keeps the loads above ahead of the chunk-count test (they would
    // otherwise be moved behind it, and wait for it)
    asm volatile("" ::: "memory");
    if (c >= nchunks) return;
    t0 = dsc.y;
    len = dsc.z;
    const bool active = 32 * rb < len;  // wavefront-uniform
    load_x(h_first);

    // ---- per-group operands of this wavefront's row block, prepared once for all heads
    // C row i_l (raw bf16), 8 values per K-step.  Rows past the chunk end
    // repeat its last row: their outputs are never stored, and in C.B^T they
    // only meet x rows that are zero, so they just need to be finite.
    u32x4 cq[KS];
    const int64_t rstride = (int64_t)p.G * N;  // elements between consecutive tokens of B and C
    {
        const uint16_t *crow = p.C + (t0 + min(i_l, len - 1)) * rstride + (int64_t)g * N + 8 * hl;
#pragma unroll
        for (int k = 0; k < KS; ++k) cq[k] = *reinterpret_cast<const u32x4 *>(crow + 16 * k);
    }
    // this row block's C.B^T tiles into LDS, each lane its own 32 bytes, read
    // back only by the same lane (no barrier needed)
    {
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t <= rb && 32 * t < len) {
                u32x4 *d = reinterpret_cast<u32x4 *>(sm.g) + (rb * (rb + 1) / 2 + t) * 128 + lane;
                d[0] = ga[t];
                d[64] = gb[t];
            }
        }
    }
    const int sg = p.gexp[((int64_t)c * p.G + g) * 4 + min(rb, 7 - rb)];  // exponent of this row block's tiles
    // C rows to fp16 under this wavefront's exponent sc
    int sc;
    {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < KS; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) m = max(m, max(cq[k][q] & 0x7FFFu, (cq[k][q] >> 16) & 0x7FFFu));
        sc = f16_scale_exponent(wave_max(__uint_as_float(m << 16)));
        const float cs = ldexpf(1.0f, sc);
#pragma unroll
        for (int k = 0; k < KS; ++k) {
            u32x4 o;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                o[q] = pack_f16x2(__uint_as_float(cq[k][q] << 16) * cs, __uint_as_float(cq[k][q] & 0xFFFF0000u) * cs);
            cq[k] = o;
        }
    }

    stage_tabs(0);
    // the first head's x is complete before the next loads are issued, so at
    // the loop head, on either path, x is older than everything still in flight
#pragma unroll
    for (int e = 0; e < 2; ++e) asm volatile("" : "+v"(xr[e][0]), "+v"(xr[e][1]));
    load_tabs(min(h_first + 1, h_last));
    __syncthreads();

#pragma unroll 1
    for (int hh = 0; hh < HB; ++hh) {
        const int h = h_first + hh;
        const int b = hh & 1;
        const float *cs2 = sm.cs2[b];
        const float *dts = sm.dts[b];
        // keep the per-group operands opaque across heads, so values derived
        // from them (fp32 copies of the tiles) are not hoisted out of the loop
        // and held in registers for all heads
#pragma unroll
        for (int k = 0; k < KS; ++k) asm volatile("" : "+v"(cq[k]));
        // likewise the lane-derived indices, so masks and addresses are
        // recomputed per head instead of being held in registers
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        const int lane = tid & 63;
        const int l32 = lane & 31;
        const int hl = lane >> 5;
        const int i_l = 32 * rb + l32;
        const int pq = tid & 3;
        const int pair = tid >> 2;

        // ======== P(hh)
        // ---- off-diagonal part: y^T_off = h_in (LDS) x C^T (registers).
        // Wavefronts past the chunk end run it too and discard it.  Of the
        // two wavefronts on a SIMD, the one with the lower row block runs
        // these products first and the staging below after them, the other
        // the reverse, so one's matrix products overlap the other's
        // vector work.
        f32x16 acc[2];
        auto offdiag = [&] {
            // h_in fragments read kPre K-steps ahead of their products
            constexpr int kPre = KS < 4 ? KS : 4;
            const uint32_t *hrow = sm.h + l32 * H_STRIDE + 4 * hl;
            u32x4 hb[kPre][2];
#pragma unroll
            for (int k = 0; k < kPre; ++k)
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
                    hb[k][pt] = *reinterpret_cast<const u32x4 *>(hrow + 32 * pt * H_STRIDE + 8 * k);
#pragma unroll
            for (int k = 0; k < KS; ++k) {
                const f16x8 cf = __builtin_bit_cast(f16x8, cq[k]);
                const u32x4 h0 = hb[k % kPre][0], h1 = hb[k % kPre][1];
                if (k + kPre < KS) {
#pragma unroll
                    for (int pt = 0; pt < 2; ++pt)
                        hb[k % kPre][pt] = *reinterpret_cast<const u32x4 *>(hrow + 32 * pt * H_STRIDE + 8 * (k + kPre));
                }
                // keeps the reads ahead (the scheduler would sink them to their use)
                __builtin_amdgcn_sched_barrier(0);
                acc[0] = mfma32_f16(__builtin_bit_cast(f16x8, h0), cf, k == 0 ? f32x16{} : acc[0]);
                acc[1] = mfma32_f16(__builtin_bit_cast(f16x8, h1), cf, k == 0 ? f32x16{} : acc[1]);
            }
        };
        if (rb < 4) offdiag();

        // ---- x^T: one power of two for the chunk and head, none where x
        // already sits well inside fp16's normal range
        const int xe_raw = sm.xexp[b];
        const float dh = sm.dd[b];
        const int xe = (xe_raw >= 0 && xe_raw <= 20) ? 0 : xe_raw;
        {
            if (len < kChunk) {  // wavefront-uniform: only a partial chunk has rows to clear
#pragma unroll
                for (int e = 0; e < 2; ++e)
                    if (pair * 2 + e >= len) xr[e][0] = xr[e][1] = u32x4{};  // past the chunk end
            }
            if (xe == 0) {
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t a = xr[0][k >> 3][(k >> 1) & 3];
                    const uint32_t b2 = xr[1][k >> 3][(k >> 1) & 3];
                    sm.xt[(pq * 16 + k) * XT_STRIDE + (pair ^ (16 * pq))] =
                        pack_f16x2(__uint_as_float((k & 1) ? (a & 0xFFFF0000u) : (a << 16)),
                                   __uint_as_float((k & 1) ? (b2 & 0xFFFF0000u) : (b2 << 16)));
                }
            } else {
                const float s0 = ldexpf(1.0f, xe);
#pragma unroll
                for (int k = 0; k < 16; ++k) {
                    const uint32_t a = xr[0][k >> 3][(k >> 1) & 3];
                    const uint32_t b2 = xr[1][k >> 3][(k >> 1) & 3];
                    sm.xt[(pq * 16 + k) * XT_STRIDE + (pair ^ (16 * pq))] =
                        pack_f16x2(__uint_as_float((k & 1) ? (a & 0xFFFF0000u) : (a << 16)) * s0,
                                   __uint_as_float((k & 1) ? (b2 & 0xFFFF0000u) : (b2 << 16)) * s0);
                }
            }
        }
        load_x(min(h + 1, h_last));  // next head's x in flight during this head's products

        // ---- bounds, the same in every wavefront: dmax = max |dts|, dgrow =
        // the chunk's total growth when A > 0 (1 otherwise)
        const float4 dm4 = *reinterpret_cast<const float4 *>(sm.dmx[b]);
        const float dmax = fmaxf(fmaxf(dm4.x, dm4.y), fmaxf(dm4.z, dm4.w));
        const float cap = fmaxf(0.f, cs2[kChunk - 1] - cs2[0]);
        const float dgrow = fast_exp2(cap);
        // table scale 2^-kw with |table| < 1
        const float vbound = dmax * dgrow;
        const int kw = vbound > 0.f ? min((int)((__float_as_uint(vbound) >> 23) & 0xFF) - 126, 126) : 0;
        // |M| in units of 2^-xe: |G| dts (decay <= dgrow) < 2^(15 - sg) dmax dgrow, plus |D| on the diagonal
        const int smx = f16_scale_exponent(ldexpf(ldexpf(dmax * dgrow, 15 - sg) + fabsf(dh), -xe));

        // ---- decay table of the tiles below the diagonal blocks
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int d = tid + it * kThreads;
            const int r = d >> 7;
            const int t = (d >> 4) & 7;
            if (t < r) {
                const int j = 32 * t + 8 * ((d >> 1) & 3) + 4 * ((d >> 3) & 1) + 2 * (d & 1);
                const float2 c2 = *reinterpret_cast<const float2 *>(cs2 + j);
                const float2 w2 = *reinterpret_cast<const float2 *>(dts + j);
                const float cr = cs2[32 * r];
                const float sk = ldexpf(1.0f, -kw);
                sm.v[d] = pack_f16x2(fast_exp2(cr - c2.x) * w2.x * sk, fast_exp2(cr - c2.y) * w2.y * sk);
            }
        }

        // ---- this lane's row factors for Q (see there), formed ahead of the barrier
        const float cs_i = cs2[i_l];
        const float cr = cs2[32 * rb];
        // the off-diagonal products' scale: exp2(cs2_i) in the M scale for row
        // block 0, exp2(cs2[32 rb]) in the scale of the tiles below the
        // diagonal block for the others
        float fq = rb > 0 ? ldexpf(fast_exp2(cr), sg + xe - sc - kw) : ldexpf(fast_exp2(cs_i), smx - sc);
        // exp2(cs2_i - cs2[32 rb]) * 2^(kw - sg - xe + smx): below-diagonal scale to the M scale
        float rs = ldexpf(fast_exp2(cs_i - cr), kw - sg - xe + smx);
        const float lmg = (float)(smx - sg - xe);
        float ci = cs_i + lmg;
        asm volatile("" : "+v"(fq), "+v"(rs), "+v"(ci));

        if (rb >= 4) offdiag();
        __syncthreads();  // x^T and the table are complete; h_in is no longer read

        // ======== Q(hh)
        if (active) {  // wavefront-uniform
            // undo the C and h_in scalings and decay column i: in row block 0
            // by exp2(cs2_i), in the M scale; in the others by exp2(cs2[32 rb])
            // only, in the scale of the tiles below the diagonal block, which
            // then accumulate onto it before the rest of the decay
            // (exp2(cs2_i - cs2[32 rb])) is applied per row
#pragma unroll
            for (int pt = 0; pt < 2; ++pt) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 s4 = *reinterpret_cast<const float4 *>(sm.hs[b] + 32 * pt + 8 * a + 4 * hl);
                    acc[pt][4 * a + 0] *= fq * s4.x;
                    acc[pt][4 * a + 1] *= fq * s4.y;
                    acc[pt][4 * a + 2] *= fq * s4.z;
                    acc[pt][4 * a + 3] *= fq * s4.w;
                }
            }
            // ---- diagonal block: the tiles below its diagonal tile (code
            // specialised per row block), then the per-row decay to the M
            // scale, then the diagonal tile itself
            if (rb > 0) {  // wavefront-uniform
                switch (rb) {
                case 1: below_diag<N, 1>(sm, acc, lane); break;
                case 2: below_diag<N, 2>(sm, acc, lane); break;
                case 3: below_diag<N, 3>(sm, acc, lane); break;
                case 4: below_diag<N, 4>(sm, acc, lane); break;
                case 5: below_diag<N, 5>(sm, acc, lane); break;
                case 6: below_diag<N, 6>(sm, acc, lane); break;
                default: below_diag<N, 7>(sm, acc, lane); break;
                }
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int e = 0; e < 16; ++e) acc[pt][e] *= rs;
            }
            diag_tile(sm, cs2, dts, acc, lane, rb, ci, cap + lmg, ldexpf(dh, smx - xe));
            // ---- back to unit scale, store bf16.  Lane l holds p = 32 pt + 8a +
            // 4(l/32) + 0..3 of token i_l (a = 0..3).  Stores that write whole
            // 128-byte lines (8 tokens x 64 p per instruction) run at about twice
            // the rate of 32-byte pieces of 32 lines, so three exchanges first
            // move the p bits above 2 into lane bits and token bits into the
            // register index: a 32-lane swap trades p bit 2 (lane bit 5) for p
            // bit 3, a 16-lane swap p bit 4 for token bit 4 (lane bit 4), and a
            // quad exchange p bit 5 for token bit 0 (lane bit 0).  Lane l then
            // holds the 16-byte piece 4(l & 1) + 2((l >> 4) & 1) + (l >> 5) of
            // the tokens 32 rb + 16 t4 + (l & 14) + b (t4, b = 0, 1), one store
            // each.
            // The buffer store's range check (the chunk's rows of y) drops the
            // tokens past the chunk end without a branch.
            {
                const float inv = ldexpf(1.0f, -smx);
                uint32_t e[2][2][2][2];  // [p bit 5][p bit 4][p bit 2][p bit 1]
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int a = 0; a < 4; a += 2)
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint32_t lo = pack_bf16x2(acc[pt][4 * a + 2 * q] * inv, acc[pt][4 * a + 2 * q + 1] * inv);
                            const uint32_t hi = pack_bf16x2(acc[pt][4 * a + 4 + 2 * q] * inv, acc[pt][4 * a + 5 + 2 * q] * inv);
                            const auto sw = __builtin_amdgcn_permlane32_swap(lo, hi, false, false);
                            e[pt][a >> 1][0][q] = sw[0];
                            e[pt][a >> 1][1][q] = sw[1];
                        }
                uint32_t f[2][2][2][2];  // [p bit 5][token bit 4][p bit 2][p bit 1]
#pragma unroll
                for (int pt = 0; pt < 2; ++pt)
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const auto sw = __builtin_amdgcn_permlane16_swap(e[pt][0][u][q], e[pt][1][u][q], false, false);
                            f[pt][0][u][q] = sw[0];
                            f[pt][1][u][q] = sw[1];
                        }
                const bool odd = lane & 1;
                const uint64_t ybase = reinterpret_cast<uint64_t>(p.y + t0 * p.H * kHeadDim);
                // readfirstlane returns int: widen each word through uint32_t
                // (a direct cast would sign-extend the low word into the high one)
                const uint64_t yb = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)ybase) |
                                    ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(ybase >> 32)) << 32);
                const __amdgpu_buffer_rsrc_t yr = __builtin_amdgcn_make_buffer_rsrc(
                    reinterpret_cast<void *>(yb), 0, len * p.H * kHeadDim * 2, kBufferFormat32);
                const int piece = 4 * (lane & 1) + 2 * ((lane >> 4) & 1) + (lane >> 5);
                const int tok = 32 * rb + (lane & 14);
#pragma unroll
                for (int t4 = 0; t4 < 2; ++t4) {
                    uint32_t g[2][2][2];  // [token bit 0][p bit 2][p bit 1]
#pragma unroll
                    for (int u = 0; u < 2; ++u)
#pragma unroll
                        for (int q = 0; q < 2; ++q) {
                            const uint32_t send = odd ? f[0][t4][u][q] : f[1][t4][u][q];
                            const uint32_t got = __builtin_amdgcn_update_dpp(0u, send, kQuadSwap01, 0xF, 0xF, false);
                            g[0][u][q] = odd ? got : f[0][t4][u][q];
                            g[1][u][q] = odd ? f[1][t4][u][q] : got;
                        }
#pragma unroll
                    for (int t0b = 0; t0b < 2; ++t0b)
                        __builtin_amdgcn_raw_buffer_store_b128(
                            u32x4{g[t0b][0][0], g[t0b][0][1], g[t0b][1][0], g[t0b][1][1]}, yr,
                            ((tok + 16 * t4 + t0b) * p.H + h) * (kHeadDim * 2) + 16 * piece, 0, 0);
                }
            }
        }
        // h_in and tables of the next head, then those of the one after in
        // flight.  Also after the last head (restaging it into the spare
        // buffer), so every path back to the loop head passes the same loads.
        stage_tabs(b ^ 1);
        load_tabs(min(h + 2, h_last));
        __syncthreads();
    }
}

// Heads per workgroup: the largest of 16, 8, 4, 2, 1 that divides the heads
// of a group and still gives at least one workgroup per compute unit (a
// workgroup fills a compute unit; more heads per workgroup amortise its
// shared operands and its start-up loads).
static int heads_per_block(const Params &p) {
    const int hg = p.H / p.G;
    const int64_t chunks = (p.nchunks_grid + 7) / 8 * 8;
    for (int hb = 16; hb > 1; hb /= 2)
        if (hg % hb == 0 && chunks * (p.H / hb) >= (int64_t)p.num_cus) return hb;
    return 1;
}

template <int N, int HB>
static hipError_t launch_nh(const Params &p, const Launch &l) {
    const int64_t slots = (p.nchunks_grid + 7) / 8 * (p.H / HB);
    return launch_kernel(ssd_chunk_scan_kernel<N, HB>, dim3((unsigned)(slots * 8)), dim3(kThreads), l, p);
}

template <int N>
static hipError_t launch_n(const Params &p, const Launch &l) {
    switch (heads_per_block(p)) {
    case 16: return launch_nh<N, 16>(p, l);
    case 8: return launch_nh<N, 8>(p, l);
    case 4: return launch_nh<N, 4>(p, l);
    case 2: return launch_nh<N, 2>(p, l);
    default: return launch_nh<N, 1>(p, l);
    }
}

hipError_t launch_chunk_scan(const Params &p, const Launch &l) {
    switch (p.N) {
    case 64: return launch_n<64>(p, l);
    case 128: return launch_n<128>(p, l);
    case 256: return launch_n<256>(p, l);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
