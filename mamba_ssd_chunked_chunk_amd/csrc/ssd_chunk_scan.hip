// Step 4 of the scan: the outputs of one chunk ("chunk_scan").
//
// For chunk c of sequence b, head h (group g), and rows i, j of the chunk
// (cs2 = log2(e) * cumulative A*dts, h_in = state entering the chunk):
//   G[i][j]   = sum_n C[i,g,n] * B[j,g,n]
//   M[i][j]   = G[i][j] * exp2(cs2_i - cs2_j) * dts_j     for j <= i, else 0
//   y[i][p]   = sum_j M[i][j] * x[j,h,p]                              (diagonal block)
//             + exp2(cs2_i) * sum_n C[i,g,n] * h_in[p][n]             (off-diagonal part)
//             + D[h] * x[i,h,p]                                       (skip term)
// This is the chunked form of "Mamba chunk scan with segsum" (description:
// intra-chunk attention-like block from segment sums, inter-chunk state,
// their sum); D*x is the skip term of "mamba2_ssd_scan" ("Per-token
// recurrence").  y is rounded to bf16.
//
// Work split.  G depends only on (chunk, group), so one workgroup takes a
// chunk and HW heads of one group.  A single pass over n (32 at a time, the
// next slice prefetched into registers) forms G and, with the same C
// fragments, the off-diagonal products C * h_in^T of all HW heads.  A second
// phase then runs the diagonal block of each head from G kept in registers.
// Eight wavefronts, one 32-row block each; the two wavefronts that share a
// SIMD own row blocks k and 7-k, so each SIMD multiplies 9 of the 36
// lower-triangular 32x32 tiles.  Workgroups are numbered so that all head
// groups of a chunk land on one XCD (dispatch is round-robin over the 8 XCDs)
// and share B and C in its L2.
//
// MFMA layout (32x32x16).  G is formed transposed (rows j, columns i) over n,
// so the accumulator layout of a G tile (16 values per lane, all at one i, at
// j = 8a + 4(l/32) + b) is directly the A-operand layout of M for M*x: the 16
// j of the first K-step are {0..3, 8..11} for lanes 0-31 and {4..7, 12..15}
// for lanes 32-63 (a permutation of 0..15), likewise 16..31 for the second;
// x is read from LDS in the same order.  The C fragment of a K-step is the B
// operand of G^T and, converted to fp16, the A operand of C*h^T.
//
// Decay without one exp2 per element.  For a tile strictly below the
// diagonal block (all j < 32*rb <= i), exp2(cs2_i - cs2_j) =
// exp2(cs2_i - cs2_r) * exp2(cs2_r - cs2_j) with r = 32*rb; both factors are
// at most 1 for A <= 0.  The second factor (times dts_j and the x row scale)
// is tabulated once per head in LDS; only the diagonal blocks use exp2 per
// element.  The skip term D*x is folded into the diagonal of M.
//
// Precision.  G comes from bf16 MFMA on the exact bf16 inputs (fp32
// accumulate).  M and h_in are rounded to fp16 (11-bit significand) under
// power-of-two scales that keep them far from overflow (one per workgroup and
// head for M, one per row for h_in); C is converted to fp16 exactly after a
// power-of-two scaling per (chunk, group), and each x row after its own
// power-of-two scaling compensated inside M.  bf16 (8 bits) for M or h_in
// would put the rounding error, which scales with the typical size of y
// rather than with each y, close to the tolerance wherever y is near zero.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kThreads = 512;
constexpr int XT_STRIDE = 130;  // dwords per x^T row: 128 token pairs + pad (8-byte aligned rows)
constexpr int R_STRIDE = 20;    // dwords per staged row of 32 16-bit values + pad

template <int HW>
struct ScanSmem {
    union {
        struct {  // phase 1: one n-slice of B, C (bf16) and the heads' h_in (fp16)
            uint32_t b[kChunk * R_STRIDE];
            uint32_t c[kChunk * R_STRIDE];
            uint32_t h[HW * kHeadDim * R_STRIDE];
        } g;
        struct {  // phase 2: one head
            uint32_t xt[kHeadDim * XT_STRIDE];
            float v[8 * kChunk];  // row block r: exp2(cs2[32r]-cs2[j]) * dts_j * 2^-xe_j, j < 32r
            float ei[kChunk];     // exp2(cs2_i)
        } hd;
    } u;
    float cs2[HW][kChunk];
    float dts[HW][kChunk];
    int hexp[HW][kHeadDim];
    int xexp[kChunk];
    float red[8][2];
};

// Contents of one n-slice held in registers while the previous slice is
// being multiplied.
template <int HW>
struct SliceRegs {
    u32x4 b[2], c[2];
    u32x4 h[(HW * kHeadDim * 4 + kThreads - 1) / kThreads];
};

__device__ __forceinline__ u32x4 lds_u32x4(const uint32_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

// 8 bf16 (as 4 dwords) -> 8 fp16 scaled by `scale` (a power of two)
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(const u32x4 v, float scale) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = pack_f16x2(__uint_as_float(v[k] << 16) * scale, __uint_as_float(v[k] & 0xFFFF0000u) * scale);
    return __builtin_bit_cast(f16x8, r);
}
}  // namespace

template <int N, int HW>
__global__ __launch_bounds__(kThreads, 1) void ssd_chunk_scan_kernel(Params p) {
    constexpr int KS = N / 32;
    constexpr int HV = (HW * kHeadDim * 4 + kThreads - 1) / kThreads;  // h_in vectors per thread per slice
    __shared__ ScanSmem<HW> sm;

    // ---- XCD-aware decode: all head groups of chunk c share one XCD
    const int nhg = p.H / HW;
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / nhg) * 8 + xcd;
    const int hg = slot - (slot / nhg) * nhg;
    if (c >= p.meta[0]) return;
    const int4 dsc = p.desc[c];
    const int64_t t0 = dsc.y;
    const int len = dsc.z;
    const int h_first = hg * HW;
    const int g = h_first / (p.H / p.G);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    // row block of this wavefront: SIMD k (= wave & 3) runs blocks k and 7-k
    const int rb = (wave >> 2) ? 7 - (wave & 3) : (wave & 3);

    const int sb = p.bexp[(int64_t)c * p.G + g];
    const int sc = p.cexp[(int64_t)c * p.G + g];
    const float c_scale = ldexpf(1.0f, sc);

    for (int e = tid; e < HW * kChunk; e += kThreads) {
        const int hh = e >> 8, j = e & 255;
        const int64_t crow = ((int64_t)c * p.H + h_first + hh) * kChunk;
        sm.cs2[hh][j] = p.cs2[crow + j];
        sm.dts[hh][j] = p.dts[crow + j];
    }
    for (int e = tid; e < HW * kHeadDim; e += kThreads) {
        const int hh = e >> 6, pp = e & 63;
        sm.hexp[hh][pp] = p.hexp[((int64_t)c * p.H + h_first + hh) * kHeadDim + pp];
    }

    // ================= phase 1: G^T[j][i] and C * h_in^T for all HW heads
    auto load_slice = [&](int ks, SliceRegs<HW> &r) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int j = (tid + it * kThreads) >> 2;
            const int v = tid & 3;
            r.b[it] = u32x4{0u, 0u, 0u, 0u};
            r.c[it] = u32x4{0u, 0u, 0u, 0u};
            if (j < len) {
                const int64_t off = ((t0 + j) * p.G + g) * N + ks * 32 + v * 8;
                r.b[it] = *reinterpret_cast<const u32x4 *>(p.B + off);
                r.c[it] = *reinterpret_cast<const u32x4 *>(p.C + off);
            }
        }
#pragma unroll
        for (int it = 0; it < HV; ++it) {
            const int idx = tid + it * kThreads;
            if (idx < HW * kHeadDim * 4) {
                const int row = idx >> 2;  // hh * 64 + p
                const int v = idx & 3;
                r.h[it] = *reinterpret_cast<const u32x4 *>(
                    p.hin + (((int64_t)c * p.H + h_first + (row >> 6)) * kHeadDim + (row & 63)) * N +
                    ks * 32 + v * 8);
            }
        }
    };
    auto store_slice = [&](const SliceRegs<HW> &r) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int j = (tid + it * kThreads) >> 2;
            const int v = tid & 3;
            *reinterpret_cast<u32x4 *>(sm.u.g.b + j * R_STRIDE + v * 4) = r.b[it];
            *reinterpret_cast<u32x4 *>(sm.u.g.c + j * R_STRIDE + v * 4) = r.c[it];
        }
#pragma unroll
        for (int it = 0; it < HV; ++it) {
            const int idx = tid + it * kThreads;
            if (idx < HW * kHeadDim * 4)
                *reinterpret_cast<u32x4 *>(sm.u.g.h + (idx >> 2) * R_STRIDE + (idx & 3) * 4) = r.h[it];
        }
    };

    f32x16 accg[8];
    f32x16 accy[HW][2];
#pragma unroll
    for (int t = 0; t < 8; ++t) accg[t] = f32x16{};
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) accy[hh][0] = accy[hh][1] = f32x16{};

    SliceRegs<HW> sr;
    load_slice(0, sr);
    for (int ks = 0; ks < KS; ++ks) {
        __syncthreads();  // previous slice consumed
        store_slice(sr);
        if (ks + 1 < KS) load_slice(ks + 1, sr);  // in flight during this slice's MFMAs
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const u32x4 craw = lds_u32x4(sm.u.g.c + (32 * rb + l32) * R_STRIDE + 8 * kk + 4 * hl);
            const bf16x8 cb = __builtin_bit_cast(bf16x8, craw);
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t <= rb) {
                    const bf16x8 bb = __builtin_bit_cast(
                        bf16x8, lds_u32x4(sm.u.g.b + (32 * t + l32) * R_STRIDE + 8 * kk + 4 * hl));
                    accg[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb, cb, accg[t], 0, 0, 0);
                }
            }
            const f16x8 cf = bf16x8_to_f16x8(craw, c_scale);
#pragma unroll
            for (int hh = 0; hh < HW; ++hh)
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const f16x8 hf = __builtin_bit_cast(
                        f16x8, lds_u32x4(sm.u.g.h + (hh * kHeadDim + 32 * pt + l32) * R_STRIDE + 8 * kk + 4 * hl));
                    accy[hh][pt] = mfma32_f16(cf, hf, accy[hh][pt]);
                }
        }
    }

    // bound on |G|: |C_i . B_j| <= N max|B| max|C| < N 2^(15-sb) 2^(15-sc)
    const float gbound = ldexpf((float)N, 30 - sb - sc);

    // ================= phase 2: the diagonal block of each head
#pragma unroll
    for (int hh = 0; hh < HW; ++hh) {
        const int h = h_first + hh;
        const float *cs2 = sm.cs2[hh];
        const float *dts = sm.dts[hh];
        __syncthreads();  // phase 1 / previous head done with the shared buffers
        // x^T: thread = (quarter of p, token pair); each x row scaled by its own 2^xe
        {
            const int pq = tid & 3;
            const int pair = tid >> 2;
            u32x4 v[2][2];
            uint32_t mrow[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const int j = pair * 2 + e;
                if (j < len) {
                    const u32x4 *src = reinterpret_cast<const u32x4 *>(
                        p.x + ((t0 + j) * p.H + h) * kHeadDim + pq * 16);
                    v[e][0] = src[0];
                    v[e][1] = src[1];
                } else {
                    v[e][0] = u32x4{0u, 0u, 0u, 0u};
                    v[e][1] = u32x4{0u, 0u, 0u, 0u};
                }
                uint32_t m = 0;
#pragma unroll
                for (int a = 0; a < 2; ++a)
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const uint32_t lo = v[e][a][k] & 0x7FFFu, hi = (v[e][a][k] >> 16) & 0x7FFFu;
                        m = m > lo ? m : lo;
                        m = m > hi ? m : hi;
                    }
                // row max over the 4 lanes holding this token
                uint32_t o = (uint32_t)__shfl_xor((int)m, 1, 64);
                m = m > o ? m : o;
                o = (uint32_t)__shfl_xor((int)m, 2, 64);
                mrow[e] = m > o ? m : o;
            }
            const int xe0 = mrow[0] == 0 ? 0 : 14 - ((int)(mrow[0] >> 7) - 127);
            const int xe1 = mrow[1] == 0 ? 0 : 14 - ((int)(mrow[1] >> 7) - 127);
            if (pq == 0) {
                sm.xexp[pair * 2] = xe0;
                sm.xexp[pair * 2 + 1] = xe1;
            }
            const float s0 = ldexpf(1.0f, xe0), s1 = ldexpf(1.0f, xe1);
#pragma unroll
            for (int k = 0; k < 16; ++k) {
                const uint32_t a = v[0][k >> 3][(k >> 1) & 3];
                const uint32_t b = v[1][k >> 3][(k >> 1) & 3];
                const float lo = __uint_as_float((k & 1) ? (a & 0xFFFF0000u) : (a << 16));
                const float hi = __uint_as_float((k & 1) ? (b & 0xFFFF0000u) : (b << 16));
                sm.u.hd.xt[(pq * 16 + k) * XT_STRIDE + pair] = pack_f16x2(lo * s0, hi * s1);
            }
        }
        __syncthreads();
        // decay tables and the bound on |M|
#pragma unroll
        for (int it = 0; it < 8 * kChunk / kThreads; ++it) {
            const int e = tid + it * kThreads;
            const int r = e >> 8;
            const int j = e & 255;
            float val = 0.f;
            if (j < 32 * r) val = ldexpf(fast_exp2(cs2[32 * r] - cs2[j]) * dts[j], -sm.xexp[j]);
            sm.u.hd.v[e] = val;
        }
        float wmax = 0.f, emax = 0.f;
        if (tid < kChunk) {
            sm.u.hd.ei[tid] = fast_exp2(cs2[tid]);
            emax = ldexpf(1.0f, -sm.xexp[tid]);
            wmax = fabsf(dts[tid]) * emax;
        }
        wmax = wave_max(wmax);
        emax = wave_max(emax);
        if (lane == 0) { sm.red[wave][0] = wmax; sm.red[wave][1] = emax; }
        __syncthreads();
        wmax = fmaxf(fmaxf(sm.red[0][0], sm.red[1][0]), fmaxf(sm.red[2][0], sm.red[3][0]));
        emax = fmaxf(fmaxf(sm.red[0][1], sm.red[1][1]), fmaxf(sm.red[2][1], sm.red[3][1]));
        const float dh = p.D ? p.D[h] : 0.0f;
        // |2^-xe M| <= |G| * max(dts 2^-xe) * (decay <= 1, or the chunk's total
        // growth when A > 0) + |D| max(2^-xe) on the diagonal
        const float dgrow = fast_exp2(fmaxf(0.f, cs2[kChunk - 1] - cs2[0]));
        const int smx = f16_scale_exponent(gbound * wmax * dgrow + fabsf(dh) * emax);
        const float m_scale = ldexpf(1.0f, smx);

        // off-diagonal part: undo the C and h_in scalings, decay row i by
        // exp2(cs2_i), move to the M scale
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            const float f = ldexpf(1.0f, smx - (sc + sm.hexp[hh][32 * pt + l32]));
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const float4 d4 = *reinterpret_cast<const float4 *>(sm.u.hd.ei + 32 * rb + 8 * a + 4 * hl);
                accy[hh][pt][4 * a + 0] *= f * d4.x;
                accy[hh][pt][4 * a + 1] *= f * d4.y;
                accy[hh][pt][4 * a + 2] *= f * d4.z;
                accy[hh][pt][4 * a + 3] *= f * d4.w;
            }
        }

        // diagonal block: (2^smx M 2^-xe) (2^xe x)
        const int i_a = 32 * rb + l32;  // this lane's row in the A layout
        const float cs_i = cs2[i_a];
        const float u = fast_exp2(cs_i - cs2[32 * rb]) * m_scale;
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            if (t <= rb) {
                float mv[16];
                if (t < rb) {
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const float4 v4 = *reinterpret_cast<const float4 *>(
                            sm.u.hd.v + rb * kChunk + 32 * t + 8 * a + 4 * hl);
                        mv[4 * a + 0] = accg[t][4 * a + 0] * (v4.x * u);
                        mv[4 * a + 1] = accg[t][4 * a + 1] * (v4.y * u);
                        mv[4 * a + 2] = accg[t][4 * a + 2] * (v4.z * u);
                        mv[4 * a + 3] = accg[t][4 * a + 3] * (v4.w * u);
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 16; ++e) {
                        const int j = 32 * t + 8 * (e >> 2) + 4 * hl + (e & 3);
                        float val = accg[t][e] * fast_exp2(cs_i - cs2[j]) * dts[j];
                        if (j == i_a) val += dh;
                        mv[e] = j <= i_a ? ldexpf(val, smx - sm.xexp[j]) : 0.f;
                    }
                }
                const f16x8 mf0 = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(mv[0], mv[1]), pack_f16x2(mv[2], mv[3]),
                                                                  pack_f16x2(mv[4], mv[5]), pack_f16x2(mv[6], mv[7])});
                const f16x8 mf1 = __builtin_bit_cast(f16x8, u32x4{pack_f16x2(mv[8], mv[9]), pack_f16x2(mv[10], mv[11]),
                                                                  pack_f16x2(mv[12], mv[13]), pack_f16x2(mv[14], mv[15])});
#pragma unroll
                for (int pt = 0; pt < 2; ++pt) {
                    const uint32_t *row = sm.u.hd.xt + (32 * pt + l32) * XT_STRIDE + 16 * t + 2 * hl;
                    const f16x8 x0 = __builtin_bit_cast(f16x8, u32x4{row[0], row[1], row[4], row[5]});
                    const f16x8 x1 = __builtin_bit_cast(f16x8, u32x4{row[8], row[9], row[12], row[13]});
                    accy[hh][pt] = mfma32_f16(mf0, x0, accy[hh][pt]);
                    accy[hh][pt] = mfma32_f16(mf1, x1, accy[hh][pt]);
                }
            }
        }

        // back to unit scale, store bf16
        const float inv = ldexpf(1.0f, -smx);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int i = 32 * rb + 8 * (e >> 2) + 4 * hl + (e & 3);
            if (i < len) {
                uint16_t *dst = p.y + ((t0 + i) * p.H + h) * kHeadDim + l32;
                dst[0] = float_to_bf16_bits(accy[hh][0][e] * inv);
                dst[32] = float_to_bf16_bits(accy[hh][1][e] * inv);
            }
        }
    }
}

// Heads per workgroup (1 or 2, dividing H/G; more would not fit the
// accumulators of all heads in the register file).  One workgroup runs per CU;
// a workgroup costs about one unit for G plus one unit per head, and the grid
// runs in ceil(workgroups / CUs) rounds.  Pick the smallest
// rounds * (G + heads) estimate.
int chunk_scan_heads_per_wg(const Params &p) {
    const int hpg = p.H / p.G;
    const double g_cost = 1.4;  // G^T relative to one head, from their MFMA counts
    int best = 1;
    double best_cost = 1e300;
    for (int hw = 1; hw <= 2 && hw <= hpg; hw *= 2) {
        if (hpg % hw) continue;
        const int64_t wgs = p.nchunks_max * (p.H / hw);
        const double rounds = (double)((wgs + p.num_cus - 1) / p.num_cus);
        const double cost = rounds * (g_cost + hw);
        if (cost < best_cost) { best_cost = cost; best = hw; }
    }
    return best;
}

template <int N>
static hipError_t launch_n(const Params &p, hipStream_t s) {
    const int hw = chunk_scan_heads_per_wg(p);
    const int64_t slots = (p.nchunks_max + 7) / 8 * (p.H / hw);
    const dim3 grid((unsigned)(slots * 8));
    if (hw == 2) hipLaunchKernelGGL((ssd_chunk_scan_kernel<N, 2>), grid, dim3(kThreads), 0, s, p);
    else hipLaunchKernelGGL((ssd_chunk_scan_kernel<N, 1>), grid, dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_chunk_scan(const Params &p, hipStream_t s) {
    switch (p.N) {
    case 64: return launch_n<64>(p, s);
    case 128: return launch_n<128>(p, s);
    case 256: return launch_n<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
