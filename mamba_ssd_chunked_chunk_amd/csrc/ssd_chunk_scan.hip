// Step 4 of the scan: the outputs of one chunk ("chunk_scan").
//
// For chunk c of sequence b, head h (group g), and rows i, j of the chunk
// (cs2 = log2(e) * cumulative A*dts, h_in = state entering the chunk):
//   G[i][j]   = sum_n C[i,g,n] * B[j,g,n]                  (formed by the prep step)
//   M[i][j]   = G[i][j] * exp2(cs2_i - cs2_j) * dts_j     for j <= i, else 0
//   y[i][p]   = sum_j M[i][j] * x[j,h,p]                              (diagonal block)
//             + exp2(cs2_i) * sum_n C[i,g,n] * h_in[p][n]             (off-diagonal part)
//             + D[h] * x[i,h,p]                                       (skip term)
// This is the chunked form of "Mamba chunk scan with segsum" (description:
// intra-chunk attention-like block from segment sums, inter-chunk state,
// their sum); D*x is the skip term of "mamba2_ssd_scan" ("Per-token
// recurrence").  y is rounded to bf16.
//
// Work split.  One workgroup per (chunk, head), eight wavefronts, one 32-row
// block each; the two wavefronts that share a SIMD own row blocks k and 7-k,
// so each SIMD handles 9 of the 36 lower-triangular 32x32 tiles.  Workgroups
// are numbered so that all heads of a chunk land on one XCD (dispatch is
// round-robin over the 8 XCDs) and share C and the C.B^T tiles in its L2.
// Every global load a wavefront needs (its C rows, the head's h_in and x, its
// first C.B^T tiles) is issued at the start, so they are all in flight
// together while the workgroup stages x and builds its decay tables.
//
// MFMA layout (v_mfma_f32_32x32x16).  C.B^T is stored transposed (rows j,
// columns i) in accumulator order, so a tile's 16 values per lane (all at one
// i, at j = 8a + 4(l/32) + b) are directly the A-operand layout of M for
// M*x: the 16 j of the first K-step are {0..3, 8..11} for lanes 0-31 and
// {4..7, 12..15} for lanes 32-63 (a permutation of 0..15), likewise 16..31
// for the second; x is read from LDS in the same order.
//
// Decay without one exp2 per element.  For a tile strictly below the
// diagonal block (all j < 32*rb <= i), exp2(cs2_i - cs2_j) =
// exp2(cs2_i - cs2_r) * exp2(cs2_r - cs2_j) with r = 32*rb; both factors are
// at most 1 for A <= 0.  The second factor (times dts_j and the x row scale)
// is tabulated once in LDS; only the diagonal tile evaluates exp2 per
// element.  The skip term D*x is folded into the diagonal of M.
//
// Precision.  M and h_in are rounded to fp16 (11-bit significand) under
// power-of-two scales that keep them far from overflow (one per workgroup for
// M, one per row for h_in); C is converted to fp16 exactly after a
// power-of-two scaling per (chunk, group), and each x row after its own
// power-of-two scaling compensated inside M.  All products accumulate in
// fp32.  bf16 (8 bits) for M or h_in would put the rounding error, which
// scales with the typical size of y rather than with each y, close to the
// tolerance wherever y is near zero.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kThreads = 512;
constexpr int XT_STRIDE = 130;  // dwords per x^T row: 128 token pairs + pad (8-byte aligned rows)

template <int N>
struct __attribute__((aligned(16))) ScanSmem {
    static constexpr int H_STRIDE = N / 2 + 4;  // dwords per h_in row + pad
    uint32_t h[kHeadDim * H_STRIDE];
    uint32_t xt[kHeadDim * XT_STRIDE];
    float v[8 * kChunk];  // row block r: exp2(cs2[32r]-cs2[j]) * dts_j * 2^-xe_j, j < 32r
    float ei[kChunk];     // exp2(cs2_i)
    float cs2[kChunk];
    float dts[kChunk];
    int xexp[kChunk];
    int hexp[kHeadDim];
    float red[8][2];
};

// 8 bf16 (as 4 dwords) -> 8 fp16 scaled by `scale` (a power of two)
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(const u32x4 v, float scale) {
    u32x4 r;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r[k] = pack_f16x2(__uint_as_float(v[k] << 16) * scale, __uint_as_float(v[k] & 0xFFFF0000u) * scale);
    return __builtin_bit_cast(f16x8, r);
}

__device__ __forceinline__ f32x16 load_tile(const float *src) {
    const float4 *s4 = reinterpret_cast<const float4 *>(src);
    f32x16 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 v = s4[q];
        r[4 * q] = v.x; r[4 * q + 1] = v.y; r[4 * q + 2] = v.z; r[4 * q + 3] = v.w;
    }
    return r;
}
}  // namespace

template <int N>
__global__ __launch_bounds__(kThreads, 1) void ssd_chunk_scan_kernel(Params p) {
    constexpr int KS = N / 16;  // K-steps of the off-diagonal product
    constexpr int H_STRIDE = ScanSmem<N>::H_STRIDE;
    constexpr int HVEC = kHeadDim * (N / 8) / kThreads;  // h_in 16-byte vectors per thread
    __shared__ ScanSmem<N> sm;

    // ---- XCD-aware decode: all heads of chunk c share one XCD
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / p.H) * 8 + xcd;
    const int h = slot - (slot / p.H) * p.H;
    if (c >= p.meta[0]) return;
    const int4 dsc = p.desc[c];
    const int64_t t0 = dsc.y;
    const int len = dsc.z;
    const int g = h / (p.H / p.G);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    // row block of this wavefront: SIMD k (= wave & 3) runs blocks k and 7-k
    const int rb = (wave >> 2) ? 7 - (wave & 3) : (wave & 3);

    // ---- issue every early global load
    // C rows of this wavefront's row block, in the A-operand layout (zero past the chunk end)
    u32x4 cfr[KS];
    {
        const int i = 32 * rb + l32;
        const uint16_t *crow = p.C + ((t0 + min(i, len - 1)) * p.G + g) * N + 8 * hl;
#pragma unroll
        for (int k = 0; k < KS; ++k) cfr[k] = i < len ? *reinterpret_cast<const u32x4 *>(crow + 16 * k) : u32x4{};
    }
    // the head's h_in rows
    u32x4 hreg[HVEC];
    const uint16_t *hin_head = p.hin + ((int64_t)c * p.H + h) * kHeadDim * N;
#pragma unroll
    for (int it = 0; it < HVEC; ++it) hreg[it] = *reinterpret_cast<const u32x4 *>(hin_head + (tid + it * kThreads) * 8);
    // x: thread = (quarter of p, token pair)
    const int pq = tid & 3;
    const int pair = tid >> 2;
    u32x4 xr[2][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int j = pair * 2 + e;
        if (j < len) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(p.x + ((t0 + j) * p.H + h) * kHeadDim + pq * 16);
            xr[e][0] = src[0];
            xr[e][1] = src[1];
        } else {
            xr[e][0] = xr[e][1] = u32x4{};
        }
    }
    // the first two C.B^T tiles of this row block
    const float *cbt = p.cbt + (((int64_t)c * p.G + g) * 36 + rb * (rb + 1) / 2) * 1024 + lane * 16;
    f32x16 gt[2];
    gt[0] = load_tile(cbt);
    gt[1] = rb >= 1 ? load_tile(cbt + 1024) : f32x16{};
    const int64_t crow = ((int64_t)c * p.H + h) * kChunk;
    if (tid < kChunk) {
        sm.cs2[tid] = p.cs2[crow + tid];
        sm.dts[tid] = p.dts[crow + tid];
    } else if (tid < kChunk + kHeadDim) {
        sm.hexp[tid - kChunk] = p.hexp[((int64_t)c * p.H + h) * kHeadDim + (tid - kChunk)];
    }
    const int sc = p.cexp[(int64_t)c * p.G + g];
    const float c_scale = ldexpf(1.0f, sc);
    const float dh = p.D ? p.D[h] : 0.0f;

    // ---- stage h_in and x^T (each x row scaled by its own 2^xe)
#pragma unroll
    for (int it = 0; it < HVEC; ++it) {
        const int idx = tid + it * kThreads;
        const int row = idx / (N / 8), v = idx - row * (N / 8);
        *reinterpret_cast<u32x4 *>(sm.h + row * H_STRIDE + v * 4) = hreg[it];
    }
    {
        uint32_t mrow[2];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            uint32_t m = 0;
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = xr[e][a][k] & 0x7FFFu, hi = (xr[e][a][k] >> 16) & 0x7FFFu;
                    m = max(m, max(lo, hi));
                }
            // row max over the 4 lanes holding this token
            m = max(m, (uint32_t)__shfl_xor((int)m, 1, 64));
            mrow[e] = max(m, (uint32_t)__shfl_xor((int)m, 2, 64));
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
            const uint32_t a = xr[0][k >> 3][(k >> 1) & 3];
            const uint32_t b = xr[1][k >> 3][(k >> 1) & 3];
            const float lo = __uint_as_float((k & 1) ? (a & 0xFFFF0000u) : (a << 16));
            const float hi = __uint_as_float((k & 1) ? (b & 0xFFFF0000u) : (b << 16));
            sm.xt[(pq * 16 + k) * XT_STRIDE + pair] = pack_f16x2(lo * s0, hi * s1);
        }
    }
    __syncthreads();

    // ---- decay tables and the bound on |M|
#pragma unroll
    for (int it = 0; it < 8 * kChunk / kThreads; ++it) {
        const int e = tid + it * kThreads;
        const int r = e >> 8;
        const int j = e & 255;
        float val = 0.f;
        if (j < 32 * r) val = ldexpf(fast_exp2(sm.cs2[32 * r] - sm.cs2[j]) * sm.dts[j], -sm.xexp[j]);
        sm.v[e] = val;
    }
    float wmax = 0.f, emax = 0.f;
    if (tid < kChunk) {
        sm.ei[tid] = fast_exp2(sm.cs2[tid]);
        emax = ldexpf(1.0f, -sm.xexp[tid]);
        wmax = fabsf(sm.dts[tid]) * emax;
    }
    wmax = wave_max(wmax);
    emax = wave_max(emax);
    if (lane == 0) { sm.red[wave][0] = wmax; sm.red[wave][1] = emax; }

    // ---- off-diagonal part: C (registers, converted to fp16) x h_in^T (LDS)
    f32x16 accy[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int k = 0; k < KS; ++k) {
        const f16x8 cf = bf16x8_to_f16x8(cfr[k], c_scale);
#pragma unroll
        for (int pt = 0; pt < 2; ++pt) {
            const f16x8 hf = __builtin_bit_cast(
                f16x8, *reinterpret_cast<const u32x4 *>(sm.h + (32 * pt + l32) * H_STRIDE + 8 * k + 4 * hl));
            accy[pt] = mfma32_f16(cf, hf, accy[pt]);
        }
    }
    __syncthreads();  // tables and red[] complete
    wmax = fmaxf(fmaxf(sm.red[0][0], sm.red[1][0]), fmaxf(sm.red[2][0], sm.red[3][0]));
    emax = fmaxf(fmaxf(sm.red[0][1], sm.red[1][1]), fmaxf(sm.red[2][1], sm.red[3][1]));
    // |2^-xe M| <= |G| * max(dts 2^-xe) * (decay <= 1, or the chunk's total
    // growth when A > 0) + |D| max(2^-xe) on the diagonal, with
    // |G| = |C_i . B_j| <= N max|B| max|C| < N 2^(15-sb) 2^(15-sc)
    const int sb = p.bexp[(int64_t)c * p.G + g];
    const float gbound = ldexpf((float)N, 30 - sb - sc);
    const float dgrow = fast_exp2(fmaxf(0.f, sm.cs2[kChunk - 1] - sm.cs2[0]));
    const int smx = f16_scale_exponent(gbound * wmax * dgrow + fabsf(dh) * emax);
    const float m_scale = ldexpf(1.0f, smx);

    // undo the C and h_in scalings, decay row i by exp2(cs2_i), move to the M scale
#pragma unroll
    for (int pt = 0; pt < 2; ++pt) {
        const float f = ldexpf(1.0f, smx - (sc + sm.hexp[32 * pt + l32]));
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const float4 d4 = *reinterpret_cast<const float4 *>(sm.ei + 32 * rb + 8 * a + 4 * hl);
            accy[pt][4 * a + 0] *= f * d4.x;
            accy[pt][4 * a + 1] *= f * d4.y;
            accy[pt][4 * a + 2] *= f * d4.z;
            accy[pt][4 * a + 3] *= f * d4.w;
        }
    }

    // ---- diagonal block: (2^smx M 2^-xe) (2^xe x), M from the C.B^T tiles
    const int i_a = 32 * rb + l32;  // this lane's row in the A layout
    const float cs_i = sm.cs2[i_a];
    const float u = fast_exp2(cs_i - sm.cs2[32 * rb]) * m_scale;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t <= rb) {
            const f32x16 gv = gt[t & 1];
            if (t + 2 <= rb) gt[t & 1] = load_tile(cbt + (t + 2) * 1024);
            float mv[16];
            if (t < rb) {
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const float4 v4 = *reinterpret_cast<const float4 *>(sm.v + rb * kChunk + 32 * t + 8 * a + 4 * hl);
                    mv[4 * a + 0] = gv[4 * a + 0] * (v4.x * u);
                    mv[4 * a + 1] = gv[4 * a + 1] * (v4.y * u);
                    mv[4 * a + 2] = gv[4 * a + 2] * (v4.z * u);
                    mv[4 * a + 3] = gv[4 * a + 3] * (v4.w * u);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int j = 32 * t + 8 * (e >> 2) + 4 * hl + (e & 3);
                    float val = gv[e] * fast_exp2(cs_i - sm.cs2[j]) * sm.dts[j];
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
                const uint2 *row = reinterpret_cast<const uint2 *>(sm.xt + (32 * pt + l32) * XT_STRIDE + 16 * t + 2 * hl);
                const uint2 xa = row[0], xb = row[2], xc = row[4], xd = row[6];
                const f16x8 x0 = __builtin_bit_cast(f16x8, u32x4{xa.x, xa.y, xb.x, xb.y});
                const f16x8 x1 = __builtin_bit_cast(f16x8, u32x4{xc.x, xc.y, xd.x, xd.y});
                accy[pt] = mfma32_f16(mf0, x0, accy[pt]);
                accy[pt] = mfma32_f16(mf1, x1, accy[pt]);
            }
        }
    }

    // ---- back to unit scale, store bf16
    const float inv = ldexpf(1.0f, -smx);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const int i = 32 * rb + 8 * (e >> 2) + 4 * hl + (e & 3);
        if (i < len) {
            uint16_t *dst = p.y + ((t0 + i) * p.H + h) * kHeadDim + l32;
            dst[0] = float_to_bf16_bits(accy[0][e] * inv);
            dst[32] = float_to_bf16_bits(accy[1][e] * inv);
        }
    }
}

template <int N>
static hipError_t launch_n(const Params &p, hipStream_t s) {
    const int64_t slots = (p.nchunks_max + 7) / 8 * p.H;
    hipLaunchKernelGGL(ssd_chunk_scan_kernel<N>, dim3((unsigned)(slots * 8)), dim3(kThreads), 0, s, p);
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
