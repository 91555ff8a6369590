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
// Precision: all three products run on v_mfma_f32_16x16x32_f16 (fp32
// accumulate).  B, C and x are bf16 inputs and convert to fp16 exactly after
// a power-of-two scaling (per chunk and group for B and C, per chunk and head
// for x) that keeps them inside fp16's range; G is then exact up to fp32
// summation.  M and h_in are rounded to fp16 (11-bit significand) with their
// own power-of-two scales (per 16-row block of M, per row p of h_in).  With
// bf16 (8 bits) for M or h_in the rounding error, which scales with the
// typical size of y rather than with each y, would approach the tolerance on
// y wherever y is near zero.
//
// Workgroup = one (chunk, head), 8 wavefronts.  Wavefront w owns the 16-row
// blocks w and 15-w, which balances the causal triangle (17 of the 136
// lower-triangular 16x16 tiles each).
//   * G is formed transposed (rows j, columns i) over n, so the accumulator
//     layout of a G tile (4 consecutive j per lane at one i) is directly the
//     A-operand layout of M for the next product, with the 32 j of a K-step
//     ordered {4q..4q+3, 16+4q..16+4q+3}; x is read from LDS in that order.
//   * The C fragment of a K-step serves both G^T (as B operand) and the
//     off-diagonal product (as A operand).
// B, C and h_in are staged 32 n at a time; x is staged once, transposed to
// [p][token].
#include "ssd_common.hpp"

namespace ssd {

template <int N>
__global__ __launch_bounds__(512) void ssd_chunk_scan_kernel(Params p) {
    constexpr int KS = N / 32;
    constexpr int XT_STRIDE = 130;  // dwords per x^T row: 128 token pairs + pad (8-byte rows)
    constexpr int R_STRIDE = 20;    // dwords per staged row of 32 fp16 + pad

    const int c = blockIdx.x;
    const int h = blockIdx.y;
    if (c >= p.meta[0]) return;
    const int4 dsc = p.desc[c];
    const int64_t t0 = dsc.y;
    const int len = dsc.z;
    const int g = h / (p.H / p.G);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int lc = lane & 15;
    const int q = lane >> 4;

    __shared__ float s_cs2[kChunk];
    __shared__ float s_dts[kChunk];
    __shared__ int s_hexp[kHeadDim];
    __shared__ uint32_t s_red[8];
    __shared__ uint32_t s_xt[kHeadDim * XT_STRIDE];
    __shared__ uint32_t s_b[kChunk * R_STRIDE];
    __shared__ uint32_t s_c[kChunk * R_STRIDE];
    __shared__ uint32_t s_h[kHeadDim * R_STRIDE];

    const int64_t crow = ((int64_t)c * p.H + h) * kChunk;
    if (tid < kChunk) {
        s_cs2[tid] = p.cs2[crow + tid];
        s_dts[tid] = p.dts[crow + tid];
    } else if (tid < kChunk + kHeadDim) {
        s_hexp[tid - kChunk] = p.hexp[((int64_t)c * p.H + h) * kHeadDim + (tid - kChunk)];
    }
    const int sb = p.bexp[(int64_t)c * p.G + g];
    const int sc = p.cexp[(int64_t)c * p.G + g];

    // x^T[p][token] as scaled fp16 pairs; thread = (token pair, quarter of p)
    int sx;
    {
        const int pair = tid & 127;
        const int pq = tid >> 7;
        u32x4 v[2][2];
        uint32_t mloc = 0;
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
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = v[e][a][k] & 0x7FFFu, hi = (v[e][a][k] >> 16) & 0x7FFFu;
                    mloc = mloc > lo ? mloc : lo;
                    mloc = mloc > hi ? mloc : hi;
                }
        }
        mloc = wave_max_u32(mloc);
        if (lane == 0) s_red[wave] = mloc;
        __syncthreads();
        uint32_t mm = s_red[0];
#pragma unroll
        for (int w = 1; w < 8; ++w) mm = mm > s_red[w] ? mm : s_red[w];
        sx = mm == 0 ? 0 : 14 - ((int)(mm >> 7) - 127);
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const uint32_t a = v[0][k >> 3][(k >> 1) & 3];
            const uint32_t b = v[1][k >> 3][(k >> 1) & 3];
            const float lo = bf16_bits_to_float((k & 1) ? (a >> 16) : (a & 0xFFFFu));
            const float hi = bf16_bits_to_float((k & 1) ? (b >> 16) : (b & 0xFFFFu));
            s_xt[(pq * 16 + k) * XT_STRIDE + pair] = pack_f16x2(ldexpf(lo, sx), ldexpf(hi, sx));
        }
    }

    // tile bookkeeping: 9 K-pairs of two 16-column j-blocks
    const int rb0 = wave, rb1 = 15 - wave;
    const int P0 = (wave + 2) >> 1;  // pairs for row block rb0

    f32x4 accg[18];
    f32x4 accy[2][4];
#pragma unroll
    for (int s = 0; s < 18; ++s) accg[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int r = 0; r < 2; ++r)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) accy[r][pt] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t *hin_head = p.hin + ((int64_t)c * p.H + h) * kHeadDim * N;

    for (int ks = 0; ks < KS; ++ks) {
        __syncthreads();
        // stage B and C rows (all 256 tokens, scaled fp16) and h_in rows (64 p)
        // for n in [32ks, 32ks+32)
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int idx = tid + it * 512;
            const int j = idx >> 2;
            const int v = idx & 3;
            u32x4 bv = u32x4{0u, 0u, 0u, 0u}, cv = u32x4{0u, 0u, 0u, 0u};
            if (j < len) {
                const int64_t off = ((t0 + j) * p.G + g) * N + ks * 32 + v * 8;
                const u32x4 braw = *reinterpret_cast<const u32x4 *>(p.B + off);
                const u32x4 craw = *reinterpret_cast<const u32x4 *>(p.C + off);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    bv[k] = pack_f16x2(ldexpf(bf16_bits_to_float(braw[k] & 0xFFFFu), sb),
                                       ldexpf(bf16_bits_to_float(braw[k] >> 16), sb));
                    cv[k] = pack_f16x2(ldexpf(bf16_bits_to_float(craw[k] & 0xFFFFu), sc),
                                       ldexpf(bf16_bits_to_float(craw[k] >> 16), sc));
                }
            }
            *reinterpret_cast<u32x4 *>(s_b + j * R_STRIDE + v * 4) = bv;
            *reinterpret_cast<u32x4 *>(s_c + j * R_STRIDE + v * 4) = cv;
        }
        if (tid < 256) {
            const int pp = tid >> 2;
            const int v = tid & 3;
            *reinterpret_cast<u32x4 *>(s_h + pp * R_STRIDE + v * 4) =
                *reinterpret_cast<const u32x4 *>(hin_head + pp * N + ks * 32 + v * 8);
        }
        __syncthreads();

        const f16x8 cf0 = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
            s_c + (rb0 * 16 + lc) * R_STRIDE + q * 4));
        const f16x8 cf1 = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
            s_c + (rb1 * 16 + lc) * R_STRIDE + q * 4));
#pragma unroll
        for (int s = 0; s < 18; ++s) {
            const int k = s >> 1;
            const bool first = k < P0;
            const int rb = first ? rb0 : rb1;
            const int jb = 2 * (first ? k : k - P0) + (s & 1);
            if (jb <= rb) {
                const f16x8 bfr = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                    s_b + (jb * 16 + lc) * R_STRIDE + q * 4));
                accg[s] = mfma_f16(bfr, first ? cf0 : cf1, accg[s]);
            }
        }
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const f16x8 hf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                s_h + (pt * 16 + lc) * R_STRIDE + q * 4));
            accy[0][pt] = mfma_f16(cf0, hf, accy[0][pt]);
            accy[1][pt] = mfma_f16(cf1, hf, accy[1][pt]);
        }
    }

    // off-diagonal part: undo the C and h_in scalings, scale row i by exp2(cs2_i)
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rb = r ? rb1 : rb0;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float dec = exp2f(s_cs2[rb * 16 + q * 4 + t]);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt)
                accy[r][pt][t] = ldexpf(accy[r][pt][t], -(sc + s_hexp[pt * 16 + lc])) * dec;
        }
    }

    // M = G * decay * dts (masked), in place of the G^T accumulators;
    // track max |M| per owned row block
    float mx0 = 0.0f, mx1 = 0.0f;
#pragma unroll
    for (int s = 0; s < 18; ++s) {
        const int k = s >> 1;
        const bool first = k < P0;
        const int rb = first ? rb0 : rb1;
        const int jb = 2 * (first ? k : k - P0) + (s & 1);
        const int i = rb * 16 + lc;
        const float cs_i = s_cs2[i];
        float m = 0.0f;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int j = jb * 16 + q * 4 + t;
            float val = 0.0f;
            if (j <= i) val = ldexpf(accg[s][t], -(sb + sc)) * exp2f(cs_i - s_cs2[j]) * s_dts[j];
            accg[s][t] = val;
            m = fmaxf(m, fabsf(val));
        }
        if (first) mx0 = fmaxf(mx0, m);
        else mx1 = fmaxf(mx1, m);
    }
    const int sm0 = f16_scale_exponent(wave_max(mx0));
    const int sm1 = f16_scale_exponent(wave_max(mx1));

    // diagonal block: (2^sm M) (2^sx x), accumulated on top of the
    // off-diagonal part brought to the same scale
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            accy[0][pt][t] = ldexpf(accy[0][pt][t], sm0 + sx);
            accy[1][pt][t] = ldexpf(accy[1][pt][t], sm1 + sx);
        }
#pragma unroll
    for (int k = 0; k < 9; ++k) {
        const bool first = k < P0;
        const int m = first ? k : k - P0;
        const int sm = first ? sm0 : sm1;
        const u32x4 mp = u32x4{
            pack_f16x2(ldexpf(accg[2 * k][0], sm), ldexpf(accg[2 * k][1], sm)),
            pack_f16x2(ldexpf(accg[2 * k][2], sm), ldexpf(accg[2 * k][3], sm)),
            pack_f16x2(ldexpf(accg[2 * k + 1][0], sm), ldexpf(accg[2 * k + 1][1], sm)),
            pack_f16x2(ldexpf(accg[2 * k + 1][2], sm), ldexpf(accg[2 * k + 1][3], sm))};
        const f16x8 mf = __builtin_bit_cast(f16x8, mp);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const uint32_t *row = s_xt + (pt * 16 + lc) * XT_STRIDE + m * 16 + q * 2;
            const u32x4 xv = u32x4{row[0], row[1], row[8], row[9]};
            const f16x8 xf = __builtin_bit_cast(f16x8, xv);
            if (first) accy[0][pt] = mfma_f16(mf, xf, accy[0][pt]);
            else accy[1][pt] = mfma_f16(mf, xf, accy[1][pt]);
        }
    }

    // back to unit scale, add D * x, store bf16
    const float dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        const int rb = r ? rb1 : rb0;
        const int sh = -((r ? sm1 : sm0) + sx);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int i = rb * 16 + q * 4 + t;
            if (i < len) {
#pragma unroll
                for (int pt = 0; pt < 4; ++pt) {
                    const int pc = pt * 16 + lc;
                    const uint32_t w2 = s_xt[pc * XT_STRIDE + (i >> 1)];
                    const float xvv = ldexpf(f16_bits_to_float((i & 1) ? (w2 >> 16) : (w2 & 0xFFFFu)), -sx);
                    const float yv = ldexpf(accy[r][pt][t], sh) + dh * xvv;
                    p.y[((t0 + i) * p.H + h) * kHeadDim + pc] = float_to_bf16_bits(yv);
                }
            }
        }
    }
}

hipError_t launch_chunk_scan(const Params &p, hipStream_t s) {
    dim3 grid((unsigned)p.nchunks_max, (unsigned)p.H);
    switch (p.N) {
    case 64: hipLaunchKernelGGL(ssd_chunk_scan_kernel<64>, grid, dim3(512), 0, s, p); break;
    case 128: hipLaunchKernelGGL(ssd_chunk_scan_kernel<128>, grid, dim3(512), 0, s, p); break;
    case 256: hipLaunchKernelGGL(ssd_chunk_scan_kernel<256>, grid, dim3(512), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
