// Step 2 of the scan: each chunk's own contribution to the state ("chunk_state").
//
// For chunk c (tokens t0 .. t0+len-1 of one sequence) and head h with group g:
//   S[p][n] = sum_j exp(cs_last - cs_j) * dts_j * x[t0+j, h, p] * B[t0+j, g, n]
// i.e. the state the chunk would leave behind if it started from zero; this is
// the per-token recurrence of "mamba2_ssd_scan" ("Per-token recurrence")
// unrolled over one chunk, the inter-chunk part of the chunked scan of
// "Mamba chunk scan with segsum" (description).
//
// It is a (P x len) . (len x N) contraction over the chunk's tokens, run on
// MFMA (v_mfma_f32_16x16x32_f16, fp32 accumulate).  Precision: the weighted
// operand w_j * x is not exact in 16 bits; fp16 (11-bit significand) keeps the
// final-state error near 2e-4 where bf16 (8 bits) would give about 1.6e-3.
// Both operands are first scaled by exact powers of two (per chunk and head
// for w*x, per chunk and group for B, from the prep step) so their maxima sit
// in [2^14, 2^15), far from fp16 overflow; the accumulator is scaled back
// exactly.
//
// Workgroup = one (chunk, head), 4 wavefronts.  The chunk's weighted x is
// staged once in LDS transposed to [p][token] (fp16), B is staged 32 tokens at
// a time transposed to [n][token]; wavefront w owns n-tiles
// [w*N/64, (w+1)*N/64) for all four 16-row p-tiles.
#include "ssd_common.hpp"

namespace ssd {

template <int N>
__global__ __launch_bounds__(256) void ssd_chunk_state_kernel(Params p) {
    constexpr int NT = N / 16;     // n-tiles
    constexpr int NTW = NT / 4;    // n-tiles per wavefront
    constexpr int XT_STRIDE = 132; // dwords per XT row: 128 (256 tokens as f16 pairs) + pad
    constexpr int BT_STRIDE = 20;  // dwords per BT row: 16 (32 tokens) + pad

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

    __shared__ float s_w[kChunk];
    __shared__ float s_red[4];
    __shared__ uint32_t s_xt[kHeadDim * XT_STRIDE];
    __shared__ uint32_t s_bt[N * BT_STRIDE];

    // ---- weights w_j = exp2(cs2_last - cs2_j) * dts_j  (0 past the chunk end)
    const int64_t crow = ((int64_t)c * p.H + h) * kChunk;
    {
        const float last = p.cs2[crow + kChunk - 1];
        s_w[tid] = exp2f(last - p.cs2[crow + tid]) * p.dts[crow + tid];
    }
    __syncthreads();

    // ---- weighted x: thread = (token pair, half of p); find the max magnitude
    const int pair = tid & 127;
    const int ph = tid >> 7;
    float xv[2][32];
    float mloc = 0.0f;
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        const int j = pair * 2 + e;
        const float w = s_w[j];
        if (j < len) {
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                p.x + ((t0 + j) * p.H + h) * kHeadDim + ph * 32);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const u32x4 qv = src[v];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xv[e][v * 8 + 2 * k] = w * bf16_bits_to_float(qv[k] & 0xFFFFu);
                    xv[e][v * 8 + 2 * k + 1] = w * bf16_bits_to_float(qv[k] >> 16);
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 32; ++k) xv[e][k] = 0.0f;
        }
#pragma unroll
        for (int k = 0; k < 32; ++k) mloc = fmaxf(mloc, fabsf(xv[e][k]));
    }
    mloc = wave_max(mloc);
    if (lane == 0) s_red[wave] = mloc;
    __syncthreads();
    const float mx = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const int sx = mx > 0.0f ? 14 - float_exponent(mx) : 0;
    const int sb = p.bexp[(int64_t)c * p.G + g];
#pragma unroll
    for (int k = 0; k < 32; ++k) {
        s_xt[(ph * 32 + k) * XT_STRIDE + pair] =
            pack_f16x2(ldexpf(xv[0][k], sx), ldexpf(xv[1][k], sx));
    }

    f32x4 acc[4][NTW];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NTW; ++b) acc[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- K loop over the chunk's tokens, 32 at a time
    const int nslices = (len + 31) / 32;
    for (int ks = 0; ks < nslices; ++ks) {
        __syncthreads();  // previous slice fully consumed (and s_xt written)
        // stage B^T[n][token] for tokens 32ks .. 32ks+31, scaled, as f16 pairs
        for (int n = tid; n < N; n += 256) {
            float bv[32];
#pragma unroll
            for (int jj = 0; jj < 32; ++jj) {
                const int j = ks * 32 + jj;
                bv[jj] = j < len ? ldexpf(bf16_bits_to_float(p.B[((t0 + j) * p.G + g) * N + n]), sb)
                                 : 0.0f;
            }
            u32x4 *dst = reinterpret_cast<u32x4 *>(s_bt + n * BT_STRIDE);
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                dst[v] = u32x4{pack_f16x2(bv[8 * v + 0], bv[8 * v + 1]),
                               pack_f16x2(bv[8 * v + 2], bv[8 * v + 3]),
                               pack_f16x2(bv[8 * v + 4], bv[8 * v + 5]),
                               pack_f16x2(bv[8 * v + 6], bv[8 * v + 7])};
            }
        }
        __syncthreads();
        f16x8 af[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                s_xt + (pt * 16 + lc) * XT_STRIDE + ks * 16 + q * 4);
            af[pt] = __builtin_bit_cast(f16x8, v);
        }
#pragma unroll
        for (int b = 0; b < NTW; ++b) {
            const int nt = wave * NTW + b;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(
                s_bt + (nt * 16 + lc) * BT_STRIDE + q * 4);
            const f16x8 bf = __builtin_bit_cast(f16x8, v);
#pragma unroll
            for (int pt = 0; pt < 4; ++pt) acc[pt][b] = mfma_f16(af[pt], bf, acc[pt][b]);
        }
    }

    // ---- store S[c][h][p][n] (fp32), undoing the two scalings exactly
    const int sh = -(sx + sb);
    float *dst = p.states + ((int64_t)c * p.H + h) * kHeadDim * N;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int b = 0; b < NTW; ++b) {
            const int n = (wave * NTW + b) * 16 + lc;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int pp = pt * 16 + q * 4 + t;
                dst[pp * N + n] = ldexpf(acc[pt][b][t], sh);
            }
        }
}

hipError_t launch_chunk_state(const Params &p, hipStream_t s) {
    dim3 grid((unsigned)p.nchunks_max, (unsigned)p.H);
    switch (p.N) {
    case 64: hipLaunchKernelGGL(ssd_chunk_state_kernel<64>, grid, dim3(256), 0, s, p); break;
    case 128: hipLaunchKernelGGL(ssd_chunk_state_kernel<128>, grid, dim3(256), 0, s, p); break;
    case 256: hipLaunchKernelGGL(ssd_chunk_state_kernel<256>, grid, dim3(256), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
