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
// v_mfma_f32_32x32x16_f16 (fp32 accumulate).  Precision: the weighted operand
// w_j * x is not exact in 16 bits; fp16 (11-bit significand) keeps the
// final-state error near 2e-4 where bf16 (8 bits) would give about 1.6e-3.
// Both operands are first scaled by exact powers of two (per chunk and head
// for w*x, per chunk and group for B, from the prep step) so their maxima sit
// in [2^14, 2^15), far from fp16 overflow.  S itself is stored as fp16 under
// one power-of-two exponent per (chunk, head) (the net exponent of all
// scalings, so the reader undoes them exactly); its rounding adds about 3e-4
// relative error to the final states and halves the states traffic.
//
// Work split: one workgroup = one chunk and HW heads of one group (B is
// staged once for all of them), four wavefronts per head.  The weighted x of
// each head is staged once in LDS, transposed to [p][token]; B is staged 32
// tokens at a time, transposed to [n][token] (fp16 pairs of tokens per
// dword), the next slice prefetched into registers.  16-byte LDS chunks of
// rows 16..31 of every 32-row block are swapped pairwise so the 32 rows an
// MFMA operand reads fall on distinct banks.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int XT_STRIDE = 132;  // dwords per x^T row: 128 token pairs + pad
constexpr int BT_STRIDE = 20;   // dwords per B^T row: 16 token pairs + pad

// dword index of 16-byte chunk `q4` (in dwords, a multiple of 4) of row r
__device__ __forceinline__ int swz(int r, int q4) { return q4 ^ (((r >> 4) & 1) << 2); }
}  // namespace

template <int N, int HW>
__global__ __launch_bounds__(256 * HW) void ssd_chunk_state_kernel(Params p) {
    constexpr int kThreads = 256 * HW;
    constexpr int NT = N / 32;      // 32-wide n tiles
    constexpr int TPW = NT / 2;     // n tiles per wavefront (two p tiles x NT n tiles over 4 waves)
    constexpr int ITEMS = 16 * (N / 8);  // (token pair, 8-wide n chunk) items per B slice

    __shared__ float s_w[HW][kChunk];
    __shared__ float s_red[HW][4];
    __shared__ __attribute__((aligned(16))) uint32_t s_xt[HW][kHeadDim * XT_STRIDE];
    __shared__ __attribute__((aligned(16))) uint32_t s_bt[N * BT_STRIDE];

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
    const int sb = p.bexp[(int64_t)c * p.G + g];
    const float b_scale = ldexpf(1.0f, sb);

    // ---- weights w_j = exp2(cs2_last - cs2_j) * dts_j  (0 past the chunk end)
    for (int e = tid; e < HW * kChunk; e += kThreads) {
        const int hh = e >> 8, j = e & 255;
        const int64_t crow = ((int64_t)c * p.H + h_first + hh) * kChunk;
        s_w[hh][j] = exp2f(p.cs2[crow + kChunk - 1] - p.cs2[crow + j]) * p.dts[crow + j];
    }
    __syncthreads();

    // ---- weighted x: thread = (head, half of p, token pair); max magnitude per head
    const int xh = tid >> 8;
    const int pair = tid & 127;
    const int ph = (tid >> 7) & 1;
    {
        float xv[2][32];
        float mloc = 0.0f;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = pair * 2 + e;
            const float w = s_w[xh][j];
            if (j < len) {
                const u32x4 *src = reinterpret_cast<const u32x4 *>(
                    p.x + ((t0 + j) * p.H + h_first + xh) * kHeadDim + ph * 32);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const u32x4 qv = src[v];
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        xv[e][v * 8 + 2 * k] = w * __uint_as_float(qv[k] << 16);
                        xv[e][v * 8 + 2 * k + 1] = w * __uint_as_float(qv[k] & 0xFFFF0000u);
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
        if (lane == 0) s_red[xh][(wave & 3)] = mloc;
        __syncthreads();
        const float mx = fmaxf(fmaxf(s_red[xh][0], s_red[xh][1]), fmaxf(s_red[xh][2], s_red[xh][3]));
        const float xs = ldexpf(1.0f, f16_scale_exponent(mx));
#pragma unroll
        for (int k = 0; k < 32; ++k) {
            const int row = ph * 32 + k;
            // token pair `pair` sits in 16-byte chunk pair/4 of the row
            s_xt[xh][row * XT_STRIDE + swz(row, (pair >> 2) << 2) + (pair & 3)] =
                pack_f16x2(xv[0][k] * xs, xv[1][k] * xs);
        }
    }
    const float mx_own = fmaxf(fmaxf(s_red[wave >> 2][0], s_red[wave >> 2][1]),
                               fmaxf(s_red[wave >> 2][2], s_red[wave >> 2][3]));
    const int sx_own = f16_scale_exponent(mx_own);

    // ---- B^T staging: item = (8-wide n chunk, token pair); 4 lanes cover 4 n chunks
    auto load_b = [&](int ks, u32x4 (&r)[2][(ITEMS + kThreads - 1) / kThreads]) {
#pragma unroll
        for (int it = 0; it < (ITEMS + kThreads - 1) / kThreads; ++it) {
            const int item = tid + it * kThreads;
            const int tp = (item >> 2) & 15;
            const int nc = ((item >> 6) << 2) | (item & 3);
            r[0][it] = r[1][it] = u32x4{0u, 0u, 0u, 0u};
            if (item < ITEMS) {
                const int j = ks * 32 + 2 * tp;
                if (j < len)
                    r[0][it] = *reinterpret_cast<const u32x4 *>(p.B + ((t0 + j) * p.G + g) * N + nc * 8);
                if (j + 1 < len)
                    r[1][it] = *reinterpret_cast<const u32x4 *>(p.B + ((t0 + j + 1) * p.G + g) * N + nc * 8);
            }
        }
    };
    auto store_b = [&](const u32x4 (&r)[2][(ITEMS + kThreads - 1) / kThreads]) {
#pragma unroll
        for (int it = 0; it < (ITEMS + kThreads - 1) / kThreads; ++it) {
            const int item = tid + it * kThreads;
            if (item < ITEMS) {
                const int tp = (item >> 2) & 15;
                const int nc = ((item >> 6) << 2) | (item & 3);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const float a0 = __uint_as_float(r[0][it][k] << 16) * b_scale;
                    const float a1 = __uint_as_float(r[0][it][k] & 0xFFFF0000u) * b_scale;
                    const float c0 = __uint_as_float(r[1][it][k] << 16) * b_scale;
                    const float c1 = __uint_as_float(r[1][it][k] & 0xFFFF0000u) * b_scale;
                    const int n0 = nc * 8 + 2 * k;
                    s_bt[n0 * BT_STRIDE + swz(n0, (tp >> 2) << 2) + (tp & 3)] = pack_f16x2(a0, c0);
                    s_bt[(n0 + 1) * BT_STRIDE + swz(n0 + 1, (tp >> 2) << 2) + (tp & 3)] = pack_f16x2(a1, c1);
                }
            }
        }
    };

    // tiles of this wavefront: p tile pt, n tiles nt0 .. nt0+TPW-1
    const int wl = wave & 3;
    const int pt = (wl * TPW) / NT;
    const int nt0 = (wl * TPW) % NT;
    f32x16 acc[TPW];
#pragma unroll
    for (int u = 0; u < TPW; ++u) acc[u] = f32x16{};

    u32x4 br[2][(ITEMS + kThreads - 1) / kThreads];
    const int nslices = (len + 31) / 32;
    load_b(0, br);
    for (int ks = 0; ks < nslices; ++ks) {
        __syncthreads();  // previous slice consumed (and x^T written)
        store_b(br);
        if (ks + 1 < nslices) load_b(ks + 1, br);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const int arow = pt * 32 + l32;
            const f16x8 af = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                s_xt[wave >> 2] + arow * XT_STRIDE + swz(arow, ks * 16 + kk * 8 + hl * 4)));
#pragma unroll
            for (int u = 0; u < TPW; ++u) {
                const int brow = (nt0 + u) * 32 + l32;
                const f16x8 bf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                    s_bt + brow * BT_STRIDE + swz(brow, kk * 8 + hl * 4)));
                acc[u] = mfma32_f16(af, bf, acc[u]);
            }
        }
    }

    // ---- store S[c][h][p][n] as fp16 with one power-of-two exponent per
    // (chunk, head): the accumulator is 2^(sx+sb) S; rescale it so that
    // max |S| lands in [2^14, 2^15) (relative rounding 2^-11 per element).
    float am = 0.f;
#pragma unroll
    for (int u = 0; u < TPW; ++u)
#pragma unroll
        for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(acc[u][e]));
    am = wave_max(am);
    __syncthreads();  // all s_red reads above are done
    if (lane == 0) s_red[wave >> 2][wave & 3] = am;
    __syncthreads();
    const float amax = fmaxf(fmaxf(s_red[wave >> 2][0], s_red[wave >> 2][1]),
                             fmaxf(s_red[wave >> 2][2], s_red[wave >> 2][3]));
    const int se = f16_scale_exponent(amax);  // stored S = 2^se * acc = 2^(se + sx + sb) S
    const float rescale = ldexpf(1.0f, se);
    const int h_own = h_first + (wave >> 2);
    if ((wave & 3) == 0 && lane == 0) p.sexp[(int64_t)c * p.H + h_own] = se + sx_own + sb;
    uint16_t *dst = p.states + ((int64_t)c * p.H + h_own) * kHeadDim * N;
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
        const int n = (nt0 + u) * 32 + l32;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int pp = pt * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
            dst[pp * N + n] = __builtin_bit_cast(uint16_t, (_Float16)(acc[u][e] * rescale));
        }
    }
}

template <int N>
static hipError_t launch_n(const Params &p, hipStream_t s) {
    const int hw = ((p.H / p.G) % 2 == 0) ? 2 : 1;
    const int64_t slots = (p.nchunks_max + 7) / 8 * (p.H / hw);
    const dim3 grid((unsigned)(slots * 8));
    if (hw == 2) hipLaunchKernelGGL((ssd_chunk_state_kernel<N, 2>), grid, dim3(512), 0, s, p);
    else hipLaunchKernelGGL((ssd_chunk_state_kernel<N, 1>), grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_chunk_state(const Params &p, hipStream_t s) {
    switch (p.N) {
    case 64: return launch_n<64>(p, s);
    case 128: return launch_n<128>(p, s);
    case 256: return launch_n<256>(p, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
