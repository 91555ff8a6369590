// Step 0 + step 1 of the scan: the chunk table and the per-chunk cumulative
// decay ("chunk_cumsum"), plus the per-(chunk, group) products that do not
// depend on the head: C.B^T and the power-of-two exponents of B and C.
//
// Chunk table: sequence b owns ceil(len_b / 256) chunks (none when empty);
// chunk c of the call is found from the exclusive prefix sum of those counts,
// so no chunk ever straddles two sequences (the state resets at every
// query_start_loc boundary: "mamba2_ssd_scan", section "Per-token
// recurrence").  Every workgroup computes the prefix itself, so no separate
// launch is needed; workgroup (0, 0) also publishes it (chunk_off, nchunks)
// for the state-passing step.
//
// Cumulative decay (blockIdx.y == 0): for each head h and token j of the chunk,
//   dts_j = softplus(dt[t,h] + dt_bias[h])   (or dt + dt_bias without softplus)
//   cs2_j = log2(e) * sum_{k <= j} A[h] * dts_k
// ("mamba2_ssd_scan", "Per-token recurrence": dA = exp(A * dts); the segment
// sums of "Mamba chunk scan with segsum", description).  Past the chunk end,
// dts = 0 and cs2 stays at its last value, so cs2[255] is the chunk's total.
// One thread per token; 16 heads at a time are scanned across the workgroup.
//
// Per group (blockIdx.y == 1 + g):
//   G^T[j][i] = sum_n B[t0+j,g,n] C[t0+i,g,n] for the causal tiles (j <= i
//   blockwise), the "attention-like" intra-chunk scores of "Mamba chunk scan
//   with segsum" (description) before decay.  They are shared by every head
//   of the group, so they are formed once here (bf16 MFMA on the exact bf16
//   inputs, fp32 accumulate) and stored in MFMA accumulator order, so the
//   chunk-scan step reads each lane's 16 values as one 64-byte run.
//   Eight wavefronts, one 32-row block (of i) each; the two wavefronts that
//   share a SIMD own row blocks k and 7-k, so each SIMD forms 9 of the 36
//   lower-triangular 32x32 tiles.  B and C stream through LDS 32 dstate
//   columns at a time, three slices in flight.  The tiles are stored as fp16
//   under one power-of-two exponent per (chunk, group) that puts their
//   maximum magnitude in [2^14, 2^15).
//
// Per group (blockIdx.y == 1 + G + g): fp16 copies of the chunk's C and B,
//   the operands of the later fp16 products, converted once per group rather
//   than once per head.  Each is scaled by the power of two that puts its
//   maximum magnitude in [2^14, 2^15) (bf16 -> fp16 is then exact but for
//   values 2^24 below the maximum), rows past the chunk end are zero, C keeps
//   its [token][n] layout and B is transposed to [n][token] so that a
//   contraction over tokens reads 8 consecutive tokens as one 16-byte load.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kPrepThreads = 512;
constexpr int kHeadBlock = 16;
constexpr int R_STRIDE = 20;  // dwords per staged row of 32 bf16 + pad
}  // namespace

// max of the bf16 magnitudes (as bits) of 8 values
__device__ __forceinline__ uint32_t max_mag8(const u32x4 v) {
    uint32_t m = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) m = max(m, max(v[k] & 0x7FFFu, (v[k] >> 16) & 0x7FFFu));
    return m;
}

// exponent s putting a bf16 magnitude (as bits) in [2^14, 2^15) after scaling
// by 2^s (0 for a zero maximum): the exponent field sits in bits 7..14
__device__ __forceinline__ int bf16_scale_exponent(uint32_t mm) {
    return mm == 0 ? 0 : 14 - ((int)(mm >> 7) - 127);
}

template <int N>
__device__ void convert_group(const Params &p, int c, int g, int64_t t0, int len, uint32_t (&s_umax)[8][2]) {
    constexpr int CV = kChunk * N / 8 / kPrepThreads;  // 16-byte vectors of C per thread
    constexpr int NB = (kChunk / 8) * (N / 8);           // 8 tokens x 8 n blocks of B
    constexpr int BB = (NB + kPrepThreads - 1) / kPrepThreads;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int64_t rstride = (int64_t)p.G * N;  // elements between consecutive tokens
    const uint16_t *Cg = p.C + (t0 * p.G + g) * N;
    const uint16_t *Bg = p.B + (t0 * p.G + g) * N;

    u32x4 cv[CV];
    u32x4 bv[BB][8];
    uint32_t cm = 0, bm = 0;
#pragma unroll
    for (int it = 0; it < CV; ++it) {
        const int v = tid + it * kPrepThreads;
        const int j = v / (N / 8), q = v % (N / 8);
        cv[it] = j < len ? *reinterpret_cast<const u32x4 *>(Cg + j * rstride + 8 * q) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int it = 0; it < BB; ++it) {
        const int b = tid + it * kPrepThreads;
        const int tb = b / (N / 8), q = b % (N / 8);
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int j = 8 * tb + r;
            bv[it][r] = (b < NB && j < len) ? *reinterpret_cast<const u32x4 *>(Bg + j * rstride + 8 * q)
                                            : u32x4{0u, 0u, 0u, 0u};
        }
    }
#pragma unroll
    for (int it = 0; it < CV; ++it) cm = max(cm, max_mag8(cv[it]));
#pragma unroll
    for (int it = 0; it < BB; ++it)
#pragma unroll
        for (int r = 0; r < 8; ++r) bm = max(bm, max_mag8(bv[it][r]));
    bm = wave_max_u32(bm);
    cm = wave_max_u32(cm);
    if (lane == 0) { s_umax[wave][0] = bm; s_umax[wave][1] = cm; }
    __syncthreads();
    uint32_t bmm = 0, cmm = 0;
#pragma unroll
    for (int w = 0; w < 8; ++w) { bmm = max(bmm, s_umax[w][0]); cmm = max(cmm, s_umax[w][1]); }
    const int sb = bf16_scale_exponent(bmm), sc = bf16_scale_exponent(cmm);
    if (tid == 0) {
        p.bexp[(int64_t)c * p.G + g] = sb;
        p.cexp[(int64_t)c * p.G + g] = sc;
    }
    const float bs = ldexpf(1.0f, sb), cs = ldexpf(1.0f, sc);

    // C: same layout, 8 values per 16-byte vector
    uint16_t *cdst = p.cf16 + ((int64_t)c * p.G + g) * kChunk * N;
#pragma unroll
    for (int it = 0; it < CV; ++it) {
        const int v = tid + it * kPrepThreads;
        u32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = pack_f16x2(__uint_as_float(cv[it][k] << 16) * cs, __uint_as_float(cv[it][k] & 0xFFFF0000u) * cs);
        *reinterpret_cast<u32x4 *>(cdst + (int64_t)v * 8) = o;
    }
    // B^T: the 8x8 block (tokens 8tb.., n 8q..) transposed in registers;
    // dword k of row n holds tokens 2k and 2k+1
    uint16_t *bdst = p.bt16 + ((int64_t)c * p.G + g) * N * kChunk;
#pragma unroll
    for (int it = 0; it < BB; ++it) {
        const int b = tid + it * kPrepThreads;
        if (b < NB) {
            const int tb = b / (N / 8), q = b % (N / 8);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                u32x4 o;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t w0 = bv[it][2 * k][e >> 1], w1 = bv[it][2 * k + 1][e >> 1];
                    const float f0 = __uint_as_float((e & 1) ? (w0 & 0xFFFF0000u) : (w0 << 16));
                    const float f1 = __uint_as_float((e & 1) ? (w1 & 0xFFFF0000u) : (w1 << 16));
                    o[k] = pack_f16x2(f0 * bs, f1 * bs);
                }
                *reinterpret_cast<u32x4 *>(bdst + (int64_t)(8 * q + e) * kChunk + 8 * tb) = o;
            }
        }
    }
}

template <int N>
__global__ __launch_bounds__(kPrepThreads) void ssd_prep_kernel(Params p) {
    constexpr int KS = N / 32;
    const int c = blockIdx.x;
    const int job = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ int s_wtot[8];
    __shared__ int s_loc[2];
    __shared__ float s_hsum[8][kHeadBlock];
    __shared__ uint32_t s_umax[8][2];
    __shared__ float s_gmax[8];
    __shared__ __attribute__((aligned(16))) uint32_t s_b[kChunk * R_STRIDE];
    __shared__ __attribute__((aligned(16))) uint32_t s_c[kChunk * R_STRIDE];

    // ---- locate chunk c: exclusive prefix of per-sequence chunk counts
    if (tid == 0) { s_loc[0] = -1; s_loc[1] = 0; }
    int carry = 0;
    for (int base = 0; base < p.batch; base += kPrepThreads) {
        const int b = base + tid;
        int n = 0;
        if (b < p.batch) {
            const int len = p.qsl[b + 1] - p.qsl[b];
            n = len > 0 ? (len + kChunk - 1) / kChunk : 0;
        }
        const int wincl = wave_incl_scan(n);
        __syncthreads();  // protects s_wtot from the previous round
        if (lane == 63) s_wtot[wave] = wincl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < 8; ++w) {
            if (w < wave) before += s_wtot[w];
            total += s_wtot[w];
        }
        const int excl = carry + before + wincl - n;
        if (b < p.batch) {
            if (c >= excl && c < excl + n) { s_loc[0] = b; s_loc[1] = c - excl; }
            if (c == 0 && job == 0) p.chunk_off[b] = excl;
        }
        carry += total;
    }
    if (c == 0 && job == 0 && tid == 0) {
        p.chunk_off[p.batch] = carry;
        p.meta[0] = carry;
        p.meta[1] = 0; p.meta[2] = 0; p.meta[3] = 0;
    }
    __syncthreads();
    const int b = s_loc[0];
    if (b < 0) {
        if (tid == 0 && job == 0) p.desc[c] = make_int4(-1, 0, 0, 0);
        return;
    }
    const int64_t t0 = (int64_t)p.qsl[b] + (int64_t)s_loc[1] * kChunk;
    const int len = (int)min((int64_t)kChunk, (int64_t)p.qsl[b + 1] - t0);

    if (job == 0) {
        if (tid == 0) p.desc[c] = make_int4(b, (int)t0, len, 0);
        // ---- dts and cs2: thread = token (threads past 255 hold zeros), 16 heads at a time
        const int j = tid;
        const bool valid = j < len;
        for (int hb = 0; hb < p.H; hb += kHeadBlock) {
            float d[kHeadBlock], a[kHeadBlock];
#pragma unroll
            for (int k = 0; k < kHeadBlock; ++k) {
                const int h = hb + k;
                float ds = 0.0f;
                if (valid && h < p.H) {
                    const float v = p.dt[(t0 + j) * p.H + h] + (p.dt_bias ? p.dt_bias[h] : 0.0f);
                    ds = p.dt_softplus ? softplus_f(v) : v;
                }
                d[k] = ds;
                a[k] = h < p.H ? p.A[h] * ds : 0.0f;
            }
            // inclusive scan over the tokens, per head
#pragma unroll
            for (int k = 0; k < kHeadBlock; ++k) a[k] = wave_incl_scan(a[k]);
            __syncthreads();  // s_hsum free from the previous head block
            if (lane == 63) {
#pragma unroll
                for (int k = 0; k < kHeadBlock; ++k) s_hsum[wave][k] = a[k];
            }
            __syncthreads();
            if (j < kChunk) {
#pragma unroll
                for (int k = 0; k < kHeadBlock; ++k) {
                    float off = 0.0f;
                    for (int w = 0; w < wave; ++w) off += s_hsum[w][k];
                    const int h = hb + k;
                    if (h < p.H) {
                        const int64_t row = ((int64_t)c * p.H + h) * kChunk + j;
                        p.dts[row] = d[k];
                        p.cs2[row] = (off + a[k]) * kLog2e;
                    }
                }
            }
        }
        return;
    }

    if (job > p.G) {
        convert_group<N>(p, c, job - 1 - p.G, t0, len, s_umax);
        return;
    }

    // ---- group g: C.B^T tiles
    const int g = job - 1;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    const int rb = (wv >> 2) ? 7 - (wv & 3) : (wv & 3);
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    constexpr int PD = KS < 3 ? KS : 3;  // slices in flight
    u32x4 rbv[PD][2], rcv[PD][2];
    auto load_slice = [&](int ks, int d) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int j = (tid + it * kPrepThreads) >> 2;
            const int v = tid & 3;
            rbv[d][it] = rcv[d][it] = u32x4{0u, 0u, 0u, 0u};
            if (j < len) {
                const int64_t off = ((t0 + j) * p.G + g) * N + ks * 32 + v * 8;
                rbv[d][it] = *reinterpret_cast<const u32x4 *>(p.B + off);
                rcv[d][it] = *reinterpret_cast<const u32x4 *>(p.C + off);
            }
        }
    };
    f32x16 accg[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) accg[t] = f32x16{};

#pragma unroll
    for (int d = 0; d < PD; ++d) load_slice(d, d);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        __syncthreads();  // previous slice consumed
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int j = (tid + it * kPrepThreads) >> 2;
            const int v = tid & 3;
            *reinterpret_cast<u32x4 *>(s_b + j * R_STRIDE + v * 4) = rbv[ks % PD][it];
            *reinterpret_cast<u32x4 *>(s_c + j * R_STRIDE + v * 4) = rcv[ks % PD][it];
        }
        if (ks + PD < KS) load_slice(ks + PD, ks % PD);  // in flight during the next slices' MFMAs
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 cb = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(s_c + (32 * rb + l32) * R_STRIDE + 8 * kk + 4 * hl));
#pragma unroll
            for (int t = 0; t < 8; ++t) {
                if (t <= rb) {
                    const bf16x8 bb = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const u32x4 *>(s_b + (32 * t + l32) * R_STRIDE + 8 * kk + 4 * hl));
                    accg[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb, cb, accg[t], 0, 0, 0);
                }
            }
        }
    }
    // one power-of-two scale for all tiles of the chunk and group
    float gm = 0.f;
#pragma unroll
    for (int t = 0; t < 8; ++t)
        if (t <= rb)
#pragma unroll
            for (int e = 0; e < 16; ++e) gm = fmaxf(gm, fabsf(accg[t][e]));
    gm = wave_max(gm);
    if (lane == 0) s_gmax[wave] = gm;
    __syncthreads();
    float gmax = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) gmax = fmaxf(gmax, s_gmax[w]);
    const int sg = f16_scale_exponent(gmax);
    if (tid == 0) p.gexp[(int64_t)c * p.G + g] = sg;
    const float gs = ldexpf(1.0f, sg);
    // tiles in accumulator order: tile rb(rb+1)/2 + t, 64 lanes x 16 fp16
    uint16_t *dst = p.cbt + ((int64_t)c * p.G + g) * 36 * 1024;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        if (t <= rb) {
            u32x4 *o = reinterpret_cast<u32x4 *>(dst + (rb * (rb + 1) / 2 + t) * 1024 + lane * 16);
#pragma unroll
            for (int q = 0; q < 2; ++q)
                o[q] = u32x4{pack_f16x2(accg[t][8 * q] * gs, accg[t][8 * q + 1] * gs),
                             pack_f16x2(accg[t][8 * q + 2] * gs, accg[t][8 * q + 3] * gs),
                             pack_f16x2(accg[t][8 * q + 4] * gs, accg[t][8 * q + 5] * gs),
                             pack_f16x2(accg[t][8 * q + 6] * gs, accg[t][8 * q + 7] * gs)};
        }
    }
}

hipError_t launch_prep(const Params &p, hipStream_t s) {
    const dim3 grid((unsigned)p.nchunks_max, (unsigned)(1 + 2 * p.G));
    switch (p.N) {
    case 64: hipLaunchKernelGGL(ssd_prep_kernel<64>, grid, dim3(kPrepThreads), 0, s, p); break;
    case 128: hipLaunchKernelGGL(ssd_prep_kernel<128>, grid, dim3(kPrepThreads), 0, s, p); break;
    case 256: hipLaunchKernelGGL(ssd_prep_kernel<256>, grid, dim3(kPrepThreads), 0, s, p); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace ssd
