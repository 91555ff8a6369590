// Step 0 of the scan: the chunk table, each chunk's cumulative decay per
// head ("chunk_cumsum"), and the per-(chunk, group) operands that do not
// depend on the head: C.B^T and B^T in MFMA operand order.
//
// Chunk table: sequence b owns ceil(len_b / 256) chunks (none when empty);
// chunk c of the call is found from the exclusive prefix sum of those counts,
// so no chunk ever straddles two sequences (the state resets at every
// query_start_loc boundary: "mamba2_ssd_scan", section "Per-token
// recurrence").  Every workgroup computes the prefix itself, so no separate
// launch is needed; workgroup (0, 0, 0) also publishes it (chunk_off,
// nchunks) for the state chain.  Sequences the short path takes
// (short_max > 0: 0 .. short_max tokens) own no chunks; workgroup (0, 0, 0)
// then also writes the list of the sequences the state chain walks (the
// others) and the list of those of 1 .. recur_max tokens for the
// token-recurrence kernel, with their counts (meta[1], meta[2]).  The grid is
// sized to the host's bound on the chunks that can reach it.  Workgroups
// (c, 0, 0) write the chunk's descriptor {sequence, first token, length}.
//
// Workgroup (c, g, q), q = 0..3, for chunk c and group g:
//   - chunk_cumsum of the group's heads i = q, q + 4, ... (one wavefront per
//     head): dts = softplus(dt + dt_bias) (0 past the chunk end) and
//     cs2 = log2(e) * cumsum(A dts), the segment sums of "Mamba chunk scan
//     with segsum" (description) in base 2;
//   - the C.B^T tiles of row blocks q and 7-q (9 of the 36 lower-triangular
//     32x32 tiles, so the four workgroups of a chunk share the triangle
//     evenly): G^T[j][i] = sum_n B[t0+j,g,n] C[t0+i,g,n] for j <= i blockwise
//     (the diagonal tiles hold zeros where j > i), the "attention-like"
//     intra-chunk scores before decay.  They are shared by every head of the
//     group, so they are formed once here (bf16 MFMA on the exact bf16
//     inputs, fp32 accumulate) and stored in MFMA accumulator order, as fp16
//     under one power-of-two exponent per row-block pair (gexp[c][g][q]) that
//     puts their maximum magnitude in [2^14, 2^15);
//   - B^T as fp16 MFMA A operands for the state chain (bfrag) for the
//     32-column slices ks = q, q + 4, ...: each slice, already staged for the
//     product above, is read back token-contiguous, scaled by the power of
//     two that puts its max |B| in [2^14, 2^15) (bexp) and stored in operand
//     order, 0 past the chunk end.
// B (all 256 rows) and the two row blocks of C stream through LDS 32 dstate
// columns at a time, several slices in flight in registers.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kPrepThreads = 512;
constexpr int kPrepWaves = kPrepThreads / 64;
constexpr int R_STRIDE = 20;  // dwords per staged row of 32 bf16 + pad
}  // namespace

// Tile i (0..8) of row-block pair q: row block q for i <= q (column blocks
// 0..q), else row block 7-q (column blocks 0..7-q).  Wavefront W of the
// workgroup takes tiles W and W+8.
__host__ __device__ constexpr int pair_rb(int q, int i) { return i <= q ? q : 7 - q; }
__host__ __device__ constexpr int pair_t(int q, int i) { return i <= q ? i : i - q - 1; }
__host__ __device__ constexpr int wave_ntiles(int W) { return W == 0 ? 2 : 1; }

// The C.B^T tiles of wavefront W for chunk c, group g, row-block pair q, and
// the B^T operand slices of the pair, PD0 slices in flight in registers.  W
// is a template parameter so that the number of tiles, and with it every
// MFMA, is fixed at compile time.
template <int N, int W, int PD0>
__device__ __forceinline__ void gram_tiles(const Params &p, int c, int g, int q, int64_t t0, int len, uint32_t *s_b,
                                           uint32_t *s_c, float *s_red, float (*s_bmax)[kPrepWaves]) {
    constexpr int KS = N / 32;
    constexpr int NTW = wave_ntiles(W);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    constexpr int PD = KS < PD0 ? KS : PD0;  // slices in flight
    constexpr int BV = kChunk * 4 / kPrepThreads;  // 16-byte pieces of B per thread and slice
    // this thread's pieces: B row (tid + kPrepThreads it) / 4, C local row
    // (tid % 256) / 4 (rows 0..31: row block q, 32..63: row block 7-q; the
    // threads from 256 on load the same pieces again and do not store them),
    // piece tid % 4
    const int v = tid & 3;
    const int cr = (tid & 255) >> 2;
    const int crow = cr < 32 ? 32 * q + cr : 32 * (7 - q) + cr - 32;
    u32x4 rbv[PD][BV], rcv[PD];
    auto load_slice = [&](int ks, int d) {
        // rows past the chunk end repeat its last row: the tiles' entries
        // there meet only zero x rows or unstored outputs later
#pragma unroll
        for (int it = 0; it < BV; ++it) {
            const int j = (tid + it * kPrepThreads) >> 2;
            rbv[d][it] = *reinterpret_cast<const u32x4 *>(p.B + ((t0 + min(j, len - 1)) * p.G + g) * N + ks * 32 + v * 8);
        }
        rcv[d] = *reinterpret_cast<const u32x4 *>(p.C + ((t0 + min(crow, len - 1)) * p.G + g) * N + ks * 32 + v * 8);
    };
    f32x16 accg[NTW];
#pragma unroll
    for (int i = 0; i < NTW; ++i) accg[i] = f32x16{};

#pragma unroll
    for (int d = 0; d < PD; ++d) load_slice(d, d);
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
        __syncthreads();  // previous slice consumed
#pragma unroll
        for (int it = 0; it < BV; ++it) {
            const int j = (tid + it * kPrepThreads) >> 2;
            *reinterpret_cast<u32x4 *>(s_b + j * R_STRIDE + v * 4) = rbv[ks % PD][it];
        }
        if (tid < 256) *reinterpret_cast<u32x4 *>(s_c + cr * R_STRIDE + v * 4) = rcv[ks % PD];
        const bool frag = (ks & 3) == q;  // uniform: this workgroup writes slice ks's B^T operands
        if (frag) {
            // max |B| of this thread's share of the slice (rows past the chunk
            // end repeat its last row: no new maximum)
            u16x2 mb2 = u16x2{0, 0};
#pragma unroll
            for (int it = 0; it < BV; ++it)
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    mb2 = __builtin_elementwise_max(mb2, __builtin_bit_cast(u16x2, rbv[ks % PD][it][w] & 0x7FFF7FFFu));
            s_bmax[ks & 1][W] = wave_max(__uint_as_float(max((uint32_t)mb2[0], (uint32_t)mb2[1]) << 16));
        }
        if (ks + PD < KS) load_slice(ks + PD, ks % PD);  // in flight during the next slices' MFMAs
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int ti = W + kPrepWaves * i;
                const int rb = pair_rb(q, ti), t = pair_t(q, ti);
                const int lr = rb == q ? 0 : 32;  // local C row block
                const bf16x8 cb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(s_c + (lr + l32) * R_STRIDE + 8 * kk + 4 * hl));
                const bf16x8 bb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(s_b + (32 * t + l32) * R_STRIDE + 8 * kk + 4 * hl));
                accg[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb, cb, accg[i], 0, 0, 0);
            }
        }
        // ---- B^T of this slice (n tile ks) as fp16 MFMA A operands:
        // fragment (K-step s, lane l) holds rows n = 32 ks + l%32, tokens
        // 16 s + 8 (l/32) + 0..7 (0 past the chunk end), scaled by 2^bexp
        if (frag) {
            float bm = 0.f;
#pragma unroll
            for (int w = 0; w < kPrepWaves; ++w) bm = fmaxf(bm, s_bmax[ks & 1][w]);
            const int sb = f16_scale_exponent(bm);
            const float bs = ldexpf(1.0f, sb);
            const int64_t tile = ((int64_t)c * p.G + g) * (N / 32) + ks;
            if (tid == 0) p.bexp[tile] = sb;
            const uint16_t *sb16 = reinterpret_cast<const uint16_t *>(s_b);
#pragma unroll
            for (int it = 0; it < 1024 / kPrepThreads; ++it) {
                const int f = tid + it * kPrepThreads;  // fragment: K-step f / 64, lane f % 64
                const int col = f & 31;
                const int j0 = 16 * (f >> 6) + 8 * ((f >> 5) & 1);
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = j0 + 2 * e;
                    const float lo = j < len ? bf16_bits_to_float(sb16[j * 2 * R_STRIDE + col]) * bs : 0.0f;
                    const float hi = j + 1 < len ? bf16_bits_to_float(sb16[(j + 1) * 2 * R_STRIDE + col]) * bs : 0.0f;
                    o[e] = pack_f16x2(lo, hi);
                }
                *reinterpret_cast<u32x4 *>(p.bfrag + (tile * 1024 + f) * 8) = u32x4{o[0], o[1], o[2], o[3]};
            }
        }
    }
    // the diagonal tiles keep only j <= i (element e of lane l: j - 32 rb =
    // 8(e/4) + 4(l/32) + e%4, i - 32 rb = l%32), so readers need no mask
#pragma unroll
    for (int i = 0; i < NTW; ++i)
        if (pair_rb(q, W + kPrepWaves * i) == pair_t(q, W + kPrepWaves * i))
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + 4 * hl + (e & 3) > l32) accg[i][e] = 0.f;
    // one power-of-two scale for the pair's tiles
    float gm = 0.f;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) gm = fmaxf(gm, fabsf(accg[i][e]));
    gm = wave_max(gm);
    if (lane == 0) s_red[W] = gm;
    __syncthreads();
    float gmax = 0.f;
#pragma unroll
    for (int w = 0; w < kPrepWaves; ++w) gmax = fmaxf(gmax, s_red[w]);
    const int sg = f16_scale_exponent(gmax);
    if (tid == 0) p.gexp[((int64_t)c * p.G + g) * 4 + q] = sg;
    const float gs = ldexpf(1.0f, sg);
    // tiles in accumulator order: tile rb(rb+1)/2 + t, 64 lanes x 16 fp16
    uint16_t *dst = p.cbt + ((int64_t)c * p.G + g) * 36 * 1024;
#pragma unroll
    for (int i = 0; i < NTW; ++i) {
        const int rb = pair_rb(q, W + kPrepWaves * i), t = pair_t(q, W + kPrepWaves * i);
        u32x4 *o = reinterpret_cast<u32x4 *>(dst + (rb * (rb + 1) / 2 + t) * 1024 + lane * 16);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            o[h2] = u32x4{pack_f16x2(accg[i][8 * h2] * gs, accg[i][8 * h2 + 1] * gs),
                          pack_f16x2(accg[i][8 * h2 + 2] * gs, accg[i][8 * h2 + 3] * gs),
                          pack_f16x2(accg[i][8 * h2 + 4] * gs, accg[i][8 * h2 + 5] * gs),
                          pack_f16x2(accg[i][8 * h2 + 6] * gs, accg[i][8 * h2 + 7] * gs)};
    }
}

template <int N, int PD>
__global__ __launch_bounds__(kPrepThreads) void ssd_prep_kernel(Params p) {
    // XCD-aware decode: workgroup ids go to the eight XCDs round-robin; every
    // workgroup (group, pair) of chunk c gets an id congruent to c mod 8, so
    // they all run on one XCD and read the chunk's B and C into one L2
    const int xcd = blockIdx.x & 7;
    const int slot = blockIdx.x >> 3;
    const int per = 4 * p.G;  // workgroups per chunk
    const int c = (slot / per) * 8 + xcd;
    const int rem = slot - (slot / per) * per;
    const int g = rem >> 2;
    const int q = rem & 3;
    if (c >= p.nchunks_grid) return;  // the grid's padding to a multiple of 8 chunks (uniform)
    const bool lead = g == 0 && q == 0;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ int s_wtot[kPrepWaves];
    __shared__ int s_loc[2];
    __shared__ float s_red[kPrepWaves];
    __shared__ float s_bmax[2][kPrepWaves];
    __shared__ __attribute__((aligned(16))) uint32_t s_b[kChunk * R_STRIDE];
    __shared__ __attribute__((aligned(16))) uint32_t s_c[64 * R_STRIDE];

    // ---- locate chunk c: exclusive prefix of per-sequence chunk counts
    if (tid == 0) { s_loc[0] = -1; s_loc[1] = 0; }
    int carry = 0;
    for (int base = 0; base < p.batch; base += kPrepThreads) {
        const int b = base + tid;
        int n = 0;
        if (b < p.batch) {
            const int len = p.qsl[b + 1] - p.qsl[b];
            n = !is_short_sequence(len, p.short_max) && len > 0 ? (len + kChunk - 1) / kChunk : 0;
        }
        const int wincl = wave_incl_scan(n);
        __syncthreads();  // protects s_wtot from the previous round
        if (lane == 63) s_wtot[wave] = wincl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < kPrepWaves; ++w) {
            if (w < wave) before += s_wtot[w];
            total += s_wtot[w];
        }
        const int excl = carry + before + wincl - n;
        if (b < p.batch) {
            if (c >= excl && c < excl + n) { s_loc[0] = b; s_loc[1] = c - excl; }
            if (c == 0 && lead) p.chunk_off[b] = excl;
        }
        carry += total;
    }
    if (c == 0 && lead) {
        // the sequences the state chain walks: all of them when no sequence
        // can take the short path, else those longer than its limit
        // and, in a second list, the sequences the token recurrence takes
        // (both counts packed in one scan: low 16 bits and high 16 bits per
        // round of kPrepThreads sequences)
        int carry2 = 0, carry3 = 0;
        for (int base = 0; base < p.batch; base += kPrepThreads) {
            const int b = base + tid;
            int f = 0, r = 0;
            if (b < p.batch) {
                const int len = p.qsl[b + 1] - p.qsl[b];
                f = !is_short_sequence(len, p.short_max);
                r = len >= 1 && len <= p.recur_max;
            }
            const int wincl = wave_incl_scan(f | (r << 16));
            __syncthreads();
            if (lane == 63) s_wtot[wave] = wincl;
            __syncthreads();
            int before = 0, total = 0;
            for (int w = 0; w < kPrepWaves; ++w) {
                if (w < wave) before += s_wtot[w];
                total += s_wtot[w];
            }
            const int incl = before + wincl;
            if (f) p.seq_list[carry2 + (incl & 0xFFFF) - 1] = b;
            if (r) p.recur_list[carry3 + (incl >> 16) - 1] = b;
            carry2 += total & 0xFFFF;
            carry3 += total >> 16;
        }
        if (tid == 0) {
            p.chunk_off[p.batch] = carry;
            p.meta[0] = carry;
            p.meta[1] = carry2; p.meta[2] = carry3; p.meta[3] = 0;
        }
    }
    __syncthreads();
    const int b = s_loc[0];
    if (b < 0) {
        if (tid == 0 && lead) p.desc[c] = make_int4(-1, 0, 0, 0);
        return;
    }
    const int64_t t0 = (int64_t)p.qsl[b] + (int64_t)s_loc[1] * kChunk;
    const int len = (int)min((int64_t)kChunk, (int64_t)p.qsl[b + 1] - t0);

    if (lead && tid == 0) p.desc[c] = make_int4(b, (int)t0, len, 0);

    // ---- chunk_cumsum of heads q, q + 4, ... of the group, one wavefront per
    // head; lane l takes tokens 4l .. 4l+3 (past the chunk end: dt of its
    // last token, which chunk_cumsum4 discards)
    {
        const int hg = p.H / p.G;
        for (int i = q + 4 * wave; i < hg; i += 4 * kPrepWaves) {  // uniform per wavefront
            const int h = g * hg + i;
            float dtv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) dtv[e] = p.dt[(t0 + min(4 * lane + e, len - 1)) * p.H + h];
            const float bias = p.dt_bias != nullptr ? p.dt_bias[h] : 0.0f;
            float dts[4], cs2[4];
            chunk_cumsum4(dtv, bias, p.A[h], p.dt_softplus != 0, len, dts, cs2);
            const int64_t r = ((int64_t)c * p.H + h) * kChunk + 4 * lane;
            *reinterpret_cast<float4 *>(p.dts + r) = make_float4(dts[0], dts[1], dts[2], dts[3]);
            *reinterpret_cast<float4 *>(p.cs2 + r) = make_float4(cs2[0], cs2[1], cs2[2], cs2[3]);
        }
    }

    // ---- C.B^T tiles of row blocks q and 7-q, B^T operands of slices q, q+4, ...
    switch (__builtin_amdgcn_readfirstlane(wave)) {
    case 0: gram_tiles<N, 0, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 1: gram_tiles<N, 1, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 2: gram_tiles<N, 2, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 3: gram_tiles<N, 3, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 4: gram_tiles<N, 4, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 5: gram_tiles<N, 5, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    case 6: gram_tiles<N, 6, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    default: gram_tiles<N, 7, PD>(p, c, g, q, t0, len, s_b, s_c, s_red, s_bmax); break;
    }
}

template <int PD>
static hipError_t launch_pd(const Params &p, const Launch &l, dim3 grid) {
    switch (p.N) {
    case 64: return launch_kernel(ssd_prep_kernel<64, PD>, grid, dim3(kPrepThreads), l, p);
    case 128: return launch_kernel(ssd_prep_kernel<128, PD>, grid, dim3(kPrepThreads), l, p);
    case 256: return launch_kernel(ssd_prep_kernel<256, PD>, grid, dim3(kPrepThreads), l, p);
    default: return hipErrorInvalidValue;
    }
}

// Slices in flight: all of them at dstate 64 and 128 (76 and 100 registers);
// at 256, all eight while the full chunks fit one workgroup per compute unit
// (the workgroup's latency is then the kernel's; 148 registers, one workgroup
// per CU), else three (120 registers, two workgroups per CU, which hide each
// other's latency).
hipError_t launch_prep(const Params &p, const Launch &l) {
    const dim3 grid((unsigned)((p.nchunks_grid + 7) / 8 * 8 * 4 * p.G));
    const bool all = p.N < 256 || p.T / kChunk * 4 * p.G <= p.num_cus;
    return all ? launch_pd<8>(p, l, grid) : launch_pd<3>(p, l, grid);
}

}  // namespace ssd
