// Step 0 + step 1 of the scan: the chunk table and the per-chunk cumulative
// decay ("chunk_cumsum"), plus the per-(chunk, group) product that does not
// depend on the head: C.B^T.
//
// Chunk table: sequence b owns ceil(len_b / 256) chunks (none when empty);
// chunk c of the call is found from the exclusive prefix sum of those counts,
// so no chunk ever straddles two sequences (the state resets at every
// query_start_loc boundary: "mamba2_ssd_scan", section "Per-token
// recurrence").  Every workgroup computes the prefix itself, so no separate
// launch is needed; workgroup (0, 0) also publishes it (chunk_off, nchunks)
// for the state-passing step.  Sequences the short path takes (short_max > 0:
// 0 .. short_max tokens) own no chunks; workgroup (0, 0) then also writes
// the list of the sequences the state chain walks (the others) and the list
// of those of 1 .. recur_max tokens for the token-recurrence kernel, with
// their counts (meta[1], meta[2]).  The grid is sized to the host's bound on
// the chunks that can reach it.
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
//   blockwise; the diagonal tiles hold zeros where j > i), the
//   "attention-like" intra-chunk scores of "Mamba chunk scan with segsum"
//   (description) before decay.  They are shared by every head
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
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kPrepThreads = 512;
constexpr int kHeadBlock = 16;
constexpr int R_STRIDE = 20;  // dwords per staged row of 32 bf16 + pad
}  // namespace

// Tiles of the C.B^T job per wavefront.  SIMD s (= W & 3) owns row blocks s
// and 7-s, 9 tiles: its first wavefront (W < 4) takes all of row block s and
// the first 4-s tiles of row block 7-s (5 tiles), its second wavefront the
// other 4 tiles of row block 7-s.  Tile i of wavefront W is (row block
// tile_rb, column block tile_t), with t <= rb.
__host__ __device__ constexpr int gram_ntiles(int W) { return W < 4 ? 5 : 4; }
__host__ __device__ constexpr int gram_tile_rb(int W, int i) {
    return W < 4 ? (i <= (W & 3) ? (W & 3) : 7 - (W & 3)) : 7 - (W & 3);
}
__host__ __device__ constexpr int gram_tile_t(int W, int i) {
    return W < 4 ? (i <= (W & 3) ? i : i - ((W & 3) + 1)) : (4 - (W & 3)) + i;
}

// The C.B^T tiles of wavefront W (above) for chunk c and group g.  W is a
// template parameter so that the tile list, and with it every MFMA, is fixed
// at compile time.
template <int N, int W>
__device__ __forceinline__ void gram_tiles(const Params &p, int c, int g, int64_t t0, int len, uint32_t *s_b,
                                           uint32_t *s_c, float *s_gmax) {
    constexpr int KS = N / 32;
    constexpr int NTW = gram_ntiles(W);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    constexpr int PD = KS < 4 ? KS : 4;  // slices in flight
    u32x4 rbv[PD][2], rcv[PD][2];
    auto load_slice = [&](int ks, int d) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
            const int j = (tid + it * kPrepThreads) >> 2;
            const int v = tid & 3;
            // rows past the chunk end repeat its last row: the tiles' entries
            // there meet only zero x rows or unstored outputs later
            const int64_t off = ((t0 + min(j, len - 1)) * p.G + g) * N + ks * 32 + v * 8;
            rbv[d][it] = *reinterpret_cast<const u32x4 *>(p.B + off);
            rcv[d][it] = *reinterpret_cast<const u32x4 *>(p.C + off);
        }
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
#pragma unroll
            for (int i = 0; i < NTW; ++i) {
                const int rb = gram_tile_rb(W, i), t = gram_tile_t(W, i);
                const bf16x8 cb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(s_c + (32 * rb + l32) * R_STRIDE + 8 * kk + 4 * hl));
                const bf16x8 bb = __builtin_bit_cast(
                    bf16x8, *reinterpret_cast<const u32x4 *>(s_b + (32 * t + l32) * R_STRIDE + 8 * kk + 4 * hl));
                accg[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb, cb, accg[i], 0, 0, 0);
            }
        }
    }
    // the diagonal tiles keep only j <= i (element e of lane l: j - 32 rb =
    // 8(e/4) + 4(l/32) + e%4, i - 32 rb = l%32), so readers need no mask
#pragma unroll
    for (int i = 0; i < NTW; ++i)
        if (gram_tile_rb(W, i) == gram_tile_t(W, i))
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + 4 * hl + (e & 3) > l32) accg[i][e] = 0.f;
    // one power-of-two scale for all tiles of the chunk and group
    float gm = 0.f;
#pragma unroll
    for (int i = 0; i < NTW; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) gm = fmaxf(gm, fabsf(accg[i][e]));
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
    for (int i = 0; i < NTW; ++i) {
        const int rb = gram_tile_rb(W, i), t = gram_tile_t(W, i);
        u32x4 *o = reinterpret_cast<u32x4 *>(dst + (rb * (rb + 1) / 2 + t) * 1024 + lane * 16);
#pragma unroll
        for (int q = 0; q < 2; ++q)
            o[q] = u32x4{pack_f16x2(accg[i][8 * q] * gs, accg[i][8 * q + 1] * gs),
                         pack_f16x2(accg[i][8 * q + 2] * gs, accg[i][8 * q + 3] * gs),
                         pack_f16x2(accg[i][8 * q + 4] * gs, accg[i][8 * q + 5] * gs),
                         pack_f16x2(accg[i][8 * q + 6] * gs, accg[i][8 * q + 7] * gs)};
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
            n = !is_short_sequence(len, p.short_max) && len > 0 ? (len + kChunk - 1) / kChunk : 0;
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
    if (c == 0 && job == 0) {
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
            for (int w = 0; w < 8; ++w) {
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
        if (tid == 0 && job == 0) p.desc[c] = make_int4(-1, 0, 0, 0);
        return;
    }
    const int64_t t0 = (int64_t)p.qsl[b] + (int64_t)s_loc[1] * kChunk;
    const int len = (int)min((int64_t)kChunk, (int64_t)p.qsl[b + 1] - t0);

    if (job == 0) {
        if (tid == 0) p.desc[c] = make_int4(b, (int)t0, len, 0);
        // ---- dts and cs2: thread = (token j, half of a 16-head block); each
        // half-block of 8 heads is scanned over the 256 tokens by 4 wavefronts
        const int j = tid & (kChunk - 1);
        const int half = tid >> 8;
        const int wq = wave & 3;  // wavefront within the half
        const bool valid = j < len;
        constexpr int K = kHeadBlock / 2;
        // this thread's raw inputs of a head block (dt of its token, dt_bias and
        // A of its 8 heads), loaded one head block ahead so the loop waits for
        // memory once; the loads are unconditional (rows past the chunk end read
        // its last row, heads past H the last head, the last block itself again
        // past the end), their values discarded below where they do not apply
        const float *dt_row = p.dt + (t0 + min(j, len - 1)) * p.H;
        const float *bias = p.dt_bias ? p.dt_bias : p.A;  // a valid address either way
        const int last_hb = (p.H - 1) / kHeadBlock * kHeadBlock;
        float r_dt[K], r_bias[K], r_a[K];
        auto load_block = [&](int hb) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int h = min(hb + half * K + k, p.H - 1);
                r_dt[k] = dt_row[h];
                r_bias[k] = bias[h];
                r_a[k] = p.A[h];
            }
        };
        load_block(0);
        for (int hb = 0; hb < p.H; hb += kHeadBlock) {
            float v_dt[K], v_bias[K], v_a[K];
#pragma unroll
            for (int k = 0; k < K; ++k) { v_dt[k] = r_dt[k]; v_bias[k] = r_bias[k]; v_a[k] = r_a[k]; }
            load_block(min(hb + kHeadBlock, last_hb));
            float d[K], a[K];
#pragma unroll
            for (int k = 0; k < K; ++k) {
                const int h = hb + half * K + k;
                float ds = 0.0f;
                if (valid && h < p.H) {
                    const float v = v_dt[k] + (p.dt_bias ? v_bias[k] : 0.0f);
                    ds = p.dt_softplus ? softplus_f(v) : v;
                }
                d[k] = ds;
                a[k] = h < p.H ? v_a[k] * ds : 0.0f;
            }
            // inclusive scan over the tokens, per head
#pragma unroll
            for (int k = 0; k < K; ++k) a[k] = wave_incl_scan(a[k]);
            __syncthreads();  // s_hsum free from the previous head block
            if (lane == 63) {
#pragma unroll
                for (int k = 0; k < K; ++k) s_hsum[wave][k] = a[k];
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < K; ++k) {
                float off = 0.0f;
#pragma unroll
                for (int w = 0; w < 3; ++w) off += w < wq ? s_hsum[4 * half + w][k] : 0.0f;
                const int h = hb + half * K + k;
                if (h < p.H) {
                    const int64_t row = ((int64_t)c * p.H + h) * kChunk + j;
                    p.dts[row] = d[k];
                    p.cs2[row] = (off + a[k]) * kLog2e;
                }
            }
        }
        return;
    }

    // ---- group g: C.B^T tiles; SIMD k (= wave & 3) runs the 9 tiles of row
    // blocks k and 7-k, split 5 + 4 between its two wavefronts
    const int g = job - 1;
    switch (__builtin_amdgcn_readfirstlane(wave)) {
    case 0: gram_tiles<N, 0>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 1: gram_tiles<N, 1>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 2: gram_tiles<N, 2>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 3: gram_tiles<N, 3>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 4: gram_tiles<N, 4>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 5: gram_tiles<N, 5>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    case 6: gram_tiles<N, 6>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    default: gram_tiles<N, 7>(p, c, g, t0, len, s_b, s_c, s_gmax); break;
    }
}

hipError_t launch_prep(const Params &p, const Launch &l) {
    const dim3 grid((unsigned)p.nchunks_grid, (unsigned)(1 + p.G));
    switch (p.N) {
    case 64: return launch_kernel(ssd_prep_kernel<64>, grid, dim3(kPrepThreads), l, p);
    case 128: return launch_kernel(ssd_prep_kernel<128>, grid, dim3(kPrepThreads), l, p);
    case 256: return launch_kernel(ssd_prep_kernel<256>, grid, dim3(kPrepThreads), l, p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
