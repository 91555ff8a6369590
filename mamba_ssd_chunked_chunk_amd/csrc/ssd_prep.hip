// Step 0 + step 1 of the scan: the chunk table and the per-chunk cumulative
// decay ("chunk_cumsum"), plus the power-of-two exponents of B and C.
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
// One thread per token; 16 heads at a time are scanned across the 256 threads.
//
// B and C exponents (blockIdx.y == 1 + array * G + g): the contractions feed
// B and C to fp16 MFMA after an exact power-of-two scaling; the exponent that
// puts max|B| (or max|C|) of the chunk's rows of group g in [2^14, 2^15) is
// computed here, once per (chunk, group).
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kPrepThreads = 256;
constexpr int kHeadBlock = 16;
}  // namespace

__global__ __launch_bounds__(kPrepThreads) void ssd_prep_kernel(Params p) {
    const int c = blockIdx.x;
    const int job = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ int s_wtot[4];
    __shared__ int s_loc[2];
    __shared__ float s_hsum[4][kHeadBlock];
    __shared__ uint32_t s_umax[4];

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
        int before = 0;
        for (int w = 0; w < wave; ++w) before += s_wtot[w];
        const int total = s_wtot[0] + s_wtot[1] + s_wtot[2] + s_wtot[3];
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
        // ---- dts and cs2: thread = token, 16 heads at a time
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
            // inclusive scan over the 256 tokens, per head
#pragma unroll
            for (int k = 0; k < kHeadBlock; ++k) a[k] = wave_incl_scan(a[k]);
            __syncthreads();  // s_hsum free from the previous head block
            if (lane == 63) {
#pragma unroll
                for (int k = 0; k < kHeadBlock; ++k) s_hsum[wave][k] = a[k];
            }
            __syncthreads();
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
        return;
    }

    // ---- B or C exponent for one group: max |value| over the chunk's rows
    const int which = (job - 1) / p.G;
    const int g = (job - 1) - which * p.G;
    const uint16_t *src = which ? p.C : p.B;
    const int nvec = p.N / 8;  // 16-byte vectors per token row
    const int total = len * nvec;
    uint32_t m = 0;
    for (int base = tid; base < total; base += kPrepThreads * 8) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = base + u * kPrepThreads;
            v[u] = u32x4{0u, 0u, 0u, 0u};
            if (i < total) {
                const int jj = i / nvec;
                const int vv = i - jj * nvec;
                v[u] = *reinterpret_cast<const u32x4 *>(src + ((t0 + jj) * p.G + g) * p.N + vv * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t lo = v[u][k] & 0x7FFFu, hi = (v[u][k] >> 16) & 0x7FFFu;
                m = m > lo ? m : lo;
                m = m > hi ? m : hi;
            }
    }
    m = wave_max_u32(m);
    if (lane == 0) s_umax[wave] = m;
    __syncthreads();
    if (tid == 0) {
        uint32_t mm = s_umax[0];
        for (int w = 1; w < 4; ++w) mm = mm > s_umax[w] ? mm : s_umax[w];
        // bf16 magnitude bits: exponent field in bits 7..14
        const int e = (int)(mm >> 7) - 127;
        int32_t *dst = which ? p.cexp : p.bexp;
        dst[(int64_t)c * p.G + g] = mm == 0 ? 0 : 14 - e;
    }
}

hipError_t launch_prep(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL(ssd_prep_kernel, dim3((unsigned)p.nchunks_max, (unsigned)(1 + 2 * p.G)),
                       dim3(kPrepThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace ssd
