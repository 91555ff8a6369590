// Step 0 + step 1 of the scan: the chunk table and the per-chunk cumulative
// decay ("chunk_cumsum").
//
// Chunk table: sequence b owns ceil(len_b / 256) chunks (none when empty);
// chunk c of the call is found from the exclusive prefix sum of those counts,
// so no chunk ever straddles two sequences (the state resets at every
// query_start_loc boundary: "mamba2_ssd_scan", section "Per-token
// recurrence").  Every workgroup computes the prefix itself, so no separate
// launch is needed; workgroup 0 also publishes it (chunk_off, nchunks) for the
// state-passing step.
//
// Cumulative decay: for each head h and token j of the chunk,
//   dts_j = softplus(dt[t,h] + dt_bias[h])   (or dt + dt_bias without softplus)
//   cs2_j = log2(e) * sum_{k <= j} A[h] * dts_k
// ("mamba2_ssd_scan", "Per-token recurrence": dA = exp(A * dts); the segment
// sums of "Mamba chunk scan with segsum", description).  Past the chunk end,
// dts = 0 and cs2 stays at its last value, so cs2[255] is the chunk's total.
//
// B and C exponents: the contractions feed B and C to fp16 MFMA after an exact
// power-of-two scaling; the exponents that put max|B| and max|C| of the chunk
// in [2^14, 2^15) are computed here once per (chunk, group).
#include "ssd_common.hpp"

namespace ssd {

__global__ __launch_bounds__(256) void ssd_prep_kernel(Params p) {
    const int c = blockIdx.x;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;

    __shared__ int s_wtot[4];
    __shared__ int s_loc[2];
    __shared__ uint32_t s_umax[4];

    // ---- locate chunk c: exclusive prefix of per-sequence chunk counts
    if (tid == 0) { s_loc[0] = -1; s_loc[1] = 0; }
    int carry = 0;
    for (int base = 0; base < p.batch; base += 256) {
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
            if (c == 0) p.chunk_off[b] = excl;
        }
        carry += total;
    }
    if (c == 0 && tid == 0) {
        p.chunk_off[p.batch] = carry;
        p.meta[0] = carry;
        p.meta[1] = 0; p.meta[2] = 0; p.meta[3] = 0;
    }
    __syncthreads();
    const int b = s_loc[0];
    if (b < 0) {
        if (tid == 0) p.desc[c] = make_int4(-1, 0, 0, 0);
        return;
    }
    const int64_t t0 = (int64_t)p.qsl[b] + (int64_t)s_loc[1] * kChunk;
    const int len = (int)min((int64_t)kChunk, (int64_t)p.qsl[b + 1] - t0);
    if (tid == 0) p.desc[c] = make_int4(b, (int)t0, len, 0);

    // ---- dts and cs2 per head: one wavefront per head, 4 tokens per lane
    for (int h = wave; h < p.H; h += 4) {
        const float a_h = p.A[h];
        const float bias = p.dt_bias ? p.dt_bias[h] : 0.0f;
        float d[4], s[4];
        float run = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int j = lane * 4 + i;
            float ds = 0.0f;
            if (j < len) {
                const float v = p.dt[(t0 + j) * p.H + h] + bias;
                ds = p.dt_softplus ? softplus_f(v) : v;
            }
            d[i] = ds;
            run += a_h * ds;
            s[i] = run;
        }
        const float incl = wave_incl_scan(run);
        const float off = incl - run;
        float4 dv = make_float4(d[0], d[1], d[2], d[3]);
        float4 cv = make_float4((off + s[0]) * kLog2e, (off + s[1]) * kLog2e,
                                (off + s[2]) * kLog2e, (off + s[3]) * kLog2e);
        const int64_t row = ((int64_t)c * p.H + h) * kChunk + lane * 4;
        *reinterpret_cast<float4 *>(p.dts + row) = dv;
        *reinterpret_cast<float4 *>(p.cs2 + row) = cv;
    }

    // ---- per-group B and C exponents: max |B|, max |C| over the chunk's tokens
    const int nvec = p.N / 8;  // 16-byte vectors per token row
    for (int which = 0; which < 2; ++which) {
        const uint16_t *src = which ? p.C : p.B;
        int32_t *dst = which ? p.cexp : p.bexp;
        for (int g = 0; g < p.G; ++g) {
            uint32_t m = 0;
            for (int i = tid; i < len * nvec; i += 256) {
                const int j = i / nvec;
                const int v = i - j * nvec;
                const u32x4 q = *reinterpret_cast<const u32x4 *>(
                    src + ((t0 + j) * p.G + g) * p.N + v * 8);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const uint32_t lo = q[k] & 0x7FFFu, hi = (q[k] >> 16) & 0x7FFFu;
                    m = m > lo ? m : lo;
                    m = m > hi ? m : hi;
                }
            }
            m = wave_max_u32(m);
            __syncthreads();
            if (lane == 0) s_umax[wave] = m;
            __syncthreads();
            if (tid == 0) {
                uint32_t mm = s_umax[0];
                for (int w = 1; w < 4; ++w) mm = mm > s_umax[w] ? mm : s_umax[w];
                // bf16 magnitude bits: exponent field in bits 7..14
                const int e = (int)(mm >> 7) - 127;
                dst[(int64_t)c * p.G + g] = mm == 0 ? 0 : 14 - e;
            }
        }
    }
}

hipError_t launch_prep(const Params &p, hipStream_t s) {
    hipLaunchKernelGGL(ssd_prep_kernel, dim3((unsigned)p.nchunks_max), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ssd
