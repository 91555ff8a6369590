// Steps 3 and 5 of the scan: the inter-chunk state recurrence ("state_passing")
// and the in-place pool write-back.
//
// For sequence b, head h and every state element (p, n), walking the
// sequence's chunks k in order:
//   h_in[first]  = has_initial_state[b] ? ssm_pool[cache_indices[b]][h][p][n] : 0
//   h_in[k + 1]  = exp(cs_last(k)) * h_in[k] + S[k]
//   final        = exp(cs_last(K-1)) * h_in[K-1] + S[K-1]
//   ssm_pool[cache_indices[b]][h][p][n] = final
// This is the "inter-chunk state recurrence with exponential decay" of
// "Mamba chunk scan with segsum" (description); the reset at each sequence
// start and the final state at each sequence end come from "mamba2_ssd_scan"
// ("Per-token recurrence"); reading the initial state from, and writing the
// final state to, slot cache_indices[b] of the pool is
// "Mamba2SSDChunkScanVarlenFwdInplace" (struct description).  A sequence with
// no tokens writes its initial state (or zeros) back.
//
// Chunk contributions arrive as fp16 under one power-of-two exponent per
// 32x32 tile of (chunk, head).  The chain is fp32.  h_in only feeds the outputs y; it is stored as fp16
// with one power-of-two scale per row p (11 significant bits: bf16's 8 would
// put the off-diagonal part's rounding error near the tolerance of y).
// Each thread owns four consecutive (p, n) elements of one (sequence, head),
// reads its pool element before the sequence's loop and writes it after, so
// the in-place read-then-write of a slot never races.  The chunk
// contributions are loaded kDepth chunks ahead of their use, so that many
// loads per thread are in flight while the chain advances.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kDepth = 4;
}

__global__ __launch_bounds__(256) void ssd_state_passing_kernel(Params p) {
    const int b = blockIdx.x;
    const int h = blockIdx.y;
    const int64_t head_elems = (int64_t)kHeadDim * p.N;
    const int64_t e0 = ((int64_t)blockIdx.z * 256 + threadIdx.x) * 4;
    if (e0 >= head_elems) return;

    // clamped to the table so malformed query_start_loc cannot index past it
    const int k1 = (int)min((int64_t)p.chunk_off[b + 1], p.nchunks_max);
    const int k0 = min(p.chunk_off[b], k1);
    const int64_t slot = p.cache_idx[b];
    const bool init = p.has_init != nullptr && p.has_init[b] != 0;
    float4 *pool4 = reinterpret_cast<float4 *>(p.pool + (slot * p.H + h) * head_elems + e0);

    float4 st = init ? *pool4 : make_float4(0.f, 0.f, 0.f, 0.f);
    const int64_t stride = (int64_t)p.H * head_elems;  // one chunk of states
    const uint16_t *S = p.states + ((int64_t)k0 * p.H + h) * head_elems + e0;
    // exponent of this thread's 32x32 tile (p / 32, n / 32) in each chunk
    const int NT = p.N / 32;
    const int tile = (int)((e0 / p.N) >> 5) * NT + (int)((e0 % p.N) >> 5);
    const int32_t *sexp = p.sexp + ((int64_t)k0 * p.H + h) * 2 * NT + tile;
    const int64_t sexp_stride = (int64_t)p.H * 2 * NT;
    const float *cs_last = p.cs2 + ((int64_t)k0 * p.H + h) * kChunk + kChunk - 1;
    const int64_t cs_stride = (int64_t)p.H * kChunk;
    uint16_t *hin = p.hin + ((int64_t)k0 * p.H + h) * head_elems + e0;
    int32_t *hexp = p.hexp + ((int64_t)k0 * p.H + h) * kHeadDim + e0 / p.N;
    const int nk = k1 - k0;

    // ring of the next kDepth chunk contributions: fp16 values, their exponent, cs2_last
    uint2 s[kDepth];
    int se[kDepth];
    float d[kDepth];
#pragma unroll
    for (int q = 0; q < kDepth; ++q) {
        s[q] = make_uint2(0u, 0u);
        se[q] = 0;
        d[q] = 0.f;
        if (q < nk) {
            s[q] = *reinterpret_cast<const uint2 *>(S + q * stride);
            se[q] = sexp[q * sexp_stride];
            d[q] = cs_last[q * cs_stride];
        }
    }
    for (int kb = 0; kb < nk; kb += kDepth) {
#pragma unroll
        for (int q = 0; q < kDepth; ++q) {
            const int k = kb + q;
            if (k < nk) {
                // h_in row p as fp16, scaled by the power of two that puts the
                // row's max |h| in [2^14, 2^15); the N/4 lanes of one row share it
                float m = fmaxf(fmaxf(fabsf(st.x), fabsf(st.y)), fmaxf(fabsf(st.z), fabsf(st.w)));
                // row max: rows are N/4 consecutive lanes (16, 32 or 64)
                m = row16_max(m);
                if (p.N >= 128) m = fmaxf(m, __shfl_xor(m, 16, 64));
                if (p.N >= 256) m = fmaxf(m, __shfl_xor(m, 32, 64));
                const int sh = f16_scale_exponent(m);
                const float sc = ldexpf(1.0f, sh);
                uint2 hv;
                hv.x = pack_f16x2(st.x * sc, st.y * sc);
                hv.y = pack_f16x2(st.z * sc, st.w * sc);
                *reinterpret_cast<uint2 *>(hin + (int64_t)k * stride) = hv;
                if (e0 % p.N == 0) hexp[(int64_t)k * p.H * kHeadDim] = sh;
                const float dec = fast_exp2(d[q]);
                const float us = ldexpf(1.0f, -se[q]);
                st.x = dec * st.x + f16_bits_to_float(s[q].x & 0xFFFFu) * us;
                st.y = dec * st.y + f16_bits_to_float(s[q].x >> 16) * us;
                st.z = dec * st.z + f16_bits_to_float(s[q].y & 0xFFFFu) * us;
                st.w = dec * st.w + f16_bits_to_float(s[q].y >> 16) * us;
                if (k + kDepth < nk) {  // refill this ring slot kDepth chunks ahead
                    s[q] = *reinterpret_cast<const uint2 *>(S + (int64_t)(k + kDepth) * stride);
                    se[q] = sexp[(int64_t)(k + kDepth) * sexp_stride];
                    d[q] = cs_last[(int64_t)(k + kDepth) * cs_stride];
                }
            }
        }
    }
    *pool4 = st;
}

hipError_t launch_state_passing(const Params &p, hipStream_t s) {
    const int64_t head_elems = (int64_t)kHeadDim * p.N;
    const unsigned zb = (unsigned)((head_elems / 4 + 255) / 256);
    dim3 grid((unsigned)p.batch, (unsigned)p.H, zb);
    hipLaunchKernelGGL(ssd_state_passing_kernel, grid, dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace ssd
