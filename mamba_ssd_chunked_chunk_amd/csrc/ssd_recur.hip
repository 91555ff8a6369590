// Very short sequences (decode steps) as the plain recurrence: every
// sequence of 1 .. recur_max tokens (at most kRecurMax; dstate 64 or 128, the
// short path on) is scanned token by token, as in "mamba2_ssd_scan"
// ("Per-token recurrence"):
//   dts = softplus(dt + dt_bias),  state = state * exp(A dts) + dts x B,
//   y = C . state + D x,
// reading the initial state from, and writing the final state to, its slot.
// This is the cooperative dstate-split form the pages describe for short
// sequences: each thread holds 8 consecutive dstate elements of state rows
// (16-byte loads and stores; the N/8 threads of a row cover it
// contiguously), so the state is read once and written once, and every token
// costs 16 FMAs per element group plus a sum over the row's lanes (DPP) for
// y.  Longer short sequences go to the MFMA short kernel, whose state I/O is
// the same but whose per-token arithmetic is not.
//
// A grid of at most 16384 workgroups of 512 threads walks the (sequence,
// head) items of the sequences listed for it (recur_list, written by the
// chunk-state step), each workgroup a block of consecutive items, so a batch with few of them costs
// few live workgroups.  Per item, every load the head needs (its
// state rows, x and dt of its tokens, the tokens' B and C rows, staged in
// LDS) is issued before any arithmetic, so the item waits for memory once; at
// about 60 registers four workgroups share a compute unit.
#include <algorithm>

#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kRThreads = 512;

// sum over each aligned group of LANES (8 or 16) lanes; every lane receives it
template <int LANES>
__device__ __forceinline__ float group_sum(float v) {
    v = dpp_add_all<0xB1>(v);   // quad_perm [1,0,3,2]
    v = dpp_add_all<0x4E>(v);   // quad_perm [2,3,0,1]
    v = dpp_add_all<0x141>(v);  // row_half_mirror: groups of 8
    if constexpr (LANES >= 16) v = dpp_add_all<0x140>(v);  // row_mirror: rows of 16
    return v;
}
}  // namespace

template <int N, bool SB>
__global__ __launch_bounds__(kRThreads) void ssd_recur_kernel(Params p) {
    static_assert(N == 64 || N == 128, "the recurrence path covers dstate 64 and 128");
    constexpr int RL = N / 8;             // threads per state row
    constexpr int RP = kRThreads / RL;    // rows per pass
    constexpr int NPASS = kHeadDim / RP;  // passes over the 64 rows
    constexpr int L = kRecurMax;
    __shared__ __attribute__((aligned(16))) uint32_t s_b[L][N / 2];  // B rows of the tokens (bf16 pairs)
    __shared__ __attribute__((aligned(16))) uint32_t s_c[L][N / 2];

    if (p.N != N) return;
    const int tid = threadIdx.x;
    const int rr = tid / RL;        // row within a pass
    const int n0 = (tid % RL) * 8;  // first of this thread's 8 dstate elements
    const void *state_src = p.state_in != nullptr ? p.state_in : p.state_out;
    // this workgroup's block of consecutive items (a run of heads of one or
    // two sequences): a sequence's bookkeeping is read once per run
    const int64_t items = (int64_t)p.meta[2] * p.H;
    const int64_t per = (items + gridDim.x - 1) / gridDim.x;
    const int64_t i0 = (int64_t)blockIdx.x * per;
    const int64_t i1 = items < i0 + per ? items : i0 + per;
    int64_t kc = -1, t0 = 0, slot = 0;
    int len = 1;
    bool init = false;
#pragma unroll 1
    for (int64_t it = i0; it < i1; ++it) {
        const int64_t k = it / p.H;
        const int h = (int)(it - k * p.H);
        if (k != kc) {  // uniform
            kc = k;
            const int b = p.recur_list[k];
            t0 = p.qsl[b];
            len = p.qsl[b + 1] - (int)t0;  // 1 .. recur_max
            slot = p.cache_idx != nullptr ? (int64_t)p.cache_idx[b] : (int64_t)b;
            init = p.init_all != 0 || (p.has_init != nullptr && p.has_init[b] != 0);
        }
        const int g = h / (p.H / p.G);
        const int64_t base = ((slot * p.H + h) * kHeadDim + rr) * N + n0;

        // ---- every load first: the tokens' B and C rows into LDS (tokens past
        // the end repeat the last one), the state rows rr + RP*k, x of those rows
        // and dt of every token, the head's scalars
        if (tid < L * (N / 8)) {
            const int t = tid / (N / 8), c8 = (tid % (N / 8)) * 8;
            const int64_t r = ((t0 + min(t, len - 1)) * p.G + g) * N + c8;
            *reinterpret_cast<u32x4 *>(&s_b[t][c8 / 2]) = *reinterpret_cast<const u32x4 *>(p.B + r);
            *reinterpret_cast<u32x4 *>(&s_c[t][c8 / 2]) = *reinterpret_cast<const u32x4 *>(p.C + r);
        }
        float s[NPASS][8], xv[NPASS][L], dtv[L];
#pragma unroll
        for (int k = 0; k < NPASS; ++k) {
            if (init) {
                load_state8<SB>(state_src, base + (int64_t)k * RP * N, s[k]);
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) s[k][e] = 0.f;
            }
        }
#pragma unroll
        for (int t = 0; t < L; ++t) {
            const int64_t tok = t0 + min(t, len - 1);
            dtv[t] = p.dt[tok * p.H + h];
#pragma unroll
            for (int k = 0; k < NPASS; ++k) xv[k][t] = bf16_bits_to_float(p.x[(tok * p.H + h) * kHeadDim + rr + k * RP]);
        }
        const float ah = p.A[h] * kLog2e;
        const float hb = p.dt_bias != nullptr ? p.dt_bias[h] : 0.f;
        const float dh = p.D != nullptr ? p.D[h] : 0.f;
        __syncthreads();  // B and C staged

#pragma unroll
        for (int t = 0; t < L; ++t) {
            if (t < len) {  // uniform
                const float v = dtv[t] + hb;
                const float dts = p.dt_softplus ? softplus_f(v) : v;
                const float dA = fast_exp2(ah * dts);
                const u32x4 bq = *reinterpret_cast<const u32x4 *>(&s_b[t][n0 / 2]);
                const u32x4 cq = *reinterpret_cast<const u32x4 *>(&s_c[t][n0 / 2]);
#pragma unroll
                for (int k = 0; k < NPASS; ++k) {
                    const float u = dts * xv[k][t];
                    float part = 0.f;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        s[k][2 * q] = s[k][2 * q] * dA + u * bf16x2_lo(bq[q]);
                        s[k][2 * q + 1] = s[k][2 * q + 1] * dA + u * bf16x2_hi(bq[q]);
                        part += bf16x2_lo(cq[q]) * s[k][2 * q] + bf16x2_hi(cq[q]) * s[k][2 * q + 1];
                    }
                    const float yv = group_sum<RL>(part) + dh * xv[k][t];
                    if (tid % RL == 0) p.y[((t0 + t) * p.H + h) * kHeadDim + rr + k * RP] = float_to_bf16_bits(yv);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < NPASS; ++k) store_state8<SB>(p.state_out, base + (int64_t)k * RP * N, s[k]);
        __syncthreads();  // B and C of this item no longer read
    }
}

hipError_t launch_recur(const Params &p, const Launch &l) {
    // one workgroup per possible item, up to 16384 (then blocks of items)
    const dim3 grid((unsigned)std::min<int64_t>((int64_t)p.batch * p.H, 16384));
    const dim3 block(kRThreads);
    switch (p.N) {
    case 64:
        return p.state_bf16 ? launch_kernel(ssd_recur_kernel<64, true>, grid, block, l, p)
                            : launch_kernel(ssd_recur_kernel<64, false>, grid, block, l, p);
    case 128:
        return p.state_bf16 ? launch_kernel(ssd_recur_kernel<128, true>, grid, block, l, p)
                            : launch_kernel(ssd_recur_kernel<128, false>, grid, block, l, p);
    default:  // no sequence takes it at other dstates (not launched there); a one-workgroup no-op
        return launch_kernel(ssd_recur_kernel<128, false>, dim3(1), block, l, p);  // p.N != 128: exits
    }
}

}  // namespace ssd
