// Short sequences in one pass ("short path"): every sequence of recur_max+1
// .. short_max tokens (at most 128; dstate 64 or 128) is scanned whole by one
// kernel, instead of going through the chunk table, the chunk-state and
// state-passing steps and their fp16 intermediates in the workspace (the
// shortest, 1 .. recur_max tokens, take the token-recurrence kernel).  With
// the path on, zero-length sequences are also finished here (their final
// state is the initial one, or zeros).
//
// For sequence b (tokens t0 .. t0+l-1), group g and each head h of the group,
// with dts, cs2 = log2(e) * cumulative A*dts and the initial state h0 (the
// pool slot or initial_states row, or zero):
//   y[i][p]    = exp2(cs2_i) * sum_n C[i,n] h0[p][n]                     (state carried in)
//              + sum_{j<=i} (C_i . B_j) exp2(cs2_i - cs2_j) dts_j x[j][p]  (within the sequence)
//              + D x[i][p]
//   final[p][n] = exp2(cs2_last) h0[p][n] + sum_j exp2(cs2_last - cs2_j) dts_j x[j][p] B[j][n]
// which is the chunked form of "Mamba chunk scan with segsum" (description)
// for a single chunk, i.e. the per-token recurrence of "mamba2_ssd_scan"
// ("Per-token recurrence") unrolled over the whole sequence; the final state
// goes straight to its slot (the pool in place, or final_states).
//
// Work split: one workgroup of eight wavefronts per (sequence, group, slice
// of the group's heads), walking its heads; workgroup ids run over the
// sequences slowest, so a sequence's workgroups spread over the XCDs.
// Wavefront w owns
//   - y rows 32 rb .. +31 with rb = 0, 0, 1, 1, 3, 3, 2, 2 for w = 0..7 (the
//     two wavefronts on a SIMD, w and w+4, hold 5 causal tiles between them;
//     blocks past the end skip their products), p columns 32 (w%2) .. +31,
//     with its row block's C.B^T tiles (bf16 MFMA on the exact inputs, kept as
//     fp16 under a power of two in registers for all heads);
//   - the 32x32 tile (p tile w%2, n tile w/2) of the final state, when
//     w/2 < dstate/32, whose h0 elements it holds in registers.
// B^T and C are staged once in LDS as fp16.  Per head, two barriers: before
// the first, x^T and (w x)^T (fp16 under one power of two) and h0 (fp16
// under a power of two per row p) are staged from registers loaded during the
// previous head, and the next head's x, dt, h0 and scalars are loaded
// (unconditionally: after the last head it loads itself again, so no wait
// depends on a branch).  Between the barriers: the state tile's S = B^T (w x),
// the off-diagonal part h0 C^T, the causal tiles (below the diagonal as a
// column-factor table times one row factor; the diagonal tile with its decay
// per element); then, once the next head's loads have landed, its maxima and
// decay tables go to the other half of a double buffer, and only then are
// this head's y and final state (exp2(cs2_last) h0 + S, straight into the
// slot) stored: a vector-memory wait also waits for the stores before it.
#include <type_traits>

#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kSThreads = 512;
constexpr int kSWaves = kSThreads / 64;
constexpr int kLS = kShortMax;   // tokens per sequence at most
constexpr int XS = kLS / 2 + 2;  // dwords per x^T row: 64 token pairs + pad (8-byte reads)
constexpr int BS = kLS / 2 + 4;  // dwords per B^T row: 64 token pairs + pad (16-byte reads)
static_assert(kLS == 128, "the short path's layouts assume 128 tokens at most");

template <int N>
struct __attribute__((aligned(16))) ShortSmem {
    static constexpr int HS = N / 2 + 4;  // dwords per h0 row and per C row
    static constexpr int NT = N / 32;
    uint32_t bt[N * BS];            // B^T fp16, [n][token pair], scaled by 2^sb
    uint32_t ct[kLS * HS];          // C fp16, [token][n pair], row block rb scaled by 2^sc[rb]
    uint32_t xt[kHeadDim * XS];     // x^T fp16, [p][token pair], scaled by 2^xe
    uint32_t wxt[kHeadDim * XS];    // (w x)^T fp16, the same layout, scaled by 2^(xe - kw)
    uint32_t h0[kHeadDim * HS];     // h0 fp16, [p][n pair], row p scaled by 2^hx[p]
    float cs[2][kLS];               // cs2 (past the end: the last token's value)
    float dts[2][kLS];              // dts (0 past the end)
    float w[2][kLS];                // exp2(cs2_last - cs2_j) dts_j 2^-kw, |.| < 1
    float u[2][3][kLS];             // row block r+1: dts_j exp2(cs2_{32(r+1)-1} - cs2_j) for j < 32(r+1)
    float rowmax[2][NT][kHeadDim];  // max |h0| of row p over each n tile
    float xmx[2][kSWaves];          // max |x| of each wavefront's share
    float hdr[2][4];                // {cs2_last, kw, max dts, unused}
    float hs[kHeadDim];             // 2^-hx[p]
    float red[kSWaves];             // max |B| of each wavefront's share (prologue)
};

// A 32x32 state tile in the MFMA accumulator layout holds, in lane (l, h =
// l/32), the elements n = 8a + 4h + 0..3 (a = 0..3) of row l%32.  With bf16
// storage each lane instead loads or stores 16 bytes, n = 16h + 8c + 0..7
// (c = 0, 1): dword d of group c is (n = 16h + 8c + 2d, +1).  Lane h = 0
// keeps its own n 0..3 and 8..11 and takes n 16..19 and 24..27 from lane
// l+32; lane h = 1 the mirror image: one v_permlane32_swap per dword pair.
__device__ __forceinline__ void to_acc_layout(const u32x4 &q0, const u32x4 &q1, f32x4 (&hn)[4]) {
    uint32_t w[4][2];  // [a][pair of e]
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(q0[d], q0[d + 2], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(q1[d], q1[d + 2], false, false);
        w[0][d] = s0[0];
        w[2][d] = s0[1];
        w[1][d] = s1[0];
        w[3][d] = s1[1];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
        hn[a] = f32x4{bf16x2_lo(w[a][0]), bf16x2_hi(w[a][0]), bf16x2_lo(w[a][1]), bf16x2_hi(w[a][1])};
}
__device__ __forceinline__ void from_acc_layout(const f32x4 (&o)[4], u32x4 &q0, u32x4 &q1) {
    uint32_t w[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
        w[a][0] = pack_bf16x2(o[a][0], o[a][1]);
        w[a][1] = pack_bf16x2(o[a][2], o[a][3]);
    }
#pragma unroll
    for (int d = 0; d < 2; ++d) {
        const auto s0 = __builtin_amdgcn_permlane32_swap(w[0][d], w[2][d], false, false);
        const auto s1 = __builtin_amdgcn_permlane32_swap(w[1][d], w[3][d], false, false);
        q0[d] = s0[0];
        q0[d + 2] = s0[1];
        q1[d] = s1[0];
        q1[d + 2] = s1[1];
    }
}

// running maximum of bf16 magnitudes (as bit patterns) over a dword's two halves
__device__ __forceinline__ uint32_t bf16_absmax2(uint32_t m, uint32_t w) {
    return max(m, max(w & 0x7FFFu, (w >> 16) & 0x7FFFu));
}
}  // namespace

// SB: states stored as bf16 (read widened to fp32, final state rounded once).
template <int N, bool SB>
__global__ __launch_bounds__(kSThreads) void ssd_short_kernel(Params p) {
    static_assert(N == 64 || N == 128, "the short path covers dstate 64 and 128");
    constexpr int NT = N / 32;  // n tiles
    constexpr int KN = N / 16;  // K-steps over n
    constexpr int HS = ShortSmem<N>::HS;
    __shared__ ShortSmem<N> sm;

    if (p.N != N) return;
    // workgroup id -> (sequence, group, slice of the group's heads), the
    // sequence slowest: ids are dealt to the eight XCDs round-robin, so the
    // workgroups of one sequence spread over several XCDs (with the sequence
    // fastest, all of them would share one, and a batch's few short sequences
    // could crowd a single XCD)
    const int per_seq = (int)(gridDim.x / (unsigned)p.batch);  // groups * slices
    const int hz = per_seq / p.G;
    const int b = (int)(blockIdx.x / (unsigned)per_seq);
    const int rem = (int)blockIdx.x - b * per_seq;
    const int g = rem / hz;
    const int64_t t0 = p.qsl[b];
    const int len = p.qsl[b + 1] - (int)t0;
    if (!is_short_sequence(len, p.short_max)) return;  // the chunked path takes it
    if (len >= 1 && len <= p.recur_max) return;                      // the token-recurrence kernel takes it
    const int64_t slot = p.cache_idx != nullptr ? (int64_t)p.cache_idx[b] : (int64_t)b;
    const bool init = p.init_all != 0 || (p.has_init != nullptr && p.has_init[b] != 0);
    const int hg = p.H / p.G;
    const int hpw = hg / hz;
    const int h_begin = g * hg + (rem - g * hz) * hpw;
    const int h_end = h_begin + hpw;
    const void *state_src = p.state_in != nullptr ? p.state_in : p.state_out;
    if (len == 0) {  // no tokens: the final state is the initial one (or zeros)
        constexpr int64_t head_bytes = (int64_t)kHeadDim * N * (SB ? 2 : 4);  // a multiple of 16 * kSThreads
        for (int h = h_begin; h < h_end; ++h) {
            const char *src = static_cast<const char *>(state_src) + (slot * p.H + h) * head_bytes;
            char *dst = static_cast<char *>(p.state_out) + (slot * p.H + h) * head_bytes;
            if (init && src == dst) continue;  // in place: already there
            for (int64_t e = 16 * (int64_t)threadIdx.x; e < head_bytes; e += 16 * kSThreads)
                *reinterpret_cast<u32x4 *>(dst + e) = init ? *reinterpret_cast<const u32x4 *>(src + e) : u32x4{};
        }
        return;
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    // y row block: 0, 0, 1, 1, 3, 3, 2, 2 for wavefronts 0..7, so the two
    // wavefronts on each SIMD (w and w+4) hold row blocks with 5 causal tiles
    // between them
    const int rb = (wave >> 1) ^ ((wave >> 2) & 1);
    const int pty = wave & 1;           // y p tile
    const bool active = 32 * rb < len;  // wavefront-uniform
    const int pts = wave & 1;           // state tile: p tile
    const int nt = wave >> 1;           //             n tile
    const bool owner = nt < NT;         // wavefront-uniform
    const int nks = (len + 15) / 16;    // K-steps over tokens (wavefront-uniform)
    const int64_t rstride = (int64_t)p.G * N;  // elements between consecutive tokens of B and C
    const uint16_t *Bg = p.B + (t0 * p.G + g) * N;
    const uint16_t *Cg = p.C + (t0 * p.G + g) * N;

    // ---- B^T into LDS as fp16 under one power of two sb.  Thread item q:
    // token pair (lane), 8 n starting at 8 * (8q + wave)
    constexpr int BQ = N / 64;
    u32x4 braw[BQ][2];
    uint32_t bm = 0;
#pragma unroll
    for (int q = 0; q < BQ; ++q) {
        const int ng = kSWaves * q + wave;
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            // rows past the end repeat the last one (their weights w are 0)
            const int j = 2 * lane + e;
            const u32x4 v = *reinterpret_cast<const u32x4 *>(Bg + (int64_t)min(j, len - 1) * rstride + 8 * ng);
            braw[q][e] = v;
#pragma unroll
            for (int k = 0; k < 4; ++k) bm = bf16_absmax2(bm, v[k]);
        }
    }
    // C rows of this wavefront's row block (raw bf16, row i_l; rows past the
    // end repeat the last one: their outputs are never stored)
    const int i_l = 32 * rb + l32;
    u32x4 cq[KN];
    {
        const uint16_t *crow = Cg + (int64_t)min(i_l, len - 1) * rstride + 8 * hl;
#pragma unroll
        for (int k = 0; k < KN; ++k) cq[k] = *reinterpret_cast<const u32x4 *>(crow + 16 * k);
    }
    {
        const float m = wave_max(__uint_as_float(bm << 16));
        if (lane == 0) sm.red[wave] = m;
    }

    // ---- C.B^T tiles of the row block: tile t (t <= rb) at lane l, element e
    // holds G^T[j][i] = B_j . C_i with j = 32t + 8(e/4) + 4(l/32) + e%4,
    // i = i_l; zero where j > i.  Kept as fp16 under 2^ge.
    uint32_t gt[4][8];
    int ge = 0;
    float gmax = 0.f;
    {
        f32x16 gf[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
        if (active) {
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                if (t <= rb) {  // wavefront-uniform
                    const uint16_t *brow = Bg + (int64_t)min(32 * t + l32, len - 1) * rstride + 8 * hl;
#pragma unroll
                    for (int k = 0; k < KN; ++k) {
                        const bf16x8 a =
                            __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(brow + 16 * k));
                        gf[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, __builtin_bit_cast(bf16x8, cq[k]),
                                                                       gf[t], 0, 0, 0);
                    }
                }
            }
        }
        const int dl = l32 - 4 * hl;  // element 8a + b of tile rb is on the diagonal when 8a + b == dl
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                if (t > rb || (t == rb && 8 * (e >> 2) + (e & 3) > dl)) gf[t][e] = 0.f;
                gmax = fmaxf(gmax, fabsf(gf[t][e]));
            }
        gmax = wave_max(gmax);
        ge = f16_scale_exponent(gmax);
        const float s = ldexpf(1.0f, ge);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int q = 0; q < 8; ++q) gt[t][q] = pack_f16x2(gf[t][2 * q] * s, gf[t][2 * q + 1] * s);
    }
    // C rows of the row block into LDS as fp16 under exponent sc (the same
    // in both wavefronts of the block; the p-tile-0 one writes them)
    int sc;
    {
        uint32_t m = 0;
#pragma unroll
        for (int k = 0; k < KN; ++k)
#pragma unroll
            for (int q = 0; q < 4; ++q) m = bf16_absmax2(m, cq[k][q]);
        sc = f16_scale_exponent(wave_max(__uint_as_float(m << 16)));
        const float cs = ldexpf(1.0f, sc);
        if (pty == 0) {
#pragma unroll
            for (int k = 0; k < KN; ++k) {
                u32x4 o;
#pragma unroll
                for (int q = 0; q < 4; ++q) o[q] = pack_f16x2(bf16x2_lo(cq[k][q]) * cs, bf16x2_hi(cq[k][q]) * cs);
                *reinterpret_cast<u32x4 *>(sm.ct + i_l * HS + 8 * k + 4 * hl) = o;
            }
        }
    }
    __syncthreads();  // sm.red: B maxima
    int sb;
    {
        float m = 0.f;
#pragma unroll
        for (int v = 0; v < kSWaves; ++v) m = fmaxf(m, sm.red[v]);
        sb = f16_scale_exponent(m);
        const float bs = ldexpf(1.0f, sb);
#pragma unroll
        for (int q = 0; q < BQ; ++q) {
            const int n0 = 8 * (kSWaves * q + wave);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t a = braw[q][0][k >> 1], c = braw[q][1][k >> 1];
                const float lo = (k & 1) ? bf16x2_hi(a) : bf16x2_lo(a);
                const float hi = (k & 1) ? bf16x2_hi(c) : bf16x2_lo(c);
                sm.bt[(n0 + k) * BS + lane] = pack_f16x2(lo * bs, hi * bs);
            }
        }
    }

    // ---- per-head inputs, loaded one head ahead.  x: token pair tid/8, p =
    // 8 (tid%8) .. +7 (eight lanes read a token's 128-byte row); dt
    // (wavefront 0): tokens 2 lane, 2 lane + 1; h0 (state-tile owners): row
    // p = 32 pts + l32, n = 32 nt + 8a + 4 hl + 0..3.
    // Tokens past the end repeat the last one: nothing selects on the loaded
    // values here (that would wait for them), and their weights are 0.  The
    // per-head scalars A, dt_bias and D come with them, so that no load is
    // waited for between these points.
    const int xm8 = tid >> 3;  // token pair of the x loads
    const int xg8 = tid & 7;   // p group of the x loads
    u32x4 xr[2];
    float dtr[2] = {0.f, 0.f};
    f32x4 hn[4] = {f32x4{}, f32x4{}, f32x4{}, f32x4{}};
    float anx = 0.f, bnx = 0.f, dnx = 0.f;
    auto load_inputs = [&](int h) {
        if (p.D != nullptr) dnx = p.D[h];
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = 2 * xm8 + e;
            xr[e] = *reinterpret_cast<const u32x4 *>(p.x + ((t0 + min(j, len - 1)) * p.H + h) * kHeadDim +
                                                     8 * xg8);
        }
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < 2; ++e) dtr[e] = p.dt[(t0 + min(2 * lane + e, len - 1)) * p.H + h];
            anx = p.A[h];
            if (p.dt_bias != nullptr) bnx = p.dt_bias[h];
        }
        if (owner && init) {  // both uniform over the wavefront
            const int64_t row = ((slot * p.H + h) * kHeadDim + 32 * pts + l32) * N + 32 * nt;
            if constexpr (SB) {
                // bf16: 16 bytes per lane (n = 32 nt + 16 hl + 8c .. +7), then
                // lanes l and l+32 trade halves into the accumulator layout
                const uint16_t *src = static_cast<const uint16_t *>(state_src) + row + 16 * hl;
                const u32x4 q0 = *reinterpret_cast<const u32x4 *>(src);
                const u32x4 q1 = *reinterpret_cast<const u32x4 *>(src + 8);
                to_acc_layout(q0, q1, hn);
            } else {
#pragma unroll
                for (int a = 0; a < 4; ++a) hn[a] = load_state4<SB>(state_src, row + 4 * hl + 8 * a);
            }
        }
    };
    // maxima and decay table of the loaded head h into buffer nb
    auto summarize = [&](int nb) {
        {
            uint32_t m = 0;
#pragma unroll
            for (int e = 0; e < 2; ++e)
#pragma unroll
                for (int k = 0; k < 4; ++k) m = bf16_absmax2(m, xr[e][k]);
            const float mx = wave_max(__uint_as_float(m << 16));
            if (lane == 0) sm.xmx[nb][wave] = mx;
        }
        if (owner) {
            float m = 0.f;
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) m = fmaxf(m, fabsf(hn[a][e]));
            const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
            m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // lanes l and l^32: the same row
            if (hl == 0) sm.rowmax[nb][nt][32 * pts + l32] = m;
        }
        if (wave == 0) {  // the decay table of the head
            const float ah = anx;
            float d[2];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                const float v = dtr[e] + bnx;
                d[e] = 2 * lane + e < len ? (p.dt_softplus ? softplus_f(v) : v) : 0.f;
            }
            const float a1 = ah * d[1];
            const float incl = wave_incl_scan(ah * d[0] + a1);
            const float c1 = incl * kLog2e, c0 = (incl - a1) * kLog2e;
            const float last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(incl), 63)) * kLog2e;
            const float w0 = fast_exp2(last - c0) * d[0], w1 = fast_exp2(last - c1) * d[1];
            const float wm = wave_max(fmaxf(fabsf(w0), fabsf(w1)));
            const int kw = wm > 0.f ? min((int)((__float_as_uint(wm) >> 23) & 0xFF) - 126, 126) : 0;
            const float wsc = ldexpf(1.0f, -kw);
            const float dm = wave_max(fmaxf(fabsf(d[0]), fabsf(d[1])));
            // column factors of the tiles below the diagonal of row blocks 1..3
            // (the sequence's log2 growth caps the exponent: 0 for A <= 0)
            const float c_first = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(c0)));
            const float capg = fmaxf(0.f, last - c_first);
#pragma unroll
            for (int r = 0; r < 3; ++r) {
                const float ref =
                    __int_as_float(__builtin_amdgcn_readlane(__float_as_int(c1), 16 * (r + 1) - 1));  // token 32(r+1)-1
                const bool in0 = 2 * lane < 32 * (r + 1);  // both tokens of the lane fall on the same side
                *reinterpret_cast<float2 *>(&sm.u[nb][r][2 * lane]) =
                    in0 ? make_float2(d[0] * fast_exp2(fminf(ref - c0, capg)), d[1] * fast_exp2(fminf(ref - c1, capg)))
                        : make_float2(0.f, 0.f);
            }
            *reinterpret_cast<float2 *>(&sm.cs[nb][2 * lane]) = make_float2(c0, c1);
            *reinterpret_cast<float2 *>(&sm.dts[nb][2 * lane]) = make_float2(d[0], d[1]);
            *reinterpret_cast<float2 *>(&sm.w[nb][2 * lane]) = make_float2(w0 * wsc, w1 * wsc);
            if (lane == 0) {
                sm.hdr[nb][0] = last;
                sm.hdr[nb][1] = (float)kw;
                sm.hdr[nb][2] = dm;
            }
        }
    };

    load_inputs(h_begin);
    summarize(0);
    __syncthreads();  // B^T staged; buffer 0 holds the first head's maxima and table

#pragma unroll 1
    for (int h = h_begin; h < h_end; ++h) {
        const int cur = (h - h_begin) & 1;
        // ======== stage x^T and h0 of head h from registers
        float xm = 0.f;
#pragma unroll
        for (int v = 0; v < kSWaves; ++v) xm = fmaxf(xm, sm.xmx[cur][v]);
        const int xe = f16_scale_exponent(xm);
        {
            const float s0 = ldexpf(1.0f, xe);
            const float2 w2 = *reinterpret_cast<const float2 *>(&sm.w[cur][2 * xm8]);
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t a = xr[0][k >> 1], c = xr[1][k >> 1];
                const float lo = ((k & 1) ? bf16x2_hi(a) : bf16x2_lo(a)) * s0;
                const float hi = ((k & 1) ? bf16x2_hi(c) : bf16x2_lo(c)) * s0;
                sm.xt[(8 * xg8 + k) * XS + xm8] = pack_f16x2(lo, hi);
                sm.wxt[(8 * xg8 + k) * XS + xm8] = pack_f16x2(lo * w2.x, hi * w2.y);
            }
        }
        f32x4 hc[4];  // h0 of head h (the loads below refill hn with head h+1)
        const float dh = dnx;
        if (owner) {
            const int pp = 32 * pts + l32;
            float m = 0.f;
#pragma unroll
            for (int v = 0; v < NT; ++v) m = fmaxf(m, sm.rowmax[cur][v][pp]);
            const int hx = f16_scale_exponent(m);
            const float s = ldexpf(1.0f, hx);
            uint32_t *dst = sm.h0 + pp * HS + 16 * nt + 2 * hl;
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                hc[a] = hn[a];
                *reinterpret_cast<u32x2 *>(dst + 4 * a) =
                    u32x2{pack_f16x2(hn[a][0] * s, hn[a][1] * s), pack_f16x2(hn[a][2] * s, hn[a][3] * s)};
            }
            if (nt == 0 && hl == 0) sm.hs[pp] = ldexpf(1.0f, -hx);
        }
        // the next head's inputs (after the last head: the last one again,
        // unconditionally, so that no wait depends on a branch)
        load_inputs(min(h + 1, h_end - 1));
        __syncthreads();  // (1) x^T, (w x)^T, h0 and the decay tables of head h

        const float cs_last = sm.hdr[cur][0];
        const int kw = (int)sm.hdr[cur][1];
        const float dmax = sm.hdr[cur][2];
        // ======== final-state tile: S^T = B^T (w x)
        f32x16 sacc = f32x16{};
        if (owner) {
            f32x16 acc = f32x16{};
            const uint32_t *xrow = sm.wxt + (32 * pts + l32) * XS + 4 * hl;
            const uint32_t *brow = sm.bt + (32 * nt + l32) * BS + 4 * hl;
            // K-steps of 16 tokens in unrolled blocks of 2, 4 or 8 (steps past
            // the end add zeros: w is 0 there)
            auto steps = [&](auto kn) {
#pragma unroll
                for (int k = 0; k < decltype(kn)::value; ++k) {
                    // tokens 16k + 8hl .. +7 (8-byte reads of (w x)^T)
                    const u32x2 xa = *reinterpret_cast<const u32x2 *>(xrow + 8 * k);
                    const u32x2 xb = *reinterpret_cast<const u32x2 *>(xrow + 8 * k + 2);
                    const f16x8 aop = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(brow + 8 * k));
                    acc = mfma32_f16(aop, __builtin_bit_cast(f16x8, u32x4{xa[0], xa[1], xb[0], xb[1]}), acc);
                }
            };
            if (nks <= 2) steps(std::integral_constant<int, 2>{});
            else if (nks <= 4) steps(std::integral_constant<int, 4>{});
            else steps(std::integral_constant<int, 8>{});
            sacc = acc;
        }

        // ======== y rows of this wavefront's row block, p tile pty
        f32x16 yacc = f32x16{};
        float yinv = 0.f;
        if (active) {  // wavefront-uniform
            const float *csv = sm.cs[cur];
            const float *dtv = sm.dts[cur];
            const float cs_i = csv[min(i_l, len - 1)];
            const float cap = fmaxf(0.f, cs_last - csv[0]);
            // |M| < 2^(15 - smx): |G| dts (decay <= 2^cap) plus |D| on the
            // diagonal; capped so that 2^(smx + xe) times the off-diagonal
            // part stays far from fp32 overflow when the bound is tiny
            const int smx = min(f16_scale_exponent(gmax * dmax * fast_exp2(cap) + fabsf(dh)), 64 - xe);
            // off-diagonal part h0 C^T, in the units of the causal part (2^(smx + xe))
            f32x16 acc = f32x16{};
            const uint32_t *hrow = sm.h0 + (32 * pty + l32) * HS + 4 * hl;
            const uint32_t *crow = sm.ct + i_l * HS + 4 * hl;
#pragma unroll
            for (int k = 0; k < KN; ++k) {
                const f16x8 hf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(hrow + 8 * k));
                const f16x8 cf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(crow + 8 * k));
                acc = mfma32_f16(hf, cf, acc);
            }
            const float f = ldexpf(fast_exp2(cs_i), smx + xe - sc);
#pragma unroll
            for (int a = 0; a < 4; ++a) {
                const f32x4 s4 = *reinterpret_cast<const f32x4 *>(sm.hs + 32 * pty + 8 * a + 4 * hl);
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[4 * a + e] *= f * s4[e];
            }
            // causal tiles t <= rb: M^T per element (G^T is zero above the
            // diagonal), then (2^xe x_t)^T M^T.  x^T rows 32 pty + l32, the
            // tokens in M's K order: step 0 takes j = 32t + 8a + 4hl + 0..3
            // for a = 0, 1, step 1 for a = 2, 3.
            const float gs = ldexpf(1.0f, smx - ge);
            const uint32_t *xrow = sm.xt + (32 * pty + l32) * XS + 2 * hl;
            auto causal_tile = [&](int t, const float (&mv)[16], f32x16 &c) {
                const f16x8 mf0 = __builtin_bit_cast(
                    f16x8, u32x4{pack_f16x2(mv[0], mv[1]), pack_f16x2(mv[2], mv[3]), pack_f16x2(mv[4], mv[5]),
                                 pack_f16x2(mv[6], mv[7])});
                const f16x8 mf1 = __builtin_bit_cast(
                    f16x8, u32x4{pack_f16x2(mv[8], mv[9]), pack_f16x2(mv[10], mv[11]), pack_f16x2(mv[12], mv[13]),
                                 pack_f16x2(mv[14], mv[15])});
                const u32x2 *row = reinterpret_cast<const u32x2 *>(xrow + 16 * t);
                const u32x2 xa = row[0], xb = row[2], xc = row[4], xd = row[6];
                c = mfma32_f16(__builtin_bit_cast(f16x8, u32x4{xa[0], xa[1], xb[0], xb[1]}), mf0, c);
                c = mfma32_f16(__builtin_bit_cast(f16x8, u32x4{xc[0], xc[1], xd[0], xd[1]}), mf1, c);
            };
            // tiles below the diagonal: exp2(cs2_i - cs2_j) = exp2(cs2_i - ref)
            // exp2(ref - cs2_j) with ref = cs2 of token 32 rb - 1; the column
            // factor (with dts_j) comes from the table, the row factor
            // multiplies their sum
            if (rb > 0) {
                f32x16 below = f32x16{};
                const float *ur = sm.u[cur][rb - 1];
#pragma unroll
                for (int t = 0; t < 3; ++t) {
                    if (t < rb) {  // wavefront-uniform
                        float mv[16];
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
                            const f32x4 u4 = *reinterpret_cast<const f32x4 *>(ur + 32 * t + 8 * a + 4 * hl);
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const f16x2 g2 = __builtin_bit_cast(f16x2, gt[t][2 * a + q]);
                                mv[4 * a + 2 * q] = (float)g2[0] * (gs * u4[2 * q]);
                                mv[4 * a + 2 * q + 1] = (float)g2[1] * (gs * u4[2 * q + 1]);
                            }
                        }
                        causal_tile(t, mv, below);
                    }
                }
                const float vr = fast_exp2(fminf(cs_i - csv[32 * rb - 1], cap));
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[e] += below[e] * vr;
            }
            // the diagonal tile: the decay per element, D on the diagonal
            {
                const float dx = ldexpf(dh, smx);
                const int dl = l32 - 4 * hl;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    if (t == rb) {  // wavefront-uniform
                        float mv[16];
#pragma unroll
                        for (int a = 0; a < 4; ++a) {
                            const int j0 = 32 * t + 8 * a + 4 * hl;
                            const f32x4 c4 = *reinterpret_cast<const f32x4 *>(csv + j0);
                            const f32x4 d4 = *reinterpret_cast<const f32x4 *>(dtv + j0);
#pragma unroll
                            for (int q = 0; q < 2; ++q) {
                                const f16x2 g2 = __builtin_bit_cast(f16x2, gt[t][2 * a + q]);
#pragma unroll
                                for (int r = 0; r < 2; ++r) {
                                    const int bb = 2 * q + r;
                                    const float m =
                                        (float)g2[r] * gs * fast_exp2(fminf(cs_i - c4[bb], cap)) * d4[bb];
                                    mv[4 * a + bb] = 8 * a + bb == dl ? m + dx : m;
                                }
                            }
                        }
                        causal_tile(t, mv, acc);
                    }
                }
            }
            yacc = acc;
            yinv = ldexpf(1.0f, -(smx + xe));
        }
        // the next head's maxima and table, before this head's stores: a
        // vector-memory wait also waits for every store issued before it
        summarize(cur ^ 1);

        // ======== stores.  Final state: lane l holds S^T[n][p] for p = 32 pts
        // + l%32, n = 32 nt + 8a + 4(l/32) + 0..3
        if (owner) {
            const float dec = fast_exp2(cs_last);
            const float us = ldexpf(1.0f, kw - sb - xe);
            const int64_t row = ((slot * p.H + h) * kHeadDim + 32 * pts + l32) * N + 32 * nt;
            f32x4 o[4];
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int e = 0; e < 4; ++e) o[a][e] = dec * hc[a][e] + sacc[4 * a + e] * us;
            if constexpr (SB) {  // the load's trade in reverse: 16 bytes per lane
                u32x4 q0, q1;
                from_acc_layout(o, q0, q1);
                uint16_t *dst = static_cast<uint16_t *>(p.state_out) + row + 16 * hl;
                *reinterpret_cast<u32x4 *>(dst) = q0;
                *reinterpret_cast<u32x4 *>(dst + 8) = q1;
            } else {
#pragma unroll
                for (int a = 0; a < 4; ++a) store_state4<SB>(p.state_out, row + 4 * hl + 8 * a, o[a]);
            }
        }
        // y back to unit scale, bf16; lanes l and l+32 trade groups so each
        // stores 8 consecutive p (16 bytes)
        if (active && i_l < len) {
            uint16_t *dsty = p.y + ((t0 + i_l) * p.H + h) * kHeadDim + 32 * pty + 8 * hl;
#pragma unroll
            for (int a = 0; a < 4; a += 2) {
                const uint32_t a0 = pack_bf16x2(yacc[4 * a] * yinv, yacc[4 * a + 1] * yinv);
                const uint32_t a1 = pack_bf16x2(yacc[4 * a + 2] * yinv, yacc[4 * a + 3] * yinv);
                const uint32_t b0 = pack_bf16x2(yacc[4 * a + 4] * yinv, yacc[4 * a + 5] * yinv);
                const uint32_t b1 = pack_bf16x2(yacc[4 * a + 6] * yinv, yacc[4 * a + 7] * yinv);
                const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                *reinterpret_cast<u32x4 *>(dsty + 8 * a) = u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
        }
        __syncthreads();  // (2) this head's LDS no longer read; the next head's buffer written
    }
}

hipError_t launch_short(const Params &p, const Launch &l) {
    const dim3 grid((unsigned)((int64_t)p.batch * p.G * short_head_slices(p)));
    const dim3 block(kSThreads);
    switch (p.N) {
    case 64:
        return p.state_bf16 ? launch_kernel(ssd_short_kernel<64, true>, grid, block, l, p)
                            : launch_kernel(ssd_short_kernel<64, false>, grid, block, l, p);
    case 128:
        return p.state_bf16 ? launch_kernel(ssd_short_kernel<128, true>, grid, block, l, p)
                            : launch_kernel(ssd_short_kernel<128, false>, grid, block, l, p);
    default:  // no sequence is short at other dstates (not launched there); a one-workgroup no-op
        return launch_kernel(ssd_short_kernel<128, false>, dim3(1, 1, 1), block, l, p);  // p.N != 128: exits
    }
}

}  // namespace ssd
