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
// w*x is scaled by the power of two that puts its maximum (per chunk and
// head) in [2^14, 2^15), and each 32-column slice of B by its own (so bf16 ->
// fp16 is exact but for values 2^24 below the slice's maximum).  S itself is stored as fp16
// under one power-of-two exponent per 32x32 tile of (chunk, head), the net
// exponent of all scalings, so the reader undoes them exactly; its rounding
// adds about 3e-4 relative error to the final states and halves the states
// traffic.
//
// Work split: one workgroup = one chunk and a block of HB heads of one group.
// The products are formed transposed, S^T[n][p] = sum_j B^T[n][j] (w_j
// x_j[p]); each wavefront owns one n tile and one or both p tiles, and keeps
// the B^T fragments of its n tile (16 K-steps of 16 tokens) in registers
// while the workgroup walks its heads, so B is read and converted once per
// block of heads: the wavefront loads its 32 columns of B for every token,
// stages them (128 tokens at a time) in an LDS region of its own and reads
// them back token-contiguous.  Each head's weighted x is
// staged in LDS, transposed to [p][token] (fp16 pairs of tokens per dword;
// 16-byte chunks of rows 16..31 of every 32-row block swapped pairwise so the
// 32 rows an MFMA operand reads fall on distinct banks); the next head's x,
// dts and cs2 are loaded into registers during the current head's products.
// Each lane ends up with 4 consecutive n of one p; lanes l and l+32 trade
// halves so that each stores 8 consecutive n as one 16-byte write.
// The exponent that scales the chunk's largest |x| of each head into
// [2^14, 2^15) is stored for the chunk-scan step, which stages x under it.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int XT_STRIDE = 132;  // dwords per x^T row: 128 token pairs + pad

// dword index of 16-byte chunk `q4` (in dwords, a multiple of 4) of row r
__device__ __forceinline__ int swz(int r, int q4) { return q4 ^ (((r >> 4) & 1) << 2); }

template <int N>
struct StateShape {
    static constexpr int NT = N / 32;                      // n tiles
    static constexpr int WAVES = 2 * NT < 8 ? 2 * NT : 8;  // 4 for dstate 64, else 8
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int PTW = WAVES == NT ? 2 : 1;        // p tiles per wavefront
    static constexpr int PQ = THREADS / 128;               // threads per token pair (p parts)
    static constexpr int PPT = kHeadDim / PQ;              // p values per thread in staging
};
}  // namespace

template <int N, int HB>
__global__ __launch_bounds__(StateShape<N>::THREADS) void ssd_chunk_state_kernel(Params p) {
    using S = StateShape<N>;
    constexpr int kThreads = S::THREADS;
    constexpr int kWaves = S::WAVES;
    constexpr int PTW = S::PTW;
    constexpr int PPT = S::PPT;
    constexpr int XV = PPT / 8;  // 16-byte x vectors per token per thread

    constexpr int BR = 20;  // dwords per staged B row: 32 bf16 + 16-byte pad
    __shared__ float s_red[2][kWaves][2];
    __shared__ __attribute__((aligned(16))) uint32_t s_xt[2][kHeadDim * XT_STRIDE];
    __shared__ __attribute__((aligned(16))) uint32_t s_b[kWaves][128 * BR];

    const int nhb = p.H / HB;
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / nhb) * 8 + xcd;
    const int hb = slot - (slot / nhb) * nhb;
    if (c >= p.meta[0]) return;
    const int4 dsc = p.desc[c];
    const int64_t t0 = dsc.y;
    const int len = dsc.z;
    const int h_first = hb * HB;
    const int g = h_first / (p.H / p.G);
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int l32 = lane & 31;
    const int hl = lane >> 5;

    // this wavefront's tiles: n tile nt, p tiles pt0 .. pt0+PTW-1
    const int nt = wave % S::NT;
    const int pt0 = PTW == 2 ? 0 : wave / S::NT;

    // ---- per-head inputs: thread = (p part, token pair).  The head loop is
    // software-pipelined over two phases, each closed by a barrier:
    //   A(k): the MFMAs of head k (x^T of head k in buffer k & 1), meanwhile
    //         weighting x of head k+1 and its wavefront maxima
    //   B(k): staging x^T of head k+1 into the other buffer, storing S of head k
    // so the products of one head overlap the VALU work of the next.  Inputs
    // are loaded two heads ahead; past the last head the loads repeat it (no
    // branch, so the compiler's wait counts stay exact).
    const int pair = tid & 127;
    const int pp = tid >> 7;  // p part: p = pp * PPT ..
    const int h_last = h_first + HB - 1;
    u32x4 xr[2][XV];
    float cs_tok[2], dt_tok[2], cs_last;
    auto load_head = [&](int h) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const int j = pair * 2 + e;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(
                p.x + ((t0 + min(j, len - 1)) * p.H + h) * kHeadDim + pp * PPT);
#pragma unroll
            for (int v = 0; v < XV; ++v) xr[e][v] = src[v];
            const int64_t crow = ((int64_t)c * p.H + h) * kChunk;
            cs_tok[e] = p.cs2[crow + j];
            dt_tok[e] = p.dts[crow + j];  // 0 past the chunk end
            cs_last = p.cs2[crow + kChunk - 1];
        }
    };
    // weighted x of the loaded head into xv, the wavefront maxima of |w x| and
    // |x| into s_red[b] (rows past the chunk end repeat its last row, with w = 0)
    float xv[2][PPT];
    auto weigh = [&](int b) {
        float mloc = 0.0f;
        u16x2 mraw2 = u16x2{0, 0};
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const float w = fast_exp2(cs_last - cs_tok[e]) * dt_tok[e];
#pragma unroll
            for (int v = 0; v < XV; ++v)
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    xv[e][v * 8 + 2 * k] = w * __uint_as_float(xr[e][v][k] << 16);
                    xv[e][v * 8 + 2 * k + 1] = w * __uint_as_float(xr[e][v][k] & 0xFFFF0000u);
                    mraw2 = __builtin_elementwise_max(mraw2, __builtin_bit_cast(u16x2, xr[e][v][k] & 0x7FFF7FFFu));
                }
#pragma unroll
            for (int k = 0; k < PPT; ++k) mloc = fmaxf(mloc, fabsf(xv[e][k]));
        }
        mloc = wave_max(mloc);
        const float mraw = wave_max(__uint_as_float(max((uint32_t)mraw2[0], (uint32_t)mraw2[1]) << 16));
        s_red[b][wave][0] = mloc;  // the same value from every lane
        s_red[b][wave][1] = mraw;
    };
    // x^T of the weighed head into s_xt[b] under the power of two that puts
    // its maximum in [2^14, 2^15); returns that exponent.  Also stores the
    // head's x exponent for the chunk-scan step.
    auto stage = [&](int b, int h) -> int {
        float mx = 0.f, mxr = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) { mx = fmaxf(mx, s_red[b][w][0]); mxr = fmaxf(mxr, s_red[b][w][1]); }
        const int sx = f16_scale_exponent(mx);
        p.xexp[(int64_t)c * p.H + h] = f16_scale_exponent(mxr);  // the same value from every thread
        const float xs = ldexpf(1.0f, sx);
#pragma unroll
        for (int k = 0; k < PPT; ++k) {
            const int row = pp * PPT + k;
            // token pair `pair` sits in 16-byte chunk pair/4 of the row
            s_xt[b][row * XT_STRIDE + swz(row, (pair >> 2) << 2) + (pair & 3)] =
                pack_f16x2(xv[0][k] * xs, xv[1][k] * xs);
        }
        return sx;
    };

    // the first head's inputs are in flight while the B^T fragments are prepared
    load_head(h_first);

    // ---- B^T fragments of n tile nt: row n = 32 nt + l32, tokens 16 k + 8 hl .. +8,
    // as fp16 scaled by 2^sb (sb: this n tile's exponent)
    u32x4 bq[16];
    int sb;
    {
        // lane: token (lane / 4) + 16 s, 16-byte chunk lane % 4 of the tile's 64 bytes
        const int64_t rstride = (int64_t)p.G * N;
        const uint16_t *bcol = p.B + (t0 * p.G + g) * N + 32 * nt + 8 * (lane & 3);
        u32x4 raw[16];
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2) {
            const int j = (lane >> 2) + 16 * s2;
            raw[s2] = *reinterpret_cast<const u32x4 *>(bcol + min(j, len - 1) * rstride);
            if (j >= len) raw[s2] = u32x4{};
        }
        uint32_t m = 0;
#pragma unroll
        for (int s2 = 0; s2 < 16; ++s2)
#pragma unroll
            for (int k = 0; k < 4; ++k) m = max(m, max(raw[s2][k] & 0x7FFFu, (raw[s2][k] >> 16) & 0x7FFFu));
        sb = f16_scale_exponent(wave_max(__uint_as_float(m << 16)));
        const float bs = ldexpf(1.0f, sb);
        uint32_t *reg = s_b[wave];
        const uint16_t *reg16 = reinterpret_cast<const uint16_t *>(reg);
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            // rows = tokens 128 half .. +128 (wavefront-private region; LDS
            // accesses of one wavefront complete in order)
#pragma unroll
            for (int s2 = 0; s2 < 8; ++s2)
                *reinterpret_cast<u32x4 *>(reg + ((lane >> 2) + 16 * s2) * BR + 4 * (lane & 3)) = raw[8 * half + s2];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const int r0 = 16 * k + 8 * hl;  // local row of the fragment's first token
                u32x4 f;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const uint32_t lo = reg16[(r0 + 2 * q) * 2 * BR + l32];
                    const uint32_t hi = reg16[(r0 + 2 * q + 1) * 2 * BR + l32];
                    f[q] = pack_f16x2(__uint_as_float(lo << 16) * bs, __uint_as_float(hi << 16) * bs);
                }
                bq[8 * half + k] = f;
            }
        }
    }

    // ---- prologue: head 0 weighed and staged, head 1 in flight
    weigh(0);
    load_head(min(h_first + 1, h_last));
    __syncthreads();
    int sx = stage(0, h_first);
    __syncthreads();

#pragma unroll
    for (int hh = 0; hh < HB; ++hh) {
        const int h = h_first + hh;
        const int b = hh & 1;
#pragma unroll
        for (int k = 0; k < 16; ++k) asm volatile("" : "+v"(bq[k]));
        // this head's prefetched inputs are first touched here: otherwise the
        // scheduler hoists their unpacking into the previous head, right
        // behind the loads, and the wait for them stalls that head
#pragma unroll
        for (int e = 0; e < 2; ++e) {
#pragma unroll
            for (int v = 0; v < XV; ++v) asm volatile("" : "+v"(xr[e][v]));
            asm volatile("" : "+v"(cs_tok[e]), "+v"(dt_tok[e]));
        }
        asm volatile("" : "+v"(cs_last));

        // ======== A(hh): S^T tiles of head hh (rows n of tile nt, columns p of
        // tiles pt0..); all 16 K-steps: both operands are zero past the chunk end
        f32x16 acc[PTW];
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            const f16x8 bf = __builtin_bit_cast(f16x8, bq[k]);
#pragma unroll
            for (int u = 0; u < PTW; ++u) {
                const int xrow = (pt0 + u) * 32 + l32;
                const f16x8 xf = __builtin_bit_cast(f16x8, *reinterpret_cast<const u32x4 *>(
                    s_xt[b] + xrow * XT_STRIDE + swz(xrow, 8 * k + 4 * hl)));
                acc[u] = mfma32_f16(bf, xf, k == 0 ? f32x16{} : acc[u]);
            }
        }
        // meanwhile: the next head weighed, the one after it in flight
        weigh(b ^ 1);
        load_head(min(h + 2, h_last));
        __syncthreads();  // x^T of head hh is no longer read; s_red[b ^ 1] complete

        // ======== B(hh): stage the next head, store S of this one
        const int sx_next = stage(b ^ 1, min(h + 1, h_last));
        // S[c][h][p][n] as fp16, one power-of-two exponent per tile: the
        // accumulator is 2^(sx+sb) S; rescale so that the tile's max |S|
        // lands in [2^14, 2^15) (relative rounding 2^-11 per element)
        uint16_t *dst = p.states + ((int64_t)c * p.H + h) * kHeadDim * N;
        int32_t *sexp = p.sexp + ((int64_t)c * p.H + h) * 2 * S::NT;
#pragma unroll
        for (int u = 0; u < PTW; ++u) {
            float am = 0.f;
#pragma unroll
            for (int e = 0; e < 16; ++e) am = fmaxf(am, fabsf(acc[u][e]));
            am = wave_max(am);
            const int se = f16_scale_exponent(am);  // stored S = 2^se * acc = 2^(se + sx + sb) S
            const float rescale = ldexpf(1.0f, se);
            const int pt = pt0 + u;
            // every lane stores the same value: no branch, so the compiler
            // counts this store on every path and its waits stay exact
            sexp[pt * S::NT + nt] = se + sx + sb;
            // lane l holds n = 8a + 4(l/32) + 0..3 of row p; per pair of groups
            // (a, a+1) a v_permlane32_swap per dword gives lanes l and l+32
            // 8 consecutive n each: one 16-byte store, 32 contiguous bytes per row
            uint16_t *row = dst + (int64_t)(pt * 32 + l32) * N + nt * 32 + 8 * hl;
#pragma unroll
            for (int a = 0; a < 4; a += 2) {
                const uint32_t a0 = pack_f16x2(acc[u][4 * a] * rescale, acc[u][4 * a + 1] * rescale);
                const uint32_t a1 = pack_f16x2(acc[u][4 * a + 2] * rescale, acc[u][4 * a + 3] * rescale);
                const uint32_t b0 = pack_f16x2(acc[u][4 * a + 4] * rescale, acc[u][4 * a + 5] * rescale);
                const uint32_t b1 = pack_f16x2(acc[u][4 * a + 6] * rescale, acc[u][4 * a + 7] * rescale);
                const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                *reinterpret_cast<u32x4 *>(row + 8 * a) = u32x4{s0[0], s1[0], s0[1], s1[1]};
            }
        }
        sx = sx_next;
        __syncthreads();  // x^T of the next head complete
    }
}

// Heads per workgroup: the largest of 16, 8, 4, 2, 1 that divides the heads of
// a group and still gives at least one workgroup per compute unit (a workgroup
// fills a compute unit; more heads per workgroup amortise its shared
// operands).
static int state_heads_per_block(const Params &p) {
    const int hg = p.H / p.G;
    const int64_t chunks = (p.nchunks_grid + 7) / 8 * 8;
    for (int hb = 16; hb > 1; hb /= 2)
        if (hg % hb == 0 && chunks * (p.H / hb) >= (int64_t)p.num_cus) return hb;
    return 1;
}

template <int N, int HB>
static hipError_t launch_nh(const Params &p, const Launch &l) {
    const int64_t slots = (p.nchunks_grid + 7) / 8 * (p.H / HB);
    return launch_kernel(ssd_chunk_state_kernel<N, HB>, dim3((unsigned)(slots * 8)), dim3(StateShape<N>::THREADS), l,
                         p);
}

template <int N>
static hipError_t launch_n(const Params &p, const Launch &l) {
    switch (state_heads_per_block(p)) {
    case 16: return launch_nh<N, 16>(p, l);
    case 8: return launch_nh<N, 8>(p, l);
    case 4: return launch_nh<N, 4>(p, l);
    case 2: return launch_nh<N, 2>(p, l);
    default: return launch_nh<N, 1>(p, l);
    }
}

hipError_t launch_chunk_state(const Params &p, const Launch &l) {
    switch (p.N) {
    case 64: return launch_n<64>(p, l);
    case 128: return launch_n<128>(p, l);
    case 256: return launch_n<256>(p, l);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
