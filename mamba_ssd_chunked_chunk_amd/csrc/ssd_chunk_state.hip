// Step 1 of the scan for the chunked sequences: each chunk's own state
// contribution ("chunk_state"),
//   S_k[p][n] = sum_j exp2(cs2_last - cs2_j) dts_j x[t0+j,h,p] B[t0+j,g,n]
// for chunk k (tokens t0 .. t0+len-1) of head h, group g, with dts and
// cs2 = log2(e) * cumsum(A dts) of the chunk from the prep step.  This is the
// per-token recurrence of "mamba2_ssd_scan" ("Per-token recurrence") summed
// over one chunk from a zero state: each token's B x, decayed to the chunk
// end; the "inter-chunk state" of "Mamba chunk scan with segsum"
// (description) is built from these by the state-passing step.  The scale of
// each chunk's x for the chunk-scan step (xexp) is written here too.
//
// Work split.  One workgroup per (chunk, block of HB heads of one group); no
// chunk waits for another.  Sixteen wavefronts in two roles:
//   - consumers (wavefronts 0-7): wavefront w owns n tile w (dstate 256), or
//     n tile w/2 and p tile w%2 (dstate 128, 64; at 64 only wavefronts 0-3).
//     Its B^T operands, formed once per chunk and group by the prep step,
//     are loaded into registers once and serve all HB heads.  Per head, each
//     S^T tile is 16 v_mfma_f32_32x32x16_f16 over the chunk's 256 tokens
//     (fp32 accumulate), stored as fp16.
//   - producers (wavefronts 8-15): load each head's x and the dts and cs2 of
//     its tokens two heads ahead, form the token weights
//     w_j = exp2(cs2_last - cs2_j) dts_j and the maxima of |w| and |x| one
//     head ahead, and stage (w x)^T into one of two LDS buffers as fp16 under
//     the power of two that puts max|w| max|x| in [2^14, 2^15).
// One barrier per head: while the consumers multiply head k-1 out of one
// buffer (and store head k-2), the producers stage head k into the other, so
// the vector work of the staging and the matrix products overlap.
// Workgroups are numbered so that all head blocks of a chunk land on one XCD
// (dispatch is round-robin over the 8 XCDs) and share the chunk's B operands
// in its L2.
// Output: S as fp16 in [chunk][head][p][n], each 32x32 tile under the power
// of two that puts its max |S| in [2^14, 2^15) (sexp).  The tiles go through
// a double-buffered LDS area and are stored one phase later as whole rows
// (16 bytes per lane, N/8 lanes per row): stores of a tile's 32 rows x 64
// bytes straight from the MFMA layout touch 32 cache lines per instruction
// and took about twice as long for the same bytes.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kConsumers = 8;
constexpr int kProducers = 8;
constexpr int kThreads = 64 * (kConsumers + kProducers);
// dwords per staged row: 128 token pairs + pad.  LDS serves 4-byte accesses
// 32 lanes at a time over 32 banks and 8-byte accesses 32 lanes at a time
// over 64 banks.  At this stride the MFMA operand reads (8 bytes, rows 0..31
// of one column) fall on distinct bank pairs, and so do the staging stores
// (4 bytes, rows 8v + i and 8v + 8 + i for 16 consecutive pairs each, the
// two rows 16 banks apart).
constexpr int XT_STRIDE = 130;

// dwords per row of the S staging area: N/2 (N fp16) + 2.  The consumers'
// 8-byte writes (rows 0..31 of one column per 32 lanes) then fall on distinct
// bank pairs, and the 16-byte reads for the stores are contiguous in a row.
template <int N>
struct SStride {
    static constexpr int value = N / 2 + 2;
};

template <int N>
struct __attribute__((aligned(16))) StateSmem {
    uint32_t xt[2][kHeadDim * XT_STRIDE];             // (w x)^T 2^sx: row p, fp16 token pairs; head k in buffer k & 1
    uint32_t sbuf[2][kHeadDim * SStride<N>::value];   // S of head k (fp16, per-tile scales), row p, in buffer k & 1
    float red[2][3][kProducers];                      // per producer wavefront: max |w|, max |x| over p < 32, over p >= 32
    int sx[2];                                        // scale exponent of the head in buffer b
};

// A producer thread's inputs of one head: x at token pairs pq + 64 it (two
// tokens each, 8 p), the chunk's cs2 and dts at those tokens and its last
// cs2; once analysed, the tokens' weights
struct HeadIn {
    u32x4 x[2][2];
    float2 cs[2], dt[2], w[2];
    float clast;
};

// threadIdx.x behind an empty asm: indices derived from it are recomputed
// where they are used instead of being held across the head loop
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}
}  // namespace

template <int N, int HB>
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(Params p) {
    constexpr int NT = N / 32;
    constexpr int TPW = N == 256 ? 2 : 1;  // p tiles per consumer wavefront
    __shared__ StateSmem<N> sm;

    // ---- XCD-aware decode: all head blocks of chunk c share one XCD
    const int nhb = p.H / HB;
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / nhb) * 8 + xcd;
    const int h_first = (slot - (slot / nhb) * nhb) * HB;
    if (c >= p.meta[0]) return;  // past the call's chunks (uniform)
    const int g = h_first / (p.H / p.G);
    const int4 dsc = p.desc[c];
    const int64_t t0 = dsc.y;
    const int len = dsc.z;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= kConsumers;  // wavefront-uniform
    // phases 0 .. HB+1 (products of head j-1 and stores of head j-2 in phase
    // j), rounded up to pairs
    constexpr int kPhases = (HB + 3) & ~1;

    // Phase j (j = 0 .. kPhases-1, in pairs so that the two register sets of
    // each role alternate at compile time): producers stage head j into
    // buffer j & 1 and analyse head j+1 (past the last head they repeat it);
    // consumers store head j-2 and multiply head j-1.  Each role runs its own
    // loop with the same barriers (one per phase, after a prologue barrier).
    if (producer) {
        const int pw = wave - kConsumers;  // producer wavefront 0 .. 7
        // thread t: p = 8 pv .. 8 pv + 7 of token pairs pq + 64 it, so that
        // each 32-lane half of a wavefront stages 16 consecutive pairs of two
        // rows 8 apart (distinct banks, see XT_STRIDE)
        auto coords = [&](int &pv, int &pq) {
            const int t = opaque_tid() - 64 * kConsumers;
            pv = (t & 1) | (((t >> 5) & 3) << 1);
            pq = ((t >> 1) & 15) | ((t >> 7) << 4);
        };
        // a head's inputs (past the last head: the last again; rows past the
        // chunk end repeat its last row, their dts is 0)
        auto load_head = [&](int hh, HeadIn &o) {
            const int h = h_first + min(hh, HB - 1);
            int pv, pq;
            coords(pv, pq);
            const int64_t r = ((int64_t)c * p.H + h) * kChunk;
            const uint32_t xrow = (uint32_t)p.H * kHeadDim * 2;  // bytes between tokens of x
            const char *xb = reinterpret_cast<const char *>(p.x + (t0 * p.H + h) * kHeadDim + 8 * pv);
#pragma unroll
            for (int it = 0; it < 2; ++it) {
#pragma unroll
                for (int e = 0; e < 2; ++e) {
                    const uint32_t j = (uint32_t)min(2 * (pq + 64 * it) + e, len - 1);
                    o.x[it][e] = *reinterpret_cast<const u32x4 *>(xb + j * xrow);
                }
                o.cs[it] = *reinterpret_cast<const float2 *>(p.cs2 + r + 2 * (pq + 64 * it));
                o.dt[it] = *reinterpret_cast<const float2 *>(p.dts + r + 2 * (pq + 64 * it));
            }
            o.clast = p.cs2[r + kChunk - 1 + min(opaque_tid(), 0)];  // a vector load (in-order waits)
        };
        // the token weights and the wavefront maxima of head hh into slot s2
        auto analyze = [&](HeadIn &o, int s2) {
            int pv, pq;
            coords(pv, pq);
            float wm = 0.0f;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                o.w[it].x = fast_exp2(o.clast - o.cs[it].x) * o.dt[it].x;
                o.w[it].y = fast_exp2(o.clast - o.cs[it].y) * o.dt[it].y;
                wm = fmaxf(wm, fmaxf(fabsf(o.w[it].x), fabsf(o.w[it].y)));
            }
            u16x2 mx2 = u16x2{0, 0};
#pragma unroll
            for (int it = 0; it < 2; ++it)
#pragma unroll
                for (int e = 0; e < 2; ++e)
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, o.x[it][e][q] & 0x7FFF7FFFu));
            const float mx = __uint_as_float(max((uint32_t)mx2[0], (uint32_t)mx2[1]) << 16);
            const float w_all = wave_max(wm);
            const float m0 = wave_max(pv < 4 ? mx : 0.0f);
            const float m1 = wave_max(pv < 4 ? 0.0f : mx);
            sm.red[s2][0][pw] = w_all;  // the same value from every lane
            sm.red[s2][1][pw] = m0;
            sm.red[s2][2][pw] = m1;
        };
        // head hh (analysed into slot s2) staged into buffer s2
        auto stage = [&](int hh, int s2, const HeadIn &o) {
            const int h = h_first + min(hh, HB - 1);
            float wmax = 0.0f, xm0 = 0.0f, xm1 = 0.0f;
#pragma unroll
            for (int v = 0; v < kProducers; ++v) {
                wmax = fmaxf(wmax, sm.red[s2][0][v]);
                xm0 = fmaxf(xm0, sm.red[s2][1][v]);
                xm1 = fmaxf(xm1, sm.red[s2][2][v]);
            }
            // the chunk-scan step stages x under the power of two of the
            // chunk's max |x| over each half of p (kNoExponent for an all-zero
            // half); every lane stores one of the two (the same value per
            // address)
            {
                const int t = opaque_tid();
                const float m = (t & 1) ? xm1 : xm0;
                p.xexp[((int64_t)c * p.H + h) * 2 + (t & 1)] = m > 0.0f ? f16_scale_exponent(m) : kNoExponent;
            }
            // |w x| <= max|w| max|x|: that bound's power of two keeps every
            // staged value below 2^15
            const int sx = f16_scale_exponent(wmax * fmaxf(xm0, xm1));
            sm.sx[s2] = sx;  // the same value from every lane
            const float xs = ldexpf(1.0f, sx);
            int pv, pq;
            coords(pv, pq);
            // rows 8 pv + i, pairs pq + 64 it: every store is this thread's
            // base plus a constant
            uint32_t *xt = sm.xt[s2] + 8 * pv * XT_STRIDE + pq;
#pragma unroll
            for (int it = 0; it < 2; ++it) {
                const float wx0 = o.w[it].x * xs, wx1 = o.w[it].y * xs;
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint32_t a0 = o.x[it][0][i >> 1], a1 = o.x[it][1][i >> 1];
                    const bool hi = i & 1;
                    xt[i * XT_STRIDE + 64 * it] = pack_f16x2((hi ? bf16x2_hi(a0) : bf16x2_lo(a0)) * wx0,
                                                             (hi ? bf16x2_hi(a1) : bf16x2_lo(a1)) * wx1);
                }
            }
        };
        // No branch in the phases: past the last head the work repeats it
        // (same values into the slot and buffer of the phase's parity, which
        // no consumer reads any more), so the loads in flight are never waited
        // for early.
        HeadIn r0, r1;
        load_head(0, r0);
        load_head(1, r1);
        analyze(r0, 0);
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < kPhases; j += 2) {
            stage(j, 0, r0);
            __builtin_amdgcn_sched_barrier(0);
            load_head(j + 2, r0);
            __builtin_amdgcn_sched_barrier(0);
            analyze(r1, 1);
            __syncthreads();
            stage(j + 1, 1, r1);
            __builtin_amdgcn_sched_barrier(0);
            load_head(j + 3, r1);
            __builtin_amdgcn_sched_barrier(0);
            analyze(r0, 0);
            __syncthreads();
        }
    } else {
        // this wavefront's n tile and first p tile
        const int nt = N == 256 ? wave : wave >> 1;
        const int pt0 = N == 256 ? 0 : wave & 1;
        const bool mma = wave < 2 * NT || N == 256;  // wavefront-uniform: at dstate 64, wavefronts 0-3
        // ---- B^T operands of the wavefront's n tile: K-step s, this lane
        u32x4 fr[16];
        int sb = 0;
        if (mma) {
            const int64_t tile = ((int64_t)c * p.G + g) * NT + nt;
            const u32x4 *src = reinterpret_cast<const u32x4 *>(p.bfrag) + tile * 1024 + lane;
#pragma unroll
            for (int s = 0; s < 16; ++s) fr[s] = src[64 * s];
            sb = p.bexp[tile];
        }
        // head hh's S^T tiles out of buffer hh & 1: rows n (32 nt ..), columns
        // p (32 pt ..); lane l holds p = 32 pt + l % 32, n = 32 nt + 8a + 4(l/32) + 0..3
        auto multiply = [&](int hh) {
            const int h = h_first + hh;
            const int b = hh & 1;
            const int sx = sm.sx[b];
#pragma unroll
            for (int tp = 0; tp < TPW; ++tp) {
                const int pt = pt0 + tp;
                const int t = opaque_tid();
                const int r = 32 * pt + (t & 31);
                const int hl = (t >> 5) & 1;
                // the lane's 8 tokens of K-step ks: pairs 8 ks + 4 hl .. +3, two 8-byte reads
                const u32x2 *brow = reinterpret_cast<const u32x2 *>(sm.xt[b] + r * XT_STRIDE + 4 * hl);
                auto operand = [&](int ks) {
                    const u32x2 a = brow[4 * ks], bb = brow[4 * ks + 1];
                    return u32x4{a[0], a[1], bb[0], bb[1]};
                };
                // (w x)^T operands read kPre K-steps ahead of their products
                constexpr int kPre = 4;
                u32x4 bq[kPre];
#pragma unroll
                for (int ks = 0; ks < kPre; ++ks) bq[ks] = operand(ks);
                f32x16 acc;
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) {
                    const f16x8 bf = __builtin_bit_cast(f16x8, bq[ks % kPre]);
                    if (ks + kPre < 16) bq[ks % kPre] = operand(ks + kPre);
                    // keeps the reads ahead (the scheduler would sink them to their use)
                    __builtin_amdgcn_sched_barrier(0);
                    acc = mfma32_f16(__builtin_bit_cast(f16x8, fr[ks]), bf, ks == 0 ? f32x16{} : acc);
                }
                // acc = 2^(sx + sb) S.  The tile is stored as fp16 times 2^se,
                // with se putting the tile's max |S| in [2^14, 2^15): acc is
                // scaled by 2^(se - sx - sb) = 2^f16_scale_exponent(max |acc|)
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(acc[e]));
                m = wave_max(m);
                const int ea = f16_scale_exponent(m);
                // every lane: the same value
                p.sexp[(((int64_t)c * p.H + h) * 2 + pt) * NT + nt] = ea + sx + sb;
                const float as = ldexpf(1.0f, ea);
                // into the staging area: lane l holds n = 32 nt + 8a + 4(l/32)
                // + 0..3 of row p, one 8-byte write per a
                uint32_t *srow = sm.sbuf[b] + r * SStride<N>::value + 16 * nt + 2 * hl;
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<u32x2 *>(srow + 4 * a) =
                        u32x2{pack_f16x2(acc[4 * a] * as, acc[4 * a + 1] * as),
                              pack_f16x2(acc[4 * a + 2] * as, acc[4 * a + 3] * as)};
            }
        };
        // head hh's S out of staging buffer hh & 1 into [chunk][head][p][n]:
        // N/8 lanes per row, 16 bytes each, so every store instruction writes
        // whole rows (8 rows per wavefront)
        auto store_s = [&](int hh) {
            constexpr int LPR = N / 8;            // lanes per row
            constexpr int RPI = 64 / LPR;         // rows per instruction
            const int h = h_first + hh;
            const int t = opaque_tid();
            const int l = t & 63;
            const int rr = l / LPR, ch = l % LPR;
#pragma unroll
            for (int i = 0; i < 8 / RPI; ++i) {
                const int row = 8 * wave + RPI * i + rr;
                const u32x4 v = *reinterpret_cast<const u32x4 *>(sm.sbuf[hh & 1] + row * SStride<N>::value + 4 * ch);
                *reinterpret_cast<u32x4 *>(p.states + (((int64_t)c * p.H + h) * kHeadDim + row) * N + 8 * ch) = v;
            }
        };
        // phase j: the stores of head j-2, then the products of head j-1
        // (their staging buffer is the other one); the stores of the last head
        // run in phase HB+1
        auto phase = [&](int j) {
            if (j >= 2 && j - 2 < HB) store_s(j - 2);
            if (mma && j >= 1 && j - 1 < HB) multiply(j - 1);
        };
        __syncthreads();
#pragma unroll 1
        for (int j = 0; j < kPhases; j += 2) {
            phase(j);
            __syncthreads();
            phase(j + 1);
            __syncthreads();
        }
    }
}

// Heads per workgroup: the largest of 16, 8, 4, 2, 1 that divides the heads
// of a group and still gives at least one workgroup per compute unit (the B
// operands are fetched once per workgroup, and its phases overlap staging
// and products: more heads per workgroup do both better).
static int state_heads_per_block(const Params &p) {
    const int hg = p.H / p.G;
    const int64_t chunks = (p.nchunks_grid + 7) / 8 * 8;
    for (int hb = 16; hb > 1; hb /= 2)
        if (hg % hb == 0 && chunks * (p.H / hb) >= (int64_t)p.num_cus) return hb;
    return 1;
}

template <int N, int HB>
static hipError_t launch_nh(const Params &p, const Launch &l) {
    const dim3 grid((unsigned)((p.nchunks_grid + 7) / 8 * (p.H / HB) * 8));
    return launch_kernel(ssd_chunk_state_kernel<N, HB>, grid, dim3(kThreads), l, p);
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
