// Steps 1-3 and 5 of the scan for the chunked sequences: each chunk's own
// state contribution ("chunk_state"), the inter-chunk recurrence
// ("state_passing") and the final-state write, fused into one walk per
// sequence, so that neither the chunk contributions nor the chain ever leave
// the compute unit.  Only what the output step needs is written: the state
// entering every chunk (h_in), the scale of each chunk's x and, at the end,
// the final state.
//
// For sequence b, head h with group g and chunk k (tokens t0 .. t0+len-1),
// with dts and cs2 = log2(e) * cumsum(A dts) of the chunk (from the prep
// step):
//   S_k[p][n]  = sum_j exp2(cs2_last - cs2_j) dts_j x[t0+j,h,p] B[t0+j,g,n]
//   h_in[0]    = initial ? state_in[slot][h] : 0
//   h_in[k+1]  = exp2(cs2_last(k)) h_in[k] + S_k
//   state_out[slot][h] = h_in[K]                       (K = the sequence's chunks)
// S_k is the per-token recurrence of "mamba2_ssd_scan" ("Per-token
// recurrence") unrolled over one chunk from a zero state; the chain is the
// "inter-chunk state recurrence with exponential decay" of "Mamba chunk scan
// with segsum" (description).  The reset at each sequence start (to zero or
// the initial state) and the final state at each sequence end are
// "mamba2_ssd_scan" (the paragraph after "Per-token recurrence"); reading the
// initial state from, and writing the final state to, slot cache_indices[b]
// of the pool is "Mamba2SSDChunkScanVarlenFwdInplace" (struct description).
// A sequence with no tokens writes its initial state (or zeros) back.
//
// Work split.  A work item is (sequence, head, half of p, NW dstate columns,
// NW = min(dstate, 128)): its 32 x NW block of the state is independent of
// every other block.  One workgroup walks the item's chunks in order, in two
// roles:
//   - consumers (wavefronts 0 .. NW/32 - 1): wavefront w owns the 32 x 32
//     state tile (the item's p half, n tile w of its columns) and keeps it in
//     fp32 registers for the whole sequence, in the layout of the MFMA
//     accumulator, so the chain update is elementwise on the tile the
//     products leave behind.  Per chunk: S^T tile = B^T (w x) over the
//     chunk's 256 tokens on v_mfma_f32_32x32x16_f16 (fp32 accumulate), with
//     the B^T operands loaded straight into registers, two chunks ahead, in
//     the operand order the prep step wrote them in (once per chunk and
//     group, not once per head); state = exp2(cs2_last) state + S; h_in of
//     the next chunk stored (fp16, one power-of-two exponent per 32 x 32
//     tile).
//   - producers (the next four wavefronts): load the item's half rows of x
//     and the chunk's dts and cs2 two chunks ahead, form the token weights
//     w_j = exp2(cs2_last - cs2_j) dts_j and reduce the maxima of |x| and |w|
//     one chunk ahead, and stage (w x)^T as fp16 under a power-of-two
//     scaling into one of two LDS buffers.
// One barrier per chunk: while the consumers multiply chunk k-1 out of one
// buffer, the producers stage chunk k into the other.  Items are numbered so
// that all items of one (sequence, head) land on one XCD (workgroup ids are
// dealt to the eight XCDs round-robin) and share the x rows they read in its
// L2; the heads of a sequence and group go to an XCD in blocks, as large as
// still gives every XCD two blocks, so the B operands that all heads of the
// group read are fetched into few L2s.
// Precision: w x and B are rounded to fp16 (11-bit significand) after scaling
// their maxima (per chunk and item; per chunk, group and 32 columns) into
// [2^14, 2^15); the chain is fp32; h_in is rounded to fp16 once (it only
// feeds y).
#include <algorithm>

#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int XT_STRIDE = 132;  // dwords per staged row: 128 token pairs + pad

// dword index of column `col` (a token pair) of staged row r (0 .. 31): rows
// 16 .. 31 swap their 16-pair halves of each 32 pairs.  With the 132-dword
// row stride (4 banks apart, of 64), the MFMA operand reads (16 consecutive
// rows per pass, one 16-byte chunk each, the same chunk in every row) fall
// on distinct banks, and so do the staging stores (row groups 0, 8, 16, 24
// of one instruction, 16 consecutive pairs each), which without the swap
// would meet in pairs (8 rows are 32 banks apart)
__device__ __forceinline__ int swz(int r, int col) { return col ^ (((r >> 4) & 1) << 4); }

template <int N>
struct ChainShape {
    static constexpr int NW = N < 128 ? N : 128;  // dstate columns per item
    static constexpr int CW = NW / 32;            // consumer wavefronts (n tiles per item)
    static constexpr int NS = N / NW;             // column splits of a head
    static constexpr int THREADS = 64 * (CW + 4);
};

struct __attribute__((aligned(16))) ChainSmem {
    uint32_t xt[2][32 * XT_STRIDE];  // (w x)^T 2^sx of the item's p half: row p, fp16 token pairs
    float xm[2][4], wm[2][4];        // producer wavefront maxima of |x| and of |w|
    int sx[2];                       // scale exponent of the chunk in buffer b
};

// A producer lane's inputs of one chunk: x at token pairs pq, pq + 64 (two
// tokens each), the chunk's cs2 and dts at those tokens, its last cs2, and
// (once analysed) the tokens' weights w_j = exp2(cs2_last - cs2_j) dts_j
struct Raw {
    u32x4 x[2][2];
    float2 cs[2], dt[2], w[2];
    float clast;
};

// threadIdx.x behind an empty asm: indices derived from it are recomputed
// where they are used instead of being hoisted out of the chunk loop and
// held (they would need more registers than the pipeline has)
__device__ __forceinline__ int opaque_tid() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    return t;
}

// Zero that the compiler cannot prove uniform: a load of a uniform address
// indexed with it stays a vector load.  Vector loads complete in order, so a
// wait for an older one leaves the newer ones in flight; scalar loads
// complete out of order, so waiting for any of them waits for all, including
// the prefetches issued just before.
__device__ __forceinline__ int lane_zero() { return min(opaque_tid(), 0); }
}  // namespace

// One item: sequence b, head h, p half ph, dstate columns NW ns .. NW ns + NW - 1.
template <int N, bool SB>
__device__ __forceinline__ void chain_item(const Params &p, ChainSmem &sm, int b, int h, int ph, int ns) {
    using S = ChainShape<N>;
    constexpr int NT = N / 32;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= S::CW;  // wavefront-uniform
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    const int nt = ns * S::CW + (producer ? 0 : wave);  // consumers: n tile of the state tile

    // chunk rows of the sequence, clamped to the tables so that a malformed
    // query_start_loc cannot index past them
    const int k1 = (int)min((int64_t)p.chunk_off[b + 1], p.nchunks_max);
    const int k0 = min(p.chunk_off[b], k1);
    const int nk = k1 - k0;
    const int64_t ts = p.qsl[b];
    const int len_b = (int)(p.qsl[b + 1] - ts);
    const int64_t slot = p.cache_idx != nullptr ? (int64_t)p.cache_idx[b] : (int64_t)b;
    const bool init = p.init_all != 0 || (p.has_init != nullptr && p.has_init[b] != 0);
    const int g = h / (p.H / p.G);

    // consumers: this lane's state elements, p = 32 ph + l32, n = 32 nt + 8a + 4 hl + e
    const int64_t soff = ((slot * p.H + h) * kHeadDim + 32 * ph + l32) * N + 32 * nt + 4 * hl;
    float st[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) st[e] = 0.0f;
    if (!producer && init) {
        // state_in is null only when no sequence reads it
        const void *src = p.state_in != nullptr ? p.state_in : p.state_out;
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            const f32x4 v = load_state4<SB>(src, soff + 8 * a);
#pragma unroll
            for (int e = 0; e < 4; ++e) st[4 * a + e] = v[e];
        }
    }

    // Phase j (j = 0 .. nk, and one more when nk is even, so that phases come
    // in pairs and the two register sets of each role alternate at compile
    // time): producers stage chunk j into buffer j & 1 and analyse chunk j+1;
    // consumers multiply chunk j-1 and store h_in of chunk j.  Each role runs
    // its own loop with the same barriers (one per phase, after a prologue
    // barrier): the roles are wavefront-uniform, and no register of one role
    // crosses a join with the other's code.
    if (nk > 0) {  // uniform over the workgroup
        auto chunk_len = [&](int k) { return min(kChunk, len_b - kChunk * k); };

        if (producer) {
            const int pw = wave - S::CW;  // producer wavefront 0 .. 3
            const uint32_t xrow = (uint32_t)p.H * kHeadDim * 2;  // bytes between tokens of x
            // raw inputs of chunk k: token pair pq + 64 it (pq = t / 4), token e
            // of the pair, 16-byte piece t % 4 of the half row; the chunk's
            // dts and cs2 at those tokens (from the prep step) and its last
            // cs2.  A base per chunk that is the same in every lane (scalar
            // registers) plus a 32-bit byte offset per lane, so no 64-bit
            // address per load is kept across the loop.  Rows past the chunk
            // end repeat its last row (their dts is 0).
            auto load_raw = [&](int k, Raw &o) {
                const int t = opaque_tid() - 64 * S::CW;
                const int pv = t & 3, pq = t >> 2;
                const int kk = min(k, nk - 1);
                const int64_t t0 = ts + (int64_t)kChunk * kk;
                const int len = chunk_len(kk);
                const char *xb = reinterpret_cast<const char *>(p.x + (t0 * p.H + h) * kHeadDim + 32 * ph);
                const int64_t r = ((k0 + kk) * (int64_t)p.H + h) * kChunk;
#pragma unroll
                for (int it = 0; it < 2; ++it) {
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const uint32_t tok = (uint32_t)min(2 * (pq + 64 * it) + e, len - 1);
                        o.x[it][e] = *reinterpret_cast<const u32x4 *>(xb + (tok * xrow + 16u * pv));
                    }
                    o.cs[it] = *reinterpret_cast<const float2 *>(p.cs2 + r + 2 * (pq + 64 * it));
                    o.dt[it] = *reinterpret_cast<const float2 *>(p.dts + r + 2 * (pq + 64 * it));
                }
                o.clast = p.cs2[r + kChunk - 1 + lane_zero()];
            };
            // chunk k analysed into slot s2: the token weights of this lane's
            // tokens (kept for the staging) and the wavefront maxima of |x|
            // and of |w|
            auto analyze = [&](Raw &o, int s2) {
                u16x2 mx2 = u16x2{0, 0};
#pragma unroll
                for (int it = 0; it < 2; ++it)
#pragma unroll
                    for (int e = 0; e < 2; ++e)
#pragma unroll
                        for (int w = 0; w < 4; ++w)
                            mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, o.x[it][e][w] & 0x7FFF7FFFu));
                float wm = 0.0f;
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    o.w[it].x = fast_exp2(o.clast - o.cs[it].x) * o.dt[it].x;
                    o.w[it].y = fast_exp2(o.clast - o.cs[it].y) * o.dt[it].y;
                    wm = fmaxf(wm, fmaxf(fabsf(o.w[it].x), fabsf(o.w[it].y)));
                }
                sm.xm[s2][pw] = wave_max(__uint_as_float(max((uint32_t)mx2[0], (uint32_t)mx2[1]) << 16));
                sm.wm[s2][pw] = wave_max(wm);
            };
            // chunk k (analysed into slot s2) staged into buffer s2
            auto stage = [&](int k, int s2, const Raw &o) {
                const float mx = fmaxf(fmaxf(sm.xm[s2][0], sm.xm[s2][1]), fmaxf(sm.xm[s2][2], sm.xm[s2][3]));
                const float wmx = fmaxf(fmaxf(sm.wm[s2][0], sm.wm[s2][1]), fmaxf(sm.wm[s2][2], sm.wm[s2][3]));
                // |w x| <= max|w| max|x|: that bound's power of two keeps every
                // staged value below 2^15
                const int sx = f16_scale_exponent(wmx * mx);
                sm.sx[s2] = sx;  // the same value from every lane
                // the chunk-scan step stages x under the power of two of the
                // chunk's max |x| over each half of p (kNoExponent for an
                // all-zero half; every lane of every item of the half stores
                // the same value)
                p.xexp[((k0 + k) * (int64_t)p.H + h) * 2 + ph] = mx > 0.0f ? f16_scale_exponent(mx) : kNoExponent;
                const float xs = ldexpf(1.0f, sx);
                // rows 8 pv + i, pairs pq + 64 it: swz(row, pair) =
                // (pq ^ 16 (pv / 2)) + 64 it, so every store is this lane's base
                // plus a constant
                const int t = opaque_tid() - 64 * S::CW;
                const int pv = t & 3, pq = t >> 2;
                uint32_t *xt = sm.xt[s2] + 8 * pv * XT_STRIDE + (pq ^ ((pv >> 1) << 4));
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
            // No branch in the phases: past the last chunk the work repeats it
            // (same values into the slot and buffer of the phase's parity,
            // which no consumer reads any more), so the loads in flight are
            // never waited for early.
            Raw r0, r1;
            load_raw(0, r0);
            load_raw(1, r1);
            analyze(r0, 0);
            __syncthreads();
#pragma unroll 1
            for (int j = 0; j <= nk; j += 2) {
                stage(min(j, nk - 1), 0, r0);
                __builtin_amdgcn_sched_barrier(0);
                load_raw(j + 2, r0);
                __builtin_amdgcn_sched_barrier(0);
                analyze(r1, 1);
                __syncthreads();
                stage(min(j + 1, nk - 1), 1, r1);
                __builtin_amdgcn_sched_barrier(0);
                load_raw(j + 3, r1);
                __builtin_amdgcn_sched_barrier(0);
                analyze(r0, 0);
                __syncthreads();
            }
        } else {
            // B^T operands of chunk k (this wavefront's n tile, 16 K-steps)
            // and their exponent
            auto load_frag = [&](int k, u32x4 (&fo)[16], int &sbo, float &clo) {
                const int t = opaque_tid();
                const int kk = k0 + min(k, nk - 1);
                const int64_t tile = (kk * (int64_t)p.G + g) * NT + nt;
                const u32x4 *src = reinterpret_cast<const u32x4 *>(p.bfrag) + tile * 1024 + (t & 63);
#pragma unroll
                for (int s = 0; s < 16; ++s) fo[s] = src[64 * s];
                sbo = p.bexp[tile + lane_zero()];
                clo = p.cs2[((int64_t)kk * p.H + h) * kChunk + kChunk - 1 + lane_zero()];
            };
            // chunk k's S^T tile out of buffer k & 1, and the chain step
            auto multiply = [&](int k, const u32x4 (&fi)[16], int sbi, float cli) {
                const int s2 = k & 1;
                const int t = opaque_tid();
                const int r = t & 31, hh = (t >> 5) & 1;
                const uint32_t *brow = sm.xt[s2] + r * XT_STRIDE;
                // (w x)^T operands read kPre K-steps ahead of their products
                constexpr int kPre = 4;
                u32x4 bq[kPre];
#pragma unroll
                for (int ks = 0; ks < kPre; ++ks)
                    bq[ks] = *reinterpret_cast<const u32x4 *>(brow + swz(r, 8 * ks + 4 * hh));
                f32x16 acc;
#pragma unroll
                for (int ks = 0; ks < 16; ++ks) {
                    const f16x8 bf = __builtin_bit_cast(f16x8, bq[ks % kPre]);
                    if (ks + kPre < 16)
                        bq[ks % kPre] = *reinterpret_cast<const u32x4 *>(brow + swz(r, 8 * (ks + kPre) + 4 * hh));
                    // keeps the reads ahead (the scheduler would sink them to their use)
                    __builtin_amdgcn_sched_barrier(0);
                    acc = mfma32_f16(__builtin_bit_cast(f16x8, fi[ks]), bf, ks == 0 ? f32x16{} : acc);
                }
                // acc = 2^(sx + sb) S
                const int su = -(sm.sx[s2] + sbi);
                const float decay = fast_exp2(cli);
#pragma unroll
                for (int e = 0; e < 16; ++e) st[e] = __builtin_fmaf(st[e], decay, ldexpf(acc[e], su));
            };
            // h_in of chunk k, fp16 under the power of two that puts the tile's
            // max |h| in [2^14, 2^15)
            auto store_hin = [&](int k) {
                const int64_t c = k0 + k;
                float m = 0.0f;
#pragma unroll
                for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(st[e]));
                // an all-zero tile takes the largest exponent, so that it never
                // lowers the common exponent chunk_scan gives a 32-row block
                m = wave_max(m);
                const int he = m > 0.0f ? f16_scale_exponent(m) : 126;
                p.hexp[((c * p.H + h) * NT + nt) * 2 + ph] = (int16_t)he;  // every lane: the same value
                const float hs = ldexpf(1.0f, he);
                // lane l holds n = 8a + 4(l/32) + 0..3 of row p; per pair of
                // groups (a, a+1) a v_permlane32_swap per dword gives lanes l
                // and l+32 8 consecutive n each: one 16-byte store, 32
                // contiguous bytes per row
                uint16_t *row = p.hin + ((c * p.H + h) * kHeadDim + 32 * ph + l32) * N + 32 * nt + 8 * hl;
#pragma unroll
                for (int a = 0; a < 4; a += 2) {
                    const uint32_t a0 = pack_f16x2(st[4 * a] * hs, st[4 * a + 1] * hs);
                    const uint32_t a1 = pack_f16x2(st[4 * a + 2] * hs, st[4 * a + 3] * hs);
                    const uint32_t b0 = pack_f16x2(st[4 * a + 4] * hs, st[4 * a + 5] * hs);
                    const uint32_t b1 = pack_f16x2(st[4 * a + 6] * hs, st[4 * a + 7] * hs);
                    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
                    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
                    *reinterpret_cast<u32x4 *>(row + 8 * a) = u32x4{s0[0], s1[0], s0[1], s1[1]};
                }
            };
            // phase j multiplies chunk j-1 with the register set loaded in
            // phase j-2 and reloads it with chunk j+1 (last: the producers'
            // loads of the phase, issued after their staging, then go to the
            // compute unit's memory pipeline ahead of these)
            u32x4 f0[16], f1[16];
            int sb0, sb1;
            float cl0, cl1;
            load_frag(0, f0, sb0, cl0);
            __syncthreads();
#pragma unroll 1
            for (int j = 0; j <= nk; j += 2) {
                if (j >= 1) multiply(j - 1, f1, sb1, cl1);
                if (j < nk) store_hin(j);
                load_frag(j + 1, f1, sb1, cl1);
                __syncthreads();
                if (j + 1 <= nk) multiply(j, f0, sb0, cl0);
                if (j + 1 < nk) store_hin(j + 1);
                load_frag(j + 2, f0, sb0, cl0);
                __syncthreads();
            }
        }
    }
    // ---- the final state into its slot (each element read and written by
    // this same thread, so an in-place slot never races)
    if (!producer) {
#pragma unroll
        for (int a = 0; a < 4; ++a)
            store_state4<SB>(p.state_out, soff + 8 * a, f32x4{st[4 * a], st[4 * a + 1], st[4 * a + 2], st[4 * a + 3]});
    }
}

// Heads per block: the largest divisor of the group's heads, halving, that
// still gives 16 blocks (two per XCD).
__host__ __device__ inline int chain_head_block(int nseq, int H, int G) {
    int hb = H / G;
    while ((hb & 1) == 0 && (int64_t)nseq * (H / hb) < 16) hb >>= 1;
    return hb;
}

// Items (sequence, head, p half, column split), walked grid-stride, in
// blocks of heads of one sequence and group that are dealt to the XCDs
// round-robin (workgroup ids x mod 8 run on XCD x), all items of a block on
// one XCD.  gridDim.x is a multiple of 8, so a workgroup stays on one XCD
// across its items.  LIST: the sequences are those of the list prep wrote (the short
// path is on: only sequences longer than its limit are there), else the
// batch.
template <int N, bool LIST, bool SB>
__global__ __launch_bounds__(ChainShape<N>::THREADS) void ssd_state_chain_kernel(Params p) {
    constexpr int NI = 2 * ChainShape<N>::NS;  // items per (sequence, head)
    __shared__ ChainSmem sm;
    const int nseq = LIST ? p.meta[1] : p.batch;
    const int hb = chain_head_block(nseq, p.H, p.G);
    const int nhb = p.H / hb;                     // head blocks of a sequence
    const int64_t nblk = (int64_t)nseq * nhb;
    const int64_t per_blk = (int64_t)hb * NI;     // items of a block
    const int64_t nid = (nblk + 7) / 8 * per_blk * 8;
#pragma unroll 1
    for (int64_t id = blockIdx.x; id < nid; id += gridDim.x) {
        const int xcd = (int)(id & 7);
        const int64_t sl = id >> 3;
        const int64_t kb = sl / per_blk * 8 + xcd;  // block
        if (kb >= nblk) continue;  // uniform over the workgroup
        const int r = (int)(sl % per_blk);
        const int bi = (int)(kb / nhb);
        const int h = (int)(kb - (int64_t)bi * nhb) * hb + r / NI;
        const int sub = r % NI;
        const int b = LIST ? p.seq_list[bi] : bi;
        chain_item<N, SB>(p, sm, b, h, sub & 1, sub >> 1);
    }
}

template <int N, bool SB>
static hipError_t launch_n(const Params &p, const Launch &l) {
    using S = ChainShape<N>;
    const bool list = p.short_max > 0;
    const int nseq = list ? p.nseq_grid : p.batch;
    const int hb = chain_head_block(nseq, p.H, p.G);
    const int64_t nid = ((int64_t)nseq * (p.H / hb) + 7) / 8 * hb * (2 * S::NS) * 8;
    // a multiple of 8 workgroups, at most 8 per compute unit; past that,
    // workgroups take several items
    const int64_t grid = std::max<int64_t>(8, std::min<int64_t>(nid, (int64_t)p.num_cus * 8));
    const dim3 block(S::THREADS);
    if (list) return launch_kernel(ssd_state_chain_kernel<N, true, SB>, dim3((unsigned)grid), block, l, p);
    return launch_kernel(ssd_state_chain_kernel<N, false, SB>, dim3((unsigned)grid), block, l, p);
}

hipError_t launch_state_chain(const Params &p, const Launch &l) {
    switch (p.N) {
    case 64: return p.state_bf16 ? launch_n<64, true>(p, l) : launch_n<64, false>(p, l);
    case 128: return p.state_bf16 ? launch_n<128, true>(p, l) : launch_n<128, false>(p, l);
    case 256: return p.state_bf16 ? launch_n<256, true>(p, l) : launch_n<256, false>(p, l);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
