// Steps 0 and 1 of the scan for the chunked sequences, in one launch: the
// chunk table, each chunk's cumulative decay per head ("chunk_cumsum"), the
// per-(chunk, group) C.B^T tiles of the chunk-scan step, and each chunk's own
// state contribution ("chunk_state"),
//   S_k[p][n] = sum_j exp2(cs2_last - cs2_j) dts_j x[t0+j,h,p] B[t0+j,g,n]
// for chunk k (tokens t0 .. t0+len-1) of head h, group g.  This is the
// per-token recurrence of "mamba2_ssd_scan" ("Per-token recurrence") summed
// over one chunk from a zero state: each token's B x, decayed to the chunk
// end; the "inter-chunk state" of "Mamba chunk scan with segsum"
// (description) is built from these by the state-passing step.
//
// Chunk table: sequence b owns ceil(len_b / 256) chunks (none when empty);
// chunk c of the call is found from the exclusive prefix sum of those counts,
// so no chunk ever straddles two sequences (the state resets at every
// query_start_loc boundary: "mamba2_ssd_scan", "Per-token recurrence").
// Every workgroup computes the prefix itself; the first workgroup of chunk 0
// also publishes it (chunk_off, meta) for the later steps.  Sequences the
// short path takes (short_max > 0: 0 .. short_max tokens) own no chunks; that
// workgroup then also writes the list of the sequences the state chain walks
// (the others) and the list of those of 1 .. recur_max tokens for the
// token-recurrence kernel, with their counts (meta[1], meta[2]).  The first
// workgroup of each chunk writes its descriptor {sequence, first token,
// length}.
//
// One workgroup per (chunk, block of HB heads of one group); no chunk waits
// for another.  Sixteen wavefronts.  Prologue, once per workgroup:
//   - chunk_cumsum of the block's heads (wavefronts 0-7, wavefront w taking
//     heads w and w + 8): dts = softplus(dt + dt_bias) (0 past the chunk end) and
//     cs2 = log2(e) * cumsum(A dts), the segment sums of "Mamba chunk scan
//     with segsum" (description) in base 2, stored for the later steps;
//   - the chunk's B (256 rows, zero past the chunk end) is staged in LDS
//     whole, and the C rows of this workgroup's row-block pairs stream
//     through LDS 32 dstate columns at a time, three slices in flight in
//     registers.  The C.B^T tiles G^T[j][i] = sum_n B[t0+j,g,n] C[t0+i,g,n],
//     j <= i blockwise, the "attention-like" intra-chunk scores before decay,
//     are shared by every head of the group; the workgroups of a (chunk,
//     group) split the four row-block pairs {q, 7-q} (9 of the 36
//     lower-triangular 32x32 tiles each) among themselves.  They are formed
//     with bf16 MFMA on the exact inputs (fp32 accumulate), the diagonal
//     tiles zeroed above their diagonal, and stored in MFMA accumulator order
//     as fp16 under one power-of-two exponent per pair (gexp) that puts its
//     maximum magnitude in [2^14, 2^15);
//   - then the consumer wavefronts read their n tile of the staged B back
//     token-contiguous as their B^T MFMA A operands (fp16, scaled by the
//     power of two that puts the tile's max |B| in [2^14, 2^15)) and keep
//     them in registers for all heads.
// Then the heads, in two roles:
//   - consumers (wavefronts 0-7): wavefront w owns n tile w (dstate 256), or
//     n tile w/2 and p tile w%2 (dstate 128, 64; at 64 only wavefronts 0-3).
//     Per head, each S^T tile is 16 v_mfma_f32_32x32x16_f16 over the chunk's
//     256 tokens (fp32 accumulate), stored as fp16.
//   - producers (wavefronts 8-15): load each head's x and the dts and cs2 of
//     its tokens two heads ahead, form the token weights
//     w_j = exp2(cs2_last - cs2_j) dts_j and the maxima of |w| and |x| one
//     head ahead, and stage (w x)^T into one of two LDS buffers as fp16 under
//     the power of two that puts max|w| max|x| in [2^14, 2^15).
// One barrier per head: while the consumers multiply head k-1 out of one
// buffer (and store head k-2), the producers stage head k into the other, so
// the vector work of the staging and the matrix products overlap.  The scale
// of each chunk's x for the chunk-scan step (xexp) is written here too.
// Workgroups are numbered so that all head blocks of a chunk land on one XCD
// (dispatch is round-robin over the 8 XCDs) and read the chunk's B and C
// through its L2.
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
constexpr int kWaves = kConsumers + kProducers;
constexpr int kThreads = 64 * kWaves;
// dwords per staged row: 128 token pairs + pad.  LDS serves 4-byte accesses
// 32 lanes at a time over 32 banks and 8-byte accesses 32 lanes at a time
// over 64 banks.  At this stride the MFMA operand reads (8 bytes, rows 0..31
// of one column) fall on distinct bank pairs, and so do the staging stores
// (4 bytes, rows 8v + i and 8v + 8 + i for 16 consecutive pairs each, the
// two rows 16 banks apart).
constexpr int XT_STRIDE = 130;
// dwords per row of a staged 32-column slice of C (32 bf16 + pad)
constexpr int R_STRIDE = 20;
constexpr int kPD = 3;  // prologue slices of C in flight in registers

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

// dwords per row of the staged B: N/2 (N bf16) + 4, so that the 16-byte MFMA
// operand reads of 16 consecutive rows fall on distinct groups of four banks
template <int N>
struct BStride {
    static constexpr int value = N / 2 + 4;
};

// The prologue's LDS: the chunk's B (rows = tokens), one slice of the C rows
// of the workgroup's row-block pairs (its pair k: rows 64k .. 64k+31 of row
// block q_k, rows 64k+32 .. 64k+63 of row block 7-q_k), and, past the area
// the heads reuse, the tile maxima and the chunk-table scan's totals.
template <int N>
struct __attribute__((aligned(16))) PrologueSmem {
    uint32_t b[kChunk * BStride<N>::value];
    uint32_t c[kChunk * R_STRIDE];
    float tmax[36];  // per C.B^T tile of the workgroup: max |G|
    float bmaxt[kWaves][N / 32];  // per wavefront and n tile: max |B| of its staged pieces
    int wtot[kWaves];
    int loc[2];
};

// The prologue's area is reused by the heads once the slices are consumed.
template <int N>
union __attribute__((aligned(16))) Smem {
    StateSmem<N> st;
    PrologueSmem<N> pro;
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

// Tile i (0..8) of row-block pair q: row block q for i <= q (column blocks
// 0..q), else row block 7-q (column blocks 0..7-q).
__host__ __device__ constexpr int pair_rb(int q, int i) { return i <= q ? q : 7 - q; }
__host__ __device__ constexpr int pair_t(int q, int i) { return i <= q ? i : i - q - 1; }

// The workgroup's share of the C.B^T tiles: the nwg workgroups of a (chunk,
// group) split the four row-block pairs, pair q going to workgroup
// q mod min(nwg, 4).  Pair k of this workgroup is q = w_in + k min(nwg, 4);
// its tiles are 9k .. 9k+8 of the workgroup.
struct GramShare {
    int nq, w_in, npairs;
    __device__ int pair(int k) const { return w_in + k * nq; }
};
__device__ __forceinline__ GramShare gram_share(int nwg, int w_in) {
    GramShare s;
    s.nq = nwg < 4 ? nwg : 4;
    s.w_in = w_in;
    s.npairs = w_in < s.nq ? (4 - w_in + s.nq - 1) / s.nq : 0;
    return s;
}
}  // namespace

// Locate chunk c (first token, length) from the per-sequence chunk counts;
// the lead workgroup also publishes the chunk table and the sequence lists,
// the first workgroup of the chunk its descriptor.  Returns false when the
// call has fewer than c + 1 chunks.  Every thread of the workgroup calls it.
template <int N>
__device__ __forceinline__ bool locate_chunk(const Params &p, int c, bool lead, bool first_of_chunk,
                                             PrologueSmem<N> &sp, int64_t &t0, int &len) {
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    if (tid == 0) { sp.loc[0] = -1; sp.loc[1] = 0; }
    int carry = 0;
    for (int base = 0; base < p.batch; base += kThreads) {
        const int b = base + tid;
        int n = 0;
        if (b < p.batch) {
            const int l = p.qsl[b + 1] - p.qsl[b];
            n = !is_short_sequence(l, p.short_max) && l > 0 ? (l + kChunk - 1) / kChunk : 0;
        }
        const int wincl = wave_incl_scan(n);
        __syncthreads();  // protects wtot from the previous round
        if (lane == 63) sp.wtot[wave] = wincl;
        __syncthreads();
        int before = 0, total = 0;
        for (int w = 0; w < kWaves; ++w) {
            if (w < wave) before += sp.wtot[w];
            total += sp.wtot[w];
        }
        const int excl = carry + before + wincl - n;
        if (b < p.batch) {
            if (c >= excl && c < excl + n) { sp.loc[0] = b; sp.loc[1] = c - excl; }
            if (lead) p.chunk_off[b] = excl;
        }
        carry += total;
    }
    if (lead) {
        // the sequences the state chain walks: all of them when no sequence
        // can take the short path, else those longer than its limit, and, in
        // a second list, the sequences the token recurrence takes (both counts
        // packed in one scan: low 16 bits and high 16 bits per round of
        // kThreads sequences)
        int carry2 = 0, carry3 = 0;
        for (int base = 0; base < p.batch; base += kThreads) {
            const int b = base + tid;
            int f = 0, r = 0;
            if (b < p.batch) {
                const int l = p.qsl[b + 1] - p.qsl[b];
                f = !is_short_sequence(l, p.short_max);
                r = l >= 1 && l <= p.recur_max;
            }
            const int wincl = wave_incl_scan(f | (r << 16));
            __syncthreads();
            if (lane == 63) sp.wtot[wave] = wincl;
            __syncthreads();
            int before = 0, total = 0;
            for (int w = 0; w < kWaves; ++w) {
                if (w < wave) before += sp.wtot[w];
                total += sp.wtot[w];
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
    const int b = sp.loc[0];
    if (b < 0) {
        if (tid == 0 && first_of_chunk) p.desc[c] = make_int4(-1, 0, 0, 0);
        return false;
    }
    t0 = (int64_t)p.qsl[b] + (int64_t)sp.loc[1] * kChunk;
    len = (int)min((int64_t)kChunk, (int64_t)p.qsl[b + 1] - t0);
    if (tid == 0 && first_of_chunk) p.desc[c] = make_int4(b, (int)t0, len, 0);
    return true;
}

template <int N, int HB>
__global__ __launch_bounds__(kThreads) void ssd_chunk_state_kernel(Params p) {
    constexpr int NT = N / 32;
    constexpr int TPW = N == 256 ? 2 : 1;  // p tiles per consumer wavefront
    __shared__ Smem<N> smu;
    StateSmem<N> &sm = smu.st;
    PrologueSmem<N> &sp = smu.pro;

    // ---- XCD-aware decode: all head blocks of chunk c share one XCD
    const int nhb = p.H / HB;
    const int id = blockIdx.x;
    const int xcd = id & 7;
    const int slot = id >> 3;
    const int c = (slot / nhb) * 8 + xcd;
    const int h_first = (slot - (slot / nhb) * nhb) * HB;
    if (c >= p.nchunks_grid) return;  // the grid's padding to a multiple of 8 chunks (uniform)
    const int hg = p.H / p.G;
    const int g = h_first / hg;
    const GramShare gs = gram_share(hg / HB, (h_first - g * hg) / HB);

    int64_t t0 = 0;
    int len = 1;
    if (!locate_chunk(p, c, c == 0 && h_first == 0, h_first == 0, sp, t0, len)) return;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int l32 = lane & 31;
    const int hl = lane >> 5;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const bool producer = wave >= kConsumers;  // wavefront-uniform
    const int ntiles = 9 * gs.npairs;

    // ---- prologue.  B: thread t loads the 16-byte pieces t + kThreads i of
    // the chunk's rows (N/8 pieces per row, whole rows per wavefront); rows
    // past the chunk end are loaded as its last row and staged as zeros.  C:
    // one 16-byte piece (t % 4) of local row t / 4 per slice (threads past the
    // workgroup's C rows load one of them again and do not store it); rows
    // past the chunk end repeat its last row (their outputs are never stored).
    constexpr int BS = BStride<N>::value;
    constexpr int BPR = N / 8;                    // 16-byte pieces per row of B
    constexpr int BPT = kChunk * BPR / kThreads;  // per thread
    auto load_b = [&](u32x4 (&bv)[BPT]) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int f = tid + kThreads * i;
            bv[i] = *reinterpret_cast<const u32x4 *>(p.B + ((t0 + min(f / BPR, len - 1)) * p.G + g) * N + 8 * (f % BPR));
        }
    };
    // B staged, and the maximum |B| of each n tile over this wavefront's
    // pieces (a thread's pieces all lie in n tile (t % (N/8)) / 4)
    auto stage_b = [&](const u32x4 (&bv)[BPT]) {
        u16x2 m2 = u16x2{0, 0};
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int f = tid + kThreads * i;
            const int row = f / BPR;
            const u32x4 v = row < len ? bv[i] : u32x4{};
            *reinterpret_cast<u32x4 *>(sp.b + row * BS + 4 * (f % BPR)) = v;
#pragma unroll
            for (int w = 0; w < 4; ++w) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u16x2, v[w] & 0x7FFF7FFFu));
        }
        float m = __uint_as_float(max((uint32_t)m2[0], (uint32_t)m2[1]) << 16);
        // over the lanes of one n tile: equal (lane % (N/8)) / 4
        m = dpp_max_step<0xB1, 0xF>(m);  // quad_perm [1,0,3,2]
        m = dpp_max_step<0x4E, 0xF>(m);  // quad_perm [2,3,0,1]
#pragma unroll
        for (int d = BPR; d < 64; d <<= 1) m = fmaxf(m, __shfl_xor(m, d, 64));
        if ((lane & 3) == 0 && lane < BPR) sp.bmaxt[wave][lane >> 2] = m;
    };
    const int sv = tid & 3;
    const int srow = tid >> 2;
    const int crows = 64 * gs.npairs;
    const int clocal = crows > 0 ? srow % crows : 0;
    const int cq = gs.pair(clocal >> 6);
    const int cglob = 32 * ((clocal & 63) < 32 ? cq : 7 - cq) + (clocal & 31);
    const uint16_t *csrc = p.C + ((t0 + min(cglob, len - 1)) * p.G + g) * N + sv * 8;
    auto load_c = [&](u32x4 (&rcv)[kPD], int ks, int d) {
        rcv[d] = *reinterpret_cast<const u32x4 *>(csrc + ks * 32);
    };
    auto stage_c = [&](const u32x4 (&rcv)[kPD], int ks) {
        if (srow < crows) *reinterpret_cast<u32x4 *>(sp.c + srow * R_STRIDE + sv * 4) = rcv[ks % kPD];
    };
    // tile i of the workgroup: row block rb (C rows: the columns i of G^T),
    // column block t (B rows), local C rows from lr
    auto tile_coords = [&](int i, int &rb, int &t, int &lr) {
        const int k = i / 9, ti = i - 9 * k;
        const int q = gs.pair(k);
        rb = pair_rb(q, ti);
        t = pair_t(q, ti);
        lr = 64 * k + (rb == q ? 0 : 32);
    };
    // the two K-steps of slice ks for tile i
    auto gram_step = [&](int ks, int i, f32x16 &acc) {
        int rb, t, lr;
        tile_coords(i, rb, t, lr);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            const bf16x8 cb = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(sp.c + (lr + l32) * R_STRIDE + 8 * kk + 4 * hl));
            const bf16x8 bb = __builtin_bit_cast(
                bf16x8, *reinterpret_cast<const u32x4 *>(sp.b + (32 * t + l32) * BS + 16 * ks + 8 * kk + 4 * hl));
            acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bb, cb, acc, 0, 0, 0);
        }
    };
    // a finished tile: zero above the diagonal of a diagonal tile (readers
    // need no mask), its max into tmax
    auto gram_max = [&](int i, f32x16 &acc) {
        int rb, t, lr;
        tile_coords(i, rb, t, lr);
        if (rb == t) {
            // element e of lane l: j - 32 rb = 8(e/4) + 4(l/32) + e%4, i - 32 rb = l%32
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (8 * (e >> 2) + 4 * hl + (e & 3) > l32) acc[e] = 0.f;
        }
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < 16; ++e) m = fmaxf(m, fabsf(acc[e]));
        sp.tmax[i] = wave_max(m);  // the same value from every lane
    };
    // once every tile's max is in: the pair's exponent, and the tile as fp16
    // in accumulator order (tile rb(rb+1)/2 + t, 64 lanes x 16 values)
    auto gram_store = [&](int i, const f32x16 &acc) {
        int rb, t, lr;
        tile_coords(i, rb, t, lr);
        const int k = i / 9;
        float gm = 0.f;
        for (int u = 0; u < 9; ++u) gm = fmaxf(gm, sp.tmax[9 * k + u]);
        const int sg = f16_scale_exponent(gm);
        if (i == 9 * k) p.gexp[((int64_t)c * p.G + g) * 4 + gs.pair(k)] = sg;  // every lane: the same value
        const float gsc = ldexpf(1.0f, sg);
        u32x4 *o = reinterpret_cast<u32x4 *>(p.cbt + (((int64_t)c * p.G + g) * 36 + rb * (rb + 1) / 2 + t) * 1024 +
                                             lane * 16);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2)
            o[h2] = u32x4{pack_f16x2(acc[8 * h2] * gsc, acc[8 * h2 + 1] * gsc),
                          pack_f16x2(acc[8 * h2 + 2] * gsc, acc[8 * h2 + 3] * gsc),
                          pack_f16x2(acc[8 * h2 + 4] * gsc, acc[8 * h2 + 5] * gsc),
                          pack_f16x2(acc[8 * h2 + 6] * gsc, acc[8 * h2 + 7] * gsc)};
    };
    // The prologue of both roles: `before` (the consumers' dt loads), B and
    // the first C slices in flight, B staged, `after` (the consumers'
    // cumulative decay), then the C slices with the C.B^T tiles wave + 16m of
    // this wavefront (at most 36 tiles in the workgroup).  Two barriers per C
    // slice, one for the tile maxima.
    constexpr int MAXT = 3;
    int nmine = 0;
#pragma unroll
    for (int m = 0; m < MAXT; ++m)
        if (wave + 16 * m < ntiles) nmine = m + 1;
    auto prologue = [&](auto &&before, auto &&after) {
        f32x16 acc[MAXT];
#pragma unroll
        for (int m = 0; m < MAXT; ++m) acc[m] = f32x16{};
        u32x4 rcv[kPD];
        before();
        {
            u32x4 bv[BPT];
            load_b(bv);
#pragma unroll
            for (int d = 0; d < kPD && d < NT; ++d) load_c(rcv, d, d);
            stage_b(bv);
        }
        after();
#pragma unroll
        for (int ks = 0; ks < NT; ++ks) {
            __syncthreads();  // B staged; the previous C slice consumed
            stage_c(rcv, ks);
            if (ks + kPD < NT) load_c(rcv, ks + kPD, ks % kPD);
            __syncthreads();
#pragma unroll
            for (int m = 0; m < MAXT; ++m)
                if (m < nmine) gram_step(ks, wave + 16 * m, acc[m]);
        }
#pragma unroll
        for (int m = 0; m < MAXT; ++m)
            if (m < nmine) gram_max(wave + 16 * m, acc[m]);
        __syncthreads();  // tile maxima complete
#pragma unroll
        for (int m = 0; m < MAXT; ++m)
            if (m < nmine) gram_store(wave + 16 * m, acc[m]);
    };

    // phases 0 .. HB+1 (products of head j-1 and stores of head j-2 in phase
    // j), rounded up to pairs
    constexpr int kPhases = (HB + 3) & ~1;

    // Each role runs its own loops with the same barriers: one per prologue
    // slice, one once the tiles are formed, one before the heads, one per
    // phase.  Phase j (j = 0 .. kPhases-1, in pairs so that the two register
    // sets of each role alternate at compile time): producers stage head j
    // into buffer j & 1 and analyse head j+1 (past the last head they repeat
    // it); consumers store head j-2 and multiply head j-1.
    if (producer) {
        const int pw = wave - kConsumers;  // producer wavefront 0 .. 7
        // at dstate <= 128 the producers issue ahead of the consumers (a higher
        // wave priority): measured faster there, and slower at dstate 256
        if constexpr (N <= 128) __builtin_amdgcn_s_setprio(1);
        prologue([] {}, [] {});

        // ---- heads
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
        __syncthreads();  // the consumers have read their B^T operands: the heads reuse the LDS
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
        // ---- prologue, with the cumulative decay of heads wave and wave + 8
        // of the block: their dt loaded first, the decay formed once B is
        // staged (lane l takes tokens 4l .. 4l+3; past the chunk end the dt of
        // its last token, which chunk_cumsum4 discards)
        constexpr int HC = (HB + kConsumers - 1) / kConsumers;  // heads per consumer
        float dtv[HC][4];
        prologue(
            [&] {
#pragma unroll
                for (int k = 0; k < HC; ++k) {
                    const int h = h_first + min(wave + kConsumers * k, HB - 1);
#pragma unroll
                    for (int e = 0; e < 4; ++e) dtv[k][e] = p.dt[(t0 + min(4 * lane + e, len - 1)) * p.H + h];
                }
            },
            [&] {
#pragma unroll
                for (int k = 0; k < HC; ++k) {
                    const int i = wave + kConsumers * k;
                    if (i < HB) {  // uniform per wavefront
                        const int h = h_first + i;
                        const float bias = p.dt_bias != nullptr ? p.dt_bias[h] : 0.0f;
                        float dts[4], cs2[4];
                        chunk_cumsum4(dtv[k], bias, p.A[h], p.dt_softplus != 0, len, dts, cs2);
                        const int64_t r = ((int64_t)c * p.H + h) * kChunk + 4 * lane;
                        *reinterpret_cast<float4 *>(p.dts + r) = make_float4(dts[0], dts[1], dts[2], dts[3]);
                        *reinterpret_cast<float4 *>(p.cs2 + r) = make_float4(cs2[0], cs2[1], cs2[2], cs2[3]);
                    }
                }
            });
        // ---- B^T operands of the wavefront's n tile from the staged B:
        // K-step s, this lane: rows n = 32 nt + l%32, tokens 16 s + 8 (l/32) +
        // 0..7 (rows past the chunk end are zero), scaled by 2^sb, sb putting
        // the tile's max |B| (from the staging wavefronts' maxima) in
        // [2^14, 2^15)
        u32x4 fr[16];
        int sb = 0;
        if (mma) {
            float bm = 0.f;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) bm = fmaxf(bm, sp.bmaxt[w][nt]);
            sb = f16_scale_exponent(bm);
            const float bs = ldexpf(1.0f, sb);
            const uint16_t *col = reinterpret_cast<const uint16_t *>(sp.b) + 32 * nt + l32;
#pragma unroll
            for (int s = 0; s < 16; ++s) {
                uint32_t o[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int j = 16 * s + 8 * hl + 2 * e;
                    o[e] = pack_f16x2(bf16_bits_to_float(col[j * 2 * BS]) * bs,
                                      bf16_bits_to_float(col[(j + 1) * 2 * BS]) * bs);
                }
                fr[s] = u32x4{o[0], o[1], o[2], o[3]};
                // a few K-steps of reads at a time (hoisted, they would all be live at once)
                if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);
            }
        } else {
#pragma unroll
            for (int s = 0; s < 16; ++s) fr[s] = u32x4{};
        }
        __syncthreads();  // every B^T operand read: the heads reuse the LDS

        // ---- heads
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
                const int half = (t >> 5) & 1;
                // the lane's 8 tokens of K-step ks: pairs 8 ks + 4 half .. +3, two 8-byte reads
                const u32x2 *brow = reinterpret_cast<const u32x2 *>(sm.xt[b] + r * XT_STRIDE + 4 * half);
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
                uint32_t *srowp = sm.sbuf[b] + r * SStride<N>::value + 16 * nt + 2 * half;
#pragma unroll
                for (int a = 0; a < 4; ++a)
                    *reinterpret_cast<u32x2 *>(srowp + 4 * a) =
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
// operands are formed once per workgroup, and its phases overlap staging
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
