// Steps 3 and 5 of the scan: the inter-chunk state recurrence ("state_passing")
// and the final-state write (into the pool in place, or to final_states).
//
// For sequence b, head h and every state element (p, n), walking the
// sequence's chunks k in order (slot = cache_indices[b] for the in-place
// operation, b for the other one):
//   h_in[first]  = initial ? state_in[slot][h][p][n] : 0    (fp32 or bf16 storage)
//   h_in[k + 1]  = exp(cs_last(k)) * h_in[k] + S[k]
//   final        = exp(cs_last(K-1)) * h_in[K-1] + S[K-1]
//   state_out[slot][h][p][n] = final
// This is the "inter-chunk state recurrence with exponential decay" of
// "Mamba chunk scan with segsum" (description); the reset at each sequence
// start (to zero or the initial state) and the final state at each sequence
// end come from "mamba2_ssd_scan" ("Per-token recurrence", and the paragraph
// after it: final_states of shape (batch, nheads, head_dim, dstate)); reading
// the initial state from, and writing the final state to, slot
// cache_indices[b] of the pool (initial when has_initial_state[b]) is
// "Mamba2SSDChunkScanVarlenFwdInplace" (struct description).  A sequence with
// no tokens writes its initial state (or zeros) back.  With the short path
// on, the sequences it takes (zero-length ones included) are not walked: the
// grid runs over the list of the others that the chunk-state step writes.
//
// Chunk contributions arrive as fp16 under one power-of-two exponent per
// 32x32 tile of (chunk, head).  The chain is fp32.  h_in only feeds the
// outputs y; it is stored as fp16 with one power-of-two scale per row p (11
// significant bits: bf16's 8 would put the off-diagonal part's rounding error
// near the tolerance of y).  Each thread owns eight consecutive (p, n)
// elements of one (sequence, head) (16-byte loads and stores), reads its
// initial elements before the sequence's loop and writes the final ones
// after, so the in-place read-then-write of a slot never races.  The chunk contributions are loaded
// kDepth chunks ahead of their use, so that many loads per thread are in
// flight while the chain advances.  A row p spans N/8 lanes; its maximum is
// taken with DPP within rows of 16 lanes and a v_permlane16_swap across them.
#include <algorithm>

#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kDepth = 8;
constexpr int kPer = 8;  // elements per thread

// maximum over the aligned groups of LANES (8, 16 or 32) lanes, for values >= 0
template <int LANES>
__device__ __forceinline__ float row_max(float m) {
    m = dpp_max_step<0xB1, 0xF>(m);  // quad_perm [1,0,3,2]
    m = dpp_max_step<0x4E, 0xF>(m);  // quad_perm [2,3,0,1]
    m = dpp_max_step<0x141, 0xF>(m); // row_half_mirror: groups of 8
    if constexpr (LANES >= 16) m = dpp_max_step<0x140, 0xF>(m);  // row_mirror: rows of 16
    if constexpr (LANES >= 32) {
        const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
        m = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));  // rows 2r and 2r+1
    }
    return m;
}
}  // namespace

// the chain of one item: sequence b, head h, this thread's kPer state
// elements from e0 of the head
template <int N, bool SB>
__device__ __forceinline__ void walk_chain(const Params &p, int b, int h, int e0) {
    constexpr int64_t head_elems = (int64_t)kHeadDim * N;

    // clamped to the table so malformed query_start_loc cannot index past it
    const int k1 = (int)min((int64_t)p.chunk_off[b + 1], p.nchunks_max);
    const int k0 = min(p.chunk_off[b], k1);
    const int64_t slot = p.cache_idx != nullptr ? (int64_t)p.cache_idx[b] : (int64_t)b;
    const bool init = p.init_all != 0 || (p.has_init != nullptr && p.has_init[b] != 0);
    const int64_t off = (slot * p.H + h) * head_elems + e0;
    // state_in is null only when no sequence reads it
    const void *src = p.state_in != nullptr ? p.state_in : p.state_out;

    float st[kPer];
    if (init) {
        load_state8<SB>(src, off, st);
    } else {
#pragma unroll
        for (int e = 0; e < kPer; ++e) st[e] = 0.f;
    }
    const int64_t stride = (int64_t)p.H * head_elems;  // one chunk of states
    const uint16_t *S = p.states + ((int64_t)k0 * p.H + h) * head_elems + e0;
    // exponent of this thread's 32x32 tile (p / 32, n / 32) in each chunk
    const int NT = N / 32;
    const int tile = (int)((e0 / N) >> 5) * NT + (int)((e0 % N) >> 5);
    const int32_t *sexp = p.sexp + ((int64_t)k0 * p.H + h) * 2 * NT + tile;
    const int64_t sexp_stride = (int64_t)p.H * 2 * NT;
    const float *cs_last = p.cs2 + ((int64_t)k0 * p.H + h) * kChunk + kChunk - 1;
    const int64_t cs_stride = (int64_t)p.H * kChunk;
    uint16_t *hin = p.hin + ((int64_t)k0 * p.H + h) * head_elems + e0;
    int32_t *hexp = p.hexp + ((int64_t)k0 * p.H + h) * kHeadDim + e0 / N;
    const int nk = k1 - k0;

    // one link of the chain: store h_in of chunk k (row-scaled fp16), then
    // advance the state by chunk k's decay and contribution
    auto link = [&](int k, const u32x4 &sv, int sev, float dv) {
        // h_in row p as fp16, scaled by the power of two that puts the row's
        // max |h| in [2^14, 2^15)
        float m = 0.f;
#pragma unroll
        for (int e = 0; e < kPer; ++e) m = fmaxf(m, fabsf(st[e]));
        m = row_max<N / kPer>(m);
        const int sh = f16_scale_exponent(m);
        const float sc = ldexpf(1.0f, sh);
        u32x4 hv;
#pragma unroll
        for (int e = 0; e < 4; ++e) hv[e] = pack_f16x2(st[2 * e] * sc, st[2 * e + 1] * sc);
        *reinterpret_cast<u32x4 *>(hin + (int64_t)k * stride) = hv;
        hexp[(int64_t)k * p.H * kHeadDim] = sh;  // every lane of the row: the same value
        const float dec = fast_exp2(dv);
        const float us = ldexpf(1.0f, -sev);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            st[2 * e] = dec * st[2 * e] + f16_bits_to_float(sv[e] & 0xFFFFu) * us;
            st[2 * e + 1] = dec * st[2 * e + 1] + f16_bits_to_float(sv[e] >> 16) * us;
        }
    };
    // chunk k's contribution, exponent and decay (k clamped into the sequence)
    auto fetch = [&](int k, u32x4 &sv, int &sev, float &dv) {
        const int kk = min(k, nk - 1);
        sv = *reinterpret_cast<const u32x4 *>(S + (int64_t)kk * stride);
        sev = sexp[(int64_t)kk * sexp_stride];
        dv = cs_last[(int64_t)kk * cs_stride];
    };
    int kb = 0;
    if (nk >= kDepth) {
        // ring of the next kDepth chunks; full rounds of kDepth links, each
        // refilling its slot kDepth chunks ahead (past the end: the last chunk again)
        u32x4 s[kDepth];
        int se[kDepth];
        float d[kDepth];
#pragma unroll
        for (int q = 0; q < kDepth; ++q) fetch(q, s[q], se[q], d[q]);
        for (; kb + kDepth <= nk; kb += kDepth) {
#pragma unroll
            for (int q = 0; q < kDepth; ++q) {
                link(kb + q, s[q], se[q], d[q]);
                fetch(kb + q + kDepth, s[q], se[q], d[q]);
            }
        }
    }
    for (; kb < nk; ++kb) {  // the rest, one chunk at a time
        u32x4 sv;
        int sev;
        float dv;
        fetch(kb, sv, sev, dv);
        link(kb, sv, sev, dv);
    }
    store_state8<SB>(p.state_out, off, st);
}

// An item is (sequence, slice of 256 * kPer state elements, head), the
// sequence slowest and the head fastest; each workgroup walks every
// gridDim.x-th item.  Workgroup ids are dealt to the eight XCDs round-robin,
// so the heads of one sequence land on different XCDs and every XCD gets a
// share of every sequence.  With the sequence as the fast index a sequence's
// whole chain runs on one XCD, and ragged lengths leave most XCDs idle while
// a few walk the long chains (the ragged 32-sequence workload: 421 us, 145 us
// in this order).
// LIST: the sequences are those of the list the chunk-state step wrote (the
// short path is on: only sequences longer than its limit are there), else the
// batch.
// SB: states stored as bf16 (read widened to fp32, final state rounded once).
template <int N, bool LIST, bool SB>
__global__ __launch_bounds__(256) void ssd_state_passing_kernel(Params p) {
    constexpr int ZB = kHeadDim * N / (256 * kPer);  // slices per head
    const int64_t per_seq = (int64_t)p.H * ZB;
    const int64_t items = (LIST ? (int64_t)p.meta[1] : (int64_t)p.batch) * per_seq;
#pragma unroll 1
    for (int64_t item = blockIdx.x; item < items; item += gridDim.x) {
        const int64_t bi = item / per_seq;
        const int rem = (int)(item - bi * per_seq);
        const int z = rem / p.H;
        const int h = rem - z * p.H;
        const int b = LIST ? p.seq_list[bi] : (int)bi;
        walk_chain<N, SB>(p, b, h, (z * 256 + (int)threadIdx.x) * kPer);
    }
}

hipError_t launch_state_passing(const Params &p, const Launch &l) {
    // items: (sequence, slice, head); the sequences are at most nseq_grid
    // (the list) or batch.  Up to 32 workgroups per compute unit; past that,
    // workgroups take several items.
    const int64_t items = (int64_t)(p.short_max > 0 ? p.nseq_grid : p.batch) * p.H * (kHeadDim * p.N / (256 * kPer));
    const bool list = p.short_max > 0;
    const dim3 grid((unsigned)std::max<int64_t>(1, std::min<int64_t>(items, (int64_t)p.num_cus * 32)));
    const dim3 block(256);
    if (p.state_bf16) {
        switch (p.N) {
        case 64:
            return list ? launch_kernel(ssd_state_passing_kernel<64, true, true>, grid, block, l, p)
                        : launch_kernel(ssd_state_passing_kernel<64, false, true>, grid, block, l, p);
        case 128:
            return list ? launch_kernel(ssd_state_passing_kernel<128, true, true>, grid, block, l, p)
                        : launch_kernel(ssd_state_passing_kernel<128, false, true>, grid, block, l, p);
        case 256:  // the short path does not serve dstate 256
            return launch_kernel(ssd_state_passing_kernel<256, false, true>, grid, block, l, p);
        default: return hipErrorInvalidValue;
        }
    }
    switch (p.N) {
    case 64:
        return list ? launch_kernel(ssd_state_passing_kernel<64, true, false>, grid, block, l, p)
                    : launch_kernel(ssd_state_passing_kernel<64, false, false>, grid, block, l, p);
    case 128:
        return list ? launch_kernel(ssd_state_passing_kernel<128, true, false>, grid, block, l, p)
                    : launch_kernel(ssd_state_passing_kernel<128, false, false>, grid, block, l, p);
    case 256:
        return launch_kernel(ssd_state_passing_kernel<256, false, false>, grid, block, l, p);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
