// Shared definitions of the libssd HIP kernels (gfx950 / CDNA4).
//
// The operation is the Mamba-2 SSD varlen prefill scan ("mamba2_ssd_scan",
// section "Per-token recurrence"), evaluated with the chunked segment-sum
// reformulation of "Mamba chunk scan with segsum" (description): chunks of 256
// tokens, an in-chunk causal block, an inter-chunk state recurrence with
// exponential decay, and their sum.
//
// Base-2 exponentials: every decay exp(z) is computed as exp2(z * log2 e), the
// constant being LOG2E of "mamba2_ssd_scan" (comptime values), so the kernels
// keep the prefix sums in log2 units ("cs2") and call the hardware exp2.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace ssd {

constexpr int kChunk = 256;      // chunk length (tokens)
constexpr int kHeadDim = 64;     // P the kernels take
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kShortMax = 128;   // longest sequence the short-path kernel takes
constexpr int kRecurMax = 4;     // longest sequence the token-recurrence kernel takes
constexpr int kNoExponent = 1000;  // stored scale exponent of an all-zero block of x
// Word 3 of a raw buffer resource: 32-bit data format, no swizzle; accesses at
// offsets past the resource's byte count are dropped by the range check.
constexpr int kBufferFormat32 = 0x00020000;
// DPP quad permutation [1, 0, 3, 2]: each lane reads its neighbour (lane ^ 1).
constexpr int kQuadSwap01 = 0xB1;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));

// Everything a launch needs, passed by value as the kernel argument.
struct Params {
    // sizes
    int64_t T;
    int batch, H, P, G, N, max_slots;
    int dt_softplus;
    int64_t nchunks_max;
    int num_cus;  // compute units of the device the call runs on
    // caller tensors (device)
    uint16_t *y;
    const uint16_t *x;
    const float *dt, *A;
    const uint16_t *B, *C;
    const float *D, *dt_bias;
    const int32_t *qsl;
    // where each sequence's state starts and ends, [slots][H][P][N] fp32 or bf16:
    // slot cache_idx[b] (b when cache_idx is null) of state_in, read when
    // init_all or has_init[b] (has_init may be null: no sequence), and of
    // state_out, written with the final state.  The in-place operation passes
    // the pool for both; the other one initial_states (or null, never read)
    // and final_states, with no slot indices.
    const void *state_in;   // fp32 or bf16 elements (state_bf16)
    void *state_out;
    int state_bf16;         // states stored as bf16 (arithmetic stays fp32)
    const uint8_t *has_init;
    const uint32_t *cache_idx;
    int init_all;
    // sequences of 0 .. short_max tokens are taken by the short-path kernel
    // and skipped by the chunked steps (short_max 0: none; at most kShortMax)
    int short_max;
    // launch sizes: chunks (<= nchunks_max) and sequences the chunked steps
    // can see at most, given the routing
    int64_t nchunks_grid;
    int nseq_grid;
    // of the short sequences, those of 1 .. recur_max tokens go to the
    // token-recurrence kernel (0: none)
    int recur_max;
    // workspace carve (device); nchunks_max rows per table
    int32_t *meta;       // [4]: nchunks
    int32_t *chunk_off;  // [batch+1]
    int4 *desc;          // [nchunks_max]: {seq, t0, len, 0}
    float *dts;          // [nchunks_max][H][256]: dts per token, 0 past the chunk end
    float *cs2;          // [nchunks_max][H][256]: log2(e) * inclusive cumsum of A dts
    uint16_t *cbt;       // [nchunks_max][G][36][64][16] fp16 C.B^T tiles * 2^gexp, accumulator order
    int32_t *gexp;       // [nchunks_max][G][4]: tiles of row blocks q and 7-q
    uint16_t *states;    // [nchunks_max][H][P][N] fp16 chunk contributions, 32x32 tile scaled by 2^sexp
    int32_t *sexp;       // [nchunks_max][H][2][N/32]: per 32x32 tile (p tile, n tile)
    uint16_t *hin;       // [nchunks_max][H][P][N] fp16, row p scaled by 2^hexp
    int32_t *hexp;       // [nchunks_max][H][P]: per row
    int32_t *xexp;       // [nchunks_max][H][2]: 2^xexp puts the chunk's max |x| over p half of the head in [2^14, 2^15)
    int32_t *seq_list;   // [batch]: the meta[1] sequences the state passing walks
    int32_t *recur_list; // [batch]: the meta[2] sequences the token recurrence takes
};

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
    __bf16 b = (__bf16)f;
    return __builtin_bit_cast(uint16_t, b);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (nearest even) in one dword: one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const bf16x2 h = __builtin_convertvector((f32x2){lo, hi}, bf16x2);
    return __builtin_bit_cast(uint32_t, h);
}

// two floats -> two fp16 (nearest even) in one dword: v_cvt_pk_f16_f32 on gfx950
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
    const f16x2 h = __builtin_convertvector((f32x2){lo, hi}, f16x2);
    return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

// Exponent s that puts a positive maximum m in [2^14, 2^15) after scaling by
// 2^s (0 when m is 0 or NaN), so scaled values stay well inside fp16's range.
// s is capped at 126 so that 2^s and 2^-s are both finite, normal floats:
// below 2^-112 (subnormal m included, whose exponent field reads as -127) the
// scaled maximum lands under 2^14 instead, which fp16 still holds.
__device__ __forceinline__ int f16_scale_exponent(float m) {
    if (!(m > 0.0f)) return 0;
    const int s = 14 - ((int)((__float_as_uint(m) >> 23) & 0xFF) - 127);
    return s < 126 ? s : 126;
}

__device__ __forceinline__ f32x4 mfma_bf16(const bf16x8 &a, const bf16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mfma_f16(const f16x8 &a, const f16x8 &b, const f32x4 &c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// 32x32 output tile, K = 16.  Lane l: A row l%32, k = (l/32)*8 + e; B column
// l%32, same k; D element t at row 8*(t/4) + 4*(l/32) + t%4, column l%32.
__device__ __forceinline__ f32x16 mfma32_f16(const f16x8 &a, const f16x8 &b, const f32x16 &c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Inclusive scan of one int over a 64-lane wavefront.
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        int o = __shfl_up(v, d, 64);
        if (lane >= d) v += o;
    }
    return v;
}

// Inclusive sum over a 64-lane wavefront with DPP: shifts by 1, 2, 4 and 8
// within rows of 16 lanes (lanes without a source add 0), then the row
// broadcasts carry each row's total into the rows above it.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add_step(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_incl_scan(float v) {
    v = dpp_add_step<0x111, 0xF>(v);  // row_shr:1
    v = dpp_add_step<0x112, 0xF>(v);  // row_shr:2
    v = dpp_add_step<0x114, 0xF>(v);  // row_shr:4
    v = dpp_add_step<0x118, 0xF>(v);  // row_shr:8
    v = dpp_add_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_add_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

// v plus the value of another lane by a DPP pattern with a source for every
// lane (quad permutations, row mirrors)
template <int CTRL>
__device__ __forceinline__ float dpp_add_all(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Maximum over a 64-lane wavefront for values >= 0 (magnitudes), with DPP
// row operations instead of LDS permutes: within rows of 16 lanes, then
// across rows with the row broadcasts (lanes a DPP step leaves unwritten
// contribute 0, which cannot raise a maximum of non-negative values); the
// total lands in lane 63 and is read back as a uniform value.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max_step(float v) {
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, false)));
}
// Maximum over each aligned group of 16 lanes (a DPP row), for values >= 0;
// every lane of the row receives it.
__device__ __forceinline__ float row16_max(float v) {
    v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
    return v;
}

__device__ __forceinline__ float wave_max(float v) {
    v = dpp_max_step<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_step<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_step<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max_step<0x140, 0xF>(v);  // row_mirror
    v = dpp_max_step<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_step<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) v = min(v, __shfl_xor(v, d, 64));
    return v;
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) {
        uint32_t o = (uint32_t)__shfl_xor((int)v, d, 64);
        v = v > o ? v : o;
    }
    return v;
}

// 2^x with the hardware instruction (v_exp_f32).  Used for decays, whose
// arguments are <= 0 for A <= 0: results below the smallest normal float are
// flushed toward zero, which is harmless for a decay factor.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// 2^k as a float for |k| < 127 (exact), for scaling by powers of two with a
// multiply.
__device__ __forceinline__ float pow2i(int k) {
    k = k < -126 ? -126 : (k > 127 ? 127 : k);
    return __uint_as_float((uint32_t)(k + 127) << 23);
}

// softplus(v) = log(1 + e^v) = max(v, 0) + log1p(e^-|v|), without overflow.
// e^-|v| and the logarithm use the hardware exp2 / log2; log1p(z) is taken as
// log(u) * z / (u - 1) with u = 1 + z rounded, which cancels the rounding of
// u (Goldberg, "What every computer scientist should know about
// floating-point arithmetic", the log1p formula), so small z keep their
// relative accuracy.
__device__ __forceinline__ float softplus_f(float v) {
    const float z = fast_exp2(-fabsf(v) * kLog2e);  // in (0, 1]
    const float u = 1.0f + z;
    const float l = u == 1.0f ? z : __builtin_amdgcn_logf(u) * (kLn2 * z / (u - 1.0f));
    return fmaxf(v, 0.0f) + l;
}

// ---- state storage: fp32, or bf16 (SB) rounded to nearest even when stored.
// Consecutive elements idx .. idx+3 (or +7) of a state tensor as floats.
__device__ __forceinline__ float bf16x2_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16x2_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <bool SB>
__device__ __forceinline__ f32x4 load_state4(const void *base, int64_t idx) {
    if constexpr (SB) {
        const u32x2 v = *reinterpret_cast<const u32x2 *>(static_cast<const uint16_t *>(base) + idx);
        return f32x4{bf16x2_lo(v[0]), bf16x2_hi(v[0]), bf16x2_lo(v[1]), bf16x2_hi(v[1])};
    } else {
        return *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
    }
}
template <bool SB>
__device__ __forceinline__ void store_state4(void *base, int64_t idx, const f32x4 &v) {
    if constexpr (SB)
        *reinterpret_cast<u32x2 *>(static_cast<uint16_t *>(base) + idx) =
            u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    else
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx) = v;
}
template <bool SB>
__device__ __forceinline__ void load_state8(const void *base, int64_t idx, float (&o)[8]) {
    if constexpr (SB) {
        const u32x4 v = *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(base) + idx);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[2 * k] = bf16x2_lo(v[k]);
            o[2 * k + 1] = bf16x2_hi(v[k]);
        }
    } else {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(base) + idx + 4);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            o[k] = a[k];
            o[4 + k] = b[k];
        }
    }
}
template <bool SB>
__device__ __forceinline__ void store_state8(void *base, int64_t idx, const float (&v)[8]) {
    if constexpr (SB) {
        *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(base) + idx) =
            u32x4{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
    } else {
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx) = f32x4{v[0], v[1], v[2], v[3]};
        *reinterpret_cast<f32x4 *>(static_cast<float *>(base) + idx + 4) = f32x4{v[4], v[5], v[6], v[7]};
    }
}

// Cumulative decay of one chunk and head ("chunk_cumsum"), by one wavefront
// whose lane l holds tokens 4l .. 4l+3 of the chunk:
//   dts_j = softplus(dt_j + dt_bias)  (dt_j + dt_bias without softplus), 0 for j >= len
//   cs2_j = log2(e) * sum_{k <= j} A dts_k                  (constant past the chunk end)
// ("mamba2_ssd_scan", "Per-token recurrence": dA = exp(A dts); the segment
// sums of "Mamba chunk scan with segsum", description).  Every kernel that
// needs these values calls this with the same inputs, so they agree bit for
// bit.  Returns cs2 of token 255, the chunk's total, in every lane.
__device__ __forceinline__ float chunk_cumsum4(const float (&dtv)[4], float bias, float A, bool softplus_on,
                                               int len, float (&dts)[4], float (&cs2)[4]) {
    const int lane = threadIdx.x & 63;
    float a[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float v = dtv[e] + bias;
        const float d = 4 * lane + e < len ? (softplus_on ? softplus_f(v) : v) : 0.0f;
        dts[e] = d;
        a[e] = A * d;
    }
    a[1] += a[0];
    a[2] += a[1];
    a[3] += a[2];
    const float incl = wave_incl_scan(a[3]);
    float excl = __shfl_up(incl, 1, 64);
    if (lane == 0) excl = 0.0f;
#pragma unroll
    for (int e = 0; e < 4; ++e) cs2[e] = (excl + a[e]) * kLog2e;
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs2[3]), 63));
}

// Whether a sequence of len tokens goes to the short-path kernel (with the
// path on, zero-length sequences go there too).
__host__ __device__ __forceinline__ bool is_short_sequence(int len, int short_max) {
    return short_max > 0 && len <= short_max;
}

// Exponent e with 2^e <= |m| < 2^(e+1) for a finite positive float m.
__device__ __forceinline__ int float_exponent(float m) {
    return (int)((__float_as_uint(m) >> 23) & 0xFF) - 127;
}

}  // namespace ssd

// Host-side launchers (one per kernel file).
namespace ssd {
// Where a kernel is launched: the stream, and events (or null) that the
// kernel's own dispatch records when it starts and when it completes, so
// timing adds no commands between kernels.
struct Launch {
    hipStream_t stream;
    hipEvent_t start;
    hipEvent_t stop;
};
template <typename K>
inline hipError_t launch_kernel(K kernel, dim3 grid, dim3 block, const Launch &l, const Params &p) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, l.stream, l.start, l.stop, 0, p);
    return hipGetLastError();
}

// Slices a group's heads are split into by the short-sequence kernel, whose
// workgroups are (sequence, group, slice): more while the grid is under four
// workgroups per compute unit (not every sequence of the batch need be
// short; workgroups of the others leave at once).  Each slice repeats the
// sequence's prologue, so a larger target costs more than it gains (the
// ragged 32-sequence workload: 2 per CU 56 us, 4: 39 us, 8: 51 us, 16: 74 us).
inline int short_head_slices(const Params &p) {
    const int hg = p.H / p.G;
    int hz = 1;
    while ((int64_t)p.batch * p.G * hz < 4 * (int64_t)p.num_cus && hg % (2 * hz) == 0) hz *= 2;
    return hz;
}

hipError_t launch_chunk_state(const Params &p, const Launch &l);
hipError_t launch_state_passing(const Params &p, const Launch &l);
hipError_t launch_chunk_scan(const Params &p, const Launch &l);
hipError_t launch_short(const Params &p, const Launch &l);
hipError_t launch_recur(const Params &p, const Launch &l);

// Copies of the size adapter (ssd_adapt.hip), launched on stream s.
hipError_t adapt_resize_rows(const void *src, void *dst, int64_t rows, int nin, int nout, int elem_bytes,
                             hipStream_t s);
hipError_t adapt_repeat(const float *src, float *dst, int64_t n_out, int m, hipStream_t s);
hipError_t adapt_gather_states(const void *src, void *area, const uint32_t *cache_idx, const uint8_t *has_init,
                               bool init_all, int batch, int H, int P, int N, int Pp, int Np, int elem_bytes,
                               hipStream_t s);
hipError_t adapt_scatter_states(const void *area, void *dst, const uint32_t *cache_idx, int batch, int H, int P,
                                int N, int Pp, int Np, int elem_bytes, hipStream_t s);
}  // namespace ssd
