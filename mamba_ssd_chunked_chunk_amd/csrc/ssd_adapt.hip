// Copies that map a problem onto the sizes the scan kernels take: head_dim 64
// and dstate 64, 128 or 256.  The pages allow any dstate up to 256
// ("mamba2_ssd_scan", comptime MAX_DSTATE) and do not fix head_dim.
//   - dstate N below 256 and not 64 or 128: B and C are copied into rows of the
//     next of 64, 128, 256 with zeros past N.  A zero column of B and C adds
//     nothing to any product, and its state column stays 0.
//   - head_dim P: rounded up to a multiple of 64 (x copied into zero-padded
//     rows, y cropped back); the 64 P / 64 channel blocks of a head then run
//     as that many heads of 64 channels, each with the head's dt, A, D and
//     dt_bias (repeated).  Head h's block s is head h m + s of the copy, whose
//     group (h m + s) / (m H / G) is h's group.  The per-token recurrence
//     ("Per-token recurrence") treats every channel p on its own, so the
//     split changes no value.
//   - states, when either size is padded: each sequence's initial state is
//     copied into a zero-padded [batch][H][P'][N'] area (zeros when it has
//     none), the scan runs on that area as its own initial and final states,
//     and each final state is copied back into its slot, cropped.
// Plain grid-stride kernels over the destination's elements.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kAdaptThreads = 256;
constexpr int64_t kAdaptMaxBlocks = 16384;

dim3 adapt_grid(int64_t n) {
    return dim3((unsigned)std::max<int64_t>(1, std::min<int64_t>((n + kAdaptThreads - 1) / kAdaptThreads,
                                                                 kAdaptMaxBlocks)));
}

// rows rows of nin elements into rows of nout elements: element c of a row
// is the source's when c < nin, else 0
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_resize_rows_kernel(const E *src, E *dst, int64_t rows,
                                                                        int nin, int nout) {
    const int64_t total = rows * nout;
    const int64_t stride = (int64_t)gridDim.x * kAdaptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / nout;
        const int c = (int)(i - r * nout);
        dst[i] = c < nin ? src[r * nin + c] : E(0);
    }
}

// n_out values, each source value repeated m times in a row
__global__ __launch_bounds__(kAdaptThreads) void ssd_repeat_kernel(const float *src, float *dst, int64_t n_out,
                                                                   int m) {
    const int64_t stride = (int64_t)gridDim.x * kAdaptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x; i < n_out; i += stride)
        dst[i] = src[i / m];
}

// area[b][h][p][n] (P' x N') = sequence b's initial state at [slot][h][p][n]
// (P x N), 0 past P or N and for a sequence without one.  slot =
// cache_idx[b], or b without cache_idx; a sequence has an initial state when
// init_all is set or has_init[b] != 0 (has_init may be NULL: none).
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_gather_states_kernel(
    const E *src, E *area, const uint32_t *cache_idx, const uint8_t *has_init, int init_all, int batch, int H,
    int P, int N, int Pp, int Np) {
    const int64_t total = (int64_t)batch * H * Pp * Np;
    const int64_t stride = (int64_t)gridDim.x * kAdaptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x; i < total; i += stride) {
        int64_t r = i / Np;
        const int n = (int)(i - r * Np);
        const int p = (int)(r % Pp);
        r /= Pp;
        const int h = (int)(r % H);
        const int b = (int)(r / H);
        const bool init = init_all != 0 || (has_init != nullptr && has_init[b] != 0);
        E v = E(0);
        if (init && p < P && n < N) {
            const int64_t slot = cache_idx != nullptr ? (int64_t)cache_idx[b] : b;
            v = src[((slot * H + h) * P + p) * N + n];
        }
        area[i] = v;
    }
}

// dst[slot][h][p][n] = area[b][h][p][n] for p < P, n < N (slot as above)
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_scatter_states_kernel(
    const E *area, E *dst, const uint32_t *cache_idx, int batch, int H, int P, int N, int Pp, int Np) {
    const int64_t total = (int64_t)batch * H * P * N;
    const int64_t stride = (int64_t)gridDim.x * kAdaptThreads;
    for (int64_t i = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x; i < total; i += stride) {
        int64_t r = i / N;
        const int n = (int)(i - r * N);
        const int p = (int)(r % P);
        r /= P;
        const int h = (int)(r % H);
        const int b = (int)(r / H);
        const int64_t slot = cache_idx != nullptr ? (int64_t)cache_idx[b] : b;
        dst[((slot * H + h) * P + p) * N + n] = area[((int64_t)(b * (int64_t)H + h) * Pp + p) * Np + n];
    }
}
}  // namespace

hipError_t adapt_resize_rows(const void *src, void *dst, int64_t rows, int nin, int nout, int elem_bytes,
                             hipStream_t s) {
    const int64_t n = rows * nout;
    if (n <= 0) return hipSuccess;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(ssd_resize_rows_kernel<uint16_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), rows, nin, nout);
    else
        hipLaunchKernelGGL(ssd_resize_rows_kernel<uint32_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint32_t *>(src), static_cast<uint32_t *>(dst), rows, nin, nout);
    return hipGetLastError();
}

hipError_t adapt_repeat(const float *src, float *dst, int64_t n_out, int m, hipStream_t s) {
    if (n_out <= 0) return hipSuccess;
    hipLaunchKernelGGL(ssd_repeat_kernel, adapt_grid(n_out), dim3(kAdaptThreads), 0, s, src, dst, n_out, m);
    return hipGetLastError();
}

hipError_t adapt_gather_states(const void *src, void *area, const uint32_t *cache_idx, const uint8_t *has_init,
                               bool init_all, int batch, int H, int P, int N, int Pp, int Np, int elem_bytes,
                               hipStream_t s) {
    const int64_t n = (int64_t)batch * H * Pp * Np;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(ssd_gather_states_kernel<uint16_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(area), cache_idx, has_init,
                           init_all ? 1 : 0, batch, H, P, N, Pp, Np);
    else
        hipLaunchKernelGGL(ssd_gather_states_kernel<uint32_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint32_t *>(src), static_cast<uint32_t *>(area), cache_idx, has_init,
                           init_all ? 1 : 0, batch, H, P, N, Pp, Np);
    return hipGetLastError();
}

hipError_t adapt_scatter_states(const void *area, void *dst, const uint32_t *cache_idx, int batch, int H, int P,
                                int N, int Pp, int Np, int elem_bytes, hipStream_t s) {
    const int64_t n = (int64_t)batch * H * P * N;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(ssd_scatter_states_kernel<uint16_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint16_t *>(area), static_cast<uint16_t *>(dst), cache_idx, batch, H,
                           P, N, Pp, Np);
    else
        hipLaunchKernelGGL(ssd_scatter_states_kernel<uint32_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint32_t *>(area), static_cast<uint32_t *>(dst), cache_idx, batch, H,
                           P, N, Pp, Np);
    return hipGetLastError();
}

}  // namespace ssd
