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
// Plain grid-stride kernels, one wavefront per row of the destination.
#include "ssd_common.hpp"

namespace ssd {

namespace {
constexpr int kAdaptThreads = 256;
constexpr int kRowsPerBlock = kAdaptThreads / 64;  // one wavefront per row at a time
constexpr int64_t kAdaptMaxBlocks = 16384;

dim3 adapt_grid(int64_t rows) {
    return dim3((unsigned)std::max<int64_t>(
        1, std::min<int64_t>((rows + kRowsPerBlock - 1) / kRowsPerBlock, kAdaptMaxBlocks)));
}

// rows rows of nin elements into rows of nout elements: element c of a row
// is the source's when c < nin, else 0.  Each wavefront copies whole rows,
// its lanes along the row.
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_resize_rows_kernel(const E *src, E *dst, int64_t rows,
                                                                        int nin, int nout) {
    const int lane = threadIdx.x & 63;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < rows;
         r += (int64_t)gridDim.x * kRowsPerBlock) {
        const E *s = src + r * nin;
        E *d = dst + r * nout;
        for (int c = lane; c < nout; c += 64) d[c] = c < nin ? s[c] : E(0);
    }
}

// n_src values, each written m times in a row
__global__ __launch_bounds__(kAdaptThreads) void ssd_repeat_kernel(const float *src, float *dst, int64_t n_src,
                                                                   int m) {
    const int64_t stride = (int64_t)gridDim.x * kAdaptThreads;
    for (int64_t j = (int64_t)blockIdx.x * kAdaptThreads + threadIdx.x; j < n_src; j += stride) {
        const float v = src[j];
        for (int s = 0; s < m; ++s) dst[j * m + s] = v;
    }
}

// area[b][h][p][n] (P' x N') = sequence b's initial state at [slot][h][p][n]
// (P x N), 0 past P or N and for a sequence without one.  slot =
// cache_idx[b], or b without cache_idx; a sequence has an initial state when
// init_all is set or has_init[b] != 0 (has_init may be NULL: none).  One
// wavefront per row (b, h, p) of the area.
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_gather_states_kernel(
    const E *src, E *area, const uint32_t *cache_idx, const uint8_t *has_init, int init_all, int batch, int H,
    int P, int N, int Pp, int Np) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)batch * H * Pp;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < rows;
         r += (int64_t)gridDim.x * kRowsPerBlock) {
        const int p = (int)(r % Pp);
        const int64_t bh = r / Pp;
        const int h = (int)(bh % H);
        const int b = (int)(bh / H);
        const bool init = init_all != 0 || (has_init != nullptr && has_init[b] != 0);
        E *d = area + r * Np;
        if (init && p < P) {
            const int64_t slot = cache_idx != nullptr ? (int64_t)cache_idx[b] : b;
            const E *s = src + ((slot * H + h) * P + p) * N;
            for (int n = lane; n < Np; n += 64) d[n] = n < N ? s[n] : E(0);
        } else {
            for (int n = lane; n < Np; n += 64) d[n] = E(0);
        }
    }
}

// dst[slot][h][p][n] = area[b][h][p][n] for p < P, n < N (slot as above);
// one wavefront per row (b, h, p) of the destination
template <typename E>
__global__ __launch_bounds__(kAdaptThreads) void ssd_scatter_states_kernel(
    const E *area, E *dst, const uint32_t *cache_idx, int batch, int H, int P, int N, int Pp, int Np) {
    const int lane = threadIdx.x & 63;
    const int64_t rows = (int64_t)batch * H * P;
    for (int64_t r = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6); r < rows;
         r += (int64_t)gridDim.x * kRowsPerBlock) {
        const int p = (int)(r % P);
        const int64_t bh = r / P;
        const int h = (int)(bh % H);
        const int b = (int)(bh / H);
        const int64_t slot = cache_idx != nullptr ? (int64_t)cache_idx[b] : b;
        const E *s = area + (bh * Pp + p) * Np;
        E *d = dst + ((slot * H + h) * P + p) * N;
        for (int n = lane; n < N; n += 64) d[n] = s[n];
    }
}
}  // namespace

hipError_t adapt_resize_rows(const void *src, void *dst, int64_t rows, int nin, int nout, int elem_bytes,
                             hipStream_t s) {
    if (rows <= 0 || nout <= 0) return hipSuccess;
    const int64_t n = rows;
    if (elem_bytes == 2)
        hipLaunchKernelGGL(ssd_resize_rows_kernel<uint16_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint16_t *>(src), static_cast<uint16_t *>(dst), rows, nin, nout);
    else
        hipLaunchKernelGGL(ssd_resize_rows_kernel<uint32_t>, adapt_grid(n), dim3(kAdaptThreads), 0, s,
                           static_cast<const uint32_t *>(src), static_cast<uint32_t *>(dst), rows, nin, nout);
    return hipGetLastError();
}

hipError_t adapt_repeat(const float *src, float *dst, int64_t n_out, int m, hipStream_t s) {
    const int64_t n_src = n_out / m;
    if (n_src <= 0) return hipSuccess;
    const dim3 grid((unsigned)std::max<int64_t>(
        1, std::min<int64_t>((n_src + kAdaptThreads - 1) / kAdaptThreads, kAdaptMaxBlocks)));
    hipLaunchKernelGGL(ssd_repeat_kernel, grid, dim3(kAdaptThreads), 0, s, src, dst, n_src, m);
    return hipGetLastError();
}

hipError_t adapt_gather_states(const void *src, void *area, const uint32_t *cache_idx, const uint8_t *has_init,
                               bool init_all, int batch, int H, int P, int N, int Pp, int Np, int elem_bytes,
                               hipStream_t s) {
    const int64_t n = (int64_t)batch * H * Pp;  // rows
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
    const int64_t n = (int64_t)batch * H * P;  // rows
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
