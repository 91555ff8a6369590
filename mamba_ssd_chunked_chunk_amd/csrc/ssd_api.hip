// C ABI of libssd: argument checks, workspace carve and launch order.
// The entry points and their conventions are declared in include/ssd.h.
// The argument order of the in-place compute entry point follows the execute
// method of "Mamba2SSDChunkScanVarlenFwdInplace" (Modular Mojo struct docs);
// the device context becomes a HIP stream.  The other compute entry point
// (initial_states in, final_states out: "mamba2_ssd_scan", the paragraph
// after "Per-token recurrence") runs the same kernels with a different
// source and destination for the state chain.
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "ssd.h"
#include "ssd_common.hpp"

namespace {

constexpr size_t kAlign = 256;

// Scratch of the no-allocation entry point: one copy per GPU, in device
// memory for the life of the process.  Host code never uses this name as an
// address (on the host it is a stand-in, not the device location): the
// device address of the current GPU's copy comes from hipGetSymbolAddress,
// once per device, and is kept in g_scratch.
static __device__ __attribute__((aligned(256))) unsigned char scratch[SSD_NOALLOC_SCRATCH_BYTES];
constexpr int kMaxDevices = 256;
std::mutex g_scratch_mu;
void *g_scratch[kMaxDevices];

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void *ptr, size_t a) { return ((uintptr_t)ptr % a) == 0; }

ssd_status check_problem(const ssd_problem *p) {
    if (p == nullptr) return SSD_ERR_NULL_ARG;
    if (p->total_len < 0 || p->batch < 1 || p->nheads < 1 || p->head_dim < 1 ||
        p->ngroups < 1 || p->dstate < 1 || p->max_slots < 1 || p->chunk_size < 0)
        return SSD_ERR_BAD_SHAPE;
    if (p->nheads % p->ngroups != 0) return SSD_ERR_BAD_SHAPE;
    if (p->state_dtype != SSD_STATE_F32 && p->state_dtype != SSD_STATE_BF16) return SSD_ERR_UNSUPPORTED;
    if (p->total_len > INT32_MAX) return SSD_ERR_BAD_SHAPE;  // query_start_loc is int32
    if (p->dstate > SSD_MAX_DSTATE) return SSD_ERR_UNSUPPORTED;
    if (p->head_dim > SSD_MAX_HEAD_DIM) return SSD_ERR_UNSUPPORTED;
    if (p->chunk_size != 0 && p->chunk_size != ssd::kChunk) return SSD_ERR_UNSUPPORTED;
    if (p->short_path_max > SSD_SHORT_PATH_LIMIT) return SSD_ERR_UNSUPPORTED;
    // the kernels see head_dim / 64 (rounded up) heads per head
    const int64_t hk = (int64_t)p->nheads * ((p->head_dim + ssd::kHeadDim - 1) / ssd::kHeadDim);
    if (hk > 65535) return SSD_ERR_UNSUPPORTED;  // grid y limit
    const int64_t ncm = p->total_len / ssd::kChunk + p->batch;  // bounds every routing's chunk count
    if (ncm > INT32_MAX) return SSD_ERR_UNSUPPORTED;
    return SSD_OK;
}

// How a problem maps onto the sizes the scan kernels take (head_dim 64;
// dstate 64, 128 or 256), through the copies of ssd_adapt.hip.
struct Shape {
    int m;            // heads of 64 channels per head: head_dim rounded up to 64 m
    int pp, np;       // head_dim and dstate as the kernels see them
    bool pad_x;       // head_dim not a multiple of 64: x and y through padded copies
    bool pad_bc;      // dstate not 64, 128 or 256: B and C through padded copies
    bool wide;        // m > 1: dt, A, D and dt_bias repeated per 64-channel block
    bool pad_states;  // either size padded: the states through a padded area
    bool adapted() const { return pad_x || pad_bc || wide || pad_states; }
};

Shape shape_of(const ssd_problem *p) {
    Shape s;
    s.m = (p->head_dim + ssd::kHeadDim - 1) / ssd::kHeadDim;
    s.pp = s.m * ssd::kHeadDim;
    s.np = p->dstate <= 64 ? 64 : p->dstate <= 128 ? 128 : 256;
    s.pad_x = s.pp != p->head_dim;
    s.pad_bc = s.np != p->dstate;
    s.wide = s.m > 1;
    s.pad_states = s.pad_x || s.pad_bc;
    return s;
}

// The problem the kernels run: m H heads of 64 channels, dstate np; with
// padded states, one slot per sequence (the padded area).
ssd_problem core_of(const ssd_problem *p, const Shape &s) {
    ssd_problem q = *p;
    q.nheads = p->nheads * s.m;
    q.head_dim = ssd::kHeadDim;
    q.dstate = s.np;
    if (s.pad_states) q.max_slots = p->batch;
    return q;
}

size_t state_elem_bytes(const ssd_problem *p) { return p->state_dtype == SSD_STATE_BF16 ? 2 : 4; }

// Longest sequence the short path takes in this call (0: none; the path
// serves dstate up to 128 only).
int short_max_of(const ssd_problem *p) {
    if (p->dstate > 128) return 0;
    return p->short_path_max < 0 ? ssd::kShortMax : p->short_path_max;
}

// Sequences the chunked steps can see at most, and chunks they can hold: with
// the short path on, only sequences longer than its limit reach them, at most
// T / (limit + 1) of them, each with at most one partial chunk beyond
// floor(T / 256) full ones (at least 1 each: a grid dimension cannot be 0,
// and the first workgroup of chunk_state publishes the chunk count and the
// lists).
void routed_bounds(const ssd_problem *p, int *nseq, int64_t *nchunks) {
    const int sm = short_max_of(p);
    const int64_t T = p->total_len;
    *nseq = sm > 0 ? (int)std::max<int64_t>(1, std::min<int64_t>(p->batch, T / (sm + 1))) : p->batch;
    *nchunks = std::max<int64_t>(1, T / ssd::kChunk + *nseq);
}

// The kernels' part of the workspace (a problem of kernel sizes).
void core_layout_of(const ssd_problem *p, ssd_workspace_layout *L) {
    int nseq;
    int64_t ncm;
    routed_bounds(p, &nseq, &ncm);
    const size_t H = (size_t)p->nheads, G = (size_t)p->ngroups;
    const size_t PN = (size_t)p->head_dim * (size_t)p->dstate;
    size_t off = 0;
    memset(L, 0, sizeof *L);
    L->nchunks_max = ncm;
    L->meta = off;      off = align_up(off + 4 * sizeof(int32_t));
    L->chunk_off = off; off = align_up(off + ((size_t)p->batch + 1) * sizeof(int32_t));
    L->desc = off;      off = align_up(off + (size_t)ncm * 4 * sizeof(int32_t));
    L->dts = off;       off = align_up(off + (size_t)ncm * H * ssd::kChunk * sizeof(float));
    L->cs2 = off;       off = align_up(off + (size_t)ncm * H * ssd::kChunk * sizeof(float));
    L->cbt = off;       off = align_up(off + (size_t)ncm * G * 36 * 64 * 16 * sizeof(uint16_t));
    L->gexp = off;      off = align_up(off + (size_t)ncm * G * 4 * sizeof(int32_t));
    L->states = off;    off = align_up(off + (size_t)ncm * H * PN * sizeof(uint16_t));
    L->sexp = off;      off = align_up(off + (size_t)ncm * H * 2 * ((size_t)p->dstate / 32) * sizeof(int32_t));
    L->hin = off;       off = align_up(off + (size_t)ncm * H * PN * sizeof(uint16_t));
    L->hexp = off;      off = align_up(off + (size_t)ncm * H * (size_t)p->head_dim * sizeof(int32_t));
    L->xexp = off;      off = align_up(off + (size_t)ncm * H * 2 * sizeof(int32_t));
    L->seq_list = off;  off = align_up(off + (size_t)p->batch * sizeof(int32_t));
    L->recur_list = off; off = align_up(off + (size_t)p->batch * sizeof(int32_t));
    L->total_bytes = off;
}

// The whole workspace: the kernels' part for the mapped problem, then the
// copies the mapping needs (SIZE_MAX where not needed).
void layout_of(const ssd_problem *p, ssd_workspace_layout *L) {
    const Shape s = shape_of(p);
    const ssd_problem q = core_of(p, s);
    core_layout_of(&q, L);
    L->core_nheads = q.nheads;
    L->core_dstate = q.dstate;
    L->x_pad = L->y_pad = L->bc_pad = L->head_wide = L->state_pad = SIZE_MAX;
    size_t off = L->total_bytes;
    const size_t T = (size_t)p->total_len, H = (size_t)p->nheads, G = (size_t)p->ngroups;
    if (s.pad_x) {
        L->x_pad = off; off = align_up(off + T * H * (size_t)s.pp * sizeof(uint16_t));
        L->y_pad = off; off = align_up(off + T * H * (size_t)s.pp * sizeof(uint16_t));
    }
    if (s.pad_bc) {  // B, then C
        L->bc_pad = off; off = align_up(off + 2 * align_up(T * G * (size_t)s.np * sizeof(uint16_t)));
    }
    if (s.wide) {  // dt [T][m H], then A, D, dt_bias [m H]
        L->head_wide = off;
        off = align_up(off + align_up(T * H * s.m * sizeof(float)) + 3 * align_up(H * s.m * sizeof(float)));
    }
    if (s.pad_states) {
        L->state_pad = off;
        off = align_up(off + (size_t)p->batch * H * (size_t)s.pp * (size_t)s.np * state_elem_bytes(p));
    }
    L->total_bytes = off;
}

}  // namespace

extern "C" {

int ssd_abi_version(void) { return SSD_ABI_VERSION; }

const char *ssd_status_string(int s) {
    switch (s) {
    case SSD_OK: return "SSD_OK";
    case SSD_ERR_NULL_ARG: return "SSD_ERR_NULL_ARG: a required pointer is NULL";
    case SSD_ERR_BAD_SHAPE: return "SSD_ERR_BAD_SHAPE: malformed problem sizes";
    case SSD_ERR_UNSUPPORTED: return "SSD_ERR_UNSUPPORTED: sizes beyond the library's limits";
    case SSD_ERR_WORKSPACE: return "SSD_ERR_WORKSPACE: workspace missing, misaligned or too small";
    case SSD_ERR_BAD_INPUT: return "SSD_ERR_BAD_INPUT: query_start_loc or cache_indices violate a precondition";
    case SSD_ERR_HIP: return "SSD_ERR_HIP: a HIP runtime call failed";
    case SSD_ERR_SCRATCH:
        return "SSD_ERR_SCRATCH: the problem needs more scratch than the no-allocation entry point holds "
               "(SSD_NOALLOC_SCRATCH_BYTES)";
    case SSD_ERR_MISALIGNED:
        return "SSD_ERR_MISALIGNED: y, x, B, C or a state tensor is not 16-byte aligned, or dt, A, D, dt_bias, "
               "query_start_loc or cache_indices not 4-byte aligned";
    default: return "unknown ssd_status";
    }
}

ssd_status ssd_workspace_size(const ssd_problem *prob, size_t *bytes) {
    if (bytes == nullptr) return SSD_ERR_NULL_ARG;
    const ssd_status st = check_problem(prob);
    if (st != SSD_OK) return st;
    ssd_workspace_layout L;
    layout_of(prob, &L);
    *bytes = L.total_bytes;
    return SSD_OK;
}

ssd_status ssd_workspace_get_layout(const ssd_problem *prob, ssd_workspace_layout *layout) {
    if (layout == nullptr) return SSD_ERR_NULL_ARG;
    const ssd_status st = check_problem(prob);
    if (st != SSD_OK) return st;
    layout_of(prob, layout);
    return SSD_OK;
}

static const char *const kKernelNames[] = {"ssd_chunk_state", "ssd_state_passing", "ssd_chunk_scan", "ssd_short",
                                           "ssd_recur"};
static constexpr int kNumKernels = 5;
static constexpr int kFirstShortKernel = 3;  // this and the later ones serve the short path

int ssd_kernel_count(void) { return kNumKernels; }

const char *ssd_kernel_name(int i) { return (i >= 0 && i < kNumKernels) ? kKernelNames[i] : nullptr; }

// Where the state chain starts and ends (see Params::state_in).
struct StateIO {
    const void *in;
    void *out;
    const uint8_t *has_init;
    const uint32_t *cache_idx;
    bool init_all;
};

// Host checks of a compute call's problem and tensor pointers (everything but
// the workspace): nothing here touches the device.
static ssd_status check_call(const ssd_problem *prob, const void *y, const void *x, const float *dt,
                             const float *A, const void *B, const void *C, const float *D, const float *dt_bias,
                             const int32_t *query_start_loc, const StateIO &sio) {
    ssd_status st = check_problem(prob);
    if (st != SSD_OK) return st;
    const bool has_tokens = prob->total_len > 0;
    if (A == nullptr || sio.out == nullptr || query_start_loc == nullptr || (sio.init_all && sio.in == nullptr))
        return SSD_ERR_NULL_ARG;
    if (has_tokens && (y == nullptr || x == nullptr || dt == nullptr || B == nullptr || C == nullptr))
        return SSD_ERR_NULL_ARG;
    if (!aligned(y, 16) || !aligned(x, 16) || !aligned(B, 16) || !aligned(C, 16) ||
        !aligned(sio.out, 16) || !aligned(sio.in, 16) || !aligned(dt, 4) || !aligned(A, 4) ||
        !aligned(D, 4) || !aligned(dt_bias, 4) || !aligned(query_start_loc, 4) || !aligned(sio.cache_idx, 4))
        return SSD_ERR_MISALIGNED;
    return SSD_OK;
}

// The scan kernels on a problem of their sizes (head_dim 64; dstate 64, 128
// or 256), with the workspace carved as L.
static ssd_status run_core(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    const int32_t *query_start_loc, const StateIO &sio, char *ws, const ssd_workspace_layout &L,
    void *stream, void *const *events) {
    ssd::Params p;
    p.T = prob->total_len;
    p.batch = prob->batch;
    p.H = prob->nheads;
    p.P = prob->head_dim;
    p.G = prob->ngroups;
    p.N = prob->dstate;
    p.max_slots = prob->max_slots;
    p.dt_softplus = prob->dt_softplus != 0;
    p.nchunks_max = L.nchunks_max;
    {
        int dev = 0, cus = 0;
        if (hipGetDevice(&dev) != hipSuccess ||
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            return SSD_ERR_HIP;
        p.num_cus = cus > 0 ? cus : 256;
    }
    p.y = static_cast<uint16_t *>(y);
    p.x = static_cast<const uint16_t *>(x);
    p.dt = dt;
    p.A = A;
    p.B = static_cast<const uint16_t *>(B);
    p.C = static_cast<const uint16_t *>(C);
    p.D = D;
    p.dt_bias = dt_bias;
    p.qsl = query_start_loc;
    p.state_in = sio.in;
    p.state_out = sio.out;
    p.has_init = sio.has_init;
    p.cache_idx = sio.cache_idx;
    p.init_all = sio.init_all ? 1 : 0;
    p.state_bf16 = prob->state_dtype == SSD_STATE_BF16 ? 1 : 0;
    // the short path serves dstate 64 and 128; the route of a sequence
    // depends on its own length only, so its results do not depend on the
    // rest of the batch
    p.short_max = short_max_of(prob);
    p.recur_max = std::min(p.short_max, ssd::kRecurMax);
    // the launches are sized to the bounds on what the routing lets reach the
    // chunked steps (the workspace tables have that many rows)
    routed_bounds(prob, &p.nseq_grid, &p.nchunks_grid);
    p.meta = reinterpret_cast<int32_t *>(ws + L.meta);
    p.chunk_off = reinterpret_cast<int32_t *>(ws + L.chunk_off);
    p.desc = reinterpret_cast<int4 *>(ws + L.desc);
    p.dts = reinterpret_cast<float *>(ws + L.dts);
    p.cs2 = reinterpret_cast<float *>(ws + L.cs2);
    p.hexp = reinterpret_cast<int32_t *>(ws + L.hexp);
    p.xexp = reinterpret_cast<int32_t *>(ws + L.xexp);
    p.seq_list = reinterpret_cast<int32_t *>(ws + L.seq_list);
    p.recur_list = reinterpret_cast<int32_t *>(ws + L.recur_list);
    p.cbt = reinterpret_cast<uint16_t *>(ws + L.cbt);
    p.gexp = reinterpret_cast<int32_t *>(ws + L.gexp);
    p.hin = reinterpret_cast<uint16_t *>(ws + L.hin);
    p.states = reinterpret_cast<uint16_t *>(ws + L.states);
    p.sexp = reinterpret_cast<int32_t *>(ws + L.sexp);

    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t (*const launchers[kNumKernels])(const ssd::Params &, const ssd::Launch &) = {
        ssd::launch_chunk_state, ssd::launch_state_passing, ssd::launch_chunk_scan, ssd::launch_short,
        ssd::launch_recur};
    // no sequence can take the short path (it is off, or the call's one
    // sequence is longer than its limit): its kernels would have nothing to
    // do, so they are not launched (their completion events, if any, are
    // recorded on the stream where they would have run)
    const bool no_short = p.short_max == 0 || (prob->batch == 1 && prob->total_len > p.short_max);
    for (int k = 0; k < kNumKernels; ++k) {
        if (k >= kFirstShortKernel && no_short) {
            if (events && hipEventRecord(static_cast<hipEvent_t>(events[k + 1]), s) != hipSuccess) return SSD_ERR_HIP;
            continue;
        }
        // events, if any, are recorded by the dispatches themselves: the start
        // of the first kernel and the end of every kernel
        const ssd::Launch l{s, events && k == 0 ? static_cast<hipEvent_t>(events[0]) : nullptr,
                            events ? static_cast<hipEvent_t>(events[k + 1]) : nullptr};
        if (launchers[k](p, l) != hipSuccess) return SSD_ERR_HIP;
    }
    return SSD_OK;
}

static ssd_status run_scan(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    const int32_t *query_start_loc, const StateIO &sio, void *workspace, size_t workspace_bytes,
    void *stream, void *const *events) {
    ssd_status st = check_call(prob, y, x, dt, A, B, C, D, dt_bias, query_start_loc, sio);
    if (st != SSD_OK) return st;
    ssd_workspace_layout L;
    layout_of(prob, &L);
    if (workspace == nullptr || workspace_bytes < L.total_bytes || !aligned(workspace, kAlign))
        return SSD_ERR_WORKSPACE;
    char *ws = static_cast<char *>(workspace);
    const Shape sh = shape_of(prob);
    if (!sh.adapted())
        return run_core(prob, y, x, dt, A, B, C, D, dt_bias, query_start_loc, sio, ws, L, stream, events);

    // Other sizes: copies into the kernels' sizes, the scan, copies back
    // (ssd_adapt.hip).  Only the scan's kernels carry the events.
    const ssd_problem q = core_of(prob, sh);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const int64_t T = prob->total_len;
    const int H = prob->nheads, G = prob->ngroups, P = prob->head_dim, N = prob->dstate;
    const int es = (int)state_elem_bytes(prob);
    const void *xk = x, *Bk = B, *Ck = C;
    void *yk = y;
    const float *dtk = dt, *Ak = A, *Dk = D, *biask = dt_bias;
    StateIO sk = sio;
    auto ok = [](hipError_t e) { return e == hipSuccess; };
    if (sh.pad_x && T > 0) {
        xk = ws + L.x_pad;
        yk = ws + L.y_pad;
        if (!ok(ssd::adapt_resize_rows(x, ws + L.x_pad, T * H, P, sh.pp, 2, s))) return SSD_ERR_HIP;
    }
    if (sh.pad_bc && T > 0) {
        char *bp = ws + L.bc_pad;
        char *cp = bp + align_up((size_t)T * G * sh.np * sizeof(uint16_t));
        Bk = bp;
        Ck = cp;
        if (!ok(ssd::adapt_resize_rows(B, bp, T * G, N, sh.np, 2, s)) ||
            !ok(ssd::adapt_resize_rows(C, cp, T * G, N, sh.np, 2, s)))
            return SSD_ERR_HIP;
    }
    if (sh.wide) {
        float *w = reinterpret_cast<float *>(ws + L.head_wide);
        const size_t hs = align_up((size_t)H * sh.m * sizeof(float)) / sizeof(float);
        float *dtw = w, *aw = w + align_up((size_t)T * H * sh.m * sizeof(float)) / sizeof(float);
        float *dw = aw + hs, *bw = dw + hs;
        if (T > 0) {
            if (!ok(ssd::adapt_repeat(dt, dtw, T * H * sh.m, sh.m, s))) return SSD_ERR_HIP;
            dtk = dtw;
        }
        if (!ok(ssd::adapt_repeat(A, aw, (int64_t)H * sh.m, sh.m, s))) return SSD_ERR_HIP;
        Ak = aw;
        if (D != nullptr) {
            if (!ok(ssd::adapt_repeat(D, dw, (int64_t)H * sh.m, sh.m, s))) return SSD_ERR_HIP;
            Dk = dw;
        }
        if (dt_bias != nullptr) {
            if (!ok(ssd::adapt_repeat(dt_bias, bw, (int64_t)H * sh.m, sh.m, s))) return SSD_ERR_HIP;
            biask = bw;
        }
    }
    if (sh.pad_states) {
        // every sequence's initial state (zeros without one) into the padded
        // area, which is then each sequence's initial and final state
        void *area = ws + L.state_pad;
        if (!ok(ssd::adapt_gather_states(sio.in, area, sio.cache_idx, sio.has_init, sio.init_all, prob->batch, H,
                                         P, N, sh.pp, sh.np, es, s)))
            return SSD_ERR_HIP;
        sk = StateIO{area, area, nullptr, nullptr, true};
    }
    st = run_core(&q, yk, xk, dtk, Ak, Bk, Ck, Dk, biask, query_start_loc, sk, ws, L, stream, events);
    if (st != SSD_OK) return st;
    if (sh.pad_x && T > 0 && !ok(ssd::adapt_resize_rows(ws + L.y_pad, y, T * H, sh.pp, P, 2, s)))
        return SSD_ERR_HIP;
    if (sh.pad_states && !ok(ssd::adapt_scatter_states(ws + L.state_pad, sio.out, sio.cache_idx, prob->batch, H,
                                                        P, N, sh.pp, sh.np, es, s)))
        return SSD_ERR_HIP;
    return SSD_OK;
}

static ssd_status inplace(const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
                          const void *B, const void *C, const float *D, const float *dt_bias, void *ssm_pool,
                          const int32_t *query_start_loc, const uint8_t *has_initial_state,
                          const uint32_t *cache_indices, void *workspace, size_t workspace_bytes, void *stream,
                          void *const *events) {
    if (ssm_pool == nullptr || cache_indices == nullptr) return SSD_ERR_NULL_ARG;
    const StateIO sio{ssm_pool, ssm_pool, has_initial_state, cache_indices, false};
    return run_scan(prob, y, x, dt, A, B, C, D, dt_bias, query_start_loc, sio, workspace, workspace_bytes,
                    stream, events);
}

// The current device's copy of the scratch array (looked up on its first use).
static ssd_status scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return SSD_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return SSD_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void *ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return SSD_ERR_HIP;
        g_scratch[dev] = ptr;
    }
    *out = g_scratch[dev];
    return SSD_OK;
}

static ssd_status separate(const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
                           const void *B, const void *C, const float *D, const float *dt_bias,
                           const void *initial_states, void *final_states, const int32_t *query_start_loc,
                           void *workspace, size_t workspace_bytes, void *stream, void *const *events) {
    if (prob == nullptr) return SSD_ERR_NULL_ARG;
    ssd_problem q = *prob;  // no pool: the state tensors have one slot per sequence
    q.max_slots = q.batch;
    const StateIO sio{initial_states, final_states, nullptr, nullptr, initial_states != nullptr};
    return run_scan(&q, y, x, dt, A, B, C, D, dt_bias, query_start_loc, sio, workspace, workspace_bytes,
                    stream, events);
}

static ssd_status check_events(void *const *events, int n_events) {
    if (events == nullptr) return SSD_ERR_NULL_ARG;
    if (n_events != kNumKernels + 1) return SSD_ERR_BAD_SHAPE;
    for (int k = 0; k <= kNumKernels; ++k)
        if (events[k] == nullptr) return SSD_ERR_NULL_ARG;
    return SSD_OK;
}

ssd_status ssd_chunk_scan_varlen_fwd_inplace(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias, void *ssm_pool,
    const int32_t *query_start_loc, const uint8_t *has_initial_state,
    const uint32_t *cache_indices, void *workspace, size_t workspace_bytes, void *stream) {
    return inplace(prob, y, x, dt, A, B, C, D, dt_bias, ssm_pool, query_start_loc, has_initial_state,
                   cache_indices, workspace, workspace_bytes, stream, nullptr);
}

ssd_status ssd_chunk_scan_varlen_fwd_inplace_noalloc(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias, void *ssm_pool,
    const int32_t *query_start_loc, const uint8_t *has_initial_state,
    const uint32_t *cache_indices, void *stream) {
    // every host check first, so a rejected call touches no device state
    if (ssm_pool == nullptr || cache_indices == nullptr) return SSD_ERR_NULL_ARG;
    const StateIO sio{ssm_pool, ssm_pool, has_initial_state, cache_indices, false};
    ssd_status st = check_call(prob, y, x, dt, A, B, C, D, dt_bias, query_start_loc, sio);
    if (st != SSD_OK) return st;
    size_t need = 0;
    st = ssd_workspace_size(prob, &need);
    if (st != SSD_OK) return st;
    if (need > SSD_NOALLOC_SCRATCH_BYTES) return SSD_ERR_SCRATCH;
    void *ws = nullptr;
    st = scratch_address(&ws);
    if (st != SSD_OK) return st;
    return inplace(prob, y, x, dt, A, B, C, D, dt_bias, ssm_pool, query_start_loc, has_initial_state,
                   cache_indices, ws, SSD_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

ssd_status ssd_chunk_scan_varlen_fwd_inplace_profiled(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias, void *ssm_pool,
    const int32_t *query_start_loc, const uint8_t *has_initial_state,
    const uint32_t *cache_indices, void *workspace, size_t workspace_bytes, void *stream,
    void *const *events, int n_events) {
    const ssd_status st = check_events(events, n_events);
    if (st != SSD_OK) return st;
    return inplace(prob, y, x, dt, A, B, C, D, dt_bias, ssm_pool, query_start_loc, has_initial_state,
                   cache_indices, workspace, workspace_bytes, stream, events);
}

ssd_status ssd_chunk_scan_varlen_fwd(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias, const void *initial_states,
    void *final_states, const int32_t *query_start_loc, void *workspace, size_t workspace_bytes,
    void *stream) {
    return separate(prob, y, x, dt, A, B, C, D, dt_bias, initial_states, final_states, query_start_loc,
                    workspace, workspace_bytes, stream, nullptr);
}

ssd_status ssd_chunk_scan_varlen_fwd_profiled(
    const ssd_problem *prob, void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias, const void *initial_states,
    void *final_states, const int32_t *query_start_loc, void *workspace, size_t workspace_bytes,
    void *stream, void *const *events, int n_events) {
    const ssd_status st = check_events(events, n_events);
    if (st != SSD_OK) return st;
    return separate(prob, y, x, dt, A, B, C, D, dt_bias, initial_states, final_states, query_start_loc,
                    workspace, workspace_bytes, stream, events);
}

ssd_status ssd_validate_inputs(const ssd_problem *prob, const int32_t *query_start_loc,
                               const uint32_t *cache_indices, void *stream) {
    ssd_status st = check_problem(prob);
    if (st != SSD_OK) return st;
    if (query_start_loc == nullptr || cache_indices == nullptr) return SSD_ERR_NULL_ARG;
    std::vector<int32_t> q((size_t)prob->batch + 1);
    std::vector<uint32_t> ci((size_t)prob->batch);
    if (hipStreamSynchronize(static_cast<hipStream_t>(stream)) != hipSuccess) return SSD_ERR_HIP;
    if (hipMemcpy(q.data(), query_start_loc, q.size() * sizeof(int32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return SSD_ERR_HIP;
    if (hipMemcpy(ci.data(), cache_indices, ci.size() * sizeof(uint32_t), hipMemcpyDeviceToHost) != hipSuccess)
        return SSD_ERR_HIP;
    if (q[0] != 0 || (int64_t)q[(size_t)prob->batch] != prob->total_len) return SSD_ERR_BAD_INPUT;
    for (int b = 0; b < prob->batch; ++b)
        if (q[(size_t)b + 1] < q[(size_t)b]) return SSD_ERR_BAD_INPUT;
    std::vector<uint8_t> seen((size_t)prob->max_slots, 0);
    for (int b = 0; b < prob->batch; ++b) {
        if (ci[(size_t)b] >= (uint32_t)prob->max_slots) return SSD_ERR_BAD_INPUT;
        if (seen[ci[(size_t)b]]) return SSD_ERR_BAD_INPUT;
        seen[ci[(size_t)b]] = 1;
    }
    return SSD_OK;
}

}  // extern "C"
