/*
 * libssd -- Mamba-2 SSD (state-space duality) varlen forward prefill scan
 * for AMD Instinct MI355X (gfx950).  C ABI.
 *
 * The operation (what every entry point below computes) is defined by the
 * per-token recurrence in "mamba2_ssd_scan" (Modular MAX kernels docs),
 * section "Per-token recurrence": for each head h, head_dim channel p and
 * group g = h / (nheads / ngroups),
 *     dts   = softplus(dt[t,h] + dt_bias[h])       (or dt + dt_bias when
 *                                                  dt_softplus is 0)
 *     state = state * exp(A[h] * dts) + dts * B[t,g,:] * x[t,h,p]
 *     y[t,h,p] = C[t,g,:] . state + D[h] * x[t,h,p]
 * with the state reset at every query_start_loc boundary.  The in-place pool
 * semantics (initial state read from ssm_pool[cache_indices[b]] when
 * has_initial_state[b] is set; final state written to the same slot) and the
 * tensor shapes follow "Mamba2SSDChunkScanVarlenFwdInplace" (Modular Mojo
 * struct docs), struct description, "Tensor shapes" and "Parameters".  The
 * GPU path evaluates it with the chunked segment-sum reformulation described
 * on "Mamba chunk scan with segsum" (kernelindex.com, operation 043).
 *
 * Conventions shared by all entry points:
 *   - All tensor pointers are DEVICE pointers to dense, row-major
 *     (C-contiguous) buffers owned by the caller.  The library allocates no
 *     device memory and keeps no pointer after a call returns.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Compute entry points are asynchronous and stream-ordered: they enqueue
 *     kernels and return without synchronising the host.
 *   - Host-side argument checks run before anything is enqueued; on any
 *     error status nothing is launched and no buffer is modified.
 *   - Device-side preconditions (query_start_loc[0] == 0, non-decreasing,
 *     query_start_loc[batch] == total_len; cache_indices[b] < max_slots and
 *     pairwise distinct) are NOT checked on the hot path (that would need a
 *     host synchronisation); ssd_validate_inputs checks them on demand.
 *     Violating them is undefined behaviour.
 *   - y must not alias any input; ssm_pool is the only read-write buffer.
 *   - Alignment: y, x, B, C and the state tensors (ssm_pool,
 *     initial_states, final_states) must start on a 16-byte boundary (the
 *     kernels move them 16 bytes per lane); dt, A, D, dt_bias,
 *     query_start_loc and cache_indices on a 4-byte boundary; the workspace
 *     on a 256-byte boundary.  Buffers from hipMalloc, or whole torch
 *     tensors, satisfy this; a view that starts mid-row (x[1:] of a tensor
 *     whose rows are not a multiple of 16 bytes, ...) may not.  A misaligned
 *     tensor gives SSD_ERR_MISALIGNED, a misaligned workspace
 *     SSD_ERR_WORKSPACE, before any launch.
 *   - Every option is passed per call in ssd_problem: the library keeps no
 *     mutable state, so concurrent calls (other host threads, other
 *     streams) and captured graphs see exactly the options they were given.
 *   - A call that fails while kernels run (SSD_ERR_HIP from a later status
 *     query) may leave the pool partially written.
 */
#ifndef LIBSSD_SSD_H
#define LIBSSD_SSD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SSD_ABI_VERSION 18
#define SSD_MAX_DSTATE 256  /* largest dstate, as in "mamba2_ssd_scan", comptime MAX_DSTATE */
#define SSD_MAX_HEAD_DIM 1024  /* largest head_dim the library takes (the pages fix none) */
#define SSD_SHORT_PATH_LIMIT 128  /* longest sequence the short path can take */
#define SSD_RECUR_LIMIT 4         /* of those, the longest the token recurrence takes */
/* element types of the state tensors (ssd_problem.state_dtype) */
#define SSD_STATE_F32 0
#define SSD_STATE_BF16 1

typedef enum ssd_status {
    SSD_OK = 0,
    SSD_ERR_NULL_ARG = 1,     /* a required pointer is NULL                     */
    SSD_ERR_BAD_SHAPE = 2,    /* negative/zero sizes, nheads % ngroups != 0 ...  */
    SSD_ERR_UNSUPPORTED = 3,  /* a size beyond the library's limits             */
    SSD_ERR_WORKSPACE = 4,    /* workspace NULL or smaller than required         */
    SSD_ERR_BAD_INPUT = 5,    /* ssd_validate_inputs found a violated precondition */
    SSD_ERR_HIP = 6,          /* a HIP runtime call or kernel launch failed       */
    SSD_ERR_MISALIGNED = 7,   /* a tensor pointer breaks the alignment rule above */
    SSD_ERR_SCRATCH = 8       /* the problem needs more scratch than the
                               * no-allocation entry point holds
                               * (SSD_NOALLOC_SCRATCH_BYTES)                  */
} ssd_status;

/* Problem sizes.  Dense row-major tensors:
 *   y, x           [total_len, nheads, head_dim]   bf16
 *   dt             [total_len, nheads]             fp32
 *   A, D, dt_bias  [nheads]                        fp32 (D, dt_bias optional)
 *   B, C           [total_len, ngroups, dstate]    bf16
 *   ssm_pool       [max_slots, nheads, head_dim, dstate]  fp32, or bf16 with
 *                  state_dtype = SSD_STATE_BF16 (also initial_states and
 *                  final_states of the separate-states entry point)
 *   query_start_loc [batch + 1] int32, has_initial_state [batch] uint8
 *   (optional), cache_indices [batch] uint32                                */
typedef struct ssd_problem {
    int64_t total_len;   /* T == query_start_loc[batch]; >= 0                */
    int32_t batch;       /* number of sequences; >= 1                         */
    int32_t nheads;      /* H; multiple of ngroups                            */
    int32_t head_dim;    /* P; 1 .. SSD_MAX_HEAD_DIM (see "Sizes" below)       */
    int32_t ngroups;     /* G                                                 */
    int32_t dstate;      /* N; 1 .. SSD_MAX_DSTATE (see "Sizes" below)        */
    int32_t max_slots;   /* leading dimension of ssm_pool; >= 1               */
    int32_t chunk_size;  /* 0 selects 256; only 256 is supported             */
    int32_t dt_softplus; /* nonzero: dts = softplus(dt + dt_bias); zero: dt + dt_bias */
    int32_t state_dtype; /* SSD_STATE_F32 or SSD_STATE_BF16: storage type of the states
                          * ("Mamba2SSDChunkScanVarlenFwdInplace": execute's state_dtype
                          * parameter; "Tensor shapes": a bf16 pool is storage only, the
                          * scan accumulates in fp32).  With bf16, initial states are read
                          * from bf16, the state chain and all arithmetic stay fp32, and
                          * each final state is rounded to bf16 (nearest even) once, when
                          * it is written */
    int32_t short_path_max; /* longest sequence the short path takes (see below):
                          * 0 = none (every sequence through the chunked steps),
                          * 1 .. SSD_SHORT_PATH_LIMIT, or any negative value for
                          * the default SSD_SHORT_PATH_LIMIT; larger values give
                          * SSD_ERR_UNSUPPORTED.  Only dstate up to 128 has a
                          * short path; above 128 the field is ignored. */
} ssd_problem;

/* Sizes.  The scan kernels take head_dim 64 and dstate 64, 128 or 256.  Other
 * sizes run on them through copies in the workspace (ssd_workspace_layout's
 * x_pad .. state_pad): dstate is rounded up to the next of 64, 128, 256 (B and
 * C copied with zero columns), head_dim up to a multiple of 64 (x copied with
 * zero channels, y cropped back), each 64-channel block of a head runs as a
 * head of its own (dt, A, D and dt_bias repeated per block; no copy of x, y
 * or the states when head_dim is a multiple of 64), and when either size is
 * padded the states pass through a zero-padded area of one slot per sequence
 * (copied in from the slots read, copied back into the slots written).  The
 * results are those of the same recurrence; only the time and the workspace
 * grow.  nheads * ceil(head_dim / 64) must not exceed 65535.            */

/* Offsets (bytes from the workspace base) and sizes of the intermediates the
 * compute entry point leaves in the workspace, so tests can compare each
 * step with the oracle.  nchunks_max bounds the number of chunks the call can
 * hold: floor(total_len / 256) plus the sequences the chunked steps can see
 * (batch, or with the short path on at most total_len / (short_path_max + 1)
 * of them); chunk c of the call occupies row c of each table.  Sequences
 * taken by the short path (see ssd_problem.short_path_max; there a
 * zero-length sequence is taken as well) have no chunks: chunk_off[b] ==
 * chunk_off[b+1] and no row of any table is theirs.
 *   meta      int32[4]                    {nchunks, nseq, nrecur, 0}: chunks,
 *                                         sequences the state passing walks,
 *                                         sequences the token recurrence
 *                                         takes
 *   chunk_off int32[batch + 1]            first chunk of each sequence
 *   desc      int32[nchunks_max][4]       {sequence, first token, length, 0}
 *   dts       fp32[nchunks_max][H][256]   dts per token, 0 past the chunk end
 *   cs2       fp32[nchunks_max][H][256]   log2(e) * inclusive sum of A*dts
 *   cbt       fp16[nchunks_max][G][36][64][16]  G^T[j][i] = C_i . B_j of the
 *                                         chunk, as the 36 lower-triangular
 *                                         32x32 tiles (row block rb, column
 *                                         block t <= rb, tile rb(rb+1)/2 + t),
 *                                         each in MFMA accumulator order: lane
 *                                         l, element e holds j = 32t + 8(e/4)
 *                                         + 4(l/32) + e%4, i = 32rb + l%32;
 *                                         scaled by 2^gexp[c][g][min(rb,
 *                                         7-rb)]; the diagonal tiles (t = rb)
 *                                         hold 0 where j > i
 *   gexp      int32[nchunks_max][G][4]    exponent of the cbt tiles of row
 *                                         blocks q and 7-q
 *   states    fp16[nchunks_max][H][P][N]  chunk's own state contribution,
 *                                         element (p, n) scaled by
 *                                         2^sexp[c][h][p/32][n/32]
 *   sexp      int32[nchunks_max][H][2][N/32]  exponent of each 32x32 tile
 *   hin       fp16[nchunks_max][H][P][N]  state entering the chunk, row p
 *                                         scaled by 2^hexp[c][h][p]
 *   hexp      int32[nchunks_max][H][P]    exponent of each hin row
 *   xexp      int32[nchunks_max][H][2]    2^xexp[c][h][i] puts the chunk's
 *                                         largest |x| over p = 32i .. 32i+31
 *                                         of the head in [2^14, 2^15) (1000
 *                                         if all zero)
 *   seq_list  int32[batch]                the nseq sequences the state passing
 *                                         walks, in order (all of them when
 *                                         no sequence can take the short
 *                                         path; else those longer than its
 *                                         limit)
 *   recur_list int32[batch]               the nrecur sequences of 1 ..
 *                                         min(limit, SSD_RECUR_LIMIT) tokens,
 *                                         in order                           */
typedef struct ssd_workspace_layout {
    size_t total_bytes;
    int64_t nchunks_max;
    size_t meta, chunk_off, desc, dts, cs2, cbt, gexp, states, sexp, hin, hexp, xexp, seq_list, recur_list;
    /* The tables above are those of the problem the kernels run (see
     * "Sizes"): core_nheads heads of head_dim 64 and dstate core_dstate
     * (nheads and dstate for head_dim 64 and dstate 64, 128 or 256).  The
     * copies the other sizes need (SIZE_MAX where a size needs none):
     *   x_pad, y_pad  bf16 [T][H][64 ceil(P/64)]   x and y, zero-padded channels
     *   bc_pad        bf16 [T][G][core_dstate] B, then (at the next 256-byte
     *                 boundary) the same for C, zero-padded columns
     *   head_wide     fp32 dt [T][core_nheads], then A, D, dt_bias
     *                 [core_nheads], each from a 256-byte boundary
     *   state_pad     [batch][H][64 ceil(P/64)][core_dstate] in the state dtype:
     *                 each sequence's state, zero-padded                   */
    int32_t core_nheads, core_dstate;
    size_t x_pad, y_pad, bc_pad, head_wide, state_pad;
} ssd_workspace_layout;

/* ABI version of the loaded library (SSD_ABI_VERSION it was built with). */
int ssd_abi_version(void);

/* Static, human-readable name of a status code. */
const char *ssd_status_string(int status);

/* Workspace size for a problem.  Returns SSD_OK and sets *bytes, or an error
 * status when the problem is malformed or unsupported.  Host only.        */
ssd_status ssd_workspace_size(const ssd_problem *prob, size_t *bytes);

/* Full workspace layout (see ssd_workspace_layout).  Host only.           */
ssd_status ssd_workspace_get_layout(const ssd_problem *prob, ssd_workspace_layout *layout);

/* Varlen SSD forward prefill with in-place pool write-back
 * ("Mamba2SSDChunkScanVarlenFwdInplace", execute; argument order as there).
 *   y                 OUT  bf16 [T,H,P]
 *   x                 IN   bf16 [T,H,P]
 *   dt                IN   fp32 [T,H]   raw dt (before bias and softplus)
 *   A                 IN   fp32 [H]     per-head scalar, normally negative
 *   B, C              IN   bf16 [T,G,N]
 *   D                 IN   fp32 [H] or NULL (treated as 0)
 *   dt_bias           IN   fp32 [H] or NULL (treated as 0)
 *   ssm_pool          IN/OUT fp32 (bf16 with state_dtype = SSD_STATE_BF16)
 *                     [max_slots,H,P,N]: slot cache_indices[b] is
 *                     read as sequence b's initial state when
 *                     has_initial_state[b] != 0 (otherwise not read at all) and
 *                     overwritten with its final state (also for zero-length
 *                     sequences).  Every other slot is left bit-identical.
 *   query_start_loc   IN   int32 [batch+1]
 *   has_initial_state IN   uint8 [batch] or NULL (all false)
 *   cache_indices     IN   uint32 [batch]
 *   workspace         scratch of at least ssd_workspace_size() bytes, 256-byte
 *                     aligned; its contents on return are the intermediates
 *                     described by ssd_workspace_layout.
 * Errors (all before any launch; nothing is modified): SSD_ERR_NULL_ARG for
 * a NULL problem or required pointer (y, x, dt, B, C may be NULL only when
 * total_len is 0), SSD_ERR_BAD_SHAPE / SSD_ERR_UNSUPPORTED for the sizes,
 * SSD_ERR_MISALIGNED, SSD_ERR_WORKSPACE; SSD_ERR_HIP if a launch fails.
 * Precision: y is rounded to bf16 (nearest even); the inter-chunk state chain
 * and the pool are fp32.  Results are deterministic (bitwise run to run).  */
ssd_status ssd_chunk_scan_varlen_fwd_inplace(
    const ssd_problem *prob,
    void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    void *ssm_pool, const int32_t *query_start_loc,
    const uint8_t *has_initial_state, const uint32_t *cache_indices,
    void *workspace, size_t workspace_bytes, void *stream);

/* Number of kernels one compute call enqueues, and the name of kernel i
 * (0 <= i < ssd_kernel_count(), launch order; NULL otherwise).  The last
 * two, "ssd_short" and "ssd_recur", serve the short path and are not
 * launched when no sequence can take it (dstate 256, or
 * short_path_max = 0).                                                      */
int ssd_kernel_count(void);
const char *ssd_kernel_name(int i);

/* Short-sequence path (ssd_problem.short_path_max).  At dstate 64 and 128,
 * every sequence of 1 .. short_path_max tokens is scanned whole by one fused
 * kernel instead of the chunked steps, with the final state written straight
 * to its slot: sequences of up to SSD_RECUR_LIMIT tokens (decode steps) by
 * the token recurrence of "mamba2_ssd_scan" ("Per-token recurrence") with the
 * state split over the threads along dstate ("ssd_recur"), longer ones by the
 * single-chunk case of the segment-sum form of "Mamba chunk scan with segsum"
 * (description), on MFMA ("ssd_short").  Zero-length sequences are finished
 * there too.  The route depends on the sequence's own length only (a
 * sequence's results do not depend on the rest of the batch).  Results agree
 * with the chunked path within the documented tolerances, not bitwise.
 * short_path_max = 0 sends every sequence through the chunked steps (the
 * faster choice for batches of mostly long sequences with a few short ones,
 * where the short kernel runs after the chunked ones).  The limit is read
 * from the problem of each call; nothing is remembered between calls. */

/* Same computation as ssd_chunk_scan_varlen_fwd_inplace; additionally
 * records events (each a hipEvent_t created by the caller, passed as void*)
 * through the kernels' own dispatches, so no command is enqueued between
 * kernels: events[0] when kernel 0 starts and events[i+1] when kernel i
 * completes (for a kernel that is not launched, the event is recorded on
 * the stream at its place).  hipEventElapsedTime(events[i], events[i+1]) is then kernel i's
 * time (with the gap before it, for i > 0) and (events[0],
 * events[ssd_kernel_count()]) the whole call.  n_events must equal
 * ssd_kernel_count()+1 (SSD_ERR_NULL_ARG / SSD_ERR_BAD_SHAPE otherwise,
 * before any launch).  For sizes that need the copies of "Sizes", the events
 * cover the scan's kernels only (the copies run before and after them).    */
ssd_status ssd_chunk_scan_varlen_fwd_inplace_profiled(
    const ssd_problem *prob,
    void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    void *ssm_pool, const int32_t *query_start_loc,
    const uint8_t *has_initial_state, const uint32_t *cache_indices,
    void *workspace, size_t workspace_bytes, void *stream,
    void *const *events, int n_events);

/* Varlen SSD forward prefill with separate initial and final states: the
 * same operation, where sequence b starts from initial_states[b] (or zero)
 * and its final state goes to final_states[b] ("mamba2_ssd_scan", Modular
 * MAX kernels docs, the paragraph after "Per-token recurrence": the state
 * resets to zero or to initial_states at each query_start_loc boundary, and
 * final_states of shape (batch, nheads, head_dim, dstate) is written at
 * each sequence end; "Mamba2SSDChunkScanVarlenFwd" is the operation the
 * in-place one is described against).
 *   y, x, dt, A, B, C, D, dt_bias, query_start_loc, workspace: as for
 *                     ssd_chunk_scan_varlen_fwd_inplace (prob->max_slots is
 *                     not used).
 *   initial_states    IN   fp32 (bf16 with state_dtype = SSD_STATE_BF16)
 *                     [batch,H,P,N] or NULL (every sequence starts
 *                     from zero); when given, every sequence starts from its
 *                     row (no per-sequence flag).
 *   final_states      OUT  the same type [batch,H,P,N]: every row is written, also
 *                     for zero-length sequences (their initial state).  It
 *                     may be the same buffer as initial_states (each element
 *                     is read before it is written); it must not overlap any
 *                     other argument.
 * Errors as for the in-place entry point; final_states NULL gives
 * SSD_ERR_NULL_ARG.                                                        */
ssd_status ssd_chunk_scan_varlen_fwd(
    const ssd_problem *prob,
    void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    const void *initial_states, void *final_states,
    const int32_t *query_start_loc,
    void *workspace, size_t workspace_bytes, void *stream);

/* ssd_chunk_scan_varlen_fwd with the events of
 * ssd_chunk_scan_varlen_fwd_inplace_profiled.                              */
ssd_status ssd_chunk_scan_varlen_fwd_profiled(
    const ssd_problem *prob,
    void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    const void *initial_states, void *final_states,
    const int32_t *query_start_loc,
    void *workspace, size_t workspace_bytes, void *stream,
    void *const *events, int n_events);

/* For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * operation as ssd_chunk_scan_varlen_fwd_inplace (same arguments, minus the
 * workspace), whose intermediates go to a scratch array that the library
 * holds in device memory instead: SSD_NOALLOC_SCRATCH_BYTES per GPU it runs
 * on, kept until the process ends.  The call allocates nothing (no hipMalloc,
 * no allocating library routine); its first call on a device looks up that
 * device's copy of the array once.  It runs on the current device; `stream`
 * must belong to it.  Problems whose ssd_workspace_size() exceeds
 * SSD_NOALLOC_SCRATCH_BYTES give SSD_ERR_SCRATCH before any launch (other
 * errors as for the in-place entry point).  Every call on one GPU shares
 * that GPU's array and leaves its intermediates there: calls on one stream
 * are ordered, but calls that can overlap on one GPU (other streams, other
 * host threads without ordering) race on it and must not be issued.       */
#define SSD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
ssd_status ssd_chunk_scan_varlen_fwd_inplace_noalloc(
    const ssd_problem *prob,
    void *y, const void *x, const float *dt, const float *A,
    const void *B, const void *C, const float *D, const float *dt_bias,
    void *ssm_pool, const int32_t *query_start_loc,
    const uint8_t *has_initial_state, const uint32_t *cache_indices,
    void *stream);

/* Synchronous debug check of the device-side preconditions: copies
 * query_start_loc and cache_indices to the host (after synchronising
 * `stream`) and returns SSD_ERR_BAD_INPUT if query_start_loc does not run
 * non-decreasing from 0 to total_len or a cache index is out of range or
 * repeated; SSD_OK otherwise.                                              */
ssd_status ssd_validate_inputs(const ssd_problem *prob, const int32_t *query_start_loc,
                               const uint32_t *cache_indices, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBSSD_SSD_H */
