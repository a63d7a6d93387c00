/*
 * topkf: exact FP32 row-wise Top-K over ragged score rows, for AMD MI355X
 * (gfx950).  A sample-guided exact selector after "Sample-Guided Exact Top-K
 * Selection for Long-Context Sparse Attention" (Secs. 4-5) and the operator
 * API of the HPC-Ops pull request "feat(topk): add sample-verified exact
 * Top-K" (section "API").
 *
 * Operator contract (paper Sec. 2.1, "Operator contract"; Eq. 30 in Sec. 6.1):
 * logits is an [M_cap, N] float32 matrix stored at a row pitch of row_stride
 * elements; row r has valid length L_r = ke[r] clamped to [0, N].  For every
 * live row r < M_live (M_live = *num_valid_rows clamped to [0, M_cap]):
 *   - L_r >  K: out[r, 0..K) receives K distinct indices from [0, L_r) such
 *               that no unselected valid score exceeds a selected one.  Ties at
 *               the K-th value resolve to any of the tied indices; the slots
 *               are in no particular order.
 *   - L_r <= K: out[r, j] = j for j < L_r and -1 for L_r <= j < K.
 * Rows r >= M_live are not written.  Columns at or beyond L_r are never read
 * and may hold anything.  Valid scores must be NaN-free (a NaN in a valid
 * prefix gives an unspecified, but in-bounds, result); +-inf and subnormals
 * are ordered numerically, and +0.0 ranks above -0.0.
 *
 * All pointers passed to topk_filtered are device pointers owned by the
 * caller; the library allocates no device memory.  Calls are asynchronous on
 * `stream`, never synchronize, never read device data back to the host, and
 * are capturable into a HIP graph: the launch geometry depends only on
 * (top_k, M_cap, N, row_stride, device), and M_live and ke stay on the device.
 */
#ifndef TOPKF_H
#define TOPKF_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    TOPKF_OK = 0,
    TOPKF_EINVAL = 1,       /* a host-checkable argument is invalid */
    TOPKF_EUNSUPPORTED = 2, /* valid request the library does not serve */
    TOPKF_EWORKSPACE = 3,   /* counters or workspace smaller than required */
    TOPKF_EHIP = 4          /* a HIP runtime call or kernel launch failed */
} topkf_status;

/* Largest supported top_k.  The workspace query takes no K, so buffers are
 * sized for this maximum (the pages evaluate K = 2048). */
#define TOPKF_K_MAX 2048

/*
 * Buffer sizes for topk_filtered on the current HIP device (PR "API":
 * topk_filtered_workspace_size(num_rows, max_kv_len)).
 *
 *   num_rows    M_cap, the captured row capacity (>= 0)
 *   max_kv_len  N, the allocated row width in elements (>= 1)
 *   counter_bytes, workspace_bytes  (out, host pointers) required sizes.
 *
 * The counter buffer must be zero-filled once before its first use; every
 * successful launch returns it to all-zero on the device (PR "API"), so it can
 * be reused and replayed in a graph without re-initialisation.  The workspace
 * needs no initialisation and may be retained across calls and graph replays.
 * Its size is bounded by the worker pool or, for plans that split rows, by
 * M_cap rows (paper Sec. 5.4 and Sec. 5.5).
 *
 * Returns TOPKF_EINVAL for negative num_rows, max_kv_len < 1 or null output
 * pointers, TOPKF_EHIP if the device cannot be queried.  Host only; launches
 * nothing.
 */
topkf_status topk_filtered_workspace_size(int64_t num_rows, int64_t max_kv_len,
                                          size_t* counter_bytes, size_t* workspace_bytes);

/*
 * Exact row-wise Top-K (PR "API": topk_filtered; paper Secs. 4.1-4.5).
 *
 *   logits          device, float32, element (r, i) at logits[r*row_stride + i]
 *   num_rows        M_cap
 *   max_kv_len      N
 *   row_stride      row pitch in elements, >= N.  A pitch and base that are
 *                   16-byte aligned allow 128-bit loads; any pitch works.
 *   ke              device, int32[M_cap], valid lengths (clamped to [0, N])
 *   out             device, int32[M_cap * top_k], row-major, contiguous
 *   num_valid_rows  device, one int32: M_live (clamped to [0, M_cap])
 *   top_k           K, 1 <= K <= TOPKF_K_MAX
 *   counters        device, counter_bytes bytes, all-zero on entry (see above)
 *   workspace       device, workspace_bytes bytes, any contents
 *   stream          HIP stream the work is enqueued on (0 = default stream)
 *
 * Errors returned without launching: TOPKF_EINVAL for null pointers (logits,
 * ke, out, num_valid_rows and counters may only be null when num_rows == 0),
 * num_rows < 0, max_kv_len < 1, row_stride < max_kv_len or top_k outside
 * [1, TOPKF_K_MAX]; TOPKF_EWORKSPACE when counter_bytes or workspace_bytes is
 * smaller than topk_filtered_workspace_size reports.  TOPKF_EHIP when the
 * launch fails; the counters may then be left non-zero and must be re-zeroed
 * by the caller.  One launch at a time may use a given counters/workspace
 * pair.
 */
topkf_status topk_filtered(const float* logits, int64_t num_rows, int64_t max_kv_len,
                           int64_t row_stride, const int32_t* ke, int32_t* out,
                           const int32_t* num_valid_rows, int32_t top_k, void* counters,
                           size_t counter_bytes, void* workspace, size_t workspace_bytes,
                           hipStream_t stream);

/*
 * topk_filtered for callers that cannot allocate device memory or pass
 * buffers: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Not part of the pages' API.
 *
 * Same operation, arguments, output and errors as topk_filtered, minus the
 * counter and workspace buffers: the library takes both from one device
 * array of TOPKF_NOALLOC_SCRATCH_BYTES (256 MiB) that it owns.  Every GPU the
 * library runs on holds its own copy of that array until the process ends,
 * and all calls on one GPU share it, so calls that overlap on one GPU (on
 * different streams, or from several host threads without ordering) race
 * and must not be issued.  The first call on a device also enqueues a clear
 * of the array's counter part on `stream`.  The call performs no allocation
 * (no hipMalloc, hipFree or allocating library routine) and reads no device
 * data on the host.
 *
 * Limits: the counters need (64 + 2 * num_rows) * 4 bytes of a 1 MiB counter
 * part, so num_rows <= 131040; the workspace part holds 255 MiB.  The
 * automatic plan is used when its workspace fits; otherwise the rows are
 * taken by persistent workers, as many as fit at 16 * (max_kv_len + 128)
 * bytes each.  TOPKF_EWORKSPACE when num_rows or max_kv_len exceed these
 * limits (max_kv_len above about 16.7M columns), without launching.
 */
#define TOPKF_NOALLOC_SCRATCH_BYTES (256u << 20)
topkf_status topk_filtered_noalloc(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                   int64_t row_stride, const int32_t* ke, int32_t* out,
                                   const int32_t* num_valid_rows, int32_t top_k,
                                   hipStream_t stream);

/* Static text for a status code; never null. */
const char* topkf_status_string(topkf_status status);

/* ------------------------------------------------------------------------
 * Plans and diagnostics.  Not part of the pages' API: they expose the host
 * planner of paper Sec. 5.5 ("Shape-stable dispatch") so that tests can force
 * every route and mapping, and count which route each row took.
 * ------------------------------------------------------------------------ */

/* Kernel families (paper Sec. 5.5, Fig. 6). */
#define TOPKF_FAMILY_AUTO 0
#define TOPKF_FAMILY_PERSISTENT 1 /* one 512-thread workgroup owns a row; rows from a queue */
#define TOPKF_FAMILY_KVSPLIT 2    /* P workgroups scan segments of a row, then one
                                     workgroup per row merges and refines */

typedef struct {
    int32_t family;   /* TOPKF_FAMILY_* */
    int32_t stride;   /* view stride s: 0 = no view (every row takes the exact
                         coarse route), 64 or 128 (paper Sec. 5.5: compile-time
                         s = 64 and s = 128 policies) */
    int32_t dual;     /* 1: also record the nested secondary boundary tau1
                         (paper Sec. 4.2; Sec. 6.4 "Conditional rescue") */
    int32_t splits;   /* KV-split: workgroups per row P (>= 1) */
    int32_t workers;  /* persistent: workgroups in the pool (>= 1) */
    int32_t min_segment; /* KV-split: shortest segment in elements; a row of
                            length L uses min(P, ceil(L / min_segment)) parts */
    int32_t band_quarters; /* secondary target K~1 = ceil(band_quarters * K / 4),
                              above primary_quarters and at most 32 when dual
                              (paper Sec. 6.4 uses 1.75K, i.e. 7); ignored
                              without dual */
    int32_t primary_quarters; /* primary target K~ = ceil(primary_quarters * K / 4),
                                 4..31 (paper Sec. 4.2 uses 1.5K, i.e. 6) */
} topkf_plan;

/*
 * The plan topk_filtered uses for (M_cap, N) on a device with `cu_count`
 * compute units (host only, no device access; cu_count >= 1).
 * TOPKF_EINVAL on bad arguments.
 */
topkf_status topkf_plan_for(int64_t num_rows, int64_t max_kv_len, int32_t cu_count,
                            topkf_plan* plan);

/* Buffer sizes for an explicit plan (host only).  TOPKF_EINVAL on bad
 * arguments or an invalid plan. */
topkf_status topkf_plan_workspace_size(const topkf_plan* plan, int64_t num_rows,
                                       int64_t max_kv_len, size_t* counter_bytes,
                                       size_t* workspace_bytes);

/* Route counters written by topk_filtered_debug (indices into route_stats). */
#define TOPKF_ROUTE_SENTINEL 0       /* L <= K: sentinel layout */
#define TOPKF_ROUTE_PRIMARY 1        /* certified by the primary boundary tau0 */
#define TOPKF_ROUTE_BAND 2           /* certified after the tau1 band extension */
#define TOPKF_ROUTE_EXACT_UNDERFILL 3 /* exact coarse recovery after underfill */
#define TOPKF_ROUTE_EXACT_DIRECT 4   /* exact coarse route: no view or unusable view */
#define TOPKF_ROUTE_SPILL 5          /* rows whose frontier overflowed on-chip storage */
#define TOPKF_ROUTE_HINTED 6         /* rows whose caller-supplied proposal replaced the view
                                        (counted in addition to the route they took) */
#define TOPKF_ROUTE_COUNT 8

/*
 * topk_filtered with an explicit plan and optional route statistics.
 *   plan         host pointer; null means the automatic plan
 *   route_stats  device, uint32[TOPKF_ROUTE_COUNT] or null; each row adds one
 *                to the counter of the route it took (not reset by the call)
 * Buffer sizes must satisfy topkf_plan_workspace_size for the plan used.
 * Same errors as topk_filtered, plus TOPKF_EINVAL for an invalid plan.
 */
topkf_status topk_filtered_debug(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                 int64_t row_stride, const int32_t* ke, int32_t* out,
                                 const int32_t* num_valid_rows, int32_t top_k, void* counters,
                                 size_t counter_bytes, void* workspace, size_t workspace_bytes,
                                 const topkf_plan* plan, uint32_t* route_stats,
                                 hipStream_t stream);

/*
 * topk_filtered with a caller-supplied proposal per row, as the GVR page
 * carries a threshold over from the previous decode step (its Sec. "Core
 * claim"; the paper's Sec. 2.2 "History-dependent prediction").
 *   hint  device, float[M_cap]: row r admits every valid value >= hint[r]
 *         (compared as descending keys, so +0 ranks above -0) in place of the
 *         boundary its view would propose; NaN means no proposal and the row
 *         uses its view.  A proposal is never trusted: the complete-row count
 *         certifies it, and a row it underfills takes the exact coarse route
 *         (no secondary band), so the result is exact for any hint.  A useful
 *         hint admits a little more than K values (e.g. the previous step's
 *         value near rank 1.25K); plans without a view ignore hints.
 * Other arguments, errors and buffers as topk_filtered; TOPKF_EINVAL also for
 * a null hint with num_rows > 0.
 */
topkf_status topk_filtered_hinted(const float* logits, int64_t num_rows, int64_t max_kv_len,
                                  int64_t row_stride, const int32_t* ke, int32_t* out,
                                  const int32_t* num_valid_rows, int32_t top_k, const float* hint,
                                  void* counters, size_t counter_bytes, void* workspace,
                                  size_t workspace_bytes, hipStream_t stream);

/* topk_filtered_hinted with an explicit plan and route statistics (as
 * topk_filtered_debug). */
topkf_status topk_filtered_hinted_debug(const float* logits, int64_t num_rows,
                                        int64_t max_kv_len, int64_t row_stride, const int32_t* ke,
                                        int32_t* out, const int32_t* num_valid_rows, int32_t top_k,
                                        const float* hint, void* counters, size_t counter_bytes,
                                        void* workspace, size_t workspace_bytes,
                                        const topkf_plan* plan, uint32_t* route_stats,
                                        hipStream_t stream);

/*
 * The 11-bit coarse key of paper Sec. 4.2, Eq. 11, for n device floats:
 * out[i] = kappa16(fp16_rne(x[i])) >> 5, where kappa16 is the descending
 * sortable key of the FP16 bit pattern (a larger value gets a smaller key).
 * Exposed so tests can check the device conversion against IEEE-754.
 * x, out: device pointers; n >= 0.  TOPKF_EINVAL on null pointers with n > 0.
 */
topkf_status topkf_coarse_keys(const float* x, int64_t n, uint16_t* out, hipStream_t stream);

/*
 * The inclusive FP32 cutoff T(tau) of every coarse bin (paper Sec. 4.3: the
 * largest non-NaN descending key whose value has c <= tau; kKeyFirst - 1 =
 * 0x007FFFFE when even +inf lies above tau).  The selector reads these from a
 * table computed at compile time; this call writes that table to table[0,
 * 2048) and the device's own search over the hardware conversion to
 * search[0, 2048), so that tests can check one against the other.
 * table, search: device pointers to 2048 uint32 each.  TOPKF_EINVAL on null.
 */
topkf_status topkf_coarse_cutoffs(uint32_t* table, uint32_t* search, hipStream_t stream);

/*
 * Measurement aid, not part of the pages' API: a plain streaming read of
 * `bytes` bytes at x with the same 128-bit nontemporal loads the selector
 * streams with (two 512-thread workgroups per compute unit, four loads in
 * flight per thread), so that its rate is the achievable-bandwidth reference
 * for the selector's score-row GB/s.  x: device pointer, 16-byte aligned;
 * bytes: a multiple of 16, >= 0; sink: device pointer to one uint32 that the
 * kernel writes only in an improbable case (keeps the loads live).  Returns
 * TOPKF_EINVAL for a misaligned pointer or size, TOPKF_EHIP on launch failure.
 */
topkf_status topkf_read_probe(const void* x, int64_t bytes, uint32_t* sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TOPKF_H */
