/*
 * ep.h -- MoE expert-parallel token routing on one AMD Instinct MI355X
 * (gfx950): prepare, dispatch, combine and their two backward ops, plus a
 * fused weighted combine and its backward.
 *
 * The five per-step calls follow the per-step part of the common C API in
 * "Expert Parallelism: common C API + NCCL EP backend" (section "Per-step
 * (allocation-free, CUDA-graph capturable)"), at one GPU's share of the work:
 * prepare builds the routing maps of a handle, dispatch moves token rows and
 * their routing weights into an expert-major receive buffer, combine sums the
 * expert outputs of each token back into a token row without weighting them
 * (the caller has already multiplied by the received weights), and
 * dispatch_bwd / combine_bwd are the adjoints of dispatch / combine.
 *
 * Conventions shared by every call
 *  - Routes are numbered s = t*K + k over the [T,K] routing table.
 *  - A route is valid iff 0 <= topk_idx[s] < E. The id -1 marks a masked
 *    route (one whose expert lives elsewhere; see the masking of
 *    "Expert-parallel implementations for ep_dispatch_experts", table
 *    "Implementations"). Any other id is an error: the device raises
 *    EP_STATUS_BAD_EXPERT and the route is then treated as masked.
 *  - Expert e owns the received rows [offsets[e], offsets[e+1]). Its valid
 *    routes fill the first counts[e] rows in ascending s; the segment is then
 *    padded up to a multiple of the alignment A. The pad rows of every
 *    expert-major output are written as zeros, unless the layout sets
 *    EP_LAYOUT_NO_PAD_FILL: then they are not written at all. An expert with
 *    no route has an empty segment. total = offsets[E].
 *  - Payload rows hold the layout's payload type: bf16 (the default, and the
 *    only type of the PyTorch wrapper in "[PyTorch] Expert Parallelism:
 *    PyTorch wrapper + autograd ops with symm-mem zero-copy", section
 *    "Public Python API"), fp16 or fp32 (the types the C++ tests of "Expert
 *    Parallelism: common C API + NCCL EP backend" cover, per its section
 *    "Important Files Changed"). They are passed as raw bit patterns through
 *    void pointers. Routing ids are int64, routing weights fp32. Rows are
 *    contiguous, H elements each, row-major.
 *  - Sums are taken in fp32 and rounded once to the payload type: round to
 *    nearest, ties to even, subnormals kept, overflow to infinity, and any
 *    NaN becomes the canonical quiet NaN (bf16 0x7FC0, fp16 0x7E00, fp32
 *    0x7FC00000). For fp32 payloads the only change is that NaN rule.
 *  - All pointers are device pointers unless stated otherwise. Payload
 *    pointers must be 16-byte aligned and H must be a multiple of 8. A
 *    pointer to a buffer with no element (T == 0 for [T,...] buffers,
 *    recv_capacity == 0 for [recv_capacity,...] buffers) may be NULL; every
 *    other required pointer must not be, whatever the other sizes are.
 *  - Work is enqueued on `stream` and nothing waits for it: no call below
 *    synchronises, allocates, frees or keeps a pointer after it returns,
 *    except ep_read_status, which waits for the stream. The caller owns
 *    every buffer. Outputs must not overlap inputs or each other.
 *  - Host-detectable errors return an ep_status_t before any HIP call is
 *    made; nothing is enqueued then. Data-dependent errors raise sticky bits
 *    in the handle's status word (see ep_read_status).
 *  - Calls on one handle must be ordered on the GPU (same stream, or events)
 *    with prepare first. Several handles may be in flight at once.
 */
#ifndef EP_MI355X_EP_H
#define EP_MI355X_EP_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ep_status {
  EP_OK = 0,
  EP_ERR_NULL = 1,        /* a required pointer is NULL */
  EP_ERR_SHAPE = 2,       /* a size is out of range (see ep_layout_t) */
  EP_ERR_ALIGN = 3,       /* a payload pointer is not 16-byte aligned */
  EP_ERR_HANDLE_SIZE = 4, /* handle_bytes < ep_handle_mem_size(layout) */
  EP_ERR_CAPACITY = 5,    /* recv_capacity < 0 or >= 2^31 */
  EP_ERR_DEVICE = 6,      /* the current device is not gfx950 */
  EP_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
  EP_ERR_SCRATCH = 8      /* ep_prepare_static: the layout's prepare scratch
                             exceeds EP_PREPARE_STATIC_SCRATCH_BYTES */
} ep_status_t;

/* Sticky device-side bits of a handle's status word. */
enum {
  EP_STATUS_BAD_EXPERT = 1u, /* prepare saw an id outside [0,E) other than -1 */
  EP_STATUS_OVERFLOW = 2u,   /* prepare: total > recv_capacity; routes whose row
                                would lie at or past the capacity were dropped */
  EP_STATUS_LAYOUT = 4u      /* a payload op was given a layout other than the
                                one the handle was prepared with, or a handle
                                that was never prepared; the op wrote nothing */
};

/* Payload element types (ep_layout_t.dtype). */
enum {
  EP_DTYPE_BF16 = 0,
  EP_DTYPE_FP16 = 1,
  EP_DTYPE_FP32 = 2
};

/* Layout flags (ep_layout_t.flags). EP_LAYOUT_NO_PAD_FILL: the payload ops
 * leave pad rows unwritten instead of zeroing them (dispatch's rows and
 * weights, combine_bwd's rows, the weighted backward's rows and weight
 * gradients), saving their writes when the consumer never reads pad rows
 * (combine and dispatch_bwd never do). The pages zero the pads of
 * combine_bwd's output only, and the review of "[PyTorch] Expert
 * Parallelism: PyTorch wrapper + autograd ops with symm-mem zero-copy"
 * weighs what the padded expert-major buffer costs (its buffer-sizing
 * thread); this flag makes the pad writes a choice. It does not change the
 * routing maps: one prepared handle serves both policies. */
enum {
  EP_LAYOUT_NO_PAD_FILL = 1u,
  EP_LAYOUT_ZERO_TAIL = 4u
};

/* EP_LAYOUT_ZERO_TAIL: the payload ops that write expert-major rows
 * (ep_dispatch's rows and weights, ep_combine_bwd's rows, and the weighted
 * backward's rows and weight gradients) also write +0 to every row at or past
 * min(total, recv_capacity), so that the whole [recv_capacity,...] buffer is
 * defined. This is the library's own addition: combine never reads those
 * rows, so their gradient is zero, and a caller that applies one function to
 * the whole receive buffer (a parameter shared by every row, a reduction
 * over it) then sees zeros there instead of stale memory. It costs one
 * zero write per tail row. */

/*
 * Per-layer sizes (the role of the layer configuration in the common C API,
 * passed by pointer as plain data). A zero-initialised dtype/flags pair
 * means bf16 payloads with zero-filled pads.
 *   num_tokens    T >= 0
 *   topk          K in [1, 64]
 *   num_experts   E in [1, 2048], local experts
 *   alignment     A >= 1 rows (the per-expert dispatch output alignment)
 *   dtype         EP_DTYPE_* of every payload row
 *   flags         EP_LAYOUT_* bits; other bits must be 0
 *   hidden        H >= 8, a multiple of 8 (elements per row)
 *   recv_capacity rows of every expert-major buffer, 0 <= cap < 2^31
 * T*K + E*(A-1) must be below 2^31 (every offset fits an int32). The handle
 * depends on num_tokens, topk, num_experts, alignment and recv_capacity
 * only; dtype, flags and hidden may differ between the ops that use it.
 */
typedef struct ep_layout {
  int64_t num_tokens;
  int32_t topk;
  int32_t num_experts;
  int32_t alignment;
  uint16_t dtype;
  uint16_t flags;
  int64_t hidden;
  int64_t recv_capacity;
} ep_layout_t;

/* Rows that can never overflow: every token sends min(K,E) distinct routes
 * and every expert adds at most A-1 pad rows: T*min(K,E) + E*(A-1). With
 * repeated ids in a token's top-k the bound is T*K + E*(A-1). Returns -1 for
 * out-of-range arguments. Host only. The library's own helper: the review of
 * "[PyTorch] Expert Parallelism: PyTorch wrapper + autograd ops with symm-mem
 * zero-copy" sizes the padded expert-major buffer for its worst case (the
 * thread on buffer sizing and recv_capacity_per_rank); this is that bound for
 * one GPU. */
int64_t ep_recv_capacity_worst(int64_t num_tokens, int32_t topk, int32_t num_experts,
                               int32_t alignment);

/* Bytes of device memory the caller must provide as `handle_mem` for this
 * layout. Returns 0 for an invalid layout. Host only. The handle-size query
 * of "Expert Parallelism: common C API + NCCL EP backend" (section "Public C
 * API", its "Lifecycle" list: layer registration reports the handle_mem size
 * the caller allocates); here it is a pure function of the layout, with no
 * registration step. */
size_t ep_handle_mem_size(const ep_layout_t* layout);

/* Byte offsets, inside handle_mem, of the routing maps that prepare writes,
 * so that callers can read them. The library's own addition: the handle of
 * the common C API is opaque caller memory. All int32 unless stated:
 *   status   uint32 status word (EP_STATUS_* bits)
 *   counts   [E]     valid routes per expert
 *   offsets  [E+1]   segment starts, offsets[E] = total
 *   slot     [T*K]   received row of route s, -1 if masked or dropped
 *   row_src  [recv_capacity]  route held by received row r, -1 for a pad row;
 *            entries at or past min(total, recv_capacity) are unspecified
 *   bytes    == ep_handle_mem_size(layout)
 *   maps_bytes  the size of the routing maps alone (<= bytes): the handle
 *            region every payload op reads. A handle of maps_bytes serves the
 *            payload ops; ep_prepare needs all `bytes` (its scratch closes the
 *            handle).
 *   runs     8 lists of run_list_entries (row, route) int32 pairs: the run
 *            entries that dispatch and combine_bwd copy by. The routes are
 *            cut into chunks of run_units * 512 consecutive routes; chunk c
 *            belongs to list c mod 8, and a list holds its chunks one after
 *            another, each as its routes that hold a row in ascending row
 *            order, then (-1, -1) for each of its valid routes dropped past
 *            the capacity.
 *   stream_live  int32 [8]: the number of entries in each list
 *   run_units    int32: units of 512 routes per chunk (1, 2 or 4), chosen
 *            by prepare from its layout's payload row size
 *   run_list_entries  (a count, not an offset) the entries each list can
 *            hold, 64 * ceil(T*K/512) + 2048
 * Every offset is a multiple of 256. Host only. */
typedef struct ep_handle_regions {
  size_t status;
  size_t counts;
  size_t offsets;
  size_t slot;
  size_t row_src;
  size_t bytes;
  size_t runs;
  size_t maps_bytes;
  size_t stream_live;
  size_t run_units;
  size_t run_list_entries;
} ep_handle_regions_t;

ep_status_t ep_handle_regions(const ep_layout_t* layout, ep_handle_regions_t* out);

/*
 * prepare: from the int64 routing table, write the per-expert token counts,
 * the aligned segment offsets and the slot map into the handle. The
 * per-step prepare of "Expert Parallelism: common C API + NCCL EP backend"
 * (section "Per-step (allocation-free, CUDA-graph capturable)"), with the
 * alignment taken from the layout.
 *   topk_idx        int64 [T,K]                  input
 *   token_counts    int32 [E]                    output: valid routes per expert
 *                                                (not padded)
 *   expert_offsets  int32 [E+1] or NULL          output: segment starts,
 *                                                expert_offsets[E] = total
 *   handle_mem      handle_bytes of device memory, fully (re)written here
 * After this call the handle holds, for the later ops, the received row of
 * every route (-1 if masked or dropped), the source route of every live
 * received row (-1 for pads) and the run entries (see ep_handle_regions),
 * whatever the layout's flags. Its status word is reset, then raises
 * BAD_EXPERT / OVERFLOW as described above.
 */
ep_status_t ep_prepare(const ep_layout_t* layout, const int64_t* topk_idx,
                       int32_t* token_counts, int32_t* expert_offsets, void* handle_mem,
                       size_t handle_bytes, hipStream_t stream);

/*
 * ep_prepare_static: ep_prepare for callers that cannot allocate (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation)
 * and so cannot give the handle room for prepare's scratch. The same work and
 * the same routing maps, bit for bit, but the scratch (the expert
 * histograms and bad-id flags of the prepare kernels) lives in a static
 * device array of the library, EP_PREPARE_STATIC_SCRATCH_BYTES per device,
 * held until the process ends; so handle_mem needs only the routing maps,
 * `maps_bytes` of ep_handle_regions (ep_handle_mem_size also suffices).
 * Allocates nothing: the array's device address is looked up on the first
 * call on each device. Every call on one device shares that device's array,
 * so calls of ep_prepare_static that overlap on one device (several streams,
 * no ordering between them) race and must not be made; ep_prepare and the
 * payload ops do not touch the array. A layout whose scratch exceeds the
 * array returns EP_ERR_SCRATCH before any HIP call. With U = ceil(T*K/512)
 * units of routes the scratch is 4*E*(U + B + 1) bytes of histograms (one
 * row per unit, one per block of units, B = ceil(U/4) blocks of 4 units up
 * to 256 units and ceil(U/8) blocks of 8 past that, one row of totals) plus
 * 8*U bytes of per-unit words, each part rounded up to 256 bytes: at
 * E = 256, 3614 units (about 1.85 M routes) fit.
 */
#define EP_PREPARE_STATIC_SCRATCH_BYTES (4u << 20)

ep_status_t ep_prepare_static(const ep_layout_t* layout, const int64_t* topk_idx,
                              int32_t* token_counts, int32_t* expert_offsets, void* handle_mem,
                              size_t handle_bytes, hipStream_t stream);

/*
 * dispatch (the per-step dispatch of the same section):
 * recv_tokens[r,:] = tokens[s/K,:] and recv_topk_weights[r] =
 * topk_weights[s] for every live row r holding route s (bit copies); pad
 * rows get +0 in both (not written with EP_LAYOUT_NO_PAD_FILL). Rows at or
 * past min(total, recv_capacity) are not written (+0 with
 * EP_LAYOUT_ZERO_TAIL).
 *   tokens             payload [T,H]
 *   topk_weights       fp32 [T,K] or NULL
 *   recv_tokens        payload [recv_capacity,H]
 *   recv_topk_weights  fp32 [recv_capacity]; must be NULL iff topk_weights is
 *                      (when T > 0 and recv_capacity > 0)
 */
ep_status_t ep_dispatch(const ep_layout_t* layout, const void* handle_mem,
                        size_t handle_bytes, const void* tokens,
                        const float* topk_weights, void* recv_tokens,
                        float* recv_topk_weights, hipStream_t stream);

/*
 * combine (the per-step combine of the same section, unweighted there too):
 * result[t,:] = the sum over the valid routes of t, k ascending, of
 * expert_out[slot(t,k),:], accumulated in fp32 starting from the first valid
 * row and rounded once to the payload type (see the rounding convention
 * above). A token with no valid route gets +0. Unweighted.
 *   expert_out  payload [recv_capacity,H] (only the rows of valid routes are
 *               read)
 *   result      payload [T,H]
 */
ep_status_t ep_combine(const ep_layout_t* layout, const void* handle_mem,
                       size_t handle_bytes, const void* expert_out, void* result,
                       hipStream_t stream);

/*
 * dispatch_bwd (the per-step dispatch backward of the same section; the
 * adjoint of dispatch): grad_tokens = combine(grad) with the
 * same fp32 ascending-k rule; grad_topk_weights[s] = g_recv_topk_weights[r]
 * for the row r of a valid route s, else +0. A NULL g_recv_topk_weights
 * (no gradient flowed into the received weights) gives +0 everywhere; a NULL
 * grad_topk_weights skips the weight gradient.
 *   grad                 payload [recv_capacity,H]
 *   g_recv_topk_weights  fp32 [recv_capacity] or NULL
 *   grad_tokens          payload [T,H]
 *   grad_topk_weights    fp32 [T,K] or NULL
 */
ep_status_t ep_dispatch_bwd(const ep_layout_t* layout, const void* handle_mem,
                            size_t handle_bytes, const void* grad,
                            const float* g_recv_topk_weights, void* grad_tokens,
                            float* grad_topk_weights, hipStream_t stream);

/*
 * combine_bwd (the per-step combine backward of the same section; the
 * adjoint of combine): grad_expert_out[r,:] = grad[s/K,:] for
 * every live row r holding route s; pad rows are zeroed (not written with
 * EP_LAYOUT_NO_PAD_FILL). Rows at or past min(total, recv_capacity) are not
 * written (+0 with EP_LAYOUT_ZERO_TAIL).
 *   grad             payload [T,H]
 *   grad_expert_out  payload [recv_capacity,H]
 */
ep_status_t ep_combine_bwd(const ep_layout_t* layout, const void* handle_mem,
                           size_t handle_bytes, const void* grad, void* grad_expert_out,
                           hipStream_t stream);

/*
 * Weighted combine: the weight multiply folded into combine, which the review
 * of "[PyTorch] Expert Parallelism: PyTorch wrapper + autograd ops with
 * symm-mem zero-copy" (thread on the weight multiply) settles on as an
 * option, so that the caller's separate pre-multiply pass disappears. For
 * each token, over its valid routes in ascending k with received row r: the
 * first term is the fp32 product w[r] * y[r], each later term is a fused
 * multiply-add fma(w[r], y[r], acc); the fp32 sum is rounded once to the
 * payload type; a token with no valid route gets +0.
 *   expert_out         payload [recv_capacity,H] (y; only the rows of valid
 *                      routes are read)
 *   recv_topk_weights  fp32 [recv_capacity]   (w, e.g. dispatch's output)
 *   result             payload [T,H]
 */
ep_status_t ep_combine_weighted(const ep_layout_t* layout, const void* handle_mem,
                                size_t handle_bytes, const void* expert_out,
                                const float* recv_topk_weights, void* result,
                                hipStream_t stream);

/*
 * Backward of the weighted combine. For every live received row r holding
 * route s of token t = s/K:
 *   grad_expert_out[r,:]      = payload(fp32(w[r] * grad[t,:]))  (one fp32
 *                               product, then the payload rounding)
 *   grad_recv_topk_weights[r] = sum over h of grad[t,h] * expert_out[r,h]
 * Pad rows get +0 in both (not written with EP_LAYOUT_NO_PAD_FILL). The
 * weight gradient is an fp32 dot product over H accumulated in a fixed order,
 * bit-identical from run to run but not the sequential order: the row is cut
 * into P = ceil(H * elem / 1024) pieces of 64 16-byte vectors (N elements
 * each: 8 for bf16 and fp16, 4 for fp32); each lane chains N fused
 * multiply-adds over its vector, six butterfly adds combine a piece's lanes,
 * and the P partials are added in piece order. So every product passes
 * through at most n = N + P + 5 fp32 roundings and the result is within
 * gamma_n * sum_h |grad[t,h] * expert_out[r,h]| of the exact dot product,
 * gamma_n = n u / (1 - n u), u = 2^-24. (Rows of more than 1024 pieces, or
 * sizes whose piece indices pass 2^31, take a token-group form whose lanes
 * chain N * P multiply-adds: n = N * P + 6 there.) With
 * grad_recv_topk_weights NULL only the row gradient is computed and
 * expert_out may be NULL. Rows at or past min(total, recv_capacity) are not
 * written (+0, and +0 weight gradients, with EP_LAYOUT_ZERO_TAIL).
 *   grad                    payload [T,H]
 *   expert_out              payload [recv_capacity,H] or NULL
 *   recv_topk_weights       fp32 [recv_capacity]
 *   grad_expert_out         payload [recv_capacity,H]
 *   grad_recv_topk_weights  fp32 [recv_capacity] or NULL
 */
ep_status_t ep_combine_weighted_bwd(const ep_layout_t* layout, const void* handle_mem,
                                    size_t handle_bytes, const void* grad,
                                    const void* expert_out, const float* recv_topk_weights,
                                    void* grad_expert_out, float* grad_recv_topk_weights,
                                    hipStream_t stream);

/* Copy the handle's status word (EP_STATUS_* bits) to *host_out. Waits for
 * `stream`; not for the hot path. host_out is a host pointer. The library's
 * own addition: the review of "[PyTorch] Expert Parallelism: PyTorch wrapper
 * + autograd ops with symm-mem zero-copy" (thread on recv_capacity_per_rank)
 * has a sync-free mode drop what exceeds the static capacity and raise a
 * flag; this call reads that flag, and the bad-id and layout flags, back. */
ep_status_t ep_read_status(const void* handle_mem, uint32_t* host_out, hipStream_t stream);

/* Static description of an ep_status_t. Never NULL. Host only. The
 * library's own addition. */
const char* ep_status_str(ep_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* EP_MI355X_EP_H */
