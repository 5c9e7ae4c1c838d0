/*
 * moe.h - C ABI of the one-device MoE layer library (libmoe.so), gfx950 / MI355X.
 *
 * The layer is the dispatch -> expert FFN -> combine chain of the Ascend
 * low_latency_dispatch / low_latency_combine pair (low_latency_combine API page:
 * "Function" Description and Formula, "Prototype", "Parameters") with an
 * expert-parallel world of one device, so the all-to-all becomes an on-device
 * permutation, plus its backward.  Each expert's FFN is SwiGLU with
 * intermediate size F (the --ffn_dim of the Triton-distributed ep_moe_fused
 * benchmark page) and every expert's FFN runs as one grouped GEMM.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All tensor arguments are DEVICE pointers to contiguous row-major memory
 *   owned by the caller.  The library allocates nothing, keeps no state between
 *   calls and never synchronises: every call only enqueues kernels on `stream`
 *   (a hipStream_t; NULL means the null stream) and returns.
 * - bf16 tensors are passed as `const void*` / `void*` (IEEE bfloat16, 2 bytes).
 *   Indices are int32, masks uint8 (0 = false), weights and weight gradients
 *   float32.
 * - Notation: T tokens (BS), H hidden, F expert intermediate size, K top-k,
 *   E = num_experts (routed experts), Z/C/Q = zero/copy/const expert counts,
 *   slot s = t*K + k, A = number of active routed slots (= rows actually used in
 *   the expanded buffers, known only on the device as ep_recv_counts[E-1]),
 *   capacity = rows allocated for the expanded buffers.
 * - Host-checkable rule violations return a negative moe_status before any
 *   launch and leave every output untouched.  Data rules that only the device
 *   can see (ids out of range, duplicate ids in a row, a 1-D mask that is not a
 *   prefix) are reported through the err_flag output of moe_dispatch; outputs
 *   are then unspecified but every kernel stays in bounds (offending slots are
 *   treated as inactive).
 * - Results are deterministic: no floating-point atomics anywhere (the page's
 *   "Deterministic Computation" section).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t moe_status;

#define MOE_OK 0
#define MOE_ERR_NULL_ARG (-1)    /* a required pointer is NULL */
#define MOE_ERR_BAD_SHAPE (-2)   /* a size is out of range or misaligned */
#define MOE_ERR_BAD_RANGE (-3)   /* an enum-like field has an unknown value */
#define MOE_ERR_CAPACITY (-4)    /* capacity < T * min(E, K) */
#define MOE_ERR_UNSUPPORTED (-5) /* valid but not implemented combination */
#define MOE_ERR_WORKSPACE (-6)   /* workspace missing or too small */
#define MOE_ERR_HIP (-7)         /* a HIP launch failed */

/* err_flag bits written by moe_dispatch (device int32). */
#define MOE_FLAG_ID_RANGE 1          /* topk_idx value outside [0, E+Z+C+Q) */
#define MOE_FLAG_ID_DUPLICATE 2      /* the same id twice in one row of topk_idx */
#define MOE_FLAG_MASK_NOT_PREFIX 4   /* 1-D x_active_mask with a true after a false */
#define MOE_FLAG_SYNC_TIMEOUT 8      /* moe_decode_fused: a wait for another workgroup's
                                        result timed out; the output is not valid */

#define MOE_DTYPE_BF16 0

/* Codes stored in the slot-to-row part of assist_info_for_combine. */
#define MOE_SLOT_NONE (-1)  /* inactive slot, zero expert or invalid slot */
#define MOE_SLOT_COPY (-2)  /* copy expert: the slot's value is ori_x[t] */
/* constant expert j: code -(3 + j) */

typedef struct moe_shape {
  int64_t T;                /* tokens, >= 0 */
  int64_t H;                /* hidden size, > 0, multiple of 8 */
  int64_t F;                /* expert intermediate size, multiple of 32 (FFN calls only) */
  int64_t capacity;         /* rows of expand_x / y / grad buffers, >= T*min(E,K) */
  int32_t K;                /* top-k, 1..16 and <= E+Z+C+Q */
  int32_t num_experts;      /* routed experts E, 1..1024 */
  int32_t zero_expert_num;  /* Z >= 0: ids [E, E+Z) */
  int32_t copy_expert_num;  /* C >= 0: ids [E+Z, E+Z+C) */
  int32_t const_expert_num; /* Q >= 0: ids [E+Z+C, E+Z+C+Q) */
  int32_t mask_ndim;        /* 0: no x_active_mask, 1: (T,), 2: (T, K) */
  int32_t act_dtype;        /* MOE_DTYPE_BF16 */
  int32_t comm_quant_mode;  /* 0: none; 2: int8 expert-output payload in combine (see moe_combine) */
} moe_shape;

/* One expert weight tensor in block-scaled e4m3, as moe_quantize_weights_fp8
 * writes it: codes in the (out, in) layout (the forward GEMMs' operand), the
 * transposed codes (in, out) (the data gradients' operand) and the fp32 scale
 * of every 128 x 128 block, shared by both layouts. */
typedef struct moe_fp8_weight {
  const uint8_t* codes;    /* (E, N, Kdim) */
  const uint8_t* codes_t;  /* (E, Kdim, N) */
  const float* scales;     /* (E, N/128, Kdim/128) */
} moe_fp8_weight;

/* Human-readable name of a status code (static string). */
const char* moe_status_str(moe_status st);

/* Size of assist_info_for_combine in int32 elements: T*K (slot -> row) followed
 * by capacity (row -> slot).  Its contents are opaque to callers, like the
 * page's assist_info_for_combine (Parameters; Constraints: callers hand it to combine unchanged). */
moe_status moe_assist_info_size(const moe_shape* s, int64_t* n_int32);

/* Bytes of device workspace that moe_dispatch needs (for per-chunk expert
 * histograms).  The FFN entries take no workspace. */
moe_status moe_workspace_size(const moe_shape* s, size_t* bytes);

/*
 * moe_dispatch - route tokens to experts and build the expert-sorted buffer.
 * (low_latency_combine page, Parameters: topk_idx, x_active_mask,
 * assist_info_for_combine, ep_send_counts; with one device the dispatch
 * all-to-all is the permutation below.)
 *
 *  in   x                 (T, H) bf16        tokens
 *  in   topk_idx          (T, K) int32       expert id per slot
 *  in   x_active_mask     (T,) or (T, K) uint8, or NULL when mask_ndim == 0
 *  out  expand_x          (capacity, H) bf16 row r = x[token of row r]; rows >= A untouched
 *  out  assist_info_for_combine  see moe_assist_info_size:
 *                         slot2row[s] = row (>= 0) of an active routed slot,
 *                         MOE_SLOT_NONE, MOE_SLOT_COPY or -(3+j) for const expert j;
 *                         row2slot[r] = slot of row r (r < A)
 *  out  expert_token_nums (E,) int32         active routed slots per expert
 *  out  ep_recv_counts    (E,) int32         inclusive prefix sum of expert_token_nums
 *  out  err_flag          (1,) int32         MOE_FLAG_* bits (overwritten, 0 when clean)
 *  ws   workspace         >= moe_workspace_size bytes of device memory
 *
 * Rows of one expert are contiguous and in increasing slot order, experts in
 * id order, so row(s) = prefix[e-1] + #{s' < s : active routed slot of e}.
 * A masked slot, a zero-expert slot and an invalid slot get no row.
 */
moe_status moe_dispatch(const moe_shape* s, const void* x, const int32_t* topk_idx,
                        const uint8_t* x_active_mask, void* expand_x,
                        int32_t* assist_info_for_combine, int32_t* expert_token_nums,
                        int32_t* ep_recv_counts, int32_t* err_flag, void* workspace,
                        size_t ws_bytes, void* stream);

/*
 * moe_grouped_ffn - SwiGLU FFN of every expert over its rows, as grouped GEMMs.
 * For expert e and its rows [prefix[e-1], prefix[e]):
 *   G = X Wg_e^T, U = X Wu_e^T (fp32 accumulation), h = silu(G) * U,
 *   y = h Wd_e^T.
 *  in   expand_x       (capacity, H) bf16
 *  in   w_gate, w_up   (E, F, H) bf16, (out, in) layout per expert
 *  in   w_down         (E, H, F) bf16
 *  in   ep_recv_counts (E,) int32 from moe_dispatch
 *  out  gate_up_save   (capacity, 2F) bf16: [G | U] per row, kept for backward
 *  out  h_act          (capacity, F) bf16: h
 *  out  y              (capacity, H) bf16
 * Equivalent to moe_ffn_gate_up_fwd followed by moe_ffn_down_fwd.
 * Every FFN entry (forward and backward) needs one expert's weight matrix
 * below 2 GiB (F * H * 2 bytes < 2^31 - 16; the kernels address it with
 * 32-bit offsets), else MOE_ERR_UNSUPPORTED.
 */
moe_status moe_grouped_ffn(const moe_shape* s, const void* expand_x, const void* w_gate,
                           const void* w_up, const void* w_down, const int32_t* ep_recv_counts,
                           void* gate_up_save, void* h_act, void* y, void* stream);

/* moe_dispatch_fp8 - moe_dispatch for the fp8 GEMMs: the permute writes every
 * expanded row as e4m3 codes with one fp32 scale per 128 columns, quantised once
 * per token (the rule and layout of moe_quant_rows_fp8: amax of the 128 values,
 * codes e4m3(v * (448/amax)), scale amax/448, an all-zero block codes 0 and scale 1),
 * and, when expand_x is given, the bf16 rows too (the bf16 weight gradients
 * read them).  The low_latency_combine page's dispatch returns its quantised
 * expand_x with dynamic_scales the same way (Example, quant_mode 2).
 *  out  expand_x        (capacity, H) bf16, or NULL
 *  out  expand_xq       (capacity, H) uint8 e4m3 codes
 *  out  dynamic_scales  (H/128, capacity) fp32, block-major
 *  other arguments, outputs and checks as moe_dispatch; H must be a multiple of
 *  128 (MOE_ERR_BAD_SHAPE). */
moe_status moe_dispatch_fp8(const moe_shape* s, const void* x, const int32_t* topk_idx,
                            const uint8_t* x_active_mask, void* expand_x, uint8_t* expand_xq, float* dynamic_scales,
                            int32_t* assist_info_for_combine, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                            int32_t* err_flag, void* workspace, size_t ws_bytes, void* stream);

/* moe_dispatch_noalloc - moe_dispatch for callers that cannot allocate device
 * memory: code under stream capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, outputs and checks as moe_dispatch, without the
 * workspace: the routing scratch is a fixed 256 KiB device array inside the
 * library (one per GPU, held until the process ends; its address is looked up
 * on the first call on each device).  The call allocates nothing.
 *  MOE_ERR_WORKSPACE when the shape's routing scratch (moe_workspace_size)
 *  exceeds 256 KiB; the routing's chunking keeps it at or below 129 KiB for
 *  every shape check_shape accepts, so this is a guard only.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on one GPU (different streams, threads) race; calls in one stream order are
 * safe, and nothing needs clearing between calls. */
moe_status moe_dispatch_noalloc(const moe_shape* s, const void* x, const int32_t* topk_idx,
                                const uint8_t* x_active_mask, void* expand_x, int32_t* assist_info_for_combine,
                                int32_t* expert_token_nums, int32_t* ep_recv_counts, int32_t* err_flag,
                                void* stream);

/* moe_route - the routing half of moe_dispatch alone: the same assist info,
 * expert_token_nums, ep_recv_counts and err_flag (same arguments, same checks),
 * without x and without writing expanded rows.  For callers that read the
 * tokens through the row -> slot map instead (moe_ffn_gate_up_fwd_gather). */
moe_status moe_route(const moe_shape* s, const int32_t* topk_idx, const uint8_t* x_active_mask,
                     int32_t* assist_info_for_combine, int32_t* expert_token_nums, int32_t* ep_recv_counts,
                     int32_t* err_flag, void* workspace, size_t ws_bytes, void* stream);

/* moe_ffn_gate_up_fwd_gather - moe_ffn_gate_up_fwd with the dispatch permute
 * folded into its operand loads: expanded row r is read as x[slot(r) / K],
 * slot(r) from the assist info of moe_route or moe_dispatch, so the result is
 * bit for bit that of moe_ffn_gate_up_fwd on moe_dispatch's expand_x.
 *  in   x (T, H) bf16; assist_info_for_combine as written by the routing;
 *       w_gate, w_up, ep_recv_counts as for moe_ffn_gate_up_fwd
 *  out  gate_up_save (capacity, 2F), h_act (capacity, F) bf16
 * MOE_ERR_UNSUPPORTED when (T + 1) * H * 2 bytes exceed 2^31 - 16 (31-bit
 * operand offsets). */
moe_status moe_ffn_gate_up_fwd_gather(const moe_shape* s, const void* x, const int32_t* assist_info_for_combine,
                                      const void* w_gate, const void* w_up, const int32_t* ep_recv_counts,
                                      void* gate_up_save, void* h_act, void* stream);

/* First grouped GEMM of moe_grouped_ffn (gate and up projections with the
 * SwiGLU product fused into its epilogue).  One kernel launch. */
moe_status moe_ffn_gate_up_fwd(const moe_shape* s, const void* expand_x, const void* w_gate,
                               const void* w_up, const int32_t* ep_recv_counts,
                               void* gate_up_save, void* h_act, void* stream);

/* Second grouped GEMM of moe_grouped_ffn: y = h Wd_e^T.  One kernel launch. */
moe_status moe_ffn_down_fwd(const moe_shape* s, const void* h_act, const void* w_down,
                            const int32_t* ep_recv_counts, void* y, void* stream);

/*
 * moe_combine - weighted merge of the expert outputs back to tokens
 * (low_latency_combine page, Function: Formula; Parameters).
 *   out[t] = sum over k = 0..K-1 of topk_weights[t,k] * v(t,k), then + shared_expert_x[t]
 * where v is y[row] for a routed slot, 0 for a zero expert (and for a masked
 * slot), ori_x[t] for a copy expert and alpha_1[j]*ori_x[t] + alpha_2[j]*v[j]
 * for constant expert j.  The sum runs in k order in fp32 with separately
 * rounded products (no fused multiply-add), the shared term is added last and
 * the result is rounded once to bf16.  With s->comm_quant_mode == 2 (the page's
 * int8 communication quantisation, Parameters: comm_quant_mode) every routed
 * slot's row of y is first replaced by its per-row symmetric int8 round trip,
 * clamp(rint(y * (127/amax)), -127, 127) * (amax/127), amax = max |y| over the row.
 *  in   y                        (capacity, H) bf16 (rows < A are read)
 *  in   topk_idx                 (T, K) int32  (shape check only; routing is in assist info)
 *  in   topk_weights             (T, K) float32
 *  in   assist_info_for_combine  from moe_dispatch
 *  in   ep_send_counts           (E,) int32 = ep_recv_counts of moe_dispatch
 *  in   x_active_mask            as given to moe_dispatch (already folded into assist info)
 *  in   shared_expert_x          (T, H) bf16 or NULL
 *  in   ori_x                    (T, H) bf16; required when C + Q > 0
 *  in   const_alpha_1/_2, const_v  (Q, H) bf16; required when Q > 0
 *  out  out                      (T, H) bf16
 */
moe_status moe_combine(const moe_shape* s, const void* y, const int32_t* topk_idx,
                       const float* topk_weights, const int32_t* assist_info_for_combine,
                       const int32_t* ep_send_counts, const uint8_t* x_active_mask,
                       const void* shared_expert_x, const void* ori_x, const void* const_alpha_1,
                       const void* const_alpha_2, const void* const_v, void* out, void* stream);

/*
 * moe_combine_bwd - gradient of moe_combine.
 *   grad_y[row]          = bf16(topk_weights[t,k] * grad_out[t])      (routed rows)
 *   grad_topk_weights[t,k] = <v(t,k), grad_out[t]> in fp32 (0 for masked/zero slots)
 * The gradient of shared_expert_x is grad_out itself; the copy/const terms'
 * gradient to ori_x is added by moe_dispatch_bwd.  With comm_quant_mode == 2 the
 * dot product uses the int8 round trip of y, as the forward did.
 * Either output may be NULL (not both: MOE_ERR_NULL_ARG), and the call then
 * computes the other alone, bit for bit as the call with both: grad_y alone
 * reads no y row (y may be NULL; for routing weights that need no gradient, about
 * half the bytes and time), grad_topk_weights alone writes no grad_y row.
 * One kernel launch.
 */
moe_status moe_combine_bwd(const moe_shape* s, const void* grad_out, const void* y,
                           const int32_t* topk_idx, const float* topk_weights,
                           const int32_t* assist_info_for_combine, const int32_t* ep_send_counts,
                           const uint8_t* x_active_mask, const void* ori_x,
                           const void* const_alpha_1, const void* const_alpha_2,
                           const void* const_v, void* grad_y, float* grad_topk_weights,
                           void* stream);

/* moe_ffn_gate_up_bwd_weight_gather - moe_ffn_gate_up_bwd_weight with the
 * dispatch permute folded into its expanded-row operand: expanded row r is read as
 * x[slot(r) / K] through the row -> slot map of the assist info (as
 * moe_ffn_gate_up_fwd_gather does for the forward), so a step that routes with
 * moe_route needs no expand_x at all.  Bit for bit that of
 * moe_ffn_gate_up_bwd_weight on moe_dispatch's expand_x.
 *  in   grad_gate_up (capacity, 2F) bf16; x (T, H) bf16; assist_info_for_combine
 *       as written by the routing; ep_recv_counts (E,)
 *  out  grad_w_gate, grad_w_up (E, F, H) fp32
 * MOE_ERR_UNSUPPORTED when (T + 1) * H * 2 bytes exceed 2^31 - 16 (31-bit
 * operand offsets).  One kernel launch. */
moe_status moe_ffn_gate_up_bwd_weight_gather(const moe_shape* s, const void* grad_gate_up, const void* x,
                                             const int32_t* assist_info_for_combine, const int32_t* ep_recv_counts,
                                             float* grad_w_gate, float* grad_w_up, void* stream);

/*
 * moe_grouped_ffn_bwd - backward of moe_grouped_ffn, four grouped GEMMs.
 *   dH = dY Wd_e;  with s = sigmoid(G): dG = dH*U*s*(1 + G(1-s)), dU = dH*G*s
 *   grad_gate_up = [dG | dU] (bf16), dX = [dG dU] [Wg_e; Wu_e] (bf16)
 *   dWd_e = dY^T h, dWg_e = dG^T X, dWu_e = dU^T X (fp32; experts with no rows get 0)
 *  in   grad_y (capacity, H), expand_x (capacity, H), gate_up_save (capacity, 2F),
 *       h_act (capacity, F): bf16;  w_gate, w_up, w_down as in moe_grouped_ffn
 *  out  grad_gate_up (capacity, 2F) bf16, grad_expand_x (capacity, H) bf16,
 *       grad_w_gate, grad_w_up (E, F, H) fp32, grad_w_down (E, H, F) fp32
 * Equivalent to moe_ffn_down_bwd_data, moe_ffn_down_bwd_weight,
 * moe_ffn_gate_up_bwd_data and moe_ffn_gate_up_bwd_weight in that order.
 */
moe_status moe_grouped_ffn_bwd(const moe_shape* s, const void* grad_y, const void* expand_x,
                               const void* gate_up_save, const void* h_act, const void* w_gate,
                               const void* w_up, const void* w_down,
                               const int32_t* ep_recv_counts, void* grad_gate_up,
                               void* grad_expand_x, float* grad_w_gate, float* grad_w_up,
                               float* grad_w_down, void* stream);

/* grad_gate_up = SwiGLU backward of (grad_y Wd_e).  One kernel launch. */
moe_status moe_ffn_down_bwd_data(const moe_shape* s, const void* grad_y, const void* w_down,
                                 const void* gate_up_save, const int32_t* ep_recv_counts,
                                 void* grad_gate_up, void* stream);

/* grad_w_down[e] = grad_y_e^T h_e.  One kernel launch. */
moe_status moe_ffn_down_bwd_weight(const moe_shape* s, const void* grad_y, const void* h_act,
                                   const int32_t* ep_recv_counts, float* grad_w_down,
                                   void* stream);

/*
 * The combine backward folded into the down GEMMs' operand loads.  The combine
 * backward's grad_y row of expanded row r is bf16(topk_weights[s] * grad_out[s / K])
 * with s = slot(r) (low_latency_combine page, "Function": the gradient of the
 * weighted sum); the two down-backward GEMMs below form it in registers from
 * grad_out read through the row -> slot map, so the step never writes or reads
 * grad_y (2 bytes per routed row and column each way).  The weights' gradient and
 * the down weight gradient are bit for bit those of moe_combine_bwd +
 * moe_ffn_down_bwd_weight (the weight gradient forms bf16(w * grad_out) rows in
 * registers); the down data gradient multiplies each row's fp32 product
 * grad_out[s / K] Wd_e by the row's weight (one bf16 rounding fewer than
 * moe_ffn_down_bwd_data on grad_y; within the element-wise parity bar of it).
 *
 * moe_combine_bwd_weights - grad_topk_weights as moe_combine_bwd computes it, and
 *   row_weights[r] = topk_weights[slot(r)] for every routed row r (rows past the
 *   routed ones are not written); no grad_y.  grad_topk_weights may be NULL
 *   (routing weights that need no gradient): then no y row is read.
 *  out  grad_topk_weights (T, K) fp32 or NULL, row_weights (capacity,) fp32
 *  other arguments as moe_combine_bwd.  One kernel launch.
 */
moe_status moe_combine_bwd_weights(const moe_shape* s, const void* grad_out, const void* y,
                                   const int32_t* topk_idx, const float* topk_weights,
                                   const int32_t* assist_info_for_combine, const int32_t* ep_send_counts,
                                   const uint8_t* x_active_mask, const void* ori_x, const void* const_alpha_1,
                                   const void* const_alpha_2, const void* const_v, float* grad_topk_weights,
                                   float* row_weights, void* stream);

/* moe_ffn_down_bwd_data_gather - moe_ffn_down_bwd_data with dH[r] =
 * row_weights[r] * (grad_out[slot(r) / K] Wd_e) in fp32, grad_out (T, H) bf16 read
 * through the assist info's row -> slot map, row_weights from
 * moe_combine_bwd_weights.  MOE_ERR_UNSUPPORTED when (T + 1) * H * 2 bytes
 * exceed 2^31 - 16 (31-bit operand offsets).  One kernel launch. */
moe_status moe_ffn_down_bwd_data_gather(const moe_shape* s, const void* grad_out,
                                        const int32_t* assist_info_for_combine, const float* row_weights,
                                        const void* w_down, const void* gate_up_save,
                                        const int32_t* ep_recv_counts, void* grad_gate_up, void* stream);

/* moe_ffn_down_bwd_weight_gather - moe_ffn_down_bwd_weight on grad_y rows
 * bf16(row_weights[r] * grad_out[slot(r) / K]) formed in registers (bit for bit).
 * Same limit.  One kernel launch. */
moe_status moe_ffn_down_bwd_weight_gather(const moe_shape* s, const void* grad_out,
                                          const int32_t* assist_info_for_combine, const float* row_weights,
                                          const void* h_act, const int32_t* ep_recv_counts,
                                          float* grad_w_down, void* stream);

/* grad_expand_x = grad_gate_up [Wg_e; Wu_e].  One kernel launch. */
moe_status moe_ffn_gate_up_bwd_data(const moe_shape* s, const void* grad_gate_up,
                                    const void* w_gate, const void* w_up,
                                    const int32_t* ep_recv_counts, void* grad_expand_x,
                                    void* stream);

/* grad_w_gate[e] = dG_e^T X_e, grad_w_up[e] = dU_e^T X_e.  One kernel launch. */
moe_status moe_ffn_gate_up_bwd_weight(const moe_shape* s, const void* grad_gate_up,
                                      const void* expand_x, const int32_t* ep_recv_counts,
                                      float* grad_w_gate, float* grad_w_up, void* stream);

/* moe_combine_bwd_fp8 - moe_combine_bwd for the fp8 data gradients: every dY
 * row also leaves as e4m3 codes with one fp32 scale per 128 columns, the rule
 * and layout of moe_quant_rows_fp8 applied to the bf16 dY (so the codes equal
 * that quantiser run on grad_y).
 *  out  grad_y         (capacity, H) bf16, or NULL when only the codes are needed
 *  out  grad_yq        (capacity, H) uint8 e4m3 codes
 *  out  grad_y_scales  (H/128, capacity) fp32, block-major
 *  other arguments and outputs as moe_combine_bwd; H must be a multiple of 128. */
moe_status moe_combine_bwd_fp8(const moe_shape* s, const void* grad_out, const void* y, const int32_t* topk_idx,
                               const float* topk_weights, const int32_t* assist_info_for_combine,
                               const int32_t* ep_send_counts, const uint8_t* x_active_mask, const void* ori_x,
                               const void* const_alpha_1, const void* const_alpha_2, const void* const_v,
                               void* grad_y, uint8_t* grad_yq, float* grad_y_scales, float* grad_topk_weights,
                               void* stream);

/*
 * moe_dispatch_bwd - gradient with respect to the layer input x (= ori_x).
 *   grad_x[t] = sum over k (k order) of: grad_expand_x[row] (routed slot),
 *               w * grad_out[t] (copy slot), w * (alpha_1[j] * grad_out[t])
 *               (constant slot j); then + grad_x_accum[t]; one bf16 rounding.
 *  in   grad_expand_x (capacity, H) bf16, assist_info_for_combine, topk_idx (T,K),
 *       topk_weights (T,K) fp32, x_active_mask (as for dispatch, folded already),
 *       grad_out (T,H) bf16 (required when C + Q > 0), const_alpha_1 (Q,H) bf16
 *       (required when Q > 0), grad_x_accum (T,H) bf16 or NULL (e.g. the
 *       shared expert's input gradient)
 *  out  grad_x (T, H) bf16
 */
moe_status moe_dispatch_bwd(const moe_shape* s, const void* grad_expand_x,
                            const int32_t* assist_info_for_combine, const int32_t* topk_idx,
                            const float* topk_weights, const uint8_t* x_active_mask,
                            const void* grad_out, const void* const_alpha_1,
                            const void* grad_x_accum, void* grad_x, void* stream);

/* ------------------------------------------------------------------ fp8 path
 * Block-scaled OCP e4m3 (1-4-3, bias 7, max 448, round to nearest even,
 * saturating): scale = amax/448 per block (fp32, 1 for an all-zero block),
 * code = e4m3(x * (448/amax)), value = code * scale.  The forward GEMMs and the
 * two data-gradient GEMMs of the FFN run on e4m3 operands with fp32
 * accumulation (each 128-wide K block's partial sum times its A and B scales);
 * the weight gradients keep the bf16 entries above, or run on per-128-token
 * codes (the fp8 weight-gradient entries below).  The pages name FP8 only as
 * a precision of the MoE layer performance tests (Megatron-LM page, Added Test
 * Cases); the block recipe is this library's.  H and F must be multiples of 128
 * (else MOE_ERR_BAD_SHAPE), H and 2F at most 32768 and the activation scales
 * below 2 GiB (capacity * max(H, 2F)/128 * 4 bytes; else MOE_ERR_UNSUPPORTED).
 */

/* Rows of a bf16 (R, C) matrix to e4m3 with one scale per (row, 128 columns).
 *  codes (R, C) uint8, scales (C/128, R) fp32 (column-block major: a GEMM K step
 *  reads consecutive rows' scales from consecutive words; the GEMM entries take
 *  scales of all `capacity` rows, so quantise the whole (capacity, C) buffer).
 *  nrows: optional device int32; when given only rows < *nrows are written
 *  (e.g. ep_recv_counts + E-1). */
moe_status moe_quant_rows_fp8(int64_t R, int64_t C, const void* src, const int32_t* nrows,
                              uint8_t* codes, float* scales, void* stream);

/* Expert weights (E, N, K) bf16 to e4m3 with one scale per 128 x 128 block:
 *  codes (E, N, K) uint8, scales (E, N/128, K/128) fp32, and (optional) the
 *  codes transposed per expert, codes_t (E, K, N), for the data-gradient GEMMs. */
moe_status moe_quantize_weights_fp8(int64_t E, int64_t N, int64_t K, const void* w,
                                    uint8_t* codes, uint8_t* codes_t, float* scales,
                                    void* stream);

/* fp8 moe_ffn_gate_up_fwd: xq/xs = moe_quant_rows_fp8 of expand_x (capacity, H);
 * wgq/wgs, wuq/wus = moe_quantize_weights_fp8 of w_gate, w_up.  Outputs as the
 * bf16 entry (gate_up_save, h_act in bf16). */
moe_status moe_ffn_gate_up_fwd_fp8(const moe_shape* s, const uint8_t* xq, const float* xs,
                                   const uint8_t* wgq, const float* wgs, const uint8_t* wuq,
                                   const float* wus, const int32_t* ep_recv_counts,
                                   void* gate_up_save, void* h_act, void* stream);

/* moe_ffn_gate_up_fwd_fp8 that also writes the per-128-token e4m3 codes of the
 * h_act it produces: hq_t (F, ld) / hs_t (slots, F), bit-identical to
 * moe_quant_cols_fp8 of h_act (the fp8 weight-gradient operand). */
moe_status moe_ffn_gate_up_fwd_fp8_quant(const moe_shape* s, const uint8_t* xq, const float* xs,
                                         const uint8_t* wgq, const float* wgs, const uint8_t* wuq,
                                         const float* wus, const int32_t* ep_recv_counts,
                                         void* gate_up_save, void* h_act, uint8_t* hq_t, float* hs_t,
                                         void* stream);

/* fp8 moe_ffn_down_fwd: hq/hs = moe_quant_rows_fp8 of h_act (capacity, F);
 * wdq/wds = moe_quantize_weights_fp8 of w_down.  y in bf16. */
moe_status moe_ffn_down_fwd_fp8(const moe_shape* s, const uint8_t* hq, const float* hs,
                                const uint8_t* wdq, const float* wds,
                                const int32_t* ep_recv_counts, void* y, void* stream);

/* fp8 moe_ffn_down_bwd_data: dyq/dys = moe_quant_rows_fp8 of grad_y (capacity, H);
 * wdq_t = transposed codes of w_down (E, F, H), wds its block scales. */
moe_status moe_ffn_down_bwd_data_fp8(const moe_shape* s, const uint8_t* dyq, const float* dys,
                                     const uint8_t* wdq_t, const float* wds,
                                     const void* gate_up_save, const int32_t* ep_recv_counts,
                                     void* grad_gate_up, void* stream);

/* moe_ffn_down_bwd_data_fp8 with the quantisation of its output fused in: the
 * same dG/dU, rounded to bf16, written as any of
 *   grad_gate_up (capacity, 2F) bf16               (optional),
 *   dguq (capacity, 2F) / dgus (2F/128, capacity)  = moe_quant_rows_fp8 of it
 *                                                    for rows < ep_recv_counts[E-1],
 *   dguq_t (2F, ld) / dgus_t (slots, 2F)           = moe_quant_cols_fp8 of it
 * (each code/scale pair given together or not at all; at least one output,
 * else MOE_ERR_NULL_ARG).  Bit-identical to running the quantisers on
 * grad_gate_up.  The fp8 weight-gradient path needs no bf16 dG/dU at all. */
moe_status moe_ffn_down_bwd_data_fp8_quant(const moe_shape* s, const uint8_t* dyq, const float* dys,
                                           const uint8_t* wdq_t, const float* wds,
                                           const void* gate_up_save, const int32_t* ep_recv_counts,
                                           void* grad_gate_up, uint8_t* dguq, float* dgus,
                                           uint8_t* dguq_t, float* dgus_t, void* stream);

/* fp8 moe_ffn_gate_up_bwd_data: dguq/dgus = moe_quant_rows_fp8 of grad_gate_up
 * (capacity, 2F); wgq_t/wuq_t = transposed codes of w_gate, w_up (E, H, F). */
moe_status moe_ffn_gate_up_bwd_data_fp8(const moe_shape* s, const uint8_t* dguq,
                                        const float* dgus, const uint8_t* wgq_t, const float* wgs,
                                        const uint8_t* wuq_t, const float* wus,
                                        const int32_t* ep_recv_counts, void* grad_expand_x,
                                        void* stream);

/* ------------------------------------------------------ fp8 weight gradients
 * The weight-gradient GEMMs contract over an expert's rows, so their e4m3
 * operands carry one scale per (128 tokens, column) instead of per (row, 128
 * columns): each expert's rows are cut into 128-row token slots starting at its
 * first row (the last one may be shorter), and each (slot, column) is one
 * quantisation block (same rule as above).  Expert e's slots are numbered from
 * prefix[e-1]/128 + e (prefix = ep_recv_counts), so with
 *   slots = capacity/128 + E,  ld = 128 * slots
 * a code matrix of a (capacity, D) activation is (D, ld) uint8, row d holding
 * column d with slot s at codes [128 s, 128 s + 128), and its scales are
 * (slots, D) fp32.  Codes of a slot's rows past its expert's end are 0; slots
 * that no row falls in are left unwritten (and never read).  The reading of
 * "per-128-token requantisation" and the layout are this library's.
 */

/* Per-128-token e4m3 codes of an expert-sorted bf16 (capacity, D) matrix
 * (expand_x, h_act, grad_y or grad_gate_up), D a multiple of 128.
 *  in  src (capacity, D) bf16, ep_recv_counts (E) int32 (device, from dispatch)
 *  out codes_t (D, 128 * slots) uint8, scales (slots, D) fp32
 * Errors: MOE_ERR_BAD_SHAPE (D not a positive multiple of 128, E < 1, sizes
 * beyond 2^40 codes), MOE_ERR_NULL_ARG.  One kernel launch. */
moe_status moe_quant_cols_fp8(int64_t capacity, int64_t D, int32_t num_experts, const void* src,
                              const int32_t* ep_recv_counts, uint8_t* codes_t, float* scales,
                              void* stream);

/* fp8 moe_ffn_down_bwd_weight: grad_w_down (E, H, F) fp32 = per expert the sum
 * over its token slots of (dY codes x h codes) times the two slots' column
 * scales.  dyq_t/dys = moe_quant_cols_fp8 of grad_y (D = H), hq_t/hs of h_act
 * (D = F).  Experts without rows get zero gradients.  Shape rules of the fp8
 * path; MOE_ERR_UNSUPPORTED when max(H, F) * ld reaches 2^31 bytes. */
moe_status moe_ffn_down_bwd_weight_fp8(const moe_shape* s, const uint8_t* dyq_t, const float* dys,
                                       const uint8_t* hq_t, const float* hs,
                                       const int32_t* ep_recv_counts, float* grad_w_down,
                                       void* stream);

/* fp8 moe_ffn_gate_up_bwd_weight: grad_w_gate, grad_w_up (E, F, H) fp32 from
 * dguq_t/dgus = moe_quant_cols_fp8 of grad_gate_up (D = 2F; rows < F of the
 * code matrix are the gate columns) and xq_t/xs of expand_x (D = H).
 * MOE_ERR_UNSUPPORTED when max(2F, H) * ld reaches 2^31 bytes. */
moe_status moe_ffn_gate_up_bwd_weight_fp8(const moe_shape* s, const uint8_t* dguq_t,
                                          const float* dgus, const uint8_t* xq_t, const float* xs,
                                          const int32_t* ep_recv_counts, float* grad_w_gate,
                                          float* grad_w_up, void* stream);

/* ------------------------------------------------------ microscaled fp8 (MX)
 * The fp8 GEMMs with gfx950's block-scaled MFMA doing the scaling: every e4m3
 * operand carries one E8M0 scale byte (2^(byte-127)) per 32 consecutive codes
 * of its contraction dimension.  The scale is the smallest power of two that
 * brings the block's largest magnitude within 448 (amax = M * 2^E, 1 <= M < 2:
 * 2^(E-8), or 2^(E-7) when M > 1.75; clamped to 2^-127 .. 2^127; an all-zero
 * block gets byte 0), so no code saturates; codes = e4m3(x / scale).  The
 * recipe is this library's (the survey's NEXT-2 names the hardware feature; the
 * pages give no recipe).  Weights are quantised twice: along H (the forward
 * GEMMs) and, transposed, along F or H (the data gradients).  Shape rules of
 * the fp8 path (H, F multiples of 128).
 */

/* Rows of a bf16 (R, C) matrix, C a multiple of 32: codes (R, C) uint8 and R*C/32
 * scale bytes, stored as one 4-byte word per (row, 128 columns) -- the scales of
 * the four 32-blocks in order -- with words ordered (column block, row): byte
 * ((c/128) * R + r) * 4 + (c/32) % 4 holds the scale of row r, columns c..c+31
 * (a GEMM K step then reads consecutive rows' scales from consecutive words).
 * nrows as in moe_quant_rows_fp8.  One kernel launch. */
moe_status moe_quant_rows_mx(int64_t R, int64_t C, const void* src, const int32_t* nrows,
                             uint8_t* codes, uint8_t* scales, void* stream);

/* Expert weights (E, N, K) bf16, N and K multiples of 128: codes (E, N, K) with
 * E*N*K/32 scale bytes along K (moe_quant_rows_mx layout over the E*N rows),
 * and (optional, both or neither) the transposes codes_t (E, K, N) with their
 * E*K*N/32 scale bytes along N (the same layout over the E*K rows of the
 * transposes).  Two kernel launches. */
moe_status moe_quantize_weights_mx(int64_t E, int64_t N, int64_t K, const void* w, uint8_t* codes,
                                   uint8_t* scales, uint8_t* codes_t, uint8_t* scales_t, void* stream);

/* MX moe_ffn_gate_up_fwd: xq/xs = moe_quant_rows_mx of expand_x; wgq/wgs,
 * wuq/wus = moe_quantize_weights_mx codes/scales of w_gate, w_up.  hq/hs
 * (optional, both or neither): the MX row codes of the h_act it writes, as
 * moe_quant_rows_mx of h_act would give them (codes (capacity, F), scales in its
 * layout over capacity rows) -- the down GEMM's input without a separate pass. */
moe_status moe_ffn_gate_up_fwd_mx(const moe_shape* s, const uint8_t* xq, const uint8_t* xs,
                                  const uint8_t* wgq, const uint8_t* wgs, const uint8_t* wuq,
                                  const uint8_t* wus, const int32_t* ep_recv_counts,
                                  void* gate_up_save, void* h_act, uint8_t* hq, uint8_t* hs,
                                  void* stream);

/* MX moe_ffn_down_fwd: hq/hs = moe_quant_rows_mx of h_act; wdq/wds of w_down. */
moe_status moe_ffn_down_fwd_mx(const moe_shape* s, const uint8_t* hq, const uint8_t* hs,
                               const uint8_t* wdq, const uint8_t* wds, const int32_t* ep_recv_counts,
                               void* y, void* stream);

/* MX moe_ffn_down_bwd_data: dyq/dys = moe_quant_rows_mx of grad_y; wdq_t/wds_t =
 * the transposed codes/scales of w_down.  Writes grad_gate_up (bf16, optional)
 * and/or dguq/dgus (both or neither): the MX row codes of it (capacity, 2F), as
 * moe_quant_rows_mx would give them; at least one output. */
moe_status moe_ffn_down_bwd_data_mx(const moe_shape* s, const uint8_t* dyq, const uint8_t* dys,
                                    const uint8_t* wdq_t, const uint8_t* wds_t, const void* gate_up_save,
                                    const int32_t* ep_recv_counts, void* grad_gate_up, uint8_t* dguq,
                                    uint8_t* dgus, void* stream);

/* MX moe_ffn_gate_up_bwd_data: dguq/dgus = moe_quant_rows_mx of grad_gate_up;
 * wgq_t/wgs_t, wuq_t/wus_t = transposed codes/scales of w_gate, w_up ((E, H, F),
 * (E, H, F/32)). */
moe_status moe_ffn_gate_up_bwd_data_mx(const moe_shape* s, const uint8_t* dguq, const uint8_t* dgus,
                                       const uint8_t* wgq_t, const uint8_t* wgs_t, const uint8_t* wuq_t,
                                       const uint8_t* wus_t, const int32_t* ep_recv_counts,
                                       void* grad_expand_x, void* stream);

/* ------------------------------------------------------------------ int8 path
 * The decode regime of the low_latency_combine page's examples: dispatch with
 * quant_mode 2 ("dynamic quantization") returns an int8 expand_x and
 * dynamic_scales, optionally scaling each row first by an fp32 (num_experts, H)
 * scales tensor (example programs; the page gives no formula).  Reading taken
 * here: row = x_t times scales[e] for the routed expert e (float32 products),
 * codes clamp(rint(v * (127/amax)), -127, 127) (ties to even), dynamic scale
 * amax/127 (an all-zero row: codes 0, scale 1) -- the rule of the int8 combine
 * payload.  The grouped FFN on those rows (not on the pages) runs w8a8: int8
 * weights with one scale per output channel (moe_quant_rows_int8 over the
 * E*N rows of the (out, in) matrices), exact integer sums times (row scale x
 * channel scale), bf16 outputs; h is requantised per row for the down
 * projection.  H and F multiples of 128 for the GEMMs (MOE_ERR_BAD_SHAPE).
 */

/* moe_dispatch with int8 expanded rows.  Same routing outputs (assist,
 * counts, err_flag) as moe_dispatch; expand_x (capacity, H) int8 and
 * dynamic_scales (capacity) fp32 for the rows < ep_recv_counts[E-1].
 * smooth_scales: NULL or (num_experts, H) fp32.  H <= 8192 (the row is held in
 * registers; else MOE_ERR_UNSUPPORTED).  Four kernel launches: the three routing
 * kernels of moe_dispatch and a quantising permute. */
moe_status moe_dispatch_int8(const moe_shape* s, const void* x, const int32_t* topk_idx,
                             const uint8_t* x_active_mask, const float* smooth_scales,
                             int8_t* expand_x, float* dynamic_scales, int32_t* assist_info_for_combine,
                             int32_t* expert_token_nums, int32_t* ep_recv_counts, int32_t* err_flag,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Rows of a bf16 (R, C) matrix to int8 with one scale per row (rule above),
 * C a multiple of 8: codes (R, C) int8, scales (R) fp32; nrows: optional device
 * int32, only rows < *nrows are written.  Also the weight quantiser of the int8
 * path, with R = E*N rows of K. */
moe_status moe_quant_rows_int8(int64_t R, int64_t C, const void* src, const int32_t* nrows,
                               int8_t* codes, float* scales, void* stream);

/* w8a8 moe_ffn_gate_up_fwd: xq/xs = moe_dispatch_int8 outputs; wgq/wgs,
 * wuq/wus = moe_quant_rows_int8 of w_gate, w_up ((E, F, H) codes, (E, F)
 * scales).  gate_up_save and h_act in bf16. */
moe_status moe_ffn_gate_up_fwd_int8(const moe_shape* s, const int8_t* xq, const float* xs,
                                    const int8_t* wgq, const float* wgs, const int8_t* wuq,
                                    const float* wus, const int32_t* ep_recv_counts,
                                    void* gate_up_save, void* h_act, void* stream);

/* w8a8 moe_ffn_down_fwd: hq/hs = moe_quant_rows_int8 of h_act; wdq/wds of
 * w_down ((E, H, F) codes, (E, H) scales).  y in bf16. */
moe_status moe_ffn_down_fwd_int8(const moe_shape* s, const int8_t* hq, const float* hs,
                                 const int8_t* wdq, const float* wds, const int32_t* ep_recv_counts,
                                 void* y, void* stream);

/* ------------------------------------------------------------------ router
 * The pages take topk_idx and topk_weights as inputs (low_latency_combine page,
 * "Parameters": K distinct ids per token in [0, E+Z+C+Q), one float weight per
 * token and choice) and print no router.  These two entries give the plain
 * softmax top-K gating that produces them, over every id a slot may take
 * (routed and special experts), and its backward.  Sizes: T >= 0 tokens,
 * n_ids ids per token (1 <= n_ids <= 4096), 0 < K <= min(16, n_ids), renorm 0
 * or 1 (else MOE_ERR_BAD_SHAPE / MOE_ERR_BAD_RANGE).  Logits are fp32; a NaN
 * logit counts as -inf.
 */

/* moe_router - topk_idx (T, K) int32: the ids of the K largest logits of each
 * row, in descending order, equal logits by increasing id.  topk_weights (T, K)
 * fp32: softmax(logits row)[topk_idx] (renorm = 0), or those K values divided by
 * their sum (renorm = 1, a softmax over the selected logits).
 *  in  logits (T, n_ids) fp32.  One kernel launch. */
moe_status moe_router(int64_t T, int64_t n_ids, int32_t K, int32_t renorm, const float* logits,
                      int32_t* topk_idx, float* topk_weights, void* stream);

/* moe_router_bwd - gradient of sum(grad_topk_weights * topk_weights) with
 * respect to the logits, the selection held fixed:
 *   renorm = 1: grad_logits[i] = w_i (dw_i - sum_k w_k dw_k) for a chosen id i,
 *               0 for the others (logits may be NULL);
 *   renorm = 0: grad_logits[i] = p_i ([i chosen] dw_i - sum_k w_k dw_k) for every
 *               id, p = softmax(logits row).
 *  in  logits (T, n_ids) fp32; topk_idx, topk_weights (T, K) from moe_router;
 *      grad_topk_weights (T, K) fp32 (e.g. from moe_combine_bwd)
 *  out grad_logits (T, n_ids) fp32, every element written.  One kernel launch. */
moe_status moe_router_bwd(int64_t T, int64_t n_ids, int32_t K, int32_t renorm, const float* logits,
                          const int32_t* topk_idx, const float* topk_weights,
                          const float* grad_topk_weights, float* grad_logits, void* stream);

/* Bytes of device workspace that moe_grouped_ffn_fp8 and moe_grouped_ffn_bwd_fp8
 * need (the e4m3 codes and scales they pass between their GEMMs). */
moe_status moe_ffn_fp8_workspace_size(const moe_shape* s, size_t* bytes);

/* moe_grouped_ffn_fp8 - moe_grouped_ffn on block-scaled e4m3 operands (the fp8
 * reading of the Megatron-LM MoE test page's FP8 precision, Added Test Cases):
 * the gate/up GEMM on the rows moe_dispatch_fp8 quantised, h's codes (one scale
 * per 128 columns), the down GEMM.  Three launches.
 *  in   expand_xq (capacity, H) e4m3, x_scales (H/128, capacity) fp32
 *  in   w[3]      gate, up (E, F, H) and down (E, H, F) weights, moe_fp8_weight
 *  out  gate_up_save (capacity, 2F), h_act (capacity, F), y (capacity, H) bf16
 *  ws   workspace >= moe_ffn_fp8_workspace_size bytes
 * H and F multiples of 128 (MOE_ERR_BAD_SHAPE). */
moe_status moe_grouped_ffn_fp8(const moe_shape* s, const uint8_t* expand_xq, const float* x_scales,
                               const moe_fp8_weight* w, const int32_t* ep_recv_counts, void* gate_up_save,
                               void* h_act, void* y, void* workspace, size_t ws_bytes, void* stream);

/* moe_grouped_ffn_bwd_fp8 - the backward of moe_grouped_ffn_fp8: the fp8 data
 * gradients on dY's codes (moe_combine_bwd_fp8) with the SwiGLU backward and the
 * codes of dG|dU fused into the down data gradient, and the weight gradients in
 * bf16 on the bf16 dY, h, dG|dU and expanded rows.  Four launches.
 *  in   grad_y (capacity, H) bf16; grad_yq (capacity, H) e4m3, grad_y_scales (H/128, capacity)
 *  in   expand_x (capacity, H) bf16 (moe_dispatch_fp8's bf16 rows); gate_up_save, h_act
 *  in   w[3] as for moe_grouped_ffn_fp8 (the transposed codes are read)
 *  out  grad_gate_up (capacity, 2F) bf16, grad_expand_x (capacity, H) bf16
 *  out  grad_w_gate, grad_w_up (E, F, H), grad_w_down (E, H, F) fp32
 *  ws   workspace >= moe_ffn_fp8_workspace_size bytes */
moe_status moe_grouped_ffn_bwd_fp8(const moe_shape* s, const void* grad_y, const uint8_t* grad_yq,
                                   const float* grad_y_scales, const void* expand_x, const void* gate_up_save,
                                   const void* h_act, const moe_fp8_weight* w, const int32_t* ep_recv_counts,
                                   void* grad_gate_up, void* grad_expand_x, float* grad_w_gate, float* grad_w_up,
                                   float* grad_w_down, void* workspace, size_t ws_bytes, void* stream);

/* moe_decode_fused - NOT ENABLED in this build: after validating its arguments
 * it returns MOE_ERR_UNSUPPORTED without launching (its first GPU runs did not
 * complete and the cause is not found).  What it is written to do:
 * the layer forward of a decode batch in ONE persistent
 * launch: routing (moe_dispatch's classification and stable expert order), the
 * gate/up GEMM with the SwiGLU epilogue on x rows gathered through the routing,
 * the down GEMM and the combine (moe_combine's formula, special experts, mask,
 * shared term and int8 payload).  The decode regime of the low_latency_combine
 * API page (Constraints: BS <= 512; Example: the decode flow of quant_mode 2).
 * out is bit-identical to moe_dispatch -> moe_ffn_gate_up_fwd ->
 * moe_ffn_down_fwd -> moe_combine on the same inputs (same arithmetic, same
 * K order).
 *  in   x (T, H) bf16, topk_idx (T, K) int32, topk_weights (T, K) fp32,
 *       x_active_mask as for moe_dispatch (NULL when mask_ndim is 0)
 *  in   w_gate, w_up (E, F, H), w_down (E, H, F) bf16
 *  in   shared_expert_x, ori_x, const_alpha_1/_2, const_v as for moe_combine
 *  out  out (T, H) bf16; err_flag (1,) int32: the routing's MOE_FLAG_* bits,
 *       plus MOE_FLAG_SYNC_TIMEOUT if a wait timed out
 *  ws   workspace >= moe_decode_fused_workspace_size bytes, ZERO-FILLED before
 *       its first use with this function; every call leaves its control words
 *       zero again.  It also holds the call's routing (expert counts, inclusive
 *       prefix, slot -> row and row -> slot maps) and the h and y rows.  Calls
 *       that share a workspace must not overlap (one stream).
 * One cooperative launch of one 512-thread workgroup per CU: workgroup 0 routes,
 * then all take gate/up, down and combine work items from an atomic counter;
 * down items wait for their expert's gate/up items and combine items for all
 * down items (bounded waits).  Requires T <= 512 (MOE_ERR_UNSUPPORTED), H a
 * multiple of 128 and F of 64 (MOE_ERR_BAD_SHAPE), T*H*2, F*H*2 and
 * capacity*F*2 below 2^31 bytes (MOE_ERR_UNSUPPORTED); MOE_ERR_HIP when the
 * cooperative launch fails. */
moe_status moe_decode_fused_workspace_size(const moe_shape* s, size_t* bytes);
moe_status moe_decode_fused(const moe_shape* s, const void* x, const int32_t* topk_idx,
                            const float* topk_weights, const uint8_t* x_active_mask, const void* w_gate,
                            const void* w_up, const void* w_down, const void* shared_expert_x, const void* ori_x,
                            const void* const_alpha_1, const void* const_alpha_2, const void* const_v, void* out,
                            int32_t* err_flag, void* workspace, size_t workspace_bytes, void* stream);

/* moe_hbm_stream - a reference streaming kernel (not part of the layer): the
 * measured HBM ceiling that the gather-reduce kernels are compared with.
 *  mode 0  copy   bytes from src to dst (each byte read once, written once)
 *  mode 1  read   bytes of src; writes 4096 * 256 16-byte vectors to sink (16 MiB)
 *  mode 2  write  bytes to dst (a fixed pattern)
 * 4096 workgroups, each streaming one contiguous range with 16-byte accesses,
 * eight loads in flight per lane.  bytes must be
 * a multiple of 16 (MOE_ERR_BAD_SHAPE); mode outside 0..2 gives MOE_ERR_BAD_RANGE. */
moe_status moe_hbm_stream(int32_t mode, const void* src, void* dst, int64_t bytes, void* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
