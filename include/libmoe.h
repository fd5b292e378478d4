/*
 * libmoe -- the Mixtral sparse Mixture-of-Experts feed-forward layer on AMD
 * MI355X (gfx950), as a C ABI.
 *
 * The layer (all from "Mixtral of Experts", section 2.1 "Sparse Mixture of
 * Experts", garden.houmin.site translation; the same definitions appear in
 * prose on the jerryyang.ai blog page):
 *
 *   logits   l = x . W_g                                 (a linear router)
 *   gates    G(x) = Softmax(TopK(l)),  TopK keeps the K largest logits and
 *            sets the others to -inf, so their gates are exactly 0
 *   experts  E_i(x) = (silu(x . w1_i) * (x . w3_i)) . w2_i   (SwiGLU block)
 *   output   y = sum_i G(x)_i * E_i(x),  evaluated only for the K experts
 *            with a non-zero gate (skipping zero gates is exact)
 *
 * Mixtral uses n = 8 experts and K = 2 (Table 1: dim 4096, hidden_dim 14336).
 * The same calls serve the fine-grained layout the ai360xpert.com summary
 * mentions (a token picks, for instance, 8 of 160 far narrower experts): n up
 * to 256.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Row-vector convention, row-major storage, experts outermost:
 *      x        bf16 [T][D]        (T = tokens, D = dim)
 *      w_gate   bf16 [D][n]
 *      w1, w3   bf16 [n][D][H]     (H = hidden)
 *      w2       bf16 [n][H][D]
 *  - Every pointer is a DEVICE pointer owned by the caller.  The library never
 *    allocates or frees memory and keeps no state between calls; all scratch
 *    comes from the caller's workspace (see moe_workspace_bytes).
 *  - Every call only validates its arguments on the host and enqueues kernels
 *    on `stream` (a hipStream_t; NULL is the default stream).  There is no
 *    device-to-host read and no synchronisation inside the library, so a call
 *    can be captured into a HIP graph.
 *  - Errors: arguments are checked before anything is enqueued; on an
 *    argument error the function returns a non-zero moe_status_t and enqueues
 *    nothing.  A failed kernel launch returns MOE_EHIP (kernels enqueued
 *    before it stay enqueued).  tokens == 0 is a valid no-op.  No C++
 *    exception crosses this interface.
 *  - A workspace holds a call's intermediate results until that call's last
 *    kernel has run, so calls that may run concurrently (on different
 *    streams, or in parallel branches of one graph) need separate
 *    workspaces.  Calls in order on one stream may share one.
 *  - Pointers must be 16-byte aligned; dim and hidden must be multiples of 8;
 *    1 <= top_k <= n_experts <= MOE_MAX_EXPERTS.
 *  - Ties in TopK go to the lower expert index; slot 0 of each token holds the
 *    larger logit.  Gates are fp32.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Diagnostics: with the environment variable LIBMOE_LOG set (to anything
 *    but "" or "0") when the first call is made, every call that enqueues
 *    work prints one line to stderr: the entry point, T, D, H, n, K, the
 *    output type, the expert-product path the shape selects, and the
 *    returned status.  Unset, it costs one atomic load per call.
 */
#ifndef LIBMOE_H
#define LIBMOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Rows of the permuted (expert-grouped) layout are grouped in segments whose
 * length is a multiple of this granule: expert e owns rows
 * [expert_offset[e], expert_offset[e+1]) and the first expert_count[e] of them
 * hold its token-slots. */
#define MOE_TILE_M 256
#define MOE_MAX_EXPERTS 256
/* Largest T the weight-streaming expert path takes (path STREAM). */
#define MOE_STREAM_MAX_TOKENS 128

typedef enum {
  MOE_OK = 0,
  MOE_EINVAL = 1,      /* bad argument: null/misaligned pointer, bad size */
  MOE_ENOTSUP = 2,     /* valid but unsupported shape: n_experts > 256, or a
                        * size past the 32-bit offsets the kernels use
                        * (D*H*2, T*D*2 or MOE_TILE_M*H*2 bytes >= 2^31, or
                        * moe_capacity_rows >= 2^31) */
  MOE_EWORKSPACE = 3,  /* workspace missing or smaller than moe_workspace_bytes */
  MOE_EHIP = 4         /* a HIP launch failed: hipGetLastError() after the
                        * launch was not hipSuccess (this also reports an
                        * earlier error the calling thread had not read) */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype_t;

/* Expert-product path.  AUTO takes the weight-streaming kernels for
 * T <= moe_decode_max_tokens() and the tiled matrix-core kernels above.
 * STREAM forces the weight-streaming path (T <= MOE_STREAM_MAX_TOKENS,
 * MOE_ENOTSUP above); TILED
 * forces the tiled path at any T.  Both give results within the same
 * tolerance of the exact layer; they are not bit-identical to each other. */
typedef enum { MOE_PATH_AUTO = 0, MOE_PATH_STREAM = 1, MOE_PATH_TILED = 2 } moe_path_t;

typedef struct {
  int32_t tokens;     /* T >= 0 */
  int32_t dim;        /* D, multiple of 8 */
  int32_t hidden;     /* H, multiple of 8 */
  int32_t n_experts;  /* n, 1..MOE_MAX_EXPERTS (256) */
  int32_t top_k;      /* K, 1..n */
  int32_t out_dtype;  /* moe_dtype_t of the layer output `out` */
  int32_t path;       /* moe_path_t: which expert-product kernels to use */
} moe_problem_t;

/* Number of rows of the permuted layout: T*K + n*(MOE_TILE_M-1) rounded up to
 * MOE_TILE_M (the worst case over all routings).  -1 if p is invalid. */
int64_t moe_capacity_rows(const moe_problem_t* p);

/* Bytes of device workspace that moe_forward needs; also enough for
 * moe_grouped_ffn.  0 if p is invalid.  The workspace must be 256-byte
 * aligned. */
size_t moe_workspace_bytes(const moe_problem_t* p);

/* Static text for a status code. */
const char* moe_status_string(int32_t status);

/* Router and gate: logits = x . W_g, then G(x) = Softmax(TopK(logits)).
 * (section 2.1, the G(x) and TopK definitions)
 *   x         bf16 [T][D]      in
 *   w_gate    bf16 [D][n]      in
 *   topk_idx  int32 [T][K]     out: chosen experts, slot 0 = largest logit,
 *                                   ties to the lower index
 *   topk_gate fp32 [T][K]      out: softmax over the K kept logits
 *   logits    fp32 [T][n]      out, optional (NULL to skip)
 *   ws, ws_bytes               scratch of moe_route_workspace_bytes(p) bytes
 *                              (NULL/0 when that is 0; else MOE_EWORKSPACE)
 * Logits accumulate in fp32.  From 2048 tokens with a multiple of 4 experts
 * (at most 16), they are computed on the matrix cores; when W_g (D rounded up
 * to a multiple of 32, times n, in bf16) takes at most 64 KiB, in one pass with
 * no scratch.  With more than 16 experts, or from 2048 tokens with a larger
 * W_g, they are computed in contraction slices whose partial sums pass through
 * ws and are added in slice order. */
size_t moe_route_workspace_bytes(const moe_problem_t* p);
moe_status_t moe_route(const moe_problem_t* p, const void* x, const void* w_gate,
                       int32_t* topk_idx, float* topk_gate, float* logits, void* ws,
                       size_t ws_bytes, void* stream);

/* Group token-slots by expert (the "skip experts whose gate is zero" step of
 * section 2.1: each expert sees only the tokens routed to it, in unequal
 * numbers).  Slot s = t*K + k is token t's k-th choice.
 *   topk_idx      int32 [T*K]     in: expert of each slot; a value outside
 *                                     [0, n) drops that slot (it then adds
 *                                     nothing to the output)
 *   expert_count  int32 [n]       out: slots routed to each expert
 *   expert_offset int32 [n+1]     out: segment starts, each segment padded to
 *                                     a multiple of MOE_TILE_M rows
 *   row_slot      int32 [cap]     out: slot held by each permuted row, -1 for
 *                                     padding (cap = moe_capacity_rows)
 *   slot_row      int32 [T*K]     out: permuted row of each slot (-1 if dropped)
 * Within an expert, slots keep increasing slot order (stable).  A token may
 * name an expert more than once (the router never does; a caller's routing
 * may): each such slot is a row of its own. */
moe_status_t moe_permute(const moe_problem_t* p, const int32_t* topk_idx,
                         int32_t* expert_count, int32_t* expert_offset,
                         int32_t* row_slot, int32_t* slot_row, void* stream);

/* Every selected expert's SwiGLU block on its rows (section 2.1, the expert
 * function and the final display equation):
 *   y_rows[r] = (silu(x_t . w1_e) * (x_t . w3_e)) . w2_e
 * for each permuted row r of expert e holding a slot of token t.
 *   x             bf16 [T][D]     in
 *   expert_count  int32 [n], expert_offset int32 [n+1], row_slot int32 [cap]
 *                                 in: as written by moe_permute
 *   w1, w3 bf16 [n][D][H], w2 bf16 [n][H][D]   in
 *   y_rows        fp32 [cap][D]   out: rows offset[e] .. offset[e]+count[e]-1
 *                                 of every expert; rows of padding are left
 *                                 as they were
 *   ws, ws_bytes  workspace, >= moe_workspace_bytes(p)
 * The intermediate silu(a)*b is rounded once to bf16 (it is the input of the
 * second product); products accumulate in fp32.  Every row of an expert is
 * computed, whatever its count (up to T*K when tokens repeat an expert). */
moe_status_t moe_grouped_ffn(const moe_problem_t* p, const void* x,
                             const int32_t* expert_count, const int32_t* expert_offset,
                             const int32_t* row_slot, const void* w1, const void* w3,
                             const void* w2, float* y_rows, void* ws, size_t ws_bytes,
                             void* stream);

/* Gate-weighted sum of each token's expert outputs (section 2.1, first display
 * equation), summed in slot order:
 *   out[t] = sum_k topk_gate[t][k] * y_rows[slot_row[t*K+k]]
 *   y_rows    fp32 [cap][D]   in
 *   slot_row  int32 [T*K]     in (-1 entries add nothing)
 *   topk_gate fp32 [T][K]     in
 *   out       [T][D] of p->out_dtype (fp32, or bf16 rounded to nearest even)
 */
moe_status_t moe_combine(const moe_problem_t* p, const float* y_rows,
                         const int32_t* slot_row, const float* topk_gate, void* out,
                         void* stream);

/* The whole layer: moe_route -> moe_permute -> moe_grouped_ffn -> moe_combine
 * on one stream, with every intermediate in the workspace.
 *   out        [T][D] of p->out_dtype   out
 *   topk_idx   int32 [T][K]  out, optional (NULL: kept in the workspace)
 *   topk_gate  fp32 [T][K]   out, optional (NULL: kept in the workspace)
 * For small batches (T <= moe_decode_max_tokens()) the expert products run as
 * bandwidth-bound weight streaming instead of the tiled matrix-core GEMM. */
moe_status_t moe_forward(const moe_problem_t* p, const void* x, const void* w_gate,
                         const void* w1, const void* w3, const void* w2, void* out,
                         int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                         void* stream);

/* moe_forward with stage timestamps for profiling.  `events` is NULL or an
 * array of 6 hipEvent_t created by the caller; they are recorded on `stream`
 * before the router, after the router, after the permute, after the first
 * expert product (x.w1 / x.w3 with silu), after the second (.w2) and after the
 * combine.  A NULL entry is skipped (each recorded event costs the stream a
 * few microseconds, so a caller timing one stage records only its two).  On
 * the weight-streaming path (T <= moe_decode_max_tokens()) there is no
 * permute pass: event 2 directly follows event 1.  The computation and its
 * results are exactly those of moe_forward. */
moe_status_t moe_forward_timed(const moe_problem_t* p, const void* x, const void* w_gate,
                               const void* w1, const void* w3, const void* w2, void* out,
                               int32_t* topk_idx, float* topk_gate, void* ws, size_t ws_bytes,
                               void* stream, void* const* events);

/* Routing diagnostics ("Mixtral of Experts", section 5, Routing analysis:
 * the per-expert token shares of Figure 7 and Figure 9, the consecutive-token
 * repetition rates of Table 5), as exact integer counts.
 *   topk_idx  int32 [T][K]  in: slot 0 is the first choice
 *   counts    int32 [2n+2]  out (device): [0, n) slots per expert among first
 *             choices; [n, 2n) slots per expert over all K choices; [2n] tokens
 *             t < T-1 whose first choice equals token t+1's; [2n+1] tokens
 *             t < T-1 that share any chosen expert with token t+1.
 * Ids outside [0, n) are not counted and match nothing.  Unlike the other
 * calls, T = 0 still writes the (zero) counts.  Shares and rates are these
 * counts divided by T, T*K or T-1 on the host. */
moe_status_t moe_route_stats(const moe_problem_t* p, const int32_t* topk_idx, int32_t* counts,
                             void* stream);

/* Largest T for which moe_forward and moe_grouped_ffn take the weight-streaming
 * (decode) path. */
int32_t moe_decode_max_tokens(void);

/* moe_forward without a workspace, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  The same layer, the same kernels and bit-identical
 * results as moe_forward on its weight-streaming path; every intermediate
 * lives in a library-owned device array of MOE_NOALLOC_SCRATCH_BYTES that
 * each GPU the library runs on holds until the process ends.  The call
 * allocates and frees nothing.
 *   Accepted: the batches moe_forward streams (T <= moe_decode_max_tokens()
 *   with path AUTO, T <= MOE_STREAM_MAX_TOKENS with path STREAM) whose
 *   intermediates fit the
 *   array: about 4*T*K*(2 + (2*S1 + 1/2)*H + S2*D) bytes: the first
 *   product's fp32 a and b in S1 = 1, 2 or 4 contraction partials, bf16 h,
 *   and S2 = 1..8 second-product partials (the larger counts when few experts
 *   can be touched, i.e. small T*K).  Mixtral's shape (D = 4096, H = 14336,
 *   K = 2) needs 27 MB at T = 64.  Other shapes, and path TILED, return
 *   MOE_ENOTSUP with nothing enqueued.
 *   stream must belong to the calling thread's current device (MOE_EINVAL
 *   otherwise).
 * Every call on one GPU uses that GPU's single array and leaves its contents
 * behind; no part of it needs clearing (a call reads only what it wrote).
 * Calls that may overlap in time on one GPU (other streams, host threads,
 * graph branches) race on it: the caller must order them. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
moe_status_t moe_forward_noalloc(const moe_problem_t* p, const void* x, const void* w_gate,
                                 const void* w1, const void* w3, const void* w2, void* out,
                                 int32_t* topk_idx, float* topk_gate, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMOE_H */
