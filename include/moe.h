/*
 * moe.h — C-ABI of the routed-expert MoE layer run through a bounded, quantized
 * expert cache, for AMD Instinct MI355X (gfx950).
 *
 * Sources (web pages; cited by title and section):
 *   [HF-PR]  "POC: Experts offload" (huggingface/transformers draft PR 50717):
 *            PR description and its three commit messages.
 *   [RFC]    "RFC: stream MoE experts from disk in from_pretrained":
 *            sections "Feature request", "Motivation", "How the prototype works",
 *            "Questions for maintainers".
 *   [SUBST]  BigMoeOnEdge docs "Limitations and prior art" with the commit message
 *            that adds cache-aware substitution (Skliar et al., arXiv:2412.00099).
 *   [CLASS]  "moe: expert slots in size classes" (1bit engine PR 137): PR
 *            description, commit message, and the ExpertCache constructor quoted
 *            in its review.
 *
 * ---------------------------------------------------------------------------
 * Shared conventions
 * ---------------------------------------------------------------------------
 * Ownership.  The caller allocates and owns every buffer and every stream/event.
 *   Device pointers are plain device addresses; the library never frees them.
 *   The library allocates host memory only: inside a moe_cache, a moe_store, and
 *   a moe_pipeline (whose pinned host tier and staging rows come from
 *   hipHostMalloc, with its HIP events); never device memory.
 * Asynchrony.  Every GPU entry point only enqueues work on the given stream and
 *   returns.  Its status covers host-side argument checks and launch errors.
 * Errors.  Entry points return MOE_OK (0) or a negative MOE_E_* code and set a
 *   thread-local message readable with moe_last_error().  Faults found on the
 *   device (an expert that is not resident, a slot out of range, a non-finite
 *   logit, an expert id out of range) are OR-ed as MOE_ERRW_* bits into the
 *   caller-owned device word `err_word` (uint32), which the caller reads after
 *   synchronising; rows touched by such a fault hold unspecified values.
 *   `err_word` may be NULL, in which case device faults are not reported.
 * Limits.  1 <= E <= 1024; 1 <= k <= min(E, 32); H and I multiples of 64;
 *   bits in {3, 4, 6, 8, 16}; T >= 0 (T == 0 is a no-op returning MOE_OK).
 * Streams.  hipStream_t 0 is the null stream.  No entry point synchronises.
 *
 * ---------------------------------------------------------------------------
 * Byte format of one expert row in a slot ([RFC] "How the prototype works":
 * experts are gated, concatenated, untransposed, without bias, and each expert
 * is one contiguous row; the weights are group-wise affine quantized)
 * ---------------------------------------------------------------------------
 * An expert with hidden size H and intermediate size I is two matrices:
 *   gate_up : 2I rows x H columns, rows 0..I-1 are the gate projection and rows
 *             I..2I-1 the up projection (out x in, like a linear layer: y = W x);
 *   down    : H rows x I columns.
 * Each matrix is stored as a code block followed by a scale/bias block.  The four
 * blocks sit in this order, each starting at a multiple of `align` (256) bytes:
 *   [gate_up codes][gate_up scale/bias][down codes][down scale/bias]
 * and slot_bytes is the end of the last block rounded up to `align`.
 *
 * Code block of an R x C matrix with b bits per code: row n occupies C*b/8 bytes
 * starting at n*C*b/8.  Inside a row, values come in pack units of 32: unit u
 * (columns 32u..32u+31) is b little-endian uint32 words at byte 4*b*u of the
 * row, and column 32u+i holds bits [b*i, b*i+b) of the 32*b-bit little-endian
 * integer those words form (for b = 3 and 6 a code may straddle two words).
 *
 * Scale/bias block: for row n and group g (columns 64g..64g+63), 4 bytes at
 * byte offset 4*(n*(C/64) + g): an IEEE fp16 scale s then an IEEE fp16 bias z,
 * both little-endian.  The dequantized weight is  w[n][c] = s*q + z  with q the
 * unsigned code; s*q is exact in fp32, so the only rounding is the add.
 *
 * Width 16 (unquantized experts; [RFC] "How the prototype works", Cache bullet:
 * BF16 experts run from the same pool): the "codes" are the bf16 weights
 * themselves (the rule above with b = 16 is the plain row-major little-endian
 * bf16 matrix) and the scale/bias block is empty (0 bytes), so the next block
 * starts at the same offset.  Each matrix's width is chosen separately.
 *
 * ---------------------------------------------------------------------------
 * Routing numeric contract ([RFC] "Motivation": each token uses k of E experts;
 * [SUBST] commit message: cache-aware substitution).  Per token, in fp32 with
 * no contraction of multiplies into adds unless a fused multiply-add is named:
 *   m   = max_e logit[e]
 *   e_i = exp_c(logit[i] - m)
 *   exp_c(x): x < -86 -> 0; n = rint(x * 1.44269502f); r = fma(-n, ln2_hi, x);
 *             r = fma(-n, ln2_lo, r) with ln2_hi = 0x3f317218, ln2_lo = 0xb102e308;
 *             degree-7 Taylor polynomial of e^r by Horner with fma, coefficients
 *             1/7!, 1/6!, 1/5!, 1/4!, 1/3!, 1/2, 1, 1 rounded to fp32;
 *             result times 2^n (exact).  exp_c(0) == 1.
 *   Z   = sum of e_i in a fixed order: 64 partials S_l = e_l + e_{l+64} + ...
 *         (ascending), then S_l += S_{l+32} for l < 32, S_l += S_{l+16} for
 *         l < 16, ..., S_0 += S_1; Z = S_0.
 *   p_i = e_i / Z, correctly rounded.
 *   key_i = p_i (plain mode), or p_i + c for experts with slot_table[i] >= 0 in
 *         substitution mode, where c = L * (max_e p - min_e p) (one rounded
 *         subtract, then one rounded multiply).
 *   ids  = top-k of key by repeated argmax; larger key first, equal keys ->
 *         smaller expert id first.  Output in that order.
 *   w_j  = p_{ids_j} / (p_{ids_0} + p_{ids_1} + ... summed left to right).
 * Substitution changes which experts are chosen, never how they are weighted.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK               0
#define MOE_E_INVALID       (-1) /* bad dims, bits, k, E, alignment, null pointer */
#define MOE_E_UNSUPPORTED   (-2) /* valid but not implemented                   */
#define MOE_E_NOT_RESIDENT  (-3) /* host-side check found a non-resident expert */
#define MOE_E_NO_SLOT       (-4) /* every slot of the size class is reserved   */
#define MOE_E_HIP           (-5) /* a HIP runtime call failed                   */
#define MOE_E_BUSY          (-6) /* a fill of this entry is still in flight     */
#define MOE_E_WORKSPACE     (-7) /* workspace smaller than the size query says  */
#define MOE_E_IO            (-8) /* the expert store could not be read          */

/* ---- device error-word bits --------------------------------------------- */
#define MOE_ERRW_NOT_RESIDENT  0x1u /* routed expert has slot_table[e] < 0      */
#define MOE_ERRW_BAD_SLOT      0x2u /* slot_table[e] >= n_slots                 */
#define MOE_ERRW_NONFINITE     0x4u /* a router logit is NaN or infinite        */
#define MOE_ERRW_BAD_ID        0x8u /* a top-k id outside [0, E)                */
#define MOE_ERRW_TIMEOUT      0x10u /* the fused decode kernel's h exchange gave up */

/* ---- routing modes ------------------------------------------------------- */
#define MOE_ROUTE_PLAIN  0
#define MOE_ROUTE_SUBST  1

/* ---- forward path selection --------------------------------------------- */
#define MOE_PATH_AUTO  0 /* GEMV for few pairs per expert, MFMA otherwise       */
#define MOE_PATH_GEMV  1 /* dequant-GEMV kernels (decode)                       */
#define MOE_PATH_MFMA  2 /* dequant + bf16 MFMA grouped GEMM (prefill)          */
#define MOE_PATH_GEMV3 3 /* GEMV as three launches (sort, gate/up, down)        */

/* ---- workspace --------------------------------------------------------------
 * The first MOE_WS_RESERVED_BYTES of a forward workspace belong to the fused
 * decode kernel's h exchange: MOE_WS_GEN_BYTES of call-tag counters (one per
 * workgroup slot, from dword 64), then MOE_WS_XWORDS 64-bit words, each an h
 * pair (two bf16) in its low half and the tag of the call that wrote it in its
 * high half.  The prefix must be zero before the first call on a workspace and
 * is written only by the library afterwards; every call leaves it consistent
 * for the next one.  No other buffer of any path overlaps it.                 */
#define MOE_WS_GEN_BYTES 8192
#define MOE_WS_XWORDS 32768
#define MOE_WS_RESERVED_BYTES (MOE_WS_GEN_BYTES + 8 * MOE_WS_XWORDS)

/* ---- cache install sources ----------------------------------------------- */
#define MOE_SRC_HOST    0 /* pinned host memory (hipHostMalloc)                 */
#define MOE_SRC_DEVICE  1 /* device memory                                      */

/* ---- weight element types of the one-time conversion ---------------------- */
#define MOE_DTYPE_F32   0
#define MOE_DTYPE_BF16  1

/*
 * Size class: every expert whose row has the same byte size shares one pool of
 * slots and one LRU ([CLASS] PR description: layers whose experts take the same
 * number of bytes form a class, and a class owns a separate slot pool and LRU).  Filled by
 * moe_size_class_init; all offsets are bytes from the start of a slot row.
 */
typedef struct moe_size_class_desc {
    int32_t H;            /* hidden size (multiple of 64)                      */
    int32_t I;            /* expert intermediate size (multiple of 64)         */
    int32_t bits_gu;      /* code width of gate_up: 3, 4, 6, 8 or 16 (bf16)    */
    int32_t bits_d;       /* code width of down:    3, 4, 6, 8 or 16 (bf16)    */
    int32_t group;        /* quantization group along the input dim: 64        */
    int32_t align;        /* block alignment in bytes: 256                     */
    int64_t n_slots;      /* slots in this class's pool                        */
    int64_t off_gu_codes; /* = 0                                               */
    int64_t off_gu_sb;
    int64_t off_d_codes;
    int64_t off_d_sb;
    int64_t slot_bytes;   /* bytes of one slot row (multiple of align)         */
} moe_size_class_desc;

/*
 * Fill `d` for an expert of the given shape and code widths.  group must be 64
 * and align 256 in this version.  Returns MOE_E_INVALID on bad arguments.
 * Source: [RFC] "How the prototype works" (each expert stored as a single
 * unbroken row) and [CLASS] PR description (an expert's size is the total of its
 * tensors' windows, each padded to the alignment).
 */
int moe_size_class_init(moe_size_class_desc* d, int H, int I, int bits_gu, int bits_d,
                        int group, int align, int64_t n_slots);

/*
 * Router logits of n_mats consecutive layers on one set of hidden states:
 * logits[m][t][e] = sum_i x[t][i] * w[m][e][i].  x: bf16 [T, H] (device);
 * w: bf16 [n_mats, E, H], the routers of the layers stacked in order (device);
 * logits: fp32 [n_mats, T, E] (device), fp32 sums of exact bf16 products.
 * These logits feed moe_route_topk to guess the experts the next layers will
 * ask for, before their hidden states exist.  Source: [RFC] "How the prototype
 * works", Reads bullet (the prediction for the two following layers applies
 * their router weights to the present layer's hidden state, and the predicted
 * experts are fetched while compute goes on).
 * Limits: H a positive multiple of 8, 1 <= E <= 1024, 1 <= n_mats <= 8, x and w
 * 16-byte aligned; T = 0 is a no-op.  Sized for decode batches (each four tokens
 * re-read the routers, from L2).
 */
int moe_router_logits(const void* x, int T, int H, const void* w, int n_mats, int E, float* logits,
                      hipStream_t stream);

/*
 * Router: softmax over E logits, top-k, renormalised weights, per the routing
 * numeric contract above.  In MOE_ROUTE_SUBST mode every expert with
 * slot_table[e] >= 0 gets L times the token's probability range added to its
 * selection key before top-k is taken ([SUBST] commit message); the weights
 * still come from the unbiased probabilities.
 *   logits     device fp32 [T, E], row-major.
 *   slot_table device int32 [E]; read only in MOE_ROUTE_SUBST mode (else NULL ok).
 *   topk_ids   device int32 [T, k] (out);  topk_w device fp32 [T, k] (out).
 *   err_word   device uint32 (may be NULL): MOE_ERRW_NONFINITE on NaN/inf logits.
 * Sources: [RFC] "Motivation" (each token uses 10 of 512 experts, only the top-k
 * are read); [SUBST] commit message.
 */
int moe_route_topk(const float* logits, int T, int E, int k, int mode, float L,
                   const int32_t* slot_table, int32_t* topk_ids, float* topk_w,
                   uint32_t* err_word, hipStream_t stream);

/*
 * Sort the T*k (token, slot j) pairs by expert.  Pair id p = t*k + j.
 *   expert_offsets device int32 [E+1] (out): offsets[e] = number of pairs routed
 *                  to experts < e; offsets[E] = T*k.
 *   sorted_pairs   device int32 [T*k] (out): pairs of expert e, ascending pair id,
 *                  at [offsets[e], offsets[e+1]).
 *   pass_table     device int32 [moe_pass_table_size(E, pass_experts)] (out):
 *                  [0] = n_hit (experts with at least one pair), [1] = n_passes,
 *                  [2 .. 2+E) = hit expert ids ascending, then -1;
 *                  [2+E .. 2+E+ceil(E/P)+1) = pass starts into the hit list:
 *                  pass q covers hit-list entries [start_q, start_{q+1}), at most
 *                  pass_experts (P) each; unused starts equal n_hit.
 *   ws             device scratch of moe_sort_workspace_size(T, k, E) bytes.
 *   err_word       MOE_ERRW_BAD_ID if an id is outside [0, E); such pairs are dropped.
 * Sources: [HF-PR] commit messages (the sorted prefill's batches of 64 experts);
 * [RFC] "How the prototype works", Prefill bullet (sorted gather, 64 experts per batch).
 */
int moe_sort_by_expert(const int32_t* topk_ids, int T, int k, int E, int pass_experts,
                       int32_t* expert_offsets, int32_t* sorted_pairs, int32_t* pass_table,
                       void* ws, size_t ws_bytes, uint32_t* err_word, hipStream_t stream);
size_t moe_sort_workspace_size(int T, int k, int E);
int    moe_pass_table_size(int E, int pass_experts);

/*
 * The routed experts of one layer:
 *   out[t] = sum_j topk_w[t,j] * down_e( silu(gate_e(x[t])) * up_e(x[t]) ),
 *   e = topk_ids[t,j], each linear map using the dequantized weights of the slot
 *   slot_table[e] of the pool `slot_pool` laid out as described by `d`.
 * Runs the sort internally (into ws), then gate/up + SwiGLU, down and the
 * weighted combine in fixed order (bit-reproducible run to run).
 *   x          device bf16 [T, H] (hipBfloat16 bits as uint16).
 *   topk_ids   device int32 [T, k];  topk_w device fp32 [T, k].
 *   slot_table device int32 [E]: slot of each expert, -1 if not resident.
 *   slot_pool  device bytes [d->n_slots * d->slot_bytes].
 *   out        device bf16 [T, H] (overwritten; round to nearest even).
 *   ws         device scratch of moe_forward_workspace_size(...) bytes, 256-byte
 *              aligned; its first MOE_WS_RESERVED_BYTES must be zero before the
 *              first call that uses it (the call-tag counters from byte 256 then
 *              count the fused calls).  Calls that share one ws must not overlap
 *              in time (same stream, or ordered by events).
 *   err_word   MOE_ERRW_NOT_RESIDENT / MOE_ERRW_BAD_SLOT / MOE_ERRW_BAD_ID /
 *              MOE_ERRW_TIMEOUT.
 * `path` selects the kernels (MOE_PATH_*); moe_experts_forward uses AUTO: a
 * one-launch decode kernel when the batch is one token (or T*k <= 64) and the
 * shape has a compiled variant that fits the device's LDS, the three-launch GEMV
 * kernels for other batches of at most 8 pairs, MFMA otherwise.
 * Co-residency precondition of the one-launch kernels (AUTO / GEMV at decode
 * sizes, and moe_layer_forward): their workgroups hand the SwiGLU activations to
 * one another through the workspace inside the launch, so every workgroup of the
 * grid must be running at the same time.  The grid is sized to at most one
 * workgroup per compute unit and the host checks that the kernel's resources
 * allow it, but a kernel on another stream or in another process that holds
 * compute units for long can keep a workgroup from starting.  Every wait is
 * bounded: when one expires the kernel sets MOE_ERRW_TIMEOUT, still ends, and
 * the contents of `out` are unspecified (routing results written by
 * moe_layer_forward are still exact).  MOE_PATH_GEMV3 and MOE_PATH_MFMA have no
 * waits between workgroups and no such precondition.
 * Sources: [HF-PR] PR description (the cached experts go through a gathered quantized matmul);
 * [RFC] "How the prototype works" (Cache, Prefill and Quantized experts bullets).
 */
int moe_experts_forward(const void* x, int T, const int32_t* topk_ids, const float* topk_w,
                        int k, int E, const int32_t* slot_table, const void* slot_pool,
                        const moe_size_class_desc* d, void* out, void* ws, size_t ws_bytes,
                        uint32_t* err_word, hipStream_t stream);
int moe_experts_forward_ex(const void* x, int T, const int32_t* topk_ids, const float* topk_w,
                           int k, int E, const int32_t* slot_table, const void* slot_pool,
                           const moe_size_class_desc* d, void* out, void* ws, size_t ws_bytes,
                           uint32_t* err_word, int path, hipStream_t stream);
size_t moe_forward_workspace_size(int T, int k, int E, const moe_size_class_desc* d);

/*
 * Router and routed experts of one layer: moe_route_topk followed by
 * moe_experts_forward, with the same arguments and the same results (ids and
 * weights bit-identical, outputs identical to MOE_PATH_GEMV).  For decode-sized
 * batches (T*k <= 64) both run in ONE launch: every workgroup routes the tokens
 * itself, so the layer needs no host round trip and no second kernel; the
 * routing is also written to topk_ids / topk_w.  Larger batches fall back to the
 * two calls.  Same workspace rules as moe_experts_forward.
 * Sources: "POC: Experts offload", commit messages (queued GPU work must not idle
 * between a layer's sub-steps); "RFC: stream MoE experts from disk in
 * from_pretrained", How the prototype works (with every expert resident, layers
 * never synchronise with the host).
 */
int moe_layer_forward(const float* logits, int T, int E, int k, int mode, float L, const void* x,
                      const int32_t* slot_table, const void* slot_pool, const moe_size_class_desc* d,
                      int32_t* topk_ids, float* topk_w, void* out, void* ws, size_t ws_bytes,
                      uint32_t* err_word, hipStream_t stream);

/*
 * moe_layer_forward with no workspace argument and no allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc.  Same arguments, semantics and
 * results as moe_layer_forward (bit-identical).  Its scratch is one array of
 * MOE_STATIC_SCRATCH_BYTES in the library's device memory per GPU, held until
 * the process ends; the first call on a device looks its address up and clears
 * its reserved prefix with a small kernel on `stream`.  A layer whose workspace
 * (moe_forward_workspace_size) exceeds MOE_STATIC_SCRATCH_BYTES is refused with
 * MOE_E_WORKSPACE before anything is enqueued.  Every call on one GPU shares
 * that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and give unspecified results; order them on one stream.
 * Allocates nothing: no hipMalloc, no hipFree, no allocating library routine.
 */
#define MOE_STATIC_SCRATCH_BYTES (8u << 20)
int moe_layer_forward_static(const float* logits, int T, int E, int k, int mode, float L, const void* x,
                             const int32_t* slot_table, const void* slot_pool,
                             const moe_size_class_desc* d, int32_t* topk_ids, float* topk_w, void* out,
                             uint32_t* err_word, hipStream_t stream);

/*
 * Prefill in passes.  A long prompt hits nearly every expert of a layer; its hit
 * experts run, in ascending id, in passes of at most 64, so that only one pass's
 * experts need to be resident at a time and the cache can be smaller than a
 * layer ([RFC] "How the prototype works", Prefill bullet; [HF-PR] commit
 * messages: the sorted prefill's batches of 64 experts).  One layer is:
 *   moe_prefill_sort    once: the stable sort of the T*k pairs by expert and the
 *                       pass table (the layout of moe_sort_by_expert, P = 64) plus
 *                       a permuted copy of x, all into ws;
 *   moe_prefill_pass    for passes [pass_begin, pass_end) of that table: gate/up,
 *                       SwiGLU and down of those passes' hit experts, each pair's
 *                       expert output (bf16) kept in ws; only the slots of these
 *                       experts are read, through `slot_table` as it is when the
 *                       call's kernels run (so the table and pool may change
 *                       between passes, ordered on the stream);
 *   moe_prefill_combine once, after the last pass: out[t] = sum_j w[t,j] * y[t,j]
 *                       in fp32, j ascending, bf16 round to nearest even.
 * Passes are 0 .. ceil(E/64) - 1; passes past the hit count are empty no-ops.
 * The three calls share one ws of moe_forward_workspace_size(T, k, E, d) bytes
 * (256-byte aligned; same T, k, E and d in every call) and must be ordered on
 * one stream or by events.  Running every pass in one call gives the same bits
 * as moe_experts_forward on MOE_PATH_MFMA.  Host status: MOE_E_INVALID (ranges,
 * NULL, alignment), MOE_E_WORKSPACE; device: as moe_experts_forward (an expert of
 * the passes run with no slot sets MOE_ERRW_NOT_RESIDENT; its pairs' outputs are
 * then unspecified).
 *
 * moe_pass_table_host: the same pass table computed on the host from host ids
 * (int32 [T, k] in host memory) into host memory of moe_pass_table_size(E, P)
 * int32: the hit experts of each pass, for the caller that makes a pass resident
 * before running it.  MOE_E_INVALID for an id outside [0, E).
 */
int moe_pass_table_host(const int32_t* topk_ids, int T, int k, int E, int pass_experts,
                        int32_t* pass_table);
int moe_prefill_sort(const void* x, int T, const int32_t* topk_ids, int k, int E,
                     const moe_size_class_desc* d, void* ws, size_t ws_bytes, uint32_t* err_word,
                     hipStream_t stream);
int moe_prefill_pass(int T, int k, int E, int pass_begin, int pass_end, const int32_t* slot_table,
                     const void* slot_pool, const moe_size_class_desc* d, void* ws, size_t ws_bytes,
                     uint32_t* err_word, hipStream_t stream);
int moe_prefill_combine(int T, int k, int E, const float* topk_w, const moe_size_class_desc* d,
                        void* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * One-time conversion of expert weights into slot rows of class d's format, the
 * rows a store file holds (see moe_store_open_file) and moe_cache_install copies.
 * Source: [RFC] "How the prototype works", Quantized experts bullet (an offline
 * pass converts the experts to the affine quantized format once and writes each
 * one as a single contiguous row).  The pages print no rule for scale and bias;
 * this library's reading, per row and group of 64 inputs:
 *   scale = (max - min) / (2^b - 1), bias = min, each rounded to the nearest fp16
 *   (ties to the even pattern; a zero minimum is stored as +0);
 *   code = (w - bias) / scale, computed in double from the fp16 scale and bias,
 *   rounded to nearest (ties to even) and clamped to [0, 2^b - 1]; 0 where the
 *   fp16 scale is 0.
 * Width 16 stores each weight rounded to the nearest bf16 (ties to even).
 * w_gu: [n_experts, 2I, H] (gate rows 0 .. I-1, then up rows), w_d:
 * [n_experts, H, I]; both device memory, row-major, element type `dtype`
 * (MOE_DTYPE_F32 or MOE_DTYPE_BF16), finite with |w| < 65504.
 * rows: device memory of n_experts * d->slot_bytes bytes, 256-byte aligned,
 * written whole (zero between blocks).  Asynchronous on `stream`; nothing is
 * allocated.  MOE_E_INVALID on a bad descriptor, dtype, pointer or alignment;
 * n_experts = 0 is a no-op.
 */
int moe_quantize_experts(const void* w_gu, const void* w_d, int dtype, int n_experts,
                         const moe_size_class_desc* d, void* rows, hipStream_t stream);

/*
 * Enqueue the copy of one expert row (d->slot_bytes bytes at `src`) into slot
 * `slot` of `slot_pool` on `copy_stream`, then record `done` (may be NULL) on it.
 * src_kind: MOE_SRC_HOST (pinned host memory) or MOE_SRC_DEVICE.  The copy is
 * asynchronous; the slot must not be read until `done` has completed (wait on it
 * from the compute stream).  Source: [RFC] "How the prototype works", Reads
 * bullet (a miss is a single read of the expert's row followed by a single
 * asynchronous copy to the device); [HF-PR] host-tier commit message.
 */
int moe_cache_install(void* slot_pool, const moe_size_class_desc* d, int64_t slot,
                      const void* src, int src_kind, hipStream_t copy_stream, hipEvent_t done);

/*
 * Host-side bounded expert cache: size classes, one LRU per class, per-layer
 * expert -> slot tables.  Source: [RFC] "How the prototype works", Cache bullet
 * (a fixed pool of slots allocated up front, LRU eviction, each layer's map from
 * expert to slot held on the host); [CLASS] PR description and constructor (a
 * class's slots are adjacent, slot byte offsets accumulate, unused slots are
 * queued at the LRU's tail so they are handed out before any eviction; every
 * class evicts on its own and no class borrows another's budget).
 *
 * moe_cache_create: classes[n_classes] (n_slots of each is that class's budget);
 *   layer_class[n_layers] maps each layer to its class; E experts per layer.
 *   Returns NULL on bad arguments (see moe_last_error).
 * moe_cache_acquire: make (layer, expert) resident.  Hit -> *slot, *needs_fill=0,
 *   entry moved to the LRU front.  Miss -> takes the LRU-back slot of the layer's
 *   class that is not pinned and not in flight, evicts its owner (its table entry
 *   becomes -1), *needs_fill = 1, and the entry is reserved (in flight) until
 *   moe_cache_fill_done / moe_cache_poll completes it.  MOE_E_NO_SLOT when every
 *   slot of the class is reserved or pinned.  An entry already in flight returns
 *   MOE_E_BUSY with *slot set and *needs_fill = 0.
 * moe_cache_fill_done: attach the event recorded after the install; the entry
 *   stays reserved until the event completes (checked by moe_cache_poll, and
 *   before every eviction).  ev == NULL marks the fill complete at once.
 * moe_cache_pin / moe_cache_unpin: keep (layer, expert) from eviction while a
 *   pass that reads it is queued (counted).
 * moe_cache_table: copy layer's expert -> slot table (int32 [E], -1 = absent)
 *   into host memory `table`.
 * moe_cache_stats: hits, misses, evictions since creation (any may be NULL).
 */
typedef struct moe_cache moe_cache;
moe_cache* moe_cache_create(const moe_size_class_desc* classes, int n_classes,
                            const int32_t* layer_class, int n_layers, int E);

/*
 * Eviction variants.  Sources: [RFC] "How the prototype works", Cache bullet (LRU,
 * optional LFU); [CLASS] PR description (one LRU per class, or one per layer with
 * --per-layer; each layer gets an equal fraction).
 * policy MOE_EVICT_LRU: the least recently used candidate goes.  MOE_EVICT_LFU:
 *   the candidate with the fewest acquires since it took its expert goes, ties to
 *   the least recently used.  A candidate is neither pinned nor in flight; empty
 *   slots always go first.
 * per_layer 0: one eviction order per class (moe_cache_create).  1: the class's
 *   n_slots are split between its layers in layer order, each a contiguous run of
 *   n_slots / L_c slots (the first n_slots % L_c layers one more), each with its
 *   own order; a layer never evicts another layer's expert.
 */
#define MOE_EVICT_LRU 0
#define MOE_EVICT_LFU 1
moe_cache* moe_cache_create_ex(const moe_size_class_desc* classes, int n_classes,
                               const int32_t* layer_class, int n_layers, int E, int policy,
                               int per_layer);
void moe_cache_destroy(moe_cache* c);
int  moe_cache_acquire(moe_cache* c, int layer, int expert, int64_t* slot, int* needs_fill);
int  moe_cache_fill_done(moe_cache* c, int layer, int expert, hipEvent_t ev);
int  moe_cache_poll(moe_cache* c);
int  moe_cache_pin(moe_cache* c, int layer, int expert);
int  moe_cache_unpin(moe_cache* c, int layer, int expert);
int  moe_cache_table(const moe_cache* c, int layer, int32_t* table);
int  moe_cache_lookup(const moe_cache* c, int layer, int expert, int64_t* slot);
int  moe_cache_stats(const moe_cache* c, int64_t* hits, int64_t* misses, int64_t* evictions);
int  moe_cache_class_of(const moe_cache* c, int layer);

/*
 * Cache introspection and repair.
 * moe_cache_shape: number of classes, layers and experts per layer (any may be NULL).
 * moe_cache_class_desc: copy of class `cls`'s descriptor.
 * moe_cache_class_stats: hits, misses, evictions of one class since creation;
 *   the per-class hit rate the size-class design reports ([CLASS] PR description:
 *   the hit rate is given per class, since each class evicts on its own).
 * moe_cache_abort_fill: drop an entry whose fill failed: it becomes absent and its
 *   slot empty at the LRU's back.  MOE_E_BUSY while the entry is pinned.
 */
int  moe_cache_shape(const moe_cache* c, int* n_classes, int* n_layers, int* E);
int  moe_cache_class_desc(const moe_cache* c, int cls, moe_size_class_desc* d);
int  moe_cache_class_stats(const moe_cache* c, int cls, int64_t* hits, int64_t* misses,
                           int64_t* evictions);
int  moe_cache_abort_fill(moe_cache* c, int layer, int expert);

/*
 * Expert store: where experts live when no cache holds them.  One contiguous row
 * per (layer, expert) in the slot byte format, layer-major: the row of (l, e)
 * starts at base(l) + e * slot_bytes(class(l)), base(l) = sum over l' < l of
 * E * slot_bytes(class(l')).  Sources: [RFC] "How the prototype works", Quantized
 * experts bullet (an offline conversion stores each expert as a single unbroken
 * row) and Reads bullet (a miss is one read of that row); [HF-PR] commit message
 * (one open file per shard serves every read).
 *
 * moe_store_open_file: a file at `path`, opened once read-only; every reader
 *   shares the descriptor (positioned reads).  It must hold at least
 *   moe_store_bytes() bytes.  NULL on error (MOE_E_IO: cannot open / too short).
 * moe_store_open_memory: `bytes` of caller-owned host memory at `mem` stand in
 *   for the file (kept by the caller until moe_store_close).
 * moe_store_read: synchronous read of one row into host memory `dst`.
 * moe_store_row_offset: byte offset of a row, -1 on bad arguments.
 */
typedef struct moe_store moe_store;
moe_store* moe_store_open_file(const char* path, const moe_size_class_desc* classes, int n_classes,
                               const int32_t* layer_class, int n_layers, int E);
moe_store* moe_store_open_memory(const void* mem, int64_t bytes, const moe_size_class_desc* classes,
                                 int n_classes, const int32_t* layer_class, int n_layers, int E);
void    moe_store_close(moe_store* s);
int64_t moe_store_bytes(const moe_store* s);
int64_t moe_store_row_offset(const moe_store* s, int layer, int expert);
int     moe_store_read(const moe_store* s, int layer, int expert, void* dst);

/*
 * Miss pipeline: fills a moe_cache's device pools from a moe_store, through an
 * optional pinned-host copy of expert rows.
 * Sources: [RFC] "How the prototype works", Reads bullet (the routing of a
 * layer travels to the host once; worker threads fetch each missing expert
 * with one read into a reused pinned staging buffer, then one asynchronous copy
 * moves it to the device; predicted experts of later layers are fetched ahead)
 * and Host tier bullet (a pinned host level under the device cache turns a
 * device miss into just a host-to-device copy; it can be filled at load time);
 * [HF-PR] host-tier commit message (a host row is not reused before the copy
 * reading it has finished) and mps_commit commit message (a predicted read that
 * has not landed is bypassed rather than awaited); [RFC] Cache bullet (a fully
 * resident model never makes a layer wait on the host); [CLASS] PR description
 * (each layer gets an equal fraction of its experts).
 *
 * moe_pipeline_config:
 *   host_tier_bytes  pinned host bytes for expert rows (0 = no host tier), split
 *                    between classes in proportion to the bytes of all their
 *                    experts; one LRU of rows per class.
 *   host_preload     nonzero: fill the host tier from the store at creation
 *                    (layers ascending, experts ascending, until each class's rows
 *                    are full).
 *   io_threads       store readers, 1..64.
 *   staging_rows     reused pinned staging buffers (largest row each) for store reads
 *                    that do not land in a host row; io_threads..1024.
 *
 * moe_pipeline_create: `class_pools[c]` is class c's device pool (n_slots rows of
 *   slot_bytes, 256-byte aligned); `copy_streams[0..n_copy_streams)` (1 to 4,
 *   caller-owned, default priority, not the compute stream) carry the install
 *   copies: every copy that reads one host row or staging buffer runs on that
 *   buffer's stream, and rows spread over the streams so copies overlap each
 *   other.  The current device is the pools' device.  The cache and store stay owned by the caller and must outlive the
 *   pipeline; while it exists only the pipeline acquires, fills or pins entries of
 *   that cache.  NULL on error.
 * moe_pipeline_prepare: make the experts `ids[0..n)` (duplicates allowed) of
 *   `layer` resident for a forward about to be enqueued on `compute`.  The
 *   distinct ids are acquired in the reverse of their first appearance (ascending
 *   experts then land in ascending slots, and their host-tier installs merge into
 *   one copy per run of consecutive rows and slots).  Hits are
 *   touched; each miss takes the class's LRU victim, is copied from its host row
 *   (inline) or read from the store on an I/O thread, then copied on the copy
 *   stream after the copy stream has waited for the last forward that read the
 *   victim slot.  Returns once every needed copy is enqueued (store reads done);
 *   never waits for a copy itself: `compute` is made to wait for the install
 *   events, then receives one host-to-device copy of the layer's expert -> slot
 *   table (int32 [E], -1 absent) into the device buffer `table_dev`.  The experts
 *   stay pinned until moe_pipeline_release(layer).  Errors: MOE_E_BUSY (layer
 *   prepared and not released), MOE_E_NO_SLOT (every slot of the class pinned),
 *   MOE_E_IO (store read failed; nothing stays pinned), MOE_E_HIP.
 * moe_pipeline_release: call after the layer's forward has been enqueued on
 *   `compute`: records the event that later installs into these slots wait for,
 *   and unpins the layer's experts.
 * moe_pipeline_prefetch: guessed experts of `layer`: absent ones start installs
 *   in the background without pinning; resident or in-flight ones are skipped.
 *   Never waits.  Returns the number of installs started (>= 0) or an error.
 * moe_pipeline_prefill: one layer of a prefill chunk run pass by pass through the
 *   cache, so the layer's class may hold fewer slots than the chunk hits experts
 *   (at least one pass: min(hit experts, 64)).  `ids_host` is the layer's routing
 *   brought to the host (int32 [T, k], host memory); topk_ids / topk_w are the same
 *   routing on the device; x, out, ws, err_word as moe_experts_forward (ws sized by
 *   moe_forward_workspace_size for the layer's class).  Computes the pass table on
 *   the host (moe_pass_table_host), enqueues moe_prefill_sort, then for each pass:
 *   moe_pipeline_prepare(layer, the pass's hit experts, table_dev), moe_prefill_pass
 *   of that pass on the layer's class pool, moe_pipeline_release(layer); finally
 *   moe_prefill_combine, all on `compute`.  A pass's installs overlap the kernels
 *   of the passes before it whenever their victims are not in use (a class with
 *   two passes' worth of slots).  Returns the number of passes (>= 0) or a status
 *   of the calls it makes.
 * moe_pipeline_drain: wait until every read and copy has finished.
 * moe_pipeline_stats_get: counters of one class (moe_pipeline_stats).
 * moe_pipeline_host_rows: host-tier rows of class `cls` (0 without a host tier).
 * Threads: prepare, release, prefetch, drain and destroy from one thread, and
 * prepare/release always on the same compute stream (else MOE_E_INVALID); the
 * I/O threads are internal.
 */
typedef struct moe_pipeline_config {
    int64_t host_tier_bytes;
    int32_t host_preload;
    int32_t io_threads;
    int32_t staging_rows;
    int32_t reserved0;
} moe_pipeline_config;

typedef struct moe_pipeline_stats {
    int64_t requests;          /* distinct experts asked for by prepare              */
    int64_t hits;              /* resident with the install complete                 */
    int64_t inflight_hits;     /* resident, install still in flight (e.g. a guess)   */
    int64_t host_hits;         /* installs copied from a host-tier row               */
    int64_t store_reads;       /* installs read from the store first                 */
    int64_t prefetches;        /* guesses that started an install                    */
    int64_t prefetch_skipped;  /* guesses resident, in flight, or with no free slot  */
    int64_t bytes_copied;      /* host-to-device install bytes enqueued              */
    int64_t bytes_read;        /* bytes read from the store (preload included)       */
} moe_pipeline_stats;

typedef struct moe_pipeline moe_pipeline;
moe_pipeline* moe_pipeline_create(moe_cache* cache, moe_store* store, void* const* class_pools,
                                  const moe_pipeline_config* cfg, const hipStream_t* copy_streams,
                                  int n_copy_streams);
void    moe_pipeline_destroy(moe_pipeline* p);
int     moe_pipeline_prepare(moe_pipeline* p, int layer, const int32_t* ids, int n,
                             int32_t* table_dev, hipStream_t compute);
int     moe_pipeline_release(moe_pipeline* p, int layer, hipStream_t compute);
int     moe_pipeline_prefetch(moe_pipeline* p, int layer, const int32_t* ids, int n);
int     moe_pipeline_prefill(moe_pipeline* p, int layer, const int32_t* ids_host, const void* x, int T,
                             const int32_t* topk_ids, const float* topk_w, int k, int32_t* table_dev,
                             void* out, void* ws, size_t ws_bytes, uint32_t* err_word,
                             hipStream_t compute);
int     moe_pipeline_drain(moe_pipeline* p);
int     moe_pipeline_stats_get(const moe_pipeline* p, int cls, moe_pipeline_stats* out);
int64_t moe_pipeline_host_rows(const moe_pipeline* p, int cls);

/* Thread-local message for the last failing call on this thread. */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
