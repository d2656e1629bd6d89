/*
 * moe_w4a16.h - C ABI of the grouped NVFP4 W4A16 routed-MoE prefill library (gfx950).
 *
 * The library runs the data-parallel hot path of one routed MoE layer at prefill:
 *
 *   moe_align               top-k expert ids -> expert-sorted slot order (counting sort)
 *   moe_w4a16_grouped_gemm  one launch over all experts: gathered BF16 rows x NVFP4 weights
 *   swiglu_clamp            silu(min(gate, L)) * clamp(up, -L, L)
 *   moe_combine             top-k weighted sum of the expert-sorted rows per token
 *   moe_zero_rows           the zero-first step on expert_out (absent experts add zero)
 *   moe_align_zero          moe_align and moe_zero_rows in one launch
 *   moe_w4a16_grouped_gemm_swiglu  the gate_up grouped GEMM with swiglu_clamp fused into
 *                           its epilogue (same bits as the two calls in sequence)
 *   moe_router_topk         router logits -> top-k expert ids and weights (feeds moe_align
 *                           and moe_combine)
 *   moe_dense_gate_up_swiglu_bf16, moe_dense_gemm_bf16
 *                           the shared expert (a BF16 SwiGLU MLP over all rows), whose
 *                           output is moe_combine's `shared` term
 *   moe_dense_gemm_bf16_partials, moe_combine_partials
 *                           the shared expert's down projection left as split-K partial
 *                           sums, reduced inside the combine (same bits, one launch less)
 *   moe_row_union, moe_w4a16_gemv_union, moe_w4a16_gemv_union_swiglu
 *                           the decode / verify path for a few rows: the union of the
 *                           rows' experts (no sort) and one sweep of each union expert,
 *                           outputs laid out by (row, slot)
 *
 * Sources (the pages this library follows, by title and section):
 *   [FPG]  "Module forward_prefill_gemm" (glm5next_mlp/forward_prefill_gemm), sections
 *          "What this replaces", "Layout compatibility - VERIFIED, not assumed" (the
 *          layout table), "What is NOT bit-identical" (item 2: the BF16 weight operand)
 *          and "Buffer discipline".
 *   [FWD]  "glm5next_mlp/forward.rs" (the 2026-09-25 metrale_model_arch page): the
 *          Glm5NextMlpWorkspace field docs (sorted_token_ids, sorted_expert_ids,
 *          expert_offsets, token_to_perm, expert_out), swiglu_rows, and forward_moe's
 *          zero-first memset and glm5next_moe_combine_indexed launch; forward_dense and
 *          the gemm helper above it (C = A B^T, BF16 in and out) for the shared expert.
 *          For the decode path: the workspace fields u_eid and u_slot, the doc of the
 *          row-batched GEMV (C[rows, top_k, N], each union expert swept once) and of
 *          moe_row_groups (which rows share a sweep never changes what a row adds).
 *
 * Conventions shared by every call:
 *   - Every pointer argument is a DEVICE pointer unless stated otherwise. The caller
 *     allocates and owns every buffer; the library never allocates, frees, synchronises
 *     or reads device memory from the host ([FPG] "Buffer discipline": nothing on the
 *     path allocates). There is no host<->device traffic inside any call.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream). Each call
 *     only enqueues kernels on it and returns (no allocation, no synchronisation, no
 *     memset or copy nodes), so calls may be captured into a HIP graph and replayed; the
 *     first call of some entry points sets a kernel attribute once per process, so make
 *     one call of each outside the capture first.
 *   - BF16 tensors are passed as uint16_t bit patterns. Matrices are row-major with the
 *     given leading dimension in ELEMENTS.
 *   - Return value: 0 (MOE_OK) or a moe_status code. On error nothing was enqueued and
 *     moe_w4a16_last_error() describes the failure (per calling thread).
 *   - Data that only the device can see (ids, offsets, gather indices) is bounds-checked
 *     in the kernels: out-of-range values are skipped as documented per call, never
 *     dereferenced.
 */
#ifndef MOE_W4A16_H
#define MOE_W4A16_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum moe_status {
  MOE_OK = 0,
  MOE_EINVAL = 1,    /* bad argument: NULL required pointer, bad size, misalignment */
  MOE_ECAPACITY = 2, /* an output buffer is smaller than the work needs */
  MOE_ELAUNCH = 3    /* the HIP runtime refused the kernel launch */
} moe_status;

/* Static description of a status code. Never NULL. */
const char *moe_w4a16_status_string(int status);

/* Message for the last non-zero status returned on this thread ("" if none). */
const char *moe_w4a16_last_error(void);

/* SHA-256 (64 lowercase hex digits) of the sources this library was compiled from: every
 * csrc/ source and header and this file, hashed by name and content at build time. A
 * loader compares it with the same hash of the sources on disk to refuse a library built
 * from other sources. Never NULL; a static string owned by the library. */
const char *moe_w4a16_source_sha256(void);

/* Largest expert count moe_align accepts (one workgroup holds the histograms). */
#define MOE_ALIGN_MAX_EXPERTS 2048

/* Limits of moe_router_topk (one wave per row holds the row's logits in registers). */
#define MOE_ROUTER_MAX_EXPERTS 2048
#define MOE_ROUTER_MAX_TOPK 64

/*
 * moe_router_topk - top-k expert selection per row ([FWD] forward_moe, the router launch:
 * FP32 logits, optional per-expert bias, top_k, n_group 1, routed_scale, renormalize).
 * The pages do not print the kernel's arithmetic; this is the reading the library takes:
 *
 *   scores[e] = softmax(logits[r, :])[e]                                  (FP32)
 *   key[e]    = scores[e] + bias[e] if bias != NULL, else logits[r, e]
 *   topk_ids[r, j], j = 0..top_k-1: the top_k largest keys, descending; equal keys go
 *               to the lower expert id
 *   topk_weights[r, j] = scores[id] / (renormalize ? sum of the selected scores : 1)
 *                        * routed_scale
 *
 * Without a bias the selection is the top_k logits (softmax is increasing): the same
 * experts as the top_k scores, without ties made by rounding. The bias shifts only the
 * selection, never the weights. If top_k > num_experts the extra slots are -1 with
 * weight 0 (moe_align excludes them). Logits must be finite.
 *
 *   logits        float [rows, ld_logits]   in
 *   bias          float [num_experts] or NULL
 *   topk_ids      int32 [rows * top_k]      out (row-major, slot j of row r at r*top_k+j)
 *   topk_weights  float [rows * top_k]      out
 * Requirements (else MOE_EINVAL): rows >= 0; 1 <= num_experts <= MOE_ROUTER_MAX_EXPERTS;
 * 1 <= top_k <= MOE_ROUTER_MAX_TOPK; ld_logits >= num_experts; routed_scale finite;
 * logits, topk_ids and topk_weights non-NULL when rows > 0. rows == 0 enqueues nothing.
 */
int moe_router_topk(const float *logits, int64_t ld_logits, int32_t rows, int32_t num_experts,
                    const float *bias, int32_t top_k, float routed_scale, int32_t renormalize,
                    int32_t *topk_ids, float *topk_weights, void *stream);

/*
 * moe_align - sort the routed slots by expert ([FWD] Glm5NextMlpWorkspace field docs).
 *
 * Slot t = r * top_k + j carries expert id topk_ids[t]. A slot is valid when its id is
 * in [0, num_experts); -1 (an unfilled router slot) and every other out-of-range id are
 * excluded from the sort. The sort is a stable counting sort: inside an expert's
 * segment, slots keep ascending t (hence ascending token).
 *
 *   topk_ids           int32 [rows * top_k]       in
 *   sorted_token_ids   int32 [rows * top_k]       out: sorted row p -> token row t / top_k
 *   sorted_expert_ids  int32 [rows * top_k]       out: sorted row p -> expert id
 *   expert_offsets     int32 [num_experts + 1]    out: exclusive prefix sum of the per-expert
 *                                                 slot counts; [num_experts] = valid slots
 *   token_to_perm      int32 [rows * top_k]       out: slot t -> its sorted row, -1 if invalid
 *   active_experts     int32 [num_experts] or NULL  out: experts with a non-zero count,
 *                                                 ascending, then -1 padding
 *   counters           int32 [2] or NULL          out: {number of active experts,
 *                                                 number of invalid slots}
 *
 * Sorted rows [expert_offsets[num_experts], rows * top_k) of the two sorted arrays are
 * set to -1. rows == 0 is allowed (offsets and counters become 0).
 * Errors: MOE_EINVAL if rows < 0, top_k < 1, num_experts < 1, num_experts >
 * MOE_ALIGN_MAX_EXPERTS, or a required pointer is NULL while rows * top_k > 0.
 */
int moe_align(const int32_t *topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
              int32_t *sorted_token_ids, int32_t *sorted_expert_ids, int32_t *expert_offsets,
              int32_t *token_to_perm, int32_t *active_experts, int32_t *counters,
              void *stream);

/*
 * moe_align_zero - moe_align and moe_zero_rows(zero, ld_zero, rows * top_k, zero_cols) in
 * one launch: forward_moe's routing sort and its zero-first step on expert_out ([FWD]
 * forward_moe). The zeroing runs in workgroups of its own beside the sort, so a layer whose
 * down table has absent experts pays one launch for the two steps. Outputs are those of
 * the two calls.
 *
 *   zero  bf16 [rows * top_k, ld_zero] or NULL (NULL or zero_cols == 0: moe_align alone)
 *
 * Errors: those of moe_align; MOE_EINVAL unless zero_cols >= 0 and zero_cols % 8 == 0,
 * ld_zero >= zero_cols and a multiple of 8, and zero non-NULL and 16-byte aligned when
 * rows * top_k * zero_cols > 0.
 */
int moe_align_zero(const int32_t *topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                   int32_t *sorted_token_ids, int32_t *sorted_expert_ids,
                   int32_t *expert_offsets, int32_t *token_to_perm, int32_t *active_experts,
                   int32_t *counters, uint16_t *zero, int64_t ld_zero, int32_t zero_cols,
                   void *stream);

/*
 * moe_w4a16_grouped_gemm - one launch over all experts ([FPG] "What this replaces" and
 * the layout table).
 *
 * For every expert e whose packed_ptrs[e] is non-zero and every sorted row s in
 * [expert_offsets[e], expert_offsets[e+1]) (clipped to [0, max_rows)):
 *
 *   c[s, n] = bf16( sum_k a[g(s), k] * W_e[n, k] )      n in [0, n), k in [0, k)
 *   g(s)    = a_gather ? a_gather[s] : s
 *
 * W_e is expert e's NVFP4 weight, N-major:
 *   packed_ptrs[e] -> uint8 [n, k/2]: byte of logical k in row n is n*(k/2) + k/2;
 *                     even k is the low nibble, odd k the high nibble.
 *   scale_ptrs[e]  -> uint8 [n, k/16]: E4M3 (OCP FN) block scale of k/16 in row n.
 *   scale2[e]      -> float: the expert's second-level scale.
 * Each weight is decoded through the E2M1 codebook (values 0, .5, 1, 1.5, 2, 3, 4, 6;
 * nibble bit 3 is the sign) and rounded to the BF16 operand the matrix cores take:
 *   W_e[n, k] = bf16_rne( fp32( fp32(e2m1(q) * e4m3(scale)) * scale2[e] ) )
 * ([FPG] "What is NOT bit-identical", item 2). Products accumulate in FP32.
 *
 *   a               bf16  [a_rows, lda]  activations (row g(s) is read)
 *   a_gather        int32 [max_rows] or NULL. An index outside [0, a_rows) reads a row
 *                   of zeros.
 *   packed_ptrs     uint64 [num_experts] device addresses (0 = expert not present here:
 *                   its rows of c are not written, the caller's values stand, [FPG]
 *                   layout table row "remote expert (EP)").
 *   scale_ptrs      uint64 [num_experts] device addresses (non-zero where packed is).
 *   scale2          float  [num_experts]
 *   expert_offsets  int32  [num_experts + 1] as written by moe_align: non-decreasing (a
 *                   prefix sum). Other values are not checked (device data); each row the
 *                   call writes still lies in [0, max_rows), but rows may then be missed.
 *   active_experts, counters
 *                   NULL, or moe_align's active_experts [num_experts] and counters [2]
 *                   for the same ids (the experts with rows, in order, and their count in
 *                   counters[0]). When both are given and max_rows < num_experts, the
 *                   launch visits only the listed experts (no block for an expert without
 *                   rows); the results are the same. Grid row i takes entry i, for i <
 *                   min(counters[0], max_rows): moe_align's ascending order guarantees
 *                   that an entry past max_rows has no row below max_rows. Entries outside
 *                   [0, num_experts) are skipped; a list that leaves out an expert with
 *                   rows leaves its rows unwritten (device data: not checked).
 *   c               bf16   [max_rows, ldc] output rows in expert-sorted order
 *
 * Requirements (else MOE_EINVAL): n > 0 and n % 16 == 0; k > 0 and k % 256 == 0;
 * lda >= k and ldc >= n, both multiples of 8; a and c 16-byte aligned;
 * 1 <= num_experts <= 65535;
 * max_rows >= 0; a_rows >= 1 when max_rows > 0; a, packed_ptrs, scale_ptrs, scale2,
 * expert_offsets and c non-NULL; the activation buffer and one expert's packed weights
 * below 2 GiB. Each table address must be 16-byte aligned (not checked: device data).
 * max_rows == 0 enqueues nothing.
 */
int moe_w4a16_grouped_gemm(const uint16_t *a, int64_t lda, int32_t a_rows,
                           const int32_t *a_gather, const uint64_t *packed_ptrs,
                           const uint64_t *scale_ptrs, const float *scale2,
                           const int32_t *expert_offsets, int32_t num_experts,
                           const int32_t *active_experts, const int32_t *counters, uint16_t *c,
                           int64_t ldc, int32_t max_rows, int32_t n, int32_t k, void *stream);

/*
 * moe_w4a16_grouped_gemm_swiglu - moe_w4a16_grouped_gemm over a fused gate_up weight
 * (n = 2 * mi rows: gate rows [0, mi), up rows [mi, 2 mi), the [FPG] fused gate_up
 * layout) followed by swiglu_clamp, in one launch:
 *
 *   act[s, j] = bf16( swiglu(G, U) ),   j in [0, mi)
 *   G = bf16(sum_k a[g(s), k] W_e[j, k]),   U = bf16(sum_k a[g(s), k] W_e[mi + j, k])
 *   swiglu(G, U) = silu(min(G, limit)) * clamp(U, -limit, limit) in FP32, as swiglu_clamp
 *
 * The result is bit-identical to moe_w4a16_grouped_gemm into a [max_rows, 2 mi] buffer
 * followed by swiglu_clamp on its two halves; the gate_up values are never stored. Rows,
 * gathers, null entries, expert_offsets and the active-expert list behave as in
 * moe_w4a16_grouped_gemm (rows of a null expert are not written).
 *
 *   act      bf16 [max_rows, ld_act]  output
 *   tables   packed_ptrs[e] -> uint8 [2 mi, k/2], scale_ptrs[e] -> uint8 [2 mi, k/16]
 *
 * Requirements (else MOE_EINVAL): mi > 0 and mi % 16 == 0; limit > 0; ld_act >= mi; the
 * other requirements of moe_w4a16_grouped_gemm with n = 2 mi and c = act.
 * Fusing the activation into the producing GEMM removes the gate_up buffer's write and
 * read and one launch.
 */
int moe_w4a16_grouped_gemm_swiglu(const uint16_t *a, int64_t lda, int32_t a_rows,
                                  const int32_t *a_gather, const uint64_t *packed_ptrs,
                                  const uint64_t *scale_ptrs, const float *scale2,
                                  const int32_t *expert_offsets, int32_t num_experts,
                                  const int32_t *active_experts, const int32_t *counters,
                                  uint16_t *act, int64_t ld_act, int32_t max_rows, int32_t mi,
                                  int32_t k, float limit, void *stream);

/*
 * swiglu_clamp - out[r, j] = bf16( silu(min(gate[r, j], limit)) * clamp(up[r, j], -limit,
 * limit) ), silu(x) = x / (1 + exp(-x)), computed in FP32 ([FWD] swiglu_rows). The gate is
 * clamped from above only.
 *
 *   gate, up  bf16 [rows, ld_in] (for a fused gate_up buffer: up = gate + n)
 *   out       bf16 [rows, ld_out]
 * Requirements (else MOE_EINVAL): rows >= 0, n >= 0, n % 8 == 0, ld_in >= n and
 * ld_out >= n multiples of 8, pointers 16-byte aligned and non-NULL when rows * n > 0,
 * limit > 0.
 */
int swiglu_clamp(const uint16_t *gate, const uint16_t *up, int64_t ld_in, uint16_t *out,
                 int64_t ld_out, int32_t rows, int32_t n, float limit, void *stream);

/*
 * moe_combine - out[r, h] = bf16( sum_{j < top_k} w[r, j] * expert_out[p, h] + shared[r, h] )
 * with p = token_to_perm[r * top_k + j], summed in FP32 in slot order j = 0..top_k-1,
 * the shared term added last ([FWD] forward_moe, glm5next_moe_combine_indexed). Slots
 * with p outside [0, expert_rows) are skipped (an excluded slot adds zero).
 *
 *   expert_out     bf16  [expert_rows, ld_e]  expert-sorted rows
 *   token_to_perm  int32 [rows * top_k]
 *   topk_weights   float [rows * top_k]
 *   shared         bf16  [rows, ld_s] or NULL (no shared-expert term)
 *   out            bf16  [rows, ld_out]
 * Requirements (else MOE_EINVAL): rows >= 0, hidden >= 0, hidden % 8 == 0, top_k >= 1,
 * expert_rows >= 0, leading dimensions >= hidden and multiples of 8, pointers 16-byte
 * aligned and non-NULL (shared excepted) when rows * hidden > 0.
 */
int moe_combine(const uint16_t *expert_out, int64_t ld_e, int32_t expert_rows,
                const int32_t *token_to_perm, const float *topk_weights,
                const uint16_t *shared, int64_t ld_s, uint16_t *out, int64_t ld_out,
                int32_t rows, int32_t hidden, int32_t top_k, void *stream);

/*
 * moe_combine_partials - moe_combine with the shared term taken from the shared expert's
 * down projection in its split-K partial form (moe_dense_gemm_bf16_partials) instead of
 * its BF16 output: shared[r, h] = bf16( sum_{s < ways} shared_partials[s, r, h] ), summed
 * in FP32 in split order and rounded as moe_dense_gemm_bf16 rounds its output, so the
 * result has the bits of moe_dense_gemm_bf16 (split-K form) followed by moe_combine. The
 * down projection's split-K reduction runs inside the combine ([FWD] forward_moe adds
 * the shared expert's output in this launch), which saves that reduction's launch.
 *
 *   shared_partials  float [ways, rows, hidden], contiguous (hidden fastest)
 *   ways             the split count the partials were written with, in [1, 64]
 *   partials_bytes   the size of shared_partials in bytes
 *   the other arguments as moe_combine (no shared, ld_s).
 * Requirements (else MOE_EINVAL / MOE_ECAPACITY): those of moe_combine; 1 <= ways <= 64;
 * shared_partials non-NULL and 16-byte aligned when rows * hidden > 0; partials_bytes >=
 * ways * rows * hidden * 4 (MOE_ECAPACITY, nothing enqueued).
 */
int moe_combine_partials(const uint16_t *expert_out, int64_t ld_e, int32_t expert_rows,
                         const int32_t *token_to_perm, const float *topk_weights,
                         const float *shared_partials, int32_t ways, int64_t partials_bytes,
                         uint16_t *out, int64_t ld_out, int32_t rows, int32_t hidden,
                         int32_t top_k, void *stream);

/*
 * moe_zero_rows - c[r, j] = 0 for r < rows, j < cols: forward_moe's zero-first step on
 * expert_out ([FWD] forward_moe), so that the rows of experts absent from the table
 * (never written by the down GEMM) add zero in moe_combine. A kernel, not a memset, so
 * that it may sit in a captured graph.
 *
 *   c  bf16 [rows, ldc]
 * Requirements (else MOE_EINVAL): rows >= 0; cols >= 0 and cols % 8 == 0; ldc >= cols and
 * a multiple of 8; c non-NULL and 16-byte aligned when rows * cols > 0.
 */
int moe_zero_rows(uint16_t *c, int64_t ldc, int32_t rows, int32_t cols, void *stream);

/*
 * moe_dense_gemm_bf16 - c[m, n] = bf16( sum_k a[m, k] * b[n, k] ), FP32 accumulation: the
 * pages' BF16 gemm (C[M, N] = A[M, K] B[N, K]^T) as forward_dense uses it for the shared
 * expert's down projection ([FWD] forward_dense).
 *
 *   a          bf16 [m, lda]   rows (tokens)
 *   b          bf16 [n, ldb]   weight rows, K contiguous
 *   c          bf16 [m, ldc]   output
 *   workspace  NULL, or device memory of at least moe_dense_workspace_bytes(m, n, k, 0)
 *              bytes, 256-byte aligned (no initial contents needed). With it the GEMM
 *              runs split over K with 128 x 128 tiles in two launches (FP32 partial tiles
 *              into the workspace, then a reduction in split order): fewer bytes through
 *              each CU's cache at the prefill shapes. Calls that share a workspace must not
 *              run concurrently (stream-ordered calls may share one). Without it, a single
 *              pass with 64 x 64 tiles. The two forms sum in different orders: each is
 *              deterministic, their bits differ.
 * Requirements (else MOE_EINVAL): m, n, k >= 0; n % 16 == 0; k % 64 == 0; lda >= k and
 * ldb >= k, multiples of 8 and at most 2^23; ldc >= n, a multiple of 4; c 8-byte aligned
 * and non-NULL when m * n > 0; a and b 16-byte aligned and non-NULL when also k > 0; a
 * workspace 256-byte aligned. MOE_ECAPACITY if workspace_bytes is below what the
 * split-K form needs. m == 0 or n == 0 enqueues nothing; k == 0 writes zeros (a and b
 * are not read).
 */
int moe_dense_gemm_bf16(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                        uint16_t *c, int64_t ldc, int32_t m, int32_t n, int32_t k,
                        void *workspace, int64_t workspace_bytes, void *stream);

/*
 * moe_dense_gemm_bf16_noalloc - moe_dense_gemm_bf16 in its split-K form without a
 * workspace argument, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation). The FP32 partial
 * tiles go to the library's own device array of MOE_DENSE_NOALLOC_SCRATCH_BYTES, one copy
 * per GPU, held from the library's load until the process ends. No call allocates or frees
 * anything; the first call on a device looks the array's address up (make it outside any
 * graph capture).
 *
 *   a, b, c, sizes, strides: as moe_dense_gemm_bf16. Same bits as moe_dense_gemm_bf16 with
 *   a workspace (the same kernels, split and order).
 * Every call on one GPU shares that GPU's array, which keeps the last call's contents (no
 * call needs it cleared). Calls that overlap on one GPU (concurrent streams, or other
 * host threads enqueuing at the same time) race on it: order them on one stream.
 * Errors: as moe_dense_gemm_bf16; MOE_ECAPACITY (nothing enqueued) when the split-K
 * partials of m x n at this k, moe_dense_workspace_bytes(m, n, k, 0), exceed
 * MOE_DENSE_NOALLOC_SCRATCH_BYTES (32 MiB: the shared expert's down projection at 256
 * rows of hidden 6144 needs 25.2 MB); MOE_ELAUNCH if the array's address lookup fails.
 */
#define MOE_DENSE_NOALLOC_SCRATCH_BYTES (32ll << 20)
int moe_dense_gemm_bf16_noalloc(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                                uint16_t *c, int64_t ldc, int32_t m, int32_t n, int32_t k,
                                void *stream);

/*
 * moe_dense_workspace_bytes - host-side size query: the workspace bytes the split-K form
 * of moe_dense_gemm_bf16 (swiglu = 0, n = output width) or of
 * moe_dense_gate_up_swiglu_bf16 (swiglu = 1, n = inter) needs for these sizes: an FP32
 * partial tile (128 x 128) per 128-row x 128-weight-row tile and K split (K splits 4, 2
 * or 1 ways: the most that divide the 64-k steps evenly with at least 8 per split and per
 * 128-row tile, and at most 8 / ceil(m / 128) ways).
 * Returns 0 when m <= 0, n <= 0 or k < 0. Enqueues nothing.
 */
int64_t moe_dense_workspace_bytes(int32_t m, int32_t n, int32_t k, int32_t swiglu);

/*
 * moe_dense_splitk_ways - host-side query: the number of K splits the split-K form uses
 * for m rows at this k (the count in moe_dense_workspace_bytes). Returns 1 when m <= 0,
 * k <= 0 or k is not a multiple of 64. Enqueues nothing.
 */
int32_t moe_dense_splitk_ways(int32_t m, int32_t k);

/*
 * moe_dense_gemm_bf16_partials - the first launch of moe_dense_gemm_bf16's split-K form
 * alone, its FP32 partial sums written row-major for moe_combine_partials:
 *
 *   partials[s, i, j] = sum over split s's K range of a[i, k] * b[j, k]   (FP32)
 *
 * with ways = moe_dense_splitk_ways(m, k) splits of equal length in K order. The
 * per-element values are the ones moe_dense_gemm_bf16's split-K reduction sums.
 *
 *   a, b, sizes, strides  as moe_dense_gemm_bf16 (n = output width)
 *   partials              float [ways, m, n], contiguous; partials_bytes its size in bytes
 * Requirements (else MOE_EINVAL / MOE_ECAPACITY): those of moe_dense_gemm_bf16 with c =
 * partials and ldc = n; partials 16-byte aligned; partials_bytes >= ways * m * n * 4
 * (MOE_ECAPACITY, nothing enqueued).
 */
int moe_dense_gemm_bf16_partials(const uint16_t *a, int64_t lda, const uint16_t *b, int64_t ldb,
                                 float *partials, int32_t m, int32_t n, int32_t k,
                                 int64_t partials_bytes, void *stream);

/*
 * moe_dense_gate_up_swiglu_bf16 - the gate and up projections of forward_dense and its
 * SwiGLU in one launch ([FWD] forward_dense, swiglu_rows):
 *
 *   act[m, j] = bf16( swiglu(G, U) ),   j in [0, inter)
 *   G = bf16(sum_k a[m, k] gate_w[j, k]),   U = bf16(sum_k a[m, k] up_w[j, k])
 *   swiglu(G, U) = silu(min(G, limit)) * clamp(U, -limit, limit) in FP32, as swiglu_clamp
 *
 * Bit-identical to moe_dense_gemm_bf16 with gate_w and with up_w followed by
 * swiglu_clamp; G and U are never stored.
 *
 *   a               bf16 [m, lda]
 *   gate_w, up_w    bf16 [inter, ldw] each
 *   act             bf16 [m, ld_act]
 *   workspace       as for moe_dense_gemm_bf16, sized by
 *                   moe_dense_workspace_bytes(m, inter, k, 1). The bit identity above holds
 *                   between calls of the same form (both with a workspace, or both
 *                   without).
 * Requirements (else MOE_EINVAL / MOE_ECAPACITY): limit > 0; inter % 16 == 0; the
 * requirements of moe_dense_gemm_bf16 with n = inter, b = gate_w and up_w, c = act.
 */
int moe_dense_gate_up_swiglu_bf16(const uint16_t *a, int64_t lda, const uint16_t *gate_w,
                                  const uint16_t *up_w, int64_t ldw, uint16_t *act,
                                  int64_t ld_act, int32_t m, int32_t inter, int32_t k,
                                  float limit, void *workspace, int64_t workspace_bytes,
                                  void *stream);

/*
 * moe_w4a16_dequant_bf16 - diagnostic: write the BF16 weight operand the grouped GEMM
 * feeds its matrix cores, out[n, k] = W[n, k] as defined for moe_w4a16_grouped_gemm,
 * through the same device decoder. Lets the decode be checked bit for bit.
 *
 *   packed  uint8 [n, k/2];  scales  uint8 [n, k/16];  out  bf16 [n, k]
 * Requirements (else MOE_EINVAL): n > 0, k > 0, k % 32 == 0, pointers non-NULL and
 * 16-byte aligned.
 */
int moe_w4a16_dequant_bf16(const uint8_t *packed, const uint8_t *scales, float scale2,
                           uint16_t *out, int32_t n, int32_t k, void *stream);

/*
 * moe_hbm_read_probe - diagnostic: stream `bytes` of device memory at `buf` and do nothing
 * else. It measures the practical HBM read ceiling that the weight-streaming kernels are
 * judged against ([FPG] "What this replaces" judges a kernel by its own DRAM roofline),
 * and a run over a buffer several times the last-level cache evicts that cache between
 * timed iterations. Each wave reads 1 KB per instruction with `unroll` instructions in
 * flight; `blocks` workgroups of 256 threads stride over the buffer.
 *
 *   buf   device, 16-byte aligned, `bytes` readable (contents are irrelevant)
 *   sink  device uint32 [blocks]: overwritten with meaningless values (the loads feed it)
 * Requirements (else MOE_EINVAL): non-NULL pointers, bytes > 0 and % 16 == 0,
 * 1 <= blocks <= 2^20, unroll in {4, 8, 16}.
 */
int moe_hbm_read_probe(const void *buf, int64_t bytes, uint32_t *sink, int32_t blocks,
                       int32_t unroll, void *stream);

/* Limits of the decode / verify path. */
#define MOE_UNION_MAX_IDS 1024 /* rows * top_k of moe_row_union (one workgroup) */
#define MOE_UNION_MAX_ROWS 16  /* rows of moe_w4a16_gemv_union (one matrix-core tile) */
#define MOE_UNION_GEMV_MAX_IDS 512 /* rows * top_k of moe_w4a16_gemv_union */

/*
 * moe_row_union - the union of the experts a few rows selected ([FWD] workspace fields
 * u_eid, u_slot; the union is found in one workgroup, without a sort).
 *
 * Slot t = r * top_k + j is covered when topk_ids[t] is in [0, num_experts), the expert
 * is present (below) and no lower slot of row r holds the same id (a proper top-k never
 * repeats an expert in a row; a repeat is treated like an invalid id).
 *
 *   topk_ids   int32 [rows * top_k]          in
 *   present    uint64 [num_experts] or NULL  in: with it, an expert whose entry is 0 (a
 *                                            null table entry, e.g. a projection's
 *                                            packed_ptrs) is treated like an invalid id:
 *                                            its slots are not covered and open no entry.
 *                                            The combine then skips them, so the rows of
 *                                            absent experts need no zeroing.
 *   u_eid      int32 [rows * top_k]          out: the distinct ids of the covered slots in
 *                                            order of first appearance in t, then -1
 *   u_slot     int32 [rows * top_k, rows]    out: u_slot[p, r] = j when row r's slot j is
 *                                            covered and selects u_eid[p], else -1
 *   slot_perm  int32 [rows * top_k] or NULL  out: t for a covered slot, else -1 (the
 *                                            combine's token_to_perm for outputs laid out
 *                                            [rows * top_k, n] by slot)
 *   counters   int32 [2] or NULL             out: {union size, uncovered slots}
 *
 * rows == 0 enqueues nothing. Errors: MOE_EINVAL if rows < 0, top_k < 1, num_experts < 1,
 * rows * top_k > MOE_UNION_MAX_IDS, or a required pointer is NULL while rows > 0.
 */
int moe_row_union(const int32_t *topk_ids, int32_t rows, int32_t top_k, int32_t num_experts,
                  const uint64_t *present, int32_t *u_eid, int32_t *u_slot,
                  int32_t *slot_perm, int32_t *counters, void *stream);

/*
 * moe_w4a16_gemv_union - the W4A16 product of each union expert's rows, each expert's
 * weights swept once ([FWD] the row-batched GEMV: C[rows, top_k, N] over the union).
 *
 * For every entry p with e = u_eid[p] in [0, num_experts) and packed_ptrs[e] != 0, and
 * every row r with j = u_slot[p, r] >= 0:
 *
 *   c[r * top_k + j, n] = bf16( sum_k a[src, k] * W_e[n, k] ),  src = a_per_slot ?
 *                                                          r * top_k + j : r
 *
 * with W_e decoded exactly as in moe_w4a16_grouped_gemm (same tables, same BF16 operand)
 * and FP32 accumulation. The sum's order does not depend on which rows share the sweep.
 * Rows of c that no entry covers, and rows of absent experts, are not written.
 *
 *   a       bf16 [a_rows, lda]: the rows' inputs (a_per_slot = 0: a_rows >= rows) or one
 *           input per slot (a_per_slot != 0: row r * top_k + j). A source row outside
 *           [0, a_rows) reads zeros.
 *   tables  as moe_w4a16_grouped_gemm (packed_ptrs, scale_ptrs, scale2 per global id)
 *   u_eid, u_slot  as written by moe_row_union for the same rows and top_k
 *   c       bf16 [rows * top_k, ldc] output, laid out by (row, slot)
 *
 * Requirements (else MOE_EINVAL): 0 <= rows <= MOE_UNION_MAX_ROWS; top_k >= 1 and
 * rows * top_k <= MOE_UNION_GEMV_MAX_IDS; n > 0, n % 16 == 0; k > 0, k % 256 == 0; lda >= k,
 * a multiple of 8; ldc >= n, a multiple of 4; a 16-byte and c 8-byte aligned;
 * num_experts >= 1; a_rows >= 1; required pointers non-NULL; the activation buffer and one
 * expert's packed weights below 2 GiB. rows == 0 enqueues nothing.
 */
int moe_w4a16_gemv_union(const uint16_t *a, int64_t lda, int32_t a_rows, int32_t a_per_slot,
                         const uint64_t *packed_ptrs, const uint64_t *scale_ptrs,
                         const float *scale2, const int32_t *u_eid, const int32_t *u_slot,
                         int32_t rows, int32_t top_k, int32_t num_experts, uint16_t *c,
                         int64_t ldc, int32_t n, int32_t k, void *stream);

/*
 * moe_w4a16_gemv_union_swiglu - moe_w4a16_gemv_union over a fused gate_up weight (n = 2 mi
 * rows, gate rows [0, mi), up rows [mi, 2 mi)) followed by swiglu_clamp in the epilogue:
 *
 *   act[r * top_k + j, i] = bf16( swiglu(G, U) ),  G = bf16(gate sum of row i),
 *                           U = bf16(up sum of row mi + i)
 *
 * bit-identical to moe_w4a16_gemv_union into a [rows * top_k, 2 mi] buffer followed by
 * swiglu_clamp. Requirements: mi > 0, mi % 16 == 0, limit > 0, ld_act >= mi, and those of
 * moe_w4a16_gemv_union with n = 2 mi.
 */
int moe_w4a16_gemv_union_swiglu(const uint16_t *a, int64_t lda, int32_t a_rows,
                                int32_t a_per_slot, const uint64_t *packed_ptrs,
                                const uint64_t *scale_ptrs, const float *scale2,
                                const int32_t *u_eid, const int32_t *u_slot, int32_t rows,
                                int32_t top_k, int32_t num_experts, uint16_t *act,
                                int64_t ld_act, int32_t mi, int32_t k, float limit,
                                void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_W4A16_H */
