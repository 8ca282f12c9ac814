/*
 * isa.h -- C ABI of the In-context Sparse Attention (ISA) library for
 * AMD Instinct MI355X (gfx950).
 *
 * ISA replaces full attention over a concatenated [source | context]
 * sequence Q, K, V of shape [B, H, N, D] (the first L_src tokens are the
 * source, the last L_ctx tokens the context).  Pages describing it:
 *
 *   [notes]   "Lightning Unified Video Editing via In-Context Sparse
 *             Attention", papernotes.org ICML 2026 notes: overall framework,
 *             key design 1 (Context Pre-Selection), key design 2 (block-wise
 *             0-th order Taylor sparse attention), key design 3 (grouped
 *             computation by query sharpness).
 *   [summary] "LIVEditor-14B: Lightning Unified Video Editing via In-Context
 *             Sparse Attention", paperlayer.ai summary of arXiv 2605.04569v2,
 *             sections 2 (Preliminary) and 3 (In-Context Sparse Attention).
 *
 * Conventions for every entry point:
 *   - Tensors are contiguous row-major [B, H, N, D] with D fastest; device
 *     pointers are 16-byte aligned.  The caller owns every buffer (inputs,
 *     outputs, workspace, aux) and keeps it alive until the stream has
 *     finished the work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Launches are asynchronous: no allocation, no synchronisation and no
 *     device-to-host copy happens inside an entry point.
 *   - Argument errors are detected on the host before the first launch, so
 *     on error nothing has been written.  No entry point aborts or throws.
 *   - Every setting is a plan field or an argument; this header has no global
 *     switches.  (The library's tests use the hooks of isa_testing.h.)
 *   - With the environment variable ISA_LOG set to a non-empty value other
 *     than "0", isa_plan_create prints the derived sizes of each plan it
 *     creates to stderr.
 *   - Supported on the device: block in {32, 64, 128}, D in {64, 128}, any
 *     L_src >= 1 and L_ctx >= 0 (the source and the context are each cut into
 *     b-token blocks from their own start, so the last block of each may be
 *     partial: [notes] key design 1 counts ceil(L_ctx / b) context blocks),
 *     dtype BF16 (fp32 accumulation) or FP32.  The block mask (n_ns > 0 with
 *     flat blocks) needs block = 64; the backward needs block = 64.  Other
 *     valid descriptions return ISA_ERR_UNSUPPORTED.
 */
#ifndef ISA_H
#define ISA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ISA_OK = 0,
  ISA_ERR_INVALID_ARG = 1,  /* a null pointer, a negative size, a ratio outside [0, 1] */
  ISA_ERR_UNSUPPORTED = 2,  /* a valid description this build does not run */
  ISA_ERR_WORKSPACE = 3,    /* workspace pointer null or smaller than workspace_bytes */
  ISA_ERR_HIP = 4           /* a HIP call failed; see isa_last_hip_error() */
} isa_status_t;

typedef enum { ISA_DTYPE_BF16 = 0, ISA_DTYPE_FP32 = 1 } isa_dtype_t;

/* Problem description.  N = L_src + L_ctx. */
typedef struct {
  int32_t B, H;          /* batch size and heads (0 gives an empty problem) */
  int32_t L_src, L_ctx;  /* source tokens (first, >= 1) and context tokens (last, >= 0) */
  int32_t D;             /* head dimension */
  int32_t block;         /* b: tokens per block; query blocks and key blocks share the grid */
  double alpha_s;        /* select ratio: keep ceil(alpha_s * n_ctx) context blocks   */
  double alpha_f;        /* flat ratio: floor(alpha_f * n_q) flattest query blocks go */
                         /* to the 0-th order Taylor path ([notes] key design 3)      */
  double alpha_ns;       /* no-sparsity ratio: inside each flat query block the        */
                         /* ceil(alpha_ns * n_kv) K_new blocks with the largest coarse */
                         /* score are computed exactly ([notes] key design 2 mask)    */
  isa_dtype_t dtype;     /* storage and input type of Q, K, V, O                      */
  double rope_base;      /* > 0: decoupled rotary embedding of Q and K before every  */
                         /* step ([notes] training strategy: source and context      */
                         /* positions each start at 0).  Pair (2i, 2i+1) of a token  */
                         /* at position pos turns by pos * rope_base^(-2i/D)          */
                         /* (RoFormer's rotation); the rotated values are rounded     */
                         /* once, to nearest even, to dtype.  0: no embedding.        */
} isa_plan_desc_t;

typedef struct isa_plan_s* isa_plan_t;

/* Sizes derived from a description (all per (batch, head)). */
typedef struct {
  int64_t n_src_blocks;   /* ceil(L_src / b) */
  int64_t n_ctx_blocks;   /* ceil(L_ctx / b) */
  int64_t n_q_blocks;     /* n_src + n_ctx (query blocks = key blocks) */
  int64_t k;              /* selected context blocks, ceil(alpha_s * n_ctx) */
  int64_t n_kv_blocks;    /* blocks of K_new: n_src + k */
  int64_t l_new;          /* tokens of K_new: L_src + k * b (fewer when the     */
                          /* context's partial last block is among the kept)   */
  int64_t n_flat;         /* query blocks on the Taylor path, floor(alpha_f * n_q) */
  int64_t n_sharp;        /* query blocks on the exact path, n_q - n_flat */
  size_t workspace_bytes; /* device workspace isa_forward needs */
  int64_t n_ns;           /* K_new blocks computed exactly per flat query block, */
                          /* ceil(alpha_ns * n_kv) (0: the plain Taylor path)     */
} isa_plan_info_t;

/* Optional device outputs of isa_forward (each pointer may be NULL). */
typedef struct {
  int32_t* sel;        /* [B, H, k]       selected context blocks, ascending        */
  int32_t* flat;       /* [B, H, n_flat]  query blocks on the Taylor path, ascending */
  int32_t* sharp;      /* [B, H, n_sharp] query blocks on the exact path, ascending  */
  double* ctx_score;   /* [B, H, n_ctx]   c_j, the source-query mean of the coarse   */
                       /*                 map over context block j                   */
  double* sharpness;   /* [B, H, n_q]     M_i, the variance of coarse row i          */
  int32_t* ns;         /* [B, H, n_flat, n_ns] per flat query block (in the order of */
                       /*                 flat) the positions in K_new (0..n_kv-1:   */
                       /*                 source blocks, then the kept context       */
                       /*                 blocks) computed exactly, ascending        */
} isa_aux_t;

/* Validate a description and derive the sizes; host only, never calls HIP.
 * The plan is immutable and may be shared across threads and streams.
 * Errors: ISA_ERR_INVALID_ARG (null out/desc, B/H/D/block < 1 or negative,
 * L_src < 1, L_ctx < 0, a ratio outside [0, 1] or NaN, rope_base negative,
 * infinite or NaN),
 * ISA_ERR_UNSUPPORTED (block not 32/64/128, D not 64/128, the block mask with
 * flat blocks at block != 64, more than 4096 blocks per head). */
isa_status_t isa_plan_create(isa_plan_t* out, const isa_plan_desc_t* desc);

/* Copy the derived sizes into *info.  Host only. */
isa_status_t isa_plan_get_info(isa_plan_t plan, isa_plan_info_t* info);

/* Release a plan (NULL is accepted).  Host only. */
isa_status_t isa_plan_destroy(isa_plan_t plan);

/* The ISA forward pass ([notes] overall framework, steps 1-4 and merge):
 *   1. block-mean pooling of Q, K, V and the coarse map
 *      S_coarse = softmax(Q^c K^c^T / sqrt(D)) (computed in fp64);
 *   2. Context Pre-Selection: c_j = mean over source query blocks of
 *      S_coarse[i, n_src + j]; keep the k blocks with the largest c_j
 *      (ties to the smaller j); K_new = [source ; kept blocks ascending];
 *   3. sharpness M_i = variance of S_coarse row i; the n_flat blocks with
 *      the smallest M_i (ties to the smaller i) are flat;
 *   4. sharp rows: exact softmax(q K_new^T / sqrt(D)) V_new; flat rows:
 *      0-th order Taylor attention against the block means of K_new, V_new
 *      with block-length weights ([notes] key design 2).  With n_ns > 0 the
 *      n_ns K_new blocks of largest coarse score x_ij of flat block i (ties
 *      to the smaller K_new position) enter token by token instead, in the
 *      same softmax;
 *   5. O = O / l (bf16 round-to-nearest-even for BF16), lse = m + ln l.
 * With rope_base > 0, every step sees the rotated Q and K (written into the
 * workspace by the pooling kernel).
 * Q, K, V, O: [B, H, N, D] of `dtype`.  lse: [B, H, N] float, may be NULL.
 * aux: optional decision outputs (see isa_aux_t), may be NULL.
 * workspace: device memory of at least info.workspace_bytes.
 * Errors: ISA_ERR_INVALID_ARG (null plan/Q/K/V/O), ISA_ERR_WORKSPACE,
 * ISA_ERR_HIP (launch failure). */
isa_status_t isa_forward(isa_plan_t plan, const void* Q, const void* K, const void* V,
                         void* O, float* lse, const isa_aux_t* aux,
                         void* workspace, size_t workspace_bytes, void* stream);

/* Number of stages isa_forward_profiled brackets with events:
 * 1 pool, 2 coarse row statistics + sharpness, 3 context column means,
 * 4 TopK + routing, 5 exact path, 6 0-th order Taylor path. */
#define ISA_PROFILE_STAGES 6

/* isa_forward with timing: the same launches on `stream`, plus
 * hipEventRecord(events[0]) before the first stage and events[i] after stage
 * i (i = 1..ISA_PROFILE_STAGES).  events: ISA_PROFILE_STAGES + 1 hipEvent_t
 * handles created by the caller (passed as void*).  The caller reads the stage
 * durations with hipEventElapsedTime after synchronising.  Errors: as
 * isa_forward, plus ISA_ERR_INVALID_ARG for a null events array. */
isa_status_t isa_forward_profiled(isa_plan_t plan, const void* Q, const void* K, const void* V,
                                  void* O, float* lse, const isa_aux_t* aux,
                                  void* workspace, size_t workspace_bytes, void* stream,
                                  void* const* events);

/* Largest plan workspace (info.workspace_bytes) isa_forward_noalloc serves:
 * 128 MiB, e.g. B * H = 40 heads of D = 128 up to N = 65536 without the
 * rotary embedding (whose rotated Q and K live in the workspace). */
#define ISA_STATIC_WORKSPACE_BYTES ((size_t)128 << 20)

/* isa_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same launches as isa_forward, with the workspace taken from an array of
 * ISA_STATIC_WORKSPACE_BYTES that the library holds on each device it runs on
 * (reserved when the library's device code is loaded on that device, kept
 * until the process ends).  No hipMalloc, hipFree or other allocating call;
 * the caller still passes Q, K, V, O, lse and aux as for isa_forward.  The
 * first call on a device resolves the array's address there (on the device of
 * `stream`, or the current device for the NULL stream).
 * Every call on one device shares that device's array, which keeps the last
 * call's contents: calls that overlap on a device (other streams, other
 * threads) race and give wrong results; calls ordered on one stream are safe.
 * Nothing needs clearing between calls: the forward writes every workspace
 * byte before it reads it.
 * Errors: as isa_forward; ISA_ERR_WORKSPACE when info.workspace_bytes exceeds
 * ISA_STATIC_WORKSPACE_BYTES (checked first, on the host); ISA_ERR_HIP when
 * the device or the array's address cannot be resolved. */
isa_status_t isa_forward_noalloc(isa_plan_t plan, const void* Q, const void* K, const void* V,
                                 void* O, float* lse, const isa_aux_t* aux, void* stream);

/* The gather + concat of Context Pre-Selection ([notes] key design 1;
 * [summary] 3 Pre-Selection), materialised: K_new, V_new [B, H, l_new, D] =
 * [all source tokens ; tokens of the context blocks listed in sel, in the
 * order given].  sel: device [B, H, k] int32 (as written by isa_forward).
 * The ids are read on the device and not checked: each must lie in
 * [0, n_ctx_blocks), or the copy reads outside K and V.
 * isa_forward itself never materialises K_new: its attention kernels read
 * the same rows through the block table.  Errors: ISA_ERR_INVALID_ARG,
 * ISA_ERR_UNSUPPORTED (L_src or L_ctx not a multiple of the block length: the
 * length of K_new would depend on sel), ISA_ERR_HIP. */
isa_status_t isa_gather(isa_plan_t plan, const void* K, const void* V, const int32_t* sel,
                        void* K_new, void* V_new, void* stream);

/* Dense attention softmax(Q K^T / sqrt(D)) V over all N keys ([summary] 2
 * Standard Attention): the library's own dense baseline, same kernels as the
 * exact path.  Q, K, V, O: [B, H, N, D]; lse [B, H, N] float or NULL.
 * Requires N % 64 == 0 and D in {64, 128}.  Errors: ISA_ERR_INVALID_ARG,
 * ISA_ERR_UNSUPPORTED, ISA_ERR_HIP. */
isa_status_t isa_dense_forward(int32_t B, int32_t H, int32_t N, int32_t D, isa_dtype_t dtype,
                               const void* Q, const void* K, const void* V, void* O,
                               float* lse, void* stream);

/* Backward of isa_forward with the decisions of that forward held fixed
 * (the trainable path: [notes] overall framework and highlights).  The
 * gradient flows through the exact path over K_new, V_new and through the
 * Taylor path and its block-mean pooling of K and V (dK_t += dK^c_j / w_j);
 * no gradient passes through the coarse map.  Context rows that were not
 * selected receive zero.  Q, K, V, O, dO, dQ, dK, dV: [B, H, N, D]; lse:
 * [B, H, N] float from the forward; aux: sel, flat and sharp from the
 * forward (required).  The decisions are read on the device and not checked:
 * they must be what isa_forward wrote for this plan (sel: k distinct ascending
 * context block ids; flat and sharp: together every query block once, each
 * list ascending), or the kernels read and write outside the tensors.
 * With rope_base > 0 the gradient is taken at the rotated Q and K the forward
 * used (re-rotated into the workspace, bit for bit the forward's), and dQ, dK
 * are turned back by each token's angle (the rotation is orthogonal per pair,
 * so dQ = R^T dQ'); the rounding of the rotated values is a storage step.
 * With the block mask (n_ns > 0 and flat blocks; [notes] key design 2: a
 * block pair with mask 1 takes the exact update, otherwise the representative
 * one) aux->ns is required too (n_ns distinct ascending positions in
 * [0, n_kv) per flat block): a flat row's token terms of its exact blocks
 * feed dK, dV of those tokens, its representative terms feed the pooled
 * gradient of the other blocks.
 * workspace: at least isa_backward_workspace_bytes() (with rope_base > 0 it
 * holds the rotated Q and K, two [B, H, N, D] copies; with the block mask,
 * the exact-block tables: about B * H * n_flat * (n_ns + n_kv / 32) * 4 bytes).
 * Errors: ISA_ERR_INVALID_ARG (also a null aux->ns with the block mask),
 * ISA_ERR_UNSUPPORTED (FP32), ISA_ERR_WORKSPACE, ISA_ERR_HIP.  Any plan
 * isa_plan_create accepts is taken otherwise: partial blocks (L_src or L_ctx
 * not a multiple of b; a block of w tokens enters the Taylor path with weight
 * w and its mean over those w rows) and b = 32, 64, 128. */
isa_status_t isa_backward(isa_plan_t plan, const void* Q, const void* K, const void* V,
                          const void* O, const void* dO, const float* lse, const isa_aux_t* aux,
                          void* dQ, void* dK, void* dV,
                          void* workspace, size_t workspace_bytes, void* stream);

/* Workspace isa_backward needs for this plan (0 for an invalid plan). */
size_t isa_backward_workspace_bytes(isa_plan_t plan);

/* Static description of a status code. */
const char* isa_status_string(isa_status_t status);

/* The hipError_t of the last failed HIP call on this thread (0 if none). */
int isa_last_hip_error(void);


#ifdef __cplusplus
}
#endif

#endif /* ISA_H */
