/*
 * gdpa.h - C ABI of the MI355X (gfx950) implementation of generalized dot-product attention.
 *
 * The operator (Kunlun paper review, liuzhao09.github.io, section 2.3 "GDPA" and Figure 2;
 * Kunlun reproduction README, daiwk.github.io, "Core equations"; substack "Kunlun Breakdown",
 * "The Core Architecture and Mechanics"): per sequence b and head h,
 *
 *     S = scale * Q_bh K_bh^T  [+ log sigmoid(G_bh) added to every row]
 *     O_bh = phi(S) V_bh
 *
 * with phi an element-wise activation (GELU, SiLU: the personalized-FFN form, where the keys and
 * values are per-sample weights generated from the context) or a row softmax (the gated-softmax
 * form). Self-attention is the case q_offsets == kv_offsets; a sliding window (review, section
 * 2.5) restricts query position i to key positions i-window_left .. i+window_right.
 *
 * Memory and ownership
 *   - Every tensor pointer is a DEVICE pointer owned by the caller. The library never allocates,
 *     frees or synchronizes; a call validates its arguments on the host, enqueues its kernels on
 *     `stream` (a hipStream_t; NULL = the default stream) and returns.
 *   - Layouts are dense row-major with no strides: q, o, dout, dq are [total_q, H, d]; k, v, dk, dv
 *     are [total_kv, H, d]; g, dg are [total_kv, H] float32; lse is [total_q, H] float32.
 *   - q_offsets / kv_offsets are device int32 arrays of num_seqs+1 non-decreasing entries starting
 *     at 0 and ending at total_q / total_kv; sequence b owns rows [offsets[b], offsets[b+1]). The
 *     host-side hints max_seqlen_q / max_seqlen_kv must bound the real lengths (they size the
 *     launch and the workspace).
 *   - The workspace `ws` (device memory of at least gdpa_workspace_size() bytes, 256-byte aligned)
 *     is scratch for the call's work list and, in the backward, for fp32 row accumulators (long
 *     key ranges that are processed in chunks, shared query matrices). Its first 4 bytes
 *     (GDPA_WS_ERROR_OFFSET) are the device error word described below, the next 4 the work
 *     list's signature (written by the work-list builder, read by planned calls); the rest of its
 *     contents on entry are ignored.
 *   - The library keeps no state between calls; distinct calls may run concurrently on different
 *     streams as long as they use distinct workspaces and outputs.
 *
 * Errors
 *   Every status check runs synchronously on the host before any HIP call: a non-zero return
 *   means nothing was enqueued. GDPA_ERR_HIP reports a failed kernel launch (hipGetLastError).
 *
 *   The offsets live on the device, so the host cannot check them. Instead every kernel checks the
 *   offsets of its own work item before touching memory: both row ranges inside their tensors,
 *   lengths within what the launch provisioned from the max_seqlen hints, equal query and key
 *   lengths under a window. An item that fails writes none of its outputs and sets bits of the
 *   int32 device error word at GDPA_WS_ERROR_OFFSET in the workspace (GDPA_DEVICE_ERR_*), so a
 *   violated precondition never leads to an out-of-bounds access. A call that launches kernels
 *   clears the word first, except a bf16 call with GDPA_FLAG_PLANNED, which adds its bits to
 *   what the word holds since the gdpa_plan that built its work list (gdpa_plan clears it). The
 *   caller reads the word after synchronizing.
 *
 *   Debug validation: with GDPA_FLAG_VALIDATE in a problem's flags, or the environment variable
 *   GDPA_DEBUG=1 at call time, the call first enqueues a kernel that checks every sequence by the
 *   rules of gdpa_validate_offsets() (which runs the same checks on host copies) and writes the
 *   result to the error word; when it is non-zero the main kernels then return without reading
 *   or writing anything (outputs are left untouched).
 */
#ifndef GDPA_H_
#define GDPA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDPA_MAX_GROUPS 16

/* gdpa_problem.flags: the workspace already holds the work list that gdpa_plan() built for
 * problems with the same n_groups, num_seqs and num_heads; the call skips rebuilding it. The list
 * is a permutation of (group, head, sequence) items, so a list built from older offsets of the
 * same shape is still complete (only its longest-first order may be stale). The list puts the
 * items of short-key groups (bf16, element-wise act, no head_acts, no window, no shared queries,
 * max_seqlen_kv <= 32) after every other group's, and the backward runs that tail in a kernel of
 * its own, so plan and call must also agree on which groups these are. gdpa_plan leaves a
 * signature of the item count and of that split in the workspace header; a planned call whose
 * problems give another signature writes nothing and sets GDPA_DEVICE_ERR_PLAN. */
#define GDPA_FLAG_PLANNED 1

/* gdpa_problem.flags: one query matrix shared by every sequence (learnable seed or summary-token
 * queries attending over each jagged sequence: the PMA / hierarchical seed pooling use of the
 * operator, Kunlun review, sections 2.3 and 2.4). q and dq are then [max_seqlen_q, H, d]: query row
 * i of every sequence is row i of q, and dq is the sum of the per-sequence gradients. o, lse and
 * dout keep their [total_q, ...] rows at q_offsets, and every q_offsets[b+1]-q_offsets[b] must be
 * at most max_seqlen_q. bf16 only; not with self_attention (hence no window). */
#define GDPA_FLAG_SHARED_Q 2

/* gdpa_problem.flags: float32 outputs for a bf16 problem. o (forward) and dq, dk, dv (backward)
 * are float32 arrays of the same shapes; q, k, v and dout stay bf16. The arithmetic is unchanged
 * (bf16 MFMA operands, P and dS rounded once to bf16, fp32 accumulation); only the final rounding
 * of the results to bf16 is left out, which removes the largest term of their error against the
 * exact result. Groups of one call may differ in it. No effect on a float32 problem, whose
 * outputs are float32 already. */
#define GDPA_FLAG_FP32_OUT 4

/* gdpa_problem.flags: enqueue the offsets-validation kernel before the main kernels (see Errors
 * above; the environment variable GDPA_DEBUG=1 has the same effect for every call). */
#define GDPA_FLAG_VALIDATE 8

/* gdpa_problem.flags (bf16, element-wise activations): P and dS enter every backward product as a
 * high + low bf16 pair, as they do by default for sums of at most 16 terms (items with that few
 * rows or keys) and for the softmax form. One rounding of P / dS to bf16 has a relative error of
 * up to 2^-9 per term; for the dK / dV sums of a long sequence batched with many much shorter
 * ones, that error can exceed 2e-2 of the whole tensor's RMS (which the short sequences lower).
 * The pair brings it to about 2^-17. Costs two more matrix products per score block. */
#define GDPA_FLAG_SPLIT_OPERANDS 16

/* Byte offset of the int32 device error word in the workspace. */
#define GDPA_WS_ERROR_OFFSET 0

/* Bits of the device error word (and of gdpa_validate_offsets' result). */
#define GDPA_DEVICE_ERR_OFFSETS 1 /* offsets decrease, leave their tensor, or do not start at 0 /
                                     end at total_q, total_kv */
#define GDPA_DEVICE_ERR_LENGTH 2  /* a sequence longer than max_seqlen_q / max_seqlen_kv allow */
#define GDPA_DEVICE_ERR_SELF 4    /* self-attention (or a window) with query and key sequences that
                                     differ */
#define GDPA_DEVICE_ERR_PLAN 8    /* GDPA_FLAG_PLANNED with a work list that gdpa_plan built for
                                     problems of another item count or short-key split: the call's
                                     kernels returned without touching any output */

typedef enum gdpa_status {
  GDPA_OK = 0,
  GDPA_ERR_INVALID_ARGUMENT = -1, /* null pointer, bad size, inconsistent window, ... */
  GDPA_ERR_UNSUPPORTED = -2,      /* valid request outside what the kernels implement */
  GDPA_ERR_WORKSPACE = -3,        /* workspace missing, misaligned or too small */
  GDPA_ERR_HIP = -4               /* a kernel launch failed */
} gdpa_status;

typedef enum gdpa_dtype {
  GDPA_DTYPE_BF16 = 0, /* q/k/v/o/dout/dq/dk/dv in bfloat16; MFMA with fp32 accumulation */
  GDPA_DTYPE_FP32 = 1  /* all tensors float32, fp32 arithmetic */
} gdpa_dtype;

typedef enum gdpa_act {
  GDPA_ACT_GELU = 0,   /* x * Phi(x), Phi the standard normal CDF */
  GDPA_ACT_SILU = 1,   /* x * sigmoid(x) */
  GDPA_ACT_SOFTMAX = 2 /* row softmax over the allowed keys; writes lse */
} gdpa_act;

/* One GDPA problem (one event group). */
typedef struct gdpa_problem {
  int32_t num_seqs;      /* B >= 0 */
  int32_t num_heads;     /* H, 1..256 */
  int32_t head_dim;      /* d: 32, 64 or 128 */
  int32_t dtype;         /* gdpa_dtype */
  int32_t act;           /* gdpa_act */
  float scale;           /* multiplies Q K^T (finite) */
  int32_t window_left;   /* >= 0, or -1 = unbounded; bounded only for self-attention */
  int32_t window_right;  /* >= 0, or -1 = unbounded; bounded only for self-attention */
  int64_t total_q;       /* rows of q (= q_offsets[B]) */
  int64_t total_kv;      /* rows of k and v (= kv_offsets[B]) */
  int32_t max_seqlen_q;  /* upper bound on any q_offsets[b+1]-q_offsets[b] */
  int32_t max_seqlen_kv; /* upper bound on any kv_offsets[b+1]-kv_offsets[b] */
  int32_t self_attention;/* 1: kv_offsets equal q_offsets (same sequences); 0: cross-attention */
  int32_t flags;         /* GDPA_FLAG_* bits; GDPA_FLAG_PLANNED must agree across a call */
  const int32_t* q_offsets;  /* device [B+1] */
  const int32_t* kv_offsets; /* device [B+1] */
  /* Optional DEVICE array [num_heads] of gdpa_act: head h uses head_acts[h] instead of act (the
   * review, section 2.3, lets the activation differ between heads). Trusted like the offsets.
   * When given, lse must be provided (it is written, and read back, for the softmax heads). */
  const int32_t* head_acts;
} gdpa_problem;

/* Device tensors of one problem. Unused entries may be NULL, and so may every tensor with no rows
   (total_q == 0: o, lse, dout, and q, dq unless the queries are shared, whose rows number
   max_seqlen_q; total_kv == 0: k, v, g, dk, dv, dg). A problem with
   num_seqs == 0 (then total_q == total_kv == 0) returns GDPA_OK and enqueues nothing. */
typedef struct gdpa_tensors {
  const void* q;     /* [total_q, H, d] */
  const void* k;     /* [total_kv, H, d] */
  const void* v;     /* [total_kv, H, d] */
  const float* g;    /* gate G [total_kv, H] float32, or NULL for no gate */
  void* o;           /* forward output [total_q, H, d] */
  float* lse;        /* forward output [total_q, H] natural-log row log-sum-exp; softmax only */
  const void* dout;  /* backward input: dL/dO [total_q, H, d] */
  void* dq;          /* backward outputs, same layout as q, k, v; their dtype, or float32 with
                        GDPA_FLAG_FP32_OUT (o too) */
  void* dk;
  void* dv;
  float* dg;         /* gate gradient [total_kv, H] float32; NULL if not wanted */
} gdpa_tensors;

/*
 * Bytes of workspace needed by one call covering `n_groups` problems (pass: 0 forward,
 * 1 backward). Returns 0 if the arguments are invalid.
 */
size_t gdpa_workspace_size(const gdpa_problem* problems, int32_t n_groups, int32_t pass);

/*
 * Forward: O = phi(scale Q K^T [+ log sigmoid G]) V for every sequence and head (and lse for the
 * softmax form). Reads q, k, v (g); writes o (lse). Source: the operator statement above.
 */
int gdpa_fwd(const gdpa_problem* problem, const gdpa_tensors* tensors, void* ws, size_t ws_bytes,
             void* stream);

/*
 * Backward of the same definition for the upstream gradient dout: writes dq, dk, dv (and dg when
 * non-NULL). For the softmax form it also reads lse from the forward (o is not needed: the row
 * term sum_j p_ij dp_ij is recomputed from the scores). Keys that no query sees get zero
 * gradients. (FlashAttention-style backward that keeps the score matrix on chip:
 * Kunlun review, section 2.3 / Figure 2.)
 */
int gdpa_bwd(const gdpa_problem* problem, const gdpa_tensors* tensors, void* ws, size_t ws_bytes,
             void* stream);

/* Largest workspace gdpa_bwd_noalloc can provide (bytes). */
#define GDPA_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * gdpa_bwd without a workspace argument and without any allocation, for callers that cannot
 * allocate device memory at call time (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation). The workspace is a 16 MiB array (GDPA_NOALLOC_SCRATCH_BYTES)
 * of device memory that the library holds on each GPU it runs on until the process ends; the
 * call uses the array of the current device (which must be the stream's device) and returns
 * GDPA_ERR_WORKSPACE, with nothing enqueued, when gdpa_workspace_size(problem, 1, 1) exceeds it.
 * It allocates, frees and synchronizes nothing (the first call on a device looks the array's
 * address up). GDPA_FLAG_PLANNED is refused (GDPA_ERR_INVALID_ARGUMENT): every call builds its
 * own work list. Every call on one GPU shares that GPU's array, so calls that overlap in time on
 * one GPU (other streams, other threads) race and must not be issued; the array keeps the last
 * call's contents, which no call reads before writing (the device error word is cleared by the
 * call itself, and items that fail their offsets check still write nothing, but the word is not
 * reported). Arguments, outputs and errors are otherwise those of gdpa_bwd.
 */
int gdpa_bwd_noalloc(const gdpa_problem* problem, const gdpa_tensors* tensors, void* stream);

/*
 * Grouped forward / backward: `n_groups` (1..GDPA_MAX_GROUPS) independent problems, each with its
 * own shapes, activation and tensors, in ONE launch of the main kernel (event-level
 * personalization: each event type gets its own width, head count and depth; Kunlun review,
 * section 2.5). All problems must share the dtype.
 */
int gdpa_fwd_grouped(const gdpa_problem* problems, const gdpa_tensors* tensors, int32_t n_groups,
                     void* ws, size_t ws_bytes, void* stream);
int gdpa_bwd_grouped(const gdpa_problem* problems, const gdpa_tensors* tensors, int32_t n_groups,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * Jagged work decomposition on its own: enqueue the kernel that orders the (group, head, sequence)
 * work items of `problems` longest-first from the device offsets, into `ws` (sized by
 * gdpa_workspace_size for the pass that follows). Subsequent gdpa_fwd / gdpa_bwd (and grouped)
 * calls with GDPA_FLAG_PLANNED set reuse it, e.g. one plan per training step for both passes.
 * (Tile scheduling over jagged, large-batch inputs: Kunlun review, section 2.3.)
 */
int gdpa_plan(const gdpa_problem* problems, int32_t n_groups, void* ws, size_t ws_bytes, void* stream);

/*
 * The device offsets check on host copies: q_offsets_host / kv_offsets_host are host arrays of
 * problem->num_seqs + 1 entries (the problem's own offset pointers are not read). Returns the OR
 * of GDPA_DEVICE_ERR_* bits over all sequences (0: the offsets meet every rule the kernels rely
 * on), or a negative gdpa_status if the problem itself is invalid or an array is NULL. The
 * validation kernel enqueued by GDPA_FLAG_VALIDATE / GDPA_DEBUG=1 applies the same function to
 * each sequence.
 */
int gdpa_validate_offsets(const gdpa_problem* problem, const int32_t* q_offsets_host,
                          const int32_t* kv_offsets_host);

/* Static description of a status code (never NULL). */
const char* gdpa_strerror(int status);

/* Library version, major*10000 + minor*100 + patch. */
int gdpa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GDPA_H_ */
