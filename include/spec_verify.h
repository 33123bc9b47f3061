/*
 * spec_verify.h -- C ABI of the batched speculative-decoding verify step on
 * AMD Instinct MI355X (gfx950).
 *
 * The operation (pages cited by title and section):
 *   [A] "推测解码与连续批处理深度实战：突破自回归生成的双重瓶颈", section 1.2:
 *       a draft model proposes gamma tokens (step 1); the target model scores
 *       all gamma+1 positions in one parallel pass (step 2); each draft token
 *       x at position i is accepted with probability min(1, p_i(x) / q_i(x)),
 *       and a rejected position is resampled from clip(p_i - q_i, 0)
 *       (step 3); the output then has exactly the target's distribution
 *       (step 4).
 *   [D] "大模型推理加速新范式：推测解码（Speculative Decoding）原理剖析与
 *       vLLM生产级实现", section 2.1 (verification stops at the first
 *       rejected position and every later draft is dropped) and section 2.2
 *       (the acceptance ratio min(1, p(x)/q(x)) and the resampling
 *       distribution norm(max(0, p - q))).
 *   [B] the blog.hotdry.top post on speculative decoding and dynamic
 *       batching, items 流程编排 (compare candidates in order, keep the prefix
 *       before the first mismatch) and 硬件并行 (pack the candidates of many
 *       requests into one batch), and its 结合使用 paragraph (speculative and
 *       plain-decode requests share a batch).
 *   [E] the same vLLM page, section 5.2: requests are rejected at different
 *       positions, so padded batches waste work -- hence the packed layout.
 *
 * Readings where the pages are silent (each one is fixed here):
 *   - p = softmax(l_target / T), q = softmax(l_draft / T) with one scalar
 *     temperature T > 0 for both (the pages only show temperature=0.7 as an
 *     API field, [D] section 4.2).
 *   - draft i is accepted iff u_i < p_i(x_i) / q_i(x_i) (strict).
 *   - when all gamma drafts pass, one bonus token is drawn from the target's
 *     (gamma+1)-th distribution (implied by the gamma+1 scored positions of
 *     [A] step 2).
 *   - every draw is an inverse-CDF draw over ascending token id with one
 *     pre-drawn uniform: the smallest k with C_k > u * S, where C_k is the
 *     running sum of the weights and S their total.
 *
 * Packed ragged layout (no padding), one launch for any mix of gamma_b >= 0
 * (gamma_b = 0 is a plain decode step: one draw from the target row):
 *   cu_draft[b]  = gamma_0 + ... + gamma_{b-1}      (int32, B+1 entries)
 *   target row of (b, i), 0 <= i <= gamma_b :  cu_draft[b] + b + i
 *   draft row of (b, i),  0 <= i <  gamma_b :  cu_draft[b] + i
 *   R_d = cu_draft[B] draft rows, R_t = R_d + B target rows
 *   uniforms[target row of (b, i)], i < gamma_b : accept test of draft i
 *   uniforms[target row of (b, gamma_b)]        : the final draw (resample
 *                                                 or bonus)
 *   out_tokens[target row of (b, i)] : draft i for i < n_b, the drawn token
 *                                      at i = n_b, -1 for n_b < i <= gamma_b
 *
 * Memory, ownership, threading:
 *   - Every pointer in spec_verify_args is DEVICE memory owned by the caller
 *     (allocated for example by PyTorch); the library allocates nothing and
 *     frees nothing.  The context holds only host-side state.
 *   - spec_verify_run only enqueues kernels on the given HIP stream and never
 *     synchronises; inputs must stay valid until the stream passes the call.
 *   - A context is immutable after creation.  Calls on different streams
 *     may overlap if each uses its own workspace; calls that share a
 *     workspace must be ordered (same stream).  One call is two kernel
 *     launches: a row-parallel statistics pass and a per-sequence finish;
 *     the stream orders them, and no workgroup ever waits for another.
 *
 * Errors: functions return SPEC_VERIFY_OK (0) or a negative status; no C++
 * exception or abort crosses the ABI.  Argument checks happen on the host
 * before any HIP call.  Device-data preconditions (monotone cu_draft with
 * cu_draft[B] = R_d, tokens in [0, V), uniforms in [0, 1), logits finite or
 * -inf with at least one finite entry per row, q_i(x_i) > 0) are the
 * caller's.  Out-of-range offsets and tokens never cause out-of-bounds
 * accesses: the kernels skip such sequences (their outputs become -1) and,
 * when `status` is given, OR the SPEC_VERIFY_DEV_* bits into it; with
 * SPEC_VERIFY_FLAG_CHECK the remaining preconditions are checked as well.
 */
#ifndef SPEC_VERIFY_H_
#define SPEC_VERIFY_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#if defined(__GNUC__)
#define SPEC_VERIFY_API __attribute__((visibility("default")))
#else
#define SPEC_VERIFY_API
#endif

/* Return codes. */
#define SPEC_VERIFY_OK 0
#define SPEC_VERIFY_EINVAL -1      /* NULL required pointer, B < 0, T <= 0 or
                                      non-finite, ld < V, unaligned element
                                      pointers, wrong device, bad sizes */
#define SPEC_VERIFY_EUNSUPPORTED -2 /* dtype not f32/bf16, V <= 0, V > 2^21 */
#define SPEC_VERIFY_ECAPACITY -3   /* B > max_seqs, R_d > max_draft_rows,
                                      workspace smaller than required, or a
                                      batch so large that a launch would
                                      exceed 2^32 threads (rows * ceil(V /
                                      4096) * 64, or B * 512 per finishing
                                      workgroup) */
#define SPEC_VERIFY_EHIP -4        /* a HIP call failed; see
                                      spec_verify_last_hip_error() */

/* Logit element types. */
#define SPEC_VERIFY_F32 0
#define SPEC_VERIFY_BF16 1

/* Create-time flags. */
#define SPEC_VERIFY_FLAG_CHECK 1u  /* kernels validate every device-data
                                      precondition into *status */

/* Bits the kernels OR into *status (when status != NULL). */
#define SPEC_VERIFY_DEV_BAD_OFFSETS 1u   /* cu_draft not monotone / out of range;
                                            the sequence is skipped */
#define SPEC_VERIFY_DEV_BAD_TOKEN 2u     /* a draft token outside [0, V); the
                                            sequence is skipped */
#define SPEC_VERIFY_DEV_BAD_UNIFORM 4u   /* (CHECK) a uniform outside [0, 1) */
#define SPEC_VERIFY_DEV_BAD_LOGIT 8u     /* (CHECK) a NaN or +inf logit */
#define SPEC_VERIFY_DEV_EMPTY_ROW 16u    /* (CHECK) a row with no finite logit */
#define SPEC_VERIFY_DEV_ZERO_Q 32u       /* (CHECK) q_i(x_i) = 0 */
#define SPEC_VERIFY_DEV_EMPTY_RESIDUAL 64u /* the residual summed to 0; the draw
                                              fell back to p at that position */
#define SPEC_VERIFY_DEV_BAD_TREE 128u    /* a tree with more than
                                            SPEC_VERIFY_MAX_TREE_NODES nodes, a
                                            parent not before its child, a token
                                            outside [0, V) or more than
                                            SPEC_VERIFY_MAX_TREE_CHILDREN children
                                            of one node; the sequence is skipped */

#define SPEC_VERIFY_DEV_RESIDUAL_UNRESOLVED 256u /* a residual whose mass is below
                                              2^-60 of the target row's: fp32
                                              terms below 2^-126 may be a share
                                              of it, so the draw is from its
                                              representable part */

/* Tree limits (per sequence). */
#define SPEC_VERIFY_MAX_TREE_NODES 1024
#define SPEC_VERIFY_MAX_TREE_CHILDREN 64

typedef struct spec_verify_ctx spec_verify_ctx;

typedef struct {
  int32_t num_seqs;            /* B >= 0 (host scalar); B = 0 is a no-op */
  int64_t total_draft_rows;    /* R_d = cu_draft[B] (host scalar) */
  const int32_t *cu_draft;     /* [B+1] exclusive prefix of gamma_b */
  const void *target_logits;   /* [R_t rows, pitch ld] of dtype */
  const void *draft_logits;    /* [R_d rows, pitch ld] of dtype (may be NULL
                                  when R_d = 0) */
  int64_t ld;                  /* row pitch in elements, >= V; a 16-byte
                                  aligned base and pitch take the vector path */
  const int32_t *draft_tokens; /* [R_d] the proposed tokens, in [0, V) */
  const float *uniforms;       /* [R_t] pre-drawn U[0,1) values */
  float temperature;           /* T > 0, applied to target and draft logits */
  int32_t *out_tokens;         /* [R_t] see the layout above */
  int32_t *out_num_accepted;   /* [B] n_b in [0, gamma_b] */
  float *out_p_draft;          /* [R_d] p_i(x_i), optional (NULL = skip) */
  float *out_q_draft;          /* [R_d] q_i(x_i), optional */
  float *out_residual_sum;     /* [B] sum_k max(0, p - q) at the rejected
                                  position, 0 when the bonus was drawn;
                                  optional */
  void *workspace;             /* >= spec_verify_workspace_size() bytes,
                                  256-byte aligned; no initial contents needed */
  size_t workspace_bytes;
  uint32_t *status;            /* optional device word; the kernels OR
                                  SPEC_VERIFY_DEV_* bits into it (the caller
                                  clears it) */
  void *const *timing_events;  /* optional: hipEvent_t[2 * kernels], created
                                  with timing enabled; events 2k and 2k+1 are
                                  the start and stop events of kernel k's own
                                  dispatch (hipExtLaunchKernel), in launch
                                  order (see spec_verify_num_kernels) */
} spec_verify_args;

/*
 * Create a context for one device, vocabulary size and logit dtype.
 * max_seqs / max_draft_rows bound B and R_d of later runs and fix the
 * workspace size, returned in *workspace_bytes.  The device's properties are
 * read here (this is the only call that queries the HIP runtime besides
 * run).  Returns OK, EINVAL, EUNSUPPORTED or EHIP; *out is NULL on failure.
 */
SPEC_VERIFY_API int spec_verify_create(spec_verify_ctx **out, int device,
                                       int64_t vocab, int dtype,
                                       int32_t max_seqs,
                                       int64_t max_draft_rows, uint32_t flags,
                                       size_t *workspace_bytes);

/*
 * Workspace bytes a context with these bounds needs, without creating one or
 * touching the HIP runtime (host-only; lets a caller size its allocation
 * first).  The workspace holds one 16-byte row-statistics partial per 4096
 * logits of every target and draft row (R_t + R_d = B + 2 R_d rows), four
 * doubles per 2048-logit tile of each sequence's final-draw rows (the
 * residual's tile sums), and one arrival counter per sequence (cleared
 * inside every call).  Returns OK, EINVAL or EUNSUPPORTED.
 */
SPEC_VERIFY_API int spec_verify_query_workspace(int64_t vocab, int32_t max_seqs,
                                                int64_t max_draft_rows,
                                                size_t *workspace_bytes);

/* Workspace bytes one run with this context needs (same value create gave). */
SPEC_VERIFY_API size_t spec_verify_workspace_size(const spec_verify_ctx *ctx);

/* Number of kernels one run launches (each bracketed by two timing events):
 * 2, for spec_verify_run, spec_verify_run_greedy and
 * spec_verify_run_point_drafts alike. */
SPEC_VERIFY_API int spec_verify_num_kernels(const spec_verify_ctx *ctx);

/*
 * Enqueue one verify step on `hip_stream` (a hipStream_t; NULL = the null
 * stream) on the context's device, which must be the current device.
 * Computes, for every sequence: p and q at all positions, the accepted count
 * n_b (first rejection, [D] 2.1), the emitted tokens, and the resampled or
 * bonus token ([A] 1.2 step 3).  Outputs are written only to the caller's
 * buffers and the workspace.
 */
SPEC_VERIFY_API int spec_verify_run(const spec_verify_ctx *ctx,
                                    const spec_verify_args *args,
                                    void *hip_stream);

/* Size of the library's own workspace used by spec_verify_run_static. */
#define SPEC_VERIFY_STATIC_WORKSPACE_BYTES (16u << 20)

/*
 * spec_verify_run without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  The workspace is the library's own
 * file-scope device array of SPEC_VERIFY_STATIC_WORKSPACE_BYTES (16 MiB),
 * one copy per device the library runs on, held until the process ends; its
 * device address is resolved once per device by spec_verify_create.
 * args->workspace and args->workspace_bytes are ignored; nothing is
 * allocated or freed.  The call's own need, spec_verify_query_workspace(V,
 * B, R_d) for this call's B and R_d, must fit in the array: otherwise it
 * returns SPEC_VERIFY_ECAPACITY and enqueues nothing (16 MiB holds, e.g.,
 * 1024 sequences of 8 drafts at V = 128256, which need 10.5 MiB).  Every call on one device
 * shares the array and each call clears the state it needs itself, so calls
 * ordered on one stream are safe; calls that can overlap on one device
 * (different streams, or graphs replayed concurrently) race and must not be
 * issued.  Same kernels, results and other errors as spec_verify_run.
 */
SPEC_VERIFY_API int spec_verify_run_static(const spec_verify_ctx *ctx,
                                           const spec_verify_args *args,
                                           void *hip_stream);

/*
 * Greedy verification: the temperature -> 0 limit of spec_verify_run.
 * [B] item 流程编排: the drafts are compared in order with the target's
 * choices, the prefix before the first mismatch is kept and decoding resumes
 * at the mismatched position.  Under greedy decoding the target's choice at
 * a position is the argmax of its logits, and equal maxima go to the lowest
 * token id (a reading: the page names no tie rule).  For every sequence:
 *   n_b = the first i with draft_tokens[i] != argmax(target row i), or
 *         gamma_b when every draft matches;
 *   out_tokens = the drafts before n_b, then argmax(target row n_b) (the
 *         token at the mismatch, or the bonus when n_b = gamma_b), then -1.
 * Same argument block, layout, workspace and error behaviour as
 * spec_verify_run.  Used: num_seqs, total_draft_rows, cu_draft,
 * target_logits, ld, draft_tokens, out_tokens, out_num_accepted, workspace,
 * workspace_bytes, status, timing_events.  Ignored (may be NULL / any
 * value): draft_logits, uniforms, temperature, out_p_draft, out_q_draft,
 * out_residual_sum.  Only the R_t target rows are read, once.  Logits must
 * not be NaN (SPEC_VERIFY_FLAG_CHECK reports NaN and +inf as
 * SPEC_VERIFY_DEV_BAD_LOGIT); an all -inf row has argmax 0.  Two kernels.
 */
SPEC_VERIFY_API int spec_verify_run_greedy(const spec_verify_ctx *ctx,
                                           const spec_verify_args *args,
                                           void *hip_stream);

/*
 * Verification of deterministic drafts: the draft proposes tokens without a
 * distribution (n-gram / prompt-lookup drafting: [A] sections 1.4 and 3.3,
 * and section 4.1 of [D]), so the draft distribution at position i is the
 * point mass at x_i.  The rule of spec_verify_run then reads:
 *   accept draft i iff u_i < p_i(x_i)                 (q_i(x_i) = 1);
 *   after a rejection at j, draw from norm(max(0, p_j - delta_{x_j})), which
 *   is p_j with x_j removed and renormalised;
 *   when every draft passes, the bonus is drawn from p_{gamma_b}.
 * Same argument block, uniforms, layout, workspace and error behaviour as
 * spec_verify_run; draft_logits is ignored (may be NULL) and no draft row is
 * read.  out_q_draft, when given, receives 1.0; out_residual_sum receives
 * the sum of p_j over k != x_j (0 after a bonus draw).  Two kernels.
 */
SPEC_VERIFY_API int spec_verify_run_point_drafts(const spec_verify_ctx *ctx,
                                                 const spec_verify_args *args,
                                                 void *hip_stream);

/*
 * Tree verification.  [D] section 3.2 (Tree Attention): the drafter proposes
 * its top candidates at each position, forming a tree, and the target scores
 * every node of the tree in one pass.  The page gives no acceptance rule; the
 * readings fixed here:
 *   greedy (spec_verify_tree_run_greedy): from the root, move to the
 *     lowest-index child whose token is the argmax of the current node's row
 *     (lowest id among equal maxima; [B] 流程编排); where no child matches,
 *     emit that argmax.
 *   point-mass candidates (spec_verify_tree_run_point): candidates carry no
 *     distribution, so each is a point mass ([A] 1.2 step 3 with q = delta_x).
 *     The current node's children are tried in index order; child c is
 *     accepted iff u_c < p'(x_c), p' being the node's p = softmax(l / T) with
 *     the tokens of already rejected siblings removed and renormalised (a
 *     token already rejected has p' = 0).  When every child is rejected, or
 *     at a node without children, the final token is drawn from p' with the
 *     root's uniform (inverse CDF as in spec_verify_run).  Each token is then
 *     emitted with probability exactly p_k at every depth.
 * Layout (packed, one launch for any mix of tree shapes): sequence b owns
 * the nodes g = cu_nodes[b] + n, 0 <= n < N_b, N_b >= 1; node 0 is the root
 * (the last committed token).  parent[g] is node n's parent as a local index
 * with 0 <= parent < n (root: ignored); tokens[g] its token (root: ignored);
 * target row g (pitch ld) the target's logits for the token after node n;
 * uniforms[g] node n's accept test, the root's slot the final draw.
 * Outputs at the sequence's N_b slots: out_tokens = the accepted nodes'
 * tokens, then the final token, then -1; out_path = the accepted nodes'
 * local indices (which KV entries to keep), then -1; out_num_accepted[b] =
 * the accepted depth.  The context's workspace holds the row statistics of
 * up to max_seqs + 2 * max_draft_rows nodes and at most max_seqs trees.
 * Errors as spec_verify_run; a malformed tree is skipped (outputs -1, status
 * SPEC_VERIFY_DEV_BAD_TREE).  Two kernels: a row pass over the R node rows
 * and one workgroup per tree.
 */
typedef struct {
  int32_t num_seqs;            /* B >= 0 (host scalar) */
  int64_t total_nodes;         /* R = cu_nodes[B] (host scalar) */
  const int32_t *cu_nodes;     /* [B+1] */
  const int32_t *parent;       /* [R] */
  const int32_t *tokens;       /* [R] */
  const void *target_logits;   /* [R rows, pitch ld] of the context's dtype */
  int64_t ld;                  /* >= V */
  const float *uniforms;       /* [R]; point-mass candidates only */
  float temperature;           /* T > 0; point-mass candidates only */
  int32_t *out_tokens;         /* [R] */
  int32_t *out_path;           /* [R] */
  int32_t *out_num_accepted;   /* [B] */
  void *workspace;             /* as in spec_verify_args */
  size_t workspace_bytes;
  uint32_t *status;            /* optional */
  void *const *timing_events;  /* optional, as in spec_verify_args */
} spec_verify_tree_args;

SPEC_VERIFY_API int spec_verify_tree_run_greedy(const spec_verify_ctx *ctx,
                                                const spec_verify_tree_args *args,
                                                void *hip_stream);

SPEC_VERIFY_API int spec_verify_tree_run_point(const spec_verify_ctx *ctx,
                                               const spec_verify_tree_args *args,
                                               void *hip_stream);

/* Destroy a context (NULL is accepted).  Returns OK. */
SPEC_VERIFY_API int spec_verify_destroy(spec_verify_ctx *ctx);

/* Static description of a return code. */
SPEC_VERIFY_API const char *spec_verify_status_string(int status);

/* The hipError_t of the last EHIP failure on the calling thread (0 if none). */
SPEC_VERIFY_API int spec_verify_last_hip_error(void);

/*
 * Measurement only, not part of the verify step: one streaming read of
 * `bytes` of device memory at `src` with the row pass's load pattern (one
 * wave per 8 KB, 16-byte loads, each load instruction covering 1 KB of
 * contiguous memory; non-temporal loads when `nontemporal` is nonzero), to
 * measure the chip's practical read bandwidth next to the row pass.  `src`
 * is 16-byte aligned and `bytes` a nonzero multiple of 8192; `sink` is one
 * device uint32 that is written only if the data folds (XOR) to 0x9E3779B9.
 * start_event / stop_event (hipEvent_t created with timing, both or
 * neither) become the kernel's own dispatch start / stop events.  Enqueues
 * one kernel on `hip_stream`; returns OK, EINVAL, ECAPACITY or EHIP.
 */
SPEC_VERIFY_API int spec_verify_read_probe(const void *src, size_t bytes, int nontemporal,
                                           uint32_t *sink, void *hip_stream,
                                           void *start_event, void *stop_event);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H_ */
