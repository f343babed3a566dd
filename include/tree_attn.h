/*
 * tree_attn.h -- C ABI of the MI355X (gfx950) shared-prefix tree-attention
 * library.
 *
 * What is computed
 * ----------------
 * Tokens are packed as DFS-linearized segments with parent information
 * (Megatron-LM issue "Shared-prefix training with context parallelism for
 * exact agent trajectories", section "Describe the solution you'd like";
 * Megatron-LM pull request 7387, section "Summary": DFS segments and
 * ancestor relationships).  Each query token i of segment u attends to the
 * keys/values of every strict ancestor segment of u (whole segments) plus
 * the tokens of u up to and including i ("attention for each query run
 * against only its ancestor path", same section of the issue).  Siblings and
 * other trees are invisible (draft "feat(hybrid): add opt-in shared-prefix
 * attention and Mamba execution", intro: each suffix stays causally
 * isolated).  The backward pass returns dq, dk, dv of
 * L = sum_{i,h} <dout[i,h], out[i,h]>; dk/dv of a shared prefix token sum the
 * contributions of every branch below it (same draft, intro).  No dense T x T
 * mask is built anywhere (pull request 7387, "Summary").
 *
 * Conventions
 * -----------
 * Tensors are contiguous, token-major ("THD"):
 *   q, out, dout, dq : [T, Hq, D]     k, v, dk, dv : [T, Hkv, D]
 *   lse              : [Hq, T] float32, natural log of the softmax denominator
 * element type bfloat16 or float32 (tree_attn_shape.dtype); arithmetic is
 * float32 accumulation (bf16 inputs feed bf16 matrix-core products; the
 * softmax probabilities are rounded to bf16 before the P*V product).
 * Query head h uses key/value head h / (Hq / Hkv).  softmax_scale <= 0 means
 * 1/sqrt(D); a NaN or infinite softmax_scale is INVALID_ARGUMENT.
 *
 * Ownership: the caller owns every tensor (device memory) and the
 * workspace; the library owns a plan (host + device copies of the
 * topology-derived tile lists) until tree_attn_plan_destroy.
 *
 * Errors: every entry point returns 0 on success or a negative code; the
 * message of the last failure on the calling thread is returned by
 * tree_attn_last_error().  All checks run before the first kernel launch, so
 * a rejected call writes nothing (pull request 7387, "Summary": unsupported
 * modes are rejected rather than silently ignored).  Faults inside a kernel
 * surface asynchronously at the caller's next synchronisation, as in HIP.
 *
 * Calls on different streams may share one plan; kernels are asynchronous on
 * the given stream (a hipStream_t, NULL = the default stream).
 */
#ifndef TREE_ATTN_H_
#define TREE_ATTN_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* return codes */
#define TREE_ATTN_OK 0
#define TREE_ATTN_INVALID_ARGUMENT (-1) /* null pointer, malformed topology, size mismatch, small workspace */
#define TREE_ATTN_UNSUPPORTED (-2)      /* dtype / head_dim / head grouping not implemented */
#define TREE_ATTN_HIP_ERROR (-3)        /* a HIP runtime call or launch failed, or host memory ran out */

/* element types */
#define TREE_ATTN_BF16 0
#define TREE_ATTN_FP32 1

typedef struct tree_attn_plan_s* tree_attn_plan_t;

typedef struct {
  int32_t total_tokens; /* T; must equal the plan's token count */
  int32_t num_q_heads;  /* Hq >= 1 */
  int32_t num_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;     /* D: 64 or 128 for bf16, 64 for fp32 */
  int32_t dtype;        /* TREE_ATTN_BF16 or TREE_ATTN_FP32 */
  float softmax_scale;  /* finite; <= 0: 1/sqrt(D) */
} tree_attn_shape;

typedef struct {
  int32_t total_tokens;  /* T */
  int32_t num_segments;  /* S */
  int32_t num_roots;     /* trees in the forest */
  int32_t max_depth;     /* deepest segment (root = 0) */
  int64_t max_path_len;  /* longest reconstructed root-to-leaf sequence, tokens */
  int64_t pairs;         /* sum over tokens i of |V(i)|, per head: the
                            algorithmic (query, key) pair count */
  int32_t num_spans;     /* merged ancestor spans over all segments */
  int32_t num_q_tiles;   /* query tiles of 32 tokens */
  int32_t num_kv_tiles;  /* key tiles of 64 tokens */
  int32_t on_device;     /* 1 if device tables were uploaded */
  int32_t q_begin;       /* the plan's query run [q_begin, q_end): 0 and T */
  int32_t q_end;         /* unless built by tree_attn_plan_query_run */
} tree_attn_plan_info_t;

/*
 * Build a plan from a DFS-linearized segment forest.
 *   parent[s]    -1 for a root, else the index of an earlier segment;
 *   seg_start[s] first token of segment s; seg_start[0] == 0 and
 *                seg_start[s+1] == seg_start[s] + seg_len[s] (no gaps);
 *   seg_len[s]   >= 1 tokens.
 * The order must be a DFS pre-order: parent[s] is -1 or an ancestor-or-self
 * of segment s-1.  T = sum(seg_len) must be < 2^31.  The host arrays are
 * read during the call only.  Derives depth, the merged ancestor spans of
 * every segment, the query tiles (never crossing a segment) and the key
 * tiles with the contiguous range of queries that see them, and uploads
 * them to the current HIP device with a synchronous copy.  The plan is
 * immutable and reusable across heads, layers, passes and streams on that
 * device.  Errors: TREE_ATTN_INVALID_ARGUMENT (malformed input, *out left
 * NULL), TREE_ATTN_HIP_ERROR (device allocation/copy failed).
 */
int tree_attn_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                   int32_t num_segments, tree_attn_plan_t* out);

/*
 * tree_attn_plan with a stream-ordered upload: the tables are staged in
 * pinned host memory (kept by the plan until tree_attn_plan_destroy) and
 * copied with one asynchronous copy on `stream` (a hipStream_t, NULL = the
 * default stream), so the call never waits for kernels already queued on
 * the device.  Kernels on `stream` may use the plan right away; work on
 * another stream must first be ordered after the copy (an event).  Same
 * validation, ownership and errors as tree_attn_plan.
 */
int tree_attn_plan_async(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                         int32_t num_segments, void* stream, tree_attn_plan_t* out);

/*
 * A plan for one query run: the queries are the tokens [q_begin, q_end)
 * (0 <= q_begin < q_end <= T), the keys and values still every token.  This
 * is one context-parallel rank's share when the run is the rank's local
 * tokens and K/V were gathered from the group (issue "Shared-prefix training
 * with context parallelism for exact agent trajectories", section "Describe
 * the solution you'd like": queries stay local, K/V is gathered).
 *   tree_attn_fwd writes out and lse for the run's rows only and reads q of
 *     those rows only; other rows are untouched;
 *   tree_attn_bwd writes dq for the run's rows (others untouched) and all of
 *     dk and dv: the gradient of the run's part of the loss,
 *     sum over i in the run of <dout[i], out[i]>, i.e. this rank's share,
 *     to be summed over the ranks (keys no run query sees get zeros); it
 *     reads out, dout and lse of the run's rows only.
 * So over a partition of [0, T) into runs, out, lse and dq of every row are
 * bitwise those of the whole-token plan, and dk, dv are sums of the shares.
 * Validation and errors as tree_attn_plan, plus INVALID_ARGUMENT for an
 * empty or out-of-range run. */
int tree_attn_plan_query_run(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                             int32_t num_segments, int32_t q_begin, int32_t q_end, tree_attn_plan_t* out);
/* The same, host only (see tree_attn_plan_host). */
int tree_attn_plan_query_run_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                                  int32_t num_segments, int32_t q_begin, int32_t q_end, tree_attn_plan_t* out);

/* Same validation and derivation without touching any device: the plan can
 * be inspected (info, export) but not executed. */
int tree_attn_plan_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                        int32_t num_segments, tree_attn_plan_t* out);

/* Free host and device memory of a plan; NULL is a no-op.  The caller must
 * make sure no kernel using the plan is still running. */
int tree_attn_plan_destroy(tree_attn_plan_t plan);

/* Topology statistics of a plan (FLOP accounting uses `pairs`). */
int tree_attn_plan_info(tree_attn_plan_t plan, tree_attn_plan_info_t* info);

/*
 * Bounded fragment planning with ancestor repetition (host only; issue
 * "Shared-prefix training with context parallelism for exact agent
 * trajectories", section "Describe the solution you'd like": fragments are
 * size-bounded, and ancestor segments may be duplicated in several of them).  Splits a DFS segment forest
 * (as for tree_attn_plan) into fragments of at most max_tokens tokens, each
 * a DFS forest of its own (segments contiguous from token 0) in which every
 * token sees exactly the tokens it sees in the source forest: a fragment
 * that starts inside a tree first repeats the ancestor chain of its first
 * segment, root first, and a segment split at a fragment boundary restarts
 * in the next fragment with a repeated copy of its already placed part (one
 * segment).  Every source token is owned -- carries its loss -- in exactly
 * one fragment; repeated tokens are not owned (give them zero dout, and sum
 * dk/dv over a token's copies).  Fragments are filled in DFS order.
 * Errors: INVALID_ARGUMENT for a malformed forest, max_tokens < 1, or a
 * root-to-leaf path longer than max_tokens.  The result is library-owned.
 */
typedef struct tree_attn_fragments_s* tree_attn_fragments_t;
typedef struct {
  int32_t num_fragments;
  int32_t num_segments;     /* over all fragments */
  int32_t max_tokens;
  int64_t source_tokens;    /* T of the source forest */
  int64_t fragment_tokens;  /* tokens over all fragments: T plus the repeated ones */
} tree_attn_fragments_info_t;
int tree_attn_fragment(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len, int32_t num_segments,
                       int32_t max_tokens, tree_attn_fragments_t* out);
int tree_attn_fragments_destroy(tree_attn_fragments_t fragments);
int tree_attn_fragments_info(tree_attn_fragments_t fragments, tree_attn_fragments_info_t* info);
/* Tables (int32), like tree_attn_plan_export (buf NULL: query *count):
 *   FRAG_SEG_PTR      [F+1]  fragment f's segments are [ptr[f], ptr[f+1])
 *   FRAG_TOKEN_PTR    [F+1]  fragment f's tokens are [ptr[f], ptr[f+1])
 *   FRAG_SEG_PARENT   per segment: parent within its fragment, -1 for a root
 *   FRAG_SEG_LEN      per segment (a fragment's segments start at its token 0)
 *   FRAG_TOKEN_SOURCE per fragment token: its source token
 *   FRAG_TOKEN_OWNER  per fragment token: 1 owned, 0 repeated */
#define TREE_ATTN_FRAG_SEG_PTR 0
#define TREE_ATTN_FRAG_TOKEN_PTR 1
#define TREE_ATTN_FRAG_SEG_PARENT 2
#define TREE_ATTN_FRAG_SEG_LEN 3
#define TREE_ATTN_FRAG_TOKEN_SOURCE 4
#define TREE_ATTN_FRAG_TOKEN_OWNER 5
int tree_attn_fragments_export(tree_attn_fragments_t fragments, int32_t which, int32_t* buf, int64_t cap,
                               int64_t* count);

/*
 * Sampled-edge projection and loss (Megatron-LM pull request 7387, section
 * "Summary": edge-source hidden states are picked out before the vocabulary
 * projection; issue "Shared-prefix training with context parallelism for
 * exact agent trajectories", section "Describe the solution you'd like": a
 * single loss owner per sampled action).  An edge e is a sampled token tgt[e] (a vocabulary
 * index) predicted from the hidden state of token src[e]; only those states
 * go through the vocabulary head W [V, d]:
 *   logits[e] = W h[src[e]],  lse[e] = log sum_v exp(logits[e, v]),
 *   loss[e]   = lse[e] - logits[e, tgt[e]].
 * Backward, given dloss [E]: G[e] = (softmax(logits[e]) - onehot(tgt[e]))
 * dloss[e]; dh[t] = sum over edges with src = t of G[e] W (rows of tokens
 * that are no edge's source: 0); dW = sum_e G[e]^T h[src[e]].  A token may
 * be the source of several edges (a branch point).  h, W, dh, dW are bf16
 * row-major, 16-byte aligned, d a multiple of 8; loss, lse, dloss float32.
 * Deterministic (no atomics; library GEMMs with atomics disabled).
 *
 * tree_attn_edges validates the host arrays (0 <= src < num_tokens,
 * 0 <= tgt < vocab), groups the edges by source and uploads them to the
 * current device; the object is library-owned and immutable.
 * Errors: INVALID_ARGUMENT (NULL, out of range, small workspace, other
 * device), UNSUPPORTED (d not a multiple of 8, > 262,143 edges), HIP_ERROR.
 */
typedef struct tree_attn_edges_s* tree_attn_edges_t;
int tree_attn_edges(const int32_t* edge_src, const int32_t* edge_tgt, int32_t num_edges, int32_t num_tokens,
                    int32_t vocab, tree_attn_edges_t* out);
int tree_attn_edges_destroy(tree_attn_edges_t edges);
/* Device workspace bytes of the forward and backward for hidden size d. */
size_t tree_attn_edge_loss_workspace_bytes(tree_attn_edges_t edges, int32_t hidden);
/* Bytes of the optional saved logits: every logit as fp16, relative to its
 * vocabulary chunk's row maximum (about 2 E V bytes; caller-owned). */
size_t tree_attn_edge_loss_saved_bytes(tree_attn_edges_t edges);
/* loss, lse: [E] float32 outputs.  h: [num_tokens, d]; W: [vocab, d].
 * saved: NULL, or a buffer of tree_attn_edge_loss_saved_bytes the forward
 * fills so that the backward need not recompute the logits. */
int tree_attn_edge_loss_fwd(const void* hidden, const void* weight, int32_t hidden_dim, tree_attn_edges_t edges,
                            float* loss, float* lse, void* saved, size_t saved_bytes, void* workspace,
                            size_t workspace_bytes, void* stream);
/* lse from the forward; saved: the forward's saved logits for the same
 * inputs, or NULL (the logits are recomputed); dloss [E]; dhidden
 * [num_tokens, d] and dweight [vocab, d] are overwritten. */
int tree_attn_edge_loss_bwd(const void* hidden, const void* weight, int32_t hidden_dim, tree_attn_edges_t edges,
                            const float* lse, const void* saved, size_t saved_bytes, const float* dloss,
                            void* dhidden, void* dweight, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Mamba state forking on the same forests (draft "feat(hybrid): add opt-in
 * shared-prefix attention and Mamba execution", intro: the prompt head is
 * shared, recurrent state forks into each branch, the convolution halo is
 * handled per branch and backward accumulates the branches into the shared
 * prefix; issue "Shared-prefix training with context parallelism for exact
 * agent trajectories", section "Describe the solution you'd like": the
 * convolution and recurrent state at branch points stay differentiable).
 * prev(i) is the token before i on its root-to-leaf path: the previous token
 * of its segment, or the parent segment's last token for a segment's first
 * token, -1 at a root.  Two ops run along it (all tensors float32,
 * row-major, on the plan's device):
 *
 * Depthwise causal convolution, x, y, dy, dx: [T, channels], weight
 * [channels, width], bias [channels]:
 *   y[i, c] = bias[c] + sum_{j < width} weight[c, j] x[prev^(width-1-j)(i), c]
 * (terms past a root are zero).  channels a multiple of 4, width 1..4;
 * x, y, dy, dx, weight, bias 16-byte aligned.
 *
 * Selective state-space recurrence with a scalar decay per head (Mamba-2
 * form), x, y: [T, H, 64]; dt: [T, H] (positive step sizes, after any
 * softplus); A, D: [H]; B, C: [T, G, N]; head h reads group h / (H / G):
 *   S_i = exp(dt[i,h] A[h]) S_prev(i) + dt[i,h] x[i,h,:] outer B[i,g,:],  S_-1 = 0
 *   y[i,h,:] = S_i C[i,g,:] + D[h] x[i,h,:]
 * N = state_dim is 64 or 128; x, y, dy, dx, B, C 16-byte aligned.
 *
 * tree_attn_mamba_plan validates the forest (same rules as tree_attn_plan),
 * derives prev, the convolution halo and successor tables and the scan
 * units (segments cut into units of at most unit_tokens tokens), and
 * uploads them to the current device; _host builds the tables only (for
 * inspection).  The plan is library-owned and immutable.
 * Determinism: no atomics; results are bitwise reproducible.
 * Errors: INVALID_ARGUMENT (NULL, malformed forest, small buffers, other
 * device, host-only plan), UNSUPPORTED (shapes outside the above), HIP_ERROR.
 */
typedef struct tree_attn_mamba_plan_s* tree_attn_mamba_plan_t;
typedef struct {
  int32_t num_tokens, num_segments, num_units, unit_tokens, max_depth, max_conv_width;
} tree_attn_mamba_plan_info_t;
typedef struct {
  int32_t num_tokens; /* T: rows of x, dt, B, C, y; must equal the plan's token count */
  int32_t num_heads, head_dim, num_groups, state_dim;
} tree_attn_ssm_shape;
int tree_attn_mamba_plan(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                         int32_t num_segments, tree_attn_mamba_plan_t* out);
int tree_attn_mamba_plan_host(const int32_t* parent, const int32_t* seg_start, const int32_t* seg_len,
                              int32_t num_segments, tree_attn_mamba_plan_t* out);
int tree_attn_mamba_plan_destroy(tree_attn_mamba_plan_t plan);
int tree_attn_mamba_plan_info(tree_attn_mamba_plan_t plan, tree_attn_mamba_plan_info_t* info);
/* Host tables, int32: PREV [T]; UNIT_START, UNIT_LEN, UNIT_PRED [num_units]
 * (predecessor unit, -1 at a root).  buf NULL queries *count. */
#define TREE_ATTN_MAMBA_PREV 0
#define TREE_ATTN_MAMBA_UNIT_START 1
#define TREE_ATTN_MAMBA_UNIT_LEN 2
#define TREE_ATTN_MAMBA_UNIT_PRED 3
int tree_attn_mamba_plan_export(tree_attn_mamba_plan_t plan, int32_t which, int32_t* buf, int64_t cap,
                                int64_t* count);
/* Convolution forward: writes y.  num_tokens (the rows of x and y) must
 * equal the plan's token count, else INVALID_ARGUMENT before any launch. */
int tree_attn_conv_fwd(const float* x, const float* weight, const float* bias, int32_t num_tokens,
                       int32_t channels, int32_t width, tree_attn_mamba_plan_t plan, float* y, void* stream);
size_t tree_attn_conv_bwd_workspace_bytes(tree_attn_mamba_plan_t plan, int32_t channels, int32_t width);
/* Convolution backward of sum <dy, y>: overwrites dx, dweight, dbias.
 * num_tokens (rows of x, dy, dx) must equal the plan's token count. */
int tree_attn_conv_bwd(const float* x, const float* weight, const float* dy, int32_t num_tokens, int32_t channels,
                       int32_t width, tree_attn_mamba_plan_t plan, float* dx, float* dweight, float* dbias,
                       void* workspace, size_t workspace_bytes, void* stream);
/* Bytes of the saved states (the state before every 32-token chunk of every
 * scan unit, written by the forward for the backward) and of the forward's
 * workspace. */
size_t tree_attn_ssm_states_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape);
size_t tree_attn_ssm_workspace_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape);
/* Recurrence forward: writes y and the saved states. */
int tree_attn_ssm_fwd(const float* x, const float* dt, const float* A, const float* B, const float* C,
                      const float* D, tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape, float* y,
                      float* states, size_t states_bytes, void* workspace, size_t workspace_bytes, void* stream);
size_t tree_attn_ssm_bwd_workspace_bytes(tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape);
/* Recurrence backward of sum <dy, y> (every token counted once; the
 * gradient reaching a branch point's state is the sum over its branches):
 * overwrites dx [T, H, 64], ddt [T, H], dA [H], dB, dC [T, G, N], dD [H].
 * states: the forward's saved states for the same inputs. */
int tree_attn_ssm_bwd(const float* x, const float* dt, const float* A, const float* B, const float* C,
                      const float* D, const float* dy, tree_attn_mamba_plan_t plan, const tree_attn_ssm_shape* shape,
                      const float* states, size_t states_bytes, float* dx, float* ddt, float* dA, float* dB,
                      float* dC, float* dD, void* workspace, size_t workspace_bytes, void* stream);

/* Copy one of the plan's host tables (int32 records) for inspection.
 *   which = TREE_ATTN_EXPORT_*; buf may be NULL to query *count;
 *   cap = capacity of buf in int32 elements; *count = elements available.
 * Records: SPAN_PTR int32[S+1] (CSR offsets into SPANS, per segment);
 *          SPANS {phys_start, len, virt_start, 0} per span;
 *          Q_TILES {q0, nq, seg, pos0} per 32-token query tile;
 *          KV_TILES {k0, nk, seg, q_end} per 64-token key tile;
 *          SEG_DEPTH, SEG_PREFIX (ancestor tokens A(s)), SEG_END (one past
 *          the last token of the segment's subtree) int32[S]. */
#define TREE_ATTN_EXPORT_SPAN_PTR 0
#define TREE_ATTN_EXPORT_SPANS 1
#define TREE_ATTN_EXPORT_Q_TILES 2
#define TREE_ATTN_EXPORT_KV_TILES 3
#define TREE_ATTN_EXPORT_SEG_DEPTH 4
#define TREE_ATTN_EXPORT_SEG_PREFIX 5
#define TREE_ATTN_EXPORT_SEG_END 6
int tree_attn_plan_export(tree_attn_plan_t plan, int32_t which, int32_t* buf, int64_t cap, int64_t* count);

/*
 * Forward pass.  q, k, v: device tensors (THD, shape->dtype); out: device
 * [T, Hq, D] of the same dtype; lse: device float32 [Hq, T].  Overwrites out
 * and lse.  stream: a hipStream_t (NULL = default).  Asynchronous.
 * Errors: INVALID_ARGUMENT (null pointer, shape mismatch, host-only plan,
 * plan built on another device), UNSUPPORTED (dtype/head_dim, more than
 * 2^31 elements in a tensor, or K/V of 2^32 bytes or more), HIP_ERROR.
 * A segment's ancestor path may split into any number of token spans.
 */
int tree_attn_fwd(const void* q, const void* k, const void* v, tree_attn_plan_t plan,
                  const tree_attn_shape* shape, void* out, float* lse, void* stream);

/* Bytes of device workspace tree_attn_fwd_ws needs (work-item counters;
 * 256); 0 on invalid input. */
size_t tree_attn_fwd_workspace_bytes(tree_attn_plan_t plan, const tree_attn_shape* shape);

/*
 * tree_attn_fwd with a caller workspace of at least
 * tree_attn_fwd_workspace_bytes() (device memory, 16-byte aligned, any
 * contents).  The same results, bitwise: each output row is still computed
 * by one workgroup in a fixed order; the workspace only holds the counters
 * through which one workgroup per compute unit takes query tiles until none
 * is left (first from its own XCD's share, then from the others'), so the
 * eight XCDs' clock differences do not leave the slowest one finishing
 * alone.  The counters are zeroed by a one-workgroup launch at the start of
 * every call.  Calls that overlap on one workspace race.
 * Errors: as tree_attn_fwd, plus INVALID_ARGUMENT for a NULL, misaligned or
 * small workspace.
 */
int tree_attn_fwd_ws(const void* q, const void* k, const void* v, tree_attn_plan_t plan,
                     const tree_attn_shape* shape, void* out, float* lse, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Bytes of device workspace tree_attn_bwd needs for this plan and shape
 * (two float32 [Hq, T] row-statistic arrays, 256-byte aligned, then 128
 * bytes of work-item counters); 0 on invalid input. */
size_t tree_attn_bwd_workspace_bytes(tree_attn_plan_t plan, const tree_attn_shape* shape);

/*
 * Backward pass.  Inputs q, k, v, out, lse (from tree_attn_fwd) and dout;
 * outputs dq [T, Hq, D], dk, dv [T, Hkv, D] (same dtype as q), overwritten
 * (not accumulated into).  workspace: caller-owned device memory of at least
 * tree_attn_bwd_workspace_bytes().  Every output element is produced by one
 * workgroup in a fixed order, with no atomic accumulation (atomic counters
 * only decide which workgroup takes which tile), so results are bitwise
 * reproducible run to run.  Asynchronous on `stream`.
 * Errors: as tree_attn_fwd, plus INVALID_ARGUMENT for a small workspace.
 */
int tree_attn_bwd(const void* q, const void* k, const void* v, const void* out, const float* lse,
                  const void* dout, tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq,
                  void* dk, void* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The three stages tree_attn_bwd runs, in this order, on one stream; each can
 * be called on its own (for example to time it).  They share the workspace:
 *   tree_attn_bwd_rowstat  -delta[h,i] = -sum_d dout[i,h,d] * out[i,h,d] and
 *                          -lse[h,i] * log2(e) into the workspace (two float32
 *                          [Hq, T] arrays, stored negated), and zeroes the
 *                          work-item counters of the other two stages;
 *   tree_attn_bwd_dkdv     dk, dv: for each key, the contributions of every
 *                          query that sees it, i.e. of every branch below a
 *                          shared prefix (draft "feat(hybrid): add opt-in
 *                          shared-prefix attention and Mamba execution",
 *                          intro); needs the rowstat workspace;
 *   tree_attn_bwd_dq       dq; needs the rowstat workspace.
 * Called on its own, tree_attn_bwd_dkdv or _dq first zeroes its own
 * work-item counters with a one-workgroup launch, so it needs nothing from
 * the workspace but the row statistics.
 * Arguments, checks and errors are those of tree_attn_bwd.
 */
int tree_attn_bwd_rowstat(const void* out, const float* lse, const void* dout, tree_attn_plan_t plan,
                          const tree_attn_shape* shape, void* workspace, size_t workspace_bytes, void* stream);
int tree_attn_bwd_dkdv(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                       tree_attn_plan_t plan, const tree_attn_shape* shape, void* dk, void* dv, void* workspace,
                       size_t workspace_bytes, void* stream);
int tree_attn_bwd_dq(const void* q, const void* k, const void* v, const float* lse, const void* dout,
                     tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * tree_attn_bwd without a caller workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  The workspace is a fixed array
 * of 64 MiB + 256 bytes that the library holds on each GPU it runs on until
 * the process ends, so shapes with num_q_heads * total_tokens above
 * 8,388,608 are UNSUPPORTED (before any launch).  The call allocates
 * nothing.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other threads) race and must be
 * ordered by the caller.  Outputs, checks and determinism as tree_attn_bwd.
 */
int tree_attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* out, const float* lse,
                          const void* dout, tree_attn_plan_t plan, const tree_attn_shape* shape, void* dq, void* dk,
                          void* dv, void* stream);

/* Message of the last failed call on this thread ("" if none). */
const char* tree_attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* TREE_ATTN_H_ */
