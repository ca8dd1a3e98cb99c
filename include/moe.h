/*
 * moe.h -- one GPU's share of an expert-parallel mixture-of-experts layer,
 * forward and backward, as hand-written HIP kernels for MI355X (gfx950).
 *
 * The operation is the per-device step sequence of an MoE layer described
 * in "GPU expert parallel" (aicassindra.com), section "The step timeline":
 * the router scores every token, tokens are permuted into contiguous
 * per-expert buffers, each expert's FFN runs over its rows as one grouped
 * GEMM, and the inverse permutation restores token order; backward walks
 * the same path in reverse.  Top-k and the capacity factor (tokens beyond
 * an expert's capacity are dropped) follow the distributed-training
 * tutorial (deepseekmodel.com), section "The Capacity Factor" and its EP
 * configuration block.  The all-to-all exchanges and gradient reductions of
 * those pages span several GPUs and are not part of this library.
 *
 * Conventions for every entry point
 *  - Every tensor pointer is a DEVICE pointer owned by the caller.  The
 *    library never allocates, frees or synchronises; each call only
 *    enqueues kernels on `stream` (a hipStream_t; NULL = default stream).
 *  - Row-major, densely packed.  "s" is the activation/weight type given by
 *    cfg->dtype: float (MOE_FP32) or bfloat16 bits (MOE_BF16, uint16).
 *    Router probabilities, gates, gate gradients, dXe and db are float.
 *  - Arguments are validated before anything is enqueued.  On an error the
 *    call returns a negative moe_status, enqueues nothing and writes
 *    nothing.  Device-side faults surface at the caller's next sync.
 *  - Shapes: T >= 0, 1 <= k <= 32, k <= E <= 256, d >= 1, f >= 1, and
 *    d * sizeof(s) and f * sizeof(s) multiples of 16 bytes
 *    (MOE_ERR_ALIGN otherwise); every pointer 16-byte aligned.
 *  - R = number of kept (token, expert) assignments, known only on the
 *    device (offsets[E]).  Buffers with R rows are sized Rmax =
 *    moe_rows_max(cfg); rows in [R, Rmax) are left untouched.
 *  - Results are deterministic: identical inputs give bitwise identical
 *    outputs (no result depends on the order of atomic operations).
 *  - Non-finite inputs are outside the contract.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

/* The library is built with hidden visibility; only these entry points are
 * exported. */
#if defined(__GNUC__) || defined(__clang__)
#define MOE_API __attribute__((visibility("default")))
#else
#define MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_ARG = -1,            /* null pointer or out-of-range scalar */
  MOE_ERR_DTYPE = -2,          /* unknown cfg->dtype */
  MOE_ERR_SHAPE = -3,          /* inconsistent sizes */
  MOE_ERR_ALIGN = -4,          /* row or pointer not 16-byte aligned */
  MOE_ERR_WORKSPACE = -5,      /* ws_bytes < moe_workspace_bytes(cfg) */
  MOE_ERR_LAUNCH = -6,         /* a kernel launch failed */
  MOE_ERR_UNIMPLEMENTED = -7
} moe_status;

typedef enum { MOE_FP32 = 0, MOE_BF16 = 1 } moe_dtype;

#define MOE_NO_CAPACITY (-1)

/* moe_cfg.flags bits.
 * MOE_FLAG_RECOMPUTE: selective recomputation ("GPU expert parallel",
 * section "Recomputation re-runs the dispatch unless you save the
 * permutation": keep the routing map, drop the MLP hidden states).  The
 * forward keeps A and H only in the workspace (A is not stored at all) and
 * the backward recomputes them from x_perm with the same kernel, one extra
 * grouped GEMM; the A and H arguments of moe_grouped_ffn,
 * moe_grouped_ffn_bwd and moe_ctx are then ignored and may be NULL.
 * Results are bitwise those of the default mode; the saved state shrinks
 * by 2 Rmax f s bytes and the workspace grows by as much. */
#define MOE_FLAG_RECOMPUTE 1u
/* MOE_FLAG_RENORM: gates renormalised over the k selected experts,
 * gate[t,j] = p[t,idx_j] / sum_i p[t,idx_i] (sum in selection order, fp32),
 * before the capacity drop; the router backward differentiates through the
 * normalisation.  Without it the gates are the probabilities themselves.
 * The pages fix neither; top-k routing is used both ways. */
#define MOE_FLAG_RENORM 2u
/* MOE_FLAG_SLOT_PRIORITY: the capacity walk is slot-major -- every token's
 * first choice before any token's second choice, (j, t) in lexicographic
 * order -- instead of token-major (t, j); the rows of an expert in x_perm
 * follow the same order.  Which assignments of a full expert go first is
 * not fixed by the pages ("The Capacity Factor" only says the excess is
 * dropped). */
#define MOE_FLAG_SLOT_PRIORITY 4u
/* MOE_FLAG_DROP_IDENTITY: a dropped assignment takes the identity fallback
 * path -- the token passes the expert unchanged -- instead of contributing
 * nothing: it adds gate[t,j] * x[t] to out[t], and backward gate[t,j] *
 * dOut[t] to dX[t] with dgate[t,j] = <dOut[t], x[t]>.  "The Capacity
 * Factor" lets excess tokens take a fallback path without defining it; the
 * pass-through is the plainest one.  Under it, moe_combine and
 * moe_combine_bwd need x, and moe_unpermute_bwd needs gate and dOut. */
#define MOE_FLAG_DROP_IDENTITY 8u

/* hipStream_t, passed opaquely so that this header needs no HIP headers. */
typedef void* moe_stream_t;

/* Kernel timing for benchmarks, owned entirely by the caller (the library
 * keeps no state of its own).  When cfg->probe is set, each launch of kernel
 * `kernel_id` made by a call with that cfg is bracketed by hipEventRecord of
 * begin[count] and end[count] on the launch's stream, and count is
 * incremented, until count reaches capacity.  The events are hipEvent_t
 * handles the caller created; the library neither creates, waits on nor
 * reads them.  Calls that share one probe must not run concurrently.  Kernel
 * ids: moe_kernel_id below. */
typedef struct moe_probe {
  int32_t kernel_id;
  int32_t capacity;   /* entries of begin and end */
  int32_t count;      /* launches recorded so far */
  int32_t reserved_;  /* 0 */
  void** begin;       /* hipEvent_t[capacity] */
  void** end;         /* hipEvent_t[capacity] */
} moe_probe;

typedef struct moe_cfg {
  int64_t T;          /* tokens; for the expert-share use (a ragged batch
                         that arrives already permuted) the number of rows */
  int32_t d;          /* model dim */
  int32_t E;          /* experts held by this GPU */
  int32_t k;          /* experts per token (top-k) */
  int32_t f;          /* expert FFN hidden dim */
  int32_t dtype;      /* moe_dtype of x, Wr, W1, W2 and every s tensor */
  int64_t capacity;   /* per-expert capacity C >= 0, or MOE_NO_CAPACITY */
  float route_margin; /* router certification margin (logit units); <= 0
                         selects the default 1e-3.  See moe_route. */
  uint32_t flags;     /* MOE_FLAG_* bits; others must be 0 */
  float aux_coeff;    /* coefficient alpha >= 0 of the auxiliary
                         load-balancing loss (0 = none); see moe_router_aux.
                         When > 0, moe_route_bwd and moe_layer_bwd add its
                         gradient. */
  moe_probe* probe;   /* NULL, or kernel timing (see moe_probe) */
} moe_cfg;

/* Capacity of the capacity-factor rule: C = ceil(cf * T * k / E), exact.
 * cf is read as its shortest decimal that converts back to the same double
 * (so 1.1 means 11/10, not the binary value just above it) and the ceiling
 * is taken in integer arithmetic.  cf < 0, NaN or +infinity returns
 * MOE_NO_CAPACITY (no limit), as does a T*k that does not fit int64.  A C
 * above T*k is returned as T*k: like any C >= T, it keeps every
 * assignment.
 * Distributed-training tutorial, section "The Capacity Factor". */
MOE_API int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double cf);

/* Rmax = min(T*k, E*C) (T*k without a capacity); -1 on invalid cfg. */
MOE_API int64_t moe_rows_max(const moe_cfg* cfg);

/* Bytes of device workspace that any entry point taking `ws` needs for
 * this cfg (the layer entry points need the most; one buffer of this size
 * serves all of them).  0 on invalid cfg. */
MOE_API size_t moe_workspace_bytes(const moe_cfg* cfg);

/* Human-readable text of a moe_status (static storage). */
MOE_API const char* moe_status_str(int status);

/* Validates cfg alone (the checks every entry point starts with). */
MOE_API int moe_check_cfg(const moe_cfg* cfg);

/* Text naming the kernel and HIP error of this thread's last
 * MOE_ERR_LAUNCH ("" if none since the last entry-point call). */
MOE_API const char* moe_last_error(void);

/* ---------------------------------------------------------------- forward */

/* F1 router: every token gets a score per expert ("The step timeline");
 * the router is a small replicated parameter whose decisions must agree on
 * every rank ("Sharded by expert, replicated everywhere else").
 *   x [T,d] s, Wr [d,E] s, b [E] float (NULL = zero bias)
 *   probs [T,E] float  softmax over all E of z = x Wr + b
 *   idx   [T,k] int32  the k experts in order (z descending, expert index
 *                      ascending on equal z)
 *   gate  [T,k] float  probs[t, idx[t,j]] (renormalised over the k under
 *                      MOE_FLAG_RENORM)
 * Decisions follow the canonical logit RN_fp32(sum in fp64 + b): the fast
 * fp32 logits (bf16 MFMA products, fp32 sums) are used where the top-(k+1)
 * gaps exceed cfg->route_margin, and every logit that can change the
 * decision is recomputed in fp64 otherwise.  This equals deciding on the
 * canonical logits whenever each fast logit lies within margin/2 of its
 * canonical value.  That bound is not checked at run time (the parity
 * tests assert it on their workloads with the default margin); a larger
 * margin widens it at the cost of more fp64 rescoring.  Workspace: ws of
 * ws_bytes >= moe_workspace_bytes(cfg) (holds a transposed copy of Wr and
 * the fast logits). */
MOE_API int moe_route(const moe_cfg* cfg, const void* x, const void* Wr,
              const float* b, float* probs, int32_t* idx, float* gate,
              void* ws, size_t ws_bytes, moe_stream_t stream);

/* F2 permute with capacity drop: the routed tokens are laid out in one
 * contiguous buffer per expert ("The step timeline"); assignments beyond an
 * expert's capacity are dropped ("The Capacity Factor").  Assignments are kept in
 * token order: (t,j) is kept iff fewer than C earlier tokens chose expert
 * idx[t,j] (under MOE_FLAG_SLOT_PRIORITY: fewer than C earlier assignments
 * in slot-major order (j, t)); the rows of an expert follow that order.
 *   idx [T,k] int32 (each row k distinct experts in [0,E))
 *   counts  [E]   int32  routed assignments per expert, before the drop
 *   offsets [E+1] int32  exclusive scan of min(counts, C); offsets[E] = R
 *   row_of  [T,k] int32  row of (t,j) in x_perm, -1 if dropped
 *   src_of  [Rmax] int32 t*k + j of the assignment in each row
 *   x_perm  [Rmax,d] s   x_perm[r] = x[src_of[r] / k] (bitwise copy)
 * Workspace: ws of ws_bytes >= moe_workspace_bytes(cfg). */
MOE_API int moe_permute(const moe_cfg* cfg, const void* x, const int32_t* idx,
                int32_t* counts, int32_t* offsets, int32_t* row_of,
                int32_t* src_of, void* x_perm, void* ws, size_t ws_bytes,
                moe_stream_t stream);

/* moe_permute for callers that cannot allocate device memory -- code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc: the same kernels and results as moe_permute (bitwise), with
 * no workspace argument.  Its scratch (the per-block expert histograms,
 * ceil(T'/256) * E * 4 bytes with T' = T, or T*k under
 * MOE_FLAG_SLOT_PRIORITY) lives in a fixed 4 MiB device array that each
 * GPU the library runs on holds until the process ends; a cfg needing more
 * returns MOE_ERR_WORKSPACE (moe_last_error gives both sizes) before
 * anything is enqueued.  It never calls hipMalloc or hipFree.  The array is
 * the current device's, and every call on one GPU shares it: calls that
 * overlap on one GPU (different streams, or threads) race and must be
 * ordered by the caller.  Every entry is written before it is read, so a
 * call needs nothing cleared from the previous one. */
MOE_API int moe_permute_noalloc(const moe_cfg* cfg, const void* x, const int32_t* idx,
                int32_t* counts, int32_t* offsets, int32_t* row_of,
                int32_t* src_of, void* x_perm, moe_stream_t stream);

/* F3+F4 grouped expert FFN over the ragged per-expert segments
 * [offsets[e], offsets[e+1]) of x_perm: every local expert runs on the rows
 * routed to it, as one grouped GEMM rather than one small GEMM per expert
 * ("The step timeline").  fp32 accumulation; storage rounding RNE:
 *   A = x_perm W1[e]      [Rmax,f] s   (saved for backward)
 *   H = gelu_tanh(A)      [Rmax,f] s   (from the stored A)
 *   Y = H W2[e]           [Rmax,d] s
 * W1 [E,d,f] s, W2 [E,f,d] s.  offsets lives on the device and is never
 * read back by the host.  Under MOE_FLAG_RECOMPUTE, A and H are ignored
 * (H lives in the workspace).  Workspace as above. */
MOE_API int moe_grouped_ffn(const moe_cfg* cfg, const void* x_perm,
                    const int32_t* offsets, const void* W1, const void* W2,
                    void* A, void* H, void* Y, void* ws, size_t ws_bytes,
                    moe_stream_t stream);

/* F5 combine: the inverse of the permutation puts expert outputs back in
 * token order ("The step timeline"), weighted by the gates:
 *   out[t] = sum over kept j (ascending) of gate[t,j] * Y[row_of[t,j]],
 * fp32 accumulation, one rounding to s; 0 for a token with every
 * assignment dropped.  Under MOE_FLAG_DROP_IDENTITY a dropped j adds
 * gate[t,j] * x[t] in its place (x [T,d] s; otherwise x is unused and may
 * be NULL).  out [T,d] s. */
MOE_API int moe_combine(const moe_cfg* cfg, const void* Y, const int32_t* row_of,
                const float* gate, const void* x, void* out, moe_stream_t stream);

/* Routing diagnostics and the auxiliary load-balancing loss.  The
 * distributed-training tutorial (section "The Capacity Factor") adds a
 * balancing penalty that pulls the experts' token loads together
 * (coefficient 0.01 in its EP configuration block) and asks for the drop
 * rate and the expert load distribution to be watched.  The loss is the
 * standard balancing loss
 *   L = alpha * E * sum_e f_e P_e,  f_e = counts[e] / (T k),
 *   P_e = (1/T) sum_t probs[t, e],  alpha = cfg->aux_coeff
 *   aux[0] = L (0 when alpha = 0), aux[1] = drop rate 1 - offsets[E] / (T k)
 * The expert load distribution is counts itself.  probs [T,E] float,
 * counts [E] and offsets [E+1] int32 as written by moe_permute,
 * aux [2] float, all device.  fp32 sums in a fixed order (deterministic).
 * Workspace as above. */
MOE_API int moe_router_aux(const moe_cfg* cfg, const float* probs, const int32_t* counts,
                           const int32_t* offsets, float* aux, void* ws, size_t ws_bytes,
                           moe_stream_t stream);

/* --------------------------------------------------------------- backward
 * The backward pass retraces the forward steps in reverse order ("The step
 * timeline").  The
 * upstream gradient is dOut [T,d] s, i.e. L = <out, dOut>. */

/* B5 combine backward:
 *   dYp[row_of[t,j]] = RN_s(gate[t,j] * dOut[t])  [Rmax,d] s
 *   dgate[t,j]       = <dOut[t], Y[row_of[t,j]]>  [T,k] float (0 if dropped;
 *                      <dOut[t], x[t]> under MOE_FLAG_DROP_IDENTITY, which
 *                      needs x [T,d] s -- otherwise x may be NULL)
 */
MOE_API int moe_combine_bwd(const moe_cfg* cfg, const void* dOut, const void* Y,
                    const int32_t* row_of, const float* gate, const void* x,
                    void* dYp, float* dgate, moe_stream_t stream);

/* B4+B3 grouped expert FFN backward; per expert e over its rows (under
 * MOE_FLAG_RECOMPUTE, A and H are first recomputed from x_perm into the
 * workspace, and the A and H arguments are ignored):
 *   dH  = dYp W2[e]^T               (fp32, not stored)
 *   dA  = RN_s(dH * gelu_tanh'(A))  (stored in the workspace)
 *   dXp = dA W1[e]^T                [Rmax,d] s
 *   dW2[e] = H^T dYp                [E,f,d] s
 *   dW1[e] = x_perm^T dA            [E,d,f] s
 * Experts with no rows get dW1[e] = dW2[e] = 0.  Expert weights live only
 * on their owning rank and their gradients are reduced over the expert
 * data-parallel group ("Two gradient reductions over two different
 * groups"); that reduction spans GPUs and is the caller's.  Workspace as
 * above. */
MOE_API int moe_grouped_ffn_bwd(const moe_cfg* cfg, const void* x_perm,
                        const int32_t* offsets, const void* W1,
                        const void* W2, const void* A, const void* H,
                        const void* dYp, void* dXp, void* dW1, void* dW2,
                        void* ws, size_t ws_bytes, moe_stream_t stream);

/* B2 inverse of the permute for gradients:
 *   dXe[t] = sum over kept j of dXp[row_of[t,j]]   [T,d] float
 * plus gate[t,j] * dOut[t] for each dropped j under MOE_FLAG_DROP_IDENTITY
 * (gate [T,k] float and dOut [T,d] s; otherwise both may be NULL). */
MOE_API int moe_unpermute_bwd(const moe_cfg* cfg, const void* dXp,
                      const int32_t* row_of, const float* gate, const void* dOut,
                      float* dXe, moe_stream_t stream);

/* B1 router backward (the router is a shared parameter with an ordinary
 * gradient -- "Sharded by expert, replicated everywhere else"):
 *   dp[t, e] = a_e + (dgate[t,j] if e = idx[t,j] for a kept j)
 *       with a_e = alpha * E * counts[e] / (T k T), the gradient of the
 *       load-balancing loss (alpha = cfg->aux_coeff; a_e = 0 when alpha = 0);
 *       under MOE_FLAG_RENORM the gate term is instead
 *       (dgate[t,j] - sum_i g_i dgate[t,i]) / S for every selected j, with
 *       S = sum_i probs[t, idx[t,i]] and g_i = probs[t, idx[t,i]] / S
 *       (dgate of a dropped assignment counts as 0, except under
 *       MOE_FLAG_DROP_IDENTITY, where every assignment's dgate counts)
 *   dz  = probs * (dp - sum_e probs * dp)
 *   db  = sum_t dz                       [E] float (db may be NULL)
 *   dWr = x^T dz                         [d,E] s
 *   dX  = RN_s(dXe + dz Wr^T)            [T,d] s
 * dXe [T,d] float is the unpermute-sum written by moe_unpermute_bwd (which
 * already holds the identity fallback's terms).  counts [E] may be NULL
 * when cfg->aux_coeff == 0.  moe_layer_bwd computes the same dX with the
 * unpermute-sum fused in.  Workspace as above. */
MOE_API int moe_route_bwd(const moe_cfg* cfg, const void* x, const void* Wr,
                  const float* probs, const int32_t* idx, const int32_t* row_of,
                  const int32_t* counts, const float* dgate, const float* dXe,
                  void* dX, void* dWr, float* db, void* ws, size_t ws_bytes,
                  moe_stream_t stream);

/* ------------------------------------------------------------ whole layer */

typedef struct moe_weights {
  const void* Wr;   /* [d,E] s */
  const float* b;   /* [E] float, NULL = zero */
  const void* W1;   /* [E,d,f] s */
  const void* W2;   /* [E,f,d] s */
} moe_weights;

/* Saved forward state, all caller-owned device buffers.  The small integer
 * routing map is kept and reused by backward instead of routing again
 * (section "Recomputation re-runs the dispatch unless you save the
 * permutation").  A and H may be NULL under MOE_FLAG_RECOMPUTE. */
typedef struct moe_ctx {
  float* probs;     /* [T,E] float */
  int32_t* idx;     /* [T,k] */
  float* gate;      /* [T,k] float */
  int32_t* counts;  /* [E] */
  int32_t* offsets; /* [E+1] */
  int32_t* row_of;  /* [T,k] */
  int32_t* src_of;  /* [Rmax] */
  void* x_perm;     /* [Rmax,d] s */
  void* A;          /* [Rmax,f] s */
  void* H;          /* [Rmax,f] s */
  void* Y;          /* [Rmax,d] s */
  float* aux;       /* [2] float or NULL: routing diagnostics written by
                       moe_layer_fwd, as by moe_router_aux */
} moe_ctx;

typedef struct moe_grads {
  void* dWr;        /* [d,E] s */
  float* db;        /* [E] float (may be NULL) */
  void* dW1;        /* [E,d,f] s */
  void* dW2;        /* [E,f,d] s */
} moe_grads;

/* Forward of the layer: moe_route, moe_permute, moe_grouped_ffn and
 * moe_combine in sequence on `stream`; out [T,d] s. */
MOE_API int moe_layer_fwd(const moe_cfg* cfg, const moe_weights* w, const void* x,
                  void* out, const moe_ctx* ctx, void* ws, size_t ws_bytes,
                  moe_stream_t stream);

/* Backward of the layer from the saved ctx: moe_combine_bwd,
 * moe_grouped_ffn_bwd and moe_route_bwd (dYp, dA, dXp and dgate live in
 * the workspace); dX [T,d] s. */
MOE_API int moe_layer_bwd(const moe_cfg* cfg, const moe_weights* w, const void* x,
                  const void* dOut, const moe_ctx* ctx, void* dX,
                  const moe_grads* g, void* ws, size_t ws_bytes,
                  moe_stream_t stream);

/* ----------------------------------------------------------- kernel ids
 * Values of moe_probe.kernel_id. */
typedef enum {
  MOE_KERNEL_ROUTE = 0,          /* softmax, top-k, certification */
  MOE_KERNEL_PERMUTE_COUNT = 1,
  MOE_KERNEL_PERMUTE_SCAN = 2,
  MOE_KERNEL_PERMUTE_SCATTER = 3,
  MOE_KERNEL_GEMM_UP = 4,        /* A = x_perm W1, H = gelu(A) */
  MOE_KERNEL_GEMM_DOWN = 5,      /* Y = H W2 */
  MOE_KERNEL_COMBINE = 6,
  MOE_KERNEL_COMBINE_BWD = 7,
  MOE_KERNEL_GEMM_DH = 8,        /* dA = (dYp W2^T) * gelu'(A) */
  MOE_KERNEL_GEMM_DX = 9,        /* dXp = dA W1^T */
  MOE_KERNEL_GEMM_DW2 = 10,      /* dW2 = H^T dYp */
  MOE_KERNEL_GEMM_DW1 = 11,      /* dW1 = x_perm^T dA */
  MOE_KERNEL_UNPERMUTE_BWD = 12,
  MOE_KERNEL_ROUTE_BWD_DZ = 13,
  MOE_KERNEL_ROUTE_BWD_DX = 14,
  MOE_KERNEL_ROUTE_BWD_DW = 15,
  MOE_KERNEL_SCHEDULE = 16,
  MOE_KERNEL_ROUTE_PREP = 17,    /* router weight transpose / stacking */
  MOE_KERNEL_PERMUTE_COPY = 18,  /* x -> x_perm row copy */
  MOE_KERNEL_ROUTE_LOGITS = 19,  /* fast router logits x Wr (GEMM) */
  MOE_KERNEL_ROUTE_AUX = 20,     /* load-balancing loss and drop rate */
  MOE_KERNEL_GEMM_RECOMPUTE = 21, /* A, H recomputed in backward (MOE_FLAG_RECOMPUTE) */
  MOE_KERNEL_GEMM_FIXUP = 22,    /* split-K tail sums of any row GEMM */
  MOE_KERNEL_COUNT_ = 23
} moe_kernel_id;

#ifdef __cplusplus
}
#endif

#endif /* MOE_H_ */
