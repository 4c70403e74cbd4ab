/*
 * libgdr -- chunked training of gated delta-rule linear attention on AMD
 * MI355X (gfx950): Kimi Delta Attention (KDA, per-channel log-gate) and Gated
 * DeltaNet (GDN, scalar log-decay with grouped Q/K heads), over packed
 * variable-length sequences at head dim 128.
 *
 * What the calls compute.  The FlashInfer pull-request pages this library is
 * built from name the operation and its operands but print no formula:
 *   - PR #8218 (description, workload paragraph): KDA training over one packed
 *     batch described by cu_seqlens; q, k, v BF16 [T,H,128] (q, k
 *     L2-normalised by the caller), g an FP32 pre-activated log-gate
 *     [T,H,128], beta BF16 [T,H]; no in-kernel norm, gate or beta activation;
 *     ops fwd, bwd and ckpt (= forward, recompute and backward);
 *   - PR #7723 (description): the GDN form -- BF16 q/k/v/out/dout, FP32 scalar
 *     log-decay g and beta, grouped Q/K heads (H_qk, H_v), dq/dk reduced in
 *     FP32 over the value heads of each Q/K head and converted once.
 * The recurrence taken here (per document n and value head j; Q/K head
 * i = j / (H_v / H_qk); the state restarts at every document start):
 *     S_0 = h0[n,j] (zeros when h0 is NULL)
 *     S_t = (I - beta_t k_t k_t^T) Diag(exp(g_t)) S_{t-1} + beta_t k_t v_t^T
 *     o_t = scale * S_t^T q_t                    ht[n,j] = S at the last token
 * with exp(g_t) a 128-vector (KDA) or a scalar (GDN).  The backward returns
 * the gradients of  sum(o * dout) + sum(ht * dht).
 *
 * Conventions for every call below:
 *   - All tensor pointers are device pointers to caller-owned, contiguous,
 *     row-major buffers with no padding.  bf16 tensors are passed as uint16_t
 *     bit patterns.  Token-major layouts: q, k [T, H_qk, K]; v, o, dout
 *     [T, H_v, V]; states h0, ht, dht, dh0 [N, H_v, K, V] (fp32, K index first).
 *   - The library never allocates, frees or synchronises: every kernel is
 *     enqueued on `stream` (a hipStream_t; NULL = the default stream) in call
 *     order, and the call returns without waiting for the GPU.
 *   - All argument checks run on the host before anything is enqueued.  A call
 *     that returns an error has enqueued nothing and left every output
 *     untouched.  GDR_ERR_HIP reports a launch failure after validation.
 *   - The workspace is caller-owned device memory of at least
 *     gdr_workspace_bytes(...) bytes, 256-byte aligned.  Its contents on entry
 *     do not matter.  A backward call reads what the immediately preceding
 *     forward with GDR_FWD_SAVE, on the same stream and the same workspace and
 *     problem, left there; this pairing is the caller's contract and is not
 *     checked on the device.
 *   - Outputs must not alias inputs or the workspace.
 *   - Precondition: g >= -8 element-wise (the kernels evaluate
 *     exp(+-(G_r - G_ref)) within 16-row blocks, which stays finite in fp32
 *     under that bound; the pages' gates lie in (-5, 0)).  Not checked.
 *   - Status codes are plain int32 (enum gdr_status).  gdr_last_error()
 *     returns a thread-local message for the last failing call on this thread.
 */
#ifndef GDR_H
#define GDR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gdr_status {
  GDR_OK = 0,
  GDR_ERR_INVALID_ARG = 1, /* NULL pointer, negative size, inconsistent table, ... */
  GDR_ERR_UNSUPPORTED = 2, /* K != 128, V != 128, KDA with H_qk != H_v, GDN with H_v % H_qk != 0,
                              H_v > 65536, N * H_v > 2^27 or n_chunks * H_v >= 2^31 */
  GDR_ERR_WORKSPACE = 3,   /* workspace smaller than required or not 256-byte aligned */
  GDR_ERR_HIP = 4,         /* a HIP runtime call or kernel launch failed */
  GDR_ERR_ARCH = 5         /* the current device is not gfx950 */
};

enum gdr_variant { GDR_KDA = 0, GDR_GDN = 1 };

/* Forward flag: also write the tapes a later backward reads (per-chunk
 * entering states, new values and the backward walk's chunk factors).
 * Without it the forward writes only o and ht (the first forward of a
 * checkpointed step). */
#define GDR_FWD_SAVE 1u
/* Forward without the output: o is neither computed nor written (it may be
 * NULL) and prep skips the output's operands.  With GDR_FWD_SAVE this is the
 * recompute of a checkpointed step whose tapes the backward then reads, the
 * output being already known (PR #8638 description: the checkpoint recompute
 * hands its tapes to the backward instead of the backward re-running prep and
 * the state walk).  ht is still written when non-NULL. */
#define GDR_FWD_SKIP_OUTPUT 2u

/* One packed problem.  Lifetime: read during the call that receives it. */
typedef struct gdr_problem {
  int32_t T;     /* total tokens of the packed batch, >= 0 */
  int32_t N;     /* documents, >= 0 */
  int32_t H_qk;  /* Q/K heads (KDA: == H_v) */
  int32_t H_v;   /* value heads (GDN: multiple of H_qk) */
  int32_t K;     /* key dim, must be 128 */
  int32_t V;     /* value dim, must be 128 */
  const uint16_t *q;         /* bf16 [T, H_qk, K] */
  const uint16_t *k;         /* bf16 [T, H_qk, K] */
  const uint16_t *v;         /* bf16 [T, H_v, V] */
  const float *g;            /* KDA: fp32 [T, H_v, K]; GDN: fp32 [T, H_v] (log-decay) */
  const void *beta;          /* KDA: bf16 [T, H_v]; GDN: fp32 [T, H_v] */
  const int32_t *cu_seqlens; /* device int32 [N+1], cu[0] = 0, non-decreasing, cu[N] = T */
  const int32_t *chunk_table;/* device copy of the table gdr_plan_chunks built from the same cu_seqlens */
  int32_t n_chunks;          /* the n_chunks gdr_plan_chunks returned for it */
  const float *h0;           /* fp32 [N, H_v, K, V] initial states, or NULL for zeros */
  float scale;               /* output scale; 1/sqrt(128) in every workload of the pages */
  uint32_t input_flags;      /* GDR_IN_* bits below; 0 = q, k, beta used as given */
  int32_t walk_segments;     /* segments per document of the state walks: 0 = automatic (see
                                gdr_workspace_bytes), n >= 1 = at most n and at most the automatic count */
  int32_t max_doc_chunks;    /* chunks of the longest document (the largest step of the table's
                                per-document first-chunk section), or 0 = unknown (taken as n_chunks).
                                A hint for the walks' launch layout: results never depend on it */
  int32_t walk_layout;       /* GDR_WALK_AUTO, GDR_WALK_SLICES or GDR_WALK_RINGS (below) */
  int32_t walk_plan;         /* GDR_PLAN_BALANCED (0) or GDR_PLAN_EQUAL: how segmented walks share
                                their segments among the documents (below) */
} gdr_problem;

/* Segment plan of segmented walks (gdr_problem.walk_plan).  Segmenting engages
 * when the walks' chains leave the compute units underfilled (see
 * gdr_workspace_bytes): with P segments per document on average, the pack gets
 * P * N segments per value head in all.
 * GDR_PLAN_EQUAL: every document gets min(P, its chunks) segments.
 * GDR_PLAN_BALANCED: document d of n_d chunks gets ceil(n_d / L) segments (at
 *   most 2P, 8 and n_d, at least one), L being the smallest segment length for
 *   which the pack's segments stay within P * N: the longest segment, which
 *   sets the walks' critical path, is as short as that budget allows (the
 *   pages' longest-processing-time segment rule, PR #7723 description, solves
 *   the same balance per rank).  With one document the two plans agree.
 * Results differ between plans only by fp32 rounding of the carries. */
#define GDR_PLAN_BALANCED 0
#define GDR_PLAN_EQUAL 1

/* Launch layout of the state walks (gdr_problem.walk_layout).  Both run the same
 * products in the same order for every 16-column slice of the state, so they
 * give the same bits.
 * GDR_WALK_SLICES: one wavefront per (chain, slice), each reading the chain's
 *   per-chunk operands through its own memory pipeline: the shortest chain step,
 *   but a compute unit retires about one slice step at a time.
 * GDR_WALK_RINGS: the slice wavefronts of a chain in workgroups of four that
 *   pass each chunk's shared operands through an LDS ring of two slots (forward
 *   walk 97 KB, adjoint walk 113 KB): a longer chain step, about four times the
 *   work per compute unit.
 * GDR_WALK_AUTO: the layout with the smaller estimated walk time, from the
 *   longest chain (max_doc_chunks) and the work per compute unit; segmented
 *   walks (see walk_segments) always use slices. */
#define GDR_WALK_AUTO 0
#define GDR_WALK_SLICES 1
#define GDR_WALK_RINGS 2

/* Input activations applied inside the kernels (gdr_problem.input_flags).
 * GDR_IN_QK_L2NORM: every (token, head) row of q and of k is scaled to unit L2
 * norm, x * (sum x^2 + 1e-6)^(-1/2), before use (PR #8638 shapes paragraph);
 * dq and dk are then gradients with respect to the raw rows.
 * GDR_IN_BETA_SIGMOID: beta holds logits; the kernels use sigmoid(beta) and
 * dbeta is the gradient with respect to the logits.
 * The forward and backward of one problem must use the same flags. */
#define GDR_IN_QK_L2NORM 1u
#define GDR_IN_BETA_SIGMOID 2u

/* Chunk planner (host only).  Splits every document of cu_seqlens into
 * 64-token chunks (the last one of a document may be shorter; chunks never
 * straddle documents) and orders the documents for the state walks, longest
 * first.  The pages' kernels walk such a table of chunks and chunk lengths
 * (PR #7723 description: the adjoint walk keeps its chunk table in a
 * shared-memory ring; its sequence diagram publishes the chunk lengths) over
 * one packed batch given by cu_seqlens (PR #8218, workload paragraph).  Table
 * layout (int32), NC = n_chunks:
 *     [0, NC)             first token of each chunk
 *     [NC, 2NC)           tokens in each chunk (1..64)
 *     [2NC, 3NC)          document of each chunk
 *     [3NC, 3NC+N+1)      first chunk of each document (prefix, last = NC)
 *     [3NC+N+1, 3NC+2N+1) documents by descending chunk count (ties: lower index first)
 * cu_seqlens_host: host int32 [N+1].  table_host: host buffer of `capacity`
 * int32 entries, or NULL to only query the sizes.  Writes n_chunks_out and
 * table_len_out (both may be NULL).  Errors: GDR_ERR_INVALID_ARG for a bad
 * cu_seqlens, or a non-NULL table smaller than table_len. */
int32_t gdr_plan_chunks(const int32_t *cu_seqlens_host, int32_t N, int32_t *table_host,
                        int64_t capacity, int32_t *n_chunks_out, int64_t *table_len_out);

/* Workspace bytes for a problem (host only), the counterpart of the pages'
 * workspace helpers that size the caller-held arena (PR #8218 description:
 * every facade entry, the workspace helpers included; PR #8638 description of
 * the change: workspace accounting).  flags = 0: forward without
 * tapes; flags = GDR_FWD_SAVE: forward with tapes followed by a backward (the
 * size every backward needs).  When the walks' chains (documents x value
 * heads, 8 wavefronts each) number fewer than 512 wavefronts and some document
 * spans two chunks (n_chunks > N), each document's walk is split into
 * P = min(4, 512 / (8 N H_v)) segments run in parallel
 * (the segments' affine carries, 2 x 64 KB per segment boundary and value
 * head, are part of the workspace, sized for the balanced plan's cap: up to
 * min(8, 2P) segments per document).  Returns the byte count (a multiple of 256), or
 * minus a gdr_status on invalid or unsupported sizes. */
int64_t gdr_workspace_bytes(int32_t variant, int32_t T, int32_t N, int32_t n_chunks,
                            int32_t H_qk, int32_t H_v, int32_t K, int32_t V, uint32_t flags);

/* KDA forward.  o: bf16 [T, H_v, V] (written; NULL allowed with
 * GDR_FWD_SKIP_OUTPUT).  ht: fp32 [N, H_v, K, V] final states, or NULL to
 * skip.  flags: GDR_FWD_SAVE and/or GDR_FWD_SKIP_OUTPUT. */
int32_t gdr_kda_fwd(const gdr_problem *p, uint16_t *o, float *ht, void *workspace,
                    int64_t workspace_bytes, uint32_t flags, void *stream);

/* KDA backward (after gdr_kda_fwd(..., GDR_FWD_SAVE) on the same workspace).
 * dout: bf16 [T, H_v, V].  dht: fp32 [N, H_v, K, V] or NULL (= zeros).
 * Writes dq, dk: bf16 [T, H_qk, K]; dv: bf16 [T, H_v, V]; dg: fp32
 * [T, H_v, K]; dbeta: bf16 [T, H_v]; dh0: fp32 [N, H_v, K, V] (NULL to skip;
 * it is the gradient with respect to h0, also when h0 is NULL). */
int32_t gdr_kda_bwd(const gdr_problem *p, const uint16_t *dout, const float *dht, uint16_t *dq,
                    uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* GDN forward: as gdr_kda_fwd with g fp32 [T, H_v] and beta fp32 [T, H_v]. */
int32_t gdr_gdn_fwd(const gdr_problem *p, uint16_t *o, float *ht, void *workspace,
                    int64_t workspace_bytes, uint32_t flags, void *stream);

/* GDN backward: as gdr_kda_bwd, except dg is fp32 [T, H_v], dbeta is fp32
 * [T, H_v], and dq, dk [T, H_qk, K] are the fp32 sums over each Q/K head's
 * value heads, rounded to bf16 once. */
int32_t gdr_gdn_bwd(const gdr_problem *p, const uint16_t *dout, const float *dht, uint16_t *dq,
                    uint16_t *dk, uint16_t *dv, float *dg, void *dbeta, float *dh0,
                    void *workspace, int64_t workspace_bytes, void *stream);

/* The checkpointed training step as one call (PR #8218 ops paragraph, "ckpt":
 * forward, recompute and backward): forward without tapes (writes o, ht), the
 * recompute with GDR_FWD_SAVE | GDR_FWD_SKIP_OUTPUT (tapes only), then the
 * backward on the recompute's tapes (PR #8638 description: the recompute hands
 * its tapes to the backward, outputs and gradients bitwise unchanged).  Arguments as in the fwd and
 * bwd calls of the variant; the workspace must hold gdr_workspace_bytes(...,
 * GDR_FWD_SAVE). */
int32_t gdr_kda_ckpt(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout,
                     const float *dht, uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg,
                     void *dbeta, float *dh0, void *workspace, int64_t workspace_bytes,
                     void *stream);
int32_t gdr_gdn_ckpt(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout,
                     const float *dht, uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg,
                     void *dbeta, float *dh0, void *workspace, int64_t workspace_bytes,
                     void *stream);

/* gdr_kda_ckpt without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The workspace is a static device array inside the
 * library of GDR_NOALLOC_SCRATCH_BYTES bytes: every device the library runs
 * on holds its own copy from the library's load until the process ends.  The
 * call allocates nothing (no hipMalloc, no hipFree) and, like every call here,
 * does not synchronise.  Its address is looked up once per device, on the
 * first call with that device current.
 *   - Problems whose gdr_workspace_bytes(GDR_KDA, ..., GDR_FWD_SAVE) exceeds
 *     GDR_NOALLOC_SCRATCH_BYTES are rejected with GDR_ERR_WORKSPACE before
 *     anything is enqueued (64 MiB holds about 320 chunk-heads: e.g. 20 K
 *     tokens at one head or 5 K tokens at four).
 *   - Every call on one device uses that device's one array, which keeps the
 *     last call's contents (nothing in it has to start at zero).  Calls that
 *     overlap on one device (other streams, other host threads) race and give
 *     undefined results; calls ordered on one stream are safe.
 * Other arguments, outputs and errors as gdr_kda_ckpt. */
#define GDR_NOALLOC_SCRATCH_BYTES (64ll << 20)
int32_t gdr_kda_ckpt_noalloc(const gdr_problem *p, uint16_t *o, float *ht, const uint16_t *dout,
                             const float *dht, uint16_t *dq, uint16_t *dk, uint16_t *dv, float *dg,
                             void *dbeta, float *dh0, void *stream);

/* Kernel timing (diagnostics).  gdr_timing_enable(1) makes every later call
 * bracket each of its kernel launches with a pair of hipEvents recorded on the
 * call's stream (the events are created on first use and reused; this is the
 * one place where the library creates runtime objects).  gdr_timing_read
 * waits for the recorded events, adds their elapsed times to per-kernel
 * totals, writes up to `capacity` entries (kernel name, total milliseconds,
 * number of launches) and, with reset != 0, clears the totals.  Kernel names:
 * "fwd_prep", "fwd_walk", "bwd_walk", "bwd_grad".  Not thread-safe with
 * respect to concurrent calls that are being timed. */
int32_t gdr_timing_enable(int32_t on);
int32_t gdr_timing_read(const char **names, double *total_ms, int64_t *launches, int32_t capacity,
                        int32_t *count, int32_t reset);

/* Launch layout the state walks of problem *p (variant GDR_KDA or GDR_GDN) take
 * on a device with `compute_units` compute units (0: the current device, 256 if
 * none can be queried): writes GDR_WALK_SLICES or GDR_WALK_RINGS to *layout.
 * Host only; the problem is validated as by the forward, and no device call is
 * made when compute_units > 0.  GDR_ERR_INVALID_ARG for a NULL layout or a
 * negative unit count. */
int32_t gdr_walk_layout_chosen(int32_t variant, const gdr_problem *p, int32_t compute_units, int32_t *layout);

/* Returns GDR_OK when the current HIP device is gfx950, else GDR_ERR_ARCH
 * (GDR_ERR_HIP when no device can be queried). */
int32_t gdr_check_device(void);

/* Static description of a status code (never NULL). */
const char *gdr_status_string(int32_t status);

/* Thread-local detail for the last failing call on this thread ("" if none). */
const char *gdr_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* GDR_H */
