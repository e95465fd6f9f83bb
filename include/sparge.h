/*
 * sparge.h -- C ABI of libsparge.so: block-sparse, optionally 8-bit-quantized
 * attention with an on-the-fly block-mask predictor (SpargeAttn), for AMD
 * Instinct MI355X (gfx950).
 *
 * Page legend for citations:
 *   [topgit]     "SpargeAttn: accelerate LLM inference without training" (topgit.dev)
 *   [readme]     "Sparge Attention" (GitHub README mirror, git.1-hub.cn)
 *   [chapterpal] "SpargeAttention: Accurate and Training-free Sparse Attention
 *                Accelerating Any Model Inference" (chapterpal.com summary)
 *   [gittools]   "SpargeAttention" (Chinese README mirror, gittoolsai.com)
 *   [abstract]   the paper abstract on codewithpapers.app
 *
 * Conventions shared by every entry point
 *   - Tensors are described by sparge_tensor: logical shape (B, H, N, D) as in
 *     torch's scaled_dot_product_attention ("drop-in replacement" for it,
 *     [topgit] "Key features"), element strides for B, H and N, and a unit stride
 *     for D.  Row starts and the data pointer must be 16-byte aligned, and the N
 *     stride must stay below 64 MiB (the attention kernel addresses a 64-row block
 *     with 32-bit offsets); otherwise SPARGE_E_UNSUPPORTED.
 *   - q, k, v and out share one dtype and one (B, H, N, D); D is 64 or 128;
 *     1 <= N <= 262144.  fp32 inputs are read exactly by the predictor and rounded to
 *     bfloat16 for the attention products; out is written in the input dtype.
 *   - All pointers in sparge_tensor, masks, workspaces and permutations are
 *     DEVICE pointers owned by the caller, unless a comment says "host".  The
 *     library allocates nothing and keeps no state between calls; calls are
 *     thread-safe (calls sharing one workspace must be ordered on one stream).
 *   - Every argument is validated before any work is queued; on error nothing is
 *     launched and the status says why.  Work is queued on `stream` (a
 *     hipStream_t; NULL = the default stream) and runs asynchronously; a status of
 *     SPARGE_OK means the launches were queued.  The only synchronising case is a
 *     non-NULL sparge_opts.stats, documented there.
 *   - A failing HIP launch returns SPARGE_E_HIP; no exception crosses the ABI.
 */
#ifndef SPARGE_H
#define SPARGE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SPARGE_OK = 0,
  SPARGE_E_NULL = -1,        /* a required pointer is NULL */
  SPARGE_E_SHAPE = -2,       /* shapes disagree, D not in {64, 128}, or N outside [1, 262144] */
  SPARGE_E_DTYPE = -3,       /* unknown dtype or dtypes disagree */
  SPARGE_E_ARG = -4,         /* a scalar argument is out of range */
  SPARGE_E_UNSUPPORTED = -5, /* strides / alignment the kernels do not handle */
  SPARGE_E_WORKSPACE = -6,   /* workspace NULL or smaller than required */
  SPARGE_E_HIP = -7          /* a HIP runtime call or kernel launch failed */
} sparge_status;

typedef enum { SPARGE_F32 = 0, SPARGE_F16 = 1, SPARGE_BF16 = 2 } sparge_dtype;

typedef struct {
  void* data;        /* device pointer to element (0, 0, 0, 0) */
  int32_t dtype;     /* sparge_dtype */
  int32_t reserved;  /* must be 0 */
  int64_t B, H, N, D;
  int64_t sB, sH, sN; /* element strides; the D stride is 1 */
} sparge_tensor;

/* Counters filled when sparge_opts.stats is non-NULL (host memory). */
typedef struct {
  uint64_t valid_blocks;    /* (b, h, i, j) blocks holding at least one allowed pair */
  uint64_t kept_blocks;     /* blocks the mask keeps */
  uint64_t group_updates;   /* (32-row group, kept block) pairs visited by the kernel */
  uint64_t skipped_updates; /* of those, dropped by the softmax-aware filter */
} sparge_stats;

typedef struct {
  double scale;          /* softmax scale; 0 means 1/sqrt(D) as in SDPA */
  double sim_threshold;  /* block self-similarity threshold theta (default 0.1):
                            Q/K blocks with mean cosine similarity below it are
                            always computed ([chapterpal] method paragraph) */
  double filter_lambda;  /* softmax-aware filter threshold in natural-log logit
                            units (default -10): a kept block is dropped for a
                            32-row group when every row's block max sits more
                            than |lambda| below its running max ([chapterpal]
                            method paragraph; [abstract]) */
  int32_t filter_on;     /* sparge_topk_attn default 1; block_sparse_attn default 0 */
  int32_t qk_int8;       /* 1: int8 Q K^T (SageAttention base, [topgit] "Key
                            features"): Q one scale per 32 rows, K mean-smoothed and
                            scaled per 64-row block, the block mean added back as
                            a q.kbar term (computed to ~2^-16 of |q| |kbar| from
                            two-level int8 codes).  Default 0 (16-bit Q K^T). */
  int32_t pv_fp16;       /* 1: P and V rounded to fp16 for P.V; 0: the input's
                            16-bit type (bfloat16 for fp32 inputs).  Default 0. */
  int32_t pv_fp8;        /* 1: P.V in OCP FP8 E4M3 (the 8-bit-float P.V of the
                            SageAttention2 base, [readme] "Installation" fp8
                            requirements; [topgit] "Key features"): V one fp32
                            scale per (b, h, channel) over the sequence, codes
                            e4m3(v * 448 / max|v|); each softmax numerator rounded
                            to E4M3 and the row normaliser summed over the
                            rounded numerators; fp32 accumulation.  16-bit inputs
                            only (SPARGE_E_UNSUPPORTED for fp32); may not be
                            combined with pv_fp16 (SPARGE_E_ARG).  Default 0. */
  uint8_t* mask_out;     /* optional device (B, H, ceil(N/128), ceil(N/64)) uint8:
                            receives the predicted 0/1 block mask */
  sparge_stats* stats;   /* optional HOST pointer; when set the call waits for the
                            stream to finish and fills the counters */
  void* prof_start;      /* optional hipEvent_t recorded on `stream` when the call's
                            first launch is queued (profiling; NULL = none) */
  void* prof_attn_begin; /* optional hipEvent_t recorded right before the attention
                            kernel's launch */
  void* prof_attn_end;   /* optional hipEvent_t recorded right after it */
  /* Per-head knobs ([chapterpal] recommendations: calibrate the thresholds per layer
   * and attention head).  Each is an optional HOST array of H values (H of the
   * call's tensors, shared by every batch entry) that replaces the scalar for head
   * h; NULL keeps the scalar.  Values are validated like the scalars (SPARGE_E_ARG)
   * and copied into the workspace before the call returns. */
  const double* head_select;        /* topk of sparge_topk_attn / sparge_predict_mask,
                                       cdf_threshold of sparge_cdf_attn: each in (0, 1] */
  const double* head_sim_threshold; /* theta per head (not NaN) */
  const double* head_filter_lambda; /* lambda per head (<= 0, not NaN) */
} sparge_opts;

/* Fills *opts with the defaults listed above (filter_on = 1). */
void sparge_default_opts(sparge_opts* opts);

/* Workspace bytes that sparge_topk_attn, sparge_cdf_attn, block_sparse_attn,
 * sparge_predict_mask and sparge_quantize_qk need for tensors of this shape and dtype under `opts`
 * (NULL = defaults).  Returns 0 when the shape or dtype is invalid.  The value
 * is an upper bound for every entry point, so one workspace serves them all. */
size_t sparge_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t dtype,
                              const sparge_opts* opts);

/* Plug-and-play sparse attention: spas_sage2_attn_meansim_topk_cuda(q, k, v,
 * topk, is_causal) of [topgit] "Using the plug-and-play API" and [gittools]
 * recommended-API section.  Stage 1 predicts a (B, H, ceil(N/128), ceil(N/64))
 * block mask on the fly (block means of Q and K, the self-similarity gate, the
 * compressed attention map and a per-row top-k keeping the fraction `topk` of
 * the row's candidate blocks, [chapterpal] method paragraph; [topgit] FAQ); stage
 * 2 computes attention over the kept blocks with the online filter.
 * topk must lie in (0, 1] (else SPARGE_E_ARG).  is_causal as in SDPA.
 * out may not alias q, k or v.  workspace: device, >= sparge_workspace_bytes(). */
sparge_status sparge_topk_attn(const sparge_tensor* q, const sparge_tensor* k,
                               const sparge_tensor* v, const sparge_tensor* out,
                               double topk, int32_t is_causal, const sparge_opts* opts,
                               void* workspace, size_t workspace_bytes, void* stream);

/* sparge_topk_attn for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument; the call's scratch regions (sized to its shape, dtype and options) live
 * in the library's own static device storage of SPARGE_NOALLOC_SCRATCH_BYTES, one copy
 * per GPU the library runs on, held until the process ends.  The call allocates
 * nothing.  A problem whose regions exceed the scratch returns SPARGE_E_WORKSPACE
 * before anything is queued (16-bit inputs of B=1, H=32, N=8192, D=128 fit under
 * every option; N=131072 does not).  Every call on one GPU shares that GPU's scratch,
 * which keeps the previous call's contents: calls that can overlap on one GPU
 * (different streams, or threads without ordering) race on it and must not be made.
 * Otherwise identical to sparge_topk_attn; the device is the stream's (the current
 * device for the NULL stream). */
#define SPARGE_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
sparge_status sparge_topk_attn_noalloc(const sparge_tensor* q, const sparge_tensor* k,
                                       const sparge_tensor* v, const sparge_tensor* out, double topk,
                                       int32_t is_causal, const sparge_opts* opts, void* stream);

/* Threshold variant of sparge_topk_attn (the meansim calls without topk, e.g.
 * spas_sage2_attn_meansim_cuda of [readme] "Avalible API" and [gittools] API list;
 * [chapterpal] recommendations on calibrating thresholds): identical except for the
 * per-row selection, which keeps the shortest prefix of the row's candidate blocks,
 * ranked by compressed score (descending, lower block index first on ties), whose
 * share of the row softmax of the compressed map (fp64, over the candidates)
 * reaches cdf_threshold; at least one candidate is kept.  cdf_threshold must lie in
 * (0, 1] (else SPARGE_E_ARG); opts->head_select gives it per head. */
sparge_status sparge_cdf_attn(const sparge_tensor* q, const sparge_tensor* k,
                              const sparge_tensor* v, const sparge_tensor* out,
                              double cdf_threshold, int32_t is_causal, const sparge_opts* opts,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Attention under a caller-given block mask: block_sparse_sage2_attn_cuda(q, k,
 * v, mask_id) of [gittools] custom block-sparse mask section; [topgit]
 * "Strengths".  mask_id: device uint8 (B, H, ceil(N/128), ceil(N/64)), contiguous;
 * nonzero keeps the 128x64 block; NULL keeps every block.  Not causal (the call
 * has no is_causal argument).  A query row with no kept block outputs zeros.
 * opts->head_filter_lambda applies; head_select and head_sim_threshold are
 * validated but not used. */
sparge_status block_sparse_attn(const sparge_tensor* q, const sparge_tensor* k,
                                const sparge_tensor* v, const uint8_t* mask_id,
                                const sparge_tensor* out, const sparge_opts* opts,
                                void* workspace, size_t workspace_bytes, void* stream);

/* Stage 1 only: writes the predicted block mask to mask_out (device uint8,
 * (B, H, ceil(N/128), ceil(N/64)), contiguous).  Same arguments and rules as
 * sparge_topk_attn; opts->mask_out is ignored.  With opts->head_select the topk
 * argument is replaced per head; head_filter_lambda is validated but not used. */
sparge_status sparge_predict_mask(const sparge_tensor* q, const sparge_tensor* k, double topk,
                                  int32_t is_causal, const sparge_opts* opts, uint8_t* mask_out,
                                  void* workspace, size_t workspace_bytes, void* stream);

/* The int8 operands of the qk_int8 option, for inspection (SageAttention base,
 * [topgit] "Key features"), exactly as the attention path forms them: the Q codes
 * are written by the attention kernel itself (a launch that quantizes Q in
 * registers as it does before its Q.K^T and then stops), the K codes by the pass
 * the attention path runs.  fp32 inputs are first rounded to bfloat16, as for the
 * attention products, so their codes are those of the rounded values.  All outputs
 * device, contiguous:
 *   q_codes  int8  (B, H, N, D)       codes of Q, one scale per 32 rows
 *   q_scales float (B, H, ceil(N/32)) fp32 step max|q|/127 of each 32-row group
 *   k_codes  int8  (B, H, N, D)       codes of K - kbar_j (block-smoothed)
 *   k_scales float (B, H, ceil(N/64)) fp32 step of each 64-row block
 *   k_means  float (B, H, ceil(N/64), D) the fp32 block means kbar_j
 * Rounding: half to even, clamp to [-127, 127], all in IEEE fp32.  q and k must
 * be bfloat16, fp16 or fp32. */
sparge_status sparge_quantize_qk(const sparge_tensor* q, const sparge_tensor* k, int8_t* q_codes,
                                 float* q_scales, int8_t* k_codes, float* k_scales, float* k_means,
                                 void* workspace, size_t workspace_bytes, void* stream);

/* 3D Hilbert order of a T x Hg x W token grid ([chapterpal] method paragraph and
 * recommendations: space-filling Hilbert-curve reordering for visual inputs).
 * Writes perm_host[p] = row-major index (t*Hg*W + y*W + x) of the p-th cell along
 * the curve.  Curve: Skilling's transform (AIP Conf. Proc. 707, 2004) on the
 * smallest 2^m cube holding the grid, axes (t, y, x), cells outside the grid
 * skipped.  perm_host: HOST int32 array of T*Hg*W entries.  Pure host function. */
sparge_status sparge_hilbert_perm3d(int32_t T, int32_t Hg, int32_t W, int32_t* perm_host);

/* Token reorder along dimension N, for the Hilbert order of visual tokens.
 * Rows outside [offset, offset + count) are copied unchanged; inside,
 *   inverse == 0 (gather):  y[offset + p] = x[offset + perm[p]]
 *   inverse != 0 (scatter): y[offset + perm[p]] = x[offset + p]
 * for p < count.  x, y: same dtype and shape, y must not alias x.  perm: device
 * int32 permutation of [0, count) (a non-permutation gives unspecified rows but
 * never an out-of-range access: entries are clamped into range). */
sparge_status sparge_reorder(const sparge_tensor* x, const sparge_tensor* y, const int32_t* perm,
                             int64_t offset, int64_t count, int32_t inverse, void* stream);

/* Human-readable name of a status code (static string). */
const char* sparge_status_str(int32_t status);

/* ABI version of this header (incremented on any change of the structs above). */
int32_t sparge_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPARGE_H */
