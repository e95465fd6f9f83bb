// C ABI of libsparge (declared in include/sparge.h): argument validation,
// workspace planning and the launch sequence of each entry point.  Every check
// runs before any HIP call, so argument errors never touch the device.
#include <math.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/sparge.h"
#include "sparge_internal.hpp"

namespace sparge {

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Workspace plan_workspace(const Dims& d, int dtype, const PlanNeeds* need) {
  Workspace w{};
  const size_t BH = (size_t)d.B * d.H;
  const size_t one16 = BH * (size_t)d.N * d.D * sizeof(uint16_t);
  // without `need`: every region at its largest, so that one size serves every entry
  // point and option; with it, only what that call uses
  const bool int8 = !need || need->qk_int8;
  const bool fp8 = !need || need->pv_fp8;
  size_t conv = 0;
  if (!need) {
    const size_t vt8 = BH * (size_t)d.nK * 64 * d.D;
    conv = 3 * one16 > vt8 ? 3 * one16 : vt8;
  } else if (dtype == SPARGE_F32) {
    conv = 3 * one16;                                     // Q, K and V rounded to 16 bits
  } else if (need->pv_fp8) {
    conv = BH * (size_t)d.nK * 64 * d.D;                  // E4M3 V tiles
  } else if (dtype == SPARGE_BF16 && need->pv_fp16) {
    conv = one16;                                         // V rounded to fp16
  }
  size_t off = 0;
  auto take = [&](size_t bytes) { const size_t at = off; off = align256(off + bytes); return at; };
  w.qmean = take(BH * pad16(d.nQ) * d.D * sizeof(double));
  w.qsim = take(BH * d.nQ * sizeof(double));
  w.kmean = take(BH * pad16(d.nK) * d.D * sizeof(double));
  w.ksim = take(BH * d.nK * sizeof(double));
  w.scores = take(BH * d.nQ * d.nK * sizeof(double));
  w.lists = take(BH * d.nQ * d.lstride * sizeof(uint16_t));
  w.counts = take(BH * d.nQ * sizeof(int));
  w.k8 = take(int8 ? BH * (size_t)d.nK * 64 * d.D : 0);
  w.kscale = take(int8 ? BH * d.nK * sizeof(float) : 0);
  w.kbar = take(int8 ? BH * d.nK * d.D * sizeof(float) : 0);
  w.kc = take(int8 ? BH * d.nK * 2 * d.D : 0);
  w.kcs = take(BH * sizeof(float));
  w.conv = take(conv);
  w.vmaxp = take(fp8 ? BH * d.nQ * d.D * sizeof(float) : 0);
  w.vscale = take(fp8 ? BH * d.D * sizeof(float) : 0);
  w.vinv = take(fp8 ? BH * d.D * sizeof(float) : 0);
  w.hparams = take(3 * (size_t)d.H * sizeof(double));
  w.counters = take(8 * sizeof(unsigned long long));
  w.total = off;
  return w;
}

}  // namespace sparge

using namespace sparge;

namespace {

constexpr int64_t kMaxN = 262144;  // uint16 block lists and the selector's LDS bound N

sparge_status check_tensor(const sparge_tensor* t) {
  if (!t || !t->data) return SPARGE_E_NULL;
  if (t->dtype != SPARGE_F32 && t->dtype != SPARGE_F16 && t->dtype != SPARGE_BF16)
    return SPARGE_E_DTYPE;
  if (t->reserved != 0) return SPARGE_E_ARG;
  if (t->B < 1 || t->H < 1 || t->N < 1 || t->N > kMaxN) return SPARGE_E_SHAPE;
  if (t->D != 64 && t->D != 128) return SPARGE_E_SHAPE;
  if (t->B * t->H * ((t->N + 127) / 128) > 0x7fffffffll) return SPARGE_E_SHAPE;
  const int64_t es = t->dtype == SPARGE_F32 ? 4 : 2;
  if (((uintptr_t)t->data) % 16 != 0) return SPARGE_E_UNSUPPORTED;
  if (t->sB < 0 || t->sH < 0 || t->sN < 0) return SPARGE_E_UNSUPPORTED;
  if ((t->sB * es) % 16 || (t->sH * es) % 16 || (t->sN * es) % 16) return SPARGE_E_UNSUPPORTED;
  // a 64-row block of K or V is addressed with 32-bit byte offsets
  if (t->sN * es >= ((int64_t)1 << 26)) return SPARGE_E_UNSUPPORTED;
  return SPARGE_OK;
}

bool same_shape(const sparge_tensor* a, const sparge_tensor* b) {
  return a->B == b->B && a->H == b->H && a->N == b->N && a->D == b->D;
}

Dims dims_of(const sparge_tensor* t) {
  return make_dims((int)t->B, (int)t->H, (int)t->N, (int)t->D);
}

View view_of(const sparge_tensor* t) { return View{t->data, t->sB, t->sH, t->sN}; }

sparge_status check_opts(const sparge_opts* o) {
  if (!o) return SPARGE_OK;
  if (o->pv_fp8 != 0 && o->pv_fp16 != 0) return SPARGE_E_ARG;
  if (!(o->scale >= 0.0) || isinf(o->scale)) return SPARGE_E_ARG;
  if (isnan(o->sim_threshold) || isnan(o->filter_lambda)) return SPARGE_E_ARG;
  if (o->filter_lambda > 0.0) return SPARGE_E_ARG;
  return SPARGE_OK;
}

// The per-head arrays of opts (host memory, H values each).
sparge_status check_head_params(const sparge_opts* o, int64_t H) {
  if (!o) return SPARGE_OK;
  for (int64_t h = 0; h < H; ++h) {
    if (o->head_select && !(o->head_select[h] > 0.0 && o->head_select[h] <= 1.0)) return SPARGE_E_ARG;
    if (o->head_sim_threshold && isnan(o->head_sim_threshold[h])) return SPARGE_E_ARG;
    if (o->head_filter_lambda && !(o->head_filter_lambda[h] <= 0.0)) return SPARGE_E_ARG;
  }
  return SPARGE_OK;
}

sparge_status check_qkv(const sparge_tensor* q, const sparge_tensor* k, const sparge_tensor* v,
                        const sparge_tensor* out) {
  sparge_status st;
  if ((st = check_tensor(q)) != SPARGE_OK) return st;
  if ((st = check_tensor(k)) != SPARGE_OK) return st;
  if (v && (st = check_tensor(v)) != SPARGE_OK) return st;
  if (out && (st = check_tensor(out)) != SPARGE_OK) return st;
  if (k->dtype != q->dtype || (v && v->dtype != q->dtype) || (out && out->dtype != q->dtype))
    return SPARGE_E_DTYPE;
  if (!same_shape(q, k) || (v && !same_shape(q, v)) || (out && !same_shape(q, out)))
    return SPARGE_E_SHAPE;
  if (out && (out->data == q->data || out->data == k->data || (v && out->data == v->data)))
    return SPARGE_E_ARG;
  return SPARGE_OK;
}

struct Ctx {
  Dims d;
  Workspace w;
  char* ws;
  hipStream_t s;
  unsigned long long* counters;  // nullable
  // device copies of the per-head arrays (nullable)
  const double* head_sel = nullptr;
  const double* head_theta = nullptr;
  const double* head_lambda = nullptr;
  template <typename T>
  T* at(size_t off) const { return (T*)(ws + off); }
};

#define SPARGE_TRY(expr) do { const hipError_t e__ = (expr); if (e__ != hipSuccess) return SPARGE_E_HIP; } while (0)

sparge_status begin_stats(Ctx& c, const sparge_opts* o) {
  c.counters = nullptr;
  if (o && o->prof_start) SPARGE_TRY(hipEventRecord((hipEvent_t)o->prof_start, c.s));
  if (o && o->stats) {
    c.counters = c.at<unsigned long long>(c.w.counters);
    SPARGE_TRY(hipMemsetAsync(c.counters, 0, 8 * sizeof(unsigned long long), c.s));
  }
  return SPARGE_OK;
}

// Copies the caller's per-head arrays into the workspace (pageable host memory:
// the copy has consumed the source when the call returns).
sparge_status stage_head_params(Ctx& c, const sparge_opts& o) {
  double* dst = c.at<double>(c.w.hparams);
  const size_t bytes = (size_t)c.d.H * sizeof(double);
  const double* src[3] = {o.head_select, o.head_sim_threshold, o.head_filter_lambda};
  const double** out[3] = {&c.head_sel, &c.head_theta, &c.head_lambda};
  for (int a = 0; a < 3; ++a) {
    *out[a] = nullptr;
    if (!src[a]) continue;
    SPARGE_TRY(hipMemcpyAsync(dst + a * c.d.H, src[a], bytes, hipMemcpyHostToDevice, c.s));
    *out[a] = dst + a * c.d.H;
  }
  return SPARGE_OK;
}

sparge_status end_stats(Ctx& c, const sparge_opts* o) {
  if (!c.counters) return SPARGE_OK;
  unsigned long long h[8];
  SPARGE_TRY(hipMemcpyAsync(h, c.counters, sizeof(h), hipMemcpyDeviceToHost, c.s));
  SPARGE_TRY(hipStreamSynchronize(c.s));
  o->stats->valid_blocks = h[0];
  o->stats->kept_blocks = h[1];
  o->stats->group_updates = h[2];
  o->stats->skipped_updates = h[3];
  return SPARGE_OK;
}

// The attention operands: Q and K as 16-bit views (fp32 inputs rounded to bf16
// into the workspace), V in the P.V type (converted into the workspace when it
// differs from the input's type, once per call rather than once per block).
struct Operands {
  View q, k, v;
  int in_f16;
  int dtype16;
};

sparge_status prepare_operands(Ctx& c, const sparge_tensor* q, const sparge_tensor* k,
                               const sparge_tensor* v, int pv_fp16, Operands& op) {
  const size_t one = (size_t)c.d.B * c.d.H * c.d.N * c.d.D;
  uint16_t* base = c.at<uint16_t>(c.w.conv);
  const View packed_strides{nullptr, (int64_t)c.d.H * c.d.N * c.d.D, (int64_t)c.d.N * c.d.D,
                            (int64_t)c.d.D};
  auto converted = [&](uint16_t* o) { View r = packed_strides; r.p = o; return r; };
  if (q->dtype == SPARGE_F32) {
    SPARGE_TRY(launch_convert16(view_of(q), kF32, c.d, base, 0, c.s));
    SPARGE_TRY(launch_convert16(view_of(k), kF32, c.d, base + one, 0, c.s));
    op.q = converted(base);
    op.k = converted(base + one);
    op.in_f16 = 0;
    op.dtype16 = kBF16;
  } else {
    op.q = view_of(q);
    op.k = view_of(k);
    op.in_f16 = q->dtype == SPARGE_F16;
    op.dtype16 = q->dtype;
  }
  const int v_f16 = pv_fp16 ? 1 : op.in_f16;
  const int v_native = (v->dtype == SPARGE_F16 && v_f16) || (v->dtype == SPARGE_BF16 && !v_f16);
  if (v_native) {
    op.v = view_of(v);
  } else {
    SPARGE_TRY(launch_convert16(view_of(v), v->dtype, c.d, base + 2 * one, v_f16, c.s));
    op.v = converted(base + 2 * one);
  }
  return SPARGE_OK;
}

sparge_status run_attention(Ctx& c, const Operands& op, const sparge_tensor* out,
                            const sparge_opts& o, int causal, int filter_on, bool k_ready = false) {
  AttnParams p{};
  p.q = op.q;
  p.k = op.k;
  p.v = op.v;
  p.o = out->data;
  p.osB = out->sB;
  p.osH = out->sH;
  p.osN = out->sN;
  p.in_f16 = op.in_f16;
  p.out_type = out->dtype;
  p.causal = causal;
  p.filter_on = filter_on;
  p.qk_int8 = o.qk_int8 != 0;
  p.pv_fp16 = o.pv_fp16 != 0;
  p.pv_fp8 = o.pv_fp8 != 0;
  if (p.pv_fp8) {
    p.v8t = c.at<unsigned char>(c.w.conv);
    p.vscale = c.at<float>(c.w.vscale);
  }
  const double scale = o.scale > 0.0 ? o.scale : 1.0 / sqrt((double)c.d.D);
  const double log2e = 1.4426950408889634;
  p.c = (float)(scale * log2e);
  p.lam2 = (float)(o.filter_lambda * log2e);
  p.head_lambda = c.head_lambda;
  p.lists = c.at<uint16_t>(c.w.lists);
  p.counts = c.at<int>(c.w.counts);
  p.counters = c.counters;
  if (p.qk_int8) {
    int8_t* k8 = c.at<int8_t>(c.w.k8);
    float* ks = c.at<float>(c.w.kscale);
    float* kb = c.at<float>(c.w.kbar);
    if (!k_ready)
      SPARGE_TRY(launch_quant_k(op.k, op.dtype16, c.d, k8, c.d.D, (int64_t)c.d.nK * 64 * c.d.D, ks,
                                kb, c.s));
    int8_t* kc = c.at<int8_t>(c.w.kc);
    float* kcs = c.at<float>(c.w.kcs);
    SPARGE_TRY(launch_kbar_codes(kb, c.d, kc, kcs, c.s));
    p.k8 = k8;
    p.kscale = ks;
    p.kc = kc;
    p.kcs = kcs;
  }
  if (o.prof_attn_begin) SPARGE_TRY(hipEventRecord((hipEvent_t)o.prof_attn_begin, c.s));
  SPARGE_TRY(launch_sparse_attn(p, c.d, c.s));
  if (o.prof_attn_end) SPARGE_TRY(hipEventRecord((hipEvent_t)o.prof_attn_end, c.s));
  return SPARGE_OK;
}

SelectParams select_params(const Ctx& c, double sel, int cdf, const sparge_opts& o) {
  SelectParams sp;
  sp.sel = sel;
  sp.theta = o.sim_threshold;
  sp.head_sel = c.head_sel;
  sp.head_theta = c.head_theta;
  sp.cdf = cdf;
  return sp;
}

sparge_status run_predictor(Ctx& c, const sparge_tensor* q, const sparge_tensor* k, double topk,
                            int cdf, int causal, const sparge_opts& o, uint8_t* mask_out) {
  const double scale = o.scale > 0.0 ? o.scale : 1.0 / sqrt((double)c.d.D);
  double* qmean = c.at<double>(c.w.qmean);
  double* qsim = c.at<double>(c.w.qsim);
  double* kmean = c.at<double>(c.w.kmean);
  double* ksim = c.at<double>(c.w.ksim);
  double* scores = c.at<double>(c.w.scores);
  SPARGE_TRY(launch_block_stats(view_of(q), view_of(k), q->dtype, c.d, qmean, qsim, kmean, ksim, c.s));
  SPARGE_TRY(launch_pooled_scores(qmean, kmean, c.d, causal, scale, scores, c.s));
  SPARGE_TRY(launch_select(scores, qsim, ksim, c.d, causal, select_params(c, topk, cdf, o), mask_out,
                           c.at<uint16_t>(c.w.lists), c.at<int>(c.w.counts), c.counters, c.s));
  return SPARGE_OK;
}

// 16-bit inputs: one fused pass over Q, K and V writes the predictor's block
// statistics, the int8 K when asked for, and the fp16 V when the P.V type differs
// from the input's (or, for the fp8 P.V, V's per-block channel maxima, followed by
// the scales and the E4M3 V tiles); the operands then point at the inputs or at
// those copies.
sparge_status prep16(Ctx& c, const sparge_tensor* q, const sparge_tensor* k,
                     const sparge_tensor* v, const sparge_opts& o, Operands& op) {
  op.q = view_of(q);
  op.k = view_of(k);
  op.in_f16 = q->dtype == SPARGE_F16;
  op.dtype16 = q->dtype;
  const int v_f16 = o.pv_fp16 ? 1 : op.in_f16;
  const int v_native = (v->dtype == SPARGE_F16 && v_f16) || (v->dtype == SPARGE_BF16 && !v_f16);
  uint16_t* v16 = nullptr;
  float* vmaxp = o.pv_fp8 ? c.at<float>(c.w.vmaxp) : nullptr;
  if (v_native || o.pv_fp8) {
    op.v = view_of(v);
  } else {
    v16 = c.at<uint16_t>(c.w.conv);
    op.v = View{v16, (int64_t)c.d.H * c.d.N * c.d.D, (int64_t)c.d.N * c.d.D, (int64_t)c.d.D};
  }
  const int64_t chead = (int64_t)c.d.nK * 64 * c.d.D;
  SPARGE_TRY(launch_prep(view_of(q), view_of(k), view_of(v), q->dtype, c.d, c.at<double>(c.w.qmean),
                         c.at<double>(c.w.qsim), c.at<double>(c.w.kmean), c.at<double>(c.w.ksim),
                         o.qk_int8 ? c.at<int8_t>(c.w.k8) : nullptr, chead,
                         (int64_t)c.d.nK * 64, c.at<float>(c.w.kscale), c.at<float>(c.w.kbar),
                         v16, vmaxp, c.s));
  if (o.pv_fp8)
    SPARGE_TRY(launch_vt8(view_of(v), v->dtype, c.d, vmaxp, c.at<float>(c.w.vscale),
                          c.at<float>(c.w.vinv), c.at<unsigned char>(c.w.conv), c.s));
  return SPARGE_OK;
}

// Pooled scores and selection from the block statistics already in the workspace.
sparge_status run_select(Ctx& c, double topk, int cdf, int causal, const sparge_opts& o) {
  const double scale = o.scale > 0.0 ? o.scale : 1.0 / sqrt((double)c.d.D);
  double* scores = c.at<double>(c.w.scores);
  SPARGE_TRY(launch_pooled_scores(c.at<double>(c.w.qmean), c.at<double>(c.w.kmean), c.d, causal,
                                  scale, scores, c.s));
  SPARGE_TRY(launch_select(scores, c.at<double>(c.w.qsim), c.at<double>(c.w.ksim), c.d, causal,
                           select_params(c, topk, cdf, o), o.mask_out, c.at<uint16_t>(c.w.lists),
                           c.at<int>(c.w.counts), c.counters, c.s));
  return SPARGE_OK;
}

sparge_status init_ctx(Ctx& c, const sparge_tensor* q, void* workspace, size_t workspace_bytes,
                       void* stream, const PlanNeeds* need = nullptr) {
  c.d = dims_of(q);
  c.w = plan_workspace(c.d, q->dtype, need);
  if (!workspace) return SPARGE_E_WORKSPACE;
  if (workspace_bytes < c.w.total) return SPARGE_E_WORKSPACE;
  if (((uintptr_t)workspace) % 256 != 0) return SPARGE_E_UNSUPPORTED;
  c.ws = (char*)workspace;
  c.s = (hipStream_t)stream;
  c.counters = nullptr;
  return SPARGE_OK;
}

}  // namespace

extern "C" {

void sparge_default_opts(sparge_opts* o) {
  if (!o) return;
  memset(o, 0, sizeof(*o));
  o->scale = 0.0;
  o->sim_threshold = 0.1;
  o->filter_lambda = -10.0;
  o->filter_on = 1;
  o->qk_int8 = 0;
  o->pv_fp16 = 0;
  o->pv_fp8 = 0;
}

size_t sparge_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t D, int32_t dtype,
                              const sparge_opts* opts) {
  (void)opts;
  if (B < 1 || H < 1 || N < 1 || N > kMaxN || (D != 64 && D != 128)) return 0;
  if (dtype != SPARGE_F32 && dtype != SPARGE_F16 && dtype != SPARGE_BF16) return 0;
  return plan_workspace(make_dims((int)B, (int)H, (int)N, (int)D), dtype).total;
}

}  // extern "C"

namespace {

// Argument checks of sparge_topk_attn, sparge_cdf_attn and sparge_topk_attn_noalloc
// (sel: the kept fraction or the softmax-mass threshold); fills the effective options.
sparge_status check_predicted(const sparge_tensor* q, const sparge_tensor* k, const sparge_tensor* v,
                              const sparge_tensor* out, double sel, const sparge_opts* opts,
                              sparge_opts& o) {
  sparge_status st;
  if ((st = check_qkv(q, k, v, out)) != SPARGE_OK) return st;
  if ((st = check_opts(opts)) != SPARGE_OK) return st;
  if ((st = check_head_params(opts, q->H)) != SPARGE_OK) return st;
  if (!(sel > 0.0 && sel <= 1.0)) return SPARGE_E_ARG;
  if (opts) o = *opts; else sparge_default_opts(&o);
  if (o.pv_fp8 && q->dtype == SPARGE_F32) return SPARGE_E_UNSUPPORTED;
  return SPARGE_OK;
}

// The launch sequence of the predicted-mask calls (cdf = 0: top-k, 1: threshold).
sparge_status run_predicted(Ctx& c, const sparge_tensor* q, const sparge_tensor* k,
                            const sparge_tensor* v, const sparge_tensor* out, double sel, int cdf,
                            int32_t is_causal, const sparge_opts& o) {
  sparge_status st;
  if ((st = begin_stats(c, &o)) != SPARGE_OK) return st;
  if ((st = stage_head_params(c, o)) != SPARGE_OK) return st;
  Operands op;
  if (q->dtype != SPARGE_F32) {
    if ((st = prep16(c, q, k, v, o, op)) != SPARGE_OK) return st;
    if ((st = run_select(c, sel, cdf, is_causal != 0, o)) != SPARGE_OK) return st;
    if ((st = run_attention(c, op, out, o, is_causal != 0, o.filter_on != 0, true)) != SPARGE_OK) return st;
    return end_stats(c, &o);
  }
  if ((st = prepare_operands(c, q, k, v, o.pv_fp16, op)) != SPARGE_OK) return st;
  if ((st = run_predictor(c, q, k, sel, cdf, is_causal != 0, o, o.mask_out)) != SPARGE_OK) return st;
  if ((st = run_attention(c, op, out, o, is_causal != 0, o.filter_on != 0)) != SPARGE_OK) return st;
  return end_stats(c, &o);
}

sparge_status predicted_attn(const sparge_tensor* q, const sparge_tensor* k, const sparge_tensor* v,
                             const sparge_tensor* out, double sel, int cdf, int32_t is_causal,
                             const sparge_opts* opts, void* workspace, size_t workspace_bytes,
                             void* stream) {
  sparge_status st;
  sparge_opts o;
  if ((st = check_predicted(q, k, v, out, sel, opts, o)) != SPARGE_OK) return st;
  Ctx c;
  if ((st = init_ctx(c, q, workspace, workspace_bytes, stream)) != SPARGE_OK) return st;
  return run_predicted(c, q, k, v, out, sel, cdf, is_causal, o);
}

// Scratch of sparge_topk_attn_noalloc: static device storage of the library's code
// object, so each GPU the library runs on holds its own copy for the life of the
// process.  Host code never uses the array's name as an address: the address of a
// device's copy is looked up once per device (with that device current) and kept.
constexpr size_t kScratchBytes = SPARGE_NOALLOC_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_addr[kMaxDevices];

// The address of the scratch copy of the device that `stream` belongs to (the current
// device for the NULL stream).
sparge_status scratch_for(hipStream_t stream, void** addr) {
  int dev = -1;
  if (stream) {
    hipDevice_t sd;
    if (hipStreamGetDevice(stream, &sd) != hipSuccess) return SPARGE_E_HIP;
    dev = (int)sd;
  } else if (hipGetDevice(&dev) != hipSuccess) {
    return SPARGE_E_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) return SPARGE_E_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_addr[dev]) {
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return SPARGE_E_HIP;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return SPARGE_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess || !p) return SPARGE_E_HIP;
    scratch_addr[dev] = p;
  }
  *addr = scratch_addr[dev];
  return SPARGE_OK;
}

}  // namespace

extern "C" {

sparge_status sparge_topk_attn(const sparge_tensor* q, const sparge_tensor* k,
                               const sparge_tensor* v, const sparge_tensor* out, double topk,
                               int32_t is_causal, const sparge_opts* opts, void* workspace,
                               size_t workspace_bytes, void* stream) {
  return predicted_attn(q, k, v, out, topk, 0, is_causal, opts, workspace, workspace_bytes, stream);
}

sparge_status sparge_cdf_attn(const sparge_tensor* q, const sparge_tensor* k,
                              const sparge_tensor* v, const sparge_tensor* out,
                              double cdf_threshold, int32_t is_causal, const sparge_opts* opts,
                              void* workspace, size_t workspace_bytes, void* stream) {
  return predicted_attn(q, k, v, out, cdf_threshold, 1, is_causal, opts, workspace,
                        workspace_bytes, stream);
}

sparge_status sparge_topk_attn_noalloc(const sparge_tensor* q, const sparge_tensor* k,
                                       const sparge_tensor* v, const sparge_tensor* out, double topk,
                                       int32_t is_causal, const sparge_opts* opts, void* stream) {
  sparge_status st;
  sparge_opts o;
  if ((st = check_predicted(q, k, v, out, topk, opts, o)) != SPARGE_OK) return st;
  // the regions this call uses, sized to it; beyond the scratch it cannot run
  const PlanNeeds need{o.qk_int8 != 0, o.pv_fp16 != 0, o.pv_fp8 != 0};
  if (plan_workspace(dims_of(q), q->dtype, &need).total > kScratchBytes) return SPARGE_E_WORKSPACE;
  void* ws = nullptr;
  if ((st = scratch_for((hipStream_t)stream, &ws)) != SPARGE_OK) return st;
  Ctx c;
  if ((st = init_ctx(c, q, ws, kScratchBytes, stream, &need)) != SPARGE_OK) return st;
  return run_predicted(c, q, k, v, out, topk, 0, is_causal, o);
}

sparge_status block_sparse_attn(const sparge_tensor* q, const sparge_tensor* k,
                                const sparge_tensor* v, const uint8_t* mask_id,
                                const sparge_tensor* out, const sparge_opts* opts, void* workspace,
                                size_t workspace_bytes, void* stream) {
  sparge_status st;
  if ((st = check_qkv(q, k, v, out)) != SPARGE_OK) return st;
  if ((st = check_opts(opts)) != SPARGE_OK) return st;
  sparge_opts o;
  if (opts) {
    o = *opts;
  } else {
    sparge_default_opts(&o);
    o.filter_on = 0;
  }
  if (o.pv_fp8 && q->dtype == SPARGE_F32) return SPARGE_E_UNSUPPORTED;
  if ((st = check_head_params(&o, q->H)) != SPARGE_OK) return st;
  o.head_select = nullptr;          // no selection here
  o.head_sim_threshold = nullptr;
  Ctx c;
  if ((st = init_ctx(c, q, workspace, workspace_bytes, stream)) != SPARGE_OK) return st;
  if ((st = begin_stats(c, &o)) != SPARGE_OK) return st;
  if ((st = stage_head_params(c, o)) != SPARGE_OK) return st;
  Operands op;
  bool k_ready = false;
  const int v_conv = v->dtype == SPARGE_BF16 && o.pv_fp16;
  if (q->dtype != SPARGE_F32 && (o.qk_int8 || v_conv || o.pv_fp8)) {
    // the int8 K and the fp16 or fp8 V in one pass (its block statistics go unused)
    if ((st = prep16(c, q, k, v, o, op)) != SPARGE_OK) return st;
    k_ready = true;
  } else if ((st = prepare_operands(c, q, k, v, o.pv_fp16, op)) != SPARGE_OK) {
    return st;
  }
  SPARGE_TRY(launch_compact(mask_id, c.d, c.at<uint16_t>(c.w.lists), c.at<int>(c.w.counts),
                            c.counters, c.s));
  if ((st = run_attention(c, op, out, o, 0, o.filter_on != 0, k_ready)) != SPARGE_OK) return st;
  return end_stats(c, &o);
}

sparge_status sparge_predict_mask(const sparge_tensor* q, const sparge_tensor* k, double topk,
                                  int32_t is_causal, const sparge_opts* opts, uint8_t* mask_out,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  sparge_status st;
  if ((st = check_qkv(q, k, nullptr, nullptr)) != SPARGE_OK) return st;
  if ((st = check_opts(opts)) != SPARGE_OK) return st;
  if (!mask_out) return SPARGE_E_NULL;
  if (!(topk > 0.0 && topk <= 1.0)) return SPARGE_E_ARG;
  if ((st = check_head_params(opts, q->H)) != SPARGE_OK) return st;
  sparge_opts o;
  if (opts) o = *opts; else sparge_default_opts(&o);
  o.head_filter_lambda = nullptr;   // no attention here
  Ctx c;
  if ((st = init_ctx(c, q, workspace, workspace_bytes, stream)) != SPARGE_OK) return st;
  if ((st = begin_stats(c, &o)) != SPARGE_OK) return st;
  if ((st = stage_head_params(c, o)) != SPARGE_OK) return st;
  if (q->dtype != SPARGE_F32) {
    // the statistics of the fused pass the attention path uses (no int8 K, no V)
    SPARGE_TRY(launch_prep(view_of(q), view_of(k), view_of(k), q->dtype, c.d, c.at<double>(c.w.qmean),
                           c.at<double>(c.w.qsim), c.at<double>(c.w.kmean), c.at<double>(c.w.ksim),
                           nullptr, 0, 0, nullptr, nullptr, nullptr, nullptr, c.s));
    o.mask_out = mask_out;
    if ((st = run_select(c, topk, 0, is_causal != 0, o)) != SPARGE_OK) return st;
    return end_stats(c, &o);
  }
  if ((st = run_predictor(c, q, k, topk, 0, is_causal != 0, o, mask_out)) != SPARGE_OK) return st;
  return end_stats(c, &o);
}

sparge_status sparge_quantize_qk(const sparge_tensor* q, const sparge_tensor* k, int8_t* q_codes,
                                 float* q_scales, int8_t* k_codes, float* k_scales, float* k_means,
                                 void* workspace, size_t workspace_bytes, void* stream) {
  sparge_status st;
  if ((st = check_qkv(q, k, nullptr, nullptr)) != SPARGE_OK) return st;
  if (!q_codes || !q_scales || !k_codes || !k_scales || !k_means) return SPARGE_E_NULL;
  Ctx c;
  if ((st = init_ctx(c, q, workspace, workspace_bytes, stream)) != SPARGE_OK) return st;
  // the operands exactly as the attention path forms them: fp32 inputs rounded to
  // bfloat16 first; Q's codes made by the attention kernel itself (codes-only launch);
  // K's by the pass the attention path runs
  View q16 = view_of(q), k16 = view_of(k);
  int dtype16 = q->dtype, in_f16 = q->dtype == SPARGE_F16;
  if (q->dtype == SPARGE_F32) {
    const size_t one = (size_t)c.d.B * c.d.H * c.d.N * c.d.D;
    uint16_t* base = c.at<uint16_t>(c.w.conv);
    const View packed{nullptr, (int64_t)c.d.H * c.d.N * c.d.D, (int64_t)c.d.N * c.d.D, (int64_t)c.d.D};
    SPARGE_TRY(launch_convert16(view_of(q), kF32, c.d, base, 0, c.s));
    SPARGE_TRY(launch_convert16(view_of(k), kF32, c.d, base + one, 0, c.s));
    q16 = packed;
    q16.p = base;
    k16 = packed;
    k16.p = base + one;
    dtype16 = kBF16;
    in_f16 = 0;
  }
  AttnParams p{};
  p.q = q16;
  p.k = k16;
  p.v = q16;
  p.in_f16 = in_f16;
  p.out_type = dtype16;
  p.qk_int8 = 1;
  p.pv_fp16 = 1;
  p.kcs = c.at<float>(c.w.kcs);
  p.q8_out = q_codes;
  p.q8_scale_out = q_scales;
  p.codes_only = 1;
  SPARGE_TRY(launch_sparse_attn(p, c.d, c.s));
  if (q->dtype != SPARGE_F32) {
    // the fused pass the attention path uses (its block statistics go unused)
    SPARGE_TRY(launch_prep(q16, k16, k16, dtype16, c.d, c.at<double>(c.w.qmean),
                           c.at<double>(c.w.qsim), c.at<double>(c.w.kmean), c.at<double>(c.w.ksim),
                           k_codes, (int64_t)c.d.N * c.d.D, c.d.N, k_scales, k_means, nullptr,
                           nullptr, c.s));
  } else {
    SPARGE_TRY(launch_quant_k(k16, dtype16, c.d, k_codes, c.d.D, (int64_t)c.d.N * c.d.D, k_scales,
                              k_means, c.s));
  }
  return SPARGE_OK;
}

sparge_status sparge_hilbert_perm3d(int32_t T, int32_t Hg, int32_t W, int32_t* perm_host) {
  if (!perm_host) return SPARGE_E_NULL;
  if (T < 1 || Hg < 1 || W < 1) return SPARGE_E_SHAPE;
  if ((int64_t)T * Hg * W > (1ll << 30) || T > (1 << 20) || Hg > (1 << 20) || W > (1 << 20))
    return SPARGE_E_SHAPE;
  hilbert_perm3d_host(T, Hg, W, perm_host);
  return SPARGE_OK;
}

sparge_status sparge_reorder(const sparge_tensor* x, const sparge_tensor* y, const int32_t* perm,
                             int64_t offset, int64_t count, int32_t inverse, void* stream) {
  sparge_status st;
  if ((st = check_tensor(x)) != SPARGE_OK) return st;
  if ((st = check_tensor(y)) != SPARGE_OK) return st;
  if (x->dtype != y->dtype) return SPARGE_E_DTYPE;
  if (!same_shape(x, y)) return SPARGE_E_SHAPE;
  if (x->data == y->data) return SPARGE_E_ARG;
  if (count < 0 || offset < 0 || offset + count > x->N) return SPARGE_E_ARG;
  if (count > 0 && !perm) return SPARGE_E_NULL;
  const Dims d = dims_of(x);
  const int es = x->dtype == SPARGE_F32 ? 4 : 2;
  SPARGE_TRY(launch_reorder(view_of(x), y->data, y->sB, y->sH, y->sN, es, d, perm, offset, count,
                            inverse, (hipStream_t)stream));
  return SPARGE_OK;
}

const char* sparge_status_str(int32_t s) {
  switch (s) {
    case SPARGE_OK: return "ok";
    case SPARGE_E_NULL: return "null pointer";
    case SPARGE_E_SHAPE: return "bad shape";
    case SPARGE_E_DTYPE: return "bad dtype";
    case SPARGE_E_ARG: return "bad argument";
    case SPARGE_E_UNSUPPORTED: return "unsupported layout";
    case SPARGE_E_WORKSPACE: return "workspace missing or too small";
    case SPARGE_E_HIP: return "HIP error";
    default: return "unknown status";
  }
}

int32_t sparge_abi_version(void) { return 3; }

}  // extern "C"
