// Internal declarations of libsparge: kernel argument blocks, workspace layout,
// and the host-side launch functions implemented in the .hip translation units.
// Nothing here is part of the public ABI (include/sparge.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sparge {

constexpr int kBQ = 128;  // query rows per mask block
constexpr int kBK = 64;   // key rows per mask block
constexpr int kQGroup = 32;  // rows per wavefront: filter group and int8 Q scale group

enum ElemType : int { kF32 = 0, kF16 = 1, kBF16 = 2 };

// A strided (B, H, N, D) view with unit stride along D.  Strides in elements.
struct View {
  const void* p;
  int64_t sB, sH, sN;
};

struct Dims {
  int B, H, N, D;
  int nQ, nK;   // ceil(N/128), ceil(N/64)
  int lstride;  // elements per kept-block list row: nK rounded up to 8 (16-byte rows)
};

// fp64 block means are stored per head in 16-row tiles (rows padded to a multiple of
// 16), laid out for the operand reads of the fp64 pooled-score MFMAs: inside a tile,
// row r and channel c, with kq = c / (D/4) and s = c % (D/4), sit at
// ((s/2)*64 + kq*16 + r)*2 + s%2, so that lane kq*16 + r reads channels s and s+1 of
// its row as one 16-byte load and a wavefront's load is 1 KB of contiguous memory.
inline __host__ __device__ int pad16(int n) { return (n + 15) & ~15; }
inline __host__ __device__ int64_t mean_index(int64_t bh, int rows_padded, int row, int c, int D) {
  const int q4 = D / 4, kq = c / q4, s = c % q4;
  return (bh * rows_padded + (row & ~15)) * D + (((s >> 1) * 64 + kq * 16 + (row & 15)) * 2 + (s & 1));
}

inline Dims make_dims(int B, int H, int N, int D) {
  Dims d;
  d.B = B; d.H = H; d.N = N; d.D = D;
  d.nQ = (N + kBQ - 1) / kBQ;
  d.nK = (N + kBK - 1) / kBK;
  d.lstride = (d.nK + 7) & ~7;
  return d;
}

// ---------------------------------------------------------------------------
// Workspace: one buffer, carved into 256-byte aligned regions.
// ---------------------------------------------------------------------------
struct Workspace {
  size_t qmean, qsim, kmean, ksim; // fp64 block means (tiled, see mean_index) and
                                   // self-similarities
  size_t scores;                   // fp64 pooled scores (BH, nQ, nK)
  size_t lists, counts;            // uint16 kept-block lists (BH, nQ, lstride), int32 counts
  size_t k8, kscale, kbar;         // int8 K codes (BH, nK*64, D), fp32 steps, fp32 block means
  size_t kc, kcs;                  // two-level int8 codes of the block means (BH, nK, 2D), steps (BH)
  size_t conv;                     // 16-bit copies of q, k (fp32 inputs) and v (3 x BH*N*D);
                                   // with fp8 P.V (16-bit inputs only) the E4M3 V tiles
  size_t vmaxp, vscale, vinv;      // fp8 P.V: per-block channel max |v| (BH, nQ, D), fp32
                                   // channel scales and inverses (BH, D)
  size_t hparams;                  // per-head knobs (3 x H fp64): selection, theta, lambda
  size_t counters;                 // 8 x uint64 stats counters
  size_t total;
};

// The options of one call that decide which optional regions it uses.
struct PlanNeeds {
  int qk_int8, pv_fp16, pv_fp8;
};

// need == nullptr: every region at its largest (one size for every entry point and
// option); otherwise only the regions that call uses.
Workspace plan_workspace(const Dims& d, int dtype, const PlanNeeds* need = nullptr);

// ---------------------------------------------------------------------------
// Kernel launchers (return hipSuccess or the launch error).
// ---------------------------------------------------------------------------

// fp32/bf16/fp16 -> bf16 or fp16 (RNE) copy of a strided view into a contiguous
// (B, H, N, D) buffer.
hipError_t launch_convert16(const View& x, int src_dtype, const Dims& d, uint16_t* dst,
                            int dst_f16, hipStream_t s);

// Per block (Q: 128 rows, K: 64 rows) channel means in fp64 and self-similarity.
hipError_t launch_block_stats(const View& q, const View& k, int dtype, const Dims& d,
                              double* qmean, double* qsim, double* kmean, double* ksim,
                              hipStream_t s);

// Pooled scores s_ij = scale * qbar_i . kbar_j (fp64) for every block pair that can
// be valid.
hipError_t launch_pooled_scores(const double* qmean, const double* kmean, const Dims& d,
                                int causal, double scale, double* scores, hipStream_t s);

// Per block row: similarity gate, top-k selection, mask row and kept-block list.
// Selection knobs: the scalar values, optionally replaced per head h by device
// arrays of H values.
struct SelectParams {
  double sel;                 // topk fraction, or the softmax-mass threshold when cdf
  double theta;               // self-similarity threshold
  const double* head_sel;     // nullable (H)
  const double* head_theta;   // nullable (H)
  int cdf;                    // 1: keep the shortest ranked prefix reaching mass sel
};

hipError_t launch_select(const double* scores, const double* qsim, const double* ksim,
                         const Dims& d, int causal, const SelectParams& sp,
                         uint8_t* mask_out, uint16_t* lists, int* counts,
                         unsigned long long* counters, hipStream_t s);

// User mask (or all ones when mask == nullptr) -> kept-block lists.
hipError_t launch_compact(const uint8_t* mask, const Dims& d, uint16_t* lists, int* counts,
                          unsigned long long* counters, hipStream_t s);

// Block-smoothed int8 K: codes (BH, nK*64, D), steps (BH, nK), fp32 means (BH, nK, D).
hipError_t launch_quant_k(const View& k, int dtype, const Dims& d, int8_t* codes,
                          int64_t codes_row_stride, int64_t codes_head_stride, float* kscale,
                          float* kbar, hipStream_t s);

// int8 Q K^T: per (b, h) a step sk = max |kbar| / 127 and two codes per element of
// the block means, kbar ~= sk (c1 + c2 / 256): rows (BH, nK, 2D), c1 then c2.
hipError_t launch_kbar_codes(const float* kbar, const Dims& d, int8_t* kc, float* kcs, hipStream_t s);

// Fused pass over 16-bit Q, K, V (one workgroup per Q block): the block means and
// self-similarities of launch_block_stats, plus, when codes != nullptr, the
// block-smoothed int8 K of launch_quant_k (codes with D bytes per row, rows below
// codes_rows written, those past N as zeros), and, when v16 != nullptr, V rounded
// to fp16 into a contiguous (B, H, N, D) buffer, or, when vmaxp != nullptr, the
// per-block channel maxima of |v| (B, H, nQ, D) for the fp8 P.V.
hipError_t launch_prep(const View& q, const View& k, const View& v, int dtype, const Dims& d,
                       double* qmean, double* qsim, double* kmean, double* ksim, int8_t* codes,
                       int64_t codes_head_stride, int64_t codes_rows, float* kscale, float* kbar,
                       uint16_t* v16, float* vmaxp, hipStream_t s);

// fp8 P.V: per-channel scales from the per-block maxima of launch_prep (vmaxp), then
// V as E4M3 codes in transposed 64-token tiles: vt[((bh * nK + j) * D + c) * 64 + r]
// is channel c of token 64j + r (zero for tokens past N).
hipError_t launch_vt8(const View& v, int dtype, const Dims& d, const float* vmaxp, float* vscale,
                      float* vinv, unsigned char* vt, hipStream_t s);

struct AttnParams {
  View q, k;             // 16-bit (bf16 or fp16) views of Q and K
  View v;                // V in the P.V type (fp16 when pv_fp16, else Q's type)
  void* o;               // output
  int64_t osB, osH, osN;
  int in_f16;            // q/k/v element type: 1 = fp16, 0 = bf16
  int out_type;          // ElemType of the output
  int causal, filter_on, qk_int8, pv_fp16, pv_fp8;
  float c;               // scale * log2(e)
  float lam2;            // filter lambda * log2(e)
  const uint16_t* lists;
  const int* counts;
  const int8_t* k8;      // int8 path: codes, (BH, nK*64, D)
  const float* kscale;   // (BH, nK)
  const int8_t* kc;      // two-level codes of the block means, (BH, nK, 2D)
  const float* kcs;      // their step per head, (BH)
  const double* head_lambda; // nullable (H): per-head filter lambda (natural-log units)
  const unsigned char* v8t;  // fp8 P.V: E4M3 V tiles (BH, nK, D, 64)
  const float* vscale;       // fp8 P.V: channel scales (BH, D)
  unsigned long long* counters;  // nullable: [2] = group updates, [3] = skipped updates
  // int8 Q.K^T: when q8_out is set, every wavefront also writes the int8 Q codes it
  // multiplies, (BH, N, D), and their step, (BH, ceil(N/32)); with codes_only it
  // returns right after (no attention: lists, counts, K, V and O are not touched)
  int8_t* q8_out;
  float* q8_scale_out;
  int codes_only;
};

hipError_t launch_sparse_attn(const AttnParams& p, const Dims& d, hipStream_t s);

// Token reorder along N (gather or scatter by perm over [offset, offset+count)).
hipError_t launch_reorder(const View& x, void* y, int64_t ysB, int64_t ysH, int64_t ysN,
                          int esize, const Dims& d, const int32_t* perm, int64_t offset,
                          int64_t count, int inverse, hipStream_t s);

// Host Hilbert order (Skilling forward transform + sort).
void hilbert_perm3d_host(int T, int Hg, int W, int32_t* perm);

}  // namespace sparge
