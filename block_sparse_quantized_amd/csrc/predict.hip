// Stage 1 of SpargeAttn on gfx950: the on-the-fly block-mask predictor.
//
// [chapterpal] method paragraph: sparse blocks are predicted by compressing token
// blocks with high internal similarity while non-similar blocks are always
// computed; [topgit] "Using the plug-and-play API" and FAQ: `topk` in (0, 1] is the
// fraction kept.  Readings implemented here (the library's spec):
//   * blocks: 128 query rows, 64 key rows, ragged tails kept (ceil on both axes);
//   * self-similarity of a block = mean of its full cosine-similarity matrix,
//     || sum_r x_r/||x_r|| ||^2 / n^2, similar iff >= theta;
//   * candidates of block row i: valid K blocks that are similar; row i keeps
//     k_i = min(C, max(1, ceil(topk*C - 1e-9))) of them by (score desc, index asc),
//     plus every valid block of a non-similar row or column;
//   * threshold variant ([readme] "Avalible API": the meansim calls without topk):
//     keep the shortest prefix of that ranking whose softmax mass reaches tau.
// All arithmetic that decides the mask runs in IEEE fp64 (fused multiply-adds only
// inside dot products); the threshold variant sums its fp64 softmax weights as exact
// integers in units of 2^-51.
#include "sparge_internal.hpp"

#pragma clang fp contract(off)

namespace sparge {
namespace {

__device__ __forceinline__ double readlane_f64(double v, int l) {
  long long bits = __double_as_longlong(v);
  int lo = __builtin_amdgcn_readlane((int)(bits & 0xffffffffll), l);
  int hi = __builtin_amdgcn_readlane((int)(bits >> 32), l);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

__device__ __forceinline__ double widen_bf16(unsigned short u) {
  return (double)__uint_as_float((unsigned int)u << 16);
}
__device__ __forceinline__ double widen_f16(unsigned short u) {
  return (double)(float)__builtin_bit_cast(_Float16, u);
}

template <int DT>  // DT: kF32, kF16, kBF16
__device__ __forceinline__ double ld(const void* base, int64_t idx) {
  if constexpr (DT == kF32) return (double)((const float*)base)[idx];
  else if constexpr (DT == kF16) return widen_f16(((const unsigned short*)base)[idx]);
  else return widen_bf16(((const unsigned short*)base)[idx]);
}

// One wavefront per block: Q blocks (128 rows) then K blocks (64 rows) of each
// (b, h).  Pass 1 (one row per lane) forms 1/||x_r||; pass 2 (channels across
// lanes) accumulates the channel sums and the sum of unit rows in row order; the
// means are the sums over the row count in fp64.
template <int DT, int D>
__global__ __launch_bounds__(256) void block_stats_kernel(View q, View k, Dims d, double* qmean,
                                                          double* qsim, double* kmean,
                                                          double* ksim) {
  constexpr int CPL = D / 64;  // channels per lane in pass 2
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int per = d.nQ + d.nK;
  const int64_t total = (int64_t)d.B * d.H * per;
  if (task >= total) return;
  const int bh = (int)(task / per);
  const int r = (int)(task % per);
  const bool isq = r < d.nQ;
  const int blk = isq ? r : r - d.nQ;
  const int rows = isq ? kBQ : kBK;
  const int r0 = blk * rows;
  const int n = min(rows, d.N - r0);
  const View x = isq ? q : k;
  const int b = bh / d.H, h = bh % d.H;
  const int64_t base = (int64_t)b * x.sB + (int64_t)h * x.sH + (int64_t)r0 * x.sN;

  // pass 1: inverse norms of rows lane and lane + 64
  double inv[2] = {0.0, 0.0};
  for (int half = 0; half < rows / 64; ++half) {
    const int rr = lane + 64 * half;
    if (rr < n) {
      const int64_t ro = base + (int64_t)rr * x.sN;
      double ss = 0.0;
      if constexpr (DT == kF32) {
        const float4* rp = (const float4*)((const float*)x.p + ro);
        for (int c = 0; c < D / 4; ++c) {
          const float4 f = rp[c];
          const double v0 = f.x, v1 = f.y, v2 = f.z, v3 = f.w;
          ss = ss + v0 * v0; ss = ss + v1 * v1; ss = ss + v2 * v2; ss = ss + v3 * v3;
        }
      } else {
        const uint4* rp = (const uint4*)((const unsigned short*)x.p + ro);
        for (int c = 0; c < D / 8; ++c) {
          const uint4 wv = rp[c];
          const unsigned int wd[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const unsigned short lo = (unsigned short)(wd[e] & 0xffffu), hi = (unsigned short)(wd[e] >> 16);
            const double v0 = (DT == kF16) ? widen_f16(lo) : widen_bf16(lo);
            const double v1 = (DT == kF16) ? widen_f16(hi) : widen_bf16(hi);
            ss = ss + v0 * v0;
            ss = ss + v1 * v1;
          }
        }
      }
      const double nrm = sqrt(ss);
      inv[half] = nrm > 0.0 ? 1.0 / nrm : 0.0;
    }
  }
  // pass 2: channel sums and unit-row sums
  double s[CPL], u[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) { s[c] = 0.0; u[c] = 0.0; }
  for (int rr = 0; rr < n; ++rr) {
    const double iv = readlane_f64(rr < 64 ? inv[0] : inv[1], rr & 63);
    const int64_t ro = base + (int64_t)rr * x.sN;
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const double v = ld<DT>(x.p, ro + CPL * lane + c);
      s[c] = s[c] + v;
      u[c] = u[c] + v * iv;
    }
  }
  double* means = isq ? qmean : kmean;
  const int nb = isq ? d.nQ : d.nK;
  double sq = 0.0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    means[mean_index(bh, pad16(nb), blk, CPL * lane + c, D)] = s[c] / (double)n;
    sq = sq + u[c] * u[c];
  }
  sq = wave_sum_f64(sq);
  if (lane == 0) (isq ? qsim : ksim)[(int64_t)bh * nb + blk] = sq / (double)(n * n);
}

// Pooled scores on the fp64 matrix cores (v_mfma_f64_16x16x4_f64): a wavefront
// computes a 16T x 16T tile as T x T MFMA tiles, a workgroup's four wavefronts a
// 32T x 32T one (T = 2 normally; T = 1 when that grid would leave most of the chip
// idle, as for short sequences).  In the MFMA's operand layout lane (r, kq) =
// (lane % 16, lane / 16) supplies row r of a 16-row tile at k = kq; at k-step s that
// is channel (D/4) kq + s, the same channel for the Q and the K operand.  The means
// are stored in that order (mean_index), so each 16-byte load of a wavefront (two
// k-steps of one 16-row tile) is 1 KB of contiguous memory.  Every pair sums all D
// products in fp64 in the same order for either T; only the association differs
// from a plain dot product.  Tiles and wavefront tiles holding no valid pair under
// causality are skipped; tiles past the padded ends re-read the last tile and rows
// and columns past the ends are not stored.
typedef double f64x4 __attribute__((ext_vector_type(4)));

template <int D, int T>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const double* qmean, const double* kmean,
                                                            Dims d, int causal, double scale,
                                                            double* scores) {
  constexpr int NP = D / 8;    // k-step pairs
  constexpr int CP = 4;        // pairs per chunk
  constexpr int WT = 16 * T;   // wavefront tile side
  const int j0 = blockIdx.x * 2 * WT, i0 = blockIdx.y * 2 * WT, bh = blockIdx.z;
  if (causal && j0 > 2 * (i0 + 2 * WT - 1) + 1) return;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int iw = i0 + WT * (w >> 1), jw = j0 + WT * (w & 1);
  // no barriers below, so a wavefront with no valid pair may leave early
  if (causal && jw > 2 * (iw + WT - 1) + 1) return;
  const int nQp = pad16(d.nQ), nKp = pad16(d.nK);
  const double2* qa[T];
  const double2* kb[T];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    qa[t] = (const double2*)(qmean + ((int64_t)bh * nQp + min(iw + 16 * t, nQp - 16)) * D) + lane;
    kb[t] = (const double2*)(kmean + ((int64_t)bh * nKp + min(jw + 16 * t, nKp - 16)) * D) + lane;
  }
  double2 a[2][T][CP], b[2][T][CP];   // [buffer][tile][pair]
  auto load = [&](int buf, int p0) {
#pragma unroll
    for (int t = 0; t < T; ++t)
#pragma unroll
      for (int e = 0; e < CP; ++e) {
        a[buf][t][e] = qa[t][64 * (p0 + e)];
        b[buf][t][e] = kb[t][64 * (p0 + e)];
      }
  };
  f64x4 acc[T][T];
#pragma unroll
  for (int ti = 0; ti < T; ++ti)
#pragma unroll
    for (int tj = 0; tj < T; ++tj) acc[ti][tj] = (f64x4)(0.0);
  load(0, 0);
#pragma unroll
  for (int c = 0; c < NP / CP; ++c) {
    const int cur = c & 1;
    if (c + 1 < NP / CP) load(cur ^ 1, (c + 1) * CP);
#pragma unroll
    for (int e = 0; e < CP; ++e)
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int ti = 0; ti < T; ++ti)
#pragma unroll
          for (int tj = 0; tj < T; ++tj) {
            const double av = half ? a[cur][ti][e].y : a[cur][ti][e].x;
            const double bv = half ? b[cur][tj][e].y : b[cur][tj][e].x;
            acc[ti][tj] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[ti][tj], 0, 0, 0);
          }
  }
  // lane (r, kq) holds rows kq + 4e (e = 0..3) of column r of each output tile
  const int r = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int ti = 0; ti < T; ++ti)
#pragma unroll
    for (int tj = 0; tj < T; ++tj) {
      const int j = jw + 16 * tj + r;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = iw + 16 * ti + kq + 4 * e;
        if (i < d.nQ && j < d.nK) scores[((int64_t)bh * d.nQ + i) * d.nK + j] = scale * acc[ti][tj][e];
      }
    }
}

// Order-preserving map of an fp64 score to uint64 (larger score -> larger key);
// -0.0 is folded onto +0.0 so that equal scores give equal keys.
__device__ __forceinline__ unsigned long long order_key(double s) {
  s = s + 0.0;
  const unsigned long long b = (unsigned long long)__double_as_longlong(s);
  return (b >> 63) ? ~b : (b | 0x8000000000000000ull);
}

__device__ __forceinline__ int keep_count(int C, double topk) {
  if (C == 0) return 0;
  const double x = topk * (double)C - 1e-9;
  int kk = (int)ceil(x);
  kk = kk < 1 ? 1 : kk;
  return kk > C ? C : kk;
}

// Wave-level reductions and scans on DPP lane moves and the gfx950 row swaps (no
// LDS round trips).  A butterfly inside each 16-lane row (partner lane^1 and lane^2
// by quad permutes, then the mirrored lane of the 8-lane half and of the row), then
// across rows (v_permlane16_swap: rows 0<->1 and 2<->3; v_permlane32_swap: the two
// halves); every lane receives the result.
template <int CTRL>
__device__ __forceinline__ unsigned int dpp_u32(unsigned int v) {
  return (unsigned int)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, true);
}
// the value of the partner lane in the row (S = 16) or half (S = 32) swap
template <int S>
__device__ __forceinline__ unsigned int swap_partner(unsigned int v) {
  const int lane = threadIdx.x & 63;
  if constexpr (S == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return ((lane >> 4) & 1) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane >> 5) ? r[0] : r[1];
  }
}
template <class F>
__device__ __forceinline__ unsigned int wave_allreduce_u32(unsigned int v, F op) {
  v = op(v, dpp_u32<0xb1>(v));     // quad_perm [1, 0, 3, 2]
  v = op(v, dpp_u32<0x4e>(v));     // quad_perm [2, 3, 0, 1]
  v = op(v, dpp_u32<0x141>(v));    // row_half_mirror
  v = op(v, dpp_u32<0x140>(v));    // row_mirror
  v = op(v, swap_partner<16>(v));
  v = op(v, swap_partner<32>(v));
  return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
  return (int)wave_allreduce_u32((unsigned int)v, [](unsigned int x, unsigned int y) { return x + y; });
}
template <class F>
__device__ __forceinline__ unsigned long long wave_allreduce_u64(unsigned long long v, F pick) {
  auto step = [&](unsigned int lo, unsigned int hi) {
    const unsigned long long o = ((unsigned long long)hi << 32) | lo;
    v = pick(v, o);
  };
#define SPARGE_STEP(EXPR_LO, EXPR_HI) step(EXPR_LO, EXPR_HI)
  SPARGE_STEP(dpp_u32<0xb1>((unsigned int)v), dpp_u32<0xb1>((unsigned int)(v >> 32)));
  SPARGE_STEP(dpp_u32<0x4e>((unsigned int)v), dpp_u32<0x4e>((unsigned int)(v >> 32)));
  SPARGE_STEP(dpp_u32<0x141>((unsigned int)v), dpp_u32<0x141>((unsigned int)(v >> 32)));
  SPARGE_STEP(dpp_u32<0x140>((unsigned int)v), dpp_u32<0x140>((unsigned int)(v >> 32)));
  SPARGE_STEP(swap_partner<16>((unsigned int)v), swap_partner<16>((unsigned int)(v >> 32)));
  SPARGE_STEP(swap_partner<32>((unsigned int)v), swap_partner<32>((unsigned int)(v >> 32)));
#undef SPARGE_STEP
  return v;
}
__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long v) {
  return wave_allreduce_u64(v, [](unsigned long long x, unsigned long long y) { return y > x ? y : x; });
}
__device__ __forceinline__ unsigned long long wave_min_u64(unsigned long long v) {
  return wave_allreduce_u64(v, [](unsigned long long x, unsigned long long y) { return y < x ? y : x; });
}
// Inclusive prefix sums over the lanes in lane order: shifts by 1, 2, 4 and 8 inside
// each row (lanes without a source add 0), then the last lane of row 0 (and of row
// 2) added to row 1 (row 3), then lane 31 added to rows 2 and 3.
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned int dpp_shift_u32(unsigned int v) {
  return (unsigned int)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROWS, 0xf, false);
}
template <int CTRL, int ROWS>
__device__ __forceinline__ unsigned long long dpp_shift_u64(unsigned long long v) {
  const unsigned long long lo = dpp_shift_u32<CTRL, ROWS>((unsigned int)v);
  const unsigned long long hi = dpp_shift_u32<CTRL, ROWS>((unsigned int)(v >> 32));
  return (hi << 32) | lo;
}
template <class T, class SH>
__device__ __forceinline__ T wave_incl_scan(T v, SH) {
  v += SH::template f<0x111, 0xf>(v);   // row_shr:1
  v += SH::template f<0x112, 0xf>(v);   // row_shr:2
  v += SH::template f<0x114, 0xf>(v);   // row_shr:4
  v += SH::template f<0x118, 0xf>(v);   // row_shr:8
  v += SH::template f<0x142, 0xa>(v);   // row_bcast:15 into rows 1 and 3
  v += SH::template f<0x143, 0xc>(v);   // row_bcast:31 into rows 2 and 3
  return v;
}
struct ShiftU32 {
  template <int CTRL, int ROWS> __device__ static unsigned int f(unsigned int v) { return dpp_shift_u32<CTRL, ROWS>(v); }
};
struct ShiftU64 {
  template <int CTRL, int ROWS> __device__ static unsigned long long f(unsigned long long v) {
    return dpp_shift_u64<CTRL, ROWS>(v);
  }
};
__device__ __forceinline__ unsigned int wave_incl_scan_u32(unsigned int v) { return wave_incl_scan(v, ShiftU32{}); }
__device__ __forceinline__ unsigned long long wave_incl_scan_u64(unsigned long long v) {
  return wave_incl_scan(v, ShiftU64{});
}

// Block selection, one wavefront per block row (b, h, i), four rows per workgroup
// and no workgroup barriers.  Lane l holds the keys of blocks j = l + 64m (m < MK,
// nK <= 64 MK), so every chunk m is 64 consecutive blocks in lane order.  The key T
// of the last kept rank is located exactly by a radix search over 8-bit digits: the
// leading bits shared by every candidate (from the wave's smallest and largest key)
// are skipped, then each pass histograms the keys that match the prefix found so
// far in the wavefront's own LDS bins and walks the bins from the largest digit,
// stopping as soon as a single key matches.
//   * top-k: the bins count keys; T is the key of rank k_i.
//   * threshold (CDF): the bins also sum the keys' softmax weights exp(s - s_max),
//     held as integers in units of 2^-51, so the sums are exact whatever order the
//     atomic adds land in; T is the key of the first rank whose cumulative weight
//     reaches tau times the total.
// Rows whose Q block is not similar keep every valid block, so they skip the search.
// Ties at T go to the lowest block indices; kept blocks are written in ascending
// order (one ballot per chunk).
constexpr int kSelMaxNK = 4096;   // 64 keys per lane

// inverse of order_key
__device__ __forceinline__ double key_to_double(unsigned long long k) {
  const unsigned long long b = (k >> 63) ? (k & 0x7fffffffffffffffull) : ~k;
  return __longlong_as_double((long long)b);
}

template <int MK, bool CDF>
__global__ __launch_bounds__(256) void select_wave_kernel(const double* scores, const double* qsim,
                                                          const double* ksim, Dims d, int causal,
                                                          SelectParams sp, uint8_t* mask_out,
                                                          uint16_t* lists, int* counts,
                                                          unsigned long long* counters) {
  __shared__ __attribute__((aligned(16))) unsigned int hist_s[4][256];
  __shared__ __attribute__((aligned(16))) unsigned long long whist_s[4][CDF ? 256 : 2];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * 4 + wv;
  // no workgroup barriers in this kernel, so a wavefront past the end may leave
  if (row >= (int64_t)d.B * d.H * d.nQ) return;
  unsigned int* hist = hist_s[wv];
  unsigned long long* whist = whist_s[wv];
  const int bh = (int)(row / d.nQ), i = (int)(row % d.nQ);
  const int h = bh % d.H;
  const double theta = sp.head_theta ? sp.head_theta[h] : sp.theta;
  const double sel = sp.head_sel ? sp.head_sel[h] : sp.sel;
  const int nK = d.nK;
  const int jv = causal ? min(nK, 2 * i + 2) : nK;
  const bool simq = qsim[row] >= theta;
  const double* srow = scores + row * nK;
  const double* ks = ksim + (int64_t)bh * nK;

  // similarity of the K blocks, then the scores of the valid ones.  The loads are
  // unconditional, with indices clamped into the row (lanes past the end re-read its
  // last entry), and all of a kind are in flight before the first is used.  Per-lane
  // bit masks over m record which blocks are in the row (inm), valid (validm),
  // similar (simkm) and candidates (candm).
  unsigned long long inm = 0ull, validm = 0ull, simkm = 0ull, candm = 0ull;
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    inm |= (unsigned long long)(lane + 64 * m < nK) << m;
    validm |= (unsigned long long)(lane + 64 * m < jv) << m;
  }
  {
    double kv[MK];
#pragma unroll
    for (int m = 0; m < MK; ++m) kv[m] = ks[min(lane + 64 * m, nK - 1)];
#pragma unroll
    for (int m = 0; m < MK; ++m) asm volatile("" : "+v"(kv[m]));
#pragma unroll
    for (int m = 0; m < MK; ++m) simkm |= (unsigned long long)(kv[m] >= theta) << m;
    simkm &= inm;
  }
  candm = validm & simkm;
  __builtin_amdgcn_sched_barrier(0);   // the score loads reuse the registers of these
  unsigned long long key[MK];
  {
    double sv[MK];
#pragma unroll
    for (int m = 0; m < MK; ++m) sv[m] = srow[min(lane + 64 * m, jv - 1)];
#pragma unroll
    for (int m = 0; m < MK; ++m) asm volatile("" : "+v"(sv[m]));
#pragma unroll
    for (int m = 0; m < MK; ++m) key[m] = order_key(sv[m]) & (0ull - ((candm >> m) & 1ull));
  }
  const int C = wave_sum_i32(__popcll(candm));
  auto is_cand = [&](int m) { return 64 * m < jv && ((candm >> m) & 1ull); };

  unsigned long long T = 0ull;
  int need = 0, kk = 0;
  if (simq && C > 0) {
    unsigned long long kmax = 0ull, kmin = ~0ull;
#pragma unroll
    for (int m = 0; m < MK; ++m)
      if (is_cand(m)) {
        kmax = key[m] > kmax ? key[m] : kmax;
        kmin = key[m] < kmin ? key[m] : kmin;
      }
    kmax = wave_max_u64(kmax);
    kmin = wave_min_u64(kmin);
    int krem = 0;                        // top-k: rank still to locate among prefix matches
    int n_above = 0;                     // CDF: candidates above the prefix
    unsigned long long A = 0ull;         // CDF: their weight
    unsigned long long target = 0ull;    // CDF: tau times the total weight
    unsigned long long wt[CDF ? MK : 1];
    bool found_t = false;
    if constexpr (CDF) {
      const double smax = key_to_double(kmax);
      unsigned long long zl = 0ull;
#pragma unroll
      for (int m = 0; m < MK; ++m) {
        wt[m] = 0ull;
        if (64 * m < jv) {   // chunks past the causal limit hold no candidate
          const double e = exp(key_to_double(key[m]) - smax);
          wt[m] = is_cand(m) ? (unsigned long long)(e * 0x1p51) : 0ull;
        }
        zl += wt[m];
      }
      const unsigned long long Z =
          wave_allreduce_u64(zl, [](unsigned long long x, unsigned long long y) { return x + y; });
      target = sel >= 1.0 ? Z : __umul64hi((unsigned long long)(sel * 0x1p64), Z);
      if (target == 0ull) {              // the first rank already reaches it
        T = kmax;
        found_t = true;
      }
    } else {
      kk = keep_count(C, sel);
      krem = kk;
    }
    int n_t = C;                         // keys equal to T (all of them when kmax == kmin)
    if (found_t) {
      n_t = 1;
    } else if (kmax == kmin) {
      T = kmax;                          // every candidate has the same key
    } else {
      // bytes above the highest differing bit are common to all candidates
      const int top = (63 - __clzll((long long)(kmax ^ kmin))) >> 3;
      unsigned long long pmask = top == 7 ? 0ull : (~0ull << (8 * (top + 1)));
      T = kmax & pmask;
      for (int byte = top; byte >= 0; --byte) {
        const int shift = 8 * byte;
        *(uint4*)(hist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
        if constexpr (CDF) {
          *(uint4*)(whist + 4 * lane) = make_uint4(0u, 0u, 0u, 0u);
          *(uint4*)(whist + 4 * lane + 2) = make_uint4(0u, 0u, 0u, 0u);
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int m = 0; m < MK; ++m)
          if (is_cand(m) && (key[m] & pmask) == T) {
            const unsigned int dg = (unsigned int)(key[m] >> shift) & 255u;
            atomicAdd(&hist[dg], 1u);
            if constexpr (CDF) atomicAdd(&whist[dg], wt[m]);
          }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        // lane l owns digits 255-4l .. 252-4l (descending); counts and weights above
        // it by scans over the lanes
        const uint4 cv = *(const uint4*)(hist + 252 - 4 * lane);
        const unsigned int c[4] = {cv.w, cv.z, cv.y, cv.x};
        const unsigned int tot = c[0] + c[1] + c[2] + c[3];
        unsigned int run = wave_incl_scan_u32(tot) - tot;
        unsigned long long w4[4] = {0ull, 0ull, 0ull, 0ull}, wrun = 0ull;
        if constexpr (CDF) {
#pragma unroll
          for (int e = 0; e < 4; ++e) w4[e] = whist[255 - 4 * lane - e];
          const unsigned long long wtot = (w4[0] + w4[1]) + (w4[2] + w4[3]);
          wrun = wave_incl_scan_u64(wtot) - wtot;
        }
        int found = -1;
        unsigned int above = 0u, here = 0u;
        unsigned long long wabove = 0ull;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool hit = CDF ? (c[e] > 0u && A + wrun + w4[e] >= target) : (run + c[e] >= (unsigned int)krem);
          if (found < 0 && hit) {
            found = 255 - (4 * lane + e);
            above = run;
            here = c[e];
            wabove = wrun;
          }
          run += c[e];
          wrun += w4[e];
        }
        const int src = __builtin_amdgcn_readfirstlane(__ffsll((long long)__ballot(found >= 0)) - 1);
        const int digit = __builtin_amdgcn_readlane(found, src);
        const int n_hi = __builtin_amdgcn_readlane((int)above, src);
        const unsigned int nhere = (unsigned int)__builtin_amdgcn_readlane((int)here, src);
        if constexpr (CDF) {
          A += ((unsigned long long)(unsigned int)__builtin_amdgcn_readlane((int)(wabove >> 32), src) << 32) |
               (unsigned int)__builtin_amdgcn_readlane((int)(unsigned int)wabove, src);
          n_above += n_hi;
        } else {
          krem -= n_hi;
        }
        // every lane has finished reading the bins before the next pass clears them
        __builtin_amdgcn_wave_barrier();
        T |= (unsigned long long)digit << shift;
        pmask |= 255ull << shift;
        n_t = (int)nhere;
        if (nhere == 1u && byte > 0) {
          // a single key matches the prefix: it is T
          unsigned long long mine = 0ull;
#pragma unroll
          for (int m = 0; m < MK; ++m)
            if (is_cand(m) && (key[m] & pmask) == T) mine = key[m];
          T = wave_max_u64(mine);
          break;
        }
      }
    }
    if constexpr (CDF) {
      if (found_t) {
        need = 1;
        kk = 1;
      } else {
        // the n_t keys equal to T share one weight w; in rank order the q-th of them
        // ends at cumulative weight A + q w, so the first to reach the target is
        // q = ceil((target - A) / w) (target > A > ... and A + n_t w >= target)
        unsigned long long mine = 0ull;
#pragma unroll
        for (int m = 0; m < MK; ++m)
          if (is_cand(m) && key[m] == T) mine = wt[m];
        const unsigned long long w = wave_max_u64(mine);
        const unsigned long long gap = target - A;
        unsigned long long q = w > 0ull ? (gap + w - 1ull) / w : 1ull;
        q = q < 1ull ? 1ull : (q > (unsigned long long)n_t ? (unsigned long long)n_t : q);
        need = (int)q;
        kk = n_above + need;
      }
    } else {
      need = krem;   // keys equal to T still to take, lowest block index first
    }
  }

  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_before = 0, base = 0;
  uint8_t* mrow = mask_out ? mask_out + row * nK : nullptr;
  uint16_t* lrow = lists + row * d.lstride;
  const bool selecting = simq && kk > 0;
#pragma unroll
  for (int m = 0; m < MK; ++m) {
    if (64 * m >= jv) {
      // no valid block in this chunk (causal rows): only the mask needs writing
      if (mrow && 64 * m < nK && ((inm >> m) & 1ull)) mrow[lane + 64 * m] = 0;
    } else {
      const int j = lane + 64 * m;
      const bool valid = (validm >> m) & 1ull, simk = (simkm >> m) & 1ull;
      const bool cand = (candm >> m) & 1ull;
      const bool is_eq = selecting && cand && key[m] == T;
      const unsigned long long eqm = __ballot(is_eq);
      const bool gt = selecting && cand && key[m] > T;
      const int rank = eq_before + __popcll(eqm & lt_mask);
      const bool keep = (valid && (!simq || !simk || gt)) || (is_eq && rank < need);
      if (mrow && ((inm >> m) & 1ull)) mrow[j] = keep ? 1 : 0;
      const unsigned long long km = __ballot(keep);
      if (keep) lrow[base + __popcll(km & lt_mask)] = (uint16_t)j;
      base += __popcll(km);
      eq_before += __popcll(eqm);
    }
  }
  if (lane == 0) {
    counts[row] = base;
    if (counters) {
      atomicAdd(&counters[0], (unsigned long long)jv);
      atomicAdd(&counters[1], (unsigned long long)base);
    }
  }
}

// One wavefront per block row: user mask (nonzero keeps) -> ascending list.
__global__ __launch_bounds__(64) void compact_kernel(const uint8_t* mask, Dims d, uint16_t* lists,
                                                     int* counts, unsigned long long* counters) {
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int nK = d.nK;
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  uint16_t* lrow = lists + row * d.lstride;
  for (int j0 = 0; j0 < nK; j0 += 64) {
    const int j = j0 + lane;
    const bool keep = j < nK && (mask == nullptr || mask[row * nK + j] != 0);
    const unsigned long long km = __ballot(keep);
    if (keep) lrow[base + __popcll(km & lt_mask)] = (uint16_t)j;
    base += __popcll(km);
  }
  if (lane == 0) {
    counts[row] = base;
    if (counters) {
      atomicAdd(&counters[0], (unsigned long long)nK);
      atomicAdd(&counters[1], (unsigned long long)base);
    }
  }
}

// Element-type conversion (fp32 / bf16 / fp16 -> bf16 or fp16, round to nearest
// even) into a contiguous (B, H, N, D) buffer; four elements per thread.
template <int SRC, bool DST_F16>
__global__ __launch_bounds__(256) void convert16_kernel(View x, Dims d, uint16_t* dst) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per_row = d.D / 4;
  const int64_t total = (int64_t)d.B * d.H * d.N * per_row;
  if (idx >= total) return;
  const int64_t rowi = idx / per_row;
  const int c = (int)(idx % per_row) * 4;
  const int n = (int)(rowi % d.N);
  const int64_t bhi = rowi / d.N;
  const int b = (int)(bhi / d.H), h = (int)(bhi % d.H);
  const int64_t src = (int64_t)b * x.sB + (int64_t)h * x.sH + (int64_t)n * x.sN + c;
  float vals[4];
  if constexpr (SRC == kF32) {
    const float4 v = *(const float4*)((const float*)x.p + src);
    vals[0] = v.x; vals[1] = v.y; vals[2] = v.z; vals[3] = v.w;
  } else {
    const ushort4 v = *(const ushort4*)((const unsigned short*)x.p + src);
    const unsigned short u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      vals[e] = (SRC == kF16) ? (float)__builtin_bit_cast(_Float16, u[e])
                              : __uint_as_float((unsigned int)u[e] << 16);
  }
  ushort4 w;
  unsigned short o[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if constexpr (DST_F16) o[e] = __builtin_bit_cast(unsigned short, (_Float16)vals[e]);
    else o[e] = __builtin_bit_cast(unsigned short, (__bf16)vals[e]);
  }
  w.x = o[0]; w.y = o[1]; w.z = o[2]; w.w = o[3];
  *(ushort4*)(dst + rowi * d.D + c) = w;
}

}  // namespace

hipError_t launch_block_stats(const View& q, const View& k, int dtype, const Dims& d,
                              double* qmean, double* qsim, double* kmean, double* ksim,
                              hipStream_t s) {
  const int64_t tasks = (int64_t)d.B * d.H * (d.nQ + d.nK);
  const dim3 grid((unsigned)((tasks + 3) / 4));
#define SPARGE_STATS(DTV, DV) \
  block_stats_kernel<DTV, DV><<<grid, 256, 0, s>>>(q, k, d, qmean, qsim, kmean, ksim)
  if (d.D == 64) {
    if (dtype == kF32) SPARGE_STATS(kF32, 64);
    else if (dtype == kF16) SPARGE_STATS(kF16, 64);
    else SPARGE_STATS(kBF16, 64);
  } else {
    if (dtype == kF32) SPARGE_STATS(kF32, 128);
    else if (dtype == kF16) SPARGE_STATS(kF16, 128);
    else SPARGE_STATS(kBF16, 128);
  }
#undef SPARGE_STATS
  return hipGetLastError();
}

hipError_t launch_pooled_scores(const double* qmean, const double* kmean, const Dims& d, int causal,
                                double scale, double* scores, hipStream_t s) {
  // 64 x 64 tiles per workgroup, or 32 x 32 when the larger tiles give under 1024
  // workgroups (short sequences: more, shorter wavefronts fill more of the chip)
  const int64_t big = (int64_t)((d.nK + 63) / 64) * ((d.nQ + 63) / 64) * d.B * d.H;
  const int side = big < 1024 ? 32 : 64;
  const dim3 grid((unsigned)((d.nK + side - 1) / side), (unsigned)((d.nQ + side - 1) / side),
                  (unsigned)(d.B * d.H));
#define SPARGE_POOLED(DV, TV) pooled_scores_kernel<DV, TV><<<grid, 256, 0, s>>>(qmean, kmean, d, causal, scale, scores)
  if (d.D == 64) {
    if (side == 32) SPARGE_POOLED(64, 1);
    else SPARGE_POOLED(64, 2);
  } else {
    if (side == 32) SPARGE_POOLED(128, 1);
    else SPARGE_POOLED(128, 2);
  }
#undef SPARGE_POOLED
  return hipGetLastError();
}

hipError_t launch_select(const double* scores, const double* qsim, const double* ksim,
                         const Dims& d, int causal, const SelectParams& sp, uint8_t* mask_out,
                         uint16_t* lists, int* counts, unsigned long long* counters,
                         hipStream_t s) {
  if (d.nK > kSelMaxNK) return hipErrorInvalidValue;
  const int64_t rows = (int64_t)d.B * d.H * d.nQ;
  const dim3 grid((unsigned)((rows + 3) / 4));
#define SPARGE_SEL(MKV)                                                                         \
  do {                                                                                          \
    if (sp.cdf)                                                                                 \
      select_wave_kernel<MKV, true><<<grid, 256, 0, s>>>(scores, qsim, ksim, d, causal, sp,     \
                                                         mask_out, lists, counts, counters);    \
    else                                                                                        \
      select_wave_kernel<MKV, false><<<grid, 256, 0, s>>>(scores, qsim, ksim, d, causal, sp,    \
                                                          mask_out, lists, counts, counters);   \
  } while (0)
  if (d.nK <= 64) SPARGE_SEL(1);
  else if (d.nK <= 128) SPARGE_SEL(2);
  else if (d.nK <= 256) SPARGE_SEL(4);
  else if (d.nK <= 512) SPARGE_SEL(8);
  else if (d.nK <= 1024) SPARGE_SEL(16);
  else if (d.nK <= 2048) SPARGE_SEL(32);
  else SPARGE_SEL(64);
#undef SPARGE_SEL
  return hipGetLastError();
}

hipError_t launch_compact(const uint8_t* mask, const Dims& d, uint16_t* lists, int* counts,
                          unsigned long long* counters, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)d.B * d.H * d.nQ));
  compact_kernel<<<grid, 64, 0, s>>>(mask, d, lists, counts, counters);
  return hipGetLastError();
}

hipError_t launch_convert16(const View& x, int src_dtype, const Dims& d, uint16_t* dst,
                            int dst_f16, hipStream_t s) {
  const int64_t chunks = (int64_t)d.B * d.H * d.N * (d.D / 4);
  const dim3 grid((unsigned)((chunks + 255) / 256));
#define SPARGE_CV(SV, DV) convert16_kernel<SV, DV><<<grid, 256, 0, s>>>(x, d, dst)
  if (src_dtype == kF32) { if (dst_f16) SPARGE_CV(kF32, true); else SPARGE_CV(kF32, false); }
  else if (src_dtype == kF16) { if (dst_f16) SPARGE_CV(kF16, true); else SPARGE_CV(kF16, false); }
  else { if (dst_f16) SPARGE_CV(kBF16, true); else SPARGE_CV(kBF16, false); }
#undef SPARGE_CV
  return hipGetLastError();
}

}  // namespace sparge
