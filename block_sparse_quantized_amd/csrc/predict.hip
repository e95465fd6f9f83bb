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
//     plus every valid block of a non-similar row or column.
// All arithmetic that decides the mask runs in IEEE fp64 with no fused
// multiply-adds outside the dot products, following the reference steps.
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
// lanes) accumulates the channel sums and the sum of unit rows in row order.
template <int DT, int D>
__global__ __launch_bounds__(256) void block_stats_kernel(View q, View k, Dims d, double* qsum,
                                                          double* qsim, double* ksum,
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
  double* sums = isq ? qsum : ksum;
  const int nb = isq ? d.nQ : d.nK;
  double* out = sums + ((int64_t)bh * nb + blk) * D;
  double sq = 0.0;
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    out[CPL * lane + c] = s[c];
    sq = sq + u[c] * u[c];
  }
  sq = wave_sum_f64(sq);
  if (lane == 0) (isq ? qsim : ksim)[(int64_t)bh * nb + blk] = sq / (double)(n * n);
}

// Pooled scores, one 32 (i) x 64 (j) tile per workgroup of 256 threads; means are
// formed from the sums (fp64 division) while staging through LDS in 32-channel
// chunks.  Tiles holding no valid pair under causality are skipped.
template <int D>
__global__ __launch_bounds__(256) void pooled_scores_kernel(const double* qsum, const double* ksum,
                                                            Dims d, int causal, double scale,
                                                            double* scores) {
  constexpr int DC = 32;
  __shared__ double qm[32][DC + 1];
  __shared__ double km[64][DC + 1];
  const int j0 = blockIdx.x * 64, i0 = blockIdx.y * 32, bh = blockIdx.z;
  if (causal && j0 > 2 * (i0 + 31) + 1) return;
  const int tid = threadIdx.x;
  const int ti = tid / 16, tj = tid % 16;
  double acc[2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[a][c] = 0.0;
  for (int c0 = 0; c0 < D; c0 += DC) {
    for (int e = tid; e < 32 * DC; e += 256) {
      const int ri = e / DC, cc = e % DC, i = i0 + ri;
      double v = 0.0;
      if (i < d.nQ) {
        const int n = min(kBQ, d.N - i * kBQ);
        v = qsum[((int64_t)bh * d.nQ + i) * D + c0 + cc] / (double)n;
      }
      qm[ri][cc] = v;
    }
    for (int e = tid; e < 64 * DC; e += 256) {
      const int rj = e / DC, cc = e % DC, j = j0 + rj;
      double v = 0.0;
      if (j < d.nK) {
        const int n = min(kBK, d.N - j * kBK);
        v = ksum[((int64_t)bh * d.nK + j) * D + c0 + cc] / (double)n;
      }
      km[rj][cc] = v;
    }
    __syncthreads();
#pragma unroll 4
    for (int cc = 0; cc < DC; ++cc) {
      const double a0 = qm[2 * ti][cc], a1 = qm[2 * ti + 1][cc];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double bv = km[tj + 16 * c][cc];
        acc[0][c] = fma(a0, bv, acc[0][c]);
        acc[1][c] = fma(a1, bv, acc[1][c]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int i = i0 + 2 * ti + a;
    if (i >= d.nQ) continue;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j = j0 + tj + 16 * c;
      if (j < d.nK) scores[((int64_t)bh * d.nQ + i) * d.nK + j] = scale * acc[a][c];
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

// One wavefront per block row (b, h, i).  Candidate keys sit in LDS; the k-th
// largest key is found exactly by an 8-pass radix select (8-bit digits from the
// most significant, an LDS histogram per pass and a wavefront suffix scan), ties at
// the threshold go to the lowest block indices, and the kept blocks are compacted
// in ascending order with ballots.
__global__ __launch_bounds__(64) void select_kernel(const double* scores, const double* qsim,
                                                    const double* ksim, Dims d, int causal,
                                                    double topk, double theta, uint8_t* mask_out,
                                                    uint16_t* lists, int* counts,
                                                    unsigned long long* counters) {
  extern __shared__ unsigned long long keys[];  // nK entries
  unsigned char* flags = (unsigned char*)(keys + d.nK);  // bit0 valid, bit1 similar-K
  __shared__ unsigned int hist[256];
  const int lane = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int bh = (int)(row / d.nQ), i = (int)(row % d.nQ);
  const int nK = d.nK;
  const int jv = causal ? min(nK, 2 * i + 2) : nK;
  const bool simq = qsim[row] >= theta;
  const double* srow = scores + row * nK;
  const double* ks = ksim + (int64_t)bh * nK;
  int cand_local = 0;
  for (int j = lane; j < nK; j += 64) {
    const bool valid = j < jv;
    const bool simk = ks[j] >= theta;
    flags[j] = (unsigned char)((valid ? 1 : 0) | (simk ? 2 : 0));
    keys[j] = (valid && simk) ? order_key(srow[j]) : 0ull;
    cand_local += (valid && simk) ? 1 : 0;
  }
  for (int off = 32; off >= 1; off >>= 1) cand_local += __shfl_xor(cand_local, off, 64);
  const int C = cand_local;
  const int kk = keep_count(C, topk);
  const int jhi = (jv < nK) ? jv : nK;  // candidates only exist below jv
  unsigned long long T = 0ull, pmask = 0ull;
  int need = 0;
  if (kk > 0) {
    int krem = kk;  // rank still to be located among keys matching the prefix
    for (int pass = 0; pass < 8; ++pass) {
      const int shift = 56 - 8 * pass;
      for (int b = lane; b < 256; b += 64) hist[b] = 0u;
      __syncthreads();
      for (int j = lane; j < jhi; j += 64) {
        if (flags[j] == 3) {
          const unsigned long long key = keys[j];
          if ((key & pmask) == T) atomicAdd(&hist[(unsigned int)(key >> shift) & 255u], 1u);
        }
      }
      __syncthreads();
      // lane l owns digits 255-4l .. 252-4l (descending); suffix counts by scan
      unsigned int c[4], tot = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        c[e] = hist[255 - (4 * lane + e)];
        tot += c[e];
      }
      unsigned int incl = tot;
      for (int off = 1; off < 64; off <<= 1) {
        const unsigned int y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      unsigned int run = incl - tot;  // keys with a larger digit than this lane's range
      int found = -1;
      unsigned int above = 0u;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        if (found < 0 && run + c[e] >= (unsigned int)krem) {
          found = 255 - (4 * lane + e);
          above = run;
        }
        run += c[e];
      }
      const unsigned long long fm = __ballot(found >= 0);
      const int src = __ffsll((long long)fm) - 1;
      const int dsel = __shfl(found, src, 64);
      const unsigned int abv = __shfl(above, src, 64);
      T |= (unsigned long long)dsel << shift;
      pmask |= 255ull << shift;
      krem -= (int)abv;
      __syncthreads();
    }
    need = krem;  // keys equal to T still to take (lowest block index first)
  }
  const unsigned long long lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int eq_before = 0, base = 0;
  uint8_t* mrow = mask_out ? mask_out + row * nK : nullptr;
  uint16_t* lrow = lists + row * d.lstride;
  for (int j0 = 0; j0 < nK; j0 += 64) {
    const int j = j0 + lane;
    const unsigned f = j < nK ? flags[j] : 0u;
    const bool valid = (f & 1u) != 0, simk = (f & 2u) != 0;
    const bool cand = valid && simk;
    const unsigned long long key = j < nK ? keys[j] : 0ull;
    const bool is_eq = cand && kk > 0 && key == T;
    const unsigned long long eqm = __ballot(is_eq);
    const int rank = eq_before + __popcll(eqm & lt_mask);
    eq_before += __popcll(eqm);
    const bool sel = cand && kk > 0 && (key > T || (is_eq && rank < need));
    const bool keep = valid && (!simq || !simk || sel);
    if (mrow && j < nK) mrow[j] = keep ? 1 : 0;
    const unsigned long long km = __ballot(keep);
    if (keep) lrow[base + __popcll(km & lt_mask)] = (uint16_t)j;
    base += __popcll(km);
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
                              double* qsum, double* qsim, double* ksum, double* ksim,
                              hipStream_t s) {
  const int64_t tasks = (int64_t)d.B * d.H * (d.nQ + d.nK);
  const dim3 grid((unsigned)((tasks + 3) / 4));
#define SPARGE_STATS(DTV, DV) \
  block_stats_kernel<DTV, DV><<<grid, 256, 0, s>>>(q, k, d, qsum, qsim, ksum, ksim)
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

hipError_t launch_pooled_scores(const double* qsum, const double* ksum, const Dims& d, int causal,
                                double scale, double* scores, hipStream_t s) {
  const dim3 grid((unsigned)((d.nK + 63) / 64), (unsigned)((d.nQ + 31) / 32),
                  (unsigned)(d.B * d.H));
  if (d.D == 64)
    pooled_scores_kernel<64><<<grid, 256, 0, s>>>(qsum, ksum, d, causal, scale, scores);
  else
    pooled_scores_kernel<128><<<grid, 256, 0, s>>>(qsum, ksum, d, causal, scale, scores);
  return hipGetLastError();
}

hipError_t launch_select(const double* scores, const double* qsim, const double* ksim,
                         const Dims& d, int causal, double topk, double theta, uint8_t* mask_out,
                         uint16_t* lists, int* counts, unsigned long long* counters,
                         hipStream_t s) {
  const size_t lds = (size_t)d.nK * (sizeof(unsigned long long) + 1);
  const dim3 grid((unsigned)((int64_t)d.B * d.H * d.nQ));
  select_kernel<<<grid, 64, lds, s>>>(scores, qsim, ksim, d, causal, topk, theta, mask_out, lists,
                                      counts, counters);
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
