// int8 operands of the quantized Q K^T option and the token reorder, for gfx950.
//
// int8 option (SageAttention base: 8-bit quantization with outlier smoothing,
// [topgit] "Key features"; [readme] "Avalible API").  Spec, all in IEEE fp32:
//   K: per 64-row block, kbar_j = fp32(fp64 row sum / rows); k'' = fp32(k) - kbar_j;
//      a = max|k''|; codes = clamp(rint(k'' * (127 / a)), -127, 127); step a / 127;
//   Q: per 32-row group, a = max|q|, the same rounding, step a / 127 (made by the
//      attention kernel itself, in registers).
// Every quantity that decides an integer code is computed in the same precision
// and order as the reference steps: fp64 sums, IEEE fp32 division, subtraction,
// product and round-half-to-even.
//
// Reorder ([chapterpal] method paragraph and recommendations: Hilbert-curve token
// order for visual inputs): gather / scatter of whole token rows by a permutation.
#include "sparge_internal.hpp"

#pragma clang fp contract(off)

namespace sparge {
namespace {

template <int DT>
__device__ __forceinline__ float ldf(const void* base, int64_t idx) {
  if constexpr (DT == kF32) return ((const float*)base)[idx];
  else if constexpr (DT == kF16) return (float)__builtin_bit_cast(_Float16, ((const unsigned short*)base)[idx]);
  else return __uint_as_float((unsigned int)(((const unsigned short*)base)[idx]) << 16);
}

__device__ __forceinline__ float wave_max_f32(float v) {
  for (int off = 32; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
  return v;
}

__device__ __forceinline__ signed char quant_code(float x, float inv) {
  float c = __builtin_rintf(x * inv);
  c = fminf(fmaxf(c, -127.0f), 127.0f);
  return (signed char)(int)c;
}

// One wavefront per (b, h, K block), one pass over K: lane owns D/64 channels and
// keeps the block's 64 rows of them in registers (sums in fp64 in row order, then
// the mean, the max deviation and the codes, all from registers).
template <int DT, int D>
__global__ __launch_bounds__(256) void quant_k_kernel(View k, Dims d, int8_t* codes,
                                                      int64_t crow, int64_t chead, int64_t rows_alloc,
                                                      float* kscale, float* kbar) {
  constexpr int CPL = D / 64;
  const int lane = threadIdx.x & 63;
  const int64_t task = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= (int64_t)d.B * d.H * d.nK) return;
  const int bh = (int)(task / d.nK), j = (int)(task % d.nK);
  const int b = bh / d.H, h = bh % d.H;
  const int r0 = j * kBK, n = min(kBK, d.N - r0);
  const int64_t base = (int64_t)b * k.sB + (int64_t)h * k.sH + (int64_t)r0 * k.sN;
  float x[kBK][CPL];
#pragma unroll
  for (int r = 0; r < kBK; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      x[r][c] = (r < n) ? ldf<DT>(k.p, base + (int64_t)r * k.sN + CPL * lane + c) : 0.0f;
  double s[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) s[c] = 0.0;
#pragma unroll
  for (int r = 0; r < kBK; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (r < n) s[c] = s[c] + (double)x[r][c];
  float mean[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) mean[c] = (float)(s[c] / (double)n);
  float a = 0.0f;
#pragma unroll
  for (int r = 0; r < kBK; ++r)
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      if (r < n) a = fmaxf(a, fabsf(x[r][c] - mean[c]));
  a = wave_max_f32(a);
  const float inv = a > 0.0f ? 127.0f / a : 0.0f;
  int8_t* cb = codes + (int64_t)bh * chead;
#pragma unroll
  for (int r = 0; r < kBK; ++r) {
    const int64_t row = (int64_t)r0 + r;
    if (row >= rows_alloc) break;
    signed char cc[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      cc[c] = (r < n && a > 0.0f) ? quant_code(x[r][c] - mean[c], inv) : (signed char)0;
    if constexpr (CPL == 2) {
      const unsigned short packed = (unsigned short)((unsigned char)cc[0] | ((unsigned char)cc[1] << 8));
      *(unsigned short*)(cb + row * crow + 2 * lane) = packed;
    } else {
      cb[row * crow + lane] = cc[0];
    }
  }
  if (lane == 0) kscale[(int64_t)bh * d.nK + j] = a > 0.0f ? a / 127.0f : 0.0f;
  float* mb = kbar + ((int64_t)bh * d.nK + j) * D;
#pragma unroll
  for (int c = 0; c < CPL; ++c) mb[CPL * lane + c] = mean[c];
}

// One thread per 16-byte chunk of an output row.
__global__ __launch_bounds__(256) void reorder_kernel(View x, void* y, int64_t ysB, int64_t ysH,
                                                      int64_t ysN, int esize, Dims d,
                                                      const int32_t* perm, int64_t offset,
                                                      int64_t count, int inverse) {
  const int chunks = d.D * esize / 16;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t total = (int64_t)d.B * d.H * d.N * chunks;
  if (idx >= total) return;
  const int c = (int)(idx % chunks);
  const int64_t rowi = idx / chunks;
  const int64_t n = rowi % d.N;
  const int64_t bhi = rowi / d.N;
  const int64_t b = bhi / d.H, h = bhi % d.H;
  int64_t src = n, dst = n;
  if (n >= offset && n < offset + count) {
    int64_t pp = perm[n - offset];
    pp = pp < 0 ? 0 : (pp >= count ? count - 1 : pp);
    if (inverse) dst = offset + pp;
    else src = offset + pp;
  }
  const char* xs = (const char*)x.p + (b * x.sB + h * x.sH + src * x.sN) * esize;
  char* yd = (char*)y + (b * ysB + h * ysH + dst * ysN) * esize;
  *(uint4*)(yd + 16 * c) = *(const uint4*)(xs + 16 * c);
}

// Two-level int8 codes of the block means, for the q . kbar term of the int8
// Q K^T on the int8 MFMA: one workgroup per (b, h); a = max_j,c |kbar_j[c]|,
// step a / 127 (0 when a = 0), and per element, with y = kbar * (127 / a),
// c1 = clamp(rint(y), +-127) and c2 = clamp(rint((y - c1) * 256), +-127), so that
// kbar ~= step (c1 + c2 / 256) within step / 512.
template <int D>
__global__ __launch_bounds__(1024) void kbar_codes_kernel(const float* kbar, Dims d, int8_t* kc,
                                                          float* kcs) {
  const int bh = blockIdx.x;
  const int64_t n = (int64_t)d.nK * D;
  const float* src = kbar + (int64_t)bh * n;
  float m = 0.0f;
  for (int64_t e = 4 * (int64_t)threadIdx.x; e < n; e += 4 * 1024) {
    const float4 v = *(const float4*)(src + e);
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  m = wave_max_f32(m);
  __shared__ float wm[16];
  if ((threadIdx.x & 63) == 0) wm[threadIdx.x >> 6] = m;
  __syncthreads();
  m = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; ++i) m = fmaxf(m, wm[i]);
  const float inv = m > 0.0f ? 127.0f / m : 0.0f;
  if (threadIdx.x == 0) kcs[bh] = m > 0.0f ? m / 127.0f : 0.0f;
  int8_t* dst = kc + (int64_t)bh * n * 2;
  for (int64_t e = 4 * (int64_t)threadIdx.x; e < n; e += 4 * 1024) {
    const float4 v = *(const float4*)(src + e);
    const float x[4] = {v.x, v.y, v.z, v.w};
    unsigned int w1 = 0, w2 = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = x[i] * inv;
      const float c1 = fminf(fmaxf(__builtin_rintf(y), -127.0f), 127.0f);
      const float c2 = fminf(fmaxf(__builtin_rintf((y - c1) * 256.0f), -127.0f), 127.0f);
      w1 |= ((unsigned int)(int)c1 & 0xffu) << (8 * i);
      w2 |= ((unsigned int)(int)c2 & 0xffu) << (8 * i);
    }
    const int64_t j = e / D, c = e % D;
    *(unsigned int*)(dst + j * 2 * D + c) = w1;
    *(unsigned int*)(dst + j * 2 * D + D + c) = w2;
  }
}

}  // namespace

hipError_t launch_kbar_codes(const float* kbar, const Dims& d, int8_t* kc, float* kcs, hipStream_t s) {
  const dim3 grid((unsigned)(d.B * d.H));
  if (d.D == 64) kbar_codes_kernel<64><<<grid, 1024, 0, s>>>(kbar, d, kc, kcs);
  else kbar_codes_kernel<128><<<grid, 1024, 0, s>>>(kbar, d, kc, kcs);
  return hipGetLastError();
}

hipError_t launch_quant_k(const View& k, int dtype, const Dims& d, int8_t* codes,
                          int64_t codes_row_stride, int64_t codes_head_stride, float* kscale,
                          float* kbar, hipStream_t s) {
  const int64_t tasks = (int64_t)d.B * d.H * d.nK;
  const dim3 grid((unsigned)((tasks + 3) / 4));
  const int64_t rows_alloc = codes_head_stride / codes_row_stride;
#define SPARGE_QK(DTV, DV) \
  quant_k_kernel<DTV, DV><<<grid, 256, 0, s>>>(k, d, codes, codes_row_stride, codes_head_stride, \
                                               rows_alloc, kscale, kbar)
  if (d.D == 64) {
    if (dtype == kF32) SPARGE_QK(kF32, 64);
    else if (dtype == kF16) SPARGE_QK(kF16, 64);
    else SPARGE_QK(kBF16, 64);
  } else {
    if (dtype == kF32) SPARGE_QK(kF32, 128);
    else if (dtype == kF16) SPARGE_QK(kF16, 128);
    else SPARGE_QK(kBF16, 128);
  }
#undef SPARGE_QK
  return hipGetLastError();
}

hipError_t launch_reorder(const View& x, void* y, int64_t ysB, int64_t ysH, int64_t ysN,
                          int esize, const Dims& d, const int32_t* perm, int64_t offset,
                          int64_t count, int inverse, hipStream_t s) {
  const int chunks = d.D * esize / 16;
  const int64_t total = (int64_t)d.B * d.H * d.N * chunks;
  const dim3 grid((unsigned)((total + 255) / 256));
  reorder_kernel<<<grid, 256, 0, s>>>(x, y, ysB, ysH, ysN, esize, d, perm, offset, count, inverse);
  return hipGetLastError();
}

}  // namespace sparge
