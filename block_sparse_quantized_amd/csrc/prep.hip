// Fused preparation pass of the top-k path on gfx950: one read of Q, K and V
// produces everything the predictor and the attention kernel need before the
// pooled scores.
//
//   * Q blocks (128 rows) and K blocks (64 rows): channel means in fp64 and the
//     block self-similarity || sum_r x_r/||x_r|| ||^2 / n^2 ([chapterpal] method
//     paragraph: blocks with high internal similarity are compressed to their mean;
//     [topgit] "Key features": 128 x 64 blocks);
//   * optionally the block-smoothed int8 K of the SageAttention base ([topgit]
//     "Key features"; [readme] "Avalible API"): kbar_j = fp32(fp64 row sum / rows),
//     k'' = fp32(k) - kbar_j, a = max|k''| over the block, codes =
//     clamp(rint(k'' * (127 / a)), -127, 127), step a / 127, all in IEEE fp32;
//   * optionally V rounded (to nearest even) from bf16 to fp16 for the fp16 P.V, or,
//     for the fp8 P.V, the block's per-channel max |v| (reduced over the sequence by
//     vscale_kernel; vt8_kernel then writes V as E4M3 codes in transposed 64-token
//     tiles, see below).
//
// One workgroup of 256 threads per (b, h, Q block i): Q rows 128i..128i+127, the
// K blocks 2i and 2i+1 over the same rows, and the same V rows.  Every 16-byte
// chunk of the three tiles is loaded once, up front (coalesced: sixteen (D=128)
// or eight (D=64) consecutive lanes read one row; raw buffer loads, so rows past N
// read as zeros without a predicate), and kept in registers.  Row
// norms come from the registers (lane partials, then a reduction across the
// row's lanes); the channel pass reads a copy of the tile in LDS (row pitch
// padded by 16 bytes); the int8 codes come from the registers again and leave
// as 8-byte stores.
#include "sparge_internal.hpp"

#pragma clang fp contract(off)

namespace sparge {
namespace {

constexpr int kPad = 16;  // bytes of padding per LDS tile row
constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer resource: 32-bit data format

__device__ __forceinline__ float u16_to_f32(unsigned short u, bool f16) {
  return f16 ? (float)__builtin_bit_cast(_Float16, u) : __uint_as_float((unsigned int)u << 16);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) {
  const long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(b & 0xffffffffll), m, 64);
  const int hi = __shfl_xor((int)(b >> 32), m, 64);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum of v over each group of G consecutive lanes (G = 8 or 16), returned to every
// lane of the group, by DPP lane swaps: partner lane^1, lane^2 (quad permutes),
// the mirrored lane of the 8-lane half, then of the 16-lane row.
template <int DPP>
__device__ __forceinline__ double dpp_f64(double v) {
  const long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)(b & 0xffffffffll), DPP, 0xf, 0xf, true);
  const int hi = __builtin_amdgcn_mov_dpp((int)(b >> 32), DPP, 0xf, 0xf, true);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}
template <int G>
__device__ __forceinline__ double group_sum_f64(double v) {
  v = v + dpp_f64<0xb1>(v);    // quad_perm [1, 0, 3, 2]
  v = v + dpp_f64<0x4e>(v);    // quad_perm [2, 3, 0, 1]
  v = v + dpp_f64<0x141>(v);   // row_half_mirror
  if constexpr (G == 16) v = v + dpp_f64<0x140>(v);   // row_mirror
  return v;
}

__device__ __forceinline__ signed char quant_code(float x, float inv) {
  float c = __builtin_rintf(x * inv);
  c = fminf(fmaxf(c, -127.0f), 127.0f);
  return (signed char)(int)c;
}

// VMODE: 0 leave V alone, 1 write the fp16 copy, 2 write per-channel max |v| of
// the block's rows (fp8 P.V).
template <int DT, int D, bool QUANT, int VMODE>
__global__ __launch_bounds__(256) void prep_kernel(View q, View k, View v, Dims d, double* qmean,
                                                   double* qsim, double* kmean, double* ksim,
                                                   int8_t* codes, int64_t codes_head_stride,
                                                   int64_t codes_rows, float* kscale, float* kbar,
                                                   uint16_t* v16, float* vmaxp) {
  constexpr bool VCONV = VMODE != 0;
  constexpr bool F16 = DT == kF16;
  constexpr int CH = D / 8;               // 16-byte chunks per row
  constexpr int NCH = 128 * CH / 256;     // chunks per thread
  constexpr int ROWB = 2 * D + kPad;      // LDS bytes per tile row
  constexpr int TPC = 256 / D;            // threads per channel in the channel pass
  __shared__ __attribute__((aligned(16))) unsigned char tile[128 * ROWB];
  __shared__ double inv_s[128];
  __shared__ double part_s[256], part_u[256];
  __shared__ double sq_s[4];
  __shared__ float mean_s[2][D];
  __shared__ float amax_s[4][2];
  __shared__ float vmx_s[VMODE == 2 ? 256 / (D / 8) : 1][D];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int bh = blockIdx.x / d.nQ, i = blockIdx.x - bh * d.nQ;
  const int b = bh / d.H, h = bh - b * d.H;
  const int N = d.N;
  const int r0 = 128 * i;
  const int nrows = min(128, N - r0);

  // every chunk of the three tiles, issued before any arithmetic.  Chunk kk of a thread
  // is row tid / CH + RPK kk: each slab of RPK rows is read by raw buffer loads over a
  // resource that spans the slab's rows below N (base, byte extent), so rows past N
  // read as zeros with no predicate and no 64-bit address per lane; the lane offsets
  // stay below 2^31 because row strides are below 64 MiB.
  constexpr int RPK = 256 / CH;           // rows per slab
  uint4 qr[NCH], kr[NCH], vr[NCH];
  const int lrow = tid / CH, lch = tid % CH;
  struct Slabs {
    const char* base;   // row r0 of this (b, h)
    int rowb;           // bytes per row
  };
  auto slabs = [&](const View& x) {
    return Slabs{(const char*)x.p + 2 * ((int64_t)b * x.sB + (int64_t)h * x.sH + (int64_t)r0 * x.sN),
                 (int)(2 * x.sN)};
  };
  auto slab_load = [&](const Slabs& s, int kk) -> uint4 {
    const int rows = min(RPK, nrows - RPK * kk);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(s.base + (int64_t)(RPK * kk) * s.rowb), (short)0,
        rows > 0 ? (rows - 1) * s.rowb + 2 * D : 0, kRsrcWord3);
    const auto w = __builtin_amdgcn_raw_buffer_load_b128(r, lrow * s.rowb + 16 * lch, 0, 0);
    return make_uint4(w[0], w[1], w[2], w[3]);
  };
  const Slabs qs = slabs(q), ks = slabs(k), vs = slabs(v);
#pragma unroll
  for (int kk = 0; kk < NCH; ++kk) {
    qr[kk] = slab_load(qs, kk);
    kr[kk] = slab_load(ks, kk);
    if constexpr (VCONV) vr[kk] = slab_load(vs, kk);
  }

  // V, fp8 P.V: per-channel max |v| over the block's rows (each thread's chunk is 8
  // channels of one row; rows past N were loaded as zeros)
  if constexpr (VMODE == 2) {
    float mx[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) mx[c] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      const unsigned int wd[4] = {vr[kk].x, vr[kk].y, vr[kk].z, vr[kk].w};
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        mx[2 * c] = fmaxf(mx[2 * c], fabsf(u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16)));
        mx[2 * c + 1] = fmaxf(mx[2 * c + 1], fabsf(u16_to_f32((unsigned short)(wd[c] >> 16), F16)));
      }
    }
    // thread t covers channels 8 (t % CH) .. +7 of rows t / CH + (256 / CH) kk
    const int ch = tid % CH, rg = tid / CH;
#pragma unroll
    for (int c = 0; c < 8; ++c) vmx_s[rg][8 * ch + c] = mx[c];
    __syncthreads();
    if (tid < D) {
      float m = 0.0f;
      for (int r = 0; r < 256 / CH; ++r) m = fmaxf(m, vmx_s[r][tid]);
      vmaxp[((int64_t)bh * d.nQ + i) * D + tid] = m;
    }
  }

  // V: fp16 copy, rows < N only
  if constexpr (VMODE == 1) {
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      const int e = tid + 256 * kk, row = e / CH, ch = e % CH;
      if (row < nrows) {
        const unsigned int wd[4] = {vr[kk].x, vr[kk].y, vr[kk].z, vr[kk].w};
        unsigned int o[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const _Float16 lo = (_Float16)u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16);
          const _Float16 hi = (_Float16)u16_to_f32((unsigned short)(wd[c] >> 16), F16);
          o[c] = (unsigned int)__builtin_bit_cast(unsigned short, lo) |
                 ((unsigned int)__builtin_bit_cast(unsigned short, hi) << 16);
        }
        *(uint4*)(v16 + ((int64_t)bh * N + r0 + row) * D + 8 * ch) = make_uint4(o[0], o[1], o[2], o[3]);
      }
    }
  }

  // Row norms of the tile held in x[] (1/||x_r||, 0 for a zero row) into inv_s, and
  // the tile into LDS.  The CH lanes holding a row's chunks sum their squares across
  // the lane group (every lane gets the same total: each step adds two partial sums,
  // and addition commutes); then lane ch < NCH of each group takes the square root
  // and the division for chunk ch, so each row pays for them once.  The squares of
  // 16-bit inputs are exact in fp64, so the fused multiply-adds round exactly as a
  // product and a sum would.
  auto stage = [&](const uint4 (&x)[NCH]) {
    const int ch = tid % CH;
    double tot[NCH];
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      const int e = tid + 256 * kk, row = e / CH;
      const unsigned int wd[4] = {x[kk].x, x[kk].y, x[kk].z, x[kk].w};
      double ss = 0.0;
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double lo = u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16);
        const double hi = u16_to_f32((unsigned short)(wd[c] >> 16), F16);
        ss = fma(lo, lo, ss);
        ss = fma(hi, hi, ss);
      }
      tot[kk] = group_sum_f64<CH>(ss);
      *(uint4*)(tile + row * ROWB + 16 * ch) = x[kk];
    }
    if (ch < NCH) {
      double ss = tot[0];
#pragma unroll
      for (int kk = 1; kk < NCH; ++kk) ss = (ch == kk) ? tot[kk] : ss;
      const double nrm = sqrt(ss);
      inv_s[(tid + 256 * ch) / CH] = nrm > 0.0 ? 1.0 / nrm : 0.0;
    }
  };
  // Channel sums s and unit-row sums u of tile rows [lo, hi) for this thread's
  // channel, in row order.  Eight rows at a time: their LDS reads are all issued
  // before the first sum needs one, so the pass waits for LDS once per eight rows.
  auto channel_pass = [&](int c, int lo, int hi, double& s, double& u) {
    s = 0.0;
    u = 0.0;
    int r = lo;
    for (; r + 8 <= hi; r += 8) {
      unsigned short xr[8];
      double iv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        xr[e] = *(const unsigned short*)(tile + (r + e) * ROWB + 2 * c);
        iv[e] = inv_s[r + e];
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const double x = u16_to_f32(xr[e], F16);
        s = s + x;
        u = fma(x, iv[e], u);
      }
    }
    for (; r < hi; ++r) {
      const double x = u16_to_f32(*(const unsigned short*)(tile + r * ROWB + 2 * c), F16);
      s = s + x;
      u = fma(x, inv_s[r], u);
    }
  };

  // ---- Q block i
  stage(qr);
  __syncthreads();
  {
    constexpr int RPP = 128 / TPC;
    const int c = tid % D, part = tid / D;
    double s, u;
    channel_pass(c, part * RPP, min(part * RPP + RPP, nrows), s, u);
    part_s[tid] = s;
    part_u[tid] = u;
    __syncthreads();
    double sq = 0.0;
    if (tid < D) {
      double S = 0.0, U = 0.0;
#pragma unroll
      for (int pp = 0; pp < TPC; ++pp) {
        S = S + part_s[pp * D + tid];
        U = U + part_u[pp * D + tid];
      }
      qmean[mean_index(bh, pad16(d.nQ), i, tid, D)] = S / (double)nrows;
      sq = U * U;
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sq = sq + shfl_xor_f64(sq, m);
    if (lane == 0) sq_s[wv] = sq;
    __syncthreads();
    if (tid == 0) {
      double t = 0.0;
      for (int w2 = 0; w2 < D / 64; ++w2) t = t + sq_s[w2];
      qsim[(int64_t)bh * d.nQ + i] = t / (double)(nrows * nrows);
    }
  }
  __syncthreads();  // the tile and inv_s are reused for K

  // ---- K blocks 2i and 2i+1
  stage(kr);
  __syncthreads();
  int nb[2];
  nb[0] = min(64, nrows);
  nb[1] = max(0, nrows - 64);
  {
    constexpr int PPB = TPC / 2;          // threads per (block, channel)
    constexpr int RPP = 64 / PPB;
    const int c = tid % D, part = tid / D;  // part in [0, TPC): block part / PPB
    const int blk = part / PPB, sub = part % PPB;
    double s, u;
    channel_pass(c, 64 * blk + sub * RPP, 64 * blk + min(sub * RPP + RPP, nb[blk]), s, u);
    part_s[tid] = s;
    part_u[tid] = u;
    __syncthreads();
    // thread t < 2D finalizes (block t / D, channel t % D)
    double sq = 0.0;
    if (tid < 2 * D) {
      const int fb = tid / D, fc = tid % D;
      double S = 0.0, U = 0.0;
#pragma unroll
      for (int pp = 0; pp < PPB; ++pp) {
        S = S + part_s[(fb * PPB + pp) * D + fc];
        U = U + part_u[(fb * PPB + pp) * D + fc];
      }
      const int j = 2 * i + fb;
      if (nb[fb] > 0) {
        const double mean = S / (double)nb[fb];
        kmean[mean_index(bh, pad16(d.nK), j, fc, D)] = mean;
        mean_s[fb][fc] = (float)mean;
        if constexpr (QUANT) kbar[((int64_t)bh * d.nK + j) * D + fc] = (float)mean;
      }
      sq = U * U;
    }
    // 2D threads = (2D/64) waves; the first half of them hold block 0
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) sq = sq + shfl_xor_f64(sq, m);
    if (lane == 0) sq_s[wv] = sq;
    __syncthreads();
    if (tid < 2) {
      constexpr int WPB = D / 64;  // waves per block in the finalize step
      double t = 0.0;
      for (int w2 = 0; w2 < WPB; ++w2) t = t + sq_s[tid * WPB + w2];
      if (nb[tid] > 0) ksim[(int64_t)bh * d.nK + 2 * i + tid] = t / (double)(nb[tid] * nb[tid]);
    }
  }

  if constexpr (QUANT) {
    // max |k - kbar| per block over this thread's chunks, then over the workgroup
    float am[2] = {0.0f, 0.0f};
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      const int e = tid + 256 * kk, row = e / CH, ch = e % CH;
      if (row < nrows) {
        const int blk = row >> 6;
        const unsigned int wd[4] = {kr[kk].x, kr[kk].y, kr[kk].z, kr[kk].w};
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const float lo = u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16) - mean_s[blk][8 * ch + 2 * c];
          const float hi = u16_to_f32((unsigned short)(wd[c] >> 16), F16) - mean_s[blk][8 * ch + 2 * c + 1];
          am[blk] = fmaxf(am[blk], fmaxf(fabsf(lo), fabsf(hi)));
        }
      }
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      am[0] = fmaxf(am[0], __shfl_xor(am[0], m, 64));
      am[1] = fmaxf(am[1], __shfl_xor(am[1], m, 64));
    }
    if (lane == 0) {
      amax_s[wv][0] = am[0];
      amax_s[wv][1] = am[1];
    }
    __syncthreads();
    float a[2], inv[2];
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      a[blk] = fmaxf(fmaxf(amax_s[0][blk], amax_s[1][blk]), fmaxf(amax_s[2][blk], amax_s[3][blk]));
      inv[blk] = a[blk] > 0.0f ? 127.0f / a[blk] : 0.0f;
    }
    if (tid < 2 && nb[tid] > 0) kscale[(int64_t)bh * d.nK + 2 * i + tid] = a[tid] > 0.0f ? a[tid] / 127.0f : 0.0f;
    // codes of every allocated row of the existing blocks (rows past N hold zeros)
    int8_t* cb = codes + (int64_t)bh * codes_head_stride;
#pragma unroll
    for (int kk = 0; kk < NCH; ++kk) {
      const int e = tid + 256 * kk, row = e / CH, ch = e % CH;
      const int blk = row >> 6;
      if (nb[blk] > 0 && r0 + row < codes_rows) {
        unsigned int packed[2] = {0u, 0u};
        if (row < nrows && a[blk] > 0.0f) {
          const unsigned int wd[4] = {kr[kk].x, kr[kk].y, kr[kk].z, kr[kk].w};
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const float lo = u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16) - mean_s[blk][8 * ch + 2 * c];
            const float hi = u16_to_f32((unsigned short)(wd[c] >> 16), F16) - mean_s[blk][8 * ch + 2 * c + 1];
            const unsigned int pair = (unsigned int)(unsigned char)quant_code(lo, inv[blk]) |
                                      ((unsigned int)(unsigned char)quant_code(hi, inv[blk]) << 8);
            packed[c >> 1] |= pair << (16 * (c & 1));
          }
        }
        *(uint2*)(cb + (int64_t)(r0 + row) * D + 8 * ch) = make_uint2(packed[0], packed[1]);
      }
    }
  }
}

// fp8 P.V, per (b, h): the channel maxima over all Q blocks, then the E4M3
// scale s_d = fp32(max / 448) and its inverse fp32(448 / max) (0 for an all-zero
// channel).  1024 threads: thread t reduces channel t % D over the Q blocks
// i = t / D (mod 1024 / D), eight independent loads in flight, then the
// 1024 / D partial maxima of each channel meet in LDS.
__global__ __launch_bounds__(1024) void vscale_kernel(const float* vmaxp, Dims d, float* vscale,
                                                      float* vinv) {
  __shared__ float part[1024];
  const int bh = blockIdx.x, t = threadIdx.x;
  const int c = t % d.D, r0 = t / d.D, rs = 1024 / d.D;
  const float* src = vmaxp + (int64_t)bh * d.nQ * d.D + c;
  float m[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  int i = r0;
  for (; i + 7 * rs < d.nQ; i += 8 * rs) {
#pragma unroll
    for (int u = 0; u < 8; ++u) m[u] = fmaxf(m[u], src[(int64_t)(i + u * rs) * d.D]);
  }
  for (; i < d.nQ; i += rs) m[0] = fmaxf(m[0], src[(int64_t)i * d.D]);
  part[t] = fmaxf(fmaxf(fmaxf(m[0], m[1]), fmaxf(m[2], m[3])), fmaxf(fmaxf(m[4], m[5]), fmaxf(m[6], m[7])));
  __syncthreads();
  if (t < d.D) {
    float mx = 0.0f;
    for (int r = 0; r < rs; ++r) mx = fmaxf(mx, part[r * d.D + t]);
    vscale[(int64_t)bh * d.D + t] = mx / 448.0f;
    vinv[(int64_t)bh * d.D + t] = mx > 0.0f ? 448.0f / mx : 0.0f;
  }
}

// fp8 P.V: V as E4M3 codes e4m3(fp32(v * inv_d)) (round to nearest even) in
// transposed 64-token tiles, vt[((bh * nK + j) * D + c) * 64 + r] = channel c of
// token 64j + r, tokens past N zero: the attention kernel stages one tile as one
// contiguous D * 64-byte read.  One workgroup per (b, h, 64-token block); the
// block's codes are transposed through LDS.
template <int DT, int D>
__global__ __launch_bounds__(256) void vt8_kernel(View v, Dims d, const float* vinv, unsigned char* vt) {
  constexpr bool F16 = DT == kF16;
  constexpr int TP = 64 + 4;   // LDS bytes per channel row (4-byte aligned, staggered banks)
  __shared__ __attribute__((aligned(16))) unsigned char t[D * TP];
  const int tid = threadIdx.x;
  const int bh = blockIdx.x / d.nK, j = blockIdx.x - bh * d.nK;
  const int b = bh / d.H, h = bh - b * d.H;
  const unsigned short* vb = (const unsigned short*)v.p + (int64_t)b * v.sB + (int64_t)h * v.sH;
  const float* iv = vinv + (int64_t)bh * D;
  // 64 rows x D channels: each thread converts 8 channels of one row per pass
  constexpr int CH = D / 8;
  for (int e = tid; e < 64 * CH; e += 256) {
    const int r = e / CH, ch = e % CH;
    const int n = 64 * j + r;
    uint4 w = make_uint4(0, 0, 0, 0);
    if (n < d.N) w = *(const uint4*)(vb + (int64_t)n * v.sN + 8 * ch);
    const unsigned int wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int c0 = 8 * ch + 2 * c;
      const float x0 = u16_to_f32((unsigned short)(wd[c] & 0xffffu), F16) * iv[c0];
      const float x1 = u16_to_f32((unsigned short)(wd[c] >> 16), F16) * iv[c0 + 1];
      const unsigned int pk = (unsigned int)__builtin_amdgcn_cvt_pk_fp8_f32(x0, x1, 0, false);
      t[c0 * TP + r] = (unsigned char)(pk & 0xffu);
      t[(c0 + 1) * TP + r] = (unsigned char)((pk >> 8) & 0xffu);
    }
  }
  __syncthreads();
  // the tile as D rows of 64 bytes, 16 bytes per thread
  unsigned char* dst = vt + ((int64_t)bh * d.nK + j) * (64 * D);
  for (int e = tid; e < D * 4; e += 256) {
    const int c = e >> 2, g = e & 3;
    const unsigned int* src = (const unsigned int*)(t + c * TP + 16 * g);
    *(uint4*)(dst + 16 * e) = make_uint4(src[0], src[1], src[2], src[3]);
  }
}

}  // namespace

hipError_t launch_vt8(const View& v, int dtype, const Dims& d, const float* vmaxp, float* vscale,
                      float* vinv, unsigned char* vt, hipStream_t s) {
  vscale_kernel<<<dim3((unsigned)(d.B * d.H)), 1024, 0, s>>>(vmaxp, d, vscale, vinv);
  const dim3 grid((unsigned)((int64_t)d.B * d.H * d.nK));
  if (dtype == kF16) {
    if (d.D == 64) vt8_kernel<kF16, 64><<<grid, 256, 0, s>>>(v, d, vinv, vt);
    else vt8_kernel<kF16, 128><<<grid, 256, 0, s>>>(v, d, vinv, vt);
  } else {
    if (d.D == 64) vt8_kernel<kBF16, 64><<<grid, 256, 0, s>>>(v, d, vinv, vt);
    else vt8_kernel<kBF16, 128><<<grid, 256, 0, s>>>(v, d, vinv, vt);
  }
  return hipGetLastError();
}

hipError_t launch_prep(const View& q, const View& k, const View& v, int dtype, const Dims& d,
                       double* qmean, double* qsim, double* kmean, double* ksim, int8_t* codes,
                       int64_t codes_head_stride, int64_t codes_rows, float* kscale, float* kbar,
                       uint16_t* v16, float* vmaxp, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)d.B * d.H * d.nQ));
  const bool quant = codes != nullptr;
  const int vmode = v16 != nullptr ? 1 : (vmaxp != nullptr ? 2 : 0);
#define SPARGE_PREP(DTV, DV, QV, VV)                                                             \
  prep_kernel<DTV, DV, QV, VV><<<grid, 256, 0, s>>>(q, k, v, d, qmean, qsim, kmean, ksim, codes, \
                                                    codes_head_stride, codes_rows, kscale, kbar, v16, \
                                                    vmaxp)
#define SPARGE_PREP_Q(DTV, DV, QV)                                 \
  do {                                                             \
    if (vmode == 1) SPARGE_PREP(DTV, DV, QV, 1);                   \
    else if (vmode == 2) SPARGE_PREP(DTV, DV, QV, 2);              \
    else SPARGE_PREP(DTV, DV, QV, 0);                              \
  } while (0)
#define SPARGE_PREP_D(DTV, DV)                                     \
  do {                                                             \
    if (quant) SPARGE_PREP_Q(DTV, DV, true);                       \
    else SPARGE_PREP_Q(DTV, DV, false);                            \
  } while (0)
  if (dtype == kF16) {
    if (d.D == 64) SPARGE_PREP_D(kF16, 64);
    else SPARGE_PREP_D(kF16, 128);
  } else {
    if (d.D == 64) SPARGE_PREP_D(kBF16, 64);
    else SPARGE_PREP_D(kBF16, 128);
  }
#undef SPARGE_PREP_D
#undef SPARGE_PREP_Q
#undef SPARGE_PREP
  return hipGetLastError();
}

}  // namespace sparge
