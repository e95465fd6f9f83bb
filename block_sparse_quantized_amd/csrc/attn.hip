// Stage 2 of SpargeAttn on gfx950: block-sparse flash attention over a per-row
// list of kept 64-key blocks, with the online softmax-aware filter and the
// optional int8 Q K^T path.
//
// [chapterpal] method paragraph; [abstract]: stage 2 skips the matrix products of
// masked-out blocks and an online filter drops updates that are negligible for a
// whole wavefront's rows.  [gittools] custom block-sparse mask section and
// [topgit] "Key features": 128 x 64 blocks, arbitrary per-head masks.
//
// Work decomposition (MI355X-first, not a translation of any CUDA kernel):
//   * one workgroup of 4 wavefronts per (b, h, 128-row Q block); wavefront w owns
//     query rows 32w..32w+31, which is also the filter's row group;
//   * S^T = K Q^T on v_mfma_f32_32x32x16_{bf16,f16} (or v_mfma_i32_32x32x32_i8):
//     with keys as the MFMA rows, each lane ends up owning ONE query column, so
//     the row max / row sum need one cross-half exchange, and P is already in
//     the B-operand layout of O^T = V^T P^T (no LDS round trip for P);
//   * K tiles are staged row-major and V tiles transposed (dcol-major, keys in
//     the lane order the P fragments use) in LDS, double buffered, with the next
//     kept block's global loads in flight during the current block's math;
//   * grid order: XCD-aware (each of the 8 XCDs gets a contiguous range of
//     tiles, head-major so co-resident workgroups share K/V in that XCD's L2),
//     longest causal rows first.
#include "sparge_internal.hpp"

namespace sparge {
namespace {

typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
typedef unsigned short u16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_inff();

template <bool F16>
__device__ __forceinline__ f32x16 mma16(u16x8 a, u16x8 b, f32x16 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float u16_to_f32(unsigned short u, bool f16) {
  return f16 ? (float)__builtin_bit_cast(_Float16, u) : __uint_as_float((unsigned int)u << 16);
}

template <bool F16>
__device__ __forceinline__ unsigned short f32_to_u16(float x) {
  if constexpr (F16) return __builtin_bit_cast(unsigned short, (_Float16)x);
  else return __builtin_bit_cast(unsigned short, (__bf16)x);
}

__device__ __forceinline__ int xcd_remap(int bid, int G) {
  // Workgroups are dispatched round-robin over the 8 XCDs; give XCD x the
  // contiguous tile range [x*q + min(x, r), ...) so neighbouring tiles share an L2.
  const int q = G >> 3, r = G & 7;
  const int x = bid & 7, loc = bid >> 3;
  return x < r ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
}

// Position, inside a 16-key group of the transposed V tile, of the 4-key run that
// starts at key offset 4*g (g = 0..3): lane half h of the P.V MFMA holds keys
// {4h..4h+3, 8+4h..8+4h+3} of the group as its 8 consecutive k slots.
__device__ __forceinline__ int vpos4(int g) { return (g == 1) ? 8 : (g == 2 ? 4 : 4 * g); }

template <int D, bool IN_F16, bool PV_F16, bool QK8>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnParams p, Dims d) {
  constexpr int KS16 = D / 16;                 // k-steps of the 16-bit Q K^T
  constexpr int KS8 = D / 32;                  // k-steps of the int8 Q K^T
  constexpr int DT = D / 32;                   // 32-column output tiles
  constexpr int KROWB = QK8 ? (D + 16) : 2 * (D + 8);  // bytes per staged K row
  constexpr int VSTR = 64 + 8;                 // u16 elements per transposed V row
  constexpr int KCPR = QK8 ? D / 16 : D / 8;   // 16-byte chunks per K row
  constexpr int KCH = 64 * KCPR / 256;         // K chunks per thread
  constexpr int VTASK = 16 * (D / 8);          // (4-key run, 8-column chunk) tasks
  constexpr int KBSTR = D + 8;                 // u16 per row of the kbar hi/lo tiles
  constexpr int AUXB = QK8 ? ((2 * 32 * KBSTR * 2) > (4 * 32 * 33 * 4) ? (2 * 32 * KBSTR * 2)
                                                                        : (4 * 32 * 33 * 4))
                           : 16;

  __shared__ __attribute__((aligned(16))) unsigned char Ks[2][64 * KROWB];
  __shared__ __attribute__((aligned(16))) unsigned short Vs[2][D * VSTR];
  __shared__ __attribute__((aligned(16))) unsigned char Aux[AUXB];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, hf = lane >> 5, ql = lane & 31;
  const int tile = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int bh = tile / d.nQ;
  const int ii = tile - bh * d.nQ;
  const int i = p.causal ? (d.nQ - 1 - ii) : ii;
  const int b = bh / d.H, h = bh - b * d.H;
  const int N = d.N;
  const int wrow0 = i * 128 + w * 32;
  const int t = wrow0 + ql;
  const bool row_ok = t < N;

  const unsigned short* Qp = (const unsigned short*)p.q.p + b * p.q.sB + h * p.q.sH;
  const unsigned short* Kp = (const unsigned short*)p.k.p + b * p.k.sB + h * p.k.sH;
  const unsigned short* Vp = (const unsigned short*)p.v.p + b * p.v.sB + h * p.v.sH;
  const int8_t* K8p = QK8 ? p.k8 + (int64_t)bh * d.nK * 64 * D : nullptr;

  // Q fragments in the B-operand layout: lane (hf, ql) holds Q[t][16s + 8hf .. +7].
  u16x8 qf[KS16];
#pragma unroll
  for (int s = 0; s < KS16; ++s) {
    if (row_ok) qf[s] = *(const u16x8*)(Qp + (int64_t)t * p.q.sN + 16 * s + 8 * hf);
    else qf[s] = (u16x8)(0);
  }

  // int8 Q codes: lane holds Q[t][32s + 16hf .. +15], one step per wavefront.
  i32x4 q8[QK8 ? KS8 : 1];
  float dq = 0.0f;
  if constexpr (QK8) {
    float vals[KS8][16];
    float amax = 0.0f;
#pragma unroll
    for (int s = 0; s < KS8; ++s) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        u16x8 raw = (u16x8)(0);
        if (row_ok) raw = *(const u16x8*)(Qp + (int64_t)t * p.q.sN + 32 * s + 16 * hf + 8 * c);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = u16_to_f32(raw[e], IN_F16);
          vals[s][8 * c + e] = x;
          amax = fmaxf(amax, fabsf(x));
        }
      }
    }
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    const float inv = amax > 0.0f ? 127.0f / amax : 0.0f;
    dq = amax > 0.0f ? amax / 127.0f : 0.0f;
#pragma unroll
    for (int s = 0; s < KS8; ++s) {
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        unsigned int packed = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float c = __builtin_rintf(vals[s][4 * wd + e] * inv);
          c = fminf(fmaxf(c, -127.0f), 127.0f);
          packed |= ((unsigned int)((int)c) & 0xffu) << (8 * e);
        }
        q8[s][wd] = (int)packed;
      }
    }
  }

  const int cnt = p.counts[bh * d.nQ + i];
  const unsigned short* lst = p.lists + (int64_t)(bh * d.nQ + i) * d.nK;

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x16)(0.0f);
  float m_run = kNegInf, l_part = 0.0f;
  unsigned int n_skip = 0;

  u16x8 kreg[KCH];
  u16x8 vreg[4];

  auto load_tile = [&](int j) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      const int row = c / KCPR, col = c % KCPR;
      const int key = 64 * j + row;
      if constexpr (QK8) {
        kreg[u] = *(const u16x8*)(K8p + (int64_t)key * D + 16 * col);
      } else {
        if (key < N) kreg[u] = *(const u16x8*)(Kp + (int64_t)key * p.k.sN + 8 * col);
        else kreg[u] = (u16x8)(0);
      }
    }
    if (VTASK == 256 || tid < VTASK) {
      const int g4 = tid / (D / 8), dc = tid % (D / 8);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int key = 64 * j + 4 * g4 + r;
        if (key < N) vreg[r] = *(const u16x8*)(Vp + (int64_t)key * p.v.sN + 8 * dc);
        else vreg[r] = (u16x8)(0);
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      const int row = c / KCPR, col = c % KCPR;
      *(u16x8*)(&Ks[buf][row * KROWB + 16 * col]) = kreg[u];
    }
    if (VTASK == 256 || tid < VTASK) {
      const int g4 = tid / (D / 8), dc = tid % (D / 8);
      const int pos = 16 * (g4 >> 2) + vpos4(g4 & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        u16x4 v4;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const unsigned short raw = vreg[r][e];
          if constexpr (IN_F16 == PV_F16) v4[r] = raw;
          else v4[r] = f32_to_u16<PV_F16>(u16_to_f32(raw, IN_F16));
        }
        *(u16x4*)(&Vs[buf][(8 * dc + e) * VSTR + pos]) = v4;
      }
    }
  };

  if (cnt > 0) load_tile(lst[0]);
  for (int it = 0; it < cnt; ++it) {
    const int j = lst[it];
    const int buf = it & 1;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < cnt) load_tile(lst[it + 1]);

    float bias = 0.0f;   // int8 path: c * (q . kbar_j) for this lane's query
    float sc = 0.0f;     // int8 path: c * dq * dk_j
    if constexpr (QK8) {
      unsigned short* kbh = (unsigned short*)Aux;            // [32][KBSTR] hi
      unsigned short* kbl = kbh + 32 * KBSTR;                // [32][KBSTR] lo
      float* cw = (float*)Aux + w * 32 * 33;                 // per wave [32][33]
      if ((it & 31) == 0) {
        // kbar of the next 32 kept blocks as bf16 hi + lo, for q . kbar by MFMA
        for (int e = tid; e < 32 * (D / 4); e += 256) {
          const int pr = e / (D / 4), c4 = (e % (D / 4)) * 4;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (it + pr < cnt)
            v = *(const float4*)(p.kbar + ((int64_t)bh * d.nK + lst[it + pr]) * D + c4);
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            // kbar = hi + lo in the input's 16-bit type (exact to ~2^-17 relative)
            const unsigned short hi = f32_to_u16<IN_F16>(vv[q4]);
            const unsigned short lo = f32_to_u16<IN_F16>(vv[q4] - u16_to_f32(hi, IN_F16));
            kbh[pr * KBSTR + c4 + q4] = hi;
            kbl[pr * KBSTR + c4 + q4] = lo;
          }
        }
        __syncthreads();
        f32x16 cacc = (f32x16)(0.0f);
#pragma unroll
        for (int s = 0; s < KS16; ++s) {
          const u16x8 ah = *(const u16x8*)(kbh + ql * KBSTR + 16 * s + 8 * hf);
          const u16x8 al = *(const u16x8*)(kbl + ql * KBSTR + 16 * s + 8 * hf);
          cacc = mma16<IN_F16>(ah, qf[s], cacc);
          cacc = mma16<IN_F16>(al, qf[s], cacc);
        }
        __syncthreads();  // every wave is done reading kbh/kbl, which cw overlays
        // lane (hf, ql) holds C[block (r/4)*8 + 4hf + r%4][query ql]
#pragma unroll
        for (int r = 0; r < 16; ++r) cw[((r >> 2) * 8 + 4 * hf + (r & 3)) * 33 + ql] = cacc[r];
        __syncthreads();
      }
      bias = p.c * cw[(it & 31) * 33 + ql];
      sc = p.c * dq * p.kscale[(int64_t)bh * d.nK + j];
    }

    // logits (log2 units) of this lane's query against the block's 64 keys:
    // lg[kt][r] is key 32kt + (r/4)*8 + 4hf + r%4
    float lg[2][16];
    if constexpr (!QK8) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        f32x16 sacc = (f32x16)(0.0f);
#pragma unroll
        for (int s = 0; s < KS16; ++s) {
          const u16x8 kf = *(const u16x8*)(&Ks[buf][(32 * kt + ql) * KROWB + 32 * s + 16 * hf]);
          sacc = mma16<IN_F16>(kf, qf[s], sacc);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) lg[kt][r] = sacc[r] * p.c;
      }
    } else {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        i32x16 iacc = (i32x16)(0);
#pragma unroll
        for (int s = 0; s < KS8; ++s) {
          const i32x4 kf = *(const i32x4*)(&Ks[buf][(32 * kt + ql) * KROWB + 32 * s + 16 * hf]);
          iacc = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, q8[s], iacc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) lg[kt][r] = __builtin_fmaf((float)iacc[r], sc, bias);
      }
    }

    const bool need_mask = (64 * j + 64 > N) || (p.causal && 64 * j + 63 > wrow0) || (wrow0 + 31 >= N);
    if (need_mask) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = 64 * j + 32 * kt + (r >> 2) * 8 + 4 * hf + (r & 3);
          if (key >= N || (p.causal && key > t) || !row_ok) lg[kt][r] = kNegInf;
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, lg[kt][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    if (p.filter_on) {
      const bool keep = (mx != kNegInf) && (mx - m_new >= p.lam2);
      if (__ballot(keep) == 0ull) {
        ++n_skip;
        continue;
      }
    }
    const float m_use = (m_new == kNegInf) ? 0.0f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;

    float rs = 0.0f;
    u16x8 pf[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float pv = __builtin_amdgcn_exp2f(lg[kt][r] - m_use);
        rs += pv;
        pf[2 * kt + (r >> 3)][r & 7] = f32_to_u16<PV_F16>(pv);
      }
    l_part = l_part * alpha + rs;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int sg = 0; sg < 4; ++sg) {
        const u16x8 vf = *(const u16x8*)(&Vs[buf][(32 * dt + ql) * VSTR + 16 * sg + 8 * hf]);
        oacc[dt] = mma16<PV_F16>(vf, pf[sg], oacc[dt]);
      }
  }

  // epilogue: O = acc / l, this lane's query row, columns 32dt + 8g + 4hf + 0..3
  const float lt = l_part + __shfl_xor(l_part, 32, 64);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    char* ob = (char*)p.o;
    const int esz = p.out_type == kF32 ? 4 : 2;
    const int64_t rowoff = ((int64_t)b * p.osB + (int64_t)h * p.osH + (int64_t)t * p.osN) * esz;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * dt + 8 * g + 4 * hf;
        const float o0 = oacc[dt][4 * g] * inv, o1 = oacc[dt][4 * g + 1] * inv;
        const float o2 = oacc[dt][4 * g + 2] * inv, o3 = oacc[dt][4 * g + 3] * inv;
        if (p.out_type == kF32) {
          *(float4*)(ob + rowoff + (int64_t)col * 4) = make_float4(o0, o1, o2, o3);
        } else if (p.out_type == kF16) {
          u16x4 v = {f32_to_u16<true>(o0), f32_to_u16<true>(o1), f32_to_u16<true>(o2), f32_to_u16<true>(o3)};
          *(u16x4*)(ob + rowoff + (int64_t)col * 2) = v;
        } else {
          u16x4 v = {f32_to_u16<false>(o0), f32_to_u16<false>(o1), f32_to_u16<false>(o2), f32_to_u16<false>(o3)};
          *(u16x4*)(ob + rowoff + (int64_t)col * 2) = v;
        }
      }
  }
  if (p.counters && lane == 0 && wrow0 < N) {
    atomicAdd(&p.counters[2], (unsigned long long)cnt);
    atomicAdd(&p.counters[3], (unsigned long long)n_skip);
  }
}

template <int D, bool IN_F16>
hipError_t launch_d(const AttnParams& p, const Dims& d, hipStream_t s) {
  const dim3 grid((unsigned)((int64_t)d.B * d.H * d.nQ));
  if (p.qk_int8) {
    if (p.pv_fp16) sparse_attn_kernel<D, IN_F16, true, true><<<grid, 256, 0, s>>>(p, d);
    else sparse_attn_kernel<D, IN_F16, IN_F16, true><<<grid, 256, 0, s>>>(p, d);
  } else {
    if (p.pv_fp16) sparse_attn_kernel<D, IN_F16, true, false><<<grid, 256, 0, s>>>(p, d);
    else sparse_attn_kernel<D, IN_F16, IN_F16, false><<<grid, 256, 0, s>>>(p, d);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnParams& p, const Dims& d, hipStream_t s) {
  if (d.D == 64) return p.in_f16 ? launch_d<64, true>(p, d, s) : launch_d<64, false>(p, d, s);
  return p.in_f16 ? launch_d<128, true>(p, d, s) : launch_d<128, false>(p, d, s);
}

}  // namespace sparge
