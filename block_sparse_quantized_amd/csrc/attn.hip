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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

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

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded (to nearest even) into one packed 16-bit pair.
template <bool F16>
__device__ __forceinline__ unsigned int pack2(float a, float b) {
  if constexpr (F16) return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, f16x2));
  else return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// acc + (lo + hi) of a packed 16-bit pair, accumulated in fp32.
template <bool F16>
__device__ __forceinline__ float add_pair(unsigned int pr, float acc) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), (f16x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr),
                                           (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Key offset, inside a 64-key block, of register r of key tile kt for lane half 0
// (half 1 adds 4): the 32x32 MFMA result layout.
__device__ __forceinline__ constexpr int key_off(int kt, int r) { return 32 * kt + (r >> 2) * 8 + (r & 3); }

// Reference-max slack (log2 units): exponentials are taken against a reference
// max that moves only when a row's running max exceeds it by more than this, so
// O and l are rescaled rarely; P then stays below 2^8.
constexpr float kTau = 8.0f;

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
  // keys s < lim are visible to this lane's query row
  const int lim = row_ok ? (p.causal ? min(N, t + 1) : N) : 0;

  const unsigned short* Qp = (const unsigned short*)p.q.p + b * p.q.sB + h * p.q.sH;
  const char* Kb = QK8 ? (const char*)(p.k8 + (int64_t)bh * d.nK * 64 * D)
                       : (const char*)((const unsigned short*)p.k.p + b * p.k.sB + h * p.k.sH);
  const char* Vb = (const char*)((const unsigned short*)p.v.p + b * p.v.sB + h * p.v.sH);

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
  // The row's kept-block list, read through the constant address space so that
  // the (wave-uniform) reads are scalar loads: they never wait behind the vector
  // tile prefetches.  Rows are 16-byte aligned; two uint16 entries per dword.
  typedef const __attribute__((address_space(4))) unsigned int* const_u32_ptr;
  const const_u32_ptr lst32 = (const_u32_ptr)(p.lists + (int64_t)(bh * d.nQ + i) * d.lstride);
  auto list_at = [&](int k) -> int {
    const unsigned int wv = lst32[k >> 1];
    return (int)((k & 1) ? (wv >> 16) : (wv & 0xffffu));
  };

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x16)(0.0f);
  float m_true = kNegInf;   // running row max of the visited blocks (filter)
  float m_ref = kNegInf;    // reference max of the exponentials
  float m_use = 0.0f;       // m_ref, or 0 while it is -inf
  float l_acc = 0.0f;       // this lane's partial row sum (its half of the keys)
  unsigned int n_skip = 0;

  // per-thread staging addresses (bytes from the head base), fixed over the loop
  int koff[KCH], krow[KCH];
#pragma unroll
  for (int u = 0; u < KCH; ++u) {
    const int c = tid + 256 * u;
    krow[u] = c / KCPR;
    koff[u] = QK8 ? krow[u] * D + 16 * (c % KCPR) : (krow[u] * (int)p.k.sN + 8 * (c % KCPR)) * 2;
  }
  // V staging task of this thread: 4-key run g4 (16 per block) x 8-column chunk dc.
  // Sixteen consecutive lanes take the sixteen runs of one chunk, so each
  // transposed LDS store instruction covers whole 128-byte rows (no bank conflicts).
  const bool vtask = (VTASK == 256) || (tid < VTASK);
  const int g4 = tid & 15, dc = tid >> 4;
  const int voff = (4 * g4 * (int)p.v.sN + 8 * dc) * 2;
  const int vrow = (int)p.v.sN * 2;
  const int64_t kblk = QK8 ? (int64_t)64 * D : (int64_t)64 * p.k.sN * 2;
  const int64_t vblk = (int64_t)64 * p.v.sN * 2;

  u16x8 kreg[KCH];
  u16x8 vreg[4];

  auto load_tile = [&](int j) {
    const char* kb = Kb + j * kblk;
    const char* vb = Vb + j * vblk;
    if (QK8 || 64 * j + 64 <= N) {
#pragma unroll
      for (int u = 0; u < KCH; ++u) kreg[u] = *(const u16x8*)(kb + koff[u]);
      if (vtask) {
#pragma unroll
        for (int r = 0; r < 4; ++r) vreg[r] = *(const u16x8*)(vb + voff + r * vrow);
      }
    } else {  // ragged last block: rows past N read as zeros
#pragma unroll
      for (int u = 0; u < KCH; ++u)
        kreg[u] = (64 * j + krow[u] < N) ? *(const u16x8*)(kb + koff[u]) : (u16x8)(0);
      if (vtask) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[r] = (64 * j + 4 * g4 + r < N) ? *(const u16x8*)(vb + voff + r * vrow) : (u16x8)(0);
      }
    }
  };

  auto store_tile = [&](int buf) {
#pragma unroll
    for (int u = 0; u < KCH; ++u) {
      const int c = tid + 256 * u;
      *(u16x8*)(&Ks[buf][(c / KCPR) * KROWB + 16 * (c % KCPR)]) = kreg[u];
    }
    if (vtask) {
      const int pos = 16 * (g4 >> 2) + vpos4(g4 & 3);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const u16x4 v4 = {vreg[0][e], vreg[1][e], vreg[2][e], vreg[3][e]};
        *(u16x4*)(&Vs[buf][(8 * dc + e) * VSTR + pos]) = v4;
      }
    }
  };

  // Block indices travel one and two iterations ahead of their use, so that no
  // wait on a list read ever drains the tile prefetch queue.
  int j_cur = cnt > 0 ? list_at(0) : 0;
  int j_nxt = cnt > 1 ? list_at(1) : 0;
  if (cnt > 0) load_tile(j_cur);
  for (int it = 0; it < cnt; ++it) {
    const int j = j_cur;
    const int buf = it & 1;
    const int j_after = (it + 2 < cnt) ? list_at(it + 2) : 0;
    store_tile(buf);
    __syncthreads();
    if (it + 1 < cnt) load_tile(j_nxt);
    j_cur = j_nxt;
    j_nxt = j_after;

    float bias = 0.0f;   // int8 path: c * (q . kbar_j) for this lane's query
    float sc = 0.0f;     // int8 path: c * dq * dk_j
    if constexpr (QK8) {
      unsigned short* kbh = (unsigned short*)Aux;            // [32][KBSTR] hi
      unsigned short* kbl = kbh + 32 * KBSTR;                // [32][KBSTR] lo
      float* cw = (float*)Aux + w * 32 * 33;                 // per wave [32][33]
      if ((it & 31) == 0) {
        // kbar of the next 32 kept blocks as hi + lo in the input's 16-bit type,
        // so that q . kbar runs on the MFMA at near-fp32 accuracy
        for (int e = tid; e < 32 * (D / 4); e += 256) {
          const int pr = e / (D / 4), c4 = (e % (D / 4)) * 4;
          float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
          if (it + pr < cnt)
            v = *(const float4*)(p.kbar + ((int64_t)bh * d.nK + list_at(it + pr)) * D + c4);
          const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
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
      // dq * dk can be 0 (an all-zero group or block); keep the slope positive so
      // that masked (-inf) scores stay -inf
      sc = fmaxf(p.c * dq * p.kscale[(int64_t)bh * d.nK + j], 1e-30f);
    }

    // raw scores of this lane's query against the block's 64 keys:
    // sacc[kt][r] is key 64j + 4hf + key_off(kt, r)
    f32x16 sacc[2];
    if constexpr (!QK8) {
      sacc[0] = (f32x16)(0.0f);
      sacc[1] = (f32x16)(0.0f);
#pragma unroll
      for (int s = 0; s < KS16; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const u16x8 kf = *(const u16x8*)(&Ks[buf][(32 * kt + ql) * KROWB + 32 * s + 16 * hf]);
          sacc[kt] = mma16<IN_F16>(kf, qf[s], sacc[kt]);
        }
    } else {
      i32x16 iacc[2] = {(i32x16)(0), (i32x16)(0)};
#pragma unroll
      for (int s = 0; s < KS8; ++s)
#pragma unroll
        for (int kt = 0; kt < 2; ++kt) {
          const i32x4 kf = *(const i32x4*)(&Ks[buf][(32 * kt + ql) * KROWB + 32 * s + 16 * hf]);
          iacc[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(kf, q8[s], iacc[kt], 0, 0, 0);
        }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = (float)iacc[kt][r];
    }

    if ((64 * j + 64 > N) || (p.causal && 64 * j + 63 > wrow0) || (wrow0 + 31 >= N)) {
      const int rel = lim - 64 * j - 4 * hf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[kt][r] = key_off(kt, r) < rel ? sacc[kt][r] : kNegInf;
    }

    float mraw = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mraw = max3f(mraw, sacc[kt][r], sacc[kt][r + 1]);
    mraw = fmaxf(mraw, __shfl_xor(mraw, 32, 64));
    float mx;  // block max of this row in log2 units, -inf when no key is visible
    if constexpr (QK8) mx = (mraw == kNegInf) ? kNegInf : __builtin_fmaf(mraw, sc, bias);
    else mx = mraw * p.c;

    if (p.filter_on) {
      const float m_new = fmaxf(m_true, mx);
      const bool keep = (mx != kNegInf) && (mx - m_new >= p.lam2);
      if (__ballot(keep) == 0ull) {
        ++n_skip;
        continue;
      }
      m_true = m_new;
    }
    if (__ballot(mx > m_ref + kTau) != 0ull) {
      const float m_ref_new = fmaxf(m_ref, mx);
      const float mu_new = (m_ref_new == kNegInf) ? 0.0f : m_ref_new;
      const float alpha = __builtin_amdgcn_exp2f(m_ref - mu_new);
      l_acc *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
      m_ref = m_ref_new;
      m_use = mu_new;
    }

    // P = 2^(score * slope + offset - m_use), rounded to the P.V type in pairs
    const float slope = QK8 ? sc : p.c;
    const float offs = (QK8 ? bias : 0.0f) - m_use;
    u32x4 pw[4];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int sg = 0; sg < 2; ++sg)
#pragma unroll
        for (int wd = 0; wd < 4; ++wd) {
          const int r = 8 * sg + 2 * wd;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r], slope, offs));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kt][r + 1], slope, offs));
          const unsigned int pr = pack2<PV_F16>(p0, p1);
          l_acc = add_pair<PV_F16>(pr, l_acc);
          pw[2 * kt + sg][wd] = pr;
        }
#pragma unroll
    for (int sg = 0; sg < 4; ++sg)
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const u16x8 vf = *(const u16x8*)(&Vs[buf][(32 * dt + ql) * VSTR + 16 * sg + 8 * hf]);
        oacc[dt] = mma16<PV_F16>(vf, __builtin_bit_cast(u16x8, pw[sg]), oacc[dt]);
      }
  }

  // epilogue: O = acc / l, this lane's query row, columns 32dt + 8g + 4hf + 0..3
  const float lt = l_acc + __shfl_xor(l_acc, 32, 64);
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
          const uint2 v = {pack2<true>(o0, o1), pack2<true>(o2, o3)};
          *(uint2*)(ob + rowoff + (int64_t)col * 2) = v;
        } else {
          const uint2 v = {pack2<false>(o0, o1), pack2<false>(o2, o3)};
          *(uint2*)(ob + rowoff + (int64_t)col * 2) = v;
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
