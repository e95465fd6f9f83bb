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
#include <type_traits>

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
typedef int i32x8 __attribute__((ext_vector_type(8)));

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


typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Two fp32 values rounded (to nearest even) into one packed 16-bit pair.
template <bool F16>
__device__ __forceinline__ unsigned int pack2(float a, float b) {
  if constexpr (F16) return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, f16x2));
  else return __builtin_bit_cast(unsigned int, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

typedef float f32x4 __attribute__((ext_vector_type(4)));

// acc + (lo + hi) of a packed 16-bit pair, accumulated in fp32.
template <bool F16>
__device__ __forceinline__ float add_pair(unsigned int pr, float acc) {
  if constexpr (F16)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, pr), (f16x2){(_Float16)1.0f, (_Float16)1.0f}, acc, false);
  else
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pr),
                                           (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, acc, false);
}

// Row sums of a 16-bit P fragment on the MFMA.  Read as the B operand of a 16x16x32
// MFMA, the 32x32x16 fragment (lane l: query l % 32, keys 8(l / 32) .. +7) puts, for
// output column c, query c's and query c+16's keys in alternating groups of eight
// (lanes c, c+16, c+32, c+48).  With A one on the groups of query c for output rows i
// with (i / 4) even and on those of query c+16 for the others (sel), D[i][c], which
// lane c + 16(i / 4) holds, is the fragment's sum for exactly that lane's own query
// (l % 32), accumulated in fp32 from the rounded P that the P.V MFMAs multiply.
template <bool F16>
__device__ __forceinline__ f32x4 rowsum16(u16x8 sel, u16x8 pf, f32x4 c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, sel), __builtin_bit_cast(f16x8, pf),
                                                  c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, sel),
                                                   __builtin_bit_cast(bf16x8, pf), c, 0, 0, 0);
}

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Lane l ^ 32's value (v_permlane32_swap: the two lane halves trade places).
__device__ __forceinline__ float partner32(float v, int hf) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(hf ? r[0] : r[1]);
}
// max(v, value of lane l ^ 32): one of the two swapped copies is v itself.
__device__ __forceinline__ float max_xor32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return max3f(v, __uint_as_float(r[0]), __uint_as_float(r[1]));
}


// Reference-max slack (log2 units): exponentials are taken against a reference
// max that moves only when a row's running max exceeds it by more than this, so
// O and l are rescaled rarely; P then stays below 2^8.
constexpr float kTau = 8.0f;
// int8 Q.K^T: the accumulators start at 0x3e22f983, the bit pattern of the MFMA's
// inline constant 1/(2 pi).  Its mantissa field is 2292099, so for |s| below that
// (127 * 127 * D is at most 2064512) the int32 result s + 0x3e22f983 read as a float
// is exactly kScoreC0 + s * 2^-26, in the binade [1/8, 1/4): scores need no int to
// float conversion, float order is integer order, and the slope and offset of the
// exponent absorb the affine map.
constexpr int kScoreBits = 0x3e22f983;
constexpr float kScoreC0 = 0.15915493667125702f;   // the float with those bits
constexpr float kScoreUnit = 67108864.0f;           // 2^26

// The first k-step of the int8 Q.K^T: C is the inline constant itself, so no register
// block has to be filled with it.  The compiler does not see an MFMA here, so the asm
// carries the wait states it would otherwise insert: two after any VALU write of A or
// B (A comes from LDS reads with an explicit wait, B is written before the loop).
// D is read only by the next k-step's MFMA with C exactly overlapping it, which needs
// none.
__device__ __forceinline__ i32x16 mfma_i8_first(i32x4 a, i32x4 b) {
  i32x16 d;
  asm("s_nop 1\n\tv_mfma_i32_32x32x32_i8 %0, %1, %2, 0x3e22f983" : "=&v"(d) : "v"(a), "v"(b));
  return d;
}

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) unsigned char* lds_u8_ptr;

// Transposing 64-bit LDS read (ds_read_b64_tr_b16) at a per-lane LDS address plus
// an immediate offset.  Issued as inline asm so that the compiler's wait-count pass,
// which cannot tell the builtin's LDS reads apart from the direct-to-LDS loads in
// flight, does not insert a full vector-memory wait in front of it; the caller
// waits for the result itself with lds_wait.
template <int OFF>
__device__ __forceinline__ s16x4 ds_read_tr(unsigned int addr) {
  s16x4 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait until at most N LDS reads issued after the ones producing a and b are in
// flight (LDS returns in order, so this makes a and b valid); the asm operands tie
// the wait to its consumers.
template <int N>
__device__ __forceinline__ void lds_wait(s16x4& a, s16x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
// 16-byte LDS read (ds_read_b128) at a per-lane address plus an immediate offset,
// issued as inline asm for the same reason as ds_read_tr; waited with lds_wait16.
template <int OFF>
__device__ __forceinline__ u32x4 ds_read16(unsigned int addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
template <int N>
__device__ __forceinline__ void lds_wait16(u32x4& a, u32x4& b) {
  asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(a), "+v"(b) : "i"(N));
}
template <int I, int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// 16 bytes per lane from a raw buffer (resource r, this lane's byte offset) into LDS
// at dst + 16 * lane (buffer_load_dwordx4 ... lds); offsets past the resource's
// extent read as zeros.
__device__ __forceinline__ void buffer_lds16(__amdgpu_buffer_rsrc_t r, lds_void_ptr dst, unsigned int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, (int)voff, 0, 0, 0);
}

// s_waitcnt vmcnt(0) with the other counters left alone (gfx9 encoding).
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Key offset, inside a 64-key block, of register r of key tile kt: the K rows fed
// to the Q.K^T MFMA are permuted (row m of a 32-key tile holds key swap23(m)), so
// that each lane's eight P values of a P.V k-step are eight consecutive keys.
// Lane half 1 adds 8.
__device__ __forceinline__ constexpr int key_off2(int kt, int r) {
  return 32 * kt + 16 * (r >> 3) + 4 * ((r >> 2) & 1) + (r & 3);
}
__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// Granule swizzles of the LDS tiles (physical granule = logical ^ f(row)), for
// gfx950's 64-bank LDS (256 bytes per cycle: sixteen lanes of a 16-byte read,
// thirty-two lanes of an 8-byte read).  K fragment reads: sixteen lanes read one
// granule column of rows swap23(0..15); fk maps those rows to sixteen different
// bank groups for 256-, 128- and 64-byte rows.  V transposing reads: thirty-two
// lanes cover four consecutive rows x four adjacent granules; fv spreads them
// over sixteen bank groups.
template <int G>
__device__ __forceinline__ int fk(int r) {
  if constexpr (G >= 16) return r & 15;
  else if constexpr (G == 8) return (r >> 1) & 7;
  else return (r >> 2) & 3;
}
template <int G>
__device__ __forceinline__ int fv(int r) {
  if constexpr (G >= 16) return 4 * (r & 3);
  else return 4 * ((r >> 1) & 1);
}
// K swizzle of the fp8 P.V variant, whose sixteen lanes read rows {0..7, 32..39} +
// a multiple of 8 (row bits 0, 1, 2 and 5 vary): those bits go to distinct bank
// groups for 256-, 128- and 64-byte rows.
template <int G, bool PV8>
__device__ __forceinline__ int fkx(int r) {
  if constexpr (!PV8) return fk<G>(r);
  else if constexpr (G >= 16) return (r & 7) | ((r >> 2) & 8);
  else if constexpr (G == 8) return ((r >> 1) & 3) | ((r >> 3) & 4);
  else return ((r >> 2) & 1) | ((r >> 4) & 2);
}

// fp8 P.V (OCP E4M3): four fp32 values rounded to nearest even into one word, the
// first in the low byte.
__device__ __forceinline__ int pack_fp8x4(float a, float b, float c, float e) {
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, e, lo, true);
}
// C += A B on v_mfma_scale_f32_32x32x64_f8f6f4 with both operands E4M3 and unit
// block scales (exponent code 127); lane (h, m) holds A[m][32h .. 32h+31] and
// B[32h .. 32h+31][m].
__device__ __forceinline__ f32x16 mma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// E4M3 16x16x128 with unit scales: the row sums of an fp8 P fragment, as rowsum16
// does for 16-bit P (the 32x32x64 fragment puts query c's and c+16's keys in
// alternating groups of 32 for output column c).
__device__ __forceinline__ f32x4 rowsum_fp8(i32x8 sel, i32x8 pf, f32x4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(sel, pf, c, 0, 0, 0, 127, 0, 127);
}

template <int D, bool IN_F16, bool PV_F16, bool QK8, bool PV8>
__global__ __launch_bounds__(256, 2) void sparse_attn_kernel(AttnParams p, Dims d) {
  constexpr int KS16 = D / 16;                // k-steps of the 16-bit Q K^T
  constexpr int KS8 = D / 32;                 // k-steps of the int8 Q K^T
  constexpr int DT = D / 32;                  // 32-column output tiles
  constexpr int KROW = QK8 ? D : 2 * D;       // bytes per K row in LDS (no padding)
  constexpr int VROW = 2 * D;                 // bytes per V row in LDS (16-bit P.V)
  constexpr int KG = KROW / 16;               // 16-byte granules per K row
  constexpr int VG = VROW / 16;
  // fp8 P.V stages the block's transposed E4M3 tile: D channel rows of 64 bytes
  constexpr int VTILE = PV8 ? 64 * D : 64 * VROW;
  constexpr int KCHUNK = 64 * KROW / 1024;    // 1 KB DMA chunks per K tile
  constexpr int VCHUNK = VTILE / 1024;
  constexpr int kNU = 4 * DT;                 // (k-step, column tile) pairs of P.V
  constexpr int kVAhead = 4;                  // P.V pairs whose V reads run ahead
  // int8 path: the q . kbar term from LDS only (see the pass in the step): this
  // workgroup's Q residual codes per wave and k-step in the B-fragment order, two
  // code rows of kbar for 16 kept blocks, and per wave q . kbar of those blocks
  constexpr int R8B = QK8 ? 4 * KS8 * 64 * 16 : 16;
  constexpr int KCB = QK8 ? 16 * 2 * D : 16;
  constexpr int CWB = QK8 ? 4 * 16 * 32 * 4 : 16;
  // LDS tiles are written by direct-to-LDS loads (one 1 KB chunk per wavefront
  // instruction, lane-linear) and stored row-major with each row's 16-byte granules
  // XOR-swizzled by a function of the row (fk, fv), so fragment reads are free of
  // bank conflicts.
  // One variable per stage and tile: the compiler then knows that a DMA into one
  // stage never aliases reads of the other, and does not wait for it.
  __shared__ __attribute__((aligned(1024))) unsigned char Ks0[64 * KROW];
  __shared__ __attribute__((aligned(1024))) unsigned char Ks1[64 * KROW];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs0[VTILE];
  __shared__ __attribute__((aligned(1024))) unsigned char Vs1[VTILE];
  __shared__ __attribute__((aligned(16))) unsigned char R8s[R8B];
  __shared__ __attribute__((aligned(1024))) unsigned char KCs[KCB];
  __shared__ __attribute__((aligned(16))) float CWs[CWB / 4];

  const int tid = threadIdx.x;
  const int lane = tid & 63, hf = lane >> 5, ql = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_remap((int)blockIdx.x, (int)gridDim.x);
  const int bh = tile / d.nQ;
  const int ii = tile - bh * d.nQ;
  const int i = p.causal ? (d.nQ - 1 - ii) : ii;
  const int b = bh / d.H, h = bh - b * d.H;
  const int N = d.N;
  // filter threshold in log2 units, per head when the caller gave per-head values
  const float lam2 = p.head_lambda ? (float)(p.head_lambda[h] * 1.4426950408889634) : p.lam2;
  const int wrow0 = i * 128 + w * 32;
  const int t = wrow0 + ql;
  const bool row_ok = t < N;
  // keys s < lim are visible to this lane's query row
  const int lim = row_ok ? (p.causal ? min(N, t + 1) : N) : 0;

  const unsigned short* Qp = (const unsigned short*)p.q.p + b * p.q.sB + h * p.q.sH;
  const char* Kb = QK8 ? (const char*)(p.k8 + (int64_t)bh * d.nK * 64 * D)
                       : (const char*)((const unsigned short*)p.k.p + b * p.k.sB + h * p.k.sH);
  const char* Vb = PV8 ? (const char*)(p.v8t + (int64_t)bh * d.nK * 64 * D)
                       : (const char*)((const unsigned short*)p.v.p + b * p.v.sB + h * p.v.sH);
  const int64_t ksrow = QK8 ? (int64_t)D : p.k.sN * 2;   // bytes between K rows in memory
  const int64_t vsrow = p.v.sN * 2;

  // Q fragments in the B-operand layout (16-bit Q.K^T): lane (hf, ql) holds
  // Q[t][16s + 8hf .. +7].
  auto load_qf = [&](u16x8 (&f)[KS16]) {
#pragma unroll
    for (int s = 0; s < KS16; ++s) {
      if (row_ok) f[s] = *(const u16x8*)(Qp + (int64_t)t * p.q.sN + 16 * s + 8 * hf);
      else f[s] = (u16x8)(0);
    }
  };
  u16x8 qf[QK8 ? 1 : KS16];
  if constexpr (!QK8) load_qf(qf);

  // int8 Q codes: lane holds Q[t][32s + 16hf .. +15], one step per wavefront.
  i32x4 q8[QK8 ? KS8 : 1];
  float dq = 0.0f;
  const float kc_step = QK8 ? p.kcs[bh] : 0.0f;   // step of this head's kbar codes
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
    // and the residual codes of the q . kbar term: q ~= dq (code + r / 256) with
    // r = clamp(rint((q / dq - code) * 256), -127, 127), kept in LDS (each lane reads
    // back only what it wrote)
#pragma unroll
    for (int s = 0; s < KS8; ++s) {
      i32x4 r8w;
#pragma unroll
      for (int wd = 0; wd < 4; ++wd) {
        unsigned int packed = 0, rpacked = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float y = vals[s][4 * wd + e] * inv;
          float c = __builtin_rintf(y);
          c = fminf(fmaxf(c, -127.0f), 127.0f);
          packed |= ((unsigned int)((int)c) & 0xffu) << (8 * e);
          float r = __builtin_rintf((y - c) * 256.0f);
          r = fminf(fmaxf(r, -127.0f), 127.0f);
          rpacked |= ((unsigned int)((int)r) & 0xffu) << (8 * e);
        }
        q8[s][wd] = (int)packed;
        r8w[wd] = (int)rpacked;
      }
      *(i32x4*)(R8s + ((w * KS8 + s) * 64 + lane) * 16) = r8w;
    }
    // the codes as multiplied, for inspection: lane (hf, ql) holds row t, columns
    // 32s + 16hf .. +15 of every k-step s
    if (p.q8_out) {
      if (row_ok) {
        int8_t* dst = p.q8_out + ((int64_t)bh * N + t) * D + 16 * hf;
#pragma unroll
        for (int s = 0; s < KS8; ++s) *(i32x4*)(dst + 32 * s) = q8[s];
      }
      if (lane == 0 && wrow0 < N) p.q8_scale_out[(int64_t)bh * ((N + 31) / 32) + (wrow0 >> 5)] = dq;
      if (p.codes_only) return;
    }
  }

  const int cnt = p.counts[bh * d.nQ + i];
  // The row's kept-block list, read through the constant address space so that
  // the (wave-uniform) reads are scalar loads that never wait behind vector loads.
  typedef const __attribute__((address_space(4))) unsigned int* const_u32_ptr;
  const const_u32_ptr lst32 = (const_u32_ptr)(p.lists + (int64_t)(bh * d.nQ + i) * d.lstride);
  auto list_at = [&](int k) -> int {
    const unsigned int wv = lst32[k >> 1];
    return (int)((k & 1) ? (wv >> 16) : (wv & 0xffffu));
  };
  // int8 K steps of this head's blocks, read the same way (scalar loads)
  typedef const __attribute__((address_space(4))) float* const_f32_ptr;
  const const_f32_ptr ksc = (const_f32_ptr)(p.kscale + (QK8 ? (int64_t)bh * d.nK : 0));
  auto kscale_at = [&](int j) -> float { return ksc[j]; };

  // LDS addresses of this lane's transposing V reads per 32-column tile dt (row
  // 8(g/2) + k/4 of a k-step, granule swizzled as the DMA stores it), per stage;
  // k-step sg and read q add the immediate offset (16sg + 4q) rows.
  const int gq = lane >> 4, kq = lane & 15;
  unsigned int va0[DT], va1[DT];
  {
    const int vr = 8 * (gq >> 1) + (kq >> 2);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int col = 32 * dt + 16 * (gq & 1) + 4 * (kq & 3);
      const int pg = (col >> 3) ^ fv<VG>(vr);
      const int off = vr * VROW + 16 * pg + 2 * (col & 7);
      va0[dt] = (unsigned int)(size_t)(lds_u8_ptr)Vs0 + off;
      va1[dt] = (unsigned int)(size_t)(lds_u8_ptr)Vs1 + off;
    }
  }

  // fp8 P.V: byte offsets of this lane's two 16-byte reads of V^T column tile 0
  // (channel ql, keys 32hf + 16q .. +15 = logical granule 2hf + q); tile dt adds
  // 32 rows.  Granules are swizzled by (row / 4) % 4, as the DMA stores them.
  unsigned int v8a[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) v8a[q] = (unsigned int)(ql * 64 + 16 * ((2 * hf + q) ^ ((ql >> 2) & 3)));

  f32x16 oacc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) oacc[dt] = (f32x16)(0.0f);
  // fp8 P.V: the row sums come from one more (16x16x128) MFMA whose A selects, with
  // E4M3 ones (0x38), the key groups of each lane's own query, so they add exactly
  // the rounded P that the P.V MFMAs see; element 0 of lacc then holds the lane's
  // query-row sum over all 64 keys of each block.
  f32x4 lacc = (f32x4)(0.0f);
  float m_true = kNegInf;   // running row max of the visited blocks (filter)
  float m_ref = kNegInf;    // reference max of the exponentials
  float m_use = 0.0f;       // m_ref, or 0 while it is -inf
  // 16-bit P.V after the int8 Q.K^T: row sums on the MFMA (rowsum16); element 0 holds
  // this lane's query row sum (the other elements are not rescaled and not read).
  // After the 16-bit Q.K^T (whose Q fragments take twice the registers) the extra
  // registers would spill: there the sums are v_dot2 on the packed pairs (l_acc).
  constexpr bool kSumMfma = QK8;
  f32x4 lsum = (f32x4)(0.0f);
  float l_acc = 0.0f;       // this lane's partial row sum (its half of the keys)
  const unsigned short one16 = PV_F16 ? 0x3c00 : 0x3f80;
  const u16x8 lsel = (u16x8)((((lane >> 2) & 1) == ((lane >> 4) & 1)) ? one16 : (unsigned short)0);
  unsigned int n_skip = 0;

  // Direct-to-LDS loads of one block's K tile (into K stage KS) or V tile (into V
  // stage VS): wavefront w issues chunks w, w+4, ... of the tile; lane l of chunk c
  // fills LDS bytes 1024c + 16l, i.e. row r = c*1024/ROW + l/G, physical granule
  // l%G, holding logical granule (l%G) ^ f(r).
  // Per-lane byte offsets of this wavefront's chunks (c = 4cc + w) inside a block;
  // the block's base address is wave-uniform, so each load is a buffer resource in
  // SGPRs plus one 32-bit vector offset.
  constexpr int KCW = KCHUNK / 4, VCW = VCHUNK / 4;
  unsigned int koff[KCW], voff[VCW];
#pragma unroll
  for (int cc = 0; cc < KCW; ++cc) {
    const int r = (4 * cc + w) * (1024 / KROW) + lane / KG;
    koff[cc] = (unsigned int)(r * ksrow + 16 * ((lane % KG) ^ fkx<KG, PV8>(r)));
  }
#pragma unroll
  for (int cc = 0; cc < VCW; ++cc) {
    if constexpr (PV8) {
      // chunk c: channel rows 16c .. 16c+15 of the contiguous E4M3 tile
      const int r = 16 * (4 * cc + w) + lane / 4;
      voff[cc] = (unsigned int)(r * 64 + 16 * ((lane & 3) ^ ((r >> 2) & 3)));
    } else {
      const int r = (4 * cc + w) * (1024 / VROW) + lane / VG;
      voff[cc] = (unsigned int)(r * vsrow + 16 * ((lane % VG) ^ fv<VG>(r)));
    }
  }
  // Each load is a raw buffer load to LDS (buffer_load_dwordx4 ... lds): a buffer
  // resource over the block's own rows (base, byte extent) in SGPRs and this lane's
  // 32-bit offset, so a full block and the ragged last one take the same
  // instructions: rows past N lie outside the resource's extent and read as zeros
  // (their scores are masked and their P is zero, so they contribute nothing).
  // Block bases are 32 x 32 -> 64-bit products (row strides are below 4 GB).
  constexpr int kRsrcWord3 = 0x00020000;   // gfx9 raw buffer: 32-bit data format
  const unsigned int ksrow32 = (unsigned int)ksrow, vsrow32 = (unsigned int)vsrow;
  auto dma_k = [&](int j, auto kstage) {
    unsigned char* dst = decltype(kstage)::value ? Ks1 : Ks0;
    const char* base = Kb + (uint64_t)(unsigned int)(64 * j) * ksrow32;
    const int rows = QK8 ? 64 : min(64, N - 64 * j);   // int8 codes are padded to whole blocks
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)base, (short)0, (int)((unsigned int)(rows - 1) * ksrow32 + (unsigned int)KROW), kRsrcWord3);
#pragma unroll
    for (int cc = 0; cc < KCW; ++cc)
      buffer_lds16(r, (lds_void_ptr)(dst + 1024 * (4 * cc + w)), koff[cc]);
  };
  auto dma_v = [&](int j, auto vstage) {
    unsigned char* dst = decltype(vstage)::value ? Vs1 : Vs0;
    // fp8 tiles are whole (tokens past N are stored as zeros)
    const char* base = PV8 ? Vb + (uint64_t)(unsigned int)j * (64 * D)
                           : Vb + (uint64_t)(unsigned int)(64 * j) * vsrow32;
    const unsigned int extent = PV8 ? (unsigned int)(64 * D)
                                    : (unsigned int)(min(64, N - 64 * j) - 1) * vsrow32 + (unsigned int)VROW;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)extent, kRsrcWord3);
#pragma unroll
    for (int cc = 0; cc < VCW; ++cc)
      buffer_lds16(r, (lds_void_ptr)(dst + 1024 * (4 * cc + w)), voff[cc]);
  };

  // per-lane row of the Q.K^T A fragments, granule 2s+hf: 32kt + swap23(ql), or for
  // the fp8 P.V 16kt + krow_l with keys 32hf' .. 32hf'+31 of the P.V MFMA on the
  // rows of lane half hf' (row m holds key 32((m/4)%2) + 16kt + 4(m/8) + m%4)
  const int krow_l = PV8 ? (32 * ((ql >> 2) & 1) + 4 * (ql >> 3) + (ql & 3)) : swap23(ql);
  constexpr int KTROW = PV8 ? 16 : 32;
  typedef std::conditional_t<QK8, i32x16, f32x16> acc_t;
  static_assert(!QK8 || 127 * 127 * D < (kScoreBits & 0x7fffff), "int8 scores leave the binade");

  // Raw Q.K^T of the block staged in K stage KS (MFMAs only; no waits on results).
  // The K fragments of k-step s sit at row krow_l (kt = 0) and row krow_l + KTROW
  // (kt = 1, the same granule swizzle), granule (2s + hf) ^ f(row): per-lane offsets
  // koff_s, and the kt = 1 read is the same address plus an immediate.  The reads run
  // KSLOT - 1 k-steps ahead of the MFMAs (inline asm with explicit waits).
  constexpr int KSTEPS = QK8 ? KS8 : KS16;
  constexpr int KSLOT = 3;
  unsigned int koffs[KSTEPS];
#pragma unroll
  for (int s = 0; s < KSTEPS; ++s)
    koffs[s] = (unsigned int)(krow_l * KROW + 16 * ((2 * s + hf) ^ fkx<KG, PV8>(krow_l)));
  // cb(k-step) runs after each k-step's MFMAs (other work to interleave with them).
  // The scores land in sc as fp32 (int8 path: in the biased form kScoreC0 + s 2^-26).
  auto qk = [&](auto kstage, f32x16 (&sc)[2], auto cb) {
    const unsigned int kb = (unsigned int)(size_t)(lds_u8_ptr)(decltype(kstage)::value ? Ks1 : Ks0);
    acc_t acc[2];
    if constexpr (!QK8) {
      acc[0] = (acc_t)(0);
      acc[1] = acc[0];
    }
    u32x4 kf[KSLOT][2];
    auto kissue = [&](auto sc) {
      constexpr int s = decltype(sc)::value;
      const unsigned int a = kb + koffs[s];
      kf[s % KSLOT][0] = ds_read16<0>(a);
      kf[s % KSLOT][1] = ds_read16<KTROW * KROW>(a);
    };
    static_for<0, (KSLOT - 1 < KSTEPS ? KSLOT - 1 : KSTEPS)>(kissue);
    static_for<0, KSTEPS>([&](auto stc) {
      constexpr int s = decltype(stc)::value;
      constexpr int ahead = (KSTEPS - 1 - s) < (KSLOT - 2) ? (KSTEPS - 1 - s) : (KSLOT - 2);
      lds_wait16<2 * ahead>(kf[s % KSLOT][0], kf[s % KSLOT][1]);
      if constexpr (s + KSLOT - 1 < KSTEPS) kissue(std::integral_constant<int, s + KSLOT - 1>{});
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        if constexpr (!QK8)
          acc[kt] = mma16<IN_F16>(__builtin_bit_cast(u16x8, kf[s % KSLOT][kt]), qf[s], acc[kt]);
        else if constexpr (s == 0)
          acc[kt] = mfma_i8_first(__builtin_bit_cast(i32x4, kf[s % KSLOT][kt]), q8[s]);
        else
          acc[kt] = __builtin_amdgcn_mfma_i32_32x32x32_i8(__builtin_bit_cast(i32x4, kf[s % KSLOT][kt]),
                                                          q8[s], acc[kt], 0, 0, 0);
      }
      cb(stc);
    });
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) sc[kt] = __builtin_bit_cast(f32x16, acc[kt]);
  };
  auto no_cb = [](auto) {};

  // Invisible keys to -inf, and the row max of the raw scores (both lane halves);
  // key of sc[kt][r] is 64j + 8hf + key_off2(kt, r), or with the fp8 P.V
  // 64j + 32hf + 16kt + r.
  auto mask_max = [&](int j, f32x16 (&sc)[2]) -> float {
    if ((64 * j + 64 > N) || (p.causal && 64 * j + 63 > wrow0) || (wrow0 + 31 >= N)) {
      const int rel = lim - 64 * j - (PV8 ? 32 : 8) * hf;
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          sc[kt][r] = (PV8 ? 16 * kt + r : key_off2(kt, r)) < rel ? sc[kt][r] : kNegInf;
    }
    float mraw = kNegInf;
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int r = 0; r < 16; r += 2) mraw = max3f(mraw, sc[kt][r], sc[kt][r + 1]);
    return max_xor32(mraw);
  };

  // Software pipeline over the kept blocks.  Step `it` (block j = list[it]):
  //   wait for K(it+1) and V(it) -> barrier -> DMA K(it+2) and V(it+1) ->
  //   issue Q.K^T of block it+1 -> softmax of block it (its mask/max were done
  //   during the previous step) -> P.V of block it -> mask/max of block it+1.
  // K is staged two blocks ahead and V one block ahead in two stages each; every
  // stage is its own LDS variable and the loop is unrolled by two, so no DMA ever
  // targets a stage that is being read in the same step.
  std::integral_constant<int, 0> s0;
  std::integral_constant<int, 1> s1;
  int j_cur = cnt > 0 ? list_at(0) : 0;   // block of step it
  int j_n1 = cnt > 1 ? list_at(1) : 0;    // block it+1
  int j_n2 = cnt > 2 ? list_at(2) : 0;    // block it+2
  // The list as 32-bit words of two entries, one scalar load per two steps: at an
  // even step it, lw holds entries it+2 and it+3 and the word of it+4 and it+5 is
  // loaded for the next two steps.  Word indices are clamped into the row.
  const int lw_last = (d.lstride >> 1) - 1;
  // int8 path: the two kbar code rows of kept blocks it1 .. it1+15 (it1 a multiple of
  // 16) into KC, by direct-to-LDS loads (1 KB chunks, one per wavefront); each row's
  // 16-byte granules XOR-swizzled by the row, so that the pass's fragment reads are
  // free of bank conflicts.  Entries past the list's end load block 0.
  auto dma_kc = [&](int it1) {
    constexpr int RB = 2 * D, G = RB / 16, RPC = 1024 / RB, NCH = 16 * RB / 1024;
    if (w < NCH) {
      unsigned int lwv[RPC / 2];
#pragma unroll
      for (int q = 0; q < RPC / 2; ++q) lwv[q] = lst32[min((it1 >> 1) + (RPC * w) / 2 + q, lw_last)];
      const int rr = lane / G, row = RPC * w + rr;
      const unsigned int wv = lwv[rr >> 1];
      const int jb = (it1 + row < cnt) ? (int)((rr & 1) ? (wv >> 16) : (wv & 0xffffu)) : 0;
      const int lg = (lane % G) ^ (row & (G - 1));
      __builtin_amdgcn_global_load_lds((const void*)(p.kc + ((int64_t)bh * d.nK + jb) * RB + 16 * lg),
                                       (lds_void_ptr)(KCs + 1024 * w), 16, 0, 0);
    }
  };
  unsigned int lw = lst32[min(1, lw_last)];
  // scores of the current block, fp32 with invisible keys at -inf: two sets, so that
  // the step of parity P reads one while the next block's Q.K^T fills the other
  f32x16 scA[2], scB[2];
  float mraw_cur = kNegInf;
  float ks_cur = (QK8 && cnt > 0) ? kscale_at(j_cur) : 0.0f;
  if (cnt > 0) {
    dma_k(j_cur, s0);
    if (cnt > 1) dma_k(j_n1, s1);
    dma_v(j_cur, s0);
    if constexpr (QK8) dma_kc(0);
    wait_vmem_all();
    __syncthreads();
    qk(s0, scA, no_cb);
    mraw_cur = mask_max(j_cur, scA);
  }

  unsigned int lw_nxt = 0u;
  auto step = [&](int it, auto par) {
    constexpr int P = decltype(par)::value;        // it & 1
    // this block's scores, and the next block's made in this step
    f32x16 (&sc_cur)[2] = P ? scB : scA;
    f32x16 (&sc_nxt)[2] = P ? scA : scB;
    std::integral_constant<int, P> sp;
    std::integral_constant<int, 1 - P> sq;
    const int j = j_cur;
    int j_n3;
    if constexpr (P == 0) {
      j_n3 = (int)(lw >> 16);                              // entry it+3
      lw_nxt = lst32[min((it >> 1) + 2, lw_last)];         // entries it+4, it+5
    } else {
      j_n3 = (int)(lw_nxt & 0xffffu);                      // entry it+3 (= it+4 of the even step)
      lw = lw_nxt;
    }
    if (it + 3 >= cnt) j_n3 = 0;
    const float ks_nxt = QK8 ? kscale_at(j_n1) : 0.0f;   // K step of the next block
    wait_vmem_all();     // this wavefront's DMAs of K(it+1) and V(it) have landed
    __syncthreads();     // ... and every wavefront's; K stage P and V stage 1-P are free
    float bias = 0.0f;   // int8 path: c (q . kbar_j) for this lane's query, less the biased zero
    float slope_i8 = 0.0f;
    if constexpr (QK8) {
      float* cw = CWs + w * 16 * 32;   // per wave [16 blocks][32 queries]
      if ((it & 15) == 0) {
        // q . kbar_j of the next 16 kept blocks for this wave's queries, in integers
        // on the int8 MFMA: with q ~= dq (q8 + r8 / 256) and kbar ~= sk (c1 + c2 / 256)
        // (each second level within 1/512 of its first level's step),
        // q . kbar ~= dq sk (q8 . c1 + (q8 . c2 + r8 . c1) / 256), leaving out the
        // r8 . c2 term (2^-16 of the product's scale).  The codes of these blocks
        // were staged in KC a step ahead; rows 16..31 of the A operand repeat rows
        // 0..15 and their results are not used.  Everything a wave reads here is in
        // LDS and either shared read-only or its own, so no barrier is needed.
        constexpr int G = 2 * D / 16;   // 16-byte granules per code row
        const int krow = ql & 15;
        const unsigned char* kr = KCs + krow * 2 * D;
        i32x16 p1 = (i32x16)(0), p2 = (i32x16)(0);
#pragma unroll
        for (int s = 0; s < KS8; ++s) {
          const i32x4 a1 = *(const i32x4*)(kr + 16 * ((2 * s + hf) ^ (krow & (G - 1))));
          const i32x4 a2 = *(const i32x4*)(kr + 16 * ((G / 2 + 2 * s + hf) ^ (krow & (G - 1))));
          const i32x4 r8 = *(const i32x4*)(R8s + ((w * KS8 + s) * 64 + lane) * 16);
          p1 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, q8[s], p1, 0, 0, 0);
          p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a2, q8[s], p2, 0, 0, 0);
          p2 = __builtin_amdgcn_mfma_i32_32x32x32_i8(a1, r8, p2, 0, 0, 0);
        }
        // lane (hf, ql) holds the result of block (r/4)*8 + 4hf + r%4 and query ql;
        // blocks 0..15 are r < 8
        const float sc = dq * kc_step;
#pragma unroll
        for (int r = 0; r < 8; ++r)
          cw[((r >> 2) * 8 + 4 * hf + (r & 3)) * 32 + ql] = sc * __builtin_fmaf((float)p2[r], 0.00390625f, (float)p1[r]);
      }
      bias = p.c * cw[(it & 15) * 32 + ql];
      // dq * dk can be 0 (an all-zero group or block); keep the slope positive so
      // that masked (-inf) scores stay -inf.  Per unit of the biased score the slope
      // is 2^26 times that of s, and the offset takes away kScoreC0 times it.
      slope_i8 = fmaxf(p.c * dq * ks_cur, 1e-30f) * kScoreUnit;
      bias = __builtin_fmaf(-slope_i8, kScoreC0, bias);
    }
    // DMAs of K(it+2) and V(it+1), and before a q . kbar pass the next 16 blocks'
    // kbar codes (the pass 15 steps ago has read KC, and every wavefront has passed
    // a barrier since)
    if (it + 2 < cnt) dma_k(j_n2, sp);
    if (it + 1 < cnt) dma_v(j_n1, sq);
    if constexpr (QK8) {
      if ((it & 15) == 15 && it + 1 < cnt) dma_kc(it + 1);
    }
    // The next block's Q.K^T (in a row's last step this multiplies whatever K stage
    // 1-P holds; the result is converted but never used).  With the 16-bit P.V it is
    // issued below, interleaved with this block's first P fragment.
    if constexpr (PV8) qk(sq, sc_nxt, no_cb);
    // 16-bit P.V: the raw max of the next block's scores is taken in quarters between
    // the P.V MFMAs, in the same basic block, so that this work overlaps the MFMAs;
    // masking, when the block needs it, follows the P.V
    float mr_nxt = kNegInf;
    auto max_quarter = [&](auto qc) {
      constexpr int q = decltype(qc)::value, kt = q >> 1, r0 = 8 * (q & 1);
#pragma unroll
      for (int r = r0; r < r0 + 8; r += 2) mr_nxt = max3f(mr_nxt, sc_nxt[kt][r], sc_nxt[kt][r + 1]);
    };

    // block max of this row in log2 units, -inf when no key is visible
    float mx;
    if constexpr (QK8) mx = (mraw_cur == kNegInf) ? kNegInf : __builtin_fmaf(mraw_cur, slope_i8, bias);
    else mx = mraw_cur * p.c;

    bool skip = false;
    if (p.filter_on) {
      const float m_new = fmaxf(m_true, mx);
      const bool keep = (mx != kNegInf) && (mx - m_new >= lam2);
      if (__ballot(keep) == 0ull) {
        ++n_skip;
        skip = true;
      } else {
        m_true = m_new;
      }
    }
    if (!skip) {
      // fp8 P.V: the reference is the integer ceiling of the row's running max, moved
      // as soon as the max passes it (no slack): every P of the block is then
      // 2^(x - reference + 8) <= 2^8, inside E4M3's range with its largest values
      // near the top of it, and every rescale is an exact power of two
      if (__ballot(mx > m_ref + (PV8 ? 0.0f : kTau)) != 0ull) {
        const float m_ref_new = PV8 ? __builtin_ceilf(fmaxf(m_ref, mx)) : fmaxf(m_ref, mx);
        const float mu_new = (m_ref_new == kNegInf) ? 0.0f : m_ref_new;
        const float alpha = __builtin_amdgcn_exp2f(m_ref - mu_new);
        if constexpr (PV8) lacc[0] *= alpha;   // the only element read
        else if constexpr (kSumMfma) lsum[0] *= alpha;   // the only element read
        else l_acc *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) oacc[dt] *= alpha;
        m_ref = m_ref_new;
        m_use = mu_new;
      }
      if constexpr (PV8) {
        // V^T as E4M3: tile dt's A fragment is channel 32dt + ql, keys 32hf .. +31
        const unsigned char* Vst = P ? Vs1 : Vs0;
        u32x4 vfr[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int q = 0; q < 2; ++q) vfr[dt][q] = *(const u32x4*)(Vst + v8a[q] + 2048 * dt);
        // P = 2^(score * slope + offset - m_use + 8) as E4M3: word q holds keys
        // 32hf + 4q .. +3, which are sc_cur[q / 4][4(q % 4) .. +3]
        const float slope = QK8 ? slope_i8 : p.c;
        const float offs = (QK8 ? bias : 0.0f) - m_use + 8.0f;
        i32x8 pb;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          const int kt = q >> 2, r = 4 * (q & 3);
          float e[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) e[x] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[kt][r + x], slope, offs));
          pb[q] = pack_fp8x4(e[0], e[1], e[2], e[3]);
        }
        const i32x8 sel8 = (i32x8)((((lane >> 2) & 1) == ((lane >> 4) & 1)) ? 0x38383838 : 0);
        lacc = rowsum_fp8(sel8, pb, lacc);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const i32x8 vf = __builtin_bit_cast(
              i32x8, __builtin_shufflevector(vfr[dt][0], vfr[dt][1], 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = mma_fp8(vf, pb, oacc[dt]);
        }
      } else {
        // V^T fragments by transposing LDS reads: for k-step sg (keys 16sg..16sg+15),
        // tile dt, lane group g = lane/16 and k = lane%16, read q in {0, 1} covers keys
        // 16sg + 8(g/2) + 4q + k/4, columns 32dt + 16(g&1) + 4(k&3) .. +3.  The (sg, dt)
        // pairs u = DT*sg + dt run in order with kVAhead pairs' reads in flight; the
        // first ones are issued before the exponentials.
        const unsigned int* va = P ? va1 : va0;
        s16x4 fr[kVAhead + 1][2];
        auto issue = [&](auto uc) {
          constexpr int u = decltype(uc)::value, sg = u / DT, dt = u % DT;
          fr[u % (kVAhead + 1)][0] = ds_read_tr<16 * sg * VROW>(va[dt]);
          fr[u % (kVAhead + 1)][1] = ds_read_tr<(16 * sg + 4) * VROW>(va[dt]);
        };
        static_for<0, kVAhead>(issue);
        __builtin_amdgcn_sched_barrier(0);   // keep these reads ahead of the exponentials
        // P = 2^(score * slope + offset - m_use), rounded to the P.V type in pairs.  The
        // B fragment of k-step k (pw[k]) holds keys 32(k/2) + 16(k%2) + ..; each is made
        // just before it is needed, so the exponentials of k-step k+1 run under the
        // MFMAs of k-step k.
        const float slope = QK8 ? slope_i8 : p.c;
        const float offs = (QK8 ? bias : 0.0f) - m_use;
        u32x4 pw[4];
        auto make_pw_word = [&](auto kc, auto wc) {
          constexpr int k = decltype(kc)::value, kt = k >> 1, sg = k & 1;
          constexpr int r = 8 * sg + 2 * decltype(wc)::value;
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[kt][r], slope, offs));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sc_cur[kt][r + 1], slope, offs));
          const unsigned int pr = pack2<PV_F16>(p0, p1);
          if constexpr (!kSumMfma) l_acc = add_pair<PV_F16>(pr, l_acc);
          pw[k][decltype(wc)::value] = pr;
        };
        auto make_pw = [&](auto kc) { static_for<0, 4>([&](auto wc) { make_pw_word(kc, wc); }); };
        // words of the first P fragment after each k-step of the next block's Q.K^T
        qk(sq, sc_nxt, [&](auto stc) {
          constexpr int s = decltype(stc)::value;
          static_for<0, 4>([&](auto wc) {
            constexpr int wd = decltype(wc)::value;
            if constexpr (wd * KSTEPS / 4 == s && (KSTEPS <= 4 || wd * KSTEPS % 4 == 0))
              make_pw_word(std::integral_constant<int, 0>{}, wc);
          });
        });
        static_for<0, kNU>([&](auto uc) {
          constexpr int u = decltype(uc)::value, sg = u / DT, dt = u % DT;
          if constexpr (u + kVAhead < kNU) issue(std::integral_constant<int, u + kVAhead>{});
          constexpr int later = (kNU - 1 - u) < kVAhead ? (kNU - 1 - u) : kVAhead;
          s16x4& f0 = fr[u % (kVAhead + 1)][0];
          s16x4& f1 = fr[u % (kVAhead + 1)][1];
          lds_wait<2 * later>(f0, f1);
          const u16x8 vf = __builtin_bit_cast(u16x8, __builtin_shufflevector(f0, f1, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[dt] = mma16<PV_F16>(vf, __builtin_bit_cast(u16x8, pw[sg]), oacc[dt]);
          if constexpr (kSumMfma && dt == 1)
            lsum = rowsum16<PV_F16>(lsel, __builtin_bit_cast(u16x8, pw[sg]), lsum);
          if constexpr (dt == 0 && sg + 1 < 4) make_pw(std::integral_constant<int, sg + 1>{});
          if constexpr (u % (kNU / 4) == 1) max_quarter(std::integral_constant<int, u / (kNU / 4)>{});
        });
      }
      }
    // the next block's scores: mask and max (fp8 P.V: all of it here, under the
    // MFMAs still in flight)
    if constexpr (PV8) {
      if (it + 1 < cnt) mraw_cur = mask_max(j_n1, sc_nxt);
    } else {
      if (skip) {   // the P.V (and the Q.K^T and conversion issued inside it) did not run
        qk(sq, sc_nxt, no_cb);
        static_for<0, 4>(max_quarter);
      }
      if (it + 1 < cnt) {
        if ((64 * j_n1 + 64 > N) || (p.causal && 64 * j_n1 + 63 > wrow0) || (wrow0 + 31 >= N)) {
          const int rel = lim - 64 * j_n1 - 8 * hf;
          mr_nxt = kNegInf;
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              sc_nxt[kt][r] = key_off2(kt, r) < rel ? sc_nxt[kt][r] : kNegInf;
              mr_nxt = fmaxf(mr_nxt, sc_nxt[kt][r]);
            }
        }
        mraw_cur = max_xor32(mr_nxt);
      }
    }
    j_cur = j_n1;
    j_n1 = j_n2;
    j_n2 = j_n3;
    if constexpr (QK8) ks_cur = ks_nxt;
  };

  for (int it = 0; it < cnt; it += 2) {
    step(it, s0);
    if (it + 1 < cnt) step(it + 1, s1);
  }

  // epilogue: O = acc / l, this lane's query row, columns 32dt + 8g + 4hf + 0..3
  const float lt = PV8 ? lacc[0] : kSumMfma ? lsum[0] : l_acc + partner32(l_acc, hf);
  const float inv = lt > 0.0f ? 1.0f / lt : 0.0f;
  if (row_ok) {
    // fp8 P.V: the channel scales of the E4M3 V codes, all loaded before any store
    float4 vs[PV8 ? DT : 1][4];
    if constexpr (PV8) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int g = 0; g < 4; ++g)
          vs[dt][g] = *(const float4*)(p.vscale + (int64_t)bh * D + 32 * dt + 8 * g + 4 * hf);
    }
    char* ob = (char*)p.o;
    const int esz = p.out_type == kF32 ? 4 : 2;
    const int64_t rowoff = ((int64_t)b * p.osB + (int64_t)h * p.osH + (int64_t)t * p.osN) * esz;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = 32 * dt + 8 * g + 4 * hf;
        float o0 = oacc[dt][4 * g] * inv, o1 = oacc[dt][4 * g + 1] * inv;
        float o2 = oacc[dt][4 * g + 2] * inv, o3 = oacc[dt][4 * g + 3] * inv;
        if constexpr (PV8) {
          o0 *= vs[dt][g].x;
          o1 *= vs[dt][g].y;
          o2 *= vs[dt][g].z;
          o3 *= vs[dt][g].w;
        }
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
  if (p.pv_fp8) {
    if (p.qk_int8) sparse_attn_kernel<D, IN_F16, false, true, true><<<grid, 256, 0, s>>>(p, d);
    else sparse_attn_kernel<D, IN_F16, false, false, true><<<grid, 256, 0, s>>>(p, d);
  } else if (p.qk_int8) {
    if (p.pv_fp16) sparse_attn_kernel<D, IN_F16, true, true, false><<<grid, 256, 0, s>>>(p, d);
    else sparse_attn_kernel<D, IN_F16, IN_F16, true, false><<<grid, 256, 0, s>>>(p, d);
  } else {
    if (p.pv_fp16) sparse_attn_kernel<D, IN_F16, true, false, false><<<grid, 256, 0, s>>>(p, d);
    else sparse_attn_kernel<D, IN_F16, IN_F16, false, false><<<grid, 256, 0, s>>>(p, d);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_sparse_attn(const AttnParams& p, const Dims& d, hipStream_t s) {
  if (d.D == 64) return p.in_f16 ? launch_d<64, true>(p, d, s) : launch_d<64, false>(p, d, s);
  return p.in_f16 ? launch_d<128, true>(p, d, s) : launch_d<128, false>(p, d, s);
}

}  // namespace sparge
