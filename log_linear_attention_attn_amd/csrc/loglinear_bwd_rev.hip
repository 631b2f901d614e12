// Reverse register-state sweep of the backward, bf16 inputs, C = 64, dk = dv = 128:
//
//   y_s = sum_{t >= s} M[t,s] (c_t . x_s) a_t,   M[t,s] = lambda[t, l(t,s)] exp(cum_t - cum_s)
//   MODE 0: dV (c = q, x = k, a = dO);  MODE 1: dK (c = dO, x = v, a = q)
//
// ([P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制",
// sections 并行形式 and 训练：分块并行扫描算法; the gradient of its parallel form).
//
// The level weight sits on the summed index t, so the level states of this
// sum cannot be merged by the lssb rule of the forward.  For a chunk-level
// bit b, every aligned block of 2^(b+1) chunks pairs its right half (the t
// side) with its left half (the s side).  Walking the chunks backwards, the
// right half is visited first and accumulates
//   R_b = sum_{t in right half} lambda[t, log2C+1+b] exp(cum_t - ref) c_t a_t^T
// (ref = cum at the end of the left half), which every chunk of the left half
// then reads: y_s += exp(ref - cum_s) x_s . R_b.
//
// One workgroup = (b,h, segment of 2^S chunks, 64 output columns), eight
// waves; wave (c, h) owns output columns 16c..16c+15 and half h of the
// contraction.  Levels below S live in the wave's registers: fp32 while their
// right half accumulates, packed fp16 with a power-of-two scale while their
// left half reads them.  The levels spanning segments reach a segment as one
// suffix state (every t after the segment sees it at the level fixed by the
// highest differing segment bit), summed at the start of the sweep from
// per-(segment, level) states that the pre-pass (PREP) forms with the same
// accumulation.  Those states are sum_t w_t q_t dO_t^T for dV and their
// transposes for dK, so one pre-pass serves both.
//
// Every product runs on fp16 matrix cores.  c, x and a are staged as fp16
// rows scaled by a power of two each (their row maximum in [2^14, 2^15)),
// the masked score tiles with one power-of-two scale per 16 x 16 tile, the
// weighted a of a level update with one per (level, chunk), and the
// accumulated state carries a running exponent: every scale stays outside
// the fp16 operands, so no operand leaves fp16's normal range.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {
namespace rv {

constexpr int C = 64, DC = 128, LOGC = 6, NLEV = 5, NTH = 512, LMAX = 16;
constexpr int LDC = DC + 8;  // fp16 rows of the c and x tiles
// the pre-pass reads its c tile only transposed (level updates): rows of 80
// banks, 16 modulo 64, put the four rows and four 16-byte pieces a 16-lane
// group reads on disjoint banks (the sweeps also read c by rows, for which
// LDC's 68 banks are the conflict-free stride)
constexpr int LDC_PREP = DC + 32;
constexpr int LDA = 64 + 8;  // fp16 rows of the a tile (the group's 64 columns)
// LDS layouts.  The tiles and row data read in phase 2 are double-buffered
// by chunk parity; everything else is written after the chunk's first
// barrier and read before the next chunk's first barrier.  The pre-pass keeps
// only c, a, the row data, the weights and lambda, so two of its workgroups
// share a CU.
template <bool PREP>
struct Lay;
template <>
struct Lay<false> {
  static constexpr int CH = 0;                         // c fp16 [2][64][LDC]
  static constexpr int XH = CH + 2 * C * LDC * 2;      // x fp16 [2][64][LDC]
  static constexpr int AH = XH + 2 * C * LDC * 2;      // a fp16 [2][64][LDA]
  static constexpr int AL = AH + 2 * C * LDA * 2;      // fp16 residual of a (fp32 a only) [2][64][LDA]
  static constexpr int PS = AL + 2 * C * LDA * 2;      // score tiles fp16 [hi, lo][4 sb][4 tb][64 lanes] x 8 B
  static constexpr int XC = PS + 2 * 16 * 64 * 8;      // partner partial sums [8][2][64] f32x4
  static constexpr int ROW = XC + 8 * 2 * 64 * 16;     // [2] x {cl (log2), ec, ex, ea} [64]
  static constexpr int RF = ROW + 2 * 4 * C * 4;       // left-read row factors [64]
  static constexpr int WT = RF + C * 4;                // level-update token weights fp16 [NLEV][64]
  static constexpr int KE = WT + NLEV * C * 2;         // the states' new exponents [NLEV], tile exponents [16]
  static constexpr int LAM = KE + 32 * 4;              // lambda rows of the chunk [64][L]
  // dV sweep only: v of the group's columns, fp16 [64][LDA], its row
  // exponents [64], the in-chunk dlambda row sums [2][64][8] and the v . dV
  // row sums of the four 16-column slices [2][64][4]
  static constexpr int VH = LAM + C * LMAX * 4;
  static constexpr int EV = VH + C * LDA * 2;
  static constexpr int ISL = EV + C * 4;
  static constexpr int VSL = ISL + 2 * C * 8 * 4;
  static constexpr int BYTES = VSL + 2 * C * 4 * 4;
};
template <>
struct Lay<true> {
  static constexpr int CH = 0;
  static constexpr int AH = CH + 2 * C * LDC_PREP * 2;
  static constexpr int ROW = AH + 2 * C * LDA * 2;
  static constexpr int WT = ROW + 2 * 4 * C * 4;
  static constexpr int KE = WT + NLEV * C * 2;
  static constexpr int LAM = KE + 32 * 4;
  static constexpr int BYTES = LAM + C * LMAX * 4;
  static constexpr int XH = 0, AL = 0, PS = 0, XC = 0, RF = 0, VH = 0, EV = 0, ISL = 0, VSL = 0;  // not used by the pre-pass
};
// register levels of the pre-pass variant that shares a CU with another
constexpr int NL_SMALL = 3;

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef _Float16 __attribute__((ext_vector_type(4))) f16x4;
typedef int __attribute__((ext_vector_type(4))) i32x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int __attribute__((ext_vector_type(4))) u32x4;

// Transposed 8-byte LDS read: within each 16-lane group, lane i receives
// element (i & 3) of the 4-element vectors addressed by lanes 4k + (i >> 2).
__device__ __forceinline__ f16x4 tr_read(const _Float16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<__attribute__((address_space(3))) char*>(reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(f16x4, v);
}
__device__ __forceinline__ f16x8 cat(f16x4 a, f16x4 b) { return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7); }
__device__ __forceinline__ f32x4 mma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
// Maxima of non-negative floats compare as unsigned integers.
template <int CTRL>
__device__ __forceinline__ unsigned dpp_umax(unsigned x) {
  return max(x, static_cast<unsigned>(
                    __builtin_amdgcn_update_dpp(0, static_cast<int>(x), CTRL, 0xf, 0xf, false)));
}
// max over the 64 lanes of a non-negative value, wave-uniform
__device__ __forceinline__ float wave_max(float v) {
  unsigned x = __float_as_uint(v);
  x = dpp_umax<0xb1>(x);   // quad_perm [1,0,3,2]
  x = dpp_umax<0x4e>(x);   // quad_perm [2,3,0,1]
  x = dpp_umax<0x124>(x);  // row_ror 4
  x = dpp_umax<0x128>(x);  // row_ror 8
  const unsigned a0 = __builtin_amdgcn_readlane(x, 0), a1 = __builtin_amdgcn_readlane(x, 16);
  const unsigned a2 = __builtin_amdgcn_readlane(x, 32), a3 = __builtin_amdgcn_readlane(x, 48);
  return __uint_as_float(max(max(a0, a1), max(a2, a3)));
}
// max over each aligned group of 16 lanes (one DPP row), non-negative values
__device__ __forceinline__ float row16_max(float v) {
  unsigned m = __float_as_uint(v);
  m = dpp_umax<0x121>(m);
  m = dpp_umax<0x122>(m);
  m = dpp_umax<0x124>(m);
  return __uint_as_float(dpp_umax<0x128>(m));
}
// max over each aligned group of 8 lanes, non-negative values
__device__ __forceinline__ float row8_max(float v) {
  unsigned m = __float_as_uint(v);
  m = dpp_umax<0xb1>(m);
  m = dpp_umax<0x4e>(m);
  return __uint_as_float(dpp_umax<0x141>(m));  // row_half_mirror
}
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sums over the 16 lanes of a 16-lane group of x[0..3]; lane li returns the
// total of x[li >> 2]: a reduce-scatter over lane bits 3 and 2 (each lane
// keeps half of its values and adds its partner's copy of them), then a sum
// over the four lanes of a quad.
__device__ __forceinline__ float rowsum16(const float x[4], int li) {
  const bool h8 = li & 8, h4 = li & 4;
  const float k0 = h8 ? x[2] : x[0], k1 = h8 ? x[3] : x[1];
  // the values a lane sends depend on its own lane bits: each is made opaque
  // (an empty asm) before the DPP read, so the compiler cannot substitute the
  // receiving lane's select into the sending lane's value
  float s0 = h8 ? x[0] : x[2], s1 = h8 ? x[1] : x[3];
  asm volatile("" : "+v"(s0), "+v"(s1));
  const float y0 = k0 + dpp_mov<0x128>(s0);  // row_ror 8: lane li ^ 8
  const float y1 = k1 + dpp_mov<0x128>(s1);
  float send = h4 ? y0 : y1;
  asm volatile("" : "+v"(send));
  // lane li ^ 4 in one exchange for every lane (ds_swizzle, bit mode: xor 4):
  // a per-lane choice between two DPP rotations can be compiled as a branch,
  // and a DPP read of a lane outside EXEC returns 0
  const float from = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(send), 0x101F));
  float z = (h4 ? y1 : y0) + from;
  z += dpp_mov<0xb1>(z);  // quad_perm [1,0,3,2]
  z += dpp_mov<0x4e>(z);  // quad_perm [2,3,0,1]
  return z;
}
// Sums over the 16 lanes of a 16-lane group of x[0..7]; lanes li and li ^ 1
// return the total of x[(li >> 1) & 7]: a reduce-scatter over lane bits 3,
// 2 and 1 as above, then a sum over lane bit 0.
__device__ __forceinline__ float rowsum16x8(const float x[8], int li) {
  const bool h8 = li & 8, h4 = li & 4, h2 = li & 2;
  float y[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float sd = h8 ? x[m] : x[4 + m];
    asm volatile("" : "+v"(sd));
    y[m] = (h8 ? x[4 + m] : x[m]) + dpp_mov<0x128>(sd);  // row_ror 8: lane li ^ 8
  }
  float z[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    float sd = h4 ? y[m] : y[2 + m];
    asm volatile("" : "+v"(sd));
    z[m] = (h4 ? y[2 + m] : y[m]) + __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(sd), 0x101F));
  }
  float sd = h2 ? z[0] : z[1];
  asm volatile("" : "+v"(sd));
  float u = (h2 ? z[1] : z[0]) + dpp_mov<0x4e>(sd);  // quad_perm [2,3,0,1]: lane li ^ 2
  u += dpp_mov<0xb1>(u);                              // quad_perm [1,0,3,2]: lane li ^ 1
  return u;
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
// inclusive prefix sum over the 64 lanes
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_add<0x111, 0xf>(x);
  x = dpp_add<0x112, 0xf>(x);
  x = dpp_add<0x114, 0xf>(x);
  x = dpp_add<0x118, 0xf>(x);
  x = dpp_add<0x142, 0xa>(x);
  x = dpp_add<0x143, 0xc>(x);
  return x;
}
// exponent e with mx * 2^-e in [2^14, 2^15); 0 for mx == 0; clamped
__device__ __forceinline__ int scale_exp(float mx) {
  if (!(mx > 0.f)) return 0;
  const int e = static_cast<int>((__float_as_uint(mx) >> 23) & 0xff) - 127 - 14;
  return max(-110, min(110, e));
}
__device__ __forceinline__ float ldexp_(float x, int e) { return __builtin_amdgcn_ldexpf(x, e); }
__device__ __forceinline__ int uniform_i(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}
constexpr float kLog2e = 1.4426950408889634f;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), static_cast<int>(bytes),
                                           0x00020000);
}
__device__ __forceinline__ u32x4 load_u4(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// One row segment of 8 values (bf16 or fp32) held by a lane.
struct Row8 {
  float v[8];
  __device__ __forceinline__ void from_bf16(u32x4 x) {
    const bf16x8 b = __builtin_bit_cast(bf16x8, x);
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = static_cast<float>(b[e]);
  }
  __device__ __forceinline__ void from_f32(u32x4 x0, u32x4 x1) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[e] = __uint_as_float(x0[e]);
      v[4 + e] = __uint_as_float(x1[e]);
    }
  }
  __device__ __forceinline__ float amax() const {
    float m = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(v[e]));
    return m;
  }
  __device__ __forceinline__ f16x8 scaled(int e2) const {
    f16x8 h;
#pragma unroll
    for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(ldexp_(v[e], -e2));
    return h;
  }
  // the rounding residual of scaled(e2)
  __device__ __forceinline__ f16x8 residual(int e2, f16x8 h) const {
    f16x8 l;
#pragma unroll
    for (int e = 0; e < 8; ++e) l[e] = static_cast<_Float16>(ldexp_(v[e], -e2) - static_cast<float>(h[e]));
    return l;
  }
};

}  // namespace rv

// MODE 0: dV; MODE 1: dK.  PREP (MODE 0 only): the per-(segment, level)
// states of the segments after the first (see the file comment); the dK sweep
// reads their transposes.  NL: levels held in registers.
template <int MODE, bool PREP, int NL>
__device__ __forceinline__ void rev_body(const BwdRevArgs& a, unsigned char* smem) {
  using namespace rv;
  using LY = Lay<PREP>;
  f16x4* Ps = reinterpret_cast<f16x4*>(smem + LY::PS);  // [hi, lo][sb][tb][lane]
  f32x4* Xc = reinterpret_cast<f32x4*>(smem + LY::XC);  // [wave][2][lane]
  float* rf_s = reinterpret_cast<float*>(smem + LY::RF);
  _Float16* WT = reinterpret_cast<_Float16*>(smem + LY::WT);
  int* ke_s = reinterpret_cast<int*>(smem + LY::KE);  // [0, NLEV): level updates; [16, 32): score tiles
  float* lam_s = reinterpret_cast<float*>(smem + LY::LAM);

  const int id = blockIdx.x;
  const int px = id & 7, rest = id >> 3;
  const int dg = rest & 1, pg = rest >> 1;  // two groups of 64 output columns
  const int p = pg * 8 + px;
  if (p >= a.BH * a.nseg) return;
  const int bh = p / a.nseg, seg = p - bh * a.nseg;
  if (PREP && seg == 0) return;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int cs = w & 3, hh = w >> 2;
  const int c0 = 16 * cs;
  const int T = a.T, L = a.L;
  const int N = (T + C - 1) / C;
  const int S = a.seg_log2;
  const int n0 = seg << S;
  const int n1 = min(N, n0 + (1 << S));
  const int col0 = dg * 64;
  const size_t bhT = (size_t)bh * T;
  // c: q (bf16) / dO (fp32); x: k / v (bf16); a: dO (fp32) / q (bf16)
  const rsrc_t cr = MODE == 0 ? make_rsrc(static_cast<const bf16*>(a.q) + bhT * DC, T * DC * 2)
                              : make_rsrc(a.dout + bhT * DC, T * DC * 4);
  const rsrc_t xr = make_rsrc(static_cast<const bf16*>(MODE == 0 ? a.k : a.v) + bhT * DC, T * DC * 2);
  const rsrc_t ar = MODE == 0 ? make_rsrc(a.dout + bhT * DC, T * DC * 4)
                              : make_rsrc(static_cast<const bf16*>(a.q) + bhT * DC, T * DC * 2);
  const rsrc_t lar = make_rsrc(a.log_a + bhT, T * 4);
  const rsrc_t lamr = make_rsrc(a.lam + bhT * L, T * L * 4);
  const rsrc_t yr = make_rsrc((MODE == 0 ? a.dv_out : a.dk_out) + bhT * DC, T * DC * 4);
  // dV sweep: v of the group's columns, for the in-chunk dlambda
  constexpr bool INTRA = MODE == 0 && !PREP;
  const bool intra = INTRA && a.intra_part != nullptr;
  const rsrc_t vr = make_rsrc(static_cast<const bf16*>(a.v) + bhT * DC, T * DC * 2);
  _Float16* Vh = reinterpret_cast<_Float16*>(smem + LY::VH);
  int* ev_s = reinterpret_cast<int*>(smem + LY::EV);
  float* isl = reinterpret_cast<float*>(smem + LY::ISL);
  float* vsl = reinterpret_cast<float*>(smem + LY::VSL);
  const int own0 = hh ? 1 : 0, own1 = hh ? 2 : 3;
  const int oth0 = hh ? 0 : 1, oth1 = hh ? 3 : 2;
  // levels held in registers: the chunk-level bits below S; in the pre-pass
  // the segment-level bits j of the segment that are set (lambda column
  // log2C + 1 + S + j)
  const int nlev = PREP ? a.nj : S;

  // ---- level states.  R[b][t], t = 2 kl + half, element r: contraction
  // index 64 hh + 32 kl + 8 g4 + 4 half + r, output column c0 + li of the
  // group; true value R * 2^kr[b].  Once the right half is complete, R[b][0]
  // and R[b][1] hold the fp16 read operand (element e of R[b][kl]:
  // contraction 64 hh + 32 kl + 8 g4 + e), true value * 2^er[b].
  f32x4 R[NL][4];
  int kr[NL], er[NL];
  float g2[NL];  // log2 decay from the end of the current chunk to the end of the left half
#pragma unroll
  for (int b = 0; b < NL; ++b) {
    kr[b] = 0;
    er[b] = 0;
    g2[b] = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t) R[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // ---- register prefetch of one chunk ----------------------------------------
  u32x4 pc[2][2], px8[2], pa[2], pv8;
  float plam[2], pla;
  const uint32_t off_a = static_cast<uint32_t>((tid >> 3) * DC + col0 + (tid & 7) * 8);
  auto prefetch = [&](int n) {
    const uint32_t tok0 = static_cast<uint32_t>(n * C);
    {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(lamr, (tok0 * L + 2 * tid) * 4, 0, 0);
      plam[0] = __uint_as_float(x[0]);
      plam[1] = __uint_as_float(x[1]);
    }
    pla = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lar, (tok0 + lane) * 4, 0, 0));
    const uint32_t ce = tok0 * DC;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + NTH * i;
      const uint32_t off = ce + (v >> 4) * DC + (v & 15) * 8;
      if constexpr (MODE == 0) {
        pc[i][0] = load_u4(cr, off * 2);
      } else {
        pc[i][0] = load_u4(cr, off * 4);
        pc[i][1] = load_u4(cr, off * 4 + 16);
      }
      if constexpr (!PREP) px8[i] = load_u4(xr, off * 2);
    }
    if constexpr (MODE == 0) {
      pa[0] = load_u4(ar, (ce + off_a) * 4);
      pa[1] = load_u4(ar, (ce + off_a) * 4 + 16);
      if constexpr (INTRA) pv8 = load_u4(vr, (ce + off_a) * 2);
    } else {
      pa[0] = load_u4(ar, (ce + off_a) * 2);
    }
  };
  prefetch(n1 - 1);

  // ---- the suffix state: sum over the later segments g' of
  //   exp(cum at the start of g' - cum at the end of this segment) P[g', j]
  // with j the highest bit in which g' and this segment differ
  f16x8 Rh[2] = {f16x8{}, f16x8{}};
  int eh = 0;
  const bool has_suffix = !PREP && seg + 1 < a.nseg;
  if (has_suffix) {
    f32x4 x[4] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f},
                  f32x4{0.f, 0.f, 0.f, 0.f}};
    float d2 = 0.f;
    for (int gq = seg + 1; gq < a.nseg; ++gq) {
      const int j = 31 - __clz(seg ^ gq);
      const float wgt = __builtin_amdgcn_exp2f(d2);
      const float* __restrict__ st = a.seg_part + ((size_t)(bh * a.nseg + gq) * a.nj + j) * DC * DC;
      if constexpr (MODE == 0) {
        const float* __restrict__ src = st + (col0 + c0 + li) * DC + 64 * hh + 8 * g4;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 y = *reinterpret_cast<const f32x4*>(src + 32 * ks + 4 * h);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[2 * ks + h][e] += wgt * y[e];
          }
      } else {
        // the dK state is the transpose of the dV one: sum w dO_t q_t^T
        const float* __restrict__ src = st + (64 * hh + 8 * g4) * DC + col0 + c0 + li;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int e = 0; e < 8; ++e) x[2 * ks + (e >> 2)][e & 3] += wgt * src[(32 * ks + e) * DC];
      }
      d2 += a.seg_tot2[bh * a.nseg + gq];
    }
    float mx = 0.f;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fabsf(x[t][e]));
    eh = scale_exp(wave_max(mx));
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        Rh[ks][e] = static_cast<_Float16>(ldexp_(x[2 * ks][e], -eh));
        Rh[ks][4 + e] = static_cast<_Float16>(ldexp_(x[2 * ks + 1][e], -eh));
      }
  }
  float dn2 = 0.f;  // log2 decay from the end of the current chunk to the end of the segment
  float tot2 = 0.f;

  // diagonal score tiles (s = 16 sb + li, t = 16 sb + 4 g4 + r): level and
  // the mask t >= s from the in-block positions
  int dlev[4];
  unsigned dmask = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    dlev[r] = level_of(li, 4 * g4 + r);
    dmask |= (4 * g4 + r >= li ? 1u : 0u) << r;
  }
  // chunk nc's in-chunk dlambda: one thread per (row, level); level 5 is the
  // key block next to the row's (odd row blocks), level 6 key blocks 0 and 1
  // (row blocks 2 and 3)
  // the helpers below derive their lane indices from an opaque copy of the
  // thread index, so the compiler recomputes them per chunk instead of
  // keeping them (and what it derives from them) live across the loop
  auto opaque = [](int x) {
    asm volatile("" : "+v"(x));
    return x;
  };
  auto flush_intra = [&](int nc) {
    const int tid_ = opaque(tid);
    if (tid_ < C * (LOGC + 1)) {
      const float* sl = isl + (nc & 1) * (C * 8);
      const int row = tid_ / (LOGC + 1), lv = tid_ - row * (LOGC + 1);
      const int tb = row >> 4, t = nc * C + row;
      float x;
      if (lv <= 4) x = sl[row * 8 + lv];
      else if (lv == 5) x = (tb & 1) ? sl[row * 8 + 5 + tb - 1] : 0.f;
      else x = tb >= 2 ? sl[row * 8 + 5] + sl[row * 8 + 6] : 0.f;
      if (t < T) a.intra_part[(((size_t)dg * a.BH + bh) * T + t) * 8 + lv] = x;
    }
  };
  // v_t . dV_t over the group's columns, the term the decay gradient
  // subtracts (the in-chunk products of this sweep are exact enough for the
  // cancellation of its diagonal terms against dO_t . O_t).  The wave's own
  // rows of chunk nv take v from global memory (read two chunks earlier, so
  // mostly from L2) at the chunk's store, where dV is final, loaded and used
  // within the store so that no register is held across the sweep's phases;
  // the reduction over the wave's 16 columns goes to word cs of the row in
  // the chunk's parity buffer, and the four slices' words are added (in
  // slice order) into word 7 of the row record one chunk later, after a
  // barrier
  constexpr bool VDV = INTRA;
  const bool vdv = intra;
  unsigned short vq[2][4];
  auto load_vdv = [&](int nv) {
    const int ln = opaque(lane);
    const int off = ((nv * C + 4 * (ln >> 4)) * DC + col0 + c0 + (ln & 15)) * 2;
#pragma unroll
    for (int o = 0; o < 2; ++o)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        vq[o][r] = __builtin_amdgcn_raw_buffer_load_b16(
            vr, static_cast<uint32_t>(off + ((16 * (o ? own1 : own0) + r) * DC) * 2), 0, 0);
  };
  auto vdv_rows = [&](int nv, const float f0[4], const float f1[4]) {
    float x[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      x[r] = __uint_as_float(static_cast<uint32_t>(vq[0][r]) << 16) * f0[r];
      x[4 + r] = __uint_as_float(static_cast<uint32_t>(vq[1][r]) << 16) * f1[r];
    }
    const int ln = opaque(lane), lj = ln & 15;
    const float sum = rowsum16x8(x, lj);
    const int j = (lj >> 1) & 7;
    if (!(lj & 1)) vsl[((nv & 1) * C + 16 * ((j >> 2) ? own1 : own0) + 4 * (ln >> 4) + (j & 3)) * 4 + cs] = sum;
  };
  auto flush_vdv = [&](int nv) {
    const int tid_ = opaque(tid);
    if (tid_ < C) {
      const float* sl = vsl + ((nv & 1) * C + tid_) * 4;
      const int t = nv * C + tid_;
      if (t < T) a.intra_part[(((size_t)dg * a.BH + bh) * T + t) * 8 + 7] = ((sl[0] + sl[1]) + sl[2]) + sl[3];
    }
  };
  f32x4 O0 = f32x4{0.f, 0.f, 0.f, 0.f}, O1 = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int n = n1 - 1; n >= n0; --n) {
    const int tok0 = n * C, par = n & 1;
    constexpr int LDCH = PREP ? LDC_PREP : LDC;  // row stride of the c tile
    // dK sweep: its c tile is read by rows (score tiles) and transposed (level
    // updates); 16-byte piece p of row r sits at p ^ ((r & 3) << 2), which
    // puts both a row read's 16 rows and a transposed read's four rows and
    // four pieces on disjoint banks at the 68-bank stride.  (The dV sweep has
    // no registers left for the swizzle's terms: 5 to 12 spilled.)
    constexpr bool CSWZ = MODE == 1 && !PREP;
    _Float16* Ch = reinterpret_cast<_Float16*>(smem + LY::CH) + par * (C * LDCH);
    _Float16* Xh = reinterpret_cast<_Float16*>(smem + LY::XH) + par * (C * LDC);
    _Float16* Ah = reinterpret_cast<_Float16*>(smem + LY::AH) + par * (C * LDA);
    _Float16* Al = reinterpret_cast<_Float16*>(smem + LY::AL) + par * (C * LDA);
    float* cl_s = reinterpret_cast<float*>(smem + LY::ROW) + par * (4 * C);
    int* ec_s = reinterpret_cast<int*>(cl_s + C);
    int* ex_s = ec_s + C;
    int* ea_s = ex_s + C;
    // ---------------- stage: fp16 rows with their power-of-two scales ----------
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
      Row8 c;
      if constexpr (MODE == 0) c.from_bf16(pc[i][0]);
      else c.from_f32(pc[i][0], pc[i][1]);
      const int e2 = scale_exp(row16_max(c.amax()));
      *reinterpret_cast<f16x8*>(Ch + row * LDCH + (CSWZ ? (((col >> 3) ^ ((row & 3) << 2)) << 3) : col)) = c.scaled(e2);
      if ((tid & 15) == 0) ec_s[row] = e2;
      if constexpr (!PREP) {
        Row8 x;
        x.from_bf16(px8[i]);
        const int e3 = scale_exp(row16_max(x.amax()));
        *reinterpret_cast<f16x8*>(Xh + row * LDC + col) = x.scaled(e3);
        if ((tid & 15) == 0) ex_s[row] = e3;
      }
    }
    {
      const int row = tid >> 3, col = (tid & 7) * 8;
      Row8 av;
      if constexpr (MODE == 0) av.from_f32(pa[0], pa[1]);
      else av.from_bf16(pa[0]);
      const int e2 = scale_exp(row8_max(av.amax()));
      const f16x8 h = av.scaled(e2);
      *reinterpret_cast<f16x8*>(Ah + row * LDA + col) = h;
      if constexpr (MODE == 0 && !PREP) *reinterpret_cast<f16x8*>(Al + row * LDA + col) = av.residual(e2, h);
      if ((tid & 7) == 0) ea_s[row] = e2;
      if constexpr (INTRA) {
        Row8 vv;
        vv.from_bf16(pv8);
        const int e4 = scale_exp(row8_max(vv.amax()));
        *reinterpret_cast<f16x8*>(Vh + row * LDA + col) = vv.scaled(e4);
        if ((tid & 7) == 0) ev_s[row] = e4;
      }
    }
    if (tid * 2 < C * L) {
      lam_s[tid * 2] = plam[0];
      lam_s[tid * 2 + 1] = plam[1];
    }
    const float cl2 = wave_prefix_sum(pla) * kLog2e;  // lane = token
    const float A2 = uniform(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl2), 63)));
    if (w == 0) cl_s[lane] = cl2;
    if constexpr (VDV) {
      if (vdv && n + 1 < n1) load_vdv(n + 1);
    }
    __syncthreads();

    // ---------------- chunk n + 1: add the partner's partial sums, store ---------
    if (!PREP && n + 1 < n1) {
      const int partner = w ^ 4;
      const f32x4 x0 = Xc[(partner * 2 + 0) * 64 + lane];
      const f32x4 x1 = Xc[(partner * 2 + 1) * 64 + lane];
      const int tp = tok0 + C;
      float f0[4], f1[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t0 = tp + 16 * own0 + 4 * g4 + r;
        const int t1 = tp + 16 * own1 + 4 * g4 + r;
        f0[r] = O0[r] + x0[r];
        f1[r] = O1[r] + x1[r];
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f0[r]), yr, (t0 * DC + col0 + c0 + li) * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f1[r]), yr, (t1 * DC + col0 + c0 + li) * 4, 0, 0);
      }
      if constexpr (INTRA) {
        if (intra) flush_intra(n + 1);
      }
      if constexpr (VDV) {
        if (vdv) {
          vdv_rows(n + 1, f0, f1);
          if (n + 2 < n1) flush_vdv(n + 2);
        }
      }
    }
    if (n > n0) prefetch(n - 1);

    // ---------------- phase 1 ---------------------------------------------------
    if constexpr (!PREP) {
      // masked score tiles (sb, tb), tb >= sb: waves 0..3 (w, w); waves 4..7
      // (0,1) (0,2) (1,2) (0,3); waves 0 and 1 also (1,3) and (2,3)
      const int ntile = w < 2 ? 2 : 1;
      int sbt[2], tbt[2];
      if (w < 4) { sbt[0] = w; tbt[0] = w; }
      else if (w == 4) { sbt[0] = 0; tbt[0] = 1; }
      else if (w == 5) { sbt[0] = 0; tbt[0] = 2; }
      else if (w == 6) { sbt[0] = 1; tbt[0] = 2; }
      else { sbt[0] = 0; tbt[0] = 3; }
      sbt[1] = w == 0 ? 1 : 2;
      tbt[1] = 3;
      f32x4 acc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int it = 0; it < 2; ++it)
          if (it < ntile) {
            const int swr = CSWZ ? (li & 3) << 2 : 0;  // (row & 3) << 2
            const f16x8 ca = *reinterpret_cast<const f16x8*>(
                Ch + (16 * tbt[it] + li) * LDCH + (CSWZ ? ((4 * ks + g4) ^ swr) << 3 : 32 * ks + 8 * g4));
            const f16x8 xb = *reinterpret_cast<const f16x8*>(Xh + (16 * sbt[it] + li) * LDC + 32 * ks + 8 * g4);
            acc[it] = mma32(ca, xb, acc[it]);  // acc[r] = c_t . x_s, s = 16 sb + li, t = 16 tb + 4 g4 + r (scaled)
          }
#pragma unroll
      for (int it = 0; it < 2; ++it)
        if (it < ntile) {
          const int sb = sbt[it], tb = tbt[it];
          const int si = 16 * sb + li;
          // P[t,s] 2^ea_t: the score, its two row scales, lambda and the decay
          const float sfac = static_cast<float>(ex_s[si]) - cl_s[si];
          const f32x4 clt = *reinterpret_cast<const f32x4*>(cl_s + 16 * tb + 4 * g4);
          const i32x4 ect = *reinterpret_cast<const i32x4*>(ec_s + 16 * tb + 4 * g4);
          const i32x4 eat = *reinterpret_cast<const i32x4*>(ea_s + 16 * tb + 4 * g4);
          float pv[4], ev[4];
          float mx = 0.f;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int ti = 16 * tb + 4 * g4 + r;
            const float ex = clt[r] + sfac + static_cast<float>(ect[r] + eat[r]);
            const float lam = tb > sb ? lam_s[ti * L + 4 + (32 - __clz(sb ^ tb))] : lam_s[ti * L + dlev[r]];
            ev[r] = acc[it][r] * __builtin_amdgcn_exp2f(ex);  // the pair's weight before lambda, times 2^ea_t
            const float x = ev[r] * lam;
            pv[r] = (tb > sb || ((dmask >> r) & 1)) ? x : 0.f;
            mx = fmaxf(mx, fabsf(pv[r]));
          }
          if constexpr (INTRA) {
            if (intra) {
              // in-chunk dlambda over this group's columns:
              //   D[t,s] = (dO_t . v_s)(q_t . k_s) exp(cum_t - cum_s)
              // dO_t . v_s from the fp16 hi + lo dO rows and the scaled v rows
              // (the diagonal terms cancel in the decay gradient, so they
              // keep ~2^-20); rows summed over s per level
              f32x4 s1 = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
              for (int ks = 0; ks < 2; ++ks) {
                const f16x8 vb = *reinterpret_cast<const f16x8*>(Vh + (16 * sb + li) * LDA + 32 * ks + 8 * g4);
                const f16x8 ah = *reinterpret_cast<const f16x8*>(Ah + (16 * tb + li) * LDA + 32 * ks + 8 * g4);
                const f16x8 al = *reinterpret_cast<const f16x8*>(Al + (16 * tb + li) * LDA + 32 * ks + 8 * g4);
                s1 = mma32(ah, vb, s1);
                s1 = mma32(al, vb, s1);
              }
              const float evs = ldexp_(1.f, ev_s[si]);
              float d[4];
#pragma unroll
              for (int r = 0; r < 4; ++r) d[r] = (tb > sb || ((dmask >> r) & 1)) ? (s1[r] * evs) * ev[r] : 0.f;
              float* slot = isl + par * (C * 8) + (16 * tb + 4 * g4 + (li >> 2)) * 8;
              const bool writer = (li & 3) == 0;
              if (tb > sb) {
                const float z = rowsum16(d, li);
                if (writer) slot[5 + sb] = z;
              } else {
#pragma unroll
                for (int lv = 0; lv <= 4; ++lv) {
                  float x[4];
#pragma unroll
                  for (int r = 0; r < 4; ++r) x[r] = dlev[r] == lv ? d[r] : 0.f;
                  const float z = rowsum16(x, li);
                  if (writer) slot[lv] = z;
                }
              }
            }
          }
          // fp16 hi + lo: the in-chunk terms carry the diagonal ones, which
          // cancel in the decay gradient (dO_t . O_t - v_t . dV_t)
          const int pe = scale_exp(wave_max(mx));
          f16x4 h, l;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = ldexp_(pv[r], -pe);
            h[r] = static_cast<_Float16>(x);
            l[r] = static_cast<_Float16>(x - static_cast<float>(h[r]));
          }
          Ps[(sb * 4 + tb) * 64 + lane] = h;
          Ps[1024 + (sb * 4 + tb) * 64 + lane] = l;
          if (lane == 0) ke_s[16 + sb * 4 + tb] = pe;
        }
      // left-read row factor (lane = row s): exp(cum at the end of the chunk
      // - cum_s) 2^ex_s
      if (w == 7) rf_s[lane] = __builtin_amdgcn_exp2f(A2 - cl2 + static_cast<float>(ex_s[lane]));
    }
    // level-update token weights (lane = t): wave b forms level b's
    //   lambda[t, lvl] exp(cum_t - cum at the end of chunk n - 1) 2^(ec_t + ea_t)
    // in units of the state's new exponent kn (fp16, below 1): kn is the
    // chunk's own exponent k (maximum in [1/2, 1)) or, if larger, that of the
    // decayed state, so the state never grows by more than a factor 2 per chunk
    {
      const bool act = w < nlev && (PREP ? ((seg >> w) & 1) : ((n >> w) & 1));
      if (act) {
        const int lvl = PREP ? LOGC + 1 + S + w : LOGC + 1 + w;
        const float raw = lam_s[lane * L + lvl] *
                          __builtin_amdgcn_exp2f(cl2 + static_cast<float>(ec_s[lane] + ea_s[lane]));
        const int kc = scale_exp(wave_max(fabsf(raw))) + 15;
        int krw = kr[0];
#pragma unroll
        for (int b = 1; b < NL; ++b)
          if (w == b) krw = kr[b];
        const int base = (n >> (w + 1)) << (w + 1);
        const bool first = PREP ? n == n1 - 1 : n == min(n1, base + (2 << w)) - 1;
        const int kn = first ? kc : max(kc, krw + static_cast<int>(floorf(fmaxf(A2, -1.0e4f))));
        WT[w * C + lane] = static_cast<_Float16>(ldexp_(raw, -kn));
        if (lane == 0) ke_s[w] = kn;
      }
    }
    __syncthreads();

    // ---------------- phase 2 ------------------------------------------------------
    if constexpr (!PREP) {
      // left reads over this wave's contraction half, all four row tiles:
      // Op[mi] = sum_b u_b x_h . R_b, times the row factor
      float ub[NL + 1];
      bool live[NL + 1];
#pragma unroll
      for (int b = 0; b < NL; ++b) {
        const int base = (n >> (b + 1)) << (b + 1);
        live[b] = b < S && !((n >> b) & 1) && base + (1 << b) < n1;
        ub[b] = __builtin_amdgcn_exp2f(g2[b] + static_cast<float>(er[b]));
      }
      live[NL] = has_suffix;
      ub[NL] = __builtin_amdgcn_exp2f(dn2 + static_cast<float>(eh));
      f32x4 Op[4];
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        Op[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
        const f16x8 xa0 = *reinterpret_cast<const f16x8*>(Xh + (16 * mi + li) * LDC + 64 * hh + 8 * g4);
        const f16x8 xa1 = *reinterpret_cast<const f16x8*>(Xh + (16 * mi + li) * LDC + 64 * hh + 32 + 8 * g4);
#pragma unroll
        for (int b = 0; b <= NL; ++b) {
          if (live[b]) {
            const f16x8 gr0 = b < NL ? __builtin_bit_cast(f16x8, R[b][0]) : Rh[0];
            const f16x8 gr1 = b < NL ? __builtin_bit_cast(f16x8, R[b][1]) : Rh[1];
            f32x4 acc = mma32(xa0, gr0, f32x4{0.f, 0.f, 0.f, 0.f});
            acc = mma32(xa1, gr1, acc);
#pragma unroll
            for (int r = 0; r < 4; ++r) Op[mi][r] += ub[b] * acc[r];
          }
        }
        const f32x4 rf = *reinterpret_cast<const f32x4*>(rf_s + 16 * mi + 4 * g4);
#pragma unroll
        for (int r = 0; r < 4; ++r) Op[mi][r] *= rf[r];
      }
      Xc[(w * 2 + 0) * 64 + lane] = Op[oth0];
      Xc[(w * 2 + 1) * 64 + lane] = Op[oth1];
      // in-chunk part for this wave's two row tiles: y_s += sum_{t >= s} P[t,s] a_t,
      // 16 x 16 x 16 products per score tile, each tile with its own scale:
      // P_hi a_hi + P_lo a_hi (+ P_hi a_lo for fp32 a)
      O0 = Op[own0];
      O1 = Op[own1];
#pragma unroll
      for (int tb = 0; tb < 4; ++tb) {
        if (tb >= own0 || tb >= own1) {
          const int ao = (16 * tb + 4 * g4 + (li >> 2)) * LDA + c0 + 4 * (li & 3);
          const f16x4 ab = tr_read(Ah + ao);
          f16x4 al = f16x4{};
          if constexpr (MODE == 0) al = tr_read(Al + ao);
#pragma unroll
          for (int o = 0; o < 2; ++o) {
            const int own = o ? own1 : own0;
            if (tb >= own) {
              const f16x4 ph = Ps[(own * 4 + tb) * 64 + lane], pl = Ps[1024 + (own * 4 + tb) * 64 + lane];
              f32x4 acc = mma16(ph, ab, f32x4{0.f, 0.f, 0.f, 0.f});
              acc = mma16(pl, ab, acc);
              if constexpr (MODE == 0) acc = mma16(ph, al, acc);
              const int pe = ke_s[16 + own * 4 + tb];
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                if (o) O1[r] += ldexp_(acc[r], pe);
                else O0[r] += ldexp_(acc[r], pe);
              }
            }
          }
        }
      }
    }
    // level updates: R_b = exp(A_n) R_b + c^T (w_b a), in the chunk-state
    // fold's layout; the state's exponent follows the larger of the decayed
    // state and the chunk
#pragma unroll
    for (int b = 0; b < NL; ++b) {
      const bool upd = b < nlev && (PREP ? ((seg >> b) & 1) : ((n >> b) & 1));
      if (upd) {
        const int base = (n >> (b + 1)) << (b + 1);
        const bool first = PREP ? n == n1 - 1 : n == min(n1, base + (2 << b)) - 1;
        const int kn = uniform_i(ke_s[b]);
        // the first chunk of the right half starts the state: the register
        // contents are finite (fp32 or packed finite fp16), so a factor 0 clears them
        const float f = first ? 0.f : __builtin_amdgcn_exp2f(A2 + static_cast<float>(kr[b] - kn));
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) R[b][t][r] *= f;
        kr[b] = kn;
        f16x8 va[2];
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const _Float16* a0 = Ah + (32 * ks + 8 * g4 + (li >> 2)) * LDA + c0 + 4 * (li & 3);
          va[ks] = cat(tr_read(a0), tr_read(a0 + 4 * LDA)) *
                   *reinterpret_cast<const f16x8*>(WT + b * C + 32 * ks + 8 * g4);
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int kq = 2 * hh + (t >> 1), half = t & 1;
            const int cpc = 4 * kq + (li & 3);  // 16-byte piece of the row
            const int swt = CSWZ ? ((li >> 2) & 3) << 2 : 0;  // (row & 3) << 2
            const _Float16* k0 = Ch + (32 * ks + 8 * g4 + (li >> 2)) * LDCH + ((cpc ^ swt) << 3) + 4 * half;
            const f16x8 ca = cat(tr_read(k0), tr_read(k0 + 4 * LDCH));
            R[b][t] = mma32(ca, va[ks], R[b][t]);
          }
        // the right half's lowest chunk: from the next chunk on, the left
        // half reads the state; pack it as fp16
        if (!PREP && n == base + (1 << b)) {
          float mx = 0.f;
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(R[b][t][r]));
          const int em = scale_exp(wave_max(mx));
          f16x8 gn[2];
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) gn[t >> 1][4 * (t & 1) + r] = static_cast<_Float16>(ldexp_(R[b][t][r], -em));
          R[b][0] = __builtin_bit_cast(f32x4, gn[0]);
          R[b][1] = __builtin_bit_cast(f32x4, gn[1]);
          er[b] = uniform_i(em + kr[b]);
          g2[b] = 0.f;
        }
      } else if (!PREP && b < nlev) {
        g2[b] = uniform(g2[b] + A2);
      }
    }
    dn2 = uniform(dn2 + A2);
    tot2 += A2;
  }

  if constexpr (PREP) {
    // P[seg, j][column][contraction] = R_j 2^kr_j
#pragma unroll
    for (int b = 0; b < NL; ++b) {
      if (b < nlev && ((seg >> b) & 1)) {
        float* dst = a.seg_part + (((size_t)(bh * a.nseg + seg) * a.nj + b) * DC + col0 + c0 + li) * DC + 64 * hh +
                     8 * g4;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f32x4 y;
#pragma unroll
          for (int r = 0; r < 4; ++r) y[r] = ldexp_(R[b][t][r], kr[b]);
          *reinterpret_cast<f32x4*>(dst + 32 * (t >> 1) + 4 * (t & 1)) = y;
        }
      }
    }
    if (tid == 0 && dg == 0) a.seg_tot2[bh * a.nseg + seg] = tot2;
  } else {
    // ---------------- first chunk of the segment: partner sums, store -------------
    if constexpr (VDV) {
      if (vdv) load_vdv(n0);
    }
    __syncthreads();
    const int partner = w ^ 4;
    const f32x4 x0 = Xc[(partner * 2 + 0) * 64 + lane];
    const f32x4 x1 = Xc[(partner * 2 + 1) * 64 + lane];
    const int tp = n0 * C;
    float f0[4], f1[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t0 = tp + 16 * own0 + 4 * g4 + r;
      const int t1 = tp + 16 * own1 + 4 * g4 + r;
      f0[r] = O0[r] + x0[r];
      f1[r] = O1[r] + x1[r];
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f0[r]), yr, (t0 * DC + col0 + c0 + li) * 4, 0, 0);
      __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(f1[r]), yr, (t1 * DC + col0 + c0 + li) * 4, 0, 0);
    }
    if constexpr (INTRA) {
      if (intra) flush_intra(n0);
    }
    if constexpr (VDV) {
      if (vdv) {
        vdv_rows(n0, f0, f1);
        if (n0 + 1 < n1) flush_vdv(n0 + 1);
        __syncthreads();
        flush_vdv(n0);
      }
    }
  }
}

template <int MODE>
__global__ void __launch_bounds__(512) bwd_rev_kernel(BwdRevArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  rev_body<MODE, false, rv::NLEV>(a, smem);
}
// the pre-pass; with NL = NL_SMALL register levels it fits two workgroups per CU
template <int NL>
__global__ void __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(NL <= rv::NL_SMALL ? 4 : 2)))
bwd_rev_prep_kernel(BwdRevArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  rev_body<0, true, NL>(a, smem);
}

void bwd_rev_plan(int T, BwdRevPlan* p) {
  const int N = (T + rv::C - 1) / rv::C;
  const int nslot = N > 1 ? 32 - __builtin_clz(static_cast<unsigned>(N - 1)) : 0;
  p->seg_log2 = std::min(nslot, rv::NLEV);
  p->nseg = (N + (1 << p->seg_log2) - 1) >> p->seg_log2;
  p->nj = p->nseg > 1 ? 32 - __builtin_clz(static_cast<unsigned>(p->nseg - 1)) : 0;
}

bool bwd_rev_ok(int C, int dk, int dv, int G, int T, int L) {
  if (C != rv::C || dk != rv::DC || dv != rv::DC || G != 1 || T < 1 || L > rv::LMAX) return false;
  BwdRevPlan p;
  bwd_rev_plan(T, &p);
  return p.nj <= rv::NLEV && (long long)T * rv::DC * 4 < 0x7fffffffLL;
}

size_t bwd_rev_workspace(int BH, int T) {
  BwdRevPlan p;
  bwd_rev_plan(T, &p);
  if (p.nseg <= 1) return 0;
  return (size_t)BH * p.nseg * p.nj * rv::DC * rv::DC * 4 + (size_t)BH * p.nseg * 4;
}

template <typename K>
static int launch_grid(K kernel, std::atomic<uint64_t>& raised, int bytes, const BwdRevArgs& a, hipStream_t stream) {
  if (!raise_lds_limit(reinterpret_cast<const void*>(kernel), raised)) return LL_ERR_HIP;
  const long long pairs = (long long)a.BH * a.nseg;
  const long long nblocks = (pairs + 7) / 8 * 8 * 2;
  if (nblocks <= 0) return LL_OK;
  if (nblocks > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(kernel, dim3(static_cast<unsigned>(nblocks)), dim3(rv::NTH), bytes, stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int launch_bwd_rev(const BwdRevArgs& a, hipStream_t stream) {
  if (a.L > rv::LMAX || a.seg_log2 < 0 || a.seg_log2 > rv::NLEV || a.nj > rv::NLEV) return LL_ERR_UNSUPPORTED;
  if (a.nseg > 1 && (!a.seg_part || !a.seg_tot2)) return LL_ERR_UNSUPPORTED;
  static std::atomic<uint64_t> r0{0}, r1{0}, r2{0}, r3{0};
  int st = LL_OK;
  if (a.nseg > 1) {
    if (a.nj <= rv::NL_SMALL)
      st = launch_grid(&bwd_rev_prep_kernel<rv::NL_SMALL>, r0, rv::Lay<true>::BYTES, a, stream);
    else
      st = launch_grid(&bwd_rev_prep_kernel<rv::NLEV>, r1, rv::Lay<true>::BYTES, a, stream);
  }
  if (st == LL_OK) st = launch_grid(&bwd_rev_kernel<0>, r2, rv::Lay<false>::BYTES, a, stream);
  if (st == LL_OK) st = launch_grid(&bwd_rev_kernel<1>, r3, rv::Lay<false>::BYTES, a, stream);
  return st;
}

}  // namespace ll
