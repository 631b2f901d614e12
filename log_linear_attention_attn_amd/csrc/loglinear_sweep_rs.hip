// Register-resident chunk sweep for the bf16 forward with C = 64, dk <= 128 and
// dv a multiple of 64 (the log-linear Mamba-2 shapes).  Same decomposition as
// fwd_sweep_kernel (loglinear_fwd.hip): per (b,h, segment) the chunks are
// walked in order and the chunk-granular Fenwick bucket states are merged with
// the lssb rule ([P1] 解码：基于 lssb 的状态更新, applied to whole chunks;
// [P1] 训练：分块并行扫描算法 for the split into intra / inter chunk work).
//
//   [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
//
// Work split of one 512-thread workgroup = (b,h, segment, 64 dv columns),
// eight waves, two per SIMD:
//   phase 1  the 10 causal 16x16 score tiles of the chunk are shared out over
//            the waves; each masked tile P (Fenwick level x decay x lambda)
//            is split bf16 hi/lo and parked in LDS in MFMA A-operand order.
//   phase 2  wave w owns dv columns 16(w&3)..+15 and dk half w>>2: the
//            partial Q G_b products of its dk half for all 64 rows, P V for
//            two of the four 16-row tiles, the chunk state K^T (V*decay) of
//            its dk half and the lssb merge.  The two dk halves of a column
//            slice add their partial outputs through LDS.  The bucket states
//            G_b (64 dk x 16 columns per wave) never leave the registers;
//            they are held in fp16 with a power-of-two scale per (level,
//            wave), and the Q.G products run as fp16 MFMAs on a scaled fp16
//            copy of Q (bf16 values are exact in fp16 once scaled into
//            range).  Error ~3e-3 of the output RMS with no decay (bf16 hi/lo
//            states in the LDS-state kernel: ~1e-4).
// K, Q and V are staged row-major; the operands that contract over tokens are
// read with the LDS transpose load (ds_read_b64_tr_b16), so no transposed
// stores are needed.  The next chunk's global loads are issued before the
// current chunk's math (register prefetch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

namespace rs {

constexpr int C = 64, DKP = 128, NKS = DKP / 32, LOGC = 6;
constexpr int LDQ = DKP + 8;  // Qs, Ks row stride (bf16)
constexpr int LDV = 64 + 8;   // Vs row stride (bf16): 64 dv columns
// LDS layout of the sweep.  K, V and the in-chunk decay sums are double
// buffered by chunk parity (they are read until the end of a chunk, while the
// next chunk is staged); everything else is single.
constexpr int QS_OFF = 0;                        // Q tile, bf16 [64][LDQ]
constexpr int KS_OFF = QS_OFF + C * LDQ * 2;     // K tiles, bf16 [2][64][LDQ]
constexpr int VS_OFF = KS_OFF + 2 * C * LDQ * 2; // V tiles, bf16 [2][64][LDV]
constexpr int PS_OFF = VS_OFF + 2 * C * LDV * 2; // masked scores, hi/lo A fragments
constexpr int PS_BYTES = 4 /*mi*/ * 2 /*ks*/ * 2 /*hi,lo*/ * 64 * 16;
constexpr int XC_OFF = PS_OFF + PS_BYTES;        // partial outputs [8 waves][2][64 lanes] f32x4
constexpr int XC_BYTES = 8 * 2 * 64 * 16;
constexpr int CL_OFF = XC_OFF + XC_BYTES;        // [2] x (cl[64], esf[64]) fp32
constexpr int QM_OFF = CL_OFF + 2 * 2 * C * 4;   // per-wave max |q| [8] (padded to 64 B)
constexpr int QH_OFF = QM_OFF + 64;              // fp16 copy of Q, [64][LDQ]
constexpr int LW_OFF = QH_OFF + C * LDQ * 2;     // per-wave Q.G row weights [8][NSLOT levels][64]
// lambda of the chunk [64][L] (+ 16 words of slack) follows the row weights
__host__ __device__ constexpr int lam_off(int nsl) { return LW_OFF + 8 * nsl * C * 4; }
// register slots of a kernel instantiation for nslot chunk-level bits
__host__ __device__ constexpr int nsl_for(int nslot) { return nslot <= 8 ? 8 : 10; }

// Rows past T of a ragged last chunk look up levels up to log2(C), and the
// row weights read all inter-chunk levels of the instantiation, which a short
// sequence's lambda may lack; the slack keeps those (discarded) reads in bounds.
__host__ __device__ inline int lds_bytes(int L, int nslot) { return lam_off(nsl_for(nslot)) + (C * L + 16) * 4; }
// Backward variant (dQ as the forward of (dO, v, k), with the chunk-level
// dlambda): the forward's q tile [64][LDQO] bf16 follows lambda; the row
// weight region holds the per-wave dlambda partials [8][64 rows][slots].
constexpr int LDQO = 64 + 8;
__host__ __device__ inline int qo_off(int L, int nslot) { return (lds_bytes(L, nslot) + 15) & ~15; }
__host__ __device__ inline int lds_bytes_dlam(int L, int nslot) { return qo_off(L, nslot) + C * LDQO * 2 + C * 4; }

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef _Float16 __attribute__((ext_vector_type(4))) f16x4;
typedef unsigned short __attribute__((ext_vector_type(2))) u16x2;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed 8-byte LDS read: within each 16-lane group, lane i receives
// element (i & 3) of the 4-element vectors addressed by lanes 4k + (i >> 2),
// k = 0..3.
__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<__attribute__((address_space(3))) char*>(
          reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(bf16x4, v);
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma16(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Maxima of NON-NEGATIVE floats: their bit patterns order like the values,
// so unsigned max (which folds into the DPP form of v_max_u32) serves.
template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  const unsigned u = __float_as_uint(x);
  return __uint_as_float(max(u, static_cast<unsigned>(__builtin_amdgcn_update_dpp(0, static_cast<int>(u), CTRL, 0xf, 0xf, false))));
}
// Max over the 64 lanes of a NON-NEGATIVE value, returned wave-uniform: DPP
// swaps within quads and rotations within 16-lane rows, then the four row
// maxima compared as integers.
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max<0xb1>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4e>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x124>(x);  // row_ror:4
  x = dpp_max<0x128>(x);  // row_ror:8
  const int xi = __float_as_int(x);
  const unsigned a0 = __builtin_amdgcn_readlane(xi, 0), a1 = __builtin_amdgcn_readlane(xi, 16);
  const unsigned a2 = __builtin_amdgcn_readlane(xi, 32), a3 = __builtin_amdgcn_readlane(xi, 48);
  return __uint_as_float(max(max(a0, a1), max(a2, a3)));
}

// Two-term bf16 split with a truncated high part: hi = the top 16 bits of x,
// lo = x - hi rounded to bf16.  |x - hi| < 2^-7 |x|, so |x - hi - lo| <=
// 2^-16 |x|, the bound of the round-to-nearest split, at fewer instructions.
__device__ __forceinline__ void split_bf16_t(float x, bf16& hi, bf16& lo) {
  const unsigned u = __float_as_uint(x);
  hi = __builtin_bit_cast(bf16, static_cast<unsigned short>(u >> 16));
  lo = static_cast<bf16>(x - __uint_as_float(u & 0xffff0000u));
}

// Inclusive prefix sum over the 64 lanes of a wave: shifts within each
// 16-lane row, then the row totals carried across rows by the row broadcasts
// of lanes 15 and 31 (DPP).  Lanes without a source add zero.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ float wave_prefix_sum(float x) {
  x = dpp_add<0x111, 0xf>(x);  // row_shr:1
  x = dpp_add<0x112, 0xf>(x);  // row_shr:2
  x = dpp_add<0x114, 0xf>(x);  // row_shr:4
  x = dpp_add<0x118, 0xf>(x);  // row_shr:8
  x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return x;
}

// Power-of-two scale exponent e such that mx * 2^-e lies in [2^14, 2^15)
// (fp16 holds up to 65504); 0 for mx == 0, clamped so 2^+-e stays a normal float.
__device__ __forceinline__ int scale_exp(float mx) {
  if (!(mx > 0.f)) return 0;
  const int e = static_cast<int>((__float_as_uint(mx) >> 23) & 0xff) - 127 - 14;
  return max(-110, min(110, e));
}

constexpr float kLog2e = 1.4426950408889634f;
// 2^x on the transcendental unit (v_exp_f32)
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// A wave-uniform float kept in a scalar register (readfirstlane), so per-level
// bookkeeping does not occupy vector registers.
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ float exp2_int(int e) { return __uint_as_float(static_cast<unsigned>(e + 127) << 23); }

// Raw buffer resource over [base, base + bytes): loads beyond the range return
// zero and stores beyond it are dropped, so ragged tails need no branches and
// the addresses stay 32-bit offsets from a wave-uniform base.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every range used here
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ bf16x8 load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
typedef unsigned int __attribute__((ext_vector_type(4))) u32x4;
// x + x of the lane 16 (resp. 32) apart, in every lane, through the gfx950
// row-pair swaps (v_permlane16_swap / v_permlane32_swap with both operands x:
// the two results hold the lane's own half and the partner half, lane layout
// checked by an on-GPU probe)
__device__ __forceinline__ float xor16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// four consecutive fp32 outputs as one 16-byte store (dropped past the range)
__device__ __forceinline__ void store_row(rsrc_t r, f32x4 x, uint32_t off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, off, 0, 0);
}

}  // namespace rs

// Eight waves per workgroup (two per SIMD): wave w owns dv columns
// 16*(w&3)..+15 of the workgroup's 64 and dk half h = w>>2 of the bucket
// states.  The two dk halves of a column slice add their partial Q.G sums
// through LDS; each wave finishes the output of two row tiles.
// EMIT: also write the prefill decode states (a separate instantiation, so the
// plain forward does not carry the extra live registers).
// DLAM: the backward's dQ sweep.  The kernel then runs on (q, k, v) = (dO in
// fp32, v, k) of the forward, so `out` is dQ, and it also forms the
// chunk-level dlambda: dlambda[t, log2C+1+b] = q_t . (level-b read of row t),
// the read being exactly the per-level product this sweep computes for dQ
// before its lambda weight.  Its products are taken transposed (lane = row,
// four consecutive columns), so the dot of a row's read with the forward's q
// over a wave's 16 columns is four products per lane and two row-pair swaps;
// the eight waves' partials are summed through LDS after the next barrier and
// written per 64-column group.
template <int NSLOT, bool EMIT, bool DLAM = false>
__global__ void __launch_bounds__(512)
fwd_rs_kernel(FwdArgs a) {
  using namespace rs;
  constexpr int NTH = 512;
  extern __shared__ __align__(16) unsigned char smem[];
  bf16* Qs = reinterpret_cast<bf16*>(smem + QS_OFF);
  _Float16* Qh = reinterpret_cast<_Float16*>(smem + QH_OFF);
  bf16x8* Ps = reinterpret_cast<bf16x8*>(smem + PS_OFF);  // [mi][ks][hl][lane]
  f32x4* Xc = reinterpret_cast<f32x4*>(smem + XC_OFF);    // [wave][2][lane]
  float* qmax_s = reinterpret_cast<float*>(smem + QM_OFF);
  float* lam_s = reinterpret_cast<float*>(smem + lam_off(NSLOT));
  _Float16* Qo = reinterpret_cast<_Float16*>(smem + ((lam_off(NSLOT) + (C * a.L + 16) * 4 + 15) & ~15));  // DLAM only
  int* er_s = reinterpret_cast<int*>(Qo + C * LDQO);  // DLAM: per-row fp16 scale exponent of q

  const int D = a.dv >> 6;  // 64-column groups
  const int id = blockIdx.x;
  const int px = id & 7, rest = id >> 3;
  const int dg = rest % D, pg = rest / D;
  const int p = pg * 8 + px;
  if (p >= a.BH * a.nseg) return;
  const int bh = p / a.nseg, seg = p - bh * a.nseg;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int cs = w & 3, hh = w >> 2;  // column slice, dk half
  const int c0 = 16 * cs;
  const int T = a.T, L = a.L, dk = a.dk, dv = a.dv;
  const int N = (T + C - 1) / C;
  const int n0 = seg << a.seg_log2;
  const int n1 = min(N, n0 + (1 << a.seg_log2));
  const int dv0 = dg * 64;
  const size_t bhT = (size_t)bh * T;
  // per-(b,h) slices; every slice is < 2^31 bytes (checked by the launcher)
  const size_t qkT = (size_t)(bh / a.G) * T;
  // DLAM: "q" is dO in fp32
  const rsrc_t qr = DLAM ? make_rsrc(static_cast<const float*>(a.q) + qkT * dk, T * dk * 4)
                         : make_rsrc(static_cast<const bf16*>(a.q) + qkT * dk, T * dk * 2);
  const rsrc_t kr = make_rsrc(static_cast<const bf16*>(a.k) + qkT * dk, T * dk * 2);
  const rsrc_t vr = make_rsrc(static_cast<const bf16*>(a.v) + bhT * dv, T * dv * 2);
  const rsrc_t lar = make_rsrc(a.log_a + bhT, T * 4);
  const rsrc_t lamr = make_rsrc(a.lam + bhT * L, T * L * 4);
  const rsrc_t outr = make_rsrc(a.out + bhT * dv, T * dv * 4);
  const rsrc_t qor = DLAM ? make_rsrc(static_cast<const bf16*>(a.qo) + bhT * dv, T * dv * 2) : outr;
  // row tiles whose output this wave finishes, and the two it hands over
  const int own0 = hh ? 1 : 0, own1 = hh ? 2 : 3;
  const int oth0 = hh ? 0 : 1, oth1 = hh ? 3 : 2;

  // ---- bucket states: G[b][ks] holds dk 64*hh + 32ks + 8*g4 + e (e = 0..7)
  // of column c0 + li, fp16 with a per-(level, wave) power-of-two scale:
  // true value = stored * 2^eg[b].
  f16x8 G[NSLOT][2];
  int eg[NSLOT];
  float dec[NSLOT];  // log decay since each bucket state was formed
#pragma unroll
  for (int b = 0; b < NSLOT; ++b) {
    dec[b] = 0.f;
    eg[b] = 0;
    G[b][0] = f16x8{};
    G[b][1] = f16x8{};
  }
  // Levels spanning whole segments: bit b >= seg_log2 of n0 <-> bit
  // b - seg_log2 of the segment; its bucket is the node starting at segment
  // (seg >> b') << b'.
#pragma unroll
  for (int b = 0; b < NSLOT; ++b) {
    if (b >= a.seg_log2 && ((n0 >> b) & 1)) {
      const int bp = b - a.seg_log2;
      const int gc = (seg >> bp) << bp;
      const float* __restrict__ node =
          a.nodes + ((size_t)(bh * a.nseg + gc) * dv + dv0 + c0 + li) * DKP + 64 * hh + 8 * g4;
      f32x4 x[4];
      float mx = 0.f;
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        x[2 * ks] = *reinterpret_cast<const f32x4*>(node + 32 * ks);
        x[2 * ks + 1] = *reinterpret_cast<const f32x4*>(node + 32 * ks + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) mx = fmaxf(mx, fmaxf(fabsf(x[2 * ks][e]), fabsf(x[2 * ks + 1][e])));
      }
      const int e2 = scale_exp(wave_max(mx));
      const float sc = exp2_int(-e2);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          G[b][ks][e] = static_cast<_Float16>(x[2 * ks][e] * sc);
          G[b][ks][4 + e] = static_cast<_Float16>(x[2 * ks + 1][e] * sc);
        }
      eg[b] = e2;
      float d = 0.f;
      for (int r = gc; r < seg; ++r) d += a.seg_decay[bh * a.nseg + r];
      dec[b] = uniform(d);
    }
  }

  // ---- register prefetch of one chunk ----------------------------------
  bf16x8 pq[2], pk[2], pv, pqo;
  f32x4 pqf[2][2];  // DLAM: the fp32 q values of pq
  float plam[3];  // lambda words 2*tid, 2*tid+1 and, for L > 16, 1024+tid of the chunk
  float pla;
  // per-thread parts of the chunk loads' offsets; columns past dk (padded
  // head dim) get an out-of-range offset and read zero
  uint32_t off_qk[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
    off_qk[i] = static_cast<uint32_t>((row * dk + col) * 2) | (col < dk ? 0u : kOutOfRange);
  }
  const uint32_t off_v = static_cast<uint32_t>(((tid >> 3) * dv + dv0 + (tid & 7) * 8) * 2);
  auto prefetch = [&](int n) {
    const uint32_t tok0 = static_cast<uint32_t>(n * C);
    // small loads first: vmcnt counts in order, so a later wait for one of
    // these does not also wait for the large q / k / v loads.  Lambda words
    // past C * L belong to the next chunk and are not staged.
    {
      const auto x = __builtin_amdgcn_raw_buffer_load_b64(lamr, (tok0 * L + 2 * tid) * 4, 0, 0);
      plam[0] = __uint_as_float(x[0]);
      plam[1] = __uint_as_float(x[1]);
      if (NSLOT > 8) plam[2] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lamr, (tok0 * L + 1024 + tid) * 4, 0, 0));
    }
    pla = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lar, (tok0 + lane) * 4, 0, 0));
    const uint32_t cq = tok0 * dk * 2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (DLAM) {
        const uint32_t o = off_qk[i] & kOutOfRange ? kOutOfRange : 2 * (off_qk[i] + cq);
#pragma unroll
        for (int h = 0; h < 2; ++h)
          pqf[i][h] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(qr, o + 16 * h, 0, 0));
      } else {
        pq[i] = load_b128(qr, off_qk[i] + cq);
      }
      pk[i] = load_b128(kr, off_qk[i] + cq);
    }
    pv = load_b128(vr, off_v + tok0 * dv * 2);
    if constexpr (DLAM) pqo = load_b128(qor, off_v + tok0 * dv * 2);
  };

  prefetch(n0);

  // level and causal mask of the diagonal score tiles (query 16qb + li,
  // key 16qb + 4g4 + r): functions of the in-block positions only
  int dlev[4];
  unsigned dmask = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    dlev[r] = level_of(li, 4 * g4 + r);
    dmask |= (4 * g4 + r <= li ? 1u : 0u) << r;
  }
  // DLAM: chunk nc's dlambda partials (written by the eight waves before the
  // last barrier) summed in wave order and stored for its live levels, zero
  // for the others; one thread per (row, slot), slots contiguous in memory
  auto dlam_flush = [&](int nc) {
    const float* dl = reinterpret_cast<const float*>(smem + LW_OFF);
    for (int e = tid; e < C * NSLOT; e += NTH) {
      const int row = e / NSLOT, b = e - row * NSLOT;
      const int t = nc * C + row;
      if (b >= a.nslot || t >= T) continue;
      float x = 0.f;
      if ((nc >> b) & 1) {
#pragma unroll
        for (int ww = 0; ww < 8; ++ww) x += dl[(ww * C + row) * NSLOT + b];
      }
      a.dlam_part[(((size_t)dg * a.BH + bh) * T + t) * a.nslot + b] = x;
    }
  };
  f32x4 O0, O1;      // this wave's two output row tiles, written after the next barrier
  float Aprev = 0.f;  // total log decay of the previous chunk
  float* lw = reinterpret_cast<float*>(smem + LW_OFF) + w * (NSLOT * C);  // this wave's row weights
  for (int n = n0; n < n1; ++n) {
    const int tok0 = n * C, par = n & 1;
    bf16* Ks = reinterpret_cast<bf16*>(smem + KS_OFF) + par * (C * LDQ);
    bf16* Vs = reinterpret_cast<bf16*>(smem + VS_OFF) + par * (C * LDV);
    float* cl_s = reinterpret_cast<float*>(smem + CL_OFF) + par * (2 * C);
    float* esf_s = cl_s + C;
    // ---------------- stage: registers -> LDS ------------------------------
    if constexpr (DLAM) {
      // the score tiles run in fp16: K goes to the bf16 Q tile's place as
      // fp16 (exact for bf16 values in range); q (fp32 dO) is scaled per row
      // by a power of two so the row's max |q| sits at 2^14..2^15 (the 16
      // lanes of a DPP row hold one row) and its exponent goes to er_s
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
        *reinterpret_cast<bf16x8*>(Ks + row * LDQ + col) = pk[i];
        f16x8 hk;
#pragma unroll
        for (int e = 0; e < 8; ++e) hk[e] = static_cast<_Float16>(static_cast<float>(pk[i][e]));
        *reinterpret_cast<f16x8*>(Qs + row * LDQ + col) = hk;
        float qf = 0.f;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int e = 0; e < 4; ++e) qf = fmaxf(qf, fabsf(pqf[i][h][e]));
        qf = dpp_max<0x121>(qf);  // row_ror:1, 2, 4, 8: the row's max in all 16 lanes
        qf = dpp_max<0x122>(qf);
        qf = dpp_max<0x124>(qf);
        qf = dpp_max<0x128>(qf);
        const int e2 = scale_exp(qf);
        const float sc = exp2_int(-e2);
        f16x8 hq;
#pragma unroll
        for (int e = 0; e < 8; ++e) hq[e] = static_cast<_Float16>(pqf[i][e >> 2][e & 3] * sc);
        *reinterpret_cast<f16x8*>(Qh + row * LDQ + col) = hq;
        if ((tid & 15) == 0) er_s[row] = e2;
      }
    } else {
      u16x2 qm = {0, 0};  // max |q| of this thread's values, as bf16 magnitude bits
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
        *reinterpret_cast<bf16x8*>(Qs + row * LDQ + col) = pq[i];
        *reinterpret_cast<bf16x8*>(Ks + row * LDQ + col) = pk[i];
        const uint4 bits = __builtin_bit_cast(uint4, pq[i]);
        qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.x & 0x7fff7fffu));
        qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.y & 0x7fff7fffu));
        qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.z & 0x7fff7fffu));
        qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.w & 0x7fff7fffu));
      }
      const unsigned m16 = max(static_cast<unsigned>(qm[0]), static_cast<unsigned>(qm[1]));
      const float qmw = wave_max(__uint_as_float(m16 << 16));
      if (lane == 0) qmax_s[w] = qmw;
    }
    *reinterpret_cast<bf16x8*>(Vs + (tid >> 3) * LDV + (tid & 7) * 8) = pv;
    if constexpr (DLAM) {  // the forward's q as fp16 (exact for bf16 values in range)
      f16x8 h;
#pragma unroll
      for (int e = 0; e < 8; ++e) h[e] = static_cast<_Float16>(static_cast<float>(pqo[e]));
      *reinterpret_cast<f16x8*>(Qo + (tid >> 3) * LDQO + (tid & 7) * 8) = h;
    }
    if (tid * 2 < C * L) {  // C * L is even
      lam_s[tid * 2] = plam[0];
      lam_s[tid * 2 + 1] = plam[1];
    }
    if (NSLOT > 8 && 1024 + tid < C * L) lam_s[1024 + tid] = plam[2];
    // in-chunk decay sums, every wave: cl = inclusive prefix of log_a (lane =
    // token); the decay from a token to the chunk's last token is Atot - cl
    const float cl = wave_prefix_sum(pla);
    const float Atot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 63));
    if (w == 0) {
      cl_s[lane] = cl * kLog2e;  // base-2 units for the score decays
      esf_s[lane] = __expf(Atot - cl);
    }
    __syncthreads();

    // ---------------- previous chunk: add the partner's partial sums, store
    if (n > n0) {
      const int partner = w ^ 4;
      const f32x4 x0 = Xc[(partner * 2 + 0) * 64 + lane];
      const f32x4 x1 = Xc[(partner * 2 + 1) * 64 + lane];
      const int tp = tok0 - C;
      if constexpr (DLAM) {
        // transposed tiles: row li, columns c0 + 4 g4 .. + 3
        store_row(outr, O0 + x0, ((tp + 16 * own0 + li) * dv + dv0 + c0 + 4 * g4) * 4);
        store_row(outr, O1 + x1, ((tp + 16 * own1 + li) * dv + dv0 + c0 + 4 * g4) * 4);
        dlam_flush(n - 1);
      } else {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // rows past T fall outside the output range and are dropped
          const int t0 = tp + 16 * own0 + 4 * g4 + r;
          const int t1 = tp + 16 * own1 + 4 * g4 + r;
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O0[r] + x0[r]), outr, (t0 * dv + dv0 + c0 + li) * 4, 0, 0);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O1[r] + x1[r]), outr, (t1 * dv + dv0 + c0 + li) * 4, 0, 0);
        }
      }
    }

    // fp16 copy of Q for the Q.G products, scaled by a power of two so the
    // chunk's max |q| sits at 2^14..2^15 (exact for bf16 values in range)
    int eq = 0;
    if constexpr (!DLAM) {
      float qmx = qmax_s[0];
#pragma unroll
      for (int i = 1; i < 8; ++i) qmx = fmaxf(qmx, qmax_s[i]);
      eq = scale_exp(qmx);
      const float sc = exp2_int(-eq);
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
        f16x8 hq;
#pragma unroll
        for (int e = 0; e < 8; ++e) hq[e] = static_cast<_Float16>(static_cast<float>(pq[i][e]) * sc);
        *reinterpret_cast<f16x8*>(Qh + row * LDQ + col) = hq;
      }
    }

    if (n + 1 < n1) prefetch(n + 1);

    // ---------------- phase 1: masked score tiles -> LDS -------------------
    // Waves 0..3 take the diagonal tile (w,w); waves 4..7 take (1,0) (2,0)
    // (2,1) (3,0); waves 0 and 1 also take (3,1) and (3,2).  Waves 2 and 3
    // zero the slots above the diagonal inside the last K-step of an even
    // query block, (0,1) and (2,3).
    {
      const int ntile = w < 2 ? 2 : 1;
      int qbt[2], kbt[2];
      if (w < 4) { qbt[0] = w; kbt[0] = w; }
      else if (w == 4) { qbt[0] = 1; kbt[0] = 0; }
      else if (w == 5) { qbt[0] = 2; kbt[0] = 0; }
      else if (w == 6) { qbt[0] = 2; kbt[0] = 1; }
      else { qbt[0] = 3; kbt[0] = 0; }
      qbt[1] = 3;
      kbt[1] = w == 0 ? 1 : 2;
      f32x4 acc[2];
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          if (it < ntile) {
            if constexpr (DLAM) {  // fp16 K copy (in the Q tile's place) and scaled fp16 q
              const f16x8 kh = *reinterpret_cast<const f16x8*>(reinterpret_cast<const _Float16*>(Qs) +
                                                               (16 * kbt[it] + li) * LDQ + 32 * ks + 8 * g4);
              const f16x8 qh = *reinterpret_cast<const f16x8*>(Qh + (16 * qbt[it] + li) * LDQ + 32 * ks + 8 * g4);
              acc[it] = mma16(kh, qh, acc[it]);
            } else {
              const bf16x8 ka =
                  *reinterpret_cast<const bf16x8*>(Ks + (16 * kbt[it] + li) * LDQ + 32 * ks + 8 * g4);
              const bf16x8 qb8 =
                  *reinterpret_cast<const bf16x8*>(Qs + (16 * qbt[it] + li) * LDQ + 32 * ks + 8 * g4);
              acc[it] = mma(ka, qb8, acc[it]);
            }
          }
        }
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        if (it < ntile) {
          const int qb = qbt[it], kb = kbt[it];
          // acc[r] = score(query 16qb+li, key 16kb+4g4+r)
          const int qi = 16 * qb + li;
          // DLAM: undo the row's fp16 scale through the decay exponent (base 2)
          const float clq = DLAM ? cl_s[qi] + static_cast<float>(er_s[qi]) : cl_s[qi];
          const f32x4 clk = *reinterpret_cast<const f32x4*>(cl_s + 16 * kb + 4 * g4);
          f32x4 pv4;
          if (kb < qb) {
            const float lam = lam_s[qi * L + 4 + (32 - __clz(qb ^ kb))];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv4[r] = acc[it][r] * lam * exp2f_fast(clq - clk[r]);
          } else {
            // diagonal tile: same 16-block, so the level and the causal
            // mask depend on the in-block positions only
#pragma unroll
            for (int r = 0; r < 4; ++r)
              pv4[r] = (dmask >> r) & 1 ? acc[it][r] * lam_s[qi * L + dlev[r]] * exp2f_fast(clq - clk[r]) : 0.f;
          }
          bf16x4 h, l;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16 x1, x2;
            split_bf16_t(pv4[r], x1, x2);
            h[r] = x1;
            l[r] = x2;
          }
          bf16* dst = reinterpret_cast<bf16*>(Ps + ((qb * 2 + (kb >> 1)) * 2) * 64 + lane) + 4 * (kb & 1);
          *reinterpret_cast<bf16x4*>(dst) = h;
          *reinterpret_cast<bf16x4*>(dst + 64 * 8) = l;
        }
      }
      if (w == 2 || w == 3) {
        const int qb = w == 2 ? 0 : 2;  // zero slot (qb, qb+1)
        bf16* dst = reinterpret_cast<bf16*>(Ps + ((qb * 2 + (qb >> 1)) * 2) * 64 + lane) + 4;
        *reinterpret_cast<bf16x4*>(dst) = bf16x4{};
        *reinterpret_cast<bf16x4*>(dst + 64 * 8) = bf16x4{};
      }
    }
    // Row weights of this wave's Q.G products for each live inter-chunk
    // level b (lane = row): lambda[row, log2C+1+b] * exp(cl_row + dec_b) (decay
    // from the bucket's end to the row) * 2^eq (fp16 Q scale) * 2^eg[b] (this
    // wave's state scale).  Written and read by this wave only.
    if constexpr (!DLAM) {
      const float ecl = __expf(cl) * exp2_int(eq);
      float lv[NSLOT];
#pragma unroll
      for (int b = 0; b < NSLOT; ++b) lv[b] = lam_s[lane * L + LOGC + 1 + b];
#pragma unroll
      for (int b = 0; b < NSLOT; ++b)
        if ((n >> b) & 1) lw[b * C + lane] = lv[b] * ecl * (__expf(dec[b]) * exp2_int(eg[b]));
    }
    __syncthreads();

    // ---------------- phase 2 ----------------------------------------------
    // Q.G over this wave's dk half for all four row tiles (fp16 MFMAs).
    f32x4 Op[4];
#pragma unroll
    for (int mi = 0; mi < 4; ++mi) Op[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
    {
      if constexpr (DLAM) {
        // lane li is row 16 mi + li, element r column c0 + 4 g4 + r.  Row
        // factor exp(cl_row) 2^eq; the forward's q of the row and columns.
        // Row tiles outer, levels inner: one tile's Q fragments are live at
        // a time.
        float* dlw = reinterpret_cast<float*>(smem + LW_OFF) + w * (C * NSLOT);
        float fb[NSLOT];
#pragma unroll
        for (int b = 0; b < NSLOT; ++b) fb[b] = uniform(__expf(dec[b]) * exp2_int(eg[b]));
#pragma unroll
        for (int mi = 0; mi < 4; ++mi) {
          const f16x8 qa0 = *reinterpret_cast<const f16x8*>(Qh + (16 * mi + li) * LDQ + 64 * hh + 8 * g4);
          const f16x8 qa1 = *reinterpret_cast<const f16x8*>(Qh + (16 * mi + li) * LDQ + 64 * hh + 32 + 8 * g4);
          const float ecr = exp2f_fast(cl_s[16 * mi + li]) * exp2_int(er_s[16 * mi + li]);
          const f16x4 qof = *reinterpret_cast<const f16x4*>(Qo + (16 * mi + li) * LDQO + c0 + 4 * g4);
#pragma unroll
          for (int b = 0; b < NSLOT; ++b) {
            if ((n >> b) & 1) {
              f32x4 acc = mma16(G[b][0], qa0, f32x4{0.f, 0.f, 0.f, 0.f});
              acc = mma16(G[b][1], qa1, acc);
              const float wd = ecr * fb[b];  // the level's read of this row: wd * acc
              const float wq = lam_s[(16 * mi + li) * L + LOGC + 1 + b] * wd;
#pragma unroll
              for (int r = 0; r < 4; ++r) Op[mi][r] += wq * acc[r];
              // dot of the row's read with the forward's q over this wave's
              // 16 columns: four products here, the other twelve in the
              // lanes li + 16, + 32, + 48 (same row, next column groups)
              float pd = 0.f;
#pragma unroll
              for (int r = 0; r < 4; ++r) pd += static_cast<float>(qof[r]) * acc[r];
              pd = xor16_sum(pd);
              pd = xor32_sum(pd);
              if (g4 == 0) dlw[(16 * mi + li) * NSLOT + b] = pd * wd;
            }
          }
        }
      } else {
        f16x8 qa[4][2];
#pragma unroll
        for (int mi = 0; mi < 4; ++mi)
#pragma unroll
          for (int ks = 0; ks < 2; ++ks)
            qa[mi][ks] = *reinterpret_cast<const f16x8*>(Qh + (16 * mi + li) * LDQ + 64 * hh + 32 * ks + 8 * g4);
#pragma unroll
        for (int b = 0; b < NSLOT; ++b) {
          if ((n >> b) & 1) {
            f32x4 acc[4];
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) acc[mi] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < 2; ++ks)
#pragma unroll
              for (int mi = 0; mi < 4; ++mi) acc[mi] = mma16(qa[mi][ks], G[b][ks], acc[mi]);
#pragma unroll
            for (int mi = 0; mi < 4; ++mi) {
              const f32x4 wv = *reinterpret_cast<const f32x4*>(lw + b * C + 16 * mi + 4 * g4);
#pragma unroll
              for (int r = 0; r < 4; ++r) Op[mi][r] += wv[r] * acc[mi][r];
            }
          }
        }
      }
    }
    // hand the partial sums of the partner's row tiles over (read after the
    // next barrier)
    Xc[(w * 2 + 0) * 64 + lane] = Op[oth0];
    Xc[(w * 2 + 1) * 64 + lane] = Op[oth1];
    // P V for this wave's two row tiles; keys in the score tile order
    // (32ks + 4g4 + e, then +16), V operand by transposed reads.
    O0 = Op[own0];
    O1 = Op[own1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16* v0 = Vs + (32 * ks + 4 * g4 + (li >> 2)) * LDV + c0 + 4 * (li & 3);
      const bf16x8 vb = cat(tr_read(v0), tr_read(v0 + 16 * LDV));
      if constexpr (DLAM) {  // transposed tiles
        if (2 * ks <= own0) {
          O0 = mma(vb, Ps[((own0 * 2 + ks) * 2 + 0) * 64 + lane], O0);
          O0 = mma(vb, Ps[((own0 * 2 + ks) * 2 + 1) * 64 + lane], O0);
        }
        if (2 * ks <= own1) {
          O1 = mma(vb, Ps[((own1 * 2 + ks) * 2 + 0) * 64 + lane], O1);
          O1 = mma(vb, Ps[((own1 * 2 + ks) * 2 + 1) * 64 + lane], O1);
        }
      } else {
        if (2 * ks <= own0) {
          O0 = mma(Ps[((own0 * 2 + ks) * 2 + 0) * 64 + lane], vb, O0);
          O0 = mma(Ps[((own0 * 2 + ks) * 2 + 1) * 64 + lane], vb, O0);
        }
        if (2 * ks <= own1) {
          O1 = mma(Ps[((own1 * 2 + ks) * 2 + 0) * 64 + lane], vb, O1);
          O1 = mma(Ps[((own1 * 2 + ks) * 2 + 1) * 64 + lane], vb, O1);
        }
      }
    }

    // ---------------- this chunk's state + lssb merge (registers) ----------
    // Chunk n -> n+1: its state joins the buckets the next chunk reads.  The
    // merge writes level m = lssb(n+1), which chunk n does not read (bit m of
    // n is clear), and only reads the levels below m, so it can follow this
    // chunk's Q.G products and overlap the P V products.  K and V of chunk n
    // stay in their parity buffer until the staging of chunk n+2, which comes
    // after the next chunk's second barrier.
    // The fold runs at raised wave priority: its vector work then issues ahead
    // of the partner wave's, which is still in its matrix products (measured
    // ~1.5% faster for the whole sweep).
    __builtin_amdgcn_s_setprio(1);
    if (n + 1 < n1) {
      const int m = __builtin_ctz(static_cast<unsigned>(n + 1));
      // decayed V of this wave's columns, tokens 32ks + 8g4 + e, split hi/lo
      bf16x8 vh[2], vl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const bf16* v0 = Vs + (32 * ks + 8 * g4 + (li >> 2)) * LDV + c0 + 4 * (li & 3);
        const bf16x8 x = cat(tr_read(v0), tr_read(v0 + 4 * LDV));
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 x1, x2;
          split_bf16_t(static_cast<float>(x[e]) * (e < 4 ? e0[e] : e1[e - 4]), x1, x2);
          vh[ks][e] = x1;
          vl[ks][e] = x2;
        }
      }
      // S tiles t = 2*kl + half (kl = local K-step of the dk half) cover dk
      // 64hh + 32kl + 8*(row>>2) + 4*half + (row&3); S[t][r] is element
      // 4*half + r of G[.][kl].  Lower levels, decayed to the end of chunk n,
      // are added first; hi / lo halves of V accumulate separately.
      f32x4 Sh[4], Sl[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        Sh[t] = f32x4{0.f, 0.f, 0.f, 0.f};
        Sl[t] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
#pragma unroll
      for (int b = 0; b < NSLOT - 1; ++b) {
        if (b < m) {
          const float fl = __expf(dec[b] + Atot) * exp2_int(eg[b]);
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int r = 0; r < 4; ++r) Sh[t][r] += fl * static_cast<float>(G[b][t >> 1][4 * (t & 1) + r]);
        }
      }
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int kq = 2 * hh + (t >> 1), half = t & 1;
          const bf16* k0 = Ks + (32 * ks + 8 * g4 + (li >> 2)) * LDQ + 32 * kq + 8 * (li & 3) + 4 * half;
          const bf16x8 ka = cat(tr_read(k0), tr_read(k0 + 4 * LDQ));
          Sh[t] = mma(ka, vh[ks], Sh[t]);
          Sl[t] = mma(ka, vl[ks], Sl[t]);
        }
      }
      float mx = 0.f;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          Sh[t][r] += Sl[t][r];
          mx = fmaxf(mx, fabsf(Sh[t][r]));
        }
      const int em = scale_exp(wave_max(mx));
      const float sc = exp2_int(-em);
      f16x8 gn[2];
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) gn[t >> 1][4 * (t & 1) + r] = static_cast<_Float16>(Sh[t][r] * sc);
      if constexpr (DLAM) {
        // the same merge as one uniform per-level loop: the register
        // allocation of this variant spills less with it (the forward
        // instantiations spill more with it)
#pragma unroll
        for (int b = 0; b < NSLOT; ++b) {
          if (b == m) {
            G[b][0] = gn[0];
            G[b][1] = gn[1];
            eg[b] = em;
          }
          dec[b] = uniform(b == m ? 0.f : (b > m ? dec[b] + Atot : dec[b]));
        }
      } else if (m == 0) {  // every other chunk: the new state is level 0, nothing merged
        G[0][0] = gn[0];
        G[0][1] = gn[1];
        eg[0] = em;
        dec[0] = 0.f;
#pragma unroll
        for (int b = 1; b < NSLOT; ++b) dec[b] = uniform(dec[b] + Atot);
      } else {
#pragma unroll
        for (int b = 1; b < NSLOT; ++b) {
          if (b == m) {
            G[b][0] = gn[0];
            G[b][1] = gn[1];
            eg[b] = em;
          }
          dec[b] = uniform(b == m ? 0.f : (b > m ? dec[b] + Atot : dec[b]));
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    Aprev = Atot;
    // DLAM stages the scaled dO (Qh), the forward's q (Qo) and their row
    // exponents before the chunk's first barrier, and phase 2 reads them:
    // every wave finishes this chunk before any wave stages the next one
    if constexpr (DLAM) __syncthreads();
  }

  // ---------------- last chunk: add the partner's partial sums, store -------
  __syncthreads();
  if (n1 > n0) {
    const int partner = w ^ 4;
    const f32x4 x0 = Xc[(partner * 2 + 0) * 64 + lane];
    const f32x4 x1 = Xc[(partner * 2 + 1) * 64 + lane];
    const int tp = (n1 - 1) * C;
    if constexpr (DLAM) {
      store_row(outr, O0 + x0, ((tp + 16 * own0 + li) * dv + dv0 + c0 + 4 * g4) * 4);
      store_row(outr, O1 + x1, ((tp + 16 * own1 + li) * dv + dv0 + c0 + 4 * g4) * 4);
      dlam_flush(n1 - 1);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t0 = tp + 16 * own0 + 4 * g4 + r;
        const int t1 = tp + 16 * own1 + 4 * g4 + r;
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O0[r] + x0[r]), outr, (t0 * dv + dv0 + c0 + li) * 4, 0, 0);
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(O1[r] + x1[r]), outr, (t1 * dv + dv0 + c0 + li) * 4, 0, 0);
      }
    }
  }

  // ---------------- prefill: decode states at T-1, inter-chunk levels -------
  // The last segment ends at the last chunk, whose bucket states are the
  // level-(log2C+1+b) states of its queries; decayed from each bucket's end to
  // token T-1 (cl of the last token = the chunk total, the tail reads zero).
  if (EMIT && seg == a.nseg - 1 && n1 > n0) {
    const int nl = n1 - 1;
    float* __restrict__ so = a.st_out + (size_t)bh * a.st_L * dk * dv + dv0 + c0 + li;
    for (int lev = LOGC + 1; lev < a.st_L; ++lev) {
      const int b = lev - LOGC - 1;
      float f = 0.f;
      f16x8 g[2] = {f16x8{}, f16x8{}};
#pragma unroll
      for (int bb = 0; bb < NSLOT; ++bb) {
        if (bb == b && ((nl >> bb) & 1)) {
          f = __expf(Aprev + dec[bb]) * exp2_int(eg[bb]);
          g[0] = G[bb][0];
          g[1] = G[bb][1];
        }
      }
#pragma unroll
      for (int kl = 0; kl < 2; ++kl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 64 * hh + 32 * kl + 8 * g4 + e;  // dk index of G[.][kl][e]
          if (d < dk) so[((size_t)lev * dk + d) * dv] = f * static_cast<float>(g[kl][e]);
        }
    }
  }
}

// Segment states for the register-state path (bf16, dk <= 128, dv % 64 == 0):
// T_g = sum over segment g of exp(cum[end] - cum[s]) k_s v_s^T, written as
// [dv][128] fp32, plus the segment's total log decay.  One 512-thread
// workgroup per (b,h, segment, 64 dv columns); the segment is walked in
// 64-token tiles from its end to its start, so each token's weight, the decay
// from it to the segment's end, is the tile's in-tile suffix plus the running
// total of the tiles already walked, and the running sum never needs a
// rescale.  Each tile's V is scaled by those weights and split bf16 hi/lo
// once, at staging; K and V stay row-major in LDS (double buffered, one
// barrier per tile, loads issued two tiles ahead) and are read transposed.
// Every tile's loads go through buffer resources over just that tile's rows
// inside the segment (scalar work), so the per-lane offsets are constants and
// rows past the segment's end, or tiles before its start, read zero.  Wave w
// keeps the 64 x 16 block (dk half w>>2, columns 16(w&3)) of the running sum.
// Workgroups of the same (b,h, segment) sit on the same XCD so the second
// column group finds K in L2.
namespace ss {
constexpr int NTH = 512;
// K row stride (bf16): 80 banks, 16 modulo 64, so the four rows and four
// 16-byte pieces a 16-lane group reads in a transposed read fall on disjoint
// banks (K is only read transposed here)
constexpr int LDK = 160;
constexpr int KS_OFF = 0;
constexpr int VH_OFF = KS_OFF + rs::C * LDK * 2;
constexpr int VL_OFF = VH_OFF + rs::C * rs::LDV * 2;
constexpr int BUF = VL_OFF + rs::C * rs::LDV * 2;
constexpr int LDS_BYTES = 2 * BUF;
}  // namespace ss

__global__ void __launch_bounds__(512) seg_state_rs_kernel(SegArgs a) {
  using namespace rs;
  extern __shared__ __align__(16) unsigned char smem[];
  const int D = a.dv >> 6;
  const int nsg = a.nseg - 1;  // the last segment's state is never used
  const int id = blockIdx.x;
  const int px = id & 7, rest = id >> 3;
  const int dg = rest % D, pg = rest / D;
  const int p = pg * 8 + px;
  if (p >= a.BH * nsg) return;
  const int bh = p / nsg, g = p - bh * nsg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int cs = w & 3, hh = w >> 2, c0 = 16 * cs;
  const int T = a.T, dk = a.dk, dv = a.dv;
  const int segtok = a.C << a.seg_log2;
  const int s0 = g * segtok, s1 = min(T, s0 + segtok);
  const int dv0 = dg * 64;
  const size_t bhT = (size_t)bh * T;
  const bf16* kb = static_cast<const bf16*>(a.k) + (size_t)(bh / a.G) * T * dk;
  const bf16* vb = static_cast<const bf16*>(a.v) + bhT * dv;
  const float* lb = a.log_a + bhT;
  // this lane's byte offsets inside a tile: K rows v >> 4 (16-byte pieces
  // past dk fall outside every resource), V row tid >> 3, log_a token lane
  uint32_t ko[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int v = tid + ss::NTH * i, row = v >> 4, col = (v & 15) * 8;
    ko[i] = col < dk ? static_cast<uint32_t>((row * dk + col) * 2) : kOutOfRange;
  }
  const uint32_t vo = static_cast<uint32_t>(((tid >> 3) * dv + dv0 + (tid & 7) * 8) * 2);

  // Register prefetch two tiles ahead: tiles alternate between two register
  // sets (and the two LDS buffers).
  struct Regs {
    bf16x8 k[2], v;
    float la;
  };
  auto prefetch = [&](Regs& r, int b0) {
    const int nrow = b0 >= s0 ? min(C, s1 - b0) : 0;  // rows of the tile inside the segment
    const int t0 = max(b0, 0);
    const rsrc_t kr = make_rsrc(kb + (size_t)t0 * dk, static_cast<uint32_t>(nrow * dk * 2));
    const rsrc_t vr = make_rsrc(vb + (size_t)t0 * dv, static_cast<uint32_t>(nrow * dv * 2));
    const rsrc_t lar = make_rsrc(lb + t0, static_cast<uint32_t>(nrow * 4));
    r.la = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lar, lane * 4, 0, 0));
#pragma unroll
    for (int i = 0; i < 2; ++i) r.k[i] = load_b128(kr, ko[i]);
    r.v = load_b128(vr, vo);
  };

  f32x4 S[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) S[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  float later = 0.f;  // total log decay of the tiles after the current one
  // one 64-token tile from register set r into LDS buffer buf, then its MFMAs
  auto tile = [&](Regs& r, int buf, int b0) {
    // keep the scheduler from hoisting this tile's register work above the
    // previous tile: that would wait for loads meant to stay in flight
    __builtin_amdgcn_sched_barrier(0);
    unsigned char* base = smem + buf * ss::BUF;
    bf16* Ks = reinterpret_cast<bf16*>(base + ss::KS_OFF);
    bf16* Vh = reinterpret_cast<bf16*>(base + ss::VH_OFF);
    bf16* Vl = reinterpret_cast<bf16*>(base + ss::VL_OFF);
    // decay of each token to the segment's last token, every wave redundantly
    const float cl = wave_prefix_sum(r.la);
    const float Ab = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 63));
    const float esf = __expf(Ab - cl + later);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + ss::NTH * i, row = v >> 4, col = (v & 15) * 8;
      *reinterpret_cast<bf16x8*>(Ks + row * ss::LDK + col) = r.k[i];
    }
    {
      const int row = tid >> 3, col = (tid & 7) * 8;
      const float e = __shfl(esf, row);
      bf16x8 h, l;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        bf16 x1, x2;
        split_bf16(static_cast<float>(r.v[j]) * e, x1, x2);
        h[j] = x1;
        l[j] = x2;
      }
      *reinterpret_cast<bf16x8*>(Vh + row * LDV + col) = h;
      *reinterpret_cast<bf16x8*>(Vl + row * LDV + col) = l;
    }
    later += Ab;
    prefetch(r, b0 - 2 * C);
    __syncthreads();

#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int vrow = (32 * ks + 8 * g4 + (li >> 2)) * LDV + c0 + 4 * (li & 3);
      const bf16x8 vh = cat(tr_read(Vh + vrow), tr_read(Vh + vrow + 4 * LDV));
      const bf16x8 vl = cat(tr_read(Vl + vrow), tr_read(Vl + vrow + 4 * LDV));
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int kq = 2 * hh + (t >> 1), half = t & 1;
        const bf16* k0 = Ks + (32 * ks + 8 * g4 + (li >> 2)) * ss::LDK + 32 * kq + 8 * (li & 3) + 4 * half;
        const bf16x8 ka = cat(tr_read(k0), tr_read(k0 + 4 * ss::LDK));
        S[t] = mma(ka, vh, S[t]);
        S[t] = mma(ka, vl, S[t]);
      }
    }
  };
  // Tiles from the segment's last down to its first, two per iteration (an
  // odd count ends with a tile before the segment: zeros, exp(0)); with a
  // fixed count of loads per tile the wait for a tile's registers leaves the
  // following tile's loads in flight.
  const int ntile = (s1 - s0 + C - 1) / C;
  Regs ra, rb;
  int b0 = s0 + (ntile - 1) * C;
  prefetch(ra, b0);
  prefetch(rb, b0 - C);
  for (int k = 0; k < ntile; k += 2, b0 -= 2 * C) {
    tile(ra, 0, b0);
    tile(rb, 1, b0 - C);
  }
  // element r of S[t] is dk 64hh + 32(t>>1) + 8g4 + 4(t&1) + r, column c0 + li
  float* __restrict__ Tout =
      a.seg_state + ((size_t)(bh * a.nseg + g) * dv + dv0 + c0 + li) * DKP + 64 * hh + 8 * g4;
#pragma unroll
  for (int kl = 0; kl < 2; ++kl) {
    *reinterpret_cast<f32x4*>(Tout + 32 * kl) = S[2 * kl];
    *reinterpret_cast<f32x4*>(Tout + 32 * kl + 4) = S[2 * kl + 1];
  }
  if (tid == 0 && dg == 0) a.seg_decay[bh * a.nseg + g] = later;
}

int launch_seg_state_rs(const SegArgs& a, int BH, hipStream_t stream) {
  const long long pairs = (long long)BH * (a.nseg - 1);
  const long long nblocks = (pairs + 7) / 8 * 8 * (a.dv / 64);
  if (nblocks > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  const size_t row_bytes = std::max((size_t)a.dk * 2, (size_t)a.dv * 2);
  if ((size_t)(a.T + 2 * rs::C) * row_bytes >= (size_t)1 << 31) return LL_ERR_UNSUPPORTED;
  static std::atomic<uint64_t> raised{0};
  if (!raise_lds_limit(reinterpret_cast<const void*>(&seg_state_rs_kernel), raised, ss::LDS_BYTES)) return LL_ERR_HIP;
  hipLaunchKernelGGL(seg_state_rs_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(ss::NTH), ss::LDS_BYTES,
                     stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int rs_max_slots() { return 10; }

int rs_dlam_lds_bytes(int L, int nslot) { return rs::lds_bytes_dlam(L, nslot); }

int launch_sweep_rs_dlam(const FwdArgs& a, int nblocks, hipStream_t stream) {
  const int bytes = rs::lds_bytes_dlam(a.L, a.nslot);
  if (a.nslot > 8 || a.L > 24 || bytes > kMaxLds || !a.qo || !a.dlam_part || a.G != 1 || a.st_out)
    return LL_ERR_UNSUPPORTED;
  const size_t row_bytes = std::max({(size_t)a.dk * 2, (size_t)a.dv * 4, (size_t)a.L * 4});
  if ((size_t)(a.T + 2 * rs::C) * row_bytes >= (size_t)1 << 31) return LL_ERR_UNSUPPORTED;
  static std::atomic<uint64_t> raised{0};
  if (!raise_lds_limit(reinterpret_cast<const void*>(&fwd_rs_kernel<8, false, true>), raised)) return LL_ERR_HIP;
  hipLaunchKernelGGL((fwd_rs_kernel<8, false, true>), dim3(nblocks), dim3(512), bytes, stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int rs_lds_bytes(int L, int nslot) { return rs::lds_bytes(L, nslot); }

int launch_sweep_rs(const FwdArgs& a, int nblocks, hipStream_t stream) {
  const int bytes = rs::lds_bytes(a.L, a.nslot);
  if (a.nslot > 10 || a.L > 24 || bytes > kMaxLds) return LL_ERR_UNSUPPORTED;
  // buffer offsets are 32-bit: every per-(b,h) slice, tail chunk included,
  // must stay below 2^31 bytes
  const size_t row_bytes = std::max({(size_t)a.dk * 2, (size_t)a.dv * 4, (size_t)a.L * 4});
  if ((size_t)(a.T + 2 * rs::C) * row_bytes >= (size_t)1 << 31) return LL_ERR_UNSUPPORTED;
  // instantiations: 8 register slots (up to 256 chunks) or 10 (up to 1024);
  // EMIT adds the prefill state output
  const bool wide = a.nslot > 8;
  const void* fn = wide ? (a.st_out ? reinterpret_cast<const void*>(&fwd_rs_kernel<10, true>)
                                    : reinterpret_cast<const void*>(&fwd_rs_kernel<10, false>))
                        : (a.st_out ? reinterpret_cast<const void*>(&fwd_rs_kernel<8, true>)
                                    : reinterpret_cast<const void*>(&fwd_rs_kernel<8, false>));
  // each instantiation's limit is raised to the maximum once per device
  static std::atomic<uint64_t> raised[4] = {};
  if (!raise_lds_limit(fn, raised[(wide ? 2 : 0) + (a.st_out ? 1 : 0)])) return LL_ERR_HIP;
  if (wide && a.st_out)
    hipLaunchKernelGGL((fwd_rs_kernel<10, true>), dim3(nblocks), dim3(512), bytes, stream, a);
  else if (wide)
    hipLaunchKernelGGL((fwd_rs_kernel<10, false>), dim3(nblocks), dim3(512), bytes, stream, a);
  else if (a.st_out)
    hipLaunchKernelGGL((fwd_rs_kernel<8, true>), dim3(nblocks), dim3(512), bytes, stream, a);
  else
    hipLaunchKernelGGL((fwd_rs_kernel<8, false>), dim3(nblocks), dim3(512), bytes, stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
