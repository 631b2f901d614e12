// Gradient of the fused level-weight projection of loglinear_lambda.hip
// ([P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制",
// section 循环形式与输出计算, with the map read as softplus):
//   z = x W^T + bias,  lambda = softplus(z),  m = b*T + t,  n = h*L + l
//   dz[m, n] = dlambda[b, h, t, l] * sigmoid(z[m, n])
//   dx       = dz W            ([B*T, D])
//   dW       = dz^T x          ([H*L, D])
//   dbias[n] = sum_m dz[m, n]
// sigmoid(z) is taken from the forward's output: e^-lambda = 1 / (1 + e^z), so
// sigmoid(z) = 1 - e^-lambda = -expm1(-lambda), which stays accurate where
// lambda is tiny.
//
// bf16 x and W with D % 8 == 0 (lam_dz16_kernel, lam_mm16_kernel): dz is
// split once into bf16 hi + lo arrays with padded rows, the two products run
// as 128 x 128-tile bf16 matrix-core GEMMs on exact operands (hi and lo
// products summed in fp32; dW split over row ranges of B*T into partials),
// and dW, dbias come from in-order sums of partials.  Other inputs: dz into an
// fp32 scratch matrix and one small-tile product kernel for both products
// (fp32 MFMAs for fp32 inputs, bf16 MFMAs on dz split hi / lo for bf16), with
// dbias as one extra column of ones on the x side.  No atomics anywhere, so
// results are deterministic.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

// dz[m, h*L + l] from dlambda and lambda in their [B, H, T, L] layout: one
// workgroup per (b, h, 64 tokens); the 64*L values of a (b, h) token block
// are contiguous, so reads are coalesced and each row's L outputs are one run.
__global__ void __launch_bounds__(256) lam_dz_kernel(LamBwdArgs a) {
  const int nt = (a.T + 63) / 64;
  const long long id = blockIdx.x;
  const int tb = static_cast<int>(id % nt);
  const long long bh = id / nt;
  const int h = static_cast<int>(bh % a.H);
  const long long b = bh / a.H;
  const int t0 = tb * 64;
  const int rows = min(64, a.T - t0);
  const int HL = a.H * a.L;
  const long long src = (bh * a.T + t0) * a.L;
  for (int i = threadIdx.x; i < rows * a.L; i += 256) {
    const int t = i / a.L, l = i - t * a.L;
    const float s = -expm1f(-a.lam[src + i]);
    a.dz[(b * a.T + t0 + t) * HL + h * a.L + l] = a.dlam[src + i] * s;
  }
}

namespace lg {
constexpr int BM = 64, BN = 64, BK = 32, NT = 256, LD = BK + 4;
}

template <typename T>
__device__ __forceinline__ float widen(const T* p, long long i) { return static_cast<float>(p[i]); }

// Element i (0 <= i < rows * BK / 256) of a thread's share of a (rows x BK)
// tile sits at row r0 + dr * i, k index k0 + dk * i: with k contiguous in
// memory the 256 threads walk rows of BK consecutive k, otherwise columns of
// consecutive rows, so a wave's loads are always one contiguous run.
template <int ROWS, int BK>
struct TileMap {
  int r0, k0, dr, dk;
  __device__ TileMap(int tid, bool kc) {
    constexpr int T = 256;
    if (kc) { r0 = tid / BK; k0 = tid % BK; dr = T / BK; dk = 0; }
    else { r0 = tid % ROWS; k0 = tid / ROWS; dr = 0; dk = T / ROWS; }
  }
};

// C(m, n) = sum_k A(m, k) B(k, n) over this workgroup's K range, fp32 MFMA.
// One 256-thread workgroup per (64 x 64 tile, K split); the four waves form a
// 2 x 2 grid of 32 x 32 blocks.  A and B tiles are staged in LDS as [row][k]
// with the global reads coalesced along whichever index has unit stride.
template <typename TA, typename TB>
__global__ void __launch_bounds__(lg::NT) lam_gemm_kernel(GemmArgs g) {
  using namespace lg;
  __shared__ float As[BM][LD];
  __shared__ float Bs[BN][LD];
  const int ntn = (g.N + BN - 1) / BN, ntm = (g.M + BM - 1) / BM;
  const long long id = blockIdx.x;
  const int tn = static_cast<int>(id % ntn);
  const long long rest = id / ntn;
  const int tm = static_cast<int>(rest % ntm);
  const int split = static_cast<int>(rest / ntm);
  const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
  const long long kb = (long long)split * g.kper;
  const long long ke = min((long long)g.K, kb + g.kper);
  const TA* A = static_cast<const TA*>(g.A);
  const TB* Bp = static_cast<const TB*>(g.B);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const bool a_kc = g.sak == 1, b_kc = g.sbk == 1;

  constexpr int PER = BM * BK / NT;
  const TileMap<BM, BK> am(tid, a_kc);
  const TileMap<BN, BK> bm(tid, b_kc);
  // in-tile element steps: i * step stays below 2^27 (i < 16, a step of at
  // most 8 rows of at most 2^20 elements, checked by the host)
  const int astep = static_cast<int>(am.dr * g.sam + am.dk * g.sak);
  const int bstep = static_cast<int>(bm.dk * g.sbk + bm.dr * g.sbn);
  float ra[PER], rb[PER];
  auto load = [&](long long k0) {
    const TA* pa = A + (m0 + am.r0) * g.sam + (k0 + am.k0) * g.sak;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool ok = m0 + am.r0 + am.dr * i < g.M && k0 + am.k0 + am.dk * i < ke;
      ra[i] = ok ? widen(pa, i * astep) : 0.f;
    }
    const TB* pb = Bp + (k0 + bm.k0) * g.sbk + (n0 + bm.r0) * g.sbn;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const long long n = n0 + bm.r0 + bm.dr * i;
      float v = 0.f;
      if (k0 + bm.k0 + bm.dk * i < ke) {
        if (n < g.nb_real) v = widen(pb, i * bstep);
        else if (g.ones && n == g.nb_real) v = 1.f;
      }
      rb[i] = v;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) As[am.r0 + am.dr * i][am.k0 + am.dk * i] = ra[i];
#pragma unroll
    for (int i = 0; i < PER; ++i) Bs[bm.r0 + bm.dr * i][bm.k0 + bm.dk * i] = rb[i];
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb < ke) load(kb);
  for (long long k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();  // the previous tile's reads are done
    stage();
    __syncthreads();
    if (k0 + BK < ke) load(k0 + BK);  // next tile's global reads overlap the products
#pragma unroll
    for (int kk = 0; kk < BK; kk += 4) {
      float af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = As[32 * wm + 16 * i + li][kk + g4];
#pragma unroll
      for (int j = 0; j < 2; ++j) bf[j] = Bs[32 * wn + 16 * j + li][kk + g4];
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x4f32(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
  }
  // acc[i][j][r] = C(m0 + 32wm + 16i + 4g4 + r, n0 + 32wn + 16j + li)
  float* C = g.C + split * g.split_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const long long n = n0 + 32 * wn + 16 * j + li;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long m = m0 + 32 * wm + 16 * i + 4 * g4 + r;
        if (m < g.M) C[m * g.ldc + n] = acc[i][j][r];
      }
    }
}

// The same product for a bf16 B operand on bf16 matrix cores
// (v_mfma_f32_16x16x32_bf16): the fp32 A operand (dz) is split at staging
// into bf16 hi + lo with |a - hi - lo| <= 2^-16 |a|, and each product is
// hi*B + lo*B with fp32 accumulation.  LDS rows of 64 k (+8 pad, 144 bytes).
namespace lg16 {
constexpr int BM = 64, BN = 64, BK = 64, NT = 256, LD = BK + 8, PER = BM * BK / NT;
}

__global__ void __launch_bounds__(lg16::NT) lam_gemm16_kernel(GemmArgs g) {
  using namespace lg16;
  __shared__ __align__(16) bf16 Ah[BM][LD];
  __shared__ __align__(16) bf16 Al[BM][LD];
  __shared__ __align__(16) bf16 Bs[BN][LD];
  const int ntn = (g.N + BN - 1) / BN, ntm = (g.M + BM - 1) / BM;
  const long long id = blockIdx.x;
  const int tn = static_cast<int>(id % ntn);
  const long long rest = id / ntn;
  const int tm = static_cast<int>(rest % ntm);
  const int split = static_cast<int>(rest / ntm);
  const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
  const long long kb = (long long)split * g.kper;
  const long long ke = min((long long)g.K, kb + g.kper);
  const float* A = static_cast<const float*>(g.A);
  const bf16* Bp = static_cast<const bf16*>(g.B);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int wm = w >> 1, wn = w & 1;
  const bool a_kc = g.sak == 1, b_kc = g.sbk == 1;

  const TileMap<BM, BK> am(tid, a_kc);
  const TileMap<BN, BK> bm(tid, b_kc);
  const int astep = static_cast<int>(am.dr * g.sam + am.dk * g.sak);
  const int bstep = static_cast<int>(bm.dk * g.sbk + bm.dr * g.sbn);
  float ra[PER];
  bf16 rb[PER];
  auto load = [&](long long k0) {
    const float* pa = A + (m0 + am.r0) * g.sam + (k0 + am.k0) * g.sak;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const bool ok = m0 + am.r0 + am.dr * i < g.M && k0 + am.k0 + am.dk * i < ke;
      ra[i] = ok ? pa[i * astep] : 0.f;
    }
    const bf16* pb = Bp + (k0 + bm.k0) * g.sbk + (n0 + bm.r0) * g.sbn;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const long long n = n0 + bm.r0 + bm.dr * i;
      bf16 v = static_cast<bf16>(0.f);
      if (k0 + bm.k0 + bm.dk * i < ke) {
        if (n < g.nb_real) v = pb[i * bstep];
        else if (g.ones && n == g.nb_real) v = static_cast<bf16>(1.f);
      }
      rb[i] = v;
    }
  };
  auto stage = [&]() {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      bf16 hi, lo;
      split_bf16(ra[i], hi, lo);
      Ah[am.r0 + am.dr * i][am.k0 + am.dk * i] = hi;
      Al[am.r0 + am.dr * i][am.k0 + am.dk * i] = lo;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) Bs[bm.r0 + bm.dr * i][bm.k0 + bm.dk * i] = rb[i];
  };

  f32x4 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (kb < ke) load(kb);
  for (long long k0 = kb; k0 < ke; k0 += BK) {
    __syncthreads();  // the previous tile's reads are done
    stage();
    __syncthreads();
    if (k0 + BK < ke) load(k0 + BK);  // next tile's global reads overlap the products
#pragma unroll
    for (int kk = 0; kk < BK; kk += 32) {
      bf16x8 ah[2], al[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        ah[i] = *reinterpret_cast<const bf16x8*>(&Ah[32 * wm + 16 * i + li][kk + 8 * g4]);
        al[i] = *reinterpret_cast<const bf16x8*>(&Al[32 * wm + 16 * i + li][kk + 8 * g4]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) bv[j] = *reinterpret_cast<const bf16x8*>(&Bs[32 * wn + 16 * j + li][kk + 8 * g4]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bv[j], acc[i][j], 0, 0, 0);
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bv[j], acc[i][j], 0, 0, 0);
        }
    }
  }
  // acc[i][j][r] = C(m0 + 32wm + 16i + 4g4 + r, n0 + 32wn + 16j + li)
  float* C = g.C + split * g.split_stride;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const long long n = n0 + 32 * wn + 16 * j + li;
      if (n >= g.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const long long m = m0 + 32 * wm + 16 * i + 4 * g4 + r;
        if (m < g.M) C[m * g.ldc + n] = acc[i][j][r];
      }
    }
}

// dW[n, d] and dbias[n] from the split partials [nsplit][HL][D + 1] (column D
// holds the bias sums), summed in split order; nsplit = 0 writes zeros.
__global__ void __launch_bounds__(256) lam_split_sum_kernel(const float* part, int nsplit, long long stride, int HL,
                                                           int D, float* dW, float* dbias) {
  const long long total = (long long)HL * (D + 1);
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < total; i += (long long)gridDim.x * 256) {
    float s = 0.f;
    for (int z = 0; z < nsplit; ++z) s += part[z * stride + i];
    const long long n = i / (D + 1);
    const int d = static_cast<int>(i - n * (D + 1));
    if (d < D) dW[n * D + d] = s;
    else if (dbias) dbias[n] = s;
  }
}

// ---------------------------------------------------------------------------
// bf16 inputs: dz is split once, in the dz kernel, into bf16 hi + lo arrays
// [B*T][HLp] (HLp = H*L rounded up to 128, padding zero), so both products are
// bf16 x bf16 matrix-core GEMMs on exact operands, hi and lo products summed
// in fp32.  The bias gradient comes from per-(64-token block) column sums of
// the fp32 dz, summed in order.
// ---------------------------------------------------------------------------

// dz as bf16 hi / lo for one (b, h, 64 tokens), plus that block's column sums.
// The workgroup of h == 0 also zeroes the row padding [H*L, HLp).
__global__ void __launch_bounds__(256) lam_dz16_kernel(LamBwdArgs a, bf16* dzh, bf16* dzl, int HLp, float* colsum) {
  __shared__ float zs[64 * 32];
  const int nt = (a.T + 63) / 64;
  const long long id = blockIdx.x;
  const int tb = static_cast<int>(id % nt);
  const long long bh = id / nt;
  const int h = static_cast<int>(bh % a.H);
  const long long b = bh / a.H;
  const int t0 = tb * 64;
  const int rows = min(64, a.T - t0);
  const int L = a.L, HL = a.H * L;
  const long long src = (bh * a.T + t0) * L;
  for (int i = threadIdx.x; i < rows * L; i += 256) {
    const int t = i / L, l = i - t * L;
    const float z = a.dlam[src + i] * -expm1f(-a.lam[src + i]);
    bf16 hi, lo;
    split_bf16(z, hi, lo);
    const long long o = (b * a.T + t0 + t) * HLp + h * L + l;
    dzh[o] = hi;
    dzl[o] = lo;
    zs[t * L + l] = z;
  }
  if (h == 0) {
    const int pad = HLp - HL;
    for (int i = threadIdx.x; i < rows * pad; i += 256) {
      const int t = i / pad;
      const long long o = (b * a.T + t0 + t) * HLp + HL + (i - t * pad);
      dzh[o] = static_cast<bf16>(0.f);
      dzl[o] = static_cast<bf16>(0.f);
    }
  }
  __syncthreads();
  if (threadIdx.x < L) {
    float sum = 0.f;
    for (int t = 0; t < rows; ++t) sum += zs[t * L + threadIdx.x];
    colsum[(b * nt + tb) * HL + h * L + threadIdx.x] = sum;
  }
}

// out[i] = sum_{r < nrows} in[r * stride + i] for i < count, in row order.
__global__ void __launch_bounds__(256) lam_rowsum_kernel(const float* in, int nrows, long long stride,
                                                         long long count, float* out) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count; i += (long long)gridDim.x * 256) {
    float s = 0.f;
    int r = 0;
    for (; r + 8 <= nrows; r += 8) {  // eight loads in flight, added in row order
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = in[(r + q) * stride + i];
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; r < nrows; ++r) s += in[r * stride + i];
    out[i] = s;
  }
}

// out[c] = sum_{r < nrows} in[r * ld + c] for c < ncols: one workgroup per 16
// columns, 16 row groups of strided rows, the 16 partial sums then added in
// group order (a fixed order: bitwise repeatable).
__global__ void __launch_bounds__(256) lam_colsum_kernel(const float* in, int nrows, long long ld, int ncols,
                                                         float* out) {
  __shared__ float ps[16][17];
  const int c = threadIdx.x & 15, grp = threadIdx.x >> 4;
  const long long col = (long long)blockIdx.x * 16 + c;
  float s = 0.f;
  if (col < ncols) {
    // eight loads in flight, added in row order
    int r = grp;
    for (; r + 7 * 16 < nrows; r += 8 * 16) {
      float v[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) v[q] = in[(long long)(r + 16 * q) * ld + col];
#pragma unroll
      for (int q = 0; q < 8; ++q) s += v[q];
    }
    for (; r < nrows; r += 16) s += in[(long long)r * ld + col];
  }
  ps[grp][c] = s;
  __syncthreads();
  if (grp == 0 && col < ncols) {
    float t = ps[0][c];
    for (int q = 1; q < 16; ++q) t += ps[q][c];
    out[col] = t;
  }
}

namespace lmm {
constexpr int BM = 128, BN = 128, BK = 32, NT = 256;
constexpr int LDN = BK + 8;   // [m][k] A tile row: 80 bytes
constexpr int LDT = 128 + 16; // [k][m] A tile / [k][n] B tile row: 288 bytes
constexpr int A_ELEMS = BM * LDN > BK * LDT ? BM * LDN : BK * LDT;
constexpr int B_ELEMS = BK * LDT;
constexpr int BUF = 2 * A_ELEMS + B_ELEMS;  // A hi, A lo, B (bf16 elements)

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
// Transposing 8-byte LDS read (ds_read_b64_tr_b16): within each 16-lane
// group, lane i receives element (i & 3) of the 4-element vectors addressed by
// lanes 4k + (i >> 2), k = 0..3.
__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<__attribute__((address_space(3))) char*>(reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(bf16x4, v);
}
// Fragment of a tile stored [k][col] (row stride LDT): lane (li, g4) gets
// column col0 + li, k = 8 g4 .. 8 g4 + 7.
__device__ __forceinline__ bf16x8 frag_t(const bf16* tile, int col0, int li, int g4) {
  const bf16* p = tile + (8 * g4 + (li >> 2)) * LDT + col0 + 4 * (li & 3);
  const bf16x4 a = tr_read(p), b = tr_read(p + 4 * LDT);
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
constexpr uint32_t kOut = 0x80000000u;  // an offset past every buffer range used here
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, long long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ bf16x8 ld16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
}  // namespace lmm

struct MmArgs {
  const bf16* ah;  // A, hi part
  const bf16* al;  // A, lo part
  const bf16* b;
  float* c;
  long long lda, ldb, ldc;  // row strides (elements)
  long long M, N, K;        // valid extents
  long long Kpad, kper;     // K range walked (multiple of 32) and its share per split
  long long split_stride;   // C offset between splits (elements)
  int ntm, ntn, nsplit;
};

// C[split](m, n) = sum_{k in the split's range} (Ah(m, k) + Al(m, k)) B(k, n)
// on bf16 matrix cores with fp32 accumulation.  A is stored [m][k] (AT =
// false, element at a[m * lda + k]) or [k][m] (AT = true, a[k * lda + m]); B
// is stored [k][n] (b[k * ldb + n]).  Elements with m >= M, n >= N or k >= K
// read as zero.  Host preconditions: lda, ldb multiples of 8 and 16-byte
// aligned bases; N and ldc multiples of 4 and C 16-byte aligned (float4
// rows); AT = false needs the A rows zero-padded to lda >= K rounded up to
// 32; AT = true needs lda a multiple of 128 (whole m tiles in range).
// 256 threads, a 128 x 128 tile, waves in a 2 x 2 grid of 64 x 64; K steps of
// 32 through double-buffered LDS, each step's loads issued two steps ahead into
// one of two register sets, one barrier per step.  Workgroup ids are remapped so that
// consecutive tiles share an XCD (L2 reuse of A rows across n tiles and of B
// rows across m tiles).
template <bool AT>
__global__ void __launch_bounds__(lmm::NT, 2) lam_mm16_kernel(MmArgs g) {
  using namespace lmm;
  __shared__ __align__(16) bf16 sm[2 * BUF];
  const int nb = gridDim.x;  // a multiple of 8
  const int id = blockIdx.x;
  const int lt = (id & 7) * (nb >> 3) + (id >> 3);
  const int tiles = g.ntm * g.ntn;
  if (lt >= tiles * g.nsplit) return;
  const int split = lt / tiles, tt = lt - split * tiles;
  int tm, tn;
  if (AT) { tm = tt % g.ntm; tn = tt / g.ntm; }  // m tiles of one n tile adjacent: shared B rows
  else { tn = tt % g.ntn; tm = tt / g.ntn; }     // n tiles of one m tile adjacent: shared A rows
  const long long m0 = (long long)tm * BM, n0 = (long long)tn * BN;
  const long long kb = (long long)split * g.kper;
  const long long ke = min(g.Kpad, kb + g.kper);  // an empty range writes a zero tile
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int wm = w >> 1, wn = w & 1;

  // buffer resources: rows past the valid range read zero
  const long long krows = max(0LL, min(g.K, ke) - kb);
  __amdgpu_buffer_rsrc_t rah, ral;
  if (AT) {
    rah = rsrc(g.ah + kb * g.lda, krows * g.lda * 2);
    ral = rsrc(g.al + kb * g.lda, krows * g.lda * 2);
  } else {
    const long long mrows = max(0LL, min((long long)BM, g.M - m0));
    rah = rsrc(g.ah + m0 * g.lda, mrows * g.lda * 2);
    ral = rsrc(g.al + m0 * g.lda, mrows * g.lda * 2);
  }
  const __amdgpu_buffer_rsrc_t rb = rsrc(g.b + kb * g.ldb, krows * g.ldb * 2);

  // per-thread chunk coordinates (two 8-element chunks per operand part)
  uint32_t offa[2], offb[2];
  int lda_s[2], ldb_s[2];  // LDS element offsets
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int c = tid + 256 * i;
    if (AT) {
      const int kr = c >> 4, mc = c & 15;
      offa[i] = static_cast<uint32_t>((kr * g.lda + m0 + 8 * mc) * 2);
      lda_s[i] = kr * LDT + 8 * mc;
    } else {
      const int r = c >> 2, kc = c & 3;
      offa[i] = static_cast<uint32_t>((r * g.lda + 8 * kc) * 2);
      lda_s[i] = r * LDN + 8 * kc;
    }
    const int kr = c >> 4, nc = c & 15;
    offb[i] = n0 + 8 * nc < g.N ? static_cast<uint32_t>((kr * g.ldb + n0 + 8 * nc) * 2) : kOut;
    ldb_s[i] = kr * LDT + 8 * nc;
  }
  // one K step's operand chunks in registers; two sets alternate so the
  // loads run two steps ahead of the products
  struct Regs {
    bf16x8 ah[2], al[2], b[2];
  };
  auto load = [&](Regs& r, long long k0) {
    const long long dk = k0 - kb;  // rows (AT, B) or columns (A [m][k]) from the range start
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint32_t da = AT ? static_cast<uint32_t>(dk * g.lda * 2) : static_cast<uint32_t>(k0 * 2);
      r.ah[i] = ld16(rah, offa[i] + da);
      r.al[i] = ld16(ral, offa[i] + da);
      r.b[i] = ld16(rb, offb[i] == kOut ? kOut : offb[i] + static_cast<uint32_t>(dk * g.ldb * 2));
    }
  };
  auto stage = [&](const Regs& r, int buf) {
    bf16* base = sm + buf * BUF;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      *reinterpret_cast<bf16x8*>(base + lda_s[i]) = r.ah[i];
      *reinterpret_cast<bf16x8*>(base + A_ELEMS + lda_s[i]) = r.al[i];
      *reinterpret_cast<bf16x8*>(base + 2 * A_ELEMS + ldb_s[i]) = r.b[i];
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto products = [&](const bf16* base) {
    bf16x8 ah[4], al[4], bv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (AT) {
        ah[i] = frag_t(base, 64 * wm + 16 * i, li, g4);
        al[i] = frag_t(base + A_ELEMS, 64 * wm + 16 * i, li, g4);
      } else {
        ah[i] = *reinterpret_cast<const bf16x8*>(base + (64 * wm + 16 * i + li) * LDN + 8 * g4);
        al[i] = *reinterpret_cast<const bf16x8*>(base + A_ELEMS + (64 * wm + 16 * i + li) * LDN + 8 * g4);
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) bv[j] = frag_t(base + 2 * A_ELEMS, 64 * wn + 16 * j, li, g4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah[i], bv[j], acc[i][j], 0, 0, 0);
        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al[i], bv[j], acc[i][j], 0, 0, 0);
      }
  };
  Regs ra, rb2;
  if (kb < ke) {
    load(ra, kb);
    stage(ra, 0);
    if (kb + BK < ke) load(ra, kb + BK);
  }
  __syncthreads();
  for (long long k0 = kb; k0 < ke; k0 += 2 * BK) {
    // step k0 from LDS buffer 0 (registers ra hold step k0 + BK)
    if (k0 + 2 * BK < ke) load(rb2, k0 + 2 * BK);
    products(sm);
    if (k0 + BK < ke) stage(ra, 1);
    __syncthreads();
    if (k0 + BK >= ke) break;
    // step k0 + BK from LDS buffer 1 (registers rb2 hold step k0 + 2 BK)
    if (k0 + 3 * BK < ke) load(ra, k0 + 3 * BK);
    products(sm + BUF);
    if (k0 + 2 * BK < ke) stage(rb2, 0);
    __syncthreads();
  }

  // acc[i][j][r] = C(m0 + 64wm + 16i + 4g4 + r, n0 + 64wn + 16j + li).  The
  // wave's 64 x 64 block goes out through its own LDS region (the operand
  // buffers are free after the loop's last barrier), 32 rows at a time, so
  // each row leaves as one 256-byte piece of float4 stores instead of four
  // 64-byte pieces (partial lines cost full-line writes).
  float* C = g.c + split * g.split_stride;
  constexpr int LDO = 64 + 4;  // staging row stride (floats): 16-byte aligned rows
  float* stg = reinterpret_cast<float*>(sm) + w * (32 * LDO);
  const long long mw = m0 + 64 * wm, nw = n0 + 64 * wn;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) stg[(16 * ii + 4 * g4 + r) * LDO + 16 * j + li] = acc[2 * h + ii][j][r];
#pragma unroll
    for (int it = 0; it < 8; ++it) {
      const int row = 4 * it + (lane >> 4), c4 = 4 * (lane & 15);
      const long long m = mw + 32 * h + row, n = nw + c4;
      const f32x4 x = *reinterpret_cast<const f32x4*>(stg + row * LDO + c4);
      if (m < g.M && n < g.N) __builtin_nontemporal_store(x, reinterpret_cast<f32x4*>(C + m * g.ldc + n));
    }
  }
}

namespace {
int launch_gemm(int dtype_a, int dtype_b, const GemmArgs& g, int nsplit, hipStream_t s) {
  const long long nb = (long long)((g.N + lg::BN - 1) / lg::BN) * ((g.M + lg::BM - 1) / lg::BM) * nsplit;
  if (nb == 0) return LL_OK;
  if (nb > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  const dim3 grid(static_cast<unsigned>(nb));
  if (dtype_a == LL_F32 && dtype_b == LL_F32)
    hipLaunchKernelGGL((lam_gemm_kernel<float, float>), grid, dim3(lg::NT), 0, s, g);
  else if (dtype_a == LL_F32 && dtype_b == LL_BF16)
    hipLaunchKernelGGL(lam_gemm16_kernel, grid, dim3(lg16::NT), 0, s, g);
  else
    return LL_ERR_UNSUPPORTED;
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}
}  // namespace

int lambda_bwd_nsplit(long long rows, int HL, int D) {
  // enough (tile, split) workgroups to fill the chip, each split at least
  // eight K tiles long
  const long long tiles = (long long)((HL + lg::BM - 1) / lg::BM) * ((D + 1 + lg::BN - 1) / lg::BN);
  long long ns = (2048 + tiles - 1) / tiles;
  const long long maxs = (rows + 8 * lg::BK - 1) / (8 * lg::BK);
  if (ns > maxs) ns = maxs;
  if (ns < 1) ns = 1;
  if (ns > 64) ns = 64;
  return static_cast<int>(ns);
}

long long lambda_bwd_kper(long long rows, int nsplit) {
  const long long per = (rows + nsplit - 1) / nsplit;
  return (per + 63) / 64 * 64;  // whole K tiles of both product kernels
}

bool lambda_bwd16_plan(const LamBwdArgs& a, Lam16Plan* p) {
  const long long M = (long long)a.B * a.T;
  const long long HL = (long long)a.H * a.L;
  if (M <= 0 || a.D % 8 != 0) return false;
  if ((reinterpret_cast<uintptr_t>(a.x) | reinterpret_cast<uintptr_t>(a.W) | reinterpret_cast<uintptr_t>(a.dx)) & 15)
    return false;
  const long long HLp = (HL + 127) / 128 * 128;
  const long long ntm = (HL + 127) / 128, ntn = (a.D + 127) / 128;
  long long ns = (512 + ntm * ntn - 1) / (ntm * ntn);
  ns = std::min(ns, (M + 255) / 256);  // at least eight 32-row steps per split
  ns = std::max(1LL, std::min(ns, 64LL));
  long long kper = ((M + ns - 1) / ns + 31) / 32 * 32;
  ns = (M + kper - 1) / kper;
  // 32-bit buffer offsets: W, a split's rows of x and of dz, a tile's rows of dz
  const long long lim = 1LL << 31;
  if (HL * a.D * 2 >= lim || kper * a.D * 2 >= lim || kper * HLp * 2 >= lim || 128 * HLp * 2 >= lim) return false;
  p->HLp = static_cast<int>(HLp);
  p->nsplit = static_cast<int>(ns);
  p->kper = kper;
  p->ntb = (a.T + 63) / 64;
  p->dz_bytes = (size_t)M * HLp * 2;
  p->colsum_bytes = (size_t)a.B * p->ntb * HL * 4;
  p->part_bytes = (size_t)ns * HL * a.D * 4;
  return true;
}

static size_t up256(size_t x) { return (x + 255) / 256 * 256; }

size_t lambda_bwd16_workspace(const Lam16Plan& p) {
  return 2 * up256(p.dz_bytes) + up256(p.colsum_bytes) + up256(p.part_bytes);
}

int launch_lambda_bwd16(const LamBwdArgs& a, const Lam16Plan& p, void* ws, hipStream_t s) {
  char* w = static_cast<char*>(ws);
  bf16* dzh = reinterpret_cast<bf16*>(w);
  bf16* dzl = reinterpret_cast<bf16*>(w + up256(p.dz_bytes));
  float* colsum = reinterpret_cast<float*>(w + 2 * up256(p.dz_bytes));
  float* part = reinterpret_cast<float*>(w + 2 * up256(p.dz_bytes) + up256(p.colsum_bytes));
  const long long M = (long long)a.B * a.T;
  const int HL = a.H * a.L;
  hipLaunchKernelGGL(lam_dz16_kernel, dim3(static_cast<unsigned>((long long)a.B * a.H * p.ntb)), dim3(256), 0, s, a,
                     dzh, dzl, p.HLp, colsum);
  if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
  const int ntn = (a.D + 127) / 128;
  // dx = dz W: A = dz [M][HLp] (k contiguous), B = W [HL][D]
  {
    const long long Kpad = (HL + 31) / 32 * 32;
    MmArgs g{dzh, dzl, static_cast<const bf16*>(a.W), a.dx, p.HLp, a.D, a.D, M, a.D, HL, Kpad, Kpad, 0,
             static_cast<int>((M + 127) / 128), ntn, 1};
    const long long nb = ((long long)g.ntm * g.ntn + 7) / 8 * 8;
    if (nb > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(lam_mm16_kernel<false>, dim3(static_cast<unsigned>(nb)), dim3(lmm::NT), 0, s, g);
    if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
  }
  // dW partials: A(m = n, k = row) = dz[row][n] ([k][m]), B = x [M][D]
  {
    MmArgs g{dzh, dzl, static_cast<const bf16*>(a.x), part, p.HLp, a.D, a.D, HL, a.D, M, (M + 31) / 32 * 32,
             p.kper, (long long)HL * a.D, (HL + 127) / 128, ntn, p.nsplit};
    const long long nb = ((long long)g.ntm * g.ntn * g.nsplit + 7) / 8 * 8;
    if (nb > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(lam_mm16_kernel<true>, dim3(static_cast<unsigned>(nb)), dim3(lmm::NT), 0, s, g);
    if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
  }
  const long long count = (long long)HL * a.D;
  hipLaunchKernelGGL(lam_rowsum_kernel, dim3(static_cast<unsigned>(std::min<long long>((count + 255) / 256, 4096))),
                     dim3(256), 0, s, static_cast<const float*>(part), p.nsplit, count, count, a.dW);
  if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
  if (a.dbias) {
    hipLaunchKernelGGL(lam_colsum_kernel, dim3(static_cast<unsigned>((HL + 15) / 16)), dim3(256), 0, s,
                       static_cast<const float*>(colsum), a.B * p.ntb, (long long)HL, HL, a.dbias);
    if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
  }
  return LL_OK;
}

int launch_lambda_bwd(int dtype, const LamBwdArgs& a, float* part, int nsplit, hipStream_t s) {
  const long long M = (long long)a.B * a.T;
  const int HL = a.H * a.L;
  const long long stride = (long long)HL * (a.D + 1);
  if (M > 0) {
    const long long nb = (long long)a.B * a.H * ((a.T + 63) / 64);
    if (nb > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
    hipLaunchKernelGGL(lam_dz_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, a);
    if (hipGetLastError() != hipSuccess) return LL_ERR_HIP;
    // dx = dz W: A(m, k) = dz[m][k], B(k, n) = W[k][n]
    GemmArgs gx{a.dz, a.W, a.dx, HL, 1, a.D, 1, a.D, 0, static_cast<int>(M), a.D, HL, HL, a.D, 0};
    int st = launch_gemm(LL_F32, dtype, gx, 1, s);
    if (st != LL_OK) return st;
    // dW partials: A(m = n, k = row) = dz[row][n], B(k = row, col) = x[row][col],
    // column D of B is all ones (bias sums)
    const long long kper = lambda_bwd_kper(M, nsplit);
    GemmArgs gw{a.dz, a.x, part, 1, HL, a.D, 1, a.D + 1, stride, HL, a.D + 1, static_cast<int>(M),
                static_cast<int>(kper), a.D, 1};
    st = launch_gemm(LL_F32, dtype, gw, nsplit, s);
    if (st != LL_OK) return st;
  } else {
    nsplit = 0;
  }
  const long long total = (long long)HL * (a.D + 1);
  const long long blocks = std::min<long long>((total + 255) / 256, 4096);
  hipLaunchKernelGGL(lam_split_sum_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, s,
                     static_cast<const float*>(part), nsplit, stride, HL, a.D, a.dW, a.dbias);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
