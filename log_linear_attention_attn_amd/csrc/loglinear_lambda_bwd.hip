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
// Three kernels: dz into a [B*T, H*L] fp32 scratch matrix; a tiled
// matrix-core product used for both products (fp32 MFMAs for fp32 inputs;
// for bf16 x and W, bf16 MFMAs on dz split into bf16 hi + lo), dW split over
// row ranges of B*T into partial sums with dbias as one extra column of ones
// on the x side; and an in-order sum of the partials.  No atomics, so results are
// deterministic.
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
