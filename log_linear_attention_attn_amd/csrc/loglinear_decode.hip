// O(log T) decode step of log-linear attention on gfx950.
//
// [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制",
//      section 解码：基于 lssb 的状态更新; [P5] "論文紹介：Log Linear Attention", slide 21.
//
// Per (sequence, head) the states S^l (k-major, dk x dv fp32) advance from
// t-1 to t with m = lssb(t):
//   S^{m+1} <- a_t (S^0 + ... + S^m),  S^{1..m} <- 0,
//   S^l <- a_t S^l for the live levels l > m+1,  S^0 <- k_t v_t^T,
// and o_t = sum_l lambda_t^l q_t^T S_t^l.  The work is a stream over the live
// levels (HBM bound): one workgroup per (sequence*head, 64-column dv tile);
// 16 row groups x 16 lanes of float4 give 256-byte contiguous row segments.
#include <hip/hip_runtime.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

// All loads of a row's live levels are issued before any of its stores (the
// level loop is unrolled to LMAX >= L with wave-uniform predicates), so each
// thread keeps up to L loads in flight.  Each state element is read and written
// once per step, so the state traffic uses non-temporal loads and stores
// (streaming hint: +8% measured).
template <typename IT, int LMAX>
__global__ void __launch_bounds__(256) decode_kernel(DecArgs a) {
  __shared__ f32x4 red[16][16];
  const int nh = blockIdx.x;
  const int seq = nh / a.H;
  const int tid = threadIdx.x, c = tid & 15, rg = tid >> 4;
  const int col = blockIdx.y * 64 + 4 * c;
  const bool colok = col < a.dv;  // dv is a multiple of 4
  const int L = a.L, dk = a.dk, dv = a.dv;
  const int t = a.t[seq];
  float* __restrict__ outp = a.out + (size_t)nh * dv + col;
  if (t < 0 || t >= (1 << (L - 1))) {
    if (rg == 0 && colok) {
      const float nan = __builtin_nanf("");
      *reinterpret_cast<f32x4*>(outp) = f32x4{nan, nan, nan, nan};
    }
    return;
  }
  const float at = __expf(a.log_a[nh]);
  const float* __restrict__ lam = a.lam + (size_t)nh * L;
  const IT* __restrict__ q = static_cast<const IT*>(a.q) + (size_t)(nh / a.G) * dk;
  const IT* __restrict__ k = static_cast<const IT*>(a.k) + (size_t)(nh / a.G) * dk;
  const IT* __restrict__ v = static_cast<const IT*>(a.v) + (size_t)nh * dv;
  float* __restrict__ S = a.S + (size_t)nh * L * dk * dv + col;
  const size_t lvl = (size_t)dk * dv;
  const int m = t ? lssb(static_cast<uint32_t>(t)) : -1;
  // levels holding state at t-1: level 0 and level b+1 for each set bit b of
  // t-1 (that is 0..m, and the levels above m+1 that t keeps)
  const unsigned live = t ? (1u | (static_cast<unsigned>(t - 1) << 1)) : 0u;

  f32x4 o = {0.f, 0.f, 0.f, 0.f};
  if (colok) {
    f32x4 vv;
#pragma unroll
    for (int i = 0; i < 4; ++i) vv[i] = static_cast<float>(v[col + i]);
    // output weight of each level's new state: lambda (level m+1 holds the
    // merge, the kept levels above it are decayed copies, 1..m are cleared)
    float wl[LMAX];
#pragma unroll
    for (int l = 0; l < LMAX; ++l)
      wl[l] = (l < L && l > m && ((live >> l) & 1 || l == m + 1)) ? lam[l] : 0.f;
    const float lam0 = lam[0];
    for (int r = rg; r < dk; r += 16) {
      const float qr = static_cast<float>(q[r]);
      const float kr = static_cast<float>(k[r]);
      float* __restrict__ Sr = S + (size_t)r * dv;
      f32x4 x[LMAX];
#pragma unroll
      for (int l = 0; l < LMAX; ++l) {
        x[l] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (l < L && ((live >> l) & 1)) x[l] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(Sr + l * lvl));
      }
      // merge of levels 0..m into level m+1, decayed by a_t
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int l = 0; l < LMAX; ++l)
        if (l <= m) acc += x[l];
      acc *= at;
      f32x4 ol = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int l = 1; l < LMAX; ++l) {
        if (l < L) {
          f32x4 y;
          if (l <= m || t == 0) y = f32x4{0.f, 0.f, 0.f, 0.f};  // cleared (t = 0: every level)
          else if (l == m + 1) y = acc;
          else y = x[l] * at;  // kept (zero stays zero for dead levels)
          if (t == 0 || l <= m + 1 || ((live >> l) & 1)) __builtin_nontemporal_store(y, reinterpret_cast<f32x4*>(Sr + l * lvl));
          ol += wl[l] * y;
        }
      }
      const f32x4 s0 = kr * vv;
      __builtin_nontemporal_store(s0, reinterpret_cast<f32x4*>(Sr));
      o += qr * (ol + lam0 * s0);
    }
  }
  red[rg][c] = o;
  __syncthreads();
  if (rg == 0 && colok) {
    f32x4 sum = red[0][c];
#pragma unroll
    for (int i = 1; i < 16; ++i) sum += red[i][c];
    *reinterpret_cast<f32x4*>(outp) = sum;
  }
}

int launch_decode(int dtype, const DecArgs& a, hipStream_t s) {
  const dim3 grid(a.N * a.H, (a.dv + 63) / 64);
  if (a.L > 31) return LL_ERR_UNSUPPORTED;
  const bool small = a.L <= 17;
  if (dtype == LL_BF16) {
    if (small) hipLaunchKernelGGL((decode_kernel<bf16, 17>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<bf16, 31>), grid, dim3(256), 0, s, a);
  } else {
    if (small) hipLaunchKernelGGL((decode_kernel<float, 17>), grid, dim3(256), 0, s, a);
    else hipLaunchKernelGGL((decode_kernel<float, 31>), grid, dim3(256), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
