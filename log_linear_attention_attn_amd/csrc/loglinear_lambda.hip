// Level weights from the hidden state, fused in one kernel:
//   lambda[b, h, t, l] = softplus(sum_d x[b, t, d] W[h*L + l, d] + bias[h*L + l])
// ([P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制",
// section 循环形式与输出计算: per-head linear map of the token's hidden
// representation, made non-negative; softplus is the reading of that map).
//
// A GEMM of the B*T rows of x against the H*L rows of W (both k-contiguous),
// with the bias, softplus and the [B, T, H*L] -> [B, H, T, L] reordering done
// on the accumulators before the only store, so no intermediate tensor goes
// through HBM.  bf16 inputs take the direct-to-LDS variant further down; the
// description here is that of the register-staged kernel fp32 inputs use.
// One 512-thread workgroup per (128 rows, 256 output columns);
// the eight waves form a 2 x 4 grid, wave w owning rows 64(w>>2)..+63 and
// columns 64(w&3)..+63 (4 x 4 tiles, 16 accumulators), so each staged x and W
// fragment is read from LDS by only 4 and 2 waves.
// The K loop stages 64-wide slices of x and W in LDS (row-major, padded rows);
// the global loads run three slices ahead (two for fp32) through a ring of
// registers, which covers the HBM latency a one-slice prefetch left exposed.
// x is read from HBM once per column block; the column blocks of one row
// block are launched on the same XCD so they share it through L2.
#include <hip/hip_runtime.h>

#include <atomic>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

namespace lp {
constexpr int BM = 128, NB = 256, NW = 8, NT = NW * 64;
template <typename IT>
struct Cfg {
  static constexpr int BK = sizeof(IT) == 2 ? 64 : 32;       // K slice (elements, 128 bytes)
  static constexpr int VEC = 16 / (int)sizeof(IT);           // elements per 16-byte load
  // padded LDS row: 144 bytes (36 banks), which puts the 16-byte fragment
  // reads of 16 consecutive rows on 16 disjoint groups of 4 banks
  static constexpr int LD = BK + (sizeof(IT) == 2 ? 8 : 4);
  static constexpr int XV = BM * BK / VEC / NT;               // x vectors per thread
  static constexpr int WV = NB * BK / VEC / NT;               // W vectors per thread
  static constexpr int NS = 2;                                // K slices in flight (register ring)
  // two LDS buffers (slice i in buffer i & 1), each x rows then W rows
  static constexpr int W_OFF = BM * LD * (int)sizeof(IT);
  static constexpr int BUF = W_OFF + NB * LD * (int)sizeof(IT);
  static constexpr int LDS = 2 * BUF;
};
// Raw buffer resource over [base, base + bytes): loads at offsets past the
// range return zero, so ragged rows, columns and K tails need no branches.
constexpr uint32_t kOutOfRange = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
}  // namespace lp

template <typename IT>
__global__ void __launch_bounds__(lp::NT) lambda_proj_kernel(LamProjArgs a) {
  using namespace lp;
  using Cf = Cfg<IT>;
  using F = Frag<IT>;
  using V = uint4;  // 16 bytes of IT
  extern __shared__ __align__(16) unsigned char smem[];

  // block id -> (row block, column block); the column blocks of a row block
  // share id % 8 (one XCD)
  const int ncb = a.ncb;
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int cb = rest % ncb, rb = (rest / ncb) * 8 + xcd;
  const long long M = (long long)a.B * a.T;
  const int N = a.H * a.L, D = a.D;
  const long long m0 = (long long)rb * BM;
  if (m0 >= M) return;
  const int n0 = cb * NB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  constexpr int BK = Cf::BK;
  // this block's rows of x and W (each below 2^31 bytes: at most 256 rows of
  // at most 2^20 elements, checked by the host)
  const long long mrows = min((long long)BM, M - m0);
  const int nrows = min(NB, N - n0);
  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const IT*>(a.x) + m0 * D, static_cast<uint32_t>(mrows * D * sizeof(IT)));
  const __amdgpu_buffer_rsrc_t wr_ =
      make_rsrc(static_cast<const IT*>(a.W) + (long long)n0 * D, static_cast<uint32_t>((long long)nrows * D * sizeof(IT)));

  constexpr int NS = Cf::NS;
  V rx[NS][Cf::XV], rw[NS][Cf::WV];
  // rows past the block's range fall outside the resource; columns past D
  // get an out-of-range offset (D is a multiple of the vector width)
  auto load = [&](V* rx, V* rw, int k0) {
    constexpr int VPR = BK / Cf::VEC;  // vectors per staged row
#pragma unroll
    for (int i = 0; i < Cf::XV; ++i) {
      const int v = tid + NT * i, r = v / VPR, c = (v % VPR) * Cf::VEC;
      const uint32_t off = k0 + c < D ? static_cast<uint32_t>((r * D + k0 + c) * sizeof(IT)) : kOutOfRange;
      rx[i] = __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(xr, off, 0, 0));
    }
#pragma unroll
    for (int i = 0; i < Cf::WV; ++i) {
      const int v = tid + NT * i, r = v / VPR, c = (v % VPR) * Cf::VEC;
      const uint32_t off = k0 + c < D ? static_cast<uint32_t>((r * D + k0 + c) * sizeof(IT)) : kOutOfRange;
      rw[i] = __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b128(wr_, off, 0, 0));
    }
  };
  auto stage = [&](const V* rx, const V* rw, int buf) {
    IT* Xs = reinterpret_cast<IT*>(smem + buf * Cf::BUF);
    IT* Ws = reinterpret_cast<IT*>(smem + buf * Cf::BUF + Cf::W_OFF);
    constexpr int VPR = BK / Cf::VEC;
#pragma unroll
    for (int i = 0; i < Cf::XV; ++i) {
      const int v = tid + NT * i, r = v / VPR, c = (v % VPR) * Cf::VEC;
      *reinterpret_cast<V*>(Xs + r * Cf::LD + c) = rx[i];
    }
#pragma unroll
    for (int i = 0; i < Cf::WV; ++i) {
      const int v = tid + NT * i, r = v / VPR, c = (v % VPR) * Cf::VEC;
      *reinterpret_cast<V*>(Ws + r * Cf::LD + c) = rw[i];
    }
  };

  const int wr = w >> 2, wc = w & 3;  // row half, column quarter
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ntile = min(NB, N - n0 + 15) / 16;  // column tiles holding real columns
  const int njt = min(4, ntile - 4 * wc);        // of this wave's four (may be <= 0)

  // K slices in a per-block rotated order: blocks running at the same time
  // read different slices of W (and of their x rows), so their requests do not
  // all land on the same L2 / HBM channels
  // Slices past the last one (the loop runs a multiple of NS of them) start
  // at D, so all their loads fall outside the resource and read zeros.
  const int nsl = (D + BK - 1) / BK;
  const int rot = static_cast<int>(rb % nsl);
  auto kof = [&](int i) {
    const int j = i + rot;
    return i >= nsl ? D : (j >= nsl ? j - nsl : j) * BK;
  };
  auto compute = [&](int buf) {
    if (njt <= 0) return;
    const IT* Xs = reinterpret_cast<const IT*>(smem + buf * Cf::BUF);
    const IT* Ws = reinterpret_cast<const IT*>(smem + buf * Cf::BUF + Cf::W_OFF);
#pragma unroll
    for (int kk = 0; kk < BK; kk += F::KS) {
      typename F::V af[4], bf[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) af[r] = F::load(Xs, Cf::LD, 64 * wr + 16 * r, kk, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = F::load(Ws, Cf::LD, 64 * wc + 16 * j, kk, lane);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < njt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r][j] = F::mma(af[r], bf[j], acc[r][j]);
        }
    }
  };
  // Pipeline: slice i is computed from LDS buffer i & 1 while slice i + 1 is
  // staged into the other buffer (last read in iteration i - 1, before the
  // barrier that ends it) and slice i + 1 + NS is loaded into the register
  // slot slice i + 1 vacated: one barrier per slice.  Every load and stage is
  // unconditional (slices past the end are zeros), so the count of loads in
  // flight is the same on every path and the wait for a slice's registers
  // leaves the later slices' loads outstanding.
#pragma unroll
  for (int s = 0; s < NS; ++s) load(rx[s], rw[s], kof(s));
  stage(rx[0], rw[0], 0);
  load(rx[0], rw[0], kof(NS));
  __syncthreads();
  static_assert(NS % 2 == 0, "slice i uses register slot i % NS and buffer i & 1");
  for (int ib = 0; ib < nsl; ib += NS) {
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int i = ib + s;
      compute(s & 1);
      const int sn = (s + 1) % NS;  // a constant once the loop is unrolled
      stage(rx[sn], rw[sn], (s + 1) & 1);
      load(rx[sn], rw[sn], kof(i + 1 + NS));
      __syncthreads();
    }
  }

  // epilogue: acc[i][j][r] = z(row 64wr + 16i + 4g4 + r, column n0 + 64wc + 16j + li).
  // Output offset = row part ((b*H*T + t) * L) + column part (h*T*L + l); the
  // rows of this lane are split into (b, t) once, with 32-bit divisions from
  // the block's first row.
  const long long TL = (long long)a.T * a.L;
  const long long b0 = m0 / a.T;
  const int t0 = static_cast<int>(m0 - b0 * a.T);
  long long rowoff[4][4];
  bool rowok[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ro = 64 * wr + 16 * i + 4 * g4 + r;
      const int q = (t0 + ro) / a.T;  // t0 + ro < T + BM
      const long long b = b0 + q;
      const int t = t0 + ro - q * a.T;
      rowoff[i][r] = (b * a.H * a.T + t) * a.L;
      rowok[i][r] = m0 + ro < M;
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 64 * wc + 16 * j + li;
    if (j >= njt || n >= N) continue;
    const float bn = a.bias ? a.bias[n] : 0.f;
    const int h = n / a.L, l = n - h * a.L;
    float* __restrict__ dst = a.lam + h * TL + l;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!rowok[i][r]) continue;
        const float z = acc[i][j][r] + bn;
        // softplus(z) = max(z, 0) + log(1 + e^(-|z|)): e^(-|z|) <= 1 never
        // overflows, and the absolute error of the hardware log near 1..2 is
        // ~1e-7
        dst[rowoff[i][r]] = fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
      }
  }
}

// bf16 variant staged by direct-to-LDS loads: each lane's 16-byte global
// load lands in LDS without passing through registers (no register staging,
// no LDS stores by the waves), three K slices are in flight (three static
// buffers, one barrier per slice), and rows of 64 k (128 bytes, unpadded)
// keep their eight 16-byte chunks in the order chunk ^ ((row >> 1) & 7),
// which spreads the 16 rows a fragment read touches over all 16 bank groups.
// Tile shapes, wave grid and epilogue as above.
namespace lpd {
constexpr int BM = 128, NB = 256, BK = 64, NT = 512;
constexpr int XT = BM * BK * 2;  // bytes of one x slice
constexpr int WT = NB * BK * 2;  // bytes of one W slice
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt immediate that waits until at most n vector-memory operations
// are outstanding (vmcnt in bits 3:0 and 15:14; expcnt, lgkmcnt not waited)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }
// barrier for LDS hand-over only: the waits for the direct-to-LDS loads are
// explicit, so the barrier itself does not drain the loads still in flight
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
typedef __attribute__((address_space(3))) void lds_void;
}  // namespace lpd

__global__ void __launch_bounds__(lpd::NT) lambda_proj_dma_kernel(LamProjArgs a) {
  using namespace lpd;
  __shared__ __align__(16) unsigned char xs0[XT], xs1[XT], xs2[XT], ws0[WT], ws1[WT], ws2[WT];
  const int ncb = a.ncb;
  const int id = blockIdx.x;
  const int xcd = id & 7, rest = id >> 3;
  const int cb = rest % ncb, rb = (rest / ncb) * 8 + xcd;
  const long long M = (long long)a.B * a.T;
  const int N = a.H * a.L, D = a.D;
  const long long m0 = (long long)rb * BM;
  if (m0 >= M) return;
  const int n0 = cb * NB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform, so tile branches stay scalar
  const int li = lane & 15, g4 = lane >> 4;
  const long long mrows = min((long long)BM, M - m0);
  const int nrows = min(NB, N - n0);
  const __amdgpu_buffer_rsrc_t xr =
      lp::make_rsrc(static_cast<const bf16*>(a.x) + m0 * D, static_cast<uint32_t>(mrows * D * 2));
  const __amdgpu_buffer_rsrc_t wr_ =
      lp::make_rsrc(static_cast<const bf16*>(a.W) + (long long)n0 * D, static_cast<uint32_t>((long long)nrows * D * 2));

  // this lane's chunk of each 1 KB block (8 rows) it fills: blocks 2w, 2w+1
  // of the x slice and 4w..4w+3 of the W slice; rows past the block's range
  // fall outside the resources
  uint32_t xo[2], wo[4];
  int xc[2], wc8[4];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = (2 * w + j) * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    xo[j] = static_cast<uint32_t>(row * D * 2 + c * 16);
    xc[j] = c * 8;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int row = (4 * w + j) * 8 + (lane >> 3), c = (lane & 7) ^ swz(row);
    wo[j] = static_cast<uint32_t>(row * D * 2 + c * 16);
    wc8[j] = c * 8;
  }
  // K slices in a per-block rotated order (as above); slices past the last
  // one start at D, so all their loads fall outside the resources
  const int nsl = (D + BK - 1) / BK;
  const int rot = static_cast<int>(rb % nsl);
  auto kof = [&](int i) {
    const int j = i + rot;
    return i >= nsl ? D : (j >= nsl ? j - nsl : j) * BK;
  };
  auto issue = [&](unsigned char* xb, unsigned char* wb, int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void*)(xb + (2 * w + j) * 1024), 16,
                                               k0 + xc[j] < D ? xo[j] + k0 * 2 : lp::kOutOfRange, 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(wr_, (lds_void*)(wb + (4 * w + j) * 1024), 16,
                                               k0 + wc8[j] < D ? wo[j] + k0 * 2 : lp::kOutOfRange, 0, 0, 0);
  };

  const int wr = w >> 2, wc = w & 3;  // row half, column quarter
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int ntile = min(NB, N - n0 + 15) / 16;
  const int njt = min(4, ntile - 4 * wc);
  auto frag = [&](const unsigned char* base, int row, int c) {
    return *reinterpret_cast<const bf16x8*>(base + row * 128 + ((c ^ swz(row)) << 4));
  };
  auto compute = [&](const unsigned char* xb, const unsigned char* wb) {
    if (njt <= 0) return;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) af[r] = frag(xb, 64 * wr + 16 * r + li, 4 * kk + g4);
#pragma unroll
      for (int j = 0; j < 4; ++j) bf[j] = frag(wb, 64 * wc + 16 * j + li, 4 * kk + g4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (j < njt) {
#pragma unroll
          for (int r = 0; r < 4; ++r) acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[r], bf[j], acc[r][j], 0, 0, 0);
        }
    }
  };
  // slice i sits in buffer i % 3; before computing it, this thread's six
  // loads of slice i are waited for (those of slice i + 1 stay in flight) and
  // the barrier makes everyone's visible and frees buffer (i + 2) % 3, which
  // then receives slice i + 2.  The scheduling barriers keep the compiler from
  // moving the direct-to-LDS loads across the barrier or into the products.
  issue(xs0, ws0, kof(0));
  issue(xs1, ws1, kof(1));
  for (int ib = 0; ib < nsl; ib += 3) {
    __builtin_amdgcn_s_waitcnt(wait_vm(6));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(xs2, ws2, kof(ib + 2));
    __builtin_amdgcn_sched_barrier(0);
    compute(xs0, ws0);
    __builtin_amdgcn_s_waitcnt(wait_vm(6));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(xs0, ws0, kof(ib + 3));
    __builtin_amdgcn_sched_barrier(0);
    compute(xs1, ws1);
    __builtin_amdgcn_s_waitcnt(wait_vm(6));
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
    issue(xs1, ws1, kof(ib + 4));
    __builtin_amdgcn_sched_barrier(0);
    compute(xs2, ws2);
  }
  // the loads issued past the end (zeros) land before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  const long long TL = (long long)a.T * a.L;
  const long long b0 = m0 / a.T;
  const int t0 = static_cast<int>(m0 - b0 * a.T);
  long long rowoff[4][4];
  bool rowok[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int ro = 64 * wr + 16 * i + 4 * g4 + r;
      const int q = (t0 + ro) / a.T;
      const long long b = b0 + q;
      const int t = t0 + ro - q * a.T;
      rowoff[i][r] = (b * a.H * a.T + t) * a.L;
      rowok[i][r] = m0 + ro < M;
    }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = n0 + 64 * wc + 16 * j + li;
    if (j >= njt || n >= N) continue;
    const float bn = a.bias ? a.bias[n] : 0.f;
    const int h = n / a.L, l = n - h * a.L;
    float* __restrict__ dst = a.lam + h * TL + l;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (!rowok[i][r]) continue;
        const float z = acc[i][j][r] + bn;
        dst[rowoff[i][r]] = fmaxf(z, 0.f) + __logf(1.f + __expf(-fabsf(z)));
      }
  }
}

int lambda_proj_lds_bytes(int dtype) {
  return dtype == LL_BF16 ? 3 * (lpd::XT + lpd::WT) : lp::Cfg<float>::LDS;
}

int launch_lambda_proj(int dtype, const LamProjArgs& a, hipStream_t s) {
  const long long M = (long long)a.B * a.T;
  const long long nrb = (M + lp::BM - 1) / lp::BM;
  const long long nblocks = (nrb + 7) / 8 * 8 * a.ncb;
  if (nblocks > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  if (dtype == LL_BF16) {
    // static LDS only
    hipLaunchKernelGGL(lambda_proj_dma_kernel, dim3(static_cast<unsigned>(nblocks)), dim3(lpd::NT), 0, s, a);
  } else {
    static std::atomic<uint64_t> lds_raised{0};
    const int lds = lambda_proj_lds_bytes(dtype);
    if (!raise_lds_limit(reinterpret_cast<const void*>(&lambda_proj_kernel<float>), lds_raised, lds))
      return LL_ERR_HIP;
    hipLaunchKernelGGL(lambda_proj_kernel<float>, dim3(static_cast<unsigned>(nblocks)), dim3(lp::NT), lds, s, a);
  }
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
