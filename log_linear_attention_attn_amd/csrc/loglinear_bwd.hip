// Backward of the log-linear attention forward: gradients of sum(out * dout)
// with respect to q, k, v, log_a and lambda.
//
//   [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
//        sections 并行形式 (O = (QK^T ⊙ M^H) V), 与已有模型的组合 (⊙ M^S),
//        训练：分块并行扫描算法 (chunk decomposition).
//
// With M[t,s] = lambda[t, l(t,s)] exp(cum_t - cum_s) for s <= t:
//   dQ_t      = sum_{s<=t} M[t,s] (dO_t . v_s) k_s
//   dK_s      = sum_{t>=s} M[t,s] (dO_t . v_s) q_t
//   dV_s      = sum_{t>=s} M[t,s] (q_t . k_s) dO_t
//   dlam[t,l] = sum_{s in bucket l of t} exp(cum_t - cum_s) (q_t . k_s)(dO_t . v_s)
//   dlog_a[r] = sum_{t>=r} (dO_t . O_t - v_t . dV_t)
// (the decay of token r sits in exactly the pairs s < r <= t, whose row sums
// of dM ⊙ M are dO_t . O_t and column sums v_s . dV_s).
//
// Chunkwise, as the forward: pairs inside one C-token chunk (levels
// <= log2 C) densely, and for chunk-level bit b the pairs between the left and
// the right half of each aligned block of 2^(b+1) chunks (level log2C+1+b).
// Unlike the forward's lssb merge, every level keeps its own state here,
// because the backward's query-side states carry lambda of their level:
//   bwd_dq_kernel   forward chunk order; per level the decayed left-half sum
//                   St_b = sum v_s k_s^T, read by the right-half queries:
//                   dQ, and the inter-chunk dlam as per-slice partial sums.
//   bwd_kv_kernel   reverse chunk order; per level the right-half sum
//                   R_b = sum lambda[t,l_b] w_t a_t c_t^T, read by the
//                   left-half keys: dV (a = dO, c = q, x = k) or
//                   dK (a = q, c = dO, x = v), y_s = sum R_b x_s.
//   bwd_dlam_intra_kernel  dlam of the in-chunk levels.
//   bwd_dlam_inter_kernel  dlam of the chunk levels from the partials.
//   bwd_dcum_kernel, bwd_dlog_a_kernel  dlog_a.
//   bwd_dlam_rows_kernel, bwd_dlog_a_blk_kernel  with the reverse
//                   register-state sweeps (whose dV sweep writes per-row
//                   records of the in-chunk dlam and of v . dV): all of
//                   dlam and dc in one pass, then dlog_a as a scan over
//                   (b,h, 1024-row) workgroups.
// Each output row slice of 16 columns belongs to one workgroup (no atomics).
// All products run as fp32 matrix-core instructions (v_mfma_f32_16x16x4f32);
// bf16 inputs are widened when staged.
#include <hip/hip_runtime.h>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {
namespace bwd {

using F = Frag<float>;

template <int C>
struct Lg;
template <>
struct Lg<16> { static constexpr int v = 4; };
template <>
struct Lg<32> { static constexpr int v = 5; };
template <>
struct Lg<64> { static constexpr int v = 6; };

__host__ __device__ constexpr int al16(int x) { return (x + 15) & ~15; }

template <typename IT>
__device__ __forceinline__ float ldf(const IT* p) { return static_cast<float>(*p); }

// four consecutive elements (16 bytes of fp32, 8 of bf16) as one access
template <typename T>
struct Vec4;
template <>
struct Vec4<float> { typedef f32x4 type; };
template <>
struct Vec4<bf16> { typedef bf16x4 type; };
template <typename T>
__device__ __forceinline__ void copy4(T* dst, const T* src, bool ok) {
  typedef typename Vec4<T>::type V;
  *reinterpret_cast<V*>(dst) = ok ? *reinterpret_cast<const V*>(src) : V{};
}

// sum over the 16 lanes of each row (DPP rotations and quad swaps)
template <int CTRL>
__device__ __forceinline__ float dpp_sum(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
__device__ __forceinline__ float row_sum16(float x) {
  x = dpp_sum<0x128>(x);  // row_ror:8
  x = dpp_sum<0x124>(x);  // row_ror:4
  x = dpp_sum<0x4e>(x);   // quad_perm [2,3,0,1]
  x = dpp_sum<0xb1>(x);   // quad_perm [1,0,3,2]
  return x;
}

// Separation after a chain of fp32 matrix-core instructions whose result is
// read past a branch: the scheduling barrier keeps the MFMAs above the nops,
// which cover the read-after-write distance on every path.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 3");
  __builtin_amdgcn_sched_barrier(0);
}

// In-chunk decay sums of chunk n for one wave: lane i -> cl_i (inclusive
// prefix of log_a over the chunk; tokens past T count 0), and the chunk total.
// Kept in fp64 so that the differences cl_t - cl_s the masks exponentiate
// carry no cancellation error from the large prefix values.
template <int C>
__device__ __forceinline__ double chunk_prefix(const float* lag, int tok0, int T, int lane, double* total) {
  double la = (lane < C && tok0 + lane < T) ? (double)lag[tok0 + lane] : 0.0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(la, off);
    if (lane >= off) la += y;
  }
  *total = __shfl(la, C - 1);
  return la;
}

// ---------------------------------------------------------------------------
// bwd_dq_kernel: one workgroup per (b,h, 16-column slice js of dk).
// ---------------------------------------------------------------------------
template <typename IT, int C>
struct DqCfg {
  static constexpr int NW = C / 16, NT = NW * 64;
  __host__ __device__ static int ldd(int dv) { return dv + 4; }           // dO rows, states (fp32)
  __host__ __device__ static int ldv(int dv) { return dv + (sizeof(IT) == 2 ? 8 : 4); }
  static constexpr int LDKT = C + 4;                                       // K slice transposed [16][C]
  static constexpr int LDQ = 17;                                           // Q slice [C][16]
  __host__ __device__ static int off_v(int dv) { return al16(C * ldd(dv) * 4); }
  __host__ __device__ static int off_kt(int dv) { return off_v(dv) + al16(C * ldv(dv) * (int)sizeof(IT)); }
  __host__ __device__ static int off_q(int dv) { return off_kt(dv) + al16(16 * LDKT * 4); }
  __host__ __device__ static int off_lam(int dv) { return off_q(dv) + al16(C * LDQ * 4); }
  __host__ __device__ static int off_cl(int dv, int L) { return off_lam(dv) + al16(C * L * 4); }
  __host__ __device__ static int off_dl(int dv, int L) { return off_cl(dv, L) + al16(2 * C * 8); }
  __host__ __device__ static int off_st(int dv, int L) { return off_dl(dv, L) + 16 * 4; }
  __host__ __device__ static int bytes(int dv, int L, int nslot) {
    return off_st(dv, L) + (nslot > 0 ? nslot : 1) * 16 * ldd(dv) * 4;
  }
};

template <typename IT, int C>
__global__ void __launch_bounds__(C / 16 * 64) bwd_dq_kernel(BwdArgs a) {
  using Cfg = DqCfg<IT, C>;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, LOGC = Lg<C>::v, LDKT = Cfg::LDKT, LDQ = Cfg::LDQ;
  extern __shared__ __align__(16) unsigned char smem[];
  const int dk = a.dk, dv = a.dv, T = a.T, L = a.L, nslot = a.nslot;
  const int LDD = Cfg::ldd(dv), LDV = Cfg::ldv(dv);
  float* dOs = reinterpret_cast<float*>(smem);
  IT* Vs = reinterpret_cast<IT*>(smem + Cfg::off_v(dv));
  float* KT = reinterpret_cast<float*>(smem + Cfg::off_kt(dv));
  float* Qs = reinterpret_cast<float*>(smem + Cfg::off_q(dv));
  float* lam_s = reinterpret_cast<float*>(smem + Cfg::off_lam(dv));
  double* cl_s = reinterpret_cast<double*>(smem + Cfg::off_cl(dv, L));  // in-chunk prefix of log_a
  float* esf_s = reinterpret_cast<float*>(cl_s + C);                      // decay to the chunk end
  float* dlt_s = reinterpret_cast<float*>(smem + Cfg::off_dl(dv, L));  // per level, see below
  float* St = reinterpret_cast<float*>(smem + Cfg::off_st(dv, L));

  const int nsl = dk / 16;
  const int bh = blockIdx.x / nsl, js = blockIdx.x - bh * nsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int N = (T + C - 1) / C;
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const IT* __restrict__ qg = static_cast<const IT*>(a.q) + qkT * dk + 16 * js;
  const IT* __restrict__ kg = static_cast<const IT*>(a.k) + qkT * dk + 16 * js;
  const IT* __restrict__ vg = static_cast<const IT*>(a.v) + bhT * dv;
  const float* __restrict__ dog = a.dout + bhT * dv;
  const float* __restrict__ lag = a.log_a + bhT;
  const float* __restrict__ lamg = a.lam + bhT * L;
  float* __restrict__ dqg = a.dq + bhT * dk + 16 * js;
  float* __restrict__ part = a.dlam_part + ((size_t)js * a.BH + bh) * T * (nslot > 0 ? nslot : 1);

  // dlt_s[b]: for a level whose right half holds this chunk, the log decay
  // from the level's reference (the last token of the left half) to the token
  // before this chunk; kept by thread 0, read after the staging barrier.
  float Aprev = 0.f;
  for (int n = 0; n < N; ++n) {
    const int tok0 = n * C;
    double Atd;
    const double cl = chunk_prefix<C>(lag, tok0, T, lane, &Atd);
    const float Atot = static_cast<float>(Atd);
    if (tid == 0)
      for (int b = 0; b < nslot; ++b)
        if ((n >> b) & 1) {
          const int rs = ((n >> (b + 1)) << (b + 1)) + (1 << b);
          dlt_s[b] = n == rs ? 0.f : dlt_s[b] + Aprev;
        }
    // ---- stage the chunk
    for (int i = tid; i < C * (dv / 4); i += NT) {
      const int r = i / (dv / 4), c = (i - r * (dv / 4)) * 4;
      const bool ok = tok0 + r < T;
      copy4(dOs + r * LDD + c, dog + (size_t)(tok0 + r) * dv + c, ok);
      copy4(Vs + r * LDV + c, vg + (size_t)(tok0 + r) * dv + c, ok);
    }
    for (int i = tid; i < C * 16; i += NT) {
      const int r = i >> 4, c = i & 15;
      const bool ok = tok0 + r < T && 16 * js + c < dk;
      KT[c * LDKT + r] = ok ? ldf(kg + (size_t)(tok0 + r) * dk + c) : 0.f;
      Qs[r * LDQ + c] = ok ? ldf(qg + (size_t)(tok0 + r) * dk + c) : 0.f;
    }
    for (int i = tid; i < C * L; i += NT) lam_s[i] = tok0 + i / L < T ? lamg[(size_t)tok0 * L + i] : 0.f;
    if (w == 0 && lane < C) {
      cl_s[lane] = cl;
      esf_s[lane] = __expf(static_cast<float>(Atd - cl));
    }
    __syncthreads();

    // ---- intra chunk: dQ rows 16w.. from the masked S^T tiles (dO . v)
    const int tq = 16 * w + li;  // query of this lane in the S^T tiles
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    for (int kb = 0; kb <= w; ++kb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      #pragma unroll 8
      for (int k0 = 0; k0 < dv; k0 += 4) {
        const float av = static_cast<float>(Vs[(16 * kb + li) * LDV + k0 + g4]);
        acc = F::mma(av, dOs[(16 * w + li) * LDD + k0 + g4], acc);
      }
      // acc[r] = dO_tq . v_s with s = 16kb + 4g4 + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * kb + 4 * g4 + r;
        const float p =
            s <= tq ? acc[r] * lam_s[tq * L + level_of(tq, s)] * __expf(static_cast<float>(cl_s[tq] - cl_s[s])) : 0.f;
        O = F::mma(p, KT[li * LDKT + s], O);
      }
    }
    mfma_drain();
    // ---- inter chunk: one level per set bit b of n (right half of its block)
    for (int b = 0; b < nslot; ++b) {
      const bool right = (n >> b) & 1;
      float x[4] = {0.f, 0.f, 0.f, 0.f};
      if (right) {
        const float* stb = St + b * 16 * LDD;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll 8
        for (int k0 = 0; k0 < dv; k0 += 4) acc = F::mma(F::load(dOs, LDD, 16 * w, k0, lane), stb[li * LDD + k0 + g4], acc);
        mfma_drain();
        // acc[r] = (dO_t St_b)[j = li], t = 16w + 4g4 + r
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * w + 4 * g4 + r;
          const float wt = __expf(static_cast<float>(cl_s[t] + dlt_s[b])) * acc[r];
          O[r] += lam_s[t * L + LOGC + 1 + b] * wt;
          x[r] = wt * Qs[t * LDQ + li];
        }
      }
      // partial dlam of this slice (0 where the level has no bucket)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sx = row_sum16(x[r]);
        const int t = tok0 + 16 * w + 4 * g4 + r;
        if (li == 0 && t < T) part[(size_t)t * nslot + b] = sx;
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = tok0 + 16 * w + 4 * g4 + r;
      if (t < T) dqg[(size_t)t * dk + li] = O[r];
    }
    // ---- key side: this chunk joins the left half of every level whose bit
    // is clear and whose right half exists.  Disjoint from the levels read above.
    for (int it = w; it < dv / 16; it += NW) {
      const int i0 = 16 * it;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      #pragma unroll 8
      for (int k0 = 0; k0 < C; k0 += 4) {
        const int s = k0 + g4;
        acc = F::mma(KT[li * LDKT + s], esf_s[s] * static_cast<float>(Vs[s * LDV + i0 + li]), acc);
      }
      mfma_drain();
      // acc[r] = sum_s K[s][j] esf_s V[s][i], j = 4g4 + r, i = i0 + li
      for (int b = 0; b < nslot; ++b) {
        const int base = (n >> (b + 1)) << (b + 1);
        if (((n >> b) & 1) || base + (1 << b) >= N) continue;
        float* stb = St + b * 16 * LDD;
        const float f = n == base ? 0.f : __expf(Atot);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* p = stb + (4 * g4 + r) * LDD + i0 + li;
          *p = (n == base ? 0.f : *p * f) + acc[r];
        }
      }
    }
    Aprev = Atot;
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bwd_kv_kernel: y_s = sum_{t>=s} M[t,s] (c_t . x_s) a_t, one workgroup per
// (b,h, 16-column slice js of a).  MODE 0: dV (a = dO, c = q, x = k);
// MODE 1: dK (a = q, c = dO, x = v).  Reverse chunk order.
// ---------------------------------------------------------------------------
template <typename IT, int C, int MODE>
struct KvCfg {
  static constexpr int NW = C / 16, NT = NW * 64;
  typedef typename std::conditional<MODE == 0, IT, float>::type CT;  // c: q (MODE 0) or dO
  __host__ __device__ static int ldc(int dc) { return dc + (sizeof(CT) == 2 ? 8 : 4); }
  __host__ __device__ static int ldx(int dc) { return dc + (sizeof(IT) == 2 ? 8 : 4); }
  __host__ __device__ static int ldr(int dc) { return dc + 4; }
  static constexpr int LDAT = C + 4;  // a slice transposed [16][C]
  __host__ __device__ static int off_x(int dc) { return al16(C * ldc(dc) * (int)sizeof(CT)); }
  __host__ __device__ static int off_at(int dc) { return off_x(dc) + al16(C * ldx(dc) * (int)sizeof(IT)); }
  __host__ __device__ static int off_lam(int dc) { return off_at(dc) + al16(16 * LDAT * 4); }
  __host__ __device__ static int off_cl(int dc, int L) { return off_lam(dc) + al16(C * L * 4); }
  __host__ __device__ static int off_tot(int dc, int L) { return off_cl(dc, L) + al16(C * 8); }
  __host__ __device__ static int off_dl(int dc, int L, int N) { return off_tot(dc, L) + al16(N * 4); }
  __host__ __device__ static int off_r(int dc, int L, int N) { return off_dl(dc, L, N) + 2 * 16 * 4; }
  __host__ __device__ static int bytes(int dc, int L, int N, int nslot) {
    return off_r(dc, L, N) + (nslot > 0 ? nslot : 1) * 16 * ldr(dc) * 4;
  }
};

template <typename IT, int C, int MODE>
__global__ void __launch_bounds__(C / 16 * 64) bwd_kv_kernel(BwdArgs a) {
  using Cfg = KvCfg<IT, C, MODE>;
  using CT = typename Cfg::CT;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, LOGC = Lg<C>::v, LDAT = Cfg::LDAT;
  extern __shared__ __align__(16) unsigned char smem[];
  const int T = a.T, L = a.L, nslot = a.nslot;
  const int da = MODE == 0 ? a.dv : a.dk;  // columns of a (and of the output)
  const int dc = MODE == 0 ? a.dk : a.dv;  // contraction dim of c and x
  const int LDC = Cfg::ldc(dc), LDX = Cfg::ldx(dc), LDR = Cfg::ldr(dc);
  const int N = (T + C - 1) / C;
  CT* Cs = reinterpret_cast<CT*>(smem);
  IT* Xs = reinterpret_cast<IT*>(smem + Cfg::off_x(dc));
  float* AT = reinterpret_cast<float*>(smem + Cfg::off_at(dc));
  float* lam_s = reinterpret_cast<float*>(smem + Cfg::off_lam(dc));
  double* cl_s = reinterpret_cast<double*>(smem + Cfg::off_cl(dc, L));
  float* tot_s = reinterpret_cast<float*>(smem + Cfg::off_tot(dc, L));
  float* dlt_s = reinterpret_cast<float*>(smem + Cfg::off_dl(dc, L, N));
  float* gam_s = dlt_s + 16;
  float* R = reinterpret_cast<float*>(smem + Cfg::off_r(dc, L, N));

  const int nsl = da / 16;
  const int bh = blockIdx.x / nsl, js = blockIdx.x - bh * nsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const CT* __restrict__ cg = MODE == 0 ? reinterpret_cast<const CT*>(static_cast<const IT*>(a.q) + qkT * dc)
                                        : reinterpret_cast<const CT*>(a.dout + bhT * dc);
  const IT* __restrict__ xg = static_cast<const IT*>(MODE == 0 ? a.k : a.v) + (MODE == 0 ? qkT : bhT) * dc;
  const float* __restrict__ lag = a.log_a + bhT;
  const float* __restrict__ lamg = a.lam + bhT * L;
  float* __restrict__ yg = (MODE == 0 ? a.dvo : a.dk_out) + bhT * da + 16 * js;

  // chunk totals of log_a, every chunk (reverse-order decay bookkeeping)
  for (int nn = w; nn < N; nn += NW) {
    double tot;
    chunk_prefix<C>(lag, nn * C, T, lane, &tot);
    if (lane == 0) tot_s[nn] = static_cast<float>(tot);
  }
  __syncthreads();

  // Per level, kept by thread 0 and read after the staging barrier:
  //   dlt_s[b] (chunk in the right half): log decay from the level's reference
  //            (last token of the left half) to the token before this chunk;
  //   gam_s[b] (chunk in the left half): log decay from this chunk's last
  //            token to the reference.
  for (int n = N - 1; n >= 0; --n) {
    const int tok0 = n * C;
    double Atd;
    const double cl = chunk_prefix<C>(lag, tok0, T, lane, &Atd);
    if (tid == 0)
      for (int b = 0; b < nslot; ++b) {
        const int base = (n >> (b + 1)) << (b + 1);
        const int rs = base + (1 << b);               // first chunk of the right half
        const int re = min(N, base + (1 << (b + 1))); // one past its last chunk
        if ((n >> b) & 1) {
          if (n == re - 1) {  // first visit of this right half
            float d = 0.f;
            for (int m = rs; m < n; ++m) d += tot_s[m];
            dlt_s[b] = d;
          } else {
            dlt_s[b] -= tot_s[n];
          }
        } else if (rs < N) {
          gam_s[b] = n == rs - 1 ? 0.f : gam_s[b] + tot_s[n + 1];
        }
      }
    for (int i = tid; i < C * (dc / 4); i += NT) {
      const int r = i / (dc / 4), c = (i - r * (dc / 4)) * 4;
      const bool ok = tok0 + r < T;
      copy4(Cs + r * LDC + c, cg + (size_t)(tok0 + r) * dc + c, ok);
      copy4(Xs + r * LDX + c, xg + (size_t)(tok0 + r) * dc + c, ok);
    }
    for (int i = tid; i < C * 16; i += NT) {
      const int r = i >> 4, c = i & 15;
      const bool ok = tok0 + r < T && 16 * js + c < da;
      float x = 0.f;
      if (ok) {
        if (MODE == 0) x = a.dout[(bhT + tok0 + r) * da + 16 * js + c];
        else x = ldf(static_cast<const IT*>(a.q) + (qkT + tok0 + r) * da + 16 * js + c);
      }
      AT[c * LDAT + r] = x;
    }
    for (int i = tid; i < C * L; i += NT) lam_s[i] = tok0 + i / L < T ? lamg[(size_t)tok0 * L + i] : 0.f;
    if (w == 0 && lane < C) cl_s[lane] = cl;
    __syncthreads();

    // ---- intra chunk: output rows s = 16w.. from the masked Z tiles (c . x)
    const int s_l = 16 * w + li;  // key of this lane
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
    for (int tb = w; tb < NW; ++tb) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      #pragma unroll 8
      for (int k0 = 0; k0 < dc; k0 += 4)
        acc = F::mma(static_cast<float>(Cs[(16 * tb + li) * LDC + k0 + g4]),
                     static_cast<float>(Xs[(16 * w + li) * LDX + k0 + g4]), acc);
      // acc[r] = c_t . x_s with t = 16tb + 4g4 + r, s = s_l
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * tb + 4 * g4 + r;
        const float p = t >= s_l ? acc[r] * lam_s[t * L + level_of(t, s_l)] *
                                         __expf(static_cast<float>(cl_s[t] - cl_s[s_l]))
                                 : 0.f;
        Y = F::mma(p, AT[li * LDAT + t], Y);
      }
    }
    mfma_drain();
    // ---- key side: levels whose bit is clear read the finished right-half state
    for (int b = 0; b < nslot; ++b) {
      const int base = (n >> (b + 1)) << (b + 1);
      if (((n >> b) & 1) || base + (1 << b) >= N) continue;
      const float* rb = R + b * 16 * LDR;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      #pragma unroll 8
      for (int k0 = 0; k0 < dc; k0 += 4)
        acc = F::mma(static_cast<float>(Xs[(16 * w + li) * LDX + k0 + g4]), rb[li * LDR + k0 + g4], acc);
      mfma_drain();
      // acc[r] = x_s . R_b[j = li], s = 16w + 4g4 + r; decay from s to the reference
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * w + 4 * g4 + r;
        Y[r] += __expf(static_cast<float>(gam_s[b] + (Atd - cl_s[s]))) * acc[r];
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = tok0 + 16 * w + 4 * g4 + r;
      if (s < T) yg[(size_t)s * da + li] = Y[r];
    }
    // ---- query side: levels whose bit is set add this chunk to their state
    for (int it = w; it < dc / 16; it += NW) {
      const int i0 = 16 * it;
      for (int b = 0; b < nslot; ++b) {
        if (!((n >> b) & 1)) continue;
        const int base = (n >> (b + 1)) << (b + 1);
        const int re = min(N, base + (1 << (b + 1)));
        float* rb = R + b * 16 * LDR;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        #pragma unroll 8
        for (int k0 = 0; k0 < C; k0 += 4) {
          const int t = k0 + g4;
          const float wq = lam_s[t * L + LOGC + 1 + b] * __expf(static_cast<float>(cl_s[t] + dlt_s[b]));
          acc = F::mma(wq * AT[li * LDAT + t], static_cast<float>(Cs[t * LDC + i0 + li]), acc);
        }
        mfma_drain();
        // acc[r] = sum_t w_t a_t[j] c_t[i], j = 4g4 + r, i = i0 + li
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float* p = rb + (4 * g4 + r) * LDR + i0 + li;
          *p = (n == re - 1 ? 0.f : *p) + acc[r];
        }
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bwd_dlam_intra_kernel: dlam of the levels 0..log2 C, one workgroup per
// (b,h, chunk); wave w owns query rows 16w..
// ---------------------------------------------------------------------------
template <typename IT, int C>
__global__ void __launch_bounds__(C / 16 * 64) bwd_dlam_intra_kernel(BwdArgs a) {
  constexpr int NW = C / 16, LOGC = Lg<C>::v;
  const int T = a.T, L = a.L, dk = a.dk, dv = a.dv;
  const int N = (T + C - 1) / C;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int tok0 = n * C;
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const IT* __restrict__ qg = static_cast<const IT*>(a.q) + qkT * dk;
  const IT* __restrict__ kg = static_cast<const IT*>(a.k) + qkT * dk;
  const IT* __restrict__ vg = static_cast<const IT*>(a.v) + bhT * dv;
  const float* __restrict__ dog = a.dout + bhT * dv;
  __shared__ double cl_s[C];
  double Atot;
  const double cl = chunk_prefix<C>(a.log_a + bhT, tok0, T, lane, &Atot);
  if (w == 0 && lane < C) cl_s[lane] = cl;
  __syncthreads();
  const int tq = 16 * w + li;
  const bool qok = tok0 + tq < T;
  float acc_l[LOGC + 1];
#pragma unroll
  for (int l = 0; l <= LOGC; ++l) acc_l[l] = 0.f;
  for (int kb = 0; kb <= w; ++kb) {
    const int s_row = 16 * kb + li;  // key row this lane loads for the A operands
    const bool sok = tok0 + s_row < T;
    f32x4 z1 = {0.f, 0.f, 0.f, 0.f}, z2 = {0.f, 0.f, 0.f, 0.f};
    #pragma unroll 8
    for (int k0 = 0; k0 < dk; k0 += 4) {
      const float ka = sok ? ldf(kg + (size_t)(tok0 + s_row) * dk + k0 + g4) : 0.f;
      const float qb = qok ? ldf(qg + (size_t)(tok0 + tq) * dk + k0 + g4) : 0.f;
      z1 = F::mma(ka, qb, z1);
    }
    #pragma unroll 8
    for (int k0 = 0; k0 < dv; k0 += 4) {
      const float va = sok ? ldf(vg + (size_t)(tok0 + s_row) * dv + k0 + g4) : 0.f;
      const float db = qok ? dog[(size_t)(tok0 + tq) * dv + k0 + g4] : 0.f;
      z2 = F::mma(va, db, z2);
    }
    mfma_drain();
    // z1[r] = k_s . q_t, z2[r] = v_s . dO_t with s = 16kb + 4g4 + r, t = tq
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 16 * kb + 4 * g4 + r;
      if (s <= tq) {
        const float x = z1[r] * z2[r] * __expf(static_cast<float>(cl_s[tq] - cl_s[s]));
        const int lev = level_of(tq, s);
#pragma unroll
        for (int l = 0; l <= LOGC; ++l) acc_l[l] += l == lev ? x : 0.f;
      }
    }
  }
  // sum over the four lane groups (keys 4g4 + r) of each query
  float* __restrict__ dl = a.dlam + (bhT + tok0 + tq) * L;
#pragma unroll
  for (int l = 0; l <= LOGC; ++l) {
    float x = acc_l[l];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g4 == 0 && qok && l < L) dl[l] = x;
  }
}

// ---------------------------------------------------------------------------
// bwd_dlam_rows_kernel: everything per (b,h, t) row that follows the sweeps
// when the reverse register-state sweeps wrote their per-column-group row
// records ([nin][BH][T][8]: words 0..logc the in-chunk dlambda, word 7
// v_t . dV_t over the group's columns): dlam of the in-chunk levels (the
// records summed in group order), of the chunk levels (the dQ sweep's
// per-slice partials summed in slice order, 0 past the levels the row
// reaches), and
//   dc_t = dO_t . O_t - v_t . dV_t = sum_l lambda[t,l] dlambda[t,l] - sum_g (v . dV)_g
// in fp64, with the total of dc over the block for the decay gradient's scan.
// A workgroup takes 64 consecutive rows of one (b,h): one thread per (row,
// level) forms and writes dlam (consecutive threads on consecutive words),
// then four threads per row sum its products from LDS.
// ---------------------------------------------------------------------------
constexpr int kRowBlk = 64;     // rows per workgroup of bwd_dlam_rows_kernel
constexpr int kScanRows = 1024; // rows per workgroup of bwd_dlog_a_blk_kernel

template <int NP>
__global__ void __launch_bounds__(256) bwd_dlam_rows_kernel(BwdArgs a, int logc, int nin, int nout) {
  constexpr int R = kRowBlk;
  __shared__ float s_lam[R * 32], s_dl[R * 32];  // L <= 32
  __shared__ double s_w[4];
  const int ntb = (a.T + R - 1) / R;
  const int bh = blockIdx.x / ntb, tb = blockIdx.x - bh * ntb;
  const long long rows = (long long)a.BH * a.T;
  const long long r0 = (long long)bh * a.T + (long long)tb * R;
  const int nr = min(R, a.T - tb * R);
  const int L = a.L, nl = logc + 1, nslot = a.nslot, tid = threadIdx.x;
  const size_t istride = (size_t)rows * 8, pstride = (size_t)rows * nslot;
  const float* __restrict__ in = a.dlam_intra_part;
  const float inv_l = 1.f / static_cast<float>(L);
  // (row, level) elements e = tid + 256 i: every element's loads are issued
  // before any sum (at most NP group and NP slice partials)
  constexpr int EPT = (R * 32) / 256;
  float part_v[EPT][NP], lam_v[EPT];
  bool is_in[EPT];
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + 256 * i;
    // e / L: e < 2^11, so the rounded quotient of e + 1/2 is exact
    const int rr = __float2int_rz((static_cast<float>(e) + 0.5f) * inv_l), l = e - rr * L;
    const size_t row = r0 + rr;
    const bool ok = e < nr * L;
    is_in[i] = l < nl;
    const bool sl_ok = !is_in[i] && l - nl < nslot;
    const float* __restrict__ src = is_in[i] ? in + row * 8 + l : a.dlam_part + row * nslot + (l - nl);
    const size_t stride = is_in[i] ? istride : pstride;
    const int np = is_in[i] ? nin : (sl_ok ? nout : 0);
#pragma unroll
    for (int p = 0; p < NP; ++p) part_v[i][p] = ok && p < np ? src[p * stride] : 0.f;
    lam_v[i] = ok ? a.lam[r0 * L + e] : 0.f;
  }
#pragma unroll
  for (int i = 0; i < EPT; ++i) {
    const int e = tid + 256 * i;
    float y = 0.f;
#pragma unroll
    for (int p = 0; p < NP; ++p) y += part_v[i][p];  // partials past np are +0: the in-order sum
    if (e < nr * L) {
      a.dlam[r0 * L + e] = y;
      s_lam[e] = lam_v[i];
      s_dl[e] = y;
    }
  }
  __syncthreads();
  // row rr = tid / 4: its quarter q of the levels, then the row's sum
  const int rr = tid >> 2, q = tid & 3;
  double x = 0.0;
  if (rr < nr)
    for (int l = q; l < L; l += 4) x += (double)s_lam[rr * L + l] * s_dl[rr * L + l];
  x += __shfl_xor(x, 1);
  x += __shfl_xor(x, 2);
  if (rr < nr && q == 0) {
    const size_t row = r0 + rr;
    for (int p = 0; p < nin; ++p) x -= (double)in[p * istride + row * 8 + 7];
    a.dc[row] = x;
  } else {
    x = 0.0;
  }
  // block total: the 16 rows of each wave, then the four waves in order
#pragma unroll
  for (int off = 4; off < 64; off <<= 1) x += __shfl_xor(x, off);
  if ((tid & 63) == 0) s_w[tid >> 6] = x;
  __syncthreads();
  if (tid == 0) a.dc_blk[(size_t)bh * ntb + tb] = ((s_w[0] + s_w[1]) + s_w[2]) + s_w[3];
}

// bwd_dlog_a_blk_kernel: dlog_a = reverse prefix sum of dc over T (fp64),
// one workgroup per (b,h, 1024 rows): the later rows' total from the 64-row
// block totals, then a reverse scan of the workgroup's rows (four per thread).
__global__ void __launch_bounds__(256) bwd_dlog_a_blk_kernel(BwdArgs a) {
  constexpr int S = kScanRows, PER = S / 256;
  __shared__ double part[256];
  const int T = a.T, tid = threadIdx.x;
  const int nsb = (T + S - 1) / S, ntb = (T + kRowBlk - 1) / kRowBlk;
  const int bh = blockIdx.x / nsb, sb = blockIdx.x - bh * nsb;
  // total of the blocks after this workgroup's rows
  const int tb0 = (sb + 1) * (S / kRowBlk);
  double s = 0.0;
  for (int tb = tb0 + tid; tb < ntb; tb += 256) s += a.dc_blk[(size_t)bh * ntb + tb];
  part[tid] = s;
  __syncthreads();
  for (int off = 128; off > 0; off >>= 1) {
    if (tid < off) part[tid] += part[tid + off];
    __syncthreads();
  }
  const double later = part[0];
  __syncthreads();
  // this thread's rows t0 .. t0 + PER - 1
  const double* __restrict__ d = a.dc + (size_t)bh * T;
  float* __restrict__ out = a.dlog_a + (size_t)bh * T;
  const int t0 = sb * S + tid * PER;
  double v[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) v[i] = t0 + i < T ? d[t0 + i] : 0.0;
  double own = 0.0;
#pragma unroll
  for (int i = 0; i < PER; ++i) own += v[i];
  part[tid] = own;
  __syncthreads();
  // inclusive suffix sums of the thread totals (log-step scan)
  for (int off = 1; off < 256; off <<= 1) {
    const double u = tid + off < 256 ? part[tid + off] : 0.0;
    __syncthreads();
    part[tid] += u;
    __syncthreads();
  }
  double run = later + (tid + 1 < 256 ? part[tid + 1] : 0.0);
#pragma unroll
  for (int i = PER - 1; i >= 0; --i) {
    run += v[i];
    if (t0 + i < T) out[t0 + i] = static_cast<float>(run);
  }
}

// ---------------------------------------------------------------------------
// bwd_dlam_inter_kernel: dlam of the chunk levels, the sum of the per-slice
// partials in slice order (0 past the levels a row reaches).  One thread per
// (b,h, t, level b < nslot): the partials of one slice and (b,h) are one
// contiguous [T][nslot] block, so consecutive threads read consecutive words.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_dlam_inter_kernel(BwdArgs a, int logc, int nparts) {
  const int T = a.T, L = a.L, nslot = a.nslot;
  const int ns = nslot > 0 ? nslot : 1;  // nslot = 0: one thread per row writes its zeros
  const int bh = blockIdx.y;
  const long long e = (long long)blockIdx.x * 256 + threadIdx.x;  // t * ns + b
  if (e >= (long long)T * ns) return;
  const int t = static_cast<int>(e / ns), b = static_cast<int>(e - (long long)t * ns);
  float* __restrict__ row = a.dlam + ((size_t)bh * T + t) * L + logc + 1;
  float x = 0.f;
  if (b < nslot) {
    // every slice's load is issued before the in-order sum (nparts <= 8)
    const size_t pstride = (size_t)a.BH * T * nslot;
    const float* __restrict__ src = a.dlam_part + (size_t)bh * T * nslot + e;
    float v[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) v[p] = p < nparts ? src[p * pstride] : 0.f;
#pragma unroll
    for (int p = 0; p < 8; ++p) x += v[p];
  }
  if (b + logc + 1 < L) row[b] = x;
  if (b == ns - 1)
    for (int q = ns; q + logc + 1 < L; ++q) row[q] = 0.f;
}

// ---------------------------------------------------------------------------
// bwd_dcum_kernel: dc_t = dO_t . O_t - v_t . dV_t (fp64), one wave per token;
// dO_t . O_t is taken as sum_l lambda[t,l] dlambda[t,l] once dlambda is final.
// bwd_dlog_a_kernel: dlog_a = reverse prefix sum of dc over T, one workgroup
// per (b,h), each thread a contiguous range, fp64 (the two parts of dc largely
// cancel and the sum runs over up to T terms).
// ---------------------------------------------------------------------------
template <typename IT>
__global__ void __launch_bounds__(256) bwd_dcum_kernel(BwdArgs a, double* dc) {
  const int T = a.T, dv = a.dv;
  const size_t row = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);  // (b,h, t) flattened
  const int lane = threadIdx.x & 63;
  if (row >= (size_t)a.BH * T) return;
  // dO_t . O_t = sum_l lambda[t, l] dlambda[t, l] (both sum the same pairs
  // (q_t . k_s)(dO_t . v_s) exp(cum_t - cum_s) lambda[t, l(t,s)]), so the
  // forward output and dO need not be read again
  const int L = a.L;
  const float* __restrict__ lam = a.lam + row * L;
  const float* __restrict__ dlam = a.dlam + row * L;
  const float* __restrict__ dV = a.dvo + row * dv;
  const IT* __restrict__ v = static_cast<const IT*>(a.v) + row * dv;
  double x = 0.0;
  for (int l = lane; l < L; l += 64) x += (double)lam[l] * dlam[l];
  for (int j = lane; j < dv; j += 64) x -= (double)static_cast<float>(v[j]) * dV[j];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (lane == 0) dc[row] = x;
}

// The same for dv / 8 a power of two up to 64 (bf16 v): G = dv / 8 lanes per
// token, each with eight columns as 16-byte loads, so a wave covers 64 / G
// tokens; the lane group's sums are reduced by xor shuffles inside the group.
template <int G>
__global__ void __launch_bounds__(256) bwd_dcum16_kernel(BwdArgs a, double* dc) {
  constexpr int TPW = 64 / G;  // tokens per wave
  const int T = a.T, dv = a.dv, L = a.L;
  const int lane = threadIdx.x & 63, gl = lane & (G - 1);
  const size_t row = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW + lane / G;
  const bool ok = row < (size_t)a.BH * T;
  double x = 0.0;
  if (ok) {
    const bf16x8 vv = *reinterpret_cast<const bf16x8*>(static_cast<const bf16*>(a.v) + row * dv + 8 * gl);
    const f32x4 d0 = *reinterpret_cast<const f32x4*>(a.dvo + row * dv + 8 * gl);
    const f32x4 d1 = *reinterpret_cast<const f32x4*>(a.dvo + row * dv + 8 * gl + 4);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x -= (double)static_cast<float>(vv[e]) * d0[e];
      x -= (double)static_cast<float>(vv[e + 4]) * d1[e];
    }
    for (int l = gl; l < L; l += G) x += (double)a.lam[row * L + l] * a.dlam[row * L + l];
  }
#pragma unroll
  for (int off = G / 2; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (ok && gl == 0) dc[row] = x;
}

__global__ void __launch_bounds__(256) bwd_dlog_a_kernel(BwdArgs a, const double* dc) {
  const int bh = blockIdx.x, tid = threadIdx.x, T = a.T;
  const double* __restrict__ d = dc + (size_t)bh * T;
  float* __restrict__ out = a.dlog_a + (size_t)bh * T;
  __shared__ double part[256];
  const int per = (T + 255) / 256;
  const int t0 = min(T, tid * per), t1 = min(T, t0 + per);
  // this thread's range total, eight loads in flight
  double s = 0.0;
  int t = t0;
  for (; t + 8 <= t1; t += 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = d[t + q];
#pragma unroll
    for (int q = 0; q < 8; ++q) s += v[q];
  }
  for (; t < t1; ++t) s += d[t];
  part[tid] = s;
  __syncthreads();
  // inclusive suffix sums of the range totals (log-step scan)
  for (int off = 1; off < 256; off <<= 1) {
    const double v = tid + off < 256 ? part[tid + off] : 0.0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  double run = tid + 1 < 256 ? part[tid + 1] : 0.0;  // sum of the ranges of the threads above
  // reverse prefix over the range, eight loads in flight
  t = t1;
  for (; t - 8 >= t0; t -= 8) {
    double v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) v[q] = d[t - 1 - q];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      run += v[q];
      out[t - 1 - q] = static_cast<float>(run);
    }
  }
  for (; t > t0; --t) {
    run += d[t - 1];
    out[t - 1] = static_cast<float>(run);
  }
}

}  // namespace bwd

int bwd_lds_bytes(int dtype, int C, int dk, int dv, int L, int N, int nslot) {
  using namespace bwd;
  auto pick = [&](auto tag_it) {
    using IT = decltype(tag_it);
    int q = 0, kv0 = 0, kv1 = 0;
    switch (C) {
      case 16: q = DqCfg<IT, 16>::bytes(dv, L, nslot); kv0 = KvCfg<IT, 16, 0>::bytes(dk, L, N, nslot);
               kv1 = KvCfg<IT, 16, 1>::bytes(dv, L, N, nslot); break;
      case 32: q = DqCfg<IT, 32>::bytes(dv, L, nslot); kv0 = KvCfg<IT, 32, 0>::bytes(dk, L, N, nslot);
               kv1 = KvCfg<IT, 32, 1>::bytes(dv, L, N, nslot); break;
      default: q = DqCfg<IT, 64>::bytes(dv, L, nslot); kv0 = KvCfg<IT, 64, 0>::bytes(dk, L, N, nslot);
               kv1 = KvCfg<IT, 64, 1>::bytes(dv, L, N, nslot); break;
    }
    return max(q, max(kv0, kv1));
  };
  return dtype == LL_BF16 ? pick(bf16(0.f)) : pick(0.f);
}

template <typename IT, int C>
static int launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  using namespace bwd;
  const int N = (a.T + C - 1) / C;
  constexpr int NT = C / 16 * 64;
  // dQ and the chunk-level dlam partials (unless the register-state sweep
  // formed them already)
  if (a.dq_done) {
  } else if (sizeof(IT) == 2 && C == 64 && bwd_dq16_ok(a)) {
    const int st = launch_bwd_dq16(a, s);
    if (st != LL_OK) return st;
  } else {
    const int bytes = DqCfg<IT, C>::bytes(a.dv, a.L, a.nslot);
    if (bytes > kMaxLds) return LL_ERR_UNSUPPORTED;
    static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
    if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_dq_kernel<IT, C>), raised)) return LL_ERR_HIP;
    hipLaunchKernelGGL((bwd_dq_kernel<IT, C>), dim3(a.BH * (a.dk / 16)), dim3(NT), bytes, s, a);
  }
  // dV and dK (unless the reverse register-state sweep formed them already)
  if (a.kv_done) {
  } else if (sizeof(IT) == 2 && C == 64 && bwd_kv16_ok(a)) {
    const int st = launch_bwd_kv16(a, s);
    if (st != LL_OK) return st;
  } else {
  {
    const int bytes = KvCfg<IT, C, 0>::bytes(a.dk, a.L, N, a.nslot);
    if (bytes > kMaxLds) return LL_ERR_UNSUPPORTED;
    static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
    if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_kv_kernel<IT, C, 0>), raised)) return LL_ERR_HIP;
    hipLaunchKernelGGL((bwd_kv_kernel<IT, C, 0>), dim3(a.BH * (a.dv / 16)), dim3(NT), bytes, s, a);
  }
  {
    const int bytes = KvCfg<IT, C, 1>::bytes(a.dv, a.L, N, a.nslot);
    if (bytes > kMaxLds) return LL_ERR_UNSUPPORTED;
    static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
    if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_kv_kernel<IT, C, 1>), raised)) return LL_ERR_HIP;
    hipLaunchKernelGGL((bwd_kv_kernel<IT, C, 1>), dim3(a.BH * (a.dk / 16)), dim3(NT), bytes, s, a);
  }
  }
  if (a.intra_parts > 0) {
    // the reverse dV sweep's row records: one pass forms dlam and dc
    const long long nb = (long long)a.BH * ((a.T + kRowBlk - 1) / kRowBlk);
    const long long ns = (long long)a.BH * ((a.T + kScanRows - 1) / kScanRows);
    const int nout = a.dq_done ? a.dlam_parts : a.dk / 16;
    if (nb > 0x7fffffffLL || !a.dc_blk || a.L > 32 || a.intra_parts > 8 || nout > 8) return LL_ERR_UNSUPPORTED;
    if (a.intra_parts <= 2 && nout <= 2)
      hipLaunchKernelGGL(bwd_dlam_rows_kernel<2>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, a, Lg<C>::v,
                         a.intra_parts, nout);
    else
      hipLaunchKernelGGL(bwd_dlam_rows_kernel<8>, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, a, Lg<C>::v,
                         a.intra_parts, nout);
    hipLaunchKernelGGL(bwd_dlog_a_blk_kernel, dim3(static_cast<unsigned>(ns)), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
  }
  if (sizeof(IT) == 2 && C == 64 && bwd_dlam_intra16_ok(a)) {
    const int st = launch_bwd_dlam_intra16(a, s);
    if (st != LL_OK) return st;
  } else {
    hipLaunchKernelGGL((bwd_dlam_intra_kernel<IT, C>), dim3(a.BH * N), dim3(NT), 0, s, a);
  }
  {
    const long long elems = (long long)a.T * (a.nslot > 0 ? a.nslot : 1);
    hipLaunchKernelGGL(bwd_dlam_inter_kernel, dim3(static_cast<unsigned>((elems + 255) / 256), a.BH), dim3(256), 0, s,
                       a, Lg<C>::v, a.dq_done ? a.dlam_parts : a.dk / 16);
  }
  const size_t rows = (size_t)a.BH * a.T;
  {
    // bf16 v with dv / 8 a power of two <= 64: grouped lanes and vector loads
    const int g = a.dv / 8;
    const bool aligned = ((reinterpret_cast<uintptr_t>(a.v) | reinterpret_cast<uintptr_t>(a.dvo)) & 15) == 0;
    const bool grouped = sizeof(IT) == 2 && aligned && a.dv % 8 == 0 && g >= 1 && g <= 64 && (g & (g - 1)) == 0;
    if (grouped) {
      const size_t waves = (rows * g + 63) / 64;
      const dim3 grid(static_cast<unsigned>((waves + 3) / 4));
      switch (g) {
        case 1: hipLaunchKernelGGL(bwd_dcum16_kernel<1>, grid, dim3(256), 0, s, a, a.dc); break;
        case 2: hipLaunchKernelGGL(bwd_dcum16_kernel<2>, grid, dim3(256), 0, s, a, a.dc); break;
        case 4: hipLaunchKernelGGL(bwd_dcum16_kernel<4>, grid, dim3(256), 0, s, a, a.dc); break;
        case 8: hipLaunchKernelGGL(bwd_dcum16_kernel<8>, grid, dim3(256), 0, s, a, a.dc); break;
        case 16: hipLaunchKernelGGL(bwd_dcum16_kernel<16>, grid, dim3(256), 0, s, a, a.dc); break;
        case 32: hipLaunchKernelGGL(bwd_dcum16_kernel<32>, grid, dim3(256), 0, s, a, a.dc); break;
        default: hipLaunchKernelGGL(bwd_dcum16_kernel<64>, grid, dim3(256), 0, s, a, a.dc); break;
      }
    } else {
      hipLaunchKernelGGL((bwd_dcum_kernel<IT>), dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, s, a, a.dc);
    }
  }
  hipLaunchKernelGGL(bwd_dlog_a_kernel, dim3(a.BH), dim3(256), 0, s, a, a.dc);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int launch_bwd(int dtype, int C, const BwdArgs& a, hipStream_t s) {
  if (dtype == LL_BF16) {
    switch (C) {
      case 16: return launch_bwd_t<bf16, 16>(a, s);
      case 32: return launch_bwd_t<bf16, 32>(a, s);
      case 64: return launch_bwd_t<bf16, 64>(a, s);
    }
  } else {
    switch (C) {
      case 16: return launch_bwd_t<float, 16>(a, s);
      case 32: return launch_bwd_t<float, 32>(a, s);
      case 64: return launch_bwd_t<float, 64>(a, s);
    }
  }
  return LL_ERR_UNSUPPORTED;
}

// Gradients of q and k shared by G heads: the per-head gradients summed over
// each group, in head order (deterministic).  Four elements per thread.
__global__ void __launch_bounds__(256) group_sum_kernel(const float* __restrict__ in, float* __restrict__ out,
                                                        int G, long long elems, long long total4) {
  const long long i4 = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i4 >= total4) return;
  const long long e = i4 * 4, row = e / elems, off = e - row * elems;
  const float* src = in + (row * G) * elems + off;
  f32x4 s = *reinterpret_cast<const f32x4*>(src);
  for (int g = 1; g < G; ++g) s += *reinterpret_cast<const f32x4*>(src + (long long)g * elems);
  *reinterpret_cast<f32x4*>(out + e) = s;
}

int launch_group_sum(const float* in, float* out, long long rows, int G, long long elems, hipStream_t s) {
  if (elems % 4 != 0) return LL_ERR_UNSUPPORTED;
  const long long total4 = rows * elems / 4;
  if (total4 == 0) return LL_OK;
  const long long nb = (total4 + 255) / 256;
  if (nb > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(group_sum_kernel, dim3(static_cast<unsigned>(nb)), dim3(256), 0, s, in, out, G, elems, total4);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
