// Backward sweeps on bf16 matrix cores for bf16 inputs: the reverse sweep
// (dV and dK) and the forward sweep (dQ and the chunk-level dlambda partials),
// C = 64, contraction widths that are multiples of 32 up to 128 and up to 8
// chunk-level Fenwick bits.  Same decomposition as bwd_kv_kernel
// (loglinear_bwd.hip; [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制",
// sections 并行形式, 与已有模型的组合, 训练：分块并行扫描算法):
//
//   y_s = sum_{t >= s} M[t,s] (c_t . x_s) a_t,   M[t,s] = lambda[t, l(t,s)] exp(cum_t - cum_s)
//   MODE 0: dV (a = dO, c = q, x = k);  MODE 1: dK (a = q, c = dO, x = v).
//
// One 512-thread workgroup per (b,h, 16 output columns), two waves per SIMD;
// chunks in reverse order.  Wave w works on key rows 16(w&3)..+15 of a chunk:
// the two waves of a row tile (w>>2 = 0, 1) take one pair of score tiles and
// half of the left-half levels each and add their partial outputs through
// LDS; the state updates of the levels whose right half holds the chunk are
// shared out over all waves.  Every product runs as
// v_mfma_f32_16x16x32_bf16: bf16 inputs are exact operands, fp32 ones (dO,
// the masked scores, the level states, the weighted a) are split into bf16
// hi + lo and multiplied term by term (hi*hi + lo*hi + hi*lo where both
// sides are split), which keeps ~2^-16 of each product.
//   intra    scores c_t . x_s for the t tiles at or after the wave's s tile,
//            masked in registers; the masked tile is the A operand of the
//            product with a^T directly from the accumulator layout (the
//            contraction order over t is the same permutation on both sides).
//   left     levels whose bit of n is clear read R_b (complete: converted once
//            from fp32 to bf16 hi / lo in place when the sweep enters its left
//            half): y_s += exp(decay s -> reference) x_s . R_b.
//   right    levels whose bit is set add this chunk to their fp32 state:
//            R_b[j][i] += sum_t lambda[t, b] exp(cum_t - ref) a_t[j] c_t[i],
//            with c^T read by the LDS transpose load.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {
namespace b16 {

constexpr int C = 64, NW = 8, NT = NW * 64, LOGC = 6, NSMAX = 8;
constexpr int LDC = 136;  // bf16 rows of c and x (contraction <= 128): 272 bytes
constexpr int LDAT = 68;  // fp32 a^T rows [16][68]
constexpr int LDAB = 72;  // bf16 a^T rows [16][72]
constexpr int LDR = 136;  // level state: fp32 [16][136], or bf16 hi [16][136] + lo [16][136]
constexpr int R_BYTES = 16 * LDR * 4;

template <int MODE>
struct KvLay {
  static constexpr int NCB = MODE == 1 ? 2 : 1;  // c copies: MODE 1 holds dO as bf16 hi, lo
  static constexpr int NAB = MODE == 0 ? 2 : 1;  // bf16 a^T copies: MODE 0 holds dO hi, lo
  static constexpr int CS = 0;
  static constexpr int XS = CS + NCB * C * LDC * 2;
  static constexpr int ATF = XS + C * LDC * 2;
  static constexpr int ATB = ATF + 16 * LDAT * 4;
  static constexpr int WL = ATB + NAB * 16 * LDAB * 2;  // right-half weights [NSMAX][C]
  static constexpr int CL = WL + NSMAX * C * 4;         // in-chunk prefix of log_a, fp64 [C]
  static constexpr int R = CL + C * 8;                  // level states [NSMAX]
  static constexpr int YX = R + NSMAX * R_BYTES;        // partial outputs [4][64] f32x4
  static constexpr int LAM = YX + 4 * 64 * 16;          // lambda rows of the chunk [C][L]
  __host__ __device__ static int tot(int L) { return LAM + C * L * 4; }  // chunk totals [N]
  __host__ __device__ static int bytes(int L, int N) { return tot(L) + ((N * 4 + 15) & ~15); }
};

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

// Transposed 8-byte LDS read: within each 16-lane group, lane i receives
// element (i & 3) of the 4-element vectors addressed by lanes 4k + (i >> 2).
__device__ __forceinline__ bf16x4 tr_read(const bf16* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(reinterpret_cast<__attribute__((address_space(3))) char*>(reinterpret_cast<uintptr_t>(p))));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 frag(const bf16* base, int ld, int row0, int k0, int lane) {
  return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
}
__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// In-chunk inclusive prefix of log_a (lane = token; tokens past T count 0) and
// the chunk total, per chunk of the sweeps: fp32 DPP row shifts and row
// broadcasts (the sweeps' bf16 arithmetic keeps ~2^-17 anyway; the fp64
// shuffle version cost ~2K cycles per chunk on the critical path).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float x) {
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROWS, 0xf, false));
}
__device__ __forceinline__ double prefix_dpp(float x, int lane, double* total) {
  x = dpp_add<0x111, 0xf>(x);  // row_shr:1
  x = dpp_add<0x112, 0xf>(x);  // row_shr:2
  x = dpp_add<0x114, 0xf>(x);  // row_shr:4
  x = dpp_add<0x118, 0xf>(x);  // row_shr:8
  x = dpp_add<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_add<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  *total = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), C - 1));
  (void)lane;
  return x;
}
// fp64 version for the chunk totals the reverse sweep sums over many chunks
__device__ __forceinline__ double chunk_prefix(const float* lag, int tok0, int T, int lane, double* total) {
  double la = tok0 + lane < T ? (double)lag[tok0 + lane] : 0.0;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const double y = __shfl_up(la, off);
    if (lane >= off) la += y;
  }
  *total = __shfl(la, C - 1);
  return la;
}

}  // namespace b16

template <int MODE>
__global__ void __launch_bounds__(b16::NT) bwd_kv16_kernel(BwdArgs a) {
  using namespace b16;
  using Lay = KvLay<MODE>;
  extern __shared__ __align__(16) unsigned char smem[];
  const int T = a.T, L = a.L, nslot = a.nslot;
  const int da = MODE == 0 ? a.dv : a.dk;  // output columns
  const int dc = MODE == 0 ? a.dk : a.dv;  // contraction of c . x
  const int N = (T + C - 1) / C;
  bf16* Ch = reinterpret_cast<bf16*>(smem + Lay::CS);
  bf16* Cl = Ch + C * LDC;  // MODE 1 only
  bf16* Xs = reinterpret_cast<bf16*>(smem + Lay::XS);
  float* ATf = reinterpret_cast<float*>(smem + Lay::ATF);
  bf16* ATh = reinterpret_cast<bf16*>(smem + Lay::ATB);
  bf16* ATl = ATh + 16 * LDAB;  // MODE 0 only
  float* WL = reinterpret_cast<float*>(smem + Lay::WL);
  double* cl_s = reinterpret_cast<double*>(smem + Lay::CL);
  unsigned char* Rbase = smem + Lay::R;
  float* lam_s = reinterpret_cast<float*>(smem + Lay::LAM);
  float* tot_s = reinterpret_cast<float*>(smem + Lay::tot(L));
  f32x4* Yx = reinterpret_cast<f32x4*>(smem + Lay::YX);

  const int nsl = da / 16;
  const int bh = blockIdx.x / nsl, js = blockIdx.x - bh * nsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int st = w & 3, hf = w >> 2;  // key row tile, half
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const float* __restrict__ lag = a.log_a + bhT;
  const float* __restrict__ lamg = a.lam + bhT * L;
  float* __restrict__ yg = (MODE == 0 ? a.dvo : a.dk_out) + bhT * da + 16 * js;

  for (int nn = w; nn < N; nn += NW) {
    double tot;
    chunk_prefix(lag, nn * C, T, lane, &tot);
    if (lane == 0) tot_s[nn] = static_cast<float>(tot);
  }
  __syncthreads();

  // Per level (identical in every lane):
  //   dlt[b] (chunk in the right half): log decay from the level's reference
  //          (last token of the left half) to the token before this chunk;
  //   gam[b] (chunk in the left half): log decay from this chunk's last token
  //          to the reference.
  float dlt[NSMAX], gam[NSMAX];
#pragma unroll
  for (int b = 0; b < NSMAX; ++b) dlt[b] = gam[b] = 0.f;

  // register prefetch of one chunk (issued a chunk ahead of its staging)
  typedef typename std::conditional<MODE == 0, bf16x8, f32x4>::type CV;  // 16-byte vector of c
  constexpr int CE = MODE == 0 ? 8 : 4;  // elements of c per vector
  typedef typename std::conditional<MODE == 0, f32x4, bf16x4>::type AV;  // four columns of a
  CV pc[4];       // c rows, vectors tid + NT*i
  bf16x8 px[2];   // x rows
  AV pa;          // a slice (threads < 4C)
  float plam[4];  // lambda words tid + NT*i of the chunk
  float pla;      // log_a of token lane
  float plw;      // lambda[token lane][log2C + 1 + w]: this wave's right-half weights
  const void* cbase = MODE == 0 ? static_cast<const void*>(static_cast<const bf16*>(a.q) + qkT * dc)
                                : static_cast<const void*>(a.dout + bhT * dc);
  const bf16* xg = static_cast<const bf16*>(MODE == 0 ? a.k : a.v) + (MODE == 0 ? qkT : bhT) * dc;
  auto load = [&](int nn) {
    const int t0 = nn * C;
    pla = t0 + lane < T ? lag[t0 + lane] : 0.f;
    // level w + log2C + 1 < L whenever w < nslot
    plw = w < nslot && t0 + lane < T ? lamg[(size_t)(t0 + lane) * L + LOGC + 1 + w] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, r = idx / (dc / CE), c = (idx - r * (dc / CE)) * CE;
      if (idx < C * dc / CE)
        pc[i] = t0 + r < T ? *reinterpret_cast<const CV*>(static_cast<const char*>(cbase) +
                                                         ((size_t)(t0 + r) * dc + c) * (MODE == 0 ? 2 : 4))
                           : CV{};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, r = idx / (dc / 8), c = (idx - r * (dc / 8)) * 8;
      if (idx < C * dc / 8)
        px[i] = t0 + r < T ? *reinterpret_cast<const bf16x8*>(xg + (size_t)(t0 + r) * dc + c) : bf16x8{};
    }
    if (tid < 4 * C) {
      const int r = tid >> 2, c = (tid & 3) * 4;
      const bool ok = t0 + r < T;
      if (MODE == 0)
        pa = ok ? *reinterpret_cast<const AV*>(a.dout + (bhT + t0 + r) * da + 16 * js + c) : AV{};
      else
        pa = ok ? *reinterpret_cast<const AV*>(static_cast<const bf16*>(a.q) + (qkT + t0 + r) * da + 16 * js + c)
                : AV{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i;
      if (idx < C * L) plam[i] = t0 + idx / L < T ? lamg[(size_t)t0 * L + idx] : 0.f;
    }
  };
  load(N - 1);
  for (int n = N - 1; n >= 0; --n) {
    const int tok0 = n * C;
    double Atd;
    const double cl = prefix_dpp(pla, lane, &Atd);
    const float wl_lam = plw;  // this chunk's; the registers are refilled below
#pragma unroll
    for (int b = 0; b < NSMAX; ++b) {
      if (b < nslot) {
        const int base = (n >> (b + 1)) << (b + 1);
        const int rs = base + (1 << b), re = min(N, base + (1 << (b + 1)));
        if ((n >> b) & 1) {
          if (n == re - 1) {
            float d = 0.f;
            for (int m = rs; m < n; ++m) d += tot_s[m];
            dlt[b] = uniform(d);
          } else {
            dlt[b] = uniform(dlt[b] - tot_s[n]);
          }
        } else if (rs < N) {
          gam[b] = uniform(n == rs - 1 ? 0.f : gam[b] + tot_s[n + 1]);
        }
      }
    }
    // The level whose right half starts at chunk n + 1 is complete: its state
    // is converted to bf16 hi / lo (in place, after the staging barrier) for
    // the left-half reads from this chunk on.
    const int bc = n + 1 < N ? __builtin_ctz(static_cast<unsigned>(n + 1)) : 32;
    const bool conv = bc < nslot;
    const int per = dc / 32;  // state elements per thread: row tid >> 5, columns (tid & 31) * per ..
    float rv[4];
    if (conv) {
      const float* Rf = reinterpret_cast<const float*>(Rbase + bc * R_BYTES) + (tid >> 5) * LDR + (tid & 31) * per;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < per) rv[e] = Rf[e];
    }

    // ---- stage chunk n from the registers (tokens past T are zero), then
    // prefetch chunk n - 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, r = idx / (dc / CE), c = (idx - r * (dc / CE)) * CE;
      if (idx < C * dc / CE) {
        if (MODE == 0) {
          *reinterpret_cast<bf16x8*>(Ch + r * LDC + c) = __builtin_bit_cast(bf16x8, pc[i]);
        } else {
          const f32x4 x = __builtin_bit_cast(f32x4, pc[i]);
          bf16x4 h, l;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            bf16 x1, x2;
            split_bf16(x[e], x1, x2);
            h[e] = x1;
            l[e] = x2;
          }
          *reinterpret_cast<bf16x4*>(Ch + r * LDC + c) = h;
          *reinterpret_cast<bf16x4*>(Cl + r * LDC + c) = l;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, r = idx / (dc / 8), c = (idx - r * (dc / 8)) * 8;
      if (idx < C * dc / 8) *reinterpret_cast<bf16x8*>(Xs + r * LDC + c) = px[i];
    }
    // a^T slice [16][C]: fp32 copy (weights) and bf16 copies (operands)
    if (tid < 4 * C) {
      const int r = tid >> 2, c = (tid & 3) * 4;  // one token, four columns per thread
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = static_cast<float>(pa[e]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        ATf[(c + e) * LDAT + r] = v[e];
        bf16 x1, x2;
        split_bf16(v[e], x1, x2);
        ATh[(c + e) * LDAB + r] = x1;
        if (MODE == 0) ATl[(c + e) * LDAB + r] = x2;
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i;
      if (idx < C * L) lam_s[idx] = plam[i];
    }
    if (n > 0) load(n - 1);
    if (w == 0) cl_s[lane] = cl;
    // right-half weights: wave w forms those of level w (lane = token)
#pragma unroll
    for (int b = 0; b < NSMAX; ++b)
      if (b < nslot && b == w && ((n >> b) & 1)) WL[b * C + lane] = wl_lam * __expf(static_cast<float>(cl) + dlt[b]);
    __syncthreads();
    if (conv) {
      bf16* Rh = reinterpret_cast<bf16*>(Rbase + bc * R_BYTES) + (tid >> 5) * LDR + (tid & 31) * per;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < per) {
          bf16 x1, x2;
          split_bf16(rv[e], x1, x2);
          Rh[e] = x1;
          Rh[16 * LDR + e] = x2;
        }
      __syncthreads();
    }

    // ---- intra chunk: this half's pair of t tiles (2hf, 2hf + 1), where at
    // or after the key tile st (pair 0 is empty for st >= 2)
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
    if (2 * hf + 1 >= st) {
      f32x4 z[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int tb = 2 * hf + q;
        z[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tb >= st) {
          for (int k0 = 0; k0 < dc; k0 += 32) {
            const bf16x8 xb = frag(Xs, LDC, 16 * st, k0, lane);
            z[q] = mma(frag(Ch, LDC, 16 * tb, k0, lane), xb, z[q]);
            if (MODE == 1) z[q] = mma(frag(Cl, LDC, 16 * tb, k0, lane), xb, z[q]);
          }
        }
      }
      // z[q][r] = c_t . x_s, t = 16(2hf + q) + 4g4 + r, s = 16st + li; masked in place
      const int s = 16 * st + li;
      const double cls = cl_s[s];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int tb = 2 * hf + q, t = 16 * tb + 4 * g4 + r;
          z[q][r] = (tb >= st && t >= s)
                        ? z[q][r] * lam_s[t * L + level_of(t, s)] * __expf(static_cast<float>(cl_s[t] - cls))
                        : 0.f;
        }
      // Y[s][j] += sum_t p[t][s] a_t[j]: the lane's eight t values (4g4 + r of
      // each tile of the pair) are the contraction slots of both operands
      {
        bf16x8 ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 x1, x2;
          split_bf16(z[e >> 2][e & 3], x1, x2);
          ph[e] = x1;
          pl[e] = x2;
        }
        const int t0 = 32 * hf + 4 * g4;
        const bf16x8 bh8 = cat(*reinterpret_cast<const bf16x4*>(ATh + li * LDAB + t0),
                               *reinterpret_cast<const bf16x4*>(ATh + li * LDAB + t0 + 16));
        Y = mma(ph, bh8, Y);
        Y = mma(pl, bh8, Y);
        if (MODE == 0) {
          const bf16x8 bl8 = cat(*reinterpret_cast<const bf16x4*>(ATl + li * LDAB + t0),
                                 *reinterpret_cast<const bf16x4*>(ATl + li * LDAB + t0 + 16));
          Y = mma(ph, bl8, Y);
        }
      }
    }

    // ---- left-half levels: y_s += exp(decay s -> reference) x_s . R_b; the
    // k-th level that has one goes to half k & 1 (balanced for any bit pattern)
    {
      bf16x8 xa[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        if (32 * kq < dc) xa[kq] = frag(Xs, LDC, 16 * st, 32 * kq, lane);
      int rank = 0;
#pragma unroll
      for (int b = 0; b < NSMAX; ++b) {
        if (!(b < nslot && !((n >> b) & 1) && ((n >> (b + 1)) << (b + 1)) + (1 << b) < N)) continue;
        if (((rank++) & 1) == hf) {
          const bf16* Rh = reinterpret_cast<const bf16*>(Rbase + b * R_BYTES);
          const bf16* Rl = Rh + 16 * LDR;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kq = 0; kq < 4; ++kq)
            if (32 * kq < dc) {
              acc = mma(xa[kq], frag(Rh, LDR, 0, 32 * kq, lane), acc);
              acc = mma(xa[kq], frag(Rl, LDR, 0, 32 * kq, lane), acc);
            }
          // acc[r] = x_s . R_b[j], s = 16st + 4g4 + r, j = li
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int s = 16 * st + 4 * g4 + r;
            Y[r] += __expf(gam[b] + static_cast<float>(Atd - cl_s[s])) * acc[r];
          }
        }
      }
    }
    // the second half hands its partial sums to the first, which stores
    if (hf == 1) Yx[st * 64 + lane] = Y;
    __syncthreads();
    if (hf == 0) {
      const f32x4 y2 = Yx[st * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = tok0 + 16 * st + 4 * g4 + r;
        if (s < T) yg[(size_t)s * da + li] = Y[r] + y2[r];
      }
    }

    // ---- right-half levels: R_b[j][i] += sum_t WL_b[t] a_t[j] c_t[i] for
    // every level whose bit of n is set.  The (level, 16-column tile) items
    // are shared out evenly over the waves, each taking a contiguous run, so
    // a chunk costs popcount(n) tiles per wave rather than every tile of one
    // level; a wave forms the weighted A operand once per level it meets.
    {
      const int ntile = dc / 16;
      const unsigned live = static_cast<unsigned>(n) & ((1u << nslot) - 1u);
      const int items = __builtin_popcount(live) * ntile;
      const int per = (items + NW - 1) / NW;
      const int k0 = w * per, k1 = min(items, k0 + per);
      bf16x8 ah[2], al[2];  // A[j = li][t = 32ks + 8g4 + e] = WL_b[t] a_t[j]
      // the run [k0, k1) covers at most a few levels; each level's tiles are
      // done in batches of four with independent accumulators, written as
      // straight-line code (tile indices clamped to the level's last tile,
      // stores predicated) so the reads, products and state updates of a
      // batch overlap instead of forming one chain per tile
      for (int k = k0; k < k1;) {
        const int lv = k / ntile, it0 = k - lv * ntile;
        const int cnt = min(k1 - k, ntile - it0);
        unsigned rest = live;  // b = the lv-th set bit of live
        for (int q = 0; q < lv; ++q) rest &= rest - 1u;
        const int b = __builtin_ctz(rest);
        const int base = (n >> (b + 1)) << (b + 1);
        const bool first = n == min(N, base + (1 << (b + 1))) - 1;
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const f32x4 x0 = *reinterpret_cast<const f32x4*>(ATf + li * LDAT + 32 * ks + 8 * g4);
          const f32x4 x1 = *reinterpret_cast<const f32x4*>(ATf + li * LDAT + 32 * ks + 8 * g4 + 4);
          const f32x4 w0 = *reinterpret_cast<const f32x4*>(WL + b * C + 32 * ks + 8 * g4);
          const f32x4 w1 = *reinterpret_cast<const f32x4*>(WL + b * C + 32 * ks + 8 * g4 + 4);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            bf16 x1_, x2_;
            split_bf16(e < 4 ? x0[e] * w0[e] : x1[e - 4] * w1[e - 4], x1_, x2_);
            ah[ks][e] = x1_;
            al[ks][e] = x2_;
          }
        }
        float* Rf = reinterpret_cast<float*>(Rbase + b * R_BYTES);
        for (int j0 = 0; j0 < cnt; j0 += 4) {
          int i0[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) i0[u] = 16 * (it0 + min(j0 + u, cnt - 1));
          f32x4 acc[4];
#pragma unroll
          for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < 2; ++ks) {
            bf16x8 cb[4], cl8[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              const int off = (32 * ks + 8 * g4 + (li >> 2)) * LDC + i0[u] + 4 * (li & 3);
              cb[u] = cat(tr_read(Ch + off), tr_read(Ch + off + 4 * LDC));
              if (MODE == 1) cl8[u] = cat(tr_read(Cl + off), tr_read(Cl + off + 4 * LDC));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) {
              acc[u] = mma(ah[ks], cb[u], acc[u]);
              acc[u] = mma(al[ks], cb[u], acc[u]);
              if (MODE == 1) acc[u] = mma(ah[ks], cl8[u], acc[u]);
            }
          }
          // acc[u][r] = sum_t WL_b[t] a_t[j] c_t[i], j = 4g4 + r, i = i0[u] + li
          float old[4][4];
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int r = 0; r < 4; ++r) old[u][r] = first ? 0.f : Rf[(4 * g4 + r) * LDR + i0[u] + li];
#pragma unroll
          for (int u = 0; u < 4; ++u)
            if (j0 + u < cnt)
#pragma unroll
              for (int r = 0; r < 4; ++r) Rf[(4 * g4 + r) * LDR + i0[u] + li] = old[u][r] + acc[u][r];
        }
        k += cnt;
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// bwd_dq16_kernel: dQ and the chunk-level dlambda partials, forward chunk order
// (as bwd_dq_kernel): per level b the decayed left-half state
// St_b[j][i] = sum_s exp(cum_ref - cum_s) k_s[j] v_s[i] is read by the
// right-half queries, dQ_t[j] += lambda[t, b] exp(cum_t - ref) (dO_t . St_b[j]),
// and the same products dotted with q_t give the slice's dlambda partial.
// One 512-thread workgroup per (b,h, 16 columns of dk); wave w works on query
// rows 16(w&3)..+15 with half w>>2 of the score tiles and of the levels.
// ---------------------------------------------------------------------------
namespace b16 {
struct DqLay {
  static constexpr int LDQS = 17;                    // fp32 q slice rows [C][17]
  static constexpr int DH = 0;                       // dO rows, bf16 hi / lo [C][LDC]
  static constexpr int DL = DH + C * LDC * 2;
  static constexpr int VS = DL + C * LDC * 2;        // v rows bf16 [C][LDC]
  static constexpr int KT = VS + C * LDC * 2;        // k slice transposed bf16 [16][LDAB]
  static constexpr int QS = KT + 16 * LDAB * 2;      // q slice fp32 [C][LDQS]
  static constexpr int ESF = QS + ((C * LDQS * 4 + 15) & ~15);  // decay to the chunk end [C]
  static constexpr int CL = ESF + C * 4;             // in-chunk prefix of log_a, fp64 [C]
  static constexpr int ST = CL + C * 8;              // level states [NSMAX]
  static constexpr int YX = ST + NSMAX * R_BYTES;    // partial outputs [4][64] f32x4
  static constexpr int LAM = YX + 4 * 64 * 16;       // lambda rows [C][L]
  __host__ __device__ static int bytes(int L) { return LAM + C * L * 4; }
};

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
}  // namespace b16

__global__ void __launch_bounds__(b16::NT) bwd_dq16_kernel(BwdArgs a) {
  using namespace b16;
  using Lay = DqLay;
  extern __shared__ __align__(16) unsigned char smem[];
  const int T = a.T, L = a.L, nslot = a.nslot, dk = a.dk, dv = a.dv;
  const int N = (T + C - 1) / C;
  bf16* Dh = reinterpret_cast<bf16*>(smem + Lay::DH);
  bf16* Dl = reinterpret_cast<bf16*>(smem + Lay::DL);
  bf16* Vs = reinterpret_cast<bf16*>(smem + Lay::VS);
  bf16* KTb = reinterpret_cast<bf16*>(smem + Lay::KT);
  float* Qs = reinterpret_cast<float*>(smem + Lay::QS);
  float* esf_s = reinterpret_cast<float*>(smem + Lay::ESF);
  double* cl_s = reinterpret_cast<double*>(smem + Lay::CL);
  unsigned char* Sbase = smem + Lay::ST;
  f32x4* Yx = reinterpret_cast<f32x4*>(smem + Lay::YX);
  float* lam_s = reinterpret_cast<float*>(smem + Lay::LAM);

  const int nsl = dk / 16;
  const int bh = blockIdx.x / nsl, js = blockIdx.x - bh * nsl;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int tt = w & 3, hf = w >> 2;  // query row tile, half
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const bf16* __restrict__ qg = static_cast<const bf16*>(a.q) + qkT * dk + 16 * js;
  const bf16* __restrict__ kg = static_cast<const bf16*>(a.k) + qkT * dk + 16 * js;
  const bf16* __restrict__ vg = static_cast<const bf16*>(a.v) + bhT * dv;
  const float* __restrict__ dog = a.dout + bhT * dv;
  const float* __restrict__ lag = a.log_a + bhT;
  const float* __restrict__ lamg = a.lam + bhT * L;
  float* __restrict__ dqg = a.dq + bhT * dk + 16 * js;
  const int nsl1 = nslot > 0 ? nslot : 1;
  float* __restrict__ part = a.dlam_part + ((size_t)js * a.BH + bh) * T * nsl1;

  // dlt[b] (chunk in the right half of level b): log decay from the level's
  // reference (last token of the left half) to the token before this chunk
  float dlt[NSMAX];
#pragma unroll
  for (int b = 0; b < NSMAX; ++b) dlt[b] = 0.f;
  float Aprev = 0.f;
  // register prefetch of one chunk (issued a chunk ahead of its staging)
  f32x4 pd[4];     // dO rows, 16-byte vectors tid + NT*i
  bf16x8 pv[2];    // v rows
  bf16x4 pk, pq;   // k and q slices (threads < 4C)
  float plam[4];   // lambda words tid + NT*i of the chunk
  float pla;       // log_a of token lane
  auto load = [&](int nn) {
    const int t0 = nn * C;
    pla = t0 + lane < T ? lag[t0 + lane] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, r = idx / (dv / 4), c = (idx - r * (dv / 4)) * 4;
      if (idx < C * dv / 4)
        pd[i] = t0 + r < T ? *reinterpret_cast<const f32x4*>(dog + (size_t)(t0 + r) * dv + c) : f32x4{};
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, r = idx / (dv / 8), c = (idx - r * (dv / 8)) * 8;
      if (idx < C * dv / 8)
        pv[i] = t0 + r < T ? *reinterpret_cast<const bf16x8*>(vg + (size_t)(t0 + r) * dv + c) : bf16x8{};
    }
    if (tid < 4 * C) {
      const int r = tid >> 2, c = (tid & 3) * 4;
      const bool ok = t0 + r < T;
      pk = ok ? *reinterpret_cast<const bf16x4*>(kg + (size_t)(t0 + r) * dk + c) : bf16x4{};
      pq = ok ? *reinterpret_cast<const bf16x4*>(qg + (size_t)(t0 + r) * dk + c) : bf16x4{};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i;
      if (idx < C * L) plam[i] = t0 + idx / L < T ? lamg[(size_t)t0 * L + idx] : 0.f;
    }
  };
  load(0);
  for (int n = 0; n < N; ++n) {
    const int tok0 = n * C;
    double Atd;
    const double cl = prefix_dpp(pla, lane, &Atd);
#pragma unroll
    for (int b = 0; b < NSMAX; ++b)
      if (b < nslot && ((n >> b) & 1)) {
        const int rs = ((n >> (b + 1)) << (b + 1)) + (1 << b);
        dlt[b] = uniform(n == rs ? 0.f : dlt[b] + Aprev);
      }
    // the level whose right half starts here has a complete left-half state:
    // converted to bf16 hi / lo in place after the staging barrier
    const int bc = n > 0 ? __builtin_ctz(static_cast<unsigned>(n)) : 32;
    const bool conv = bc < nslot;
    const int per = dv / 32;
    float rv[4];
    if (conv) {
      const float* Sf = reinterpret_cast<const float*>(Sbase + bc * R_BYTES) + (tid >> 5) * LDR + (tid & 31) * per;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < per) rv[e] = Sf[e];
    }

    // ---- stage chunk n from the registers (tokens past T are zero), then
    // prefetch chunk n + 1
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i, r = idx / (dv / 4), c = (idx - r * (dv / 4)) * 4;
      if (idx < C * dv / 4) {
        bf16x4 h, l;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          bf16 x1, x2;
          split_bf16(pd[i][e], x1, x2);
          h[e] = x1;
          l[e] = x2;
        }
        *reinterpret_cast<bf16x4*>(Dh + r * LDC + c) = h;
        *reinterpret_cast<bf16x4*>(Dl + r * LDC + c) = l;
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + NT * i, r = idx / (dv / 8), c = (idx - r * (dv / 8)) * 8;
      if (idx < C * dv / 8) *reinterpret_cast<bf16x8*>(Vs + r * LDC + c) = pv[i];
    }
    if (tid < 4 * C) {  // k and q slices: one token, four columns per thread
      const int r = tid >> 2, c = (tid & 3) * 4;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        KTb[(c + e) * LDAB + r] = pk[e];
        Qs[r * DqLay::LDQS + c + e] = static_cast<float>(pq[e]);
      }
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int idx = tid + NT * i;
      if (idx < C * L) lam_s[idx] = plam[i];
    }
    if (n + 1 < N) load(n + 1);
    if (w == 0) {
      cl_s[lane] = cl;
      esf_s[lane] = tok0 + lane < T ? __expf(static_cast<float>(Atd - cl)) : 0.f;
    }
    __syncthreads();
    if (conv) {
      bf16* Sh = reinterpret_cast<bf16*>(Sbase + bc * R_BYTES) + (tid >> 5) * LDR + (tid & 31) * per;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        if (e < per) {
          bf16 x1, x2;
          split_bf16(rv[e], x1, x2);
          Sh[e] = x1;
          Sh[16 * LDR + e] = x2;
        }
      __syncthreads();
    }

    // ---- intra chunk: this half's pair of s tiles (2hf, 2hf + 1) at or before tt
    f32x4 Y = {0.f, 0.f, 0.f, 0.f};
    if (2 * hf <= tt) {
      f32x4 z[2];
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        const int sb = 2 * hf + q;
        z[q] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (sb <= tt) {
          for (int k0 = 0; k0 < dv; k0 += 32) {
            const bf16x8 va = frag(Vs, LDC, 16 * sb, k0, lane);
            z[q] = mma(va, frag(Dh, LDC, 16 * tt, k0, lane), z[q]);
            z[q] = mma(va, frag(Dl, LDC, 16 * tt, k0, lane), z[q]);
          }
        }
      }
      // z[q][r] = v_s . dO_t, s = 16(2hf + q) + 4g4 + r, t = 16tt + li; masked in place
      const int t = 16 * tt + li;
      const double clt = cl_s[t];
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int sb = 2 * hf + q, s = 16 * sb + 4 * g4 + r;
          z[q][r] = (sb <= tt && s <= t)
                        ? z[q][r] * lam_s[t * L + level_of(t, s)] * __expf(static_cast<float>(clt - cl_s[s]))
                        : 0.f;
        }
      bf16x8 ph, pl;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 x1, x2;
        split_bf16(z[e >> 2][e & 3], x1, x2);
        ph[e] = x1;
        pl[e] = x2;
      }
      // dQ[t][j] += sum_s p[t][s] k_s[j]: the lane's eight s values are the
      // contraction slots of both operands
      const int s0 = 32 * hf + 4 * g4;
      const bf16x8 kb8 = cat(*reinterpret_cast<const bf16x4*>(KTb + li * LDAB + s0),
                             *reinterpret_cast<const bf16x4*>(KTb + li * LDAB + s0 + 16));
      Y = mma(ph, kb8, Y);
      Y = mma(pl, kb8, Y);
    }
    // Y[r]: t = 16tt + 4g4 + r, j = li

    // ---- inter chunk: right-half levels; the k-th live level goes to half
    // k & 1, and the zero dlambda partials of the other levels by parity.  Run
    // at raised wave priority (measured ~0.6% faster for the whole backward).
    __builtin_amdgcn_s_setprio(1);
    {
      bf16x8 dah[4], dal[4];
#pragma unroll
      for (int kq = 0; kq < 4; ++kq)
        if (32 * kq < dv) {
          dah[kq] = frag(Dh, LDC, 16 * tt, 32 * kq, lane);
          dal[kq] = frag(Dl, LDC, 16 * tt, 32 * kq, lane);
        }
      int rank = 0;
#pragma unroll
      for (int b = 0; b < NSMAX; ++b) {
        if (b >= nslot) continue;
        if (!((n >> b) & 1)) {  // no bucket at this level: zero partial
          if ((b & 1) == hf && li == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int t = tok0 + 16 * tt + 4 * g4 + r;
              if (t < T) part[(size_t)t * nslot + b] = 0.f;
            }
          }
          continue;
        }
        if (((rank++) & 1) != hf) continue;
        float x[4];
        {
          const bf16* Sh = reinterpret_cast<const bf16*>(Sbase + b * R_BYTES);
          const bf16* Sl = Sh + 16 * LDR;
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kq = 0; kq < 4; ++kq)
            if (32 * kq < dv) {
              const bf16x8 sh = frag(Sh, LDR, 0, 32 * kq, lane);
              acc = mma(dah[kq], sh, acc);
              acc = mma(dal[kq], sh, acc);
              acc = mma(dah[kq], frag(Sl, LDR, 0, 32 * kq, lane), acc);
            }
          // acc[r] = dO_t . St_b[j], t = 16tt + 4g4 + r, j = li
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 16 * tt + 4 * g4 + r;
            const float wt = __expf(static_cast<float>(cl_s[t]) + dlt[b]) * acc[r];
            Y[r] += lam_s[t * L + LOGC + 1 + b] * wt;
            x[r] = wt * Qs[t * DqLay::LDQS + li];
          }
        }
        // this slice's dlambda partial
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const float sx = row_sum16(x[r]);
          const int t = tok0 + 16 * tt + 4 * g4 + r;
          if (li == 0 && t < T) part[(size_t)t * nslot + b] = sx;
        }
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if (hf == 1) Yx[tt * 64 + lane] = Y;
    __syncthreads();
    if (hf == 0) {
      const f32x4 y2 = Yx[tt * 64 + lane];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = tok0 + 16 * tt + 4 * g4 + r;
        if (t < T) dqg[(size_t)t * dk + li] = Y[r] + y2[r];
      }
    }

    // ---- key side: this chunk joins the left half of every level whose bit
    // is clear and whose right half exists; one 16-column tile of v per wave
    if (16 * w < dv) {
      const int i0 = 16 * w;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        // A[j][s] = esf_s k_s[j], s = 32ks + 8g4 + e
        const bf16x8 kx = *reinterpret_cast<const bf16x8*>(KTb + li * LDAB + 32 * ks + 8 * g4);
        const f32x4 e0 = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4);
        const f32x4 e1 = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4 + 4);
        bf16x8 ah, al;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 x1, x2;
          split_bf16(static_cast<float>(kx[e]) * (e < 4 ? e0[e] : e1[e - 4]), x1, x2);
          ah[e] = x1;
          al[e] = x2;
        }
        const int off = (32 * ks + 8 * g4 + (li >> 2)) * LDC + i0 + 4 * (li & 3);
        const bf16x8 vb = cat(tr_read(Vs + off), tr_read(Vs + off + 4 * LDC));
        acc = mma(ah, vb, acc);
        acc = mma(al, vb, acc);
      }
      // acc[r] = sum_s esf_s k_s[j] v_s[i], j = 4g4 + r, i = i0 + li
      const float fa = __expf(static_cast<float>(Atd));
#pragma unroll
      for (int b = 0; b < NSMAX; ++b) {
        const int base = (n >> (b + 1)) << (b + 1);
        if (b < nslot && !((n >> b) & 1) && base + (1 << b) < N) {
          float* Sf = reinterpret_cast<float*>(Sbase + b * R_BYTES);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float* p = Sf + (4 * g4 + r) * LDR + i0 + li;
            *p = (n == base ? 0.f : *p * fa) + acc[r];
          }
        }
      }
    }
    Aprev = static_cast<float>(Atd);
    __syncthreads();
  }
}

bool bwd_dq16_ok(const BwdArgs& a) {
  return a.nslot <= b16::NSMAX && a.dv % 32 == 0 && a.dv <= 128 && b16::DqLay::bytes(a.L) <= kMaxLds;
}

int launch_bwd_dq16(const BwdArgs& a, hipStream_t s) {
  const int bytes = b16::DqLay::bytes(a.L);
  static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
  if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_dq16_kernel), raised)) return LL_ERR_HIP;
  hipLaunchKernelGGL(bwd_dq16_kernel, dim3(a.BH * (a.dk / 16)), dim3(b16::NT), bytes, s, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

// ---------------------------------------------------------------------------
// bwd_dlam_intra16_kernel: dlambda of the in-chunk levels 0..log2 C,
//   dlam[t, l] = sum_{s in the chunk, l(t,s) = l} exp(cum_t - cum_s) (q_t . k_s)(dO_t . v_s),
// one 256-thread workgroup per (b,h, chunk), wave w owning query rows 16w..
// The two score products run on bf16 matrix cores with fragments loaded
// straight from global memory (no LDS): q . k exact, dO split hi / lo.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_dlam_intra16_kernel(BwdArgs a) {
  using namespace b16;
  const int T = a.T, L = a.L, dk = a.dk, dv = a.dv;
  const int N = (T + C - 1) / C;
  const int bh = blockIdx.x / N, n = blockIdx.x - bh * N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int tok0 = n * C;
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const bf16* __restrict__ qg = static_cast<const bf16*>(a.q) + (qkT + tok0) * dk;
  const bf16* __restrict__ kg = static_cast<const bf16*>(a.k) + (qkT + tok0) * dk;
  const bf16* __restrict__ vg = static_cast<const bf16*>(a.v) + (bhT + tok0) * dv;
  const float* __restrict__ dog = a.dout + (bhT + tok0) * dv;
  __shared__ double cl_s[C];
  double Atot;
  const double cl = chunk_prefix(a.log_a + bhT, tok0, T, lane, &Atot);
  if (w == 0) cl_s[lane] = cl;
  __syncthreads();
  const int t = 16 * w + li;  // query row of this lane in the B operands
  const bool tok = tok0 + t < T;
  // B operands of this wave's query rows: q (exact) and dO (hi / lo)
  bf16x8 qb[4], dh[4], dl[4];
#pragma unroll
  for (int kq = 0; kq < 4; ++kq) {
    if (32 * kq < dk) qb[kq] = tok ? *reinterpret_cast<const bf16x8*>(qg + (size_t)t * dk + 32 * kq + 8 * g4) : bf16x8{};
    if (32 * kq < dv) {
      f32x4 x0 = {0.f, 0.f, 0.f, 0.f}, x1 = {0.f, 0.f, 0.f, 0.f};
      if (tok) {
        x0 = *reinterpret_cast<const f32x4*>(dog + (size_t)t * dv + 32 * kq + 8 * g4);
        x1 = *reinterpret_cast<const f32x4*>(dog + (size_t)t * dv + 32 * kq + 8 * g4 + 4);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16 h, l;
        split_bf16(e < 4 ? x0[e] : x1[e - 4], h, l);
        dh[kq][e] = h;
        dl[kq][e] = l;
      }
    }
  }
  float acc_l[LOGC + 1];
#pragma unroll
  for (int l = 0; l <= LOGC; ++l) acc_l[l] = 0.f;
  // key tiles 0..w; each tile's k and v rows are loaded one tile ahead
  bf16x8 kn[4], vn[4];
  auto load_kv = [&](int kb) {
    const int srow = 16 * kb + li;  // key row this lane loads for the A operands
    const bool sok = tok0 + srow < T;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      if (32 * kq < dk) kn[kq] = sok ? *reinterpret_cast<const bf16x8*>(kg + (size_t)srow * dk + 32 * kq + 8 * g4) : bf16x8{};
      if (32 * kq < dv) vn[kq] = sok ? *reinterpret_cast<const bf16x8*>(vg + (size_t)srow * dv + 32 * kq + 8 * g4) : bf16x8{};
    }
  };
  load_kv(0);
  for (int kb = 0; kb <= w; ++kb) {
    bf16x8 ka[4], va[4];
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      ka[kq] = kn[kq];
      va[kq] = vn[kq];
    }
    if (kb < w) load_kv(kb + 1);
    f32x4 z1 = {0.f, 0.f, 0.f, 0.f}, z2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      if (32 * kq < dk) z1 = mma(ka[kq], qb[kq], z1);
      if (32 * kq < dv) {
        z2 = mma(va[kq], dh[kq], z2);
        z2 = mma(va[kq], dl[kq], z2);
      }
    }
    // z1[r] = k_s . q_t, z2[r] = v_s . dO_t, s = 16kb + 4g4 + r
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int s = 16 * kb + 4 * g4 + r;
      if (s <= t) {
        const float x = z1[r] * z2[r] * __expf(static_cast<float>(cl_s[t] - cl_s[s]));
        const int lev = level_of(t, s);
#pragma unroll
        for (int l = 0; l <= LOGC; ++l) acc_l[l] += l == lev ? x : 0.f;
      }
    }
  }
  // sum over the four lane groups (keys 4g4 + r) of each query
  float* __restrict__ dl_out = a.dlam + (bhT + tok0 + t) * L;
#pragma unroll
  for (int l = 0; l <= LOGC; ++l) {
    float x = acc_l[l];
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    if (g4 == 0 && tok && l < L) dl_out[l] = x;
  }
}

bool bwd_dlam_intra16_ok(const BwdArgs& a) { return a.dk % 32 == 0 && a.dk <= 128 && a.dv % 32 == 0 && a.dv <= 128; }

int launch_bwd_dlam_intra16(const BwdArgs& a, hipStream_t s) {
  const int N = (a.T + b16::C - 1) / b16::C;
  hipLaunchKernelGGL(bwd_dlam_intra16_kernel, dim3(a.BH * N), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

bool bwd_kv16_ok(const BwdArgs& a) {
  if (a.nslot > b16::NSMAX) return false;
  for (int dc : {a.dk, a.dv})
    if (dc % 32 != 0 || dc > 128) return false;
  const int N = (a.T + b16::C - 1) / b16::C;
  return b16::KvLay<1>::bytes(a.L, N) <= kMaxLds && b16::KvLay<0>::bytes(a.L, N) <= kMaxLds;
}

int launch_bwd_kv16(const BwdArgs& a, hipStream_t s) {
  const int N = (a.T + b16::C - 1) / b16::C;
  {
    const int bytes = b16::KvLay<0>::bytes(a.L, N);
    static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
    if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_kv16_kernel<0>), raised)) return LL_ERR_HIP;
    hipLaunchKernelGGL(bwd_kv16_kernel<0>, dim3(a.BH * (a.dv / 16)), dim3(b16::NT), bytes, s, a);
  }
  {
    const int bytes = b16::KvLay<1>::bytes(a.L, N);
    static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
    if (!raise_lds_limit(reinterpret_cast<const void*>(&bwd_kv16_kernel<1>), raised)) return LL_ERR_HIP;
    hipLaunchKernelGGL(bwd_kv16_kernel<1>, dim3(a.BH * (a.dk / 16)), dim3(b16::NT), bytes, s, a);
  }
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
