// Log-linear attention forward on gfx950 (MI355X).
//
//   O = (Q K^T ⊙ M^S ⊙ M^H) V,  M^H[t,s] = lambda[t, level(t,s)],
//   M^S[t,s] = exp(cum[t] - cum[s])
//
// Pages (cited by title and section):
//   [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
//   [P2] "算力终结者来了！华人天团「降维打击」注意力瓶颈，AI狂飙进对数时代"
//
// Decomposition ([P1] 训练：分块并行扫描算法; [P2] 高效训练算法).  With chunk size
// C the level of a pair (t, s) in chunks n > m is log2(C) + bit_length(n ^ m),
// and pairs inside one chunk have level <= log2(C).  So every query of chunk n
// sees, besides its own chunk (dense, "intra"), one bucket of whole chunks per
// set bit b of n: the 2^b chunks just below n's bit b, at level log2(C)+1+b.
// The bucket's contribution is q_t^T G_{n,b} with G the decayed sum of k v^T
// over the bucket, weighted by lambda[t, log2(C)+1+b] and the decay from the
// bucket's end to t.
//
// Kernels (one pass over Q, one over K/V per dv slice; states stay on chip):
//   seg_state_kernel  per (b,h, segment of 2^S chunks): decayed sum of k v^T
//                     over the segment (bf16 / fp32 matrix cores).
//   seg_node_kernel   per (b,h, segment g >= 1, state element): the bucket
//                     state that starts at g, i.e. the merge the lssb rule
//                     ([P1] 解码) makes on the step into g.
//   fwd_sweep_kernel  per (b,h, segment, 16-wide dv slice): walks the
//                     segment's chunks in order, keeping the bucket states of
//                     levels inside the segment in LDS and merging them with
//                     the lssb rule at chunk granularity; bucket states of
//                     levels that span whole segments come from
//                     seg_node_kernel.  Per chunk: intra scores with the
//                     Fenwick level mask computed in registers, P·V, one
//                     Q·G product per live level, output, chunk state.
//
// bf16 path: Q, K, V are exact bf16 MFMA operands.  The masked scores P, the
// states G and the decay-scaled keys K~ are fp32 values; each is split into
// bf16 hi + lo and fed to two MFMAs so that its rounding error is ~2^-16
// instead of 2^-9 (a single bf16 K~ costs ~2e-2 of the output RMS once the
// decay is weak enough for distant chunks to matter).  fp32 path: fp32 MFMA.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <type_traits>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

__host__ __device__ constexpr int align16(int x) { return (x + 15) & ~15; }

template <int C>
struct Log2C;
template <>
struct Log2C<16> { static constexpr int v = 4; };
template <>
struct Log2C<32> { static constexpr int v = 5; };
template <>
struct Log2C<64> { static constexpr int v = 6; };

// LDS layout of fwd_sweep_kernel (bytes).  Used by the kernel and by the host
// to size the dynamic shared memory.
template <typename IT, int C, int DKP>
struct SweepCfg {
  static constexpr bool BF = sizeof(IT) == 2;
  static constexpr int NW = C / 16;          // waves; wave w owns query rows 16w..16w+15
  static constexpr int NT = NW * 64;
  static constexpr int PADE = BF ? 8 : 4;    // row padding (elements) against bank conflicts
  static constexpr int LDQ = DKP + PADE;     // K rows: [token][dk]
  static constexpr int CK = C < 32 ? 32 : C; // key extent of transposed operands (>= one bf16 K-step)
  static constexpr int LDK = CK + PADE;      // K~^T rows [dk][key], V^T rows [dv][key]
  static constexpr int LDG = DKP + PADE;     // state rows G^T [dv][dk]
  static constexpr int VEC = 16 / (int)sizeof(IT);
  static constexpr int LOGC = Log2C<C>::v;
  static constexpr int K_OFF = 0;
  static constexpr int KT_OFF = K_OFF + align16(C * LDQ * (int)sizeof(IT));
  // K~^T: bf16 keeps hi and lo halves (two consecutive [DKP][LDK] arrays)
  static constexpr int KT_BYTES = align16(DKP * LDK * (int)sizeof(IT)) * (BF ? 2 : 1);
  static constexpr int VT_OFF = KT_OFF + KT_BYTES;
  static constexpr int CL_OFF = VT_OFF + align16(16 * LDK * (int)sizeof(IT));
  static constexpr int LAM_OFF = CL_OFF + align16(C * 4);
  // one state slot: bf16 hi [16][LDG] + bf16 lo [16][LDG], or fp32 [16][LDG]
  static constexpr int SLOT_BYTES = 16 * LDG * 4;
  __host__ __device__ static int dec_off(int L) { return LAM_OFF + align16(C * L * 4); }
  __host__ __device__ static int st_off(int L, int nslot) {
    return dec_off(L) + align16((nslot > 0 ? nslot : 1) * 4);
  }
  __host__ __device__ static int bytes(int L, int nslot) { return st_off(L, nslot) + nslot * SLOT_BYTES; }
};

template <typename IT, int VEC>
struct VecOf;
template <>
struct VecOf<bf16, 8> { typedef bf16x8 type; };
template <>
struct VecOf<float, 4> { typedef f32x4 type; };

// ---------------------------------------------------------------------------
// fwd_sweep_kernel
// ---------------------------------------------------------------------------
template <typename IT, int C, int DKP>
__global__ void __launch_bounds__(C / 16 * 64)
fwd_sweep_kernel(FwdArgs a) {
  using Cfg = SweepCfg<IT, C, DKP>;
  using F = Frag<IT>;
  using vecT = typename VecOf<IT, Cfg::VEC>::type;
  constexpr int NW = Cfg::NW, NT = Cfg::NT, LDQ = Cfg::LDQ, CK = Cfg::CK, LDK = Cfg::LDK;
  constexpr int LDG = Cfg::LDG, VEC = Cfg::VEC, LOGC = Cfg::LOGC;
  constexpr bool BF = Cfg::BF;

  extern __shared__ __align__(16) unsigned char smem[];
  IT* Ks = reinterpret_cast<IT*>(smem + Cfg::K_OFF);
  IT* KtT = reinterpret_cast<IT*>(smem + Cfg::KT_OFF);
  IT* KtL = reinterpret_cast<IT*>(smem + Cfg::KT_OFF + Cfg::KT_BYTES / 2);  // bf16 lo half
  IT* VtT = reinterpret_cast<IT*>(smem + Cfg::VT_OFF);
  float* cl_s = reinterpret_cast<float*>(smem + Cfg::CL_OFF);
  float* lam_s = reinterpret_cast<float*>(smem + Cfg::LAM_OFF);
  float* dec_s = reinterpret_cast<float*>(smem + Cfg::dec_off(a.L));
  unsigned char* st = smem + Cfg::st_off(a.L, a.nslot);

  // Workgroup -> (pair p = (b,h,segment), dv slice ds).  The dv slices of one
  // pair share Q and K; they get consecutive ids with the same id % 8 so they
  // run together on one XCD and share its L2.
  const int D = a.dv >> 4;
  const int id = blockIdx.x;
  const int px = id & 7, rest = id >> 3;
  const int ds = rest % D, pg = rest / D;
  const int p = pg * 8 + px;
  if (p >= a.BH * a.nseg) return;
  const int bh = p / a.nseg, seg = p - bh * a.nseg;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int T = a.T, L = a.L, dk = a.dk, dv = a.dv;
  const int N = (T + C - 1) / C;
  const int n0 = seg << a.seg_log2;
  const int n1 = min(N, n0 + (1 << a.seg_log2));
  const size_t bhT = (size_t)bh * T, qkT = (size_t)(bh / a.G) * T;
  const IT* __restrict__ qg = static_cast<const IT*>(a.q) + qkT * dk;
  const IT* __restrict__ kg = static_cast<const IT*>(a.k) + qkT * dk;
  const IT* __restrict__ vg = static_cast<const IT*>(a.v) + bhT * dv + 16 * ds;
  const float* __restrict__ lag = a.log_a + bhT;
  const float* __restrict__ lamg = a.lam + bhT * L;
  float* __restrict__ outg = a.out + bhT * dv + 16 * ds;

  // Key columns >= C of the transposed operands are padding and must read 0.
  for (int i = tid; i < DKP * LDK; i += NT) KtT[i] = IT(0.f);
  if constexpr (BF)
    for (int i = tid; i < DKP * LDK; i += NT) KtL[i] = IT(0.f);
  for (int i = tid; i < 16 * LDK; i += NT) VtT[i] = IT(0.f);
  for (int i = tid; i < a.nslot; i += NT) dec_s[i] = 0.f;
  __syncthreads();

  // Prologue: bucket states of the levels that span whole segments.  Bit b >=
  // seg_log2 of the first chunk index is bit b' = b - seg_log2 of the segment
  // index; its bucket is the node that starts at segment (seg >> b') << b'.
  {
    unsigned bits = static_cast<unsigned>(n0);
    while (bits) {
      const int b = __builtin_ctz(bits);
      bits &= bits - 1;
      const int bp = b - a.seg_log2;
      const int gc = (seg >> bp) << bp;
      const float* __restrict__ node = a.nodes + ((size_t)(bh * a.nseg + gc) * dv + 16 * ds) * DKP;
      unsigned char* slot = st + b * Cfg::SLOT_BYTES;
      for (int i = tid; i < 16 * DKP; i += NT) {
        const int r = i / DKP, c = i - r * DKP;
        const float x = node[(size_t)r * DKP + c];
        if constexpr (BF) {
          bf16 h, l;
          split_bf16(x, h, l);
          reinterpret_cast<bf16*>(slot)[r * LDG + c] = h;
          reinterpret_cast<bf16*>(slot)[16 * LDG + r * LDG + c] = l;
        } else {
          reinterpret_cast<float*>(slot)[r * LDG + c] = x;
        }
      }
      if (tid == 0) {
        float d = 0.f;  // decay from the start of segment gc to the start of seg
        for (int r = gc; r < seg; ++r) d += a.seg_decay[bh * a.nseg + r];
        dec_s[b] = d;
      }
    }
  }
  __syncthreads();

  float Alast = 0.f;  // total log decay of the latest chunk
  for (int n = n0; n < n1; ++n) {
    const int tok0 = n * C;

    // In-chunk decay sums (every wave computes the same values, lane i <-> i):
    // cl = inclusive prefix of log_a, sf = exclusive suffix (decay to the
    // chunk's last token), Atot = chunk total.
    float la = 0.f;
    if (lane < C && tok0 + lane < T) la = lag[tok0 + lane];
    float cl = la;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_up(cl, off);
      if (lane >= off) cl += y;
    }
    float sf = __shfl_down(la, 1);
    if (lane == 63) sf = 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(sf, off);
      if (lane + off < 64) sf += y;
    }
    const float Atot = __shfl(cl, C - 1);
    Alast = Atot;
    if (w == 0 && lane < C) cl_s[lane] = cl;

    // This wave's 16 query rows as matrix-core fragments, straight from global
    // memory: they are the B operand of the score tiles and the A operand of
    // every Q.G product, so Q never goes through LDS.
    typename F::V qf[DKP / F::KS];
    {
      const int tq = tok0 + 16 * w + li;
#pragma unroll
      for (int i = 0; i < DKP / F::KS; ++i) {
        if constexpr (BF) {
          const int col = i * F::KS + 8 * g4;
          bf16x8 x = {};
          if (tq < T && col < dk) x = *reinterpret_cast<const bf16x8*>(qg + (size_t)tq * dk + col);
          qf[i] = x;
        } else {
          const int col = i * F::KS + g4;
          qf[i] = (tq < T && col < dk) ? qg[(size_t)tq * dk + col] : 0.f;
        }
      }
    }
    // Stage K (row-major) and K~^T = (K * exp(sf))^T; bf16 splits K~ into hi + lo.
    constexpr int RV = DKP / VEC;
#pragma unroll 2
    for (int idx = tid; idx < C * RV; idx += NT) {  // uniform trip count (DKP/(4*VEC))
      const int row = idx / RV, col = (idx - row * RV) * VEC;
      const int tok = tok0 + row;
      vecT kv = {};
      if (tok < T && col < dk) kv = *reinterpret_cast<const vecT*>(kg + (size_t)tok * dk + col);
      *reinterpret_cast<vecT*>(Ks + row * LDQ + col) = kv;
      const float sc = __expf(__shfl(sf, row));
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = static_cast<float>(kv[e]) * sc;
        if constexpr (BF) {
          bf16 h, l;
          split_bf16(x, h, l);
          KtT[(col + e) * LDK + row] = h;
          KtL[(col + e) * LDK + row] = l;
        } else {
          KtT[(col + e) * LDK + row] = x;
        }
      }
    }
    // Stage V^T of this 16-wide dv slice.
    constexpr int VV = 16 / VEC;
    for (int idx = tid; idx < C * VV; idx += NT) {
      const int row = idx / VV, col = (idx - row * VV) * VEC;
      const int tok = tok0 + row;
      vecT vv = {};
      if (tok < T) vv = *reinterpret_cast<const vecT*>(vg + (size_t)tok * dv + col);
#pragma unroll
      for (int e = 0; e < VEC; ++e) VtT[(col + e) * LDK + row] = vv[e];
    }
    // Stage lambda rows of the chunk.
    for (int idx = tid; idx < C * L; idx += NT) {
      const int tok = tok0 + idx / L;
      lam_s[idx] = tok < T ? lamg[(size_t)tok0 * L + idx] : 0.f;
    }
    __syncthreads();

    // ---------------- intra chunk: levels 0..log2(C) -----------------------
    const int qi = 16 * w + li;  // query row of this lane in the score tiles
    const float cl_q = cl_s[qi];
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
    constexpr int NP = (NW + 1) / 2;
    f32x4 P[2 * NP];
#pragma unroll
    for (int kb = 0; kb < 2 * NP; ++kb) {
      P[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (kb <= w) {
        // S^T tile: rows = keys 16kb.., columns = queries 16w..
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int k0 = 0; k0 < DKP; k0 += F::KS)
          acc = F::mma(F::load(Ks, LDQ, 16 * kb, k0, lane), qf[k0 / F::KS], acc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int kj = 16 * kb + 4 * g4 + r;
          float pv = 0.f;
          if (kj <= qi)  // chunk-local indices give the same level: tok0 is a multiple of C
            pv = acc[r] * lam_s[qi * L + level_of(qi, kj)] * __expf(cl_q - cl_s[kj]);
          P[kb][r] = pv;
        }
      }
    }
    // O = P V.  The S^T tile layout already is the A-operand layout of P with
    // the key index permuted; V^T is read with the same permutation.
    if constexpr (BF) {
#pragma unroll
      for (int pp = 0; pp < NP; ++pp) {
        if (2 * pp <= w) {
          bf16x8 ah, al;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16 h, l;
            split_bf16(P[2 * pp][r], h, l);
            ah[r] = h;
            al[r] = l;
            split_bf16(P[2 * pp + 1][r], h, l);
            ah[4 + r] = h;
            al[4 + r] = l;
          }
          const bf16* vb = VtT + li * LDK + 32 * pp + 4 * g4;
          const bf16x4 v0 = *reinterpret_cast<const bf16x4*>(vb);
          const bf16x4 v1 = *reinterpret_cast<const bf16x4*>(vb + 16);
          const bf16x8 bv = __builtin_shufflevector(v0, v1, 0, 1, 2, 3, 4, 5, 6, 7);
          O = F::mma(ah, bv, O);
          O = F::mma(al, bv, O);
        }
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < NW; ++kb) {
        if (kb <= w) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            O = F::mma(P[kb][r], VtT[li * LDK + 16 * kb + 4 * g4 + r], O);
        }
      }
    }

    // ---------------- inter chunk: one bucket per set bit of n -------------
    unsigned live = static_cast<unsigned>(n);
    while (live) {
      const int b = __builtin_ctz(live);
      live &= live - 1;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      const unsigned char* slot = st + b * Cfg::SLOT_BYTES;
      if constexpr (BF) {
        const bf16* gh = reinterpret_cast<const bf16*>(slot);
        const bf16* gl = gh + 16 * LDG;
#pragma unroll
        for (int i = 0; i < DKP / F::KS; ++i) {
          acc = F::mma(qf[i], F::load(gh, LDG, 0, i * F::KS, lane), acc);
          acc = F::mma(qf[i], F::load(gl, LDG, 0, i * F::KS, lane), acc);
        }
      } else {
        const float* gf = reinterpret_cast<const float*>(slot);
#pragma unroll
        for (int i = 0; i < DKP / F::KS; ++i) acc = F::mma(qf[i], F::load(gf, LDG, 0, i * F::KS, lane), acc);
      }
      const int lev = LOGC + 1 + b;
      const float db = dec_s[b];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * w + 4 * g4 + r;
        O[r] += lam_s[row * L + lev] * __expf(cl_s[row] + db) * acc[r];
      }
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int tok = tok0 + 16 * w + 4 * g4 + r;
      if (tok < T) outg[(size_t)tok * dv + li] = O[r];
    }

    // ---------------- chunk state and lssb merge (chunk granularity) -------
    // Transition n -> n+1 with m = lssb(n+1): the new level-m bucket is chunk
    // n plus the buckets of levels < m of n, all decayed to the end of chunk n.
    if (n + 1 < n1) {
      const int m = __builtin_ctz(static_cast<unsigned>(n + 1));
      for (int t = w; t < DKP / 16; t += NW) {
        // Decayed sum of the lower levels first; the chunk state is then
        // accumulated onto it by the MFMAs, whose result is consumed in the
        // same basic block (no branch between MFMA and the accumulator read).
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const int col0 = 16 * t + 4 * g4;  // dk index of acc[0]; li is the dv column
        for (int b = 0; b < m; ++b) {
          const float f = __expf(dec_s[b] + Atot);
          const unsigned char* slot = st + b * Cfg::SLOT_BYTES;
          if constexpr (BF) {
            const bf16* gh = reinterpret_cast<const bf16*>(slot) + li * LDG + col0;
            const bf16x4 h = *reinterpret_cast<const bf16x4*>(gh);
            const bf16x4 l = *reinterpret_cast<const bf16x4*>(gh + 16 * LDG);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += f * (static_cast<float>(h[r]) + static_cast<float>(l[r]));
          } else {
            const f32x4 x = *reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(slot) + li * LDG + col0);
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[r] += f * x[r];
          }
        }
#pragma unroll
        for (int k0 = 0; k0 < CK; k0 += F::KS) {
          const typename F::V vb = F::load(VtT, LDK, 0, k0, lane);
          acc = F::mma(F::load(KtT, LDK, 16 * t, k0, lane), vb, acc);
          if constexpr (BF) acc = F::mma(F::load(KtL, LDK, 16 * t, k0, lane), vb, acc);
        }
        unsigned char* slot = st + m * Cfg::SLOT_BYTES;
        if constexpr (BF) {
          bf16x4 h, l;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16 hh, ll;
            split_bf16(acc[r], hh, ll);
            h[r] = hh;
            l[r] = ll;
          }
          bf16* gh = reinterpret_cast<bf16*>(slot) + li * LDG + col0;
          *reinterpret_cast<bf16x4*>(gh) = h;
          *reinterpret_cast<bf16x4*>(gh + 16 * LDG) = l;
        } else {
          *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(slot) + li * LDG + col0) = acc;
        }
      }
    }
    __syncthreads();
    if (tid == 0 && n + 1 < n1) {
      const int m = __builtin_ctz(static_cast<unsigned>(n + 1));
      for (int b = m + 1; b < a.nslot; ++b) dec_s[b] += Atot;
      dec_s[m] = 0.f;
    }
  }

  // Prefill: decode states at T-1, inter-chunk levels.  The last segment ends
  // at the last chunk, whose bucket states are the level-(log2C+1+b) states of
  // its queries; decayed from each bucket's end to token T-1 (cl of the last
  // token is the chunk total, the tail reads zero).
  if (a.st_out && seg == a.nseg - 1 && n1 > n0) {
    const int nl = n1 - 1;
    float* __restrict__ so = a.st_out + (size_t)bh * a.st_L * dk * dv + 16 * ds;
    for (int lev = LOGC + 1; lev < a.st_L; ++lev) {
      const int b = lev - LOGC - 1;
      const bool live = b < a.nslot && ((nl >> b) & 1);
      const float f = live ? __expf(Alast + dec_s[b]) : 0.f;
      const unsigned char* slot = st + (live ? b : 0) * Cfg::SLOT_BYTES;
      for (int i = tid; i < 16 * dk; i += NT) {
        const int r = i / dk, c = i - r * dk;  // dv column r of the slice, dk index c
        float x = 0.f;
        if (live) {
          if constexpr (BF) {
            const bf16* gh = reinterpret_cast<const bf16*>(slot) + r * LDG + c;
            x = f * (static_cast<float>(gh[0]) + static_cast<float>(gh[16 * LDG]));
          } else {
            x = f * reinterpret_cast<const float*>(slot)[r * LDG + c];
          }
        }
        so[((size_t)lev * dk + c) * dv + r] = x;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// seg_state_kernel: T_g = sum_{s in segment g} exp(cum[end] - cum[s]) k_s v_s^T,
// stored transposed ([dv][DKP], fp32), plus the segment's total log decay.
// ---------------------------------------------------------------------------
template <typename IT, int DKP>
struct SegCfg {
  static constexpr bool BF = sizeof(IT) == 2;
  static constexpr int KB = 64;   // tokens per step
  static constexpr int NT = 256;
  static constexpr int PADE = BF ? 8 : 4;
  static constexpr int LDK = KB + PADE;
  static constexpr int DVG = 128;  // dv columns per workgroup
  static constexpr int VEC = 16 / (int)sizeof(IT);
  static constexpr int MAXT = (DKP / 16) * (DVG / 16) / 4;  // accumulator tiles per wave
  static constexpr int KT_OFF = 0;
  static constexpr int KT_BYTES = align16(DKP * LDK * (int)sizeof(IT)) * (BF ? 2 : 1);  // hi (+ lo)
  static constexpr int VT_OFF = KT_BYTES;
  static constexpr int BYTES = VT_OFF + align16(DVG * LDK * (int)sizeof(IT));
};

template <typename IT, int DKP>
__global__ void __launch_bounds__(256)
seg_state_kernel(SegArgs a) {
  using Cfg = SegCfg<IT, DKP>;
  using F = Frag<IT>;
  using vecT = typename VecOf<IT, Cfg::VEC>::type;
  constexpr int KB = Cfg::KB, NT = Cfg::NT, LDK = Cfg::LDK, VEC = Cfg::VEC, MAXT = Cfg::MAXT;

  extern __shared__ __align__(16) unsigned char smem[];
  IT* KtT = reinterpret_cast<IT*>(smem + Cfg::KT_OFF);
  IT* KtL = reinterpret_cast<IT*>(smem + Cfg::KT_OFF + Cfg::KT_BYTES / 2);  // bf16 lo half
  IT* VtT = reinterpret_cast<IT*>(smem + Cfg::VT_OFF);

  const int ndvg = (a.dv + Cfg::DVG - 1) / Cfg::DVG;
  const int nsg = a.nseg - 1;  // the last segment's state is never used
  const int id = blockIdx.x;
  const int dvg = id % ndvg, rest = id / ndvg;
  const int g = rest % nsg, bh = rest / nsg;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int T = a.T, dk = a.dk, dv = a.dv;
  const int segtok = a.C << a.seg_log2;
  const int s0 = g * segtok, s1 = min(T, s0 + segtok);
  const int dv0 = dvg * Cfg::DVG;
  const int dvw = min(Cfg::DVG, dv - dv0);
  const int nu = dvw >> 4;
  const int ntile = (DKP / 16) * nu;
  const size_t bhT = (size_t)bh * T;
  const IT* __restrict__ kg = static_cast<const IT*>(a.k) + (size_t)(bh / a.G) * T * dk;
  const IT* __restrict__ vg = static_cast<const IT*>(a.v) + bhT * dv + dv0;
  const float* __restrict__ lag = a.log_a + bhT;

  f32x4 acc[MAXT];
#pragma unroll
  for (int j = 0; j < MAXT; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float Aseg = 0.f;

  for (int b0 = s0; b0 < s1; b0 += KB) {
    float la = 0.f;
    if (b0 + lane < s1) la = lag[b0 + lane];
    float sf = __shfl_down(la, 1);
    if (lane == 63) sf = 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float y = __shfl_down(sf, off);
      if (lane + off < 64) sf += y;
    }
    const float Ab = __shfl(sf, 0) + __shfl(la, 0);  // block total
    constexpr int RV = DKP / VEC;
    for (int idx = tid; idx < KB * RV; idx += NT) {  // uniform trip count
      const int row = idx / RV, col = (idx - row * RV) * VEC;
      const int tok = b0 + row;
      vecT kv = {};
      if (tok < s1 && col < dk) kv = *reinterpret_cast<const vecT*>(kg + (size_t)tok * dk + col);
      const float sc = __expf(__shfl(sf, row));
#pragma unroll
      for (int e = 0; e < VEC; ++e) {
        const float x = static_cast<float>(kv[e]) * sc;
        if constexpr (Cfg::BF) {
          bf16 h, l;
          split_bf16(x, h, l);
          KtT[(col + e) * LDK + row] = h;
          KtL[(col + e) * LDK + row] = l;
        } else {
          KtT[(col + e) * LDK + row] = x;
        }
      }
    }
    const int vrow = dvw / VEC;
    for (int idx = tid; idx < KB * vrow; idx += NT) {
      const int row = idx / vrow, col = (idx - row * vrow) * VEC;
      const int tok = b0 + row;
      vecT vv = {};
      if (tok < s1) vv = *reinterpret_cast<const vecT*>(vg + (size_t)tok * dv + col);
#pragma unroll
      for (int e = 0; e < VEC; ++e) VtT[(col + e) * LDK + row] = vv[e];
    }
    __syncthreads();
    const float fa = __expf(Ab);
#pragma unroll
    for (int j = 0; j < MAXT; ++j) {
      const int ti = w + 4 * j;
      if (ti < ntile) {
        const int t = ti / nu, u = ti - t * nu;
        f32x4 c = acc[j];
#pragma unroll
        for (int r = 0; r < 4; ++r) c[r] *= fa;
#pragma unroll
        for (int k0 = 0; k0 < KB; k0 += F::KS) {
          const typename F::V vb = F::load(VtT, LDK, 16 * u, k0, lane);
          c = F::mma(F::load(KtT, LDK, 16 * t, k0, lane), vb, c);
          if constexpr (Cfg::BF) c = F::mma(F::load(KtL, LDK, 16 * t, k0, lane), vb, c);
        }
        acc[j] = c;
      }
    }
    Aseg += Ab;
    __syncthreads();
  }
  float* __restrict__ Tout = a.seg_state + ((size_t)(bh * a.nseg + g) * dv + dv0) * DKP;
#pragma unroll
  for (int j = 0; j < MAXT; ++j) {
    const int ti = w + 4 * j;
    if (ti < ntile) {
      const int t = ti / nu, u = ti - t * nu;
      *reinterpret_cast<f32x4*>(Tout + (size_t)(16 * u + li) * DKP + 16 * t + 4 * g4) = acc[j];
    }
  }
  if (tid == 0 && dvg == 0) a.seg_decay[bh * a.nseg + g] = Aseg;
}

// ---------------------------------------------------------------------------
// seg_node_kernel: the bucket state that starts at segment g >= 1.  With
// m = lssb(g) it covers segments [g - 2^m, g) (the merge the lssb rule makes
// on the step into g, [P1] 解码), decayed to the start of g.  It is summed
// from the block states T_j of those segments (R = 2^rlog2 blocks each):
//   node_g = sum_{j = (g - 2^m) R}^{g R - 1} exp(A_{j+1} + ... + A_{gR-1}) T_j,
// A_j the total log decay of block j.  The first workgroup of each (b,h, g)
// also writes the total log decay of segment g - 1.
// One thread per (b,h, g, four state elements).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) seg_node_kernel(NodeArgs a) {
  const int e = (blockIdx.x * 256 + threadIdx.x) * 4;  // four consecutive elements
  const int g = blockIdx.y + 1;
  const int bh = blockIdx.z;
  const size_t bbase = (size_t)bh * a.nblk1;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    float sd = 0.f;
    for (int j = (g - 1) << a.rlog2; j < g << a.rlog2; ++j) sd += a.blk_decay[bbase + j];
    a.seg_decay[(size_t)bh * a.nseg + g - 1] = sd;
  }
  if (e >= a.E) return;
  const int m = lssb(static_cast<uint32_t>(g));
  const int j0 = (g - (1 << m)) << a.rlog2;
  // each term is independent: weight exp(A_{j+1} + ... + A_{gR-1}), summed
  // from the end so the weights come out of one running sum
  f32x4 x = {0.f, 0.f, 0.f, 0.f};
  float d = 0.f;
#pragma unroll 4
  for (int j = (g << a.rlog2) - 1; j >= j0; --j) {
    const float wgt = __expf(d);
    const f32x4 t = *reinterpret_cast<const f32x4*>(a.blk_state + (bbase + j) * a.E + e);
#pragma unroll
    for (int r = 0; r < 4; ++r) x[r] += wgt * t[r];
    d += a.blk_decay[bbase + j];
  }
  *reinterpret_cast<f32x4*>(a.nodes + ((size_t)bh * a.nseg + g) * a.E + e) = x;
}

// ---------------------------------------------------------------------------
// level table export (test only): same device helper as the kernels.
// ---------------------------------------------------------------------------
// handoff_intra_kernel: the levels 0..log2(C) of the decode states at
// position t = T-1 (prefill -> decode).  Their buckets lie inside the last
// chunk: level 0 is {t}, level l >= 1 (when bit l-1 of t is set) the 2^(l-1)
// tokens below t's bit l-1 (page above, section 前缀的层次化分解).  Each is
// sum_s exp(cum[t] - cum[s]) k_s v_s^T in fp32.  One workgroup per (b,h, 64
// dv columns, level): the decay of each bucket token to t is one suffix sum of
// log_a over (lo, t] (a shuffle scan in one wave), the bucket's k and decayed v
// rows (at most C/2 tokens) are staged in LDS, and each thread forms 4 x 4
// blocks of the (dk, dv) state from float4 reads and writes them as float4
// rows.
template <typename IT>
__global__ void __launch_bounds__(256) handoff_intra_kernel(HandoffArgs a) {
  __shared__ __align__(16) float ks[32][128];  // k rows of the bucket
  __shared__ __align__(16) float vw[32][64];   // exp(cum[t] - cum[s]) v_s, this workgroup's columns
  __shared__ float es[32];                     // exp(cum[t] - cum[s]) per bucket token
  const int bh = blockIdx.x, dv0 = blockIdx.y * 64, lev = blockIdx.z;
  const int tid = threadIdx.x;
  const int T = a.T, dk = a.dk, dv = a.dv;
  const int t = T - 1;
  const size_t bhT = (size_t)bh * T;
  int lo = t, hi = t + 1;  // level 0: {t}
  if (lev > 0) {
    if ((t >> (lev - 1)) & 1) {
      lo = (t >> lev) << lev;
      hi = lo + (1 << (lev - 1));
    } else {
      lo = hi = 0;  // no bucket at this level
    }
  }
  const int nb = hi - lo;  // <= C / 2 <= 32
  const int ncol = min(64, dv - dv0);
  const IT* __restrict__ kg = static_cast<const IT*>(a.k) + (size_t)(bh / a.G) * T * dk;
  const IT* __restrict__ vg = static_cast<const IT*>(a.v) + bhT * dv;
  float* __restrict__ so = a.st_out + ((size_t)bh * a.st_L + lev) * dk * dv;
  if (nb > 0) {
    if (tid < 64) {
      // lane i holds log_a of token lo + 1 + i (tokens up to t; t - lo <= C - 1 <= 63);
      // the suffix sum from lane s is the log decay from token lo + s to t
      float x = tid < t - lo ? a.log_a[bhT + lo + 1 + tid] : 0.f;
      for (int off = 1; off < 64; off <<= 1) {
        const float y = __shfl_down(x, off);
        if (tid + off < 64) x += y;
      }
      if (tid < nb) es[tid] = __expf(x);
    }
    for (int i = tid; i < nb * dk; i += 256) {
      const int s = i / dk, d = i - s * dk;
      ks[s][d] = to_float(kg[(size_t)(lo + s) * dk + d]);
    }
  }
  __syncthreads();
  if (nb > 0) {
    for (int i = tid; i < nb * 64; i += 256) {
      const int s = i >> 6, j = i & 63;
      vw[s][j] = j < ncol ? es[s] * to_float(vg[(size_t)(lo + s) * dv + dv0 + j]) : 0.f;
    }
  }
  __syncthreads();
  // thread: columns 4jq..4jq+3, rows 4dq + 64u .. +3 (u = 0, 1)
  const int jq = tid & 15, dq = tid >> 4;
  const bool vec = ((reinterpret_cast<uintptr_t>(so) | static_cast<uintptr_t>(dv0 * 4) |
                     static_cast<uintptr_t>(dv * 4)) & 15) == 0;
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int d0 = 4 * dq + 64 * u;
    if (d0 >= dk || 4 * jq >= ncol) continue;
    f32x4 acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < nb; ++s) {
      const f32x4 kv = *reinterpret_cast<const f32x4*>(&ks[s][d0]);
      const f32x4 vv = *reinterpret_cast<const f32x4*>(&vw[s][4 * jq]);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] += kv[r] * vv;
    }
    const int nc = min(4, ncol - 4 * jq);  // columns of this group inside the slice
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (d0 + r >= dk) break;
      float* p = so + (size_t)(d0 + r) * dv + dv0 + 4 * jq;
      if (vec && nc == 4) {
        *reinterpret_cast<f32x4*>(p) = acc[r];
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c)
          if (c < nc) p[c] = acc[r][c];
      }
    }
  }
}

__global__ void __launch_bounds__(256) level_table_kernel(signed char* lev, int T) {
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (size_t)T * T) return;
  const int t = static_cast<int>(idx / T), s = static_cast<int>(idx - (size_t)t * T);
  lev[idx] = s <= t ? static_cast<signed char>(level_of(t, s)) : static_cast<signed char>(-1);
}

// ---------------------------------------------------------------------------
// host-side launchers
// ---------------------------------------------------------------------------
template <typename IT, int C, int DKP>
static int launch_sweep_t(const FwdArgs& a, int nblocks, hipStream_t stream) {
  using Cfg = SweepCfg<IT, C, DKP>;
  const int bytes = Cfg::bytes(a.L, a.nslot);
  if (bytes > kMaxLds) return LL_ERR_UNSUPPORTED;
  static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
  if (!raise_lds_limit(reinterpret_cast<const void*>(&fwd_sweep_kernel<IT, C, DKP>), raised)) return LL_ERR_HIP;
  hipLaunchKernelGGL((fwd_sweep_kernel<IT, C, DKP>), dim3(nblocks), dim3(Cfg::NT), bytes, stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

template <typename IT, int DKP>
static int launch_seg_t(const SegArgs& a, int nblocks, hipStream_t stream) {
  using Cfg = SegCfg<IT, DKP>;
  static std::atomic<uint64_t> raised{0};  // once per device: to the maximum, any size fits
  if (!raise_lds_limit(reinterpret_cast<const void*>(&seg_state_kernel<IT, DKP>), raised)) return LL_ERR_HIP;
  hipLaunchKernelGGL((seg_state_kernel<IT, DKP>), dim3(nblocks), dim3(Cfg::NT), Cfg::BYTES, stream, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

template <typename IT>
static int sweep_lds_t(int C, int DKP, int L, int nslot) {
#define LL_CASE(CC, DD) \
  if (C == CC && DKP == DD) return SweepCfg<IT, CC, DD>::bytes(L, nslot);
  LL_CASE(16, 32) LL_CASE(16, 64) LL_CASE(16, 128)
  LL_CASE(32, 32) LL_CASE(32, 64) LL_CASE(32, 128)
  LL_CASE(64, 32) LL_CASE(64, 64) LL_CASE(64, 128)
#undef LL_CASE
  return -1;
}

int sweep_lds_bytes(int dtype, int C, int DKP, int L, int nslot) {
  return dtype == LL_BF16 ? sweep_lds_t<bf16>(C, DKP, L, nslot) : sweep_lds_t<float>(C, DKP, L, nslot);
}

template <typename IT>
static int launch_sweep_dispatch(int C, int DKP, const FwdArgs& a, int nblocks, hipStream_t s) {
#define LL_CASE(CC, DD) \
  if (C == CC && DKP == DD) return launch_sweep_t<IT, CC, DD>(a, nblocks, s);
  LL_CASE(16, 32) LL_CASE(16, 64) LL_CASE(16, 128)
  LL_CASE(32, 32) LL_CASE(32, 64) LL_CASE(32, 128)
  LL_CASE(64, 32) LL_CASE(64, 64) LL_CASE(64, 128)
#undef LL_CASE
  return LL_ERR_UNSUPPORTED;
}

int launch_sweep(int dtype, int C, int DKP, const FwdArgs& a, int nblocks, hipStream_t s) {
  return dtype == LL_BF16 ? launch_sweep_dispatch<bf16>(C, DKP, a, nblocks, s)
                          : launch_sweep_dispatch<float>(C, DKP, a, nblocks, s);
}

int launch_handoff_intra(int dtype, const HandoffArgs& a, hipStream_t s) {
  if (a.BH <= 0) return LL_OK;
  if (a.C > 64 || a.dk > 128) return LL_ERR_UNSUPPORTED;  // buckets of <= 32 tokens, staged k rows
  int logc = 0;
  while ((1 << logc) < a.C) ++logc;
  const int nlev = std::min(logc + 1, a.st_L);
  const dim3 grid(static_cast<unsigned>(a.BH), static_cast<unsigned>((a.dv + 63) / 64), static_cast<unsigned>(nlev));
  if (dtype == LL_BF16)
    hipLaunchKernelGGL(handoff_intra_kernel<bf16>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(handoff_intra_kernel<float>, grid, dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int launch_seg_state(int dtype, int DKP, const SegArgs& a, int nblocks, hipStream_t s) {
  if (dtype == LL_BF16) {
    if (DKP == 32) return launch_seg_t<bf16, 32>(a, nblocks, s);
    if (DKP == 64) return launch_seg_t<bf16, 64>(a, nblocks, s);
    if (DKP == 128) return launch_seg_t<bf16, 128>(a, nblocks, s);
  } else {
    if (DKP == 32) return launch_seg_t<float, 32>(a, nblocks, s);
    if (DKP == 64) return launch_seg_t<float, 64>(a, nblocks, s);
    if (DKP == 128) return launch_seg_t<float, 128>(a, nblocks, s);
  }
  return LL_ERR_UNSUPPORTED;
}

int launch_seg_nodes(const NodeArgs& a, int BH, hipStream_t s) {
  if (a.nseg < 2) return LL_OK;
  if (a.E % 4 != 0) return LL_ERR_UNSUPPORTED;  // E = dv * DKP, DKP a multiple of 32
  hipLaunchKernelGGL(seg_node_kernel, dim3((a.E / 4 + 255) / 256, a.nseg - 1, BH), dim3(256), 0, s, a);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int launch_level_table(signed char* lev, int T, hipStream_t s) {
  const size_t n = (size_t)T * T;
  hipLaunchKernelGGL(level_table_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, s, lev, T);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

}  // namespace ll
