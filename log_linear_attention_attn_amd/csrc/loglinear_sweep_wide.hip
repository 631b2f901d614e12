// Full-width register-state chunk sweep for the bf16 forward with C = 64,
// 64 < dk <= 128 and dv = 128 (the log-linear Mamba-2 head shapes of the
// LM-scale and long-context workloads).  Same decomposition as the other
// sweeps ([P1] 训练：分块并行扫描算法 for the split into intra- and inter-chunk
// work; the chunk-granular Fenwick bucket states merged with the lssb rule of
// [P1] 解码：基于 lssb 的状态更新):
//
//   [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
//
// One 512-thread workgroup per (b,h, segment) covers all 128 dv columns, so
// the score tiles and their masks are formed once per chunk.  Wave w owns the
// 16 columns 16w..16w+15 over the whole of dk: the bucket states of the levels
// inside the segment (NREG levels x 128 dk x 16 columns, fp16 with a
// power-of-two scale per (level, wave)) never leave its registers, its Q.G
// products run over all of dk, so each output element is weighted once and no
// partial sums cross waves, and its chunk-state fold and merge touch only its
// own columns.  The levels that span whole segments are constant over the
// segment; node_pack_kernel builds them once as fp16 MFMA fragments (with
// their scales), and each chunk reads its wave's fragments from L2.
//
// Per chunk:
//   stage    Q, K, V arrived in LDS by direct-to-LDS loads issued during the
//            previous chunk (K, V, lambda and the in-chunk decay sums double-
//            buffered by chunk parity); lambda goes from registers to LDS;
//            every wave forms the in-chunk decay prefix with DPP.  Barrier.
//   phase 1  fp16 copy of Q (power-of-two scale per row); the 10 causal
//            16x16 score tiles shared out over the waves (bf16 MFMA), masked
//            in registers (Fenwick level x decay x lambda), split bf16 hi/lo
//            and parked in LDS in MFMA fragment order.  Barrier.
//   phase 2  per wave, no barrier: the transposed output O^T = G^T Q^T +
//            V^T P^T of its 16 columns, so a lane holds one query row and four
//            consecutive columns: Q.G_b for every live level (fp16 MFMA), each
//            weighted once by the lane's lambda of that level, P V (bf16
//            hi/lo), one 16-byte store per row tile; then the fold of this
//            chunk's state K^T (V*decay) into the bucket states for the next
//            chunk (lssb merge).
#include <hip/hip_runtime.h>

#include <algorithm>

#include "ll_device.h"
#include "ll_internal.h"

namespace ll {

namespace wd {

constexpr int C = 64, DKP = 128, LOGC = 6, NSLOT = 10, NTH = 512, DV = 128;
// Q, K and V tiles are [64 rows][128] bf16 without padding (rows of 256
// bytes, as the direct-to-LDS loads write them: 16 bytes per lane, a wave's
// 64 lanes contiguous), with the 16-byte chunks of row r permuted by
// swz(r) (see below) so that the fragment reads do not collide in banks.
// The fp16 copy of Q is written by the threads and keeps a padded row.
constexpr int LDQ = DKP + 8;                       // Qh row stride (fp16 elements)
constexpr int TILE = C * 128 * 2;                  // one unpadded 64 x 128 bf16 tile
// The Q tile and the two (chunk parity) K and V tiles are separate static
// LDS arrays, so the compiler sees that the next chunk's loads into one
// parity's tiles do not touch the other's (its waits then cover only the
// loads a read depends on).  The rest is dynamic LDS:
constexpr int QH_OFF = 0;                          // fp16 copy of Q, [64][LDQ]
constexpr int PS_OFF = QH_OFF + C * LDQ * 2;       // masked scores, hi/lo MFMA fragments
constexpr int PS_BYTES = 4 /*mi*/ * 2 /*ks*/ * 2 /*hi,lo*/ * 64 * 16;
constexpr int CL_OFF = PS_OFF + PS_BYTES;          // [2] x (cl[64], esf[64]) fp32 (chunk parity)
constexpr int ER_OFF = CL_OFF + 2 * 2 * C * 4;     // per-row output exponent cl*log2e + eq_row [64]
constexpr int LAM_OFF = ER_OFF + C * 4;            // lambda of the chunk [2][64 * L + 16] (parity)
// Rows past T of a ragged last chunk look up levels up to log2(C), and the
// level weights read all NSLOT inter-chunk levels, which a short sequence's
// lambda may lack; the slack keeps those (discarded) reads in bounds.
__host__ __device__ constexpr int lam_words(int L) { return C * L + 16; }
__host__ __device__ constexpr int lds_bytes(int L) { return LAM_OFF + 2 * lam_words(L) * 4; }
constexpr int kStaticLds = 5 * TILE;

// Chunk permutation of the unpadded tiles: the 16-byte chunk c of row r is
// stored at chunk position c ^ swz(r).  swz is a permutation of 0..15 over
// 16 consecutive rows (row-wise fragment reads: 16 rows, one chunk) and puts
// each of 4 consecutive rows in a different group of 4 chunks (transposed
// reads: 4 rows x 4 neighbouring chunks), so neither pattern repeats a bank.
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 2) | ((r >> 2) & 3); }
// element offset of (row r, column e) in an unpadded tile
__device__ __forceinline__ int toff(int r, int e) { return r * 128 + (((e >> 3) ^ swz(r)) << 3) + (e & 7); }

typedef short __attribute__((ext_vector_type(4))) s16x4;
typedef unsigned short __attribute__((ext_vector_type(2))) u16x2;
typedef unsigned int __attribute__((ext_vector_type(4))) u32x4;
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

template <int CTRL>
__device__ __forceinline__ float dpp_max(float x) {
  return fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false)));
}
// Max over the 64 lanes of a NON-NEGATIVE value, returned wave-uniform: DPP
// swaps within quads and rotations within 16-lane rows, then the four row
// maxima compared as integers (non-negative floats order like their bits).
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
__device__ __forceinline__ float exp2f_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float uniform(float x) {
  return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

__device__ __forceinline__ float exp2_int(int e) { return __uint_as_float(static_cast<unsigned>(e + 127) << 23); }

// s_waitcnt immediates (gfx9 encoding: vmcnt bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8; a field at its maximum does not wait).
constexpr int kWaitLgkm0 = 0xC07F;                // lgkmcnt(0)
constexpr int wait_vm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70 | 0xF00; }
// Workgroup barrier for LDS traffic: this wave's LDS operations are complete
// before it arrives; the compiler keeps memory accesses on their side of it.
// (Direct-to-LDS loads are waited for explicitly where their data is needed.)
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kOutOfRange = 0x80000000u;  // an offset past every range used here
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ bf16x8 load_b128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

}  // namespace wd

// EMIT: also write the prefill decode states of the inter-chunk levels (a
// separate instantiation, so the plain forward does not carry the extra code).
template <int NREG, int NNODE, bool EMIT>
__global__ void __launch_bounds__(512)
fwd_wide_kernel(FwdArgs a) {
  using namespace wd;
  __shared__ __align__(16) unsigned char q_tile[TILE];
  __shared__ __align__(16) unsigned char k_tile0[TILE], k_tile1[TILE];
  __shared__ __align__(16) unsigned char v_tile0[TILE], v_tile1[TILE];
  extern __shared__ __align__(16) unsigned char smem[];
  const bf16* Qs = reinterpret_cast<const bf16*>(q_tile);
  _Float16* Qh = reinterpret_cast<_Float16*>(smem + QH_OFF);
  bf16x8* Ps = reinterpret_cast<bf16x8*>(smem + PS_OFF);  // [mi][ks][hl][lane]
  float* er_s = reinterpret_cast<float*>(smem + ER_OFF);

  const int id = blockIdx.x;
  const int p = (id & 7) + ((id >> 3) << 3);
  if (p >= a.BH * a.nseg) return;
  const int bh = p / a.nseg, seg = p - bh * a.nseg;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const int c0 = 16 * w;  // this wave's dv columns
  const int T = a.T, L = a.L, dk = a.dk;
  const int N = (T + C - 1) / C;
  const int n0 = seg << a.seg_log2;
  const int n1 = min(N, n0 + (1 << a.seg_log2));
  const size_t bhT = (size_t)bh * T;
  // per-(b,h) slices; every slice is < 2^31 bytes (checked by the launcher)
  const size_t qkT = (size_t)(bh / a.G) * T;
  const rsrc_t qr = make_rsrc(static_cast<const bf16*>(a.q) + qkT * dk, T * dk * 2);
  const rsrc_t kr = make_rsrc(static_cast<const bf16*>(a.k) + qkT * dk, T * dk * 2);
  const rsrc_t vr = make_rsrc(static_cast<const bf16*>(a.v) + bhT * DV, T * DV * 2);
  const rsrc_t lar = make_rsrc(a.log_a + bhT, T * 4);
  const rsrc_t lamr = make_rsrc(a.lam + bhT * L, T * L * 4);
  const rsrc_t outr = make_rsrc(a.out + bhT * DV, T * DV * 4);

  // ---- bucket states of the levels inside the segment (b < seg_log2 =
  // NREG): G[b][kl] element e holds dk 32kl + 8g4 + e of column c0 + li, fp16
  // with a per-(level, wave) power-of-two scale: true value = stored *
  // 2^eg[b].  dec[b]: log decay since the state was formed.
  f16x8 G[NREG][4];
  int eg[NREG];
  float dec[NREG];
#pragma unroll
  for (int b = 0; b < NREG; ++b) {
    dec[b] = 0.f;
    eg[b] = 0;
#pragma unroll
    for (int kl = 0; kl < 4; ++kl) G[b][kl] = f16x8{};
  }
  // Levels spanning whole segments: level NREG + i is live for every chunk of
  // the segment when bit i of the segment index is set; its bucket is the node
  // starting at segment gc = (seg >> i) << i, packed by node_pack_kernel as
  // this wave's fp16 fragments (f16x8 [4 kl][64 lanes]) with exponent egn[i].
  // decn[i]: log decay from the node's end to the current chunk.
  const f16x8* __restrict__ node16 = static_cast<const f16x8*>(a.node16);
  const f16x8* nfrag[NNODE];
  int egn[NNODE];
  float decn[NNODE];
#pragma unroll
  for (int i = 0; i < NNODE; ++i) {
    nfrag[i] = nullptr;
    egn[i] = 0;
    decn[i] = 0.f;
    if ((seg >> i) & 1) {
      const int gc = (seg >> i) << i;
      const size_t slot = ((size_t)(bh * a.nseg + gc) * 8 + w);
      nfrag[i] = node16 + slot * (4 * 64) + lane;
      egn[i] = __builtin_amdgcn_readfirstlane(a.node_exp[slot]);
      float d = 0.f;
      for (int r = gc; r < seg; ++r) d += a.seg_decay[bh * a.nseg + r];
      decn[i] = uniform(d);
    }
  }

  // ---- loads of one chunk ------------------------------------------------
  // q, k, v go straight to LDS: wave w fills the 1 KiB blocks 2w and 2w+1 of
  // each tile (rows 4b .. 4b+3, lane -> row 4b + g4, chunk position li, which
  // holds the chunk li ^ swz(row) of that row).  Columns past dk (padded head
  // dim) get an out-of-range offset and read zero.  lambda and log_a go to
  // registers (staged by the threads).
  uint32_t dq_off[2], dv_off[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int row = 4 * (2 * w + j) + g4;
    const int col = 8 * (li ^ swz(row));
    dq_off[j] = static_cast<uint32_t>((row * dk + col) * 2) | (col < dk ? 0u : kOutOfRange);
    dv_off[j] = static_cast<uint32_t>((row * DV + col) * 2);
  }
  float plam[3];  // lambda words 2*tid, 2*tid+1 and, for L > 16, 1024+tid of the chunk
  float pla;
  // chunk n's loads into the tiles of its parity
  auto load_chunk = [&](int n) {
    const uint32_t tok0 = static_cast<uint32_t>(n * C);
    const uint32_t cq = tok0 * dk * 2, cv = tok0 * DV * 2;
    unsigned char* kbuf = n & 1 ? k_tile1 : k_tile0;
    unsigned char* vbuf = n & 1 ? v_tile1 : v_tile0;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int blk = (2 * w + j) * 1024;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(qr, (__attribute__((address_space(3))) void*)(q_tile + blk), 16,
                                               dq_off[j] + cq, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (__attribute__((address_space(3))) void*)(kbuf + blk), 16,
                                               dq_off[j] + cq, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (__attribute__((address_space(3))) void*)(vbuf + blk), 16,
                                               dv_off[j] + cv, 0, 0, 0);
    }
    // lambda words past C * L belong to the next chunk and are not staged
    const auto x = __builtin_amdgcn_raw_buffer_load_b64(lamr, (tok0 * L + 2 * tid) * 4, 0, 0);
    plam[0] = __uint_as_float(x[0]);
    plam[1] = __uint_as_float(x[1]);
    plam[2] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lamr, (tok0 * L + 1024 + tid) * 4, 0, 0));
    pla = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(lar, (tok0 + lane) * 4, 0, 0));
  };

  load_chunk(n0);
  // Four stores past the output range (the buffer resource drops them), so
  // the loop head sees the same outstanding vector-memory operations from the
  // prologue as from the previous chunk: the chunk's loads, then four output
  // stores.  The staging waits for the loads only (vmcnt(4)).
#pragma unroll
  for (int mi = 0; mi < 4; ++mi)
    __builtin_amdgcn_raw_buffer_store_b128(u32x4{0u, 0u, 0u, 0u}, outr, kOutOfRange + 16 * mi, 0, 0);

  float Aprev = 0.f;  // total log decay of the previous chunk
  for (int n = n0; n < n1; ++n) {
    const int tok0 = n * C, P = n & 1;
    const bf16* Ks = reinterpret_cast<const bf16*>(P ? k_tile1 : k_tile0);
    const bf16* Vs = reinterpret_cast<const bf16*>(P ? v_tile1 : v_tile0);
    float* cl_s = reinterpret_cast<float*>(smem + CL_OFF) + P * (2 * C);
    float* esf_s = cl_s + C;
    float* lam_s = reinterpret_cast<float*>(smem + LAM_OFF) + P * lam_words(L);
    // ---------------- stage ------------------------------------------------
    // this chunk's loads are complete (only the previous chunk's four stores
    // may still be in flight); lambda to LDS; in-chunk decay sums, every
    // wave: cl = inclusive prefix of log_a (lane = token); the decay from a
    // token to the chunk's last token is Atot - cl
    __builtin_amdgcn_s_waitcnt(wait_vm(4));
    if (tid * 2 < C * L) {  // C * L is even
      lam_s[tid * 2] = plam[0];
      lam_s[tid * 2 + 1] = plam[1];
    }
    if (1024 + tid < C * L) lam_s[1024 + tid] = plam[2];
    const float cl = wave_prefix_sum(pla);
    const float Atot = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cl), 63));
    if (w == 0) {
      cl_s[lane] = cl * kLog2e;  // base-2 units for the score decays
      esf_s[lane] = __expf(Atot - cl);
    }
    lds_barrier();

    // ---------------- phase 1 ----------------------------------------------
    // fp16 copy of Q for the Q.G products, each row scaled by a power of two
    // so its max |q| sits at 2^14..2^15 (exact for bf16 values in range): the
    // 16 lanes holding a row share its max through DPP row rotations; the
    // row's exponent goes into its output factor.
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int v = tid + NTH * i, row = v >> 4, col = (v & 15) * 8;
      const bf16x8 x = *reinterpret_cast<const bf16x8*>(Qs + toff(row, col));
      const uint4 bits = __builtin_bit_cast(uint4, x);
      u16x2 qm = __builtin_bit_cast(u16x2, bits.x & 0x7fff7fffu);
      qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.y & 0x7fff7fffu));
      qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.z & 0x7fff7fffu));
      qm = __builtin_elementwise_max(qm, __builtin_bit_cast(u16x2, bits.w & 0x7fff7fffu));
      float mx = __uint_as_float(max(static_cast<unsigned>(qm[0]), static_cast<unsigned>(qm[1])) << 16);
      mx = dpp_max<0x121>(mx);  // row_ror:1
      mx = dpp_max<0x122>(mx);  // row_ror:2
      mx = dpp_max<0x124>(mx);  // row_ror:4
      mx = dpp_max<0x128>(mx);  // row_ror:8
      const int eq = scale_exp(mx);
      const float sc = exp2_int(-eq);
      f16x8 hq;
#pragma unroll
      for (int e = 0; e < 8; ++e) hq[e] = static_cast<_Float16>(static_cast<float>(x[e]) * sc);
      *reinterpret_cast<f16x8*>(Qh + row * LDQ + col) = hq;
      if ((v & 15) == 0) er_s[row] = cl_s[row] + static_cast<float>(eq);
    }

    // masked score tiles -> LDS.  Waves 0..3 take the diagonal tile (w,w)
    // (per-element levels, the costlier mask); waves 4..7 take (1,0) (2,0)
    // (2,1) (3,0), and waves 4 and 5 also (3,1) and (3,2).  Waves 2 and 3
    // zero the slots above the diagonal inside the last K-step of an even
    // query block, (0,1) and (2,3).
    {
      const int ntile = w == 4 || w == 5 ? 2 : 1;
      int qbt[2], kbt[2];
      if (w < 4) { qbt[0] = w; kbt[0] = w; }
      else if (w == 4) { qbt[0] = 1; kbt[0] = 0; }
      else if (w == 5) { qbt[0] = 2; kbt[0] = 0; }
      else if (w == 6) { qbt[0] = 2; kbt[0] = 1; }
      else { qbt[0] = 3; kbt[0] = 0; }
      qbt[1] = 3;
      kbt[1] = w == 4 ? 1 : 2;
      f32x4 acc[2];
      acc[0] = f32x4{0.f, 0.f, 0.f, 0.f};
      acc[1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          if (it < ntile) {
            const int kr_ = 16 * kbt[it] + li, qr_ = 16 * qbt[it] + li;
            const bf16x8 ka = *reinterpret_cast<const bf16x8*>(Ks + toff(kr_, 32 * ks + 8 * g4));
            const bf16x8 qb8 = *reinterpret_cast<const bf16x8*>(Qs + toff(qr_, 32 * ks + 8 * g4));
            acc[it] = mma(ka, qb8, acc[it]);
          }
        }
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        if (it < ntile) {
          const int qb = qbt[it], kb = kbt[it];
          // acc[r] = score(query 16qb+li, key 16kb+4g4+r)
          const int qi = 16 * qb + li;
          const float clq = cl_s[qi];
          const f32x4 clk = *reinterpret_cast<const f32x4*>(cl_s + 16 * kb + 4 * g4);
          f32x4 pv4;
          if (kb < qb) {
            const float lam = lam_s[qi * L + 4 + (32 - __clz(qb ^ kb))];
#pragma unroll
            for (int r = 0; r < 4; ++r) pv4[r] = acc[it][r] * lam * exp2f_fast(clq - clk[r]);
          } else {
            // diagonal tile: same 16-block, so the level (query li, key
            // 4g4 + r inside the block, 0..4) and the causal mask depend on
            // the in-block positions only; the row's five level weights are
            // read once
            float lr[5];
#pragma unroll
            for (int l = 0; l < 5; ++l) lr[l] = lam_s[qi * L + l];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int lev = level_of(li, 4 * g4 + r);
              float lam = lr[0];
#pragma unroll
              for (int l = 1; l < 5; ++l) lam = lev == l ? lr[l] : lam;
              pv4[r] = 4 * g4 + r <= li ? acc[it][r] * lam * exp2f_fast(clq - clk[r]) : 0.f;
            }
          }
          bf16x4 h, l;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            bf16 x1, x2;
            split_bf16(pv4[r], x1, x2);
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
    lds_barrier();

    // ---------------- phase 2 (per wave) -----------------------------------

    // Transposed output tiles: O^T = sum_b w_b G_b^T Q^T + V^T P^T for query
    // rows 16mi..16mi+15, one row tile at a time (Q.G, P V, store); lane
    // (li, g4) holds query 16mi + li and the columns c0 + 4g4 + r, r = 0..3.
    // The weight of level b for the lane's row is lambda[row, log2C+1+b] *
    // exp(dec_b) * 2^eg_b (per-lane scalar); the level-independent factor
    // exp(cl_row) * 2^eq_row follows once.  V^T operand: keys in the score
    // tile order (32ks + 4g4 + e, then +16), by transposed reads.
    bf16x8 vb[2];
    float fn[NNODE];
    f16x8 NG[NNODE][4];
    auto qg_pv_store = [&]() {
#pragma unroll
      for (int mi = 0; mi < 4; ++mi) {
        const int row = 16 * mi + li;
        f16x8 qa[4];
#pragma unroll
        for (int kl = 0; kl < 4; ++kl)
          qa[kl] = *reinterpret_cast<const f16x8*>(Qh + row * LDQ + 32 * kl + 8 * g4);
        const float* lrow = lam_s + row * L + LOGC + 1;
        f32x4 o = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NREG; ++b) {
          if ((n >> b) & 1) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kl = 0; kl < 4; ++kl) acc = mma16(G[b][kl], qa[kl], acc);
            const float wv = lrow[b] * (__expf(dec[b]) * exp2_int(eg[b]));
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] += wv * acc[r];
          }
        }
#pragma unroll
        for (int i = 0; i < NNODE; ++i) {
          if ((seg >> i) & 1) {
            f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kl = 0; kl < 4; ++kl) acc = mma16(NG[i][kl], qa[kl], acc);
            const float wv = lrow[NREG + i] * fn[i];
#pragma unroll
            for (int r = 0; r < 4; ++r) o[r] += wv * acc[r];
          }
        }
        const float er = exp2f_fast(er_s[row]);
#pragma unroll
        for (int r = 0; r < 4; ++r) o[r] *= er;
        // V^T P^T: row tile mi reads key steps ks <= mi / 2
#pragma unroll
        for (int ks = 0; ks <= mi / 2; ++ks) {
          o = mma(vb[ks], Ps[((mi * 2 + ks) * 2 + 0) * 64 + lane], o);
          o = mma(vb[ks], Ps[((mi * 2 + ks) * 2 + 1) * 64 + lane], o);
        }
        // rows past T fall outside the output range and are dropped
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), outr, ((tok0 + row) * DV + c0 + 4 * g4) * 4,
                                               0, 0);
      }
    };
    // ---------------- this chunk's state + lssb merge (registers) ----------
    // Chunk n -> n+1: its state joins the buckets the next chunk reads.  The
    // merge writes level m = lssb(n+1), which chunk n does not read (bit m of
    // n is clear), and only reads the levels below it.  K and V of chunk n
    // stay in their parity buffer until the loads of chunk n+2, issued after
    // the next chunk's second barrier.
    // The fold writes only level m's state and scale, which chunk n's Q.G
    // does not read, so it can go first; the decay bookkeeping of the other
    // levels is committed after both.
    const bool fold_next = n + 1 < n1;
    const int m = fold_next ? __builtin_ctz(static_cast<unsigned>(n + 1)) : 0;
    auto fold = [&]() {
      // decayed V of this wave's columns, tokens 32ks + 8g4 + e, split hi/lo
      bf16x8 vh[2], vl[2];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int r0 = 32 * ks + 8 * g4 + (li >> 2), e0 = c0 + 4 * (li & 3);
        const bf16x8 x = cat(tr_read(Vs + toff(r0, e0)), tr_read(Vs + toff(r0 + 4, e0)));
        const f32x4 e0v = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4);
        const f32x4 e1v = *reinterpret_cast<const f32x4*>(esf_s + 32 * ks + 8 * g4 + 4);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          bf16 x1, x2;
          split_bf16(static_cast<float>(x[e]) * (e < 4 ? e0v[e] : e1v[e - 4]), x1, x2);
          vh[ks][e] = x1;
          vl[ks][e] = x2;
        }
      }
      // S tiles t = 2*kl + half cover dk 32kl + 8*(row>>2) + 4*half + (row&3);
      // S[t][r] is element 4*half + r of G[.][kl].  The lower levels, decayed
      // to the end of chunk n, start the accumulators.  Two passes over dk
      // halves (kl 0-1, then 2-3) keep the live accumulators at 16 registers;
      // the new state's scale comes from the max over both.
      float flv[NREG];
#pragma unroll
      for (int b = 0; b < NREG; ++b) flv[b] = b < m ? __expf(dec[b] + Atot) * exp2_int(eg[b]) : 0.f;
      f32x4 S[2][4];
#pragma unroll
      for (int hp = 0; hp < 2; ++hp) {
#pragma unroll
        for (int t = 0; t < 4; ++t) S[hp][t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int b = 0; b < NREG - 1; ++b) {
          if (b < m) {
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
              for (int r = 0; r < 4; ++r)
                S[hp][t][r] += flv[b] * static_cast<float>(G[b][2 * hp + (t >> 1)][4 * (t & 1) + r]);
          }
        }
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int kl = 2 * hp + (t >> 1), half = t & 1;
            const int r0 = 32 * ks + 8 * g4 + (li >> 2), e0 = 32 * kl + 8 * (li & 3) + 4 * half;
            const bf16x8 ka = cat(tr_read(Ks + toff(r0, e0)), tr_read(Ks + toff(r0 + 4, e0)));
            S[hp][t] = mma(ka, vh[ks], S[hp][t]);
            S[hp][t] = mma(ka, vl[ks], S[hp][t]);
          }
        }
      }
      float mx = 0.f;
#pragma unroll
      for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(S[hp][t][r]));
      const int em = scale_exp(wave_max(mx));
      const float sc = exp2_int(-em);
      f16x8 gn[4];
#pragma unroll
      for (int hp = 0; hp < 2; ++hp)
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            gn[2 * hp + (t >> 1)][4 * (t & 1) + r] = static_cast<_Float16>(S[hp][t][r] * sc);
#pragma unroll
      for (int b = 0; b < NREG; ++b) {
        if (b == m) {
#pragma unroll
          for (int kl = 0; kl < 4; ++kl) G[b][kl] = gn[kl];
          eg[b] = em;
        }
      }
    };
    // Order: the fold and the V^T fragments (every read of this chunk's K
    // and V tiles), then the next chunk's loads into the other parity's tiles
    // and the Q tile (the compiler cannot tell the parities apart, so no read
    // of a K / V tile may follow them), then Q.G, P V and the stores.
    if (fold_next) fold();
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int r0 = 32 * ks + 4 * g4 + (li >> 2), e0 = c0 + 4 * (li & 3);
      vb[ks] = cat(tr_read(Vs + toff(r0, e0)), tr_read(Vs + toff(r0 + 16, e0)));
    }
    // the live segment-spanning levels' fragments (L2 hits: every chunk of
    // the segment reads the same ones); used last in Q.G
#pragma unroll
    for (int i = 0; i < NNODE; ++i) {
      fn[i] = uniform(__expf(decn[i]) * exp2_int(egn[i]));
#pragma unroll
      for (int kl = 0; kl < 4; ++kl) NG[i][kl] = f16x8{};
      if ((seg >> i) & 1) {  // wave-uniform; nfrag[i] is set for live levels only
#pragma unroll
        for (int kl = 0; kl < 4; ++kl) NG[i][kl] = nfrag[i][kl * 64];
      }
    }
    // (the scheduler sees these as plain global loads; the sched barriers
    // keep them after the fold's reads of the K / V tiles)
    __builtin_amdgcn_sched_barrier(0);
    load_chunk(n + 1);
    __builtin_amdgcn_sched_barrier(0);
    qg_pv_store();
    if (fold_next) {
#pragma unroll
      for (int b = 0; b < NREG; ++b) dec[b] = uniform(b == m ? 0.f : (b > m ? dec[b] + Atot : dec[b]));
    }
#pragma unroll
    for (int i = 0; i < NNODE; ++i) decn[i] = uniform(decn[i] + Atot);
    Aprev = Atot;
  }
  // the last chunk's loads of the following rows (never used) and its stores
  // are left to complete on their own; nothing reads them
  __builtin_amdgcn_s_waitcnt(wait_vm(0));

  // ---------------- prefill: decode states at T-1, inter-chunk levels -------
  // The last segment ends at the last chunk, whose bucket states are the
  // level-(log2C+1+b) states of its queries; decayed from each bucket's end to
  // token T-1 (cl of the last token = the chunk total, the tail reads zero).
  if (EMIT && seg == a.nseg - 1 && n1 > n0) {
    const int nl = n1 - 1;
    float* __restrict__ so = a.st_out + (size_t)bh * a.st_L * dk * DV + c0 + li;
    for (int lev = LOGC + 1; lev < a.st_L; ++lev) {
      const int b = lev - LOGC - 1;
      float f = 0.f;
      f16x8 g[4] = {f16x8{}, f16x8{}, f16x8{}, f16x8{}};
#pragma unroll
      for (int bb = 0; bb < NREG; ++bb) {
        if (bb == b && ((nl >> bb) & 1)) {
          f = __expf(Aprev + dec[bb]) * exp2_int(eg[bb]);
#pragma unroll
          for (int kl = 0; kl < 4; ++kl) g[kl] = G[bb][kl];
        }
      }
      // decn already holds the decay to the end of the last chunk
#pragma unroll
      for (int i = 0; i < NNODE; ++i) {
        if (NREG + i == b && ((seg >> i) & 1)) {
          f = __expf(decn[i]) * exp2_int(egn[i]);
#pragma unroll
          for (int kl = 0; kl < 4; ++kl) g[kl] = nfrag[i][kl * 64];
        }
      }
#pragma unroll
      for (int kl = 0; kl < 4; ++kl)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int d = 32 * kl + 8 * g4 + e;  // dk index of G[.][kl][e]
          if (d < dk) so[((size_t)lev * dk + d) * DV] = f * static_cast<float>(g[kl][e]);
        }
    }
  }
}

// Bucket node states packed for the full-width sweep.  The node starting at
// segment g >= 1 is the bucket formed by the lssb merge on the step into
// segment g: the decayed sum of the block states of the 2^lssb(g) segments
// before it,
//   node_g = sum_{j = (g - 2^m) R}^{g R - 1} exp(A_{j+1} + ... + A_{gR-1}) T_j,
// A_j the total log decay of block j (R blocks per segment).  Written as the
// fp16 B fragments each wave of the sweep multiplies (wave w: columns
// 16w..16w+15, lane (li, g4), fragment kl: dk 32kl + 8g4 + e) with one
// power-of-two exponent per (node, wave), so the sweep reads them with one
// 16-byte load per lane and fragment.  Workgroup (g - 1, bh) also writes the
// total log decay of segment g - 1.
__global__ void __launch_bounds__(512) node_pack_kernel(NodeArgs a, f16x8* __restrict__ out,
                                                         int* __restrict__ out_exp) {
  using namespace wd;
  const int g = blockIdx.x + 1;
  const int bh = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g4 = lane >> 4;
  const size_t bbase = (size_t)bh * a.nblk1;
  if (tid == 0) {
    float sd = 0.f;
    for (int j = (g - 1) << a.rlog2; j < g << a.rlog2; ++j) sd += a.blk_decay[bbase + j];
    a.seg_decay[(size_t)bh * a.nseg + g - 1] = sd;
  }
  const int m = lssb(static_cast<uint32_t>(g));
  const int j0 = (g - (1 << m)) << a.rlog2;
  f32x4 x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  // summed from the end so the weights come out of one running sum
  float d = 0.f;
  for (int j = (g << a.rlog2) - 1; j >= j0; --j) {
    const float wgt = __expf(d);
    const float* __restrict__ src = a.blk_state + (bbase + j) * a.E + (size_t)(16 * w + li) * DKP + 8 * g4;
#pragma unroll
    for (int kl = 0; kl < 4; ++kl)
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const f32x4 t = *reinterpret_cast<const f32x4*>(src + 32 * kl + 4 * h);
#pragma unroll
        for (int r = 0; r < 4; ++r) x[2 * kl + h][r] += wgt * t[r];
      }
    d += a.blk_decay[bbase + j];
  }
  float mx = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, fabsf(x[i][r]));
  const int e2 = scale_exp(wave_max(mx));
  const float sc = exp2_int(-e2);
  const size_t slot = ((size_t)bh * a.nseg + g) * 8 + w;
#pragma unroll
  for (int kl = 0; kl < 4; ++kl) {
    f16x8 f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      f[e] = static_cast<_Float16>(x[2 * kl][e] * sc);
      f[4 + e] = static_cast<_Float16>(x[2 * kl + 1][e] * sc);
    }
    out[(slot * 4 + kl) * 64 + lane] = f;
  }
  if (lane == 0) out_exp[slot] = e2;
}

// Instantiations: NREG = seg_log2 levels in registers, NNODE segment-spanning
// levels read per chunk.
bool sweep_wide_seg_ok(int seg_log2, int nslot) {
  switch (seg_log2) {
    case 3: case 4: case 6: return nslot <= seg_log2 + 4;
    case 5: return nslot <= 8;
    default: return false;
  }
}

bool sweep_wide_ok(int C, int dk, int dv, int L, int nslot, int seg_log2) {
  return C == wd::C && dk > 64 && dk <= wd::DKP && dv == wd::DV && nslot <= wd::NSLOT && L <= 17 &&
         wd::lds_bytes(L) + wd::kStaticLds <= kMaxLds && (seg_log2 < 0 || sweep_wide_seg_ok(seg_log2, nslot));
}

size_t node_pack_bytes(int BH, int nseg) {
  return (size_t)BH * nseg * 8 * (4 * 64 * 16 + sizeof(int));
}

int launch_node_pack(const NodeArgs& a, void* node16, int* node_exp, int BH, hipStream_t stream) {
  if (a.nseg < 2) return LL_OK;
  if (a.E != wd::DV * wd::DKP) return LL_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(node_pack_kernel, dim3(a.nseg - 1, BH), dim3(512), 0, stream, a,
                     static_cast<f16x8*>(node16), node_exp);
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

template <int NREG, int NNODE>
static int launch_wide_inst(const FwdArgs& a, unsigned nblocks, int bytes, hipStream_t stream) {
  static std::atomic<uint64_t> raised_plain{0}, raised_emit{0};
  if (a.st_out) {
    if (!raise_lds_limit(reinterpret_cast<const void*>(&fwd_wide_kernel<NREG, NNODE, true>), raised_emit,
                         kMaxLds - wd::kStaticLds))
      return LL_ERR_HIP;
    hipLaunchKernelGGL((fwd_wide_kernel<NREG, NNODE, true>), dim3(nblocks), dim3(wd::NTH), bytes, stream, a);
  } else {
    if (!raise_lds_limit(reinterpret_cast<const void*>(&fwd_wide_kernel<NREG, NNODE, false>), raised_plain,
                         kMaxLds - wd::kStaticLds))
      return LL_ERR_HIP;
    hipLaunchKernelGGL((fwd_wide_kernel<NREG, NNODE, false>), dim3(nblocks), dim3(wd::NTH), bytes, stream, a);
  }
  return hipGetLastError() == hipSuccess ? LL_OK : LL_ERR_HIP;
}

int launch_sweep_wide(const FwdArgs& a, hipStream_t stream) {
  if (!sweep_wide_ok(wd::C, a.dk, a.dv, a.L, a.nslot, a.seg_log2)) return LL_ERR_UNSUPPORTED;
  if (a.nseg > 1 && (!a.node16 || !a.node_exp)) return LL_ERR_UNSUPPORTED;
  const int bytes = wd::lds_bytes(a.L);
  // buffer offsets are 32-bit: every per-(b,h) slice, tail chunk included,
  // must stay below 2^31 bytes
  const size_t row_bytes = std::max({(size_t)a.dk * 2, (size_t)a.dv * 4, (size_t)a.L * 4});
  if ((size_t)(a.T + 2 * wd::C) * row_bytes >= (size_t)1 << 31) return LL_ERR_UNSUPPORTED;
  const long long pairs = (long long)a.BH * a.nseg;
  const long long nblocks = (pairs + 7) / 8 * 8;
  if (nblocks > 0x7fffffffLL) return LL_ERR_UNSUPPORTED;
  const unsigned nb = static_cast<unsigned>(nblocks);
  switch (a.seg_log2) {
    case 3: return launch_wide_inst<3, 4>(a, nb, bytes, stream);
    case 4: return launch_wide_inst<4, 4>(a, nb, bytes, stream);
    case 5: return launch_wide_inst<5, 3>(a, nb, bytes, stream);
    case 6: return launch_wide_inst<6, 4>(a, nb, bytes, stream);
    default: return LL_ERR_UNSUPPORTED;
  }
}

}  // namespace ll
