// Device helpers shared by the log-linear attention kernels (gfx950 only).
//
// Page abbreviation used in comments:
//   [P1] "论文阅读：Log-Linear Attention — 基于 Fenwick 树与层次矩阵的对数线性复杂度注意力机制"
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ll {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;

// Fenwick level of key s seen from query t, s <= t ([P1] 层级判定算法).  The
// bucket walk peels the low set bits of t; s lands in the bucket cut by the
// highest bit in which s and t differ, so the level is the bit length of
// t ^ s (0 when s == t, the size-one sentinel bucket).
__device__ __forceinline__ int level_of(uint32_t t, uint32_t s) {
  const uint32_t x = t ^ s;
  return x ? 32 - __clz(x) : 0;
}

// 0-based index of the lowest set bit of t > 0 ([P1] 解码：基于 lssb 的状态更新).
__device__ __forceinline__ int lssb(uint32_t t) { return __ffs(t) - 1; }

// ---------------------------------------------------------------------------
// 16x16 matrix-core fragments.  For both element types a lane l holds row
// (A) or column (B) l % 16 of its operand; the accumulator holds
// C[4*(l/16) + r][l % 16] in element r.  The order of the reduction index
// inside a fragment only has to agree between A and B, which every caller
// guarantees by loading both through the same index map.
// ---------------------------------------------------------------------------
template <typename IT>
struct Frag;

template <>
struct Frag<bf16> {
  using V = bf16x8;
  static constexpr int KS = 32;  // reduction length of one v_mfma_f32_16x16x32_bf16
  // Row-major tile (element (row, k) at base[row * ld + k]); rows row0..row0+15,
  // reduction index k0..k0+31, 8 consecutive elements per lane.
  static __device__ __forceinline__ V load(const bf16* base, int ld, int row0, int k0, int lane) {
    return *reinterpret_cast<const bf16x8*>(base + (row0 + (lane & 15)) * ld + k0 + 8 * (lane >> 4));
  }
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};

template <>
struct Frag<float> {
  using V = float;
  static constexpr int KS = 4;  // v_mfma_f32_16x16x4_f32
  static __device__ __forceinline__ V load(const float* base, int ld, int row0, int k0, int lane) {
    return base[(row0 + (lane & 15)) * ld + k0 + (lane >> 4)];
  }
  static __device__ __forceinline__ f32x4 mma(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
};

// Two-term bf16 split: x ~= hi + lo with |x - hi - lo| <= 2^-16 |x| (RNE).
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = static_cast<bf16>(x);
  lo = static_cast<bf16>(x - static_cast<float>(hi));
}

template <typename T>
__device__ __forceinline__ T from_float(float x) { return static_cast<T>(x); }
template <typename T>
__device__ __forceinline__ float to_float(T x) { return static_cast<float>(x); }

}  // namespace ll
