// Device-side helpers shared by the paged-attention kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/pa.h"

namespace pa {

constexpr int kBlock = 16;            // rows per tile (a physical block holds 1 or 2 tiles)
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;

// A physical block holds 16 << sh tokens (16 or 32, 5688vip chapter 3, section
// 3.2): per kv head, 1 << sh tiles of 16 rows, contiguous.  The 16-row tile
// index of a sequence's logical tile j, whose table entry is blk; the
// (block, kv head) scale of a 1-byte pool sits at index tile >> sh.
__device__ __forceinline__ int64_t tile_index(int blk, int hkv, int h, int j, int sh) {
  return (((int64_t)blk * hkv + h) << sh) + (j & ((1 << sh) - 1));
}
// Running-max sentinel: finite so that exp2(sentinel - sentinel) = 1 keeps an
// empty lane's (m, l, acc) = (sentinel, 0, 0) harmless in every merge.
constexpr float kNegBig = -1.0e30f;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

__host__ __device__ constexpr int dtype_bytes(int dt) {
  return dt == PA_F32 ? 4 : (dt == PA_F16 || dt == PA_BF16) ? 2 : 1;
}

// ---- scalar conversions -------------------------------------------------------------
__device__ __forceinline__ float f16_lo(uint32_t w) {
  return (float)__builtin_bit_cast(h2_t, w)[0];
}
__device__ __forceinline__ float f16_hi(uint32_t w) {
  return (float)__builtin_bit_cast(h2_t, w)[1];
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) {
  return __builtin_bit_cast(float, w & 0xffff0000u);
}

// Load one query element of dtype QT as float.
template <int QT>
__device__ __forceinline__ float load_q(const void *p, int64_t i) {
  if constexpr (QT == PA_F32) {
    return reinterpret_cast<const float *>(p)[i];
  } else if constexpr (QT == PA_F16) {
    return (float)reinterpret_cast<const _Float16 *>(p)[i];
  } else {
    uint16_t b = reinterpret_cast<const uint16_t *>(p)[i];
    return __builtin_bit_cast(float, (uint32_t)b << 16);
  }
}

// Store a float as dtype OT, rounding to nearest even.
template <int OT>
__device__ __forceinline__ void store_out(void *p, int64_t i, float x) {
  if constexpr (OT == PA_F32) {
    reinterpret_cast<float *>(p)[i] = x;
  } else if constexpr (OT == PA_F16) {
    reinterpret_cast<_Float16 *>(p)[i] = (_Float16)x;
  } else {
    reinterpret_cast<__bf16 *>(p)[i] = (__bf16)x;
  }
}

// E4M3FN pair -> two floats (gfx950 decodes the OCP format in hardware).
__device__ __forceinline__ void fp8x4_to_f32(uint32_t w, float *f) {
  auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
  auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

__device__ __forceinline__ void i8x4_to_f32(uint32_t w, float *f) {
  f[0] = (float)(int8_t)(w & 0xff);
  f[1] = (float)(int8_t)((w >> 8) & 0xff);
  f[2] = (float)(int8_t)((w >> 16) & 0xff);
  f[3] = (float)(int8_t)(w >> 24);
}

// ---- cross-lane sums inside groups of 2^k lanes (DPP, no LDS) ---------------------------
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <- lane 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <- lane 15-i within 16
constexpr int kDppRor4 = 0x124;       // lane i <- lane (i-4) mod 16 within 16
constexpr int kDppRor8 = 0x128;       // lane i <- lane i^8 within 16
constexpr int kDppRowBcast0 = 0x150;  // + n: every lane of a 16-lane row <- lane n of that row

// Reduce-scatter across one 16-lane row: on entry each lane holds NV partial values
// x[0..NV); on exit x[0..NV/16) hold full row sums of value indices
// c*(NV/16) + j, where c is the lane's index within the row.  Each step pairs a lane
// with a partner holding the complementary half (xor 8 by rotation, bit 2 by the
// half-row mirror, then xor 2 and xor 1), keeps one half and adds the partner's copy.
template <int N, int CTRL>
__device__ __forceinline__ void rs_step(float *x, bool upper) {
  constexpr int H = N / 2;
#pragma unroll
  for (int k = 0; k < H; ++k) {
    const float keep = upper ? x[k + H] : x[k];
    const float send = upper ? x[k] : x[k + H];
    x[k] = keep + dpp_f<CTRL>(send);
  }
}

template <int NV>
__device__ __forceinline__ void row_reduce_scatter(float *x, int c) {
  static_assert(NV % 16 == 0, "reduce-scatter needs a multiple of 16 values");
  rs_step<NV, kDppRor8>(x, (c >> 3) & 1);
  rs_step<NV / 2, kDppHalfMirror>(x, (c >> 2) & 1);
  rs_step<NV / 4, kDppXor2>(x, (c >> 1) & 1);
  rs_step<NV / 8, kDppXor1>(x, c & 1);
}

// Value of x held by lane n of this lane's 16-lane row (n a compile-time constant).
template <int N>
__device__ __forceinline__ float row_bcast(float x) {
  return dpp_f<kDppRowBcast0 + N>(x);
}

// Value held by lane (lane ^ MASK), for MASK in {1, 2, 8, 16, 32} without LDS:
// DPP inside a 16-lane row, v_permlane{16,32}_swap across rows (each returns the
// pair (x[lane & ~MASK], x[lane | MASK]); the partner is the one that differs).
template <int MASK>
__device__ __forceinline__ float xor_lanes(float x) {
  if constexpr (MASK == 1) {
    return dpp_f<kDppXor1>(x);
  } else if constexpr (MASK == 2) {
    return dpp_f<kDppXor2>(x);
  } else if constexpr (MASK == 8) {
    return dpp_f<kDppRor8>(x);
  } else if constexpr (MASK == 16 || MASK == 32) {
    const unsigned u = __builtin_bit_cast(unsigned, x);
    unsigned lo, hi;
    if constexpr (MASK == 16) {
      auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
      lo = r[0];
      hi = r[1];
    } else {
      auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      lo = r[0];
      hi = r[1];
    }
    const bool upper = (__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)) & MASK) != 0;
    return __builtin_bit_cast(float, upper ? lo : hi);
  } else {
    return __shfl_xor(x, MASK, 64);
  }
}

// After the call every lane holds the sum over its aligned group of N lanes.
// Lanes of one group must hold the same kind of value (a partial dot product).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
  if constexpr (N >= 2) x += dpp_f<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_f<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_f<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f<kDppMirror>(x);
  if constexpr (N >= 32) x += xor_lanes<16>(x);
  if constexpr (N >= 64) x += xor_lanes<32>(x);
  return x;
}

// Maxima as the bare v_max / v_max3 instructions.  Written through fmaxf, every
// operand that the compiler cannot prove canonical (an MFMA result, a value moved
// across lanes) first gets a v_max_f32 x, x, x of its own, which quiets a
// signalling NaN under the IEEE mode the kernels run in.  The callers' operands
// are scores and running maxima -- finite, or -inf where masked by a select --
// for which the bare instruction is the same maximum.
__device__ __forceinline__ float max_raw(float a, float b) {
  float r;
  asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
  return r;
}
__device__ __forceinline__ float max3_raw(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// max(x, x of lane ^ MASK) for MASK 16 or 32: the row swap leaves the lane's own
// value in one output and its partner's in the other, so no select is needed.
template <int MASK>
__device__ __forceinline__ float max_xor_rows(float x) {
  static_assert(MASK == 16 || MASK == 32, "row swaps only");
  const unsigned u = __builtin_bit_cast(unsigned, x);
  unsigned a, b;
  if constexpr (MASK == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    a = r[0];
    b = r[1];
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    a = r[0];
    b = r[1];
  }
  return max_raw(__builtin_bit_cast(float, a), __builtin_bit_cast(float, b));
}

// Row swap of two values (MASK 16: rows r and r^1; MASK 32: halves): afterwards x
// holds, in the even row (lower half), its own x and in the odd row (upper half) the
// partner's y, and y the partner's x in the even row and its own y in the odd one.
// So x and y are the two states of one value pair-wise: x (+) y merges x's value in
// the even rows and y's in the odd rows, with no select.
template <int MASK>
__device__ __forceinline__ void swap_rows(float &x, float &y) {
  static_assert(MASK == 16 || MASK == 32, "row swaps only");
  const unsigned u = __builtin_bit_cast(unsigned, x), v = __builtin_bit_cast(unsigned, y);
  if constexpr (MASK == 16) {
    auto r = __builtin_amdgcn_permlane16_swap(u, v, false, false);
    x = __builtin_bit_cast(float, (unsigned)r[0]);
    y = __builtin_bit_cast(float, (unsigned)r[1]);
  } else {
    auto r = __builtin_amdgcn_permlane32_swap(u, v, false, false);
    x = __builtin_bit_cast(float, (unsigned)r[0]);
    y = __builtin_bit_cast(float, (unsigned)r[1]);
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

}  // namespace pa
