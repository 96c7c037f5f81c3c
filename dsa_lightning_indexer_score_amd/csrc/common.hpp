// Shared device helpers for the gfx950 kernels of libidxc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace idxc {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kMaxK = 2048;

// 32x32x16 bf16 MFMA (gfx950). Operand layout, lane l of 64:
//   A: row (l % 32), k = 8*(l/32) + j for j = 0..7
//   B: col (l % 32), k = 8*(l/32) + j
//   C: acc[i] holds row 8*(i/4) + 4*(l/32) + (i%4), col (l % 32)
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int acc_row(int i, int lane) {
  return 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
}

// x[l] + x[l ^ 32] (identical in both lanes of the pair). permlane32_swap
// returns both halves of the swapped register pair; per lane one of them is
// the lane's own value and the other its partner's, so their sum (or max) is
// the pair reduction.
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                            false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// max(x, 0) for a finite float, on its bit pattern: non-negative floats are
// non-negative ints, negative floats (and -0.0) are negative ints, so an
// integer max with 0 is an exact ReLU that returns +0.0 for x <= 0.
__device__ __forceinline__ float relu_bits(float x) {
  return __int_as_float(max(__float_as_int(x), 0));
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// Round-to-nearest-even fp32 -> bf16 (inputs are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 pair (hardware round-to-nearest-even), low = a.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  const bf16x2 h = __builtin_convertvector(f32x2{a, b}, bf16x2);
  return __builtin_bit_cast(uint32_t, h);
}

// Order-preserving map of a finite fp32 to uint32 (larger float -> larger key);
// -0.0 is mapped like +0.0.
__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_to_float(uint32_t key) {
  uint32_t u = (key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// v of lane (l ^ M), M a power of two below 64, without LDS traffic: DPP
// quad permutes (1, 2), a row shift either way (4), a row rotate (8), or a
// permlane swap (16, 32), which returns both values of each lane pair.
template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
  static_assert(M == 1 || M == 2 || M == 4 || M == 8 || M == 16 || M == 32, "lane mask");
  const int lane = lane_id();
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const uint32_t up = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x104, 0xF, 0xF, false);  // row_shl:4
    const uint32_t dn = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);  // row_shr:4
    return (lane & 4) ? dn : up;
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (M == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane & 16) ? r[0] : r[1];
  } else {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (lane & 32) ? r[0] : r[1];
  }
}

// Wave-wide inclusive prefix sum of an int (64 lanes): Hillis-Steele steps
// within each 16-lane row (DPP row shifts, lanes shifted in from outside the
// row read 0), then each row's last value is added to the rows above it (DPP
// row broadcasts of lanes 15 and 31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15, rows 1 and 3
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31, rows 2 and 3
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, __uint_as_float(lane_xor<32>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<16>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<8>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<4>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<2>(__float_as_uint(v))));
  v = fmaxf(v, __uint_as_float(lane_xor<1>(__float_as_uint(v))));
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
  v += (int)lane_xor<32>((uint32_t)v);
  v += (int)lane_xor<16>((uint32_t)v);
  v += (int)lane_xor<8>((uint32_t)v);
  v += (int)lane_xor<4>((uint32_t)v);
  v += (int)lane_xor<2>((uint32_t)v);
  v += (int)lane_xor<1>((uint32_t)v);
  return v;
}

// Wave-wide minimum and maximum of a uint32 (every lane gets both).
__device__ __forceinline__ void wave_minmax(uint32_t& mn, uint32_t& mx) {
#define IDXC_MINMAX_STEP(M)              \
  mn = min(mn, lane_xor<M>(mn));         \
  mx = max(mx, lane_xor<M>(mx));
  IDXC_MINMAX_STEP(32)
  IDXC_MINMAX_STEP(16)
  IDXC_MINMAX_STEP(8)
  IDXC_MINMAX_STEP(4)
  IDXC_MINMAX_STEP(2)
  IDXC_MINMAX_STEP(1)
#undef IDXC_MINMAX_STEP
}

}  // namespace idxc
