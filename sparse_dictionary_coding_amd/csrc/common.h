// Device-side helpers shared by the FAD-KV kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fadkv {

enum { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2 };

// A dispatch counts work-items in 32 bits per grid dimension, so launches whose grid grows with
// the number of vectors are issued in chunks of at most 2^22 workgroups (2^31 work-items at 512
// threads); each chunk passes its first unit as `base`.
constexpr size_t kMaxBlocksPerLaunch = size_t(1) << 22;

// vector-status byte written by the screening kernel for the selection kernel
enum { VS_NORMAL = 0, VS_ZERO = 1, VS_NONFINITE = 2 };

enum { FLAG_TRIGGER = 0x01, FLAG_REPLACED = 0x02, FLAG_EXHAUSTED = 0x04, FLAG_NONFINITE = 0x08 };

template <int DT> struct Elem;
template <> struct Elem<DT_F32> { static constexpr int bytes = 4; };
template <> struct Elem<DT_F16> { static constexpr int bytes = 2; };
template <> struct Elem<DT_BF16> { static constexpr int bytes = 2; };

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float f16_bits_to_float(uint32_t b) {
  uint16_t h = (uint16_t)b;
  _Float16 f = __builtin_bit_cast(_Float16, h);
  return (float)f;
}
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// low / high element of a packed 32-bit word of two 16-bit values, as float
template <int DT> __device__ __forceinline__ float lo_f(uint32_t w) {
  return DT == DT_F16 ? f16_bits_to_float(w & 0xffffu) : bf16_bits_to_float(w & 0xffffu);
}
template <int DT> __device__ __forceinline__ float hi_f(uint32_t w) {
  return DT == DT_F16 ? f16_bits_to_float(w >> 16) : bf16_bits_to_float(w >> 16);
}

// element i of a row stored in dtype DT, as float
template <int DT> __device__ __forceinline__ float elem_f(const void *row, int i) {
  if constexpr (DT == DT_F32) {
    return reinterpret_cast<const float *>(row)[i];
  } else {
    uint32_t b = reinterpret_cast<const uint16_t *>(row)[i];
    return DT == DT_F16 ? f16_bits_to_float(b) : bf16_bits_to_float(b);
  }
}

// 2-element fp32-accumulating dot of packed 16-bit pairs
template <int DT> __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DT == DT_F16) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(half2_t, a), __builtin_bit_cast(half2_t, b),
                                  c, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                           __builtin_bit_cast(bf16x2_t, b), c, false);
  }
}

// ---- float -> storage rounding (round to nearest, ties to even) ----------------------------
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t float_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;   // hardware conversion, round to nearest even
  return __builtin_bit_cast(uint16_t, h);
}

// Round a double to the nearest value with `p` significant bits whose spacing never drops
// below 2^qmin, ties to even: r = rint(v / 2^q) * 2^q with 2^q the spacing at |v|.
__device__ __forceinline__ double round_sig_bits(double v, int p, int qmin) {
  if (v == 0.0 || !__builtin_isfinite(v)) return v;
  int e;
  (void)__builtin_frexp(v, &e);   // |v| in [2^(e-1), 2^e)
  int q = e - p;
  if (q < qmin) q = qmin;
  return __builtin_ldexp(__builtin_rint(__builtin_ldexp(v, -q)), q);
}

// double -> storage bits straight from double (no intermediate rounding to float)
template <int DT> __device__ __forceinline__ uint32_t double_to_storage_bits(double v) {
  if constexpr (DT == DT_F32) {
    return __float_as_uint((float)v);   // v_cvt_f32_f64 rounds to nearest even
  } else if constexpr (DT == DT_F16) {
    double r = round_sig_bits(v, 11, -24);
    if (__builtin_fabs(r) > 65504.0) r = __builtin_copysign(__builtin_inf(), v);
    _Float16 h = (_Float16)(float)r;   // exact: r is representable in binary16
    return __builtin_bit_cast(uint16_t, h);
  } else {
    double r = round_sig_bits(v, 8, -133);
    const double bmax = 3.3895313892515355e38;   // (2 - 2^-7) * 2^127
    if (__builtin_fabs(r) > bmax) r = __builtin_copysign(__builtin_inf(), v);
    return __float_as_uint((float)r) >> 16;   // exact: r is representable in bfloat16
  }
}

// ---- wave64 reductions ----------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// ---- wave64 reductions through DPP (row-internal patterns, then the four row leaders) ------
template <int CTRL> __device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror: afterwards every lane
// of a 16-lane row holds the row's reduction
__device__ __forceinline__ float wave_max_f32(float v) {
  v = fmaxf(v, __int_as_float(dpp_i<0xB1>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x4E>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x141>(__float_as_int(v))));
  v = fmaxf(v, __int_as_float(dpp_i<0x140>(__float_as_int(v))));
  const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}
// Maximum over the wave of non-negative floats (negative values only as "absent"), in lane 63:
// signed-integer max on the bit patterns orders such values like the floats.  Each level is
// one DPP-fused v_max_i32 (the moved-in value defaults to INT_MIN, the identity): row-internal
// patterns first, then row_bcast:15 (into rows 1 and 3) and row_bcast:31 (into rows 2 and 3).
template <int CTRL, int ROWS = 0xF> __device__ __forceinline__ int max_dpp_i(int v) {
  return max(v, __builtin_amdgcn_update_dpp((int)0x80000000, v, CTRL, ROWS, 0xF, false));
}
__device__ __forceinline__ int wave_max_nonneg_bits(int v) {
  v = max_dpp_i<0xB1>(v);
  v = max_dpp_i<0x4E>(v);
  v = max_dpp_i<0x141>(v);
  v = max_dpp_i<0x140>(v);
  v = max_dpp_i<0x142, 0xA>(v);
  v = max_dpp_i<0x143, 0xC>(v);
  return __builtin_amdgcn_readlane(v, 63);
}
__device__ __forceinline__ int wave_min_i32(int v) {
  v = min(v, dpp_i<0xB1>(v));
  v = min(v, dpp_i<0x4E>(v));
  v = min(v, dpp_i<0x141>(v));
  v = min(v, dpp_i<0x140>(v));
  const int a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const int c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return min(min(a, b), min(c, d));
}

}  // namespace fadkv
