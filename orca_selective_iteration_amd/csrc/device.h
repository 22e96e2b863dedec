// Device helpers shared by the gfx950 kernels: bf16 storage type, 16-byte
// vector access, wave-level reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace orca {

// bf16 is stored as its 16 raw bits; arithmetic happens in fp32.
struct bf16 {
  uint16_t bits;
};

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;   // MFMA operand
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;   // dot2 operand
typedef __attribute__((ext_vector_type(16))) float f32x16_t;    // 32x32 MFMA acc
typedef __attribute__((ext_vector_type(4))) float f32x4_t;      // 16x16 MFMA acc

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16, round to nearest, ties to even (NaN stays NaN).
// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 (one
// instruction for two values), which the compiler emits for __bf16 casts.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Scalar load/store of one element of T as fp32.
template <typename T> __device__ __forceinline__ float load_f32(const T* p);
template <> __device__ __forceinline__ float load_f32<float>(const float* p) { return *p; }
template <> __device__ __forceinline__ float load_f32<bf16>(const bf16* p) {
  return __uint_as_float(uint32_t(p->bits) << 16);
}
template <typename T> __device__ __forceinline__ void store_f32(T* p, float v);
template <> __device__ __forceinline__ void store_f32<float>(float* p, float v) { *p = v; }
template <> __device__ __forceinline__ void store_f32<bf16>(bf16* p, float v) {
  p->bits = f32_to_bf16_bits(v);
}

// 16 bytes of T <-> fp32 lanes (8 for bf16, 4 for fp32).
// 16-byte load with the non-temporal hint, for data read once per launch
// (streamed K/V, streamed weights): on MI355X a plain streaming read reaches
// ~6.3 TB/s, with the hint ~7.1 TB/s.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_nt16(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

template <typename T> struct Vec16;
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = __uint_as_float(v.x); f[1] = __uint_as_float(v.y);
    f[2] = __uint_as_float(v.z); f[3] = __uint_as_float(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                      __float_as_uint(f[3]));
  }
};
template <> struct Vec16<bf16> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const uint4& v, float* f) {
    f[0] = bf16_lo(v.x); f[1] = bf16_hi(v.x); f[2] = bf16_lo(v.y); f[3] = bf16_hi(v.y);
    f[4] = bf16_lo(v.z); f[5] = bf16_hi(v.z); f[6] = bf16_lo(v.w); f[7] = bf16_hi(v.w);
  }
  __device__ __forceinline__ static uint4 pack(const float* f) {
    return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                      pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
  }
};

// ---- cross-lane sums inside groups of G consecutive lanes (G | 64) --------
// DPP row operations for groups up to 16 lanes, a bpermute for 32 and 64.
__device__ __forceinline__ float dpp_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_xor2(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_half_mirror(float v) {   // lane i <-> 7-i in 8
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, true));
}
__device__ __forceinline__ float dpp_mirror(float v) {        // lane i <-> 15-i in 16
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, true));
}

template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16 || G == 32 || G == 64, "G");
  if constexpr (G >= 2) v += dpp_xor1(v);
  if constexpr (G >= 4) v += dpp_xor2(v);
  if constexpr (G >= 8) v += dpp_half_mirror(v);
  if constexpr (G >= 16) v += dpp_mirror(v);
  if constexpr (G >= 32) v += __shfl_xor(v, 16);
  if constexpr (G >= 64) v += __shfl_xor(v, 32);
  return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<64>(v); }

__device__ __forceinline__ float wave_max(float v) {
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace orca
