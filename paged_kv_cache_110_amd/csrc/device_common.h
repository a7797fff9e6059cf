// Device helpers shared by the libpkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr float kNegSentinel = -1.0e30f;  // "no score yet": finite, so exp2(x - it) never NaNs

// bf16 halves of a 32-bit word, widened exactly to fp32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 values -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// dot of two packed bf16 pairs accumulated into c (v_dot2_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane exchange inside a row of 16 lanes through DPP.
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

// Sum over aligned groups of N lanes (N in {1,2,4,8,16}); every lane of the
// group ends with the group total.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (N >= 2) x += dpp_f32<kDppXor1>(x);
  if constexpr (N >= 4) x += dpp_f32<kDppXor2>(x);
  if constexpr (N >= 8) x += dpp_f32<kDppHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_f32<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

constexpr int kDppRowRor8 = 0x128;  // lane i <- lane i ^ 8 within a row of 16

// Sum / max over the lanes l, l ^ S, l ^ 2S, ... (S in {8, 16, 32}): lanes
// that share l % S.  Every lane ends with the result.  The exchanges run on
// the vector ALU (DPP row rotate by 8, v_permlane16_swap, v_permlane32_swap:
// each swap of x with itself yields the two halves of every lane pair, so
// combining its two outputs gives the pair's sum or max in all lanes).
template <int S, bool MAX>
__device__ __forceinline__ float cross_reduce(float x) {
  static_assert(S == 8 || S == 16 || S == 32, "stride");
  auto op = [](float a, float b) { return MAX ? fmaxf(a, b) : a + b; };
  if constexpr (S <= 8) x = op(x, dpp_f32<kDppRowRor8>(x));
  if constexpr (S <= 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = op(__uint_as_float(p[0]), __uint_as_float(p[1]));
  }
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return op(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

// 16-byte global load / store helpers (addresses must be 16-byte aligned).
__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
// The same load with the non-temporal hint (`nt`), for data read once per
// call: a plain streaming read of 4 GiB measured 6.3 TB/s with plain loads and
// 7.1 TB/s with non-temporal ones on MI355X.
__device__ __forceinline__ u32x4 ld16_stream(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace pkv
