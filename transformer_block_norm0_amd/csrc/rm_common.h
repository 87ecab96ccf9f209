// Internal device helpers shared by the RankMixerBlock kernels (gfx950, wave64).
#pragma once

#include <type_traits>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rm {

// ---------------------------------------------------------------------------
// storage types.  bf16 and fp16 are carried as their 16-bit patterns.

struct bf16_t {
  uint16_t u;
};
struct f16_t {
  uint16_t u;
};

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v.u) << 16); }
__device__ __forceinline__ float to_f32(f16_t v) { return (float)__builtin_bit_cast(_Float16, v.u); }
// fp16 bit pattern -> fp32 (exact)
__device__ __forceinline__ float h_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}
// float -> fp16, round to nearest even (the hardware conversion's default mode).
__device__ __forceinline__ uint16_t f32_to_f16_bits(float f) { return __builtin_bit_cast(uint16_t, (_Float16)f); }

// float -> bf16, round to nearest even (the gfx950 conversion instruction);
// NaN stays a (quiet) NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

template <typename ST> __device__ __forceinline__ ST from_f32(float f);
template <> __device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) {
  bf16_t r;
  r.u = f32_to_bf16_bits(f);
  return r;
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float f) {
  f16_t r;
  r.u = f32_to_f16_bits(f);
  return r;
}
// 16-bit storage bits of a float, per storage type
template <typename ST> __device__ __forceinline__ uint32_t to_bits16(float f);
template <> __device__ __forceinline__ uint32_t to_bits16<bf16_t>(float f) { return f32_to_bf16_bits(f); }
template <> __device__ __forceinline__ uint32_t to_bits16<f16_t>(float f) { return f32_to_f16_bits(f); }
// the low / high element of a word of two 16-bit storage values, as fp32
template <typename ST> __device__ __forceinline__ float lo16(uint32_t w);
template <typename ST> __device__ __forceinline__ float hi16(uint32_t w);
template <> __device__ __forceinline__ float lo16<bf16_t>(uint32_t w) { return __uint_as_float(w << 16); }
template <> __device__ __forceinline__ float hi16<bf16_t>(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
template <> __device__ __forceinline__ float lo16<f16_t>(uint32_t w) { return h_to_f32(w & 0xffffu); }
template <> __device__ __forceinline__ float hi16<f16_t>(uint32_t w) { return h_to_f32(w >> 16); }
// two floats packed as two 16-bit storage values (a in the low half), round
// to nearest even: one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32
template <typename ST> __device__ __forceinline__ uint32_t pack16x2(float a, float b) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  const f32x2 v = {a, b};
  if constexpr (std::is_same<ST, f16_t>::value) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, h2));
  } else {
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
  }
}

template <typename ST> __device__ __forceinline__ float ld(const ST* p, long i) { return to_f32(p[i]); }
template <typename ST> __device__ __forceinline__ void st(ST* p, long i, float v) { p[i] = from_f32<ST>(v); }

// ---------------------------------------------------------------------------
// token mixing index map (page 1, "Exact computation": view [B,T,D] as
// [B,T,T,S] with S = D/T, swap the two T axes).  Output row i, column c reads
// input row c / S, column i*S + c % S.  The map is an involution, so the same
// function also gives the adjoint (the backward gather).
__device__ __forceinline__ void tm_source(int i, int c, int S, int& src_row, int& src_col) {
  const int j = c / S;
  src_row = j;
  src_col = i * S + (c - j * S);
}

// r1 = token_mix(norm0(x)) + x for one gathered element a of row j (nmr =
// -mu0[j] rstd0[j], rs = rstd0[j]), the gathered affine gg/bb and the
// residual xi.  Every forward prologue and norm1 backward uses it, so
// the backward recomputes the forward's r1 bit for bit.
__device__ __forceinline__ float mixed_residual(float a, float rs, float nmr, float gg, float bb, float xi) {
  return fmaf(fmaf(a, rs, nmr), gg, bb) + xi;
}

// ---------------------------------------------------------------------------
// reductions (fixed order: deterministic)

// Sum over the 64 lanes of a wave, result in every lane, without LDS: DPP
// butterflies inside each 16-lane row (pairs, quads, half-row mirror, row
// mirror), then the four row sums read from lanes 0, 16, 32, 48.  Fixed order.
__device__ __forceinline__ float wave_sum(float v) {
  auto dpp = [](float a, auto ctrl) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, a), decltype(ctrl)::value,
                                                                 0xF, 0xF, false));
  };
  v += dpp(v, std::integral_constant<int, 0xB1>{});   // quad_perm [1,0,3,2]
  v += dpp(v, std::integral_constant<int, 0x4E>{});   // quad_perm [2,3,0,1]
  v += dpp(v, std::integral_constant<int, 0x141>{});  // row_half_mirror
  v += dpp(v, std::integral_constant<int, 0x140>{});  // row_mirror
  auto rl = [](float a, int l) { return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), l)); };
  return (rl(v, 0) + rl(v, 16)) + (rl(v, 32) + rl(v, 48));
}


// sigmoid(v) = 1 / (1 + exp(-v)) with the hardware exp2 and reciprocal (about
// 2 ulp); saturates cleanly to 0 and 1 for large |v|.
__device__ __forceinline__ float sigmoidf_(float v) { return __builtin_amdgcn_rcpf(1.0f + __expf(-v)); }

}  // namespace rm
