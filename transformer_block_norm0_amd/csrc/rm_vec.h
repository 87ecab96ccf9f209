// Vector load/store of N consecutive storage elements as fp32 (16-, 8- or
// 4-byte accesses), plus block reductions for row kernels.
#pragma once

#include <type_traits>

#include "rm_common.h"

namespace rm {

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// p must be aligned to N elements.
template <int N>
__device__ __forceinline__ void ldv(const float* __restrict__ p, float (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = p[0];
  } else if constexpr (N == 2) {
    const float2 a = *reinterpret_cast<const float2*>(p);
    v[0] = a.x; v[1] = a.y;
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 a = *reinterpret_cast<const float4*>(p + i);
      v[i] = a.x; v[i + 1] = a.y; v[i + 2] = a.z; v[i + 3] = a.w;
    }
  }
}

// 16-bit storage (bf16 or fp16)
template <typename ST>
constexpr bool is_half16 = std::is_same<ST, bf16_t>::value || std::is_same<ST, f16_t>::value;

template <typename ST, int N, std::enable_if_t<is_half16<ST>, int> = 0>
__device__ __forceinline__ void ldv(const ST* __restrict__ p, float (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = to_f32(p[0]);
  } else if constexpr (N == 2) {
    const uint32_t a = *reinterpret_cast<const uint32_t*>(p);
    v[0] = lo16<ST>(a); v[1] = hi16<ST>(a);
  } else if constexpr (N == 4) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    v[0] = lo16<ST>(a.x); v[1] = hi16<ST>(a.x); v[2] = lo16<ST>(a.y); v[3] = hi16<ST>(a.y);
  } else {
    static_assert(N % 8 == 0, "16-bit vector width");
#pragma unroll
    for (int i = 0; i < N; i += 8) {
      const uint4 a = *reinterpret_cast<const uint4*>(p + i);
      v[i] = lo16<ST>(a.x); v[i + 1] = hi16<ST>(a.x); v[i + 2] = lo16<ST>(a.y); v[i + 3] = hi16<ST>(a.y);
      v[i + 4] = lo16<ST>(a.z); v[i + 5] = hi16<ST>(a.z); v[i + 6] = lo16<ST>(a.w); v[i + 7] = hi16<ST>(a.w);
    }
  }
}

template <int N>
__device__ __forceinline__ void stv(float* __restrict__ p, const float (&v)[N]) {
  if constexpr (N == 1) {
    p[0] = v[0];
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  }
}

template <typename ST, int N, std::enable_if_t<is_half16<ST>, int> = 0>
__device__ __forceinline__ void stv(ST* __restrict__ p, const float (&v)[N]) {
  if constexpr (N == 1) {
    p[0].u = (uint16_t)to_bits16<ST>(v[0]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<uint32_t*>(p) = pack16x2<ST>(v[0], v[1]);
  } else if constexpr (N == 4) {
    *reinterpret_cast<uint2*>(p) = make_uint2(pack16x2<ST>(v[0], v[1]), pack16x2<ST>(v[2], v[3]));
  } else {
#pragma unroll
    for (int i = 0; i < N; i += 8)
      *reinterpret_cast<uint4*>(p + i) =
          make_uint4(pack16x2<ST>(v[i], v[i + 1]), pack16x2<ST>(v[i + 2], v[i + 3]), pack16x2<ST>(v[i + 4], v[i + 5]),
                     pack16x2<ST>(v[i + 6], v[i + 7]));
  }
}

// Raw (still packed) storage words of N elements, for prefetching a row
// without unpacking it into N fp32 registers.
template <typename ST, int N>
struct Raw {
  static constexpr int BYTES = N * (int)sizeof(ST);
  static constexpr int W = BYTES >= 4 ? BYTES / 4 : 1;
  uint32_t w[W];
};

template <typename ST, int N>
__device__ __forceinline__ void ldr(const ST* __restrict__ p, Raw<ST, N>& r) {
  constexpr int BYTES = Raw<ST, N>::BYTES;
  if constexpr (BYTES == 2) {
    r.w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else if constexpr (BYTES == 4) {
    r.w[0] = *reinterpret_cast<const uint32_t*>(p);
  } else if constexpr (BYTES == 8) {
    const uint2 a = *reinterpret_cast<const uint2*>(p);
    r.w[0] = a.x; r.w[1] = a.y;
  } else {
#pragma unroll
    for (int i = 0; i < BYTES / 16; ++i) {
      const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(p) + 16 * i);
      r.w[4 * i] = a.x; r.w[4 * i + 1] = a.y; r.w[4 * i + 2] = a.z; r.w[4 * i + 3] = a.w;
    }
  }
}


// Hide a value from the optimiser (no code emitted): forces a recomputation
// after a barrier instead of keeping earlier results alive across it.
template <typename ST, int N>
__device__ __forceinline__ void opaque(Raw<ST, N>& r) {
#pragma unroll
  for (int i = 0; i < Raw<ST, N>::W; ++i) asm volatile("" : "+v"(r.w[i]));
}

template <int N>
__device__ __forceinline__ void unpack(const Raw<float, N>& r, float (&v)[N]) {
#pragma unroll
  for (int e = 0; e < N; ++e) v[e] = __uint_as_float(r.w[e]);
}

template <typename ST, int N, std::enable_if_t<is_half16<ST>, int> = 0>
__device__ __forceinline__ void unpack(const Raw<ST, N>& r, float (&v)[N]) {
  if constexpr (N == 1) {
    v[0] = lo16<ST>(r.w[0]);
  } else {
#pragma unroll
    for (int e = 0; e < N; e += 2) {
      v[e] = lo16<ST>(r.w[e / 2]);
      v[e + 1] = hi16<ST>(r.w[e / 2]);
    }
  }
}

// Workgroup barrier for LDS-only communication: waits for this wave's LDS
// operations (lgkmcnt(0); gfx9 s_waitcnt encoding with vmcnt/expcnt at their
// maxima) but not for its outstanding global loads, so row prefetches stay in
// flight across it.  Not a fence for global memory.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Sum 8 values over the whole block (nw waves, nw <= 16), fixed order, the
// totals in every lane.  red: 2 * 16 * 8 floats of LDS, two halves
// alternating with `parity`, so consecutive calls need one barrier each (the
// barrier waits for LDS only).  Inside the wave a transposing reduce-scatter
// halves the number of values per lane at each lane distance (32, 16, 8), so
// the wave's eight sums cost 18 VALU operations instead of eight full
// butterflies; lane l then holds the wave's sum l/8 and lanes l%8 == 0 write
// it to the wave's slots.  After the barrier lane l reads wave l%16's sums
// 2(l/16) and 2(l/16)+1 and each 16-lane row adds the 16 waves with a DPP
// butterfly, without branches: the slots of waves >= nw must hold zeros
// (zero_red before the block's first barrier).
__device__ __forceinline__ void zero_red(float* red) {
  for (int i = threadIdx.x; i < 2 * 16 * 8; i += blockDim.x) red[i] = 0.f;
}
__device__ __forceinline__ void block_sum8(float (&v)[8], float* red, int parity);

// Sum NV values over the whole block (nw waves, nw <= 16), fixed order.
// red: 2 * NV * 16 floats of LDS, used as two alternating halves selected by
// `parity`, so consecutive calls need only one barrier each.
template <int NV>
__device__ __forceinline__ void block_sum(float (&v)[NV], float* red, int nw, int parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  float* r = red + parity * NV * 16;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float s = wave_sum(v[i]);
    if (lane == 0) r[i * 16 + wave] = s;
  }
  lds_barrier();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float t = 0.f;
    for (int w = 0; w < nw; ++w) t += r[i * 16 + w];
    v[i] = t;
  }
}

// Sum over the 64 lanes of a wave, result in every lane, without LDS: DPP
// butterflies inside each 16-lane row (pairs, quads, half-row mirror, row
// mirror), then the four row sums read from lanes 0, 16, 32, 48.  Fixed order.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), l));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += dpp_mov<0xB1>(v);   // quad_perm [1,0,3,2]
  v += dpp_mov<0x4E>(v);   // quad_perm [2,3,0,1]
  v += dpp_mov<0x141>(v);  // row_half_mirror
  v += dpp_mov<0x140>(v);  // row_mirror
  return (lane_f(v, 0) + lane_f(v, 16)) + (lane_f(v, 32) + lane_f(v, 48));
}


// Lane-half and row swaps (gfx950): x holds value i, y value i' of every
// lane.  v_permlane32_swap exchanges x's lanes 32..63 with y's lanes 0..31, so
// afterwards lanes 0..31 hold (own x, partner's x) and lanes 32..63
// (partner's y, own y), partner = lane ^ 32; the sum of the pair is x summed
// over the two lanes in the lower half and y in the upper.  v_permlane16_swap
// does the same for the odd and even 16-lane rows (partner = lane ^ 16).
__device__ __forceinline__ float swap32_sum(float x, float y) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}
__device__ __forceinline__ float swap16_sum(float x, float y) {
  const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(y), false, false);
  return __uint_as_float(s[0]) + __uint_as_float(s[1]);
}

__device__ __forceinline__ void block_sum8(float (&v)[8], float* red, int parity) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // lanes 0..31: sums 0..3 over {l, l^32}; lanes 32..63: sums 4..7
  float s[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) s[i] = swap32_sum(v[i], v[i + 4]);
  // 16-lane row q (= lane/16) holds sums 2q, 2q+1 over 4 lanes
  float t[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) t[j] = swap16_sum(s[j], s[j + 2]);
  // lanes with bit 3 clear keep sum 2q, the others 2q+1, each adding its
  // partner's (lane ^ 8, row_ror:8) copy; then the 8-lane half-row butterfly
  const bool odd = (lane & 8) != 0;
  float u = (odd ? t[1] : t[0]) + dpp_mov<0x128>(odd ? t[0] : t[1]);
  u += dpp_mov<0xB1>(u);   // quad_perm [1,0,3,2]
  u += dpp_mov<0x4E>(u);   // quad_perm [2,3,0,1]
  u += dpp_mov<0x141>(u);  // row_half_mirror
  float* r = red + parity * 16 * 8;
  if ((lane & 7) == 0) r[8 * wave + (lane >> 3)] = u;  // the wave's sum lane/8
  __builtin_amdgcn_sched_barrier(0);
  lds_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const float2 b = *reinterpret_cast<const float2*>(r + 8 * (lane & 15) + 2 * (lane >> 4));
  float a[2] = {b.x, b.y};
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    a[i] += dpp_mov<0xB1>(a[i]);
    a[i] += dpp_mov<0x4E>(a[i]);
    a[i] += dpp_mov<0x141>(a[i]);
    a[i] += dpp_mov<0x140>(a[i]);  // row_mirror: the 16 waves' total in every lane of the row
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    v[2 * q] = lane_f(a[0], 16 * q);
    v[2 * q + 1] = lane_f(a[1], 16 * q);
  }
}

// Wait until every vector-memory operation of this wave has completed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_byte_addr(const void* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// floor(c / S) for 0 <= c < 2^16, 1 <= S <= 1280 (exact: the quotient's
// fractional part is at least 0.5/S away from an integer).
__device__ __forceinline__ int div_small(int c, float invS) { return (int)(((float)c + 0.5f) * invS); }

}  // namespace rm
