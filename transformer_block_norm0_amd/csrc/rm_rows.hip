// Row-wise kernels of the RankMixerBlock (LayerNorms, token mixing, gating,
// and their backward), for gfx950 wave64.  All of them are HBM-bandwidth
// bound: each reads and writes its rows once, in 16-byte (or 8-byte) vector
// chunks, and keeps statistics in fp32.
//
// Page 1 of "Subgraph-fusion-based Mega-kernel Generation", section "Exact
// computation", defines what they compute: outer LayerNorms (eps 1e-3),
// token mixing (swap the two T axes of a [B,T,T,D/T] view), the residual
// adds, and the gated inner LayerNorms (eps 1e-5) of the dense subgraph.
//
// Two shapes of kernel:
//   * one wave per row (rows are independent, no parameter gradient): the
//     forward prologue, gate forward, norm2 forward;
//   * one thread per vector chunk of the row, a workgroup walking the rows
//     (b, t) of one group of samples at one token t, with block reductions:
//     the backward kernels, whose per-column parameter-gradient partial sums
//     then stay in a few registers per thread.
#include <atomic>
#include "rm_common.h"
#include "rm_internal.h"
#include "rm_vec.h"

#include <algorithm>
#include <type_traits>

namespace rm {

namespace {

constexpr float EPS_OUTER = 1e-3f;
constexpr float EPS_INNER = 1e-5f;
constexpr int MAXD = 1280, MAXH = 3840;

template <typename ST>
__host__ __device__ __forceinline__ const ST* cptr(const void* p) { return reinterpret_cast<const ST*>(p); }

// ---------------------------------------------------------------------------
// Forward prologue, one workgroup (8 waves) per sample b, one wave per row:
//   a0 = norm0(x[b]);  r1 = token_mix(a0) + x[b];  out1 = norm1(r1).
// Token mixing is a gather: output row i, column c reads token c/S, column
// i*S + c%S of a0, recomputed from x and norm0's statistics (kept in LDS).
// N = elements per lane chunk; N > 1 needs D % N == 0 and S % N == 0 so a
// chunk's gather source is N contiguous, aligned elements.
template <typename ST, int N>
__global__ __launch_bounds__(512) void k_prologue(const ST* __restrict__ x, const ST* __restrict__ g0,
                                                  const ST* __restrict__ be0, const ST* __restrict__ g1,
                                                  const ST* __restrict__ be1, ST* __restrict__ h1,
                                                  float* __restrict__ stats, int B, int T, int D) {
  constexpr int Q = (MAXD + 64 * N - 1) / (64 * N);
  __shared__ float s_mu0[64], s_rs0[64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long NR = (long)B * T;
  const long base = (long)b * T * D;
  const int S = D / T;
  const float invS = 1.0f / (float)S, invD = 1.0f / (float)D;

  for (int j = wave; j < T; j += 8) {
    float v[Q][N];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        ldv(x + base + (long)j * D + c, v[q]);
      } else {
#pragma unroll
        for (int e = 0; e < N; ++e) v[q][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < N; ++e) s += v[q][e];
    }
    const float mean = wave_sum(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float dd = v[q][e] - mean;
          s2 += dd * dd;
        }
      }
    }
    const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
    if (lane == 0) {
      s_mu0[j] = mean;
      s_rs0[j] = rstd;
      stats[ST_MU0 * NR + (long)b * T + j] = mean;
      stats[ST_RS0 * NR + (long)b * T + j] = rstd;
    }
  }
  __syncthreads();

  for (int i = wave; i < T; i += 8) {
    float r[Q][N];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        const int j = div_small(c, invS);
        const int sc = i * S + (c - j * S);
        float a[N], gg[N], bb[N], xi[N];
        ldv(x + base + (long)j * D + sc, a);
        ldv(g0 + sc, gg);
        ldv(be0 + sc, bb);
        ldv(x + base + (long)i * D + c, xi);
        const float rs = s_rs0[j], nmr = -s_mu0[j] * rs;
#pragma unroll
        for (int e = 0; e < N; ++e) r[q][e] = mixed_residual(a[e], rs, nmr, gg[e], bb[e], xi[e]);
      } else {
#pragma unroll
        for (int e = 0; e < N; ++e) r[q][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < N; ++e) s += r[q][e];
    }
    const float mean = wave_sum(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float dd = r[q][e] - mean;
          s2 += dd * dd;
        }
      }
    }
    const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        float gg[N], bb[N], o[N];
        ldv(g1 + c, gg);
        ldv(be1 + c, bb);
#pragma unroll
        for (int e = 0; e < N; ++e) o[e] = (r[q][e] - mean) * rstd * gg[e] + bb[e];
        stv(h1 + base + (long)i * D + c, o);
      }
    }
    if (lane == 0) {
      stats[ST_MU1 * NR + (long)b * T + i] = mean;
      stats[ST_RS1 * NR + (long)b * T + i] = rstd;
    }
  }
}

// Raw buffer resource over `bytes` bytes at p (gfx9 word 3: 32-bit data
// format).  Range checks apply to the per-lane offset only (not the scalar
// one): a lane offset of 0x80000000 reads zero / drops the store.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* p, long bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)min(bytes, 0x7fffffffL), 0x00020000);
}

template <typename ST>
__device__ __forceinline__ void bld4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, Raw<ST, 4>& r) {
  if constexpr (sizeof(ST) == 2) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u a = __builtin_bit_cast(v2u, __builtin_amdgcn_raw_buffer_load_b64(rs, voff, soff, 0));
    r.w[0] = a.x; r.w[1] = a.y;
  } else {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u a = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rs, voff, soff, 0));
    r.w[0] = a.x; r.w[1] = a.y; r.w[2] = a.z; r.w[3] = a.w;
  }
}

template <typename ST>
__device__ __forceinline__ void bst4(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, const float (&v)[4]) {
  if constexpr (sizeof(ST) == 2) {
    typedef uint32_t v2u __attribute__((ext_vector_type(2)));
    const v2u a = {pack16x2<ST>(v[0], v[1]), pack16x2<ST>(v[2], v[3])};
    __builtin_amdgcn_raw_buffer_store_b64(a, rs, voff, soff, 0);
  } else {
    typedef uint32_t v4u __attribute__((ext_vector_type(4)));
    const v4u a = {__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
    __builtin_amdgcn_raw_buffer_store_b128(a, rs, voff, soff, 0);
  }
}

// N storage elements from fp32 by one buffer store (N * sizeof(ST) = 2, 4,
// 8 or 16 bytes).
template <typename ST, int N>
__device__ __forceinline__ void bstv(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff, const float (&v)[N]) {
  constexpr int BYTES = N * (int)sizeof(ST);
  static_assert(BYTES == 2 || BYTES == 4 || BYTES == 8 || BYTES == 16, "store width");
  if constexpr (BYTES == 2) {
    __builtin_amdgcn_raw_buffer_store_b16((unsigned short)to_bits16<ST>(v[0]), rs, voff, soff, 0);
  } else {
    constexpr int W = BYTES / 4;
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W; ++i) {
      if constexpr (sizeof(ST) == 2) w[i] = pack16x2<ST>(v[2 * i], v[2 * i + 1]);
      else w[i] = __float_as_uint(v[i]);
    }
    if constexpr (W == 1) {
      __builtin_amdgcn_raw_buffer_store_b32(w[0], rs, voff, soff, 0);
    } else if constexpr (W == 2) {
      typedef uint32_t v2u __attribute__((ext_vector_type(2)));
      const v2u a = {w[0], w[1]};
      __builtin_amdgcn_raw_buffer_store_b64(a, rs, voff, soff, 0);
    } else {
      typedef uint32_t v4u __attribute__((ext_vector_type(4)));
      const v4u a = {w[0], w[1], w[2], w[3]};
      __builtin_amdgcn_raw_buffer_store_b128(a, rs, voff, soff, 0);
    }
  }
}

// Resident blocks per compute unit of a kernel at a block size (cached per
// kernel; concurrent first calls store the same value).
template <auto KERNEL>
int resident_blocks(int threads) {
  static std::atomic<int> cached{0};
  int n = cached.load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, KERNEL, threads, 0) != hipSuccess || n <= 0) n = 1;
    cached.store(n, std::memory_order_relaxed);
  }
  return n;
}

// ---------------------------------------------------------------------------
// Forward prologue for 16-bit storage with the whole sample staged in LDS (T*D*2 bytes,
// at most 160 KB), so x is read from HBM once.  One workgroup (16 waves for
// the 160 KB LDS tier, fewer for smaller samples, see lds_tier) per sample b,
// one wave per row, 4-element chunks (D % 4 == 0, S % 4 == 0):
//   1. each wave loads its rows of x[b] once, computes norm0's statistics in
//      registers, writes the raw row to LDS and the statistics to `stats`;
//   2. after the barrier each lane fetches the statistics of the (at most
//      MAXD / 256) source rows its columns gather from -- the same rows for
//      every output row -- with L1-bypassing loads;
//   3. output row i: the token-mix gather and the residual read LDS, then
//      norm1 in registers and one store of out1.
constexpr int PRO_LDS_BYTES = (int)SAMPLE_LDS_BYTES;  // 160 KB: T*D bf16 for T <= 64, D <= 1280
// LDS tiers of the sample kernels: a workgroup declares the smallest tier
// that holds its sample (T*D*2 bytes) and runs as many threads as leave the
// LDS and the register file room for 160 KB / tier workgroups per CU, so a
// small sample's load, compute and store overlap with other samples'.
constexpr int lds_tier(long sample_bytes) {
  return sample_bytes <= PRO_LDS_BYTES / 4 ? PRO_LDS_BYTES / 4
         : sample_bytes <= PRO_LDS_BYTES / 2 ? PRO_LDS_BYTES / 2 : PRO_LDS_BYTES;
}
// prologue: 16 waves per CU in all (at most 128 VGPRs each)
constexpr int pro_threads(int tier) { return 1024 * tier / PRO_LDS_BYTES; }
// tail: 8 waves per CU in all (at most 256 VGPRs each), at least 4 per workgroup
constexpr int tail_threads(int tier) { return tier == PRO_LDS_BYTES ? 512 : 256; }

// Copy nbytes (a multiple of 16) from global src to LDS dst with 16-byte
// buffer loads that write LDS directly, range-checked against [src, src +
// nbytes) (an offset outside reads zeros): the wave's pieces first, first +
// stride, ... (first and stride uniform multiples of 64 pieces; piece p is
// bytes 16p .. 16p + 15 of both).  Inline assembly, so the compiler does not
// count these loads: the caller waits (vmcnt(0)) before reading the data.
__device__ __forceinline__ void copy_to_lds(const void* src, void* dst, int nbytes, int first, int stride, int lane) {
  const int np = nbytes >> 4;
  const __amdgpu_buffer_rsrc_t rs = row_rsrc(src, (long)nbytes);
  const char* d = reinterpret_cast<const char*>(dst);
  for (int p0 = first; p0 < np; p0 += stride) {
    const int p = p0 + lane;
    const uint32_t lds = lds_byte_addr(d + (long)p0 * 16);
    if (p < np) asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"((uint32_t)p * 16), "s"(rs), "{m0}"(lds) : "memory");
  }
}

__device__ __forceinline__ float load_bypass_l1(const float* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <typename ST, int LDSB>
__global__ __launch_bounds__(pro_threads(LDSB), 4) void k_prologue_lds(const ST* __restrict__ x, const ST* __restrict__ g0,
                                                       const ST* __restrict__ be0, const ST* __restrict__ g1,
                                                       const ST* __restrict__ be1, ST* __restrict__ h1,
                                                       float* __restrict__ stats, int B, int T, int D) {
  constexpr int N = 4;
  constexpr int Q = MAXD / (64 * N);
  __shared__ __attribute__((aligned(16))) char sx[LDSB];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const long NR = (long)B * T;
  const long base = (long)b * T * D;
  const int S = D / T;
  const float invS = 1.0f / (float)S, invD = 1.0f / (float)D;

  // 1. statistics of norm0 (collected one row per lane, stored after the
  // loop), raw rows into LDS
  float lmu0 = 0.f, lrs0 = 0.f;
  // the wave's next row is loaded while the current one is reduced
  Raw<ST, N> pr[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) ldr(x + base + (long)min(wave, T - 1) * D + min((lane + 64 * q) * N, D - N), pr[q]);
  for (int j = wave; j < T; j += nw) {
    Raw<ST, N> rr[Q];
    float v[Q][N];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      rr[q] = pr[q];
      ldr(x + base + (long)min(j + nw, T - 1) * D + min((lane + 64 * q) * N, D - N), pr[q]);
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      unpack(rr[q], v[q]);
      const float m = c < D ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) s += m * v[q][e];
    }
    const float mean = wave_sum_dpp(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const float m = c < D ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float dd = v[q][e] - mean;
        s2 += m * dd * dd;
      }
      if (c < D) *reinterpret_cast<uint2*>(sx + ((long)j * D + c) * 2) = make_uint2(rr[q].w[0], rr[q].w[1]);
    }
    const float rstd = rsqrtf(wave_sum_dpp(s2) * invD + EPS_OUTER);
    const int k = (j - wave) / nw;  // this wave's k-th row
    lmu0 = lane == k ? mean : lmu0;
    lrs0 = lane == k ? rstd : lrs0;
  }
  {
    const int nr = wave < T ? (T - wave + nw - 1) / nw : 0;
    if (lane < nr) {
      stats[ST_MU0 * NR + (long)b * T + wave + lane * nw] = lmu0;
      stats[ST_RS0 * NR + (long)b * T + wave + lane * nw] = lrs0;
    }
  }
  __syncthreads();

  // 2. per-lane source rows and their statistics; out1's affine for this lane's columns
  float nmr[Q], rs[Q];
  int jq[Q];
  Raw<ST, N> rg1[Q], rb1[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = (lane + 64 * q) * N;
    const int cc = min(c, D - N);
    const int j = div_small(cc, invS);
    jq[q] = j;
    rs[q] = load_bypass_l1(stats + ST_RS0 * NR + (long)b * T + j);
    nmr[q] = -load_bypass_l1(stats + ST_MU0 * NR + (long)b * T + j) * rs[q];
    ldr(g1 + cc, rg1[q]);
    ldr(be1 + cc, rb1[q]);
  }

  // 3. out1 rows; h1 by buffer stores issued on every lane (columns past D
  // get an out-of-range offset), the row statistics collected one row per
  // lane and stored after the loop, so the loop has no branches
  const __amdgpu_buffer_rsrc_t hrs = row_rsrc(h1 + base, (long)T * D * (long)sizeof(ST));
  float lmu = 0.f, lrs = 0.f;
  for (int i = wave; i < T; i += nw) {
    float r[Q][N];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const int cc = min(c, D - N);
      const int j = jq[q];
      const int sc = i * S + (cc - j * S);
      float a[N], gg[N], bb[N], xi[N];
      const uint2 ra = *reinterpret_cast<const uint2*>(sx + ((long)j * D + sc) * 2);
      const uint2 rx = *reinterpret_cast<const uint2*>(sx + ((long)i * D + cc) * 2);
      a[0] = lo16<ST>(ra.x); a[1] = hi16<ST>(ra.x); a[2] = lo16<ST>(ra.y); a[3] = hi16<ST>(ra.y);
      xi[0] = lo16<ST>(rx.x); xi[1] = hi16<ST>(rx.x); xi[2] = lo16<ST>(rx.y); xi[3] = hi16<ST>(rx.y);
      ldv(g0 + sc, gg);
      ldv(be0 + sc, bb);
      const float m = c < D ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        r[q][e] = mixed_residual(a[e], rs[q], nmr[q], gg[e], bb[e], xi[e]);
        s += m * r[q][e];
      }
    }
    const float mean = wave_sum_dpp(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const float m = c < D ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float dd = r[q][e] - mean;
        s2 += m * dd * dd;
      }
    }
    const float rstd = rsqrtf(wave_sum_dpp(s2) * invD + EPS_OUTER);
    const float nmrs = -mean * rstd;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      float gg[N], bb[N], o[N];
      unpack(rg1[q], gg);
      unpack(rb1[q], bb);
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = fmaf(fmaf(r[q][e], rstd, nmrs), gg[e], bb[e]);
      bst4<ST>(hrs, c < D ? (uint32_t)(c * (int)sizeof(ST)) : 0x80000000u, (uint32_t)(i * D * (int)sizeof(ST)), o);
    }
    const int k = (i - wave) / nw;  // this wave's k-th row
    lmu = lane == k ? mean : lmu;
    lrs = lane == k ? rstd : lrs;
  }
  const int nr = wave < T ? (T - wave + nw - 1) / nw : 0;
  if (lane < nr) {
    stats[ST_MU1 * NR + (long)b * T + wave + lane * nw] = lmu;
    stats[ST_RS1 * NR + (long)b * T + wave + lane * nw] = lrs;
  }
}

// ---------------------------------------------------------------------------
// hidden = LN_x(U) * silu(LN_gate(G)).  One workgroup per GATE_ROWS rows of
// Z, one thread per N-element chunk of U (and the matching chunk of G); the
// next row's chunks are loaded while the current row is reduced.
// The statistics come from the stored (rounded) Z, which the backward re-reads.
// One wave per row; Q = chunks of N elements per lane (Q * 64 * N >= H).
// Loads use clamped in-bounds addresses and masks instead of branches, so a
// row's loads are all in flight together.
template <typename ST, int N, int Q>
__global__ __launch_bounds__(256) void k_gate_fwd(const ST* __restrict__ Z, const ST* __restrict__ gx,
                                                  const ST* __restrict__ bx, const ST* __restrict__ gg,
                                                  const ST* __restrict__ bg, ST* __restrict__ hid,
                                                  float* __restrict__ stats, long NR, int H) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + wave;
  if (row >= NR) return;
  const ST* z = Z + row * 2 * H;
  const float invH = 1.0f / (float)H;
  Raw<ST, N> ru[Q], rg[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = min((lane + 64 * q) * N, H - N);
    ldr(z + c, ru[q]);
    ldr(z + H + c, rg[q]);
  }
  float su = 0.f, sg = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const float m = ((lane + 64 * q) * N < H) ? 1.f : 0.f;
    float u[N], g[N];
    unpack(ru[q], u);
    unpack(rg[q], g);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      su += m * u[e];
      sg += m * g[e];
    }
  }
  const float mu_u = wave_sum(su) * invH, mu_g = wave_sum(sg) * invH;
  float vu = 0.f, vg = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    // masked deviation m (z - mu) as one FMA: m z + (-m mu)
    const float m = ((lane + 64 * q) * N < H) ? 1.f : 0.f;
    const float omu = -m * mu_u, omg = -m * mu_g;
    float u[N], g[N];
    unpack(ru[q], u);
    unpack(rg[q], g);
#pragma unroll
    for (int e = 0; e < N; ++e) {
      const float du = fmaf(u[e], m, omu), dg = fmaf(g[e], m, omg);
      vu = fmaf(du, du, vu);
      vg = fmaf(dg, dg, vg);
    }
  }
  const float rs_u = rsqrtf(wave_sum(vu) * invH + EPS_INNER);
  const float rs_g = rsqrtf(wave_sum(vg) * invH + EPS_INNER);
  const float nmr_u = -mu_u * rs_u, nmr_g = -mu_g * rs_g;
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = (lane + 64 * q) * N;
    if (c < H) {
      float u[N], g[N], cgx[N], cbx[N], cgg[N], cbg[N], o[N];
      unpack(ru[q], u);
      unpack(rg[q], g);
      ldv(gx + c, cgx);
      ldv(bx + c, cbx);
      ldv(gg + c, cgg);
      ldv(bg + c, cbg);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float ux = fmaf(fmaf(u[e], rs_u, nmr_u), cgx[e], cbx[e]);
        const float ug = fmaf(fmaf(g[e], rs_g, nmr_g), cgg[e], cbg[e]);
        o[e] = ux * (ug * sigmoidf_(ug));
      }
      stv(hid + row * H + c, o);
    }
  }
  if (lane == 0) {
    stats[ST_MUX * NR + row] = mu_u;
    stats[ST_RSX * NR + row] = rs_u;
    stats[ST_MUG * NR + row] = mu_g;
    stats[ST_RSG * NR + row] = rs_g;
  }
}

// ---------------------------------------------------------------------------
// y = norm2(r2), r2 = out1 + out2 in the storage dtype.  One wave per row,
// persistent: wave w of the grid takes rows w, w + W, w + 2W, ... (W waves in
// the grid).  The affine of the wave's columns is loaded once; rows are
// loaded one ahead into two alternating register sets; y and the statistics
// are written by buffer stores issued on every lane (out-of-range offsets
// where nothing is written), so the loop has no branches.
template <typename ST, int N>
__global__ __launch_bounds__(256) void k_ln2_fwd(const ST* __restrict__ r2, const ST* __restrict__ g2,
                                                 const ST* __restrict__ be2, ST* __restrict__ y,
                                                 float* __restrict__ stats, long NR, int D) {
  constexpr int Q = (MAXD + 64 * N - 1) / (64 * N);
  constexpr int SZ = (int)sizeof(ST);
  const int lane = threadIdx.x & 63;
  const long gw = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const long W = (long)gridDim.x * 4;
  if (gw >= NR) return;
  const float invD = 1.0f / (float)D;
  Raw<ST, N> rg[Q], rb[Q], buf[2][Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int cc = min((lane + 64 * q) * N, D - N);
    ldr(g2 + cc, rg[q]);
    ldr(be2 + cc, rb[q]);
  }
  const __amdgpu_buffer_rsrc_t ys = row_rsrc(y, NR * D * SZ);
  const __amdgpu_buffer_rsrc_t ms = row_rsrc(stats + ST_MU2 * NR, NR * 4);
  const __amdgpu_buffer_rsrc_t rss = row_rsrc(stats + ST_RS2 * NR, NR * 4);
  auto load = [&](int k, long row) {
    const ST* r = r2 + min(row, NR - 1) * D;
#pragma unroll
    for (int q = 0; q < Q; ++q) ldr(r + min((lane + 64 * q) * N, D - N), buf[k][q]);
  };
  auto compute = [&](int k, long row) {
    const bool valid = row < NR;
    float v[Q][N];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float m = (lane + 64 * q) * N < D ? 1.f : 0.f;
      unpack(buf[k][q], v[q]);
#pragma unroll
      for (int e = 0; e < N; ++e) s += m * v[q][e];
    }
    const float mean = wave_sum(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float m = (lane + 64 * q) * N < D ? 1.f : 0.f;
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float dd = v[q][e] - mean;
        s2 += m * dd * dd;
      }
    }
    const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
    const uint32_t soff = (uint32_t)(min(row, NR - 1) * D * SZ);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      float gg[N], bb[N], o[N];
      unpack(rg[q], gg);
      unpack(rb[q], bb);
#pragma unroll
      for (int e = 0; e < N; ++e) o[e] = (v[q][e] - mean) * rstd * gg[e] + bb[e];
      bstv<ST, N>(ys, valid && c < D ? (uint32_t)(c * SZ) : 0x80000000u, soff, o);
    }
    const uint32_t so = valid && lane == 0 ? (uint32_t)(row * 4) : 0x80000000u;
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mean), ms, so, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(rstd), rss, so, 0, 0);
  };
  load(0, gw);
  for (long row = gw; row < NR; row += 2 * W) {
    load(1, row + W);
    compute(0, row);
    load(0, row + 2 * W);
    compute(1, row + W);
  }
}

// ---------------------------------------------------------------------------
// Backward row-group kernels: blockIdx.x = token t, blockIdx.y = group of
// rpg samples; thread k owns the N-element chunks k, k + blockDim,
// ... (QC of them) of every row it visits.  Partial sums of parameter
// gradients over the group's rows are written to part[.][group][t][col].

// The three D-wide backward kernels below use one wave per row: a workgroup
// of 4 waves walks the rows (b, t) of one group of samples at one token t,
// wave w taking b = first + w, first + w + 4, ...  Lane l owns the columns
// (l + 64q) * N; its parameter-gradient partial sums stay in registers and
// the 4 waves' sums are added in a fixed order through LDS at the end.

// Adds the four waves' per-column partials (lane-owned columns (l + 64q) * N)
// in a fixed order through LDS (4 x D floats) and writes them to out[0, D).
template <int N, int Q>
__device__ __forceinline__ void combine_waves_store(const float (&acc)[Q][N], float* lds, float* __restrict__ out,
                                                    int D) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = (lane + 64 * q) * N;
    if (c < D) stv(lds + wave * D + c, acc[q]);
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256) out[c] = (lds[c] + lds[D + c]) + (lds[2 * D + c] + lds[3 * D + c]);
}

// norm2 backward:  do2 = rstd2 * (dn - mean(dn) - n2 * mean(dn * n2)),  dn = dy * gamma2.
// Partials: dgamma2 (dy * n2), dbeta2 (dy), dbout[t] (do2).
template <typename ST, int N, int Q>
__global__ __launch_bounds__(256) void k_ln2_bwd(const ST* __restrict__ r2, const ST* __restrict__ dy,
                                                 const ST* __restrict__ g2, const float* __restrict__ stats,
                                                 ST* __restrict__ do2, float* __restrict__ part, int B, int T,
                                                 int D, int nb, int rpg) {
  __shared__ float lds[4 * MAXD];
  const int t = blockIdx.x, grp = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long NR = (long)B * T;
  const float invD = 1.0f / (float)D;
  float pg[Q][N], pb[Q][N], po[Q][N];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < N; ++e) pg[q][e] = pb[q][e] = po[q][e] = 0.f;
  const int b_end = min(B, (grp + 1) * rpg);
  for (int b = grp * rpg + wave; b < b_end; b += 4) {
    const long row = (long)b * T + t;
    const float mu = stats[ST_MU2 * NR + row], rs = stats[ST_RS2 * NR + row];
    Raw<ST, N> rr[Q];
    Raw<ST, N> rdy[Q], rgm[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = min((lane + 64 * q) * N, D - N);
      ldr(r2 + row * D + c, rr[q]);
      ldr(dy + row * D + c, rdy[q]);
      ldr(g2 + c, rgm[q]);
    }
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const float m = ((lane + 64 * q) * N < D) ? 1.f : 0.f;
      float r[N], d[N], gm[N];
      unpack(rr[q], r);
      unpack(rdy[q], d);
      unpack(rgm[q], gm);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float n2 = (r[e] - mu) * rs, dn = m * d[e] * gm[e];
        s1 += dn;
        s2 += dn * n2;
      }
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        float r[N], d[N], gm[N], o[N];
        unpack(rr[q], r);
        unpack(rdy[q], d);
        unpack(rgm[q], gm);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float n2 = (r[e] - mu) * rs;
          o[e] = rs * (d[e] * gm[e] - m1 - n2 * m2);
          pg[q][e] += d[e] * n2;
          pb[q][e] += d[e];
          po[q][e] += o[e];
        }
        stv(do2 + row * D + c, o);
      }
    }
  }
  const long blk = (long)nb * T * D;
  float* out = part + ((long)grp * T + t) * D;
  combine_waves_store(pg, lds, out, D);
  combine_waves_store(pb, lds, out + blk, D);
  combine_waves_store(po, lds, out + 2 * blk, D);
}

// Backward of hidden = LN_x(U) * silu(LN_gate(G)):
//   ux = LN_x(U), ug = LN_gate(G), s = sigmoid(ug)
//   d ux = dh * ug * s,  d ug = dh * ux * s * (1 + ug * (1 - s))
//   dU = rstd_x * (dnx - mean(dnx) - nx * mean(dnx * nx)),  dnx = d ux * gamma_x   (same for G)
// Partials: dgamma_x, dbeta_x, dgamma_g, dbeta_g, and db1[t] (the sum of dZ).
// Rows and affine constants stay packed in registers; the cheap elementwise
// terms are recomputed after the row reduction instead of being kept live,
// which keeps occupancy (and loads in flight) high.
template <typename ST, int N>
struct GateTerms {
  float nx[N], ng[N], dux[N], dug[N];
};

template <typename ST, int N>
__device__ __forceinline__ void gate_terms(const Raw<ST, N>& ru, const Raw<ST, N>& rg, const Raw<ST, N>& rdh,
                                           const Raw<ST, N>& rgx, const Raw<ST, N>& rbx, const Raw<ST, N>& rgg,
                                           const Raw<ST, N>& rbg, float mux, float rsx, float mug, float rsg,
                                           GateTerms<ST, N>& o) {
  float u[N], g[N], dh[N], cgx[N], cbx[N], cgg[N], cbg[N];
  unpack(ru, u);
  unpack(rg, g);
  unpack(rdh, dh);
  unpack(rgx, cgx);
  unpack(rbx, cbx);
  unpack(rgg, cgg);
  unpack(rbg, cbg);
#pragma unroll
  for (int e = 0; e < N; ++e) {
    o.nx[e] = fmaf(u[e], rsx, -mux * rsx);  // the forward's form of the normalised value
    o.ng[e] = fmaf(g[e], rsg, -mug * rsg);
    const float ux = o.nx[e] * cgx[e] + cbx[e];
    const float ug = o.ng[e] * cgg[e] + cbg[e];
    const float sgm = sigmoidf_(ug);
    o.dux[e] = dh[e] * ug * sgm;
    o.dug[e] = dh[e] * ux * sgm * (1.f + ug * (1.f - sgm));
  }
}

template <typename ST, int N, int QC>
struct GateBwdSlot {
  float st[4];
  Raw<ST, N> u[QC], g[QC], dh[QC];
};

// One thread per N-element chunk; RPI rows per iteration are loaded together
// (straight-line code, clamped in-bounds addresses) and share one block
// reduction, so several rows' loads are in flight per workgroup.
template <typename ST, int N, int QC, int MAXT, int RPI>
__global__ __launch_bounds__(MAXT) void k_gate_bwd(const ST* __restrict__ Z, const ST* __restrict__ dhid,
                                                   const ST* __restrict__ gx, const ST* __restrict__ bx,
                                                   const ST* __restrict__ gg, const ST* __restrict__ bg,
                                                   const float* __restrict__ stats, ST* __restrict__ dZ,
                                                   float* __restrict__ pgate, float* __restrict__ pb1, int B,
                                                   int T, int H, int nb, int rpg) {
  __shared__ float red[2 * 4 * RPI * 16];
  const int t = blockIdx.x, grp = blockIdx.y;
  const int nw = blockDim.x >> 6;
  const long NR = (long)B * T;
  const float invH = 1.0f / (float)H;
  Raw<ST, N> rgx[QC], rbx[QC], rgg[QC], rbg[QC];
  float agx[QC][N], abx[QC][N], agg[QC][N], abg[QC][N], au[QC][N], ag[QC][N];
  float msk[QC];
#pragma unroll
  for (int k = 0; k < QC; ++k) {
    const int craw = (threadIdx.x + k * blockDim.x) * N;
    const int c = min(craw, H - N);
    msk[k] = craw < H ? 1.f : 0.f;
#pragma unroll
    for (int e = 0; e < N; ++e) agx[k][e] = abx[k][e] = agg[k][e] = abg[k][e] = au[k][e] = ag[k][e] = 0.f;
    ldr(gx + c, rgx[k]);
    ldr(bx + c, rbx[k]);
    ldr(gg + c, rgg[k]);
    ldr(bg + c, rbg[k]);
  }
  const int b_begin = grp * rpg, b_end = min(B, (grp + 1) * rpg);
  int parity = 0;
  for (int b0 = b_begin; b0 < b_end; b0 += RPI) {
    GateBwdSlot<ST, N, QC> cur[RPI];
    float valid[RPI];
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
      const int b = min(b0 + r, b_end - 1);
      valid[r] = (b0 + r < b_end) ? 1.f : 0.f;
      const long row = (long)b * T + t;
      cur[r].st[0] = stats[ST_MUX * NR + row];
      cur[r].st[1] = stats[ST_RSX * NR + row];
      cur[r].st[2] = stats[ST_MUG * NR + row];
      cur[r].st[3] = stats[ST_RSG * NR + row];
#pragma unroll
      for (int k = 0; k < QC; ++k) {
        const int c = min((int)((threadIdx.x + k * blockDim.x) * N), H - N);
        ldr(Z + row * 2 * H + c, cur[r].u[k]);
        ldr(Z + row * 2 * H + H + c, cur[r].g[k]);
        ldr(dhid + row * H + c, cur[r].dh[k]);
      }
    }
    float sm[4 * RPI];
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
      const float mux = cur[r].st[0], rsx = cur[r].st[1], mug = cur[r].st[2], rsg = cur[r].st[3];
      float s0 = 0.f, s1 = 0.f, s2 = 0.f, s3 = 0.f;
#pragma unroll
      for (int k = 0; k < QC; ++k) {
        GateTerms<ST, N> gt;
        gate_terms(cur[r].u[k], cur[r].g[k], cur[r].dh[k], rgx[k], rbx[k], rgg[k], rbg[k], mux, rsx, mug, rsg, gt);
        float cgx[N], cgg[N];
        unpack(rgx[k], cgx);
        unpack(rgg[k], cgg);
        const float w = msk[k] * valid[r];
#pragma unroll
        for (int e = 0; e < N; ++e) {
          const float dux = w * gt.dux[e], dug = w * gt.dug[e];
          agx[k][e] += dux * gt.nx[e];
          abx[k][e] += dux;
          agg[k][e] += dug * gt.ng[e];
          abg[k][e] += dug;
          const float dnx = dux * cgx[e], dng = dug * cgg[e];
          s0 += dnx;
          s1 += dnx * gt.nx[e];
          s2 += dng;
          s3 += dng * gt.ng[e];
        }
      }
      sm[4 * r + 0] = s0;
      sm[4 * r + 1] = s1;
      sm[4 * r + 2] = s2;
      sm[4 * r + 3] = s3;
    }
    block_sum(sm, red, nw, parity);
    parity ^= 1;
#pragma unroll
    for (int r = 0; r < RPI; ++r)
#pragma unroll
      for (int k = 0; k < QC; ++k) {
        opaque(cur[r].u[k]);
        opaque(cur[r].g[k]);
        opaque(cur[r].dh[k]);
      }
#pragma unroll
    for (int r = 0; r < RPI; ++r) {
      if (b0 + r < b_end) {
        const long row = (long)(b0 + r) * T + t;
        const float mux = cur[r].st[0], rsx = cur[r].st[1], mug = cur[r].st[2], rsg = cur[r].st[3];
        const float m1 = sm[4 * r] * invH, m2 = sm[4 * r + 1] * invH;
        const float m3 = sm[4 * r + 2] * invH, m4 = sm[4 * r + 3] * invH;
#pragma unroll
        for (int k = 0; k < QC; ++k) {
          const int c = (threadIdx.x + k * blockDim.x) * N;
          if (c < H) {
            GateTerms<ST, N> gt;
            gate_terms(cur[r].u[k], cur[r].g[k], cur[r].dh[k], rgx[k], rbx[k], rgg[k], rbg[k], mux, rsx, mug, rsg,
                       gt);
            float cgx[N], cgg[N], du[N], dg[N];
            unpack(rgx[k], cgx);
            unpack(rgg[k], cgg);
#pragma unroll
            for (int e = 0; e < N; ++e) {
              du[e] = rsx * (gt.dux[e] * cgx[e] - m1 - gt.nx[e] * m2);
              dg[e] = rsg * (gt.dug[e] * cgg[e] - m3 - gt.ng[e] * m4);
              au[k][e] += du[e];
              ag[k][e] += dg[e];
            }
            stv(dZ + row * 2 * H + c, du);
            stv(dZ + row * 2 * H + H + c, dg);
          }
        }
      }
    }
  }
  const long blk = (long)nb * T * H;
  const long o = ((long)grp * T + t) * H;
  const long o1 = ((long)grp * T + t) * 2 * H;
#pragma unroll
  for (int k = 0; k < QC; ++k) {
    const int c = (threadIdx.x + k * blockDim.x) * N;
    if (c < H) {
      stv(pgate + o + c, agx[k]);
      stv(pgate + blk + o + c, abx[k]);
      stv(pgate + 2 * blk + o + c, agg[k]);
      stv(pgate + 3 * blk + o + c, abg[k]);
      stv(pb1 + o1 + c, au[k]);
      stv(pb1 + o1 + H + c, ag[k]);
    }
  }
}

// Gate / SiLU / inner LayerNorm backward for H % 4 == 0: one thread per
// 4-column chunk of U (and the matching chunk of G and d hidden), one
// workgroup walking the rpg rows (b, t) of one sample group at one
// token t.  Rows go two at a time: the pair's u, g, d hidden sit in a
// two-slot register ring, refilled with the next pair (unconditional loads
// from clamped rows) before the pair's one block reduction of eight sums, so
// the loads stay in flight across its LDS-only barrier; the row statistics
// are staged in LDS once.  The per-element terms are kept in registers
// between the reduction and the dZ computation.  Rows past B get zero weight
// and out-of-range (dropped) buffer stores.
//   dux = dh * ug * sigmoid(ug)                  (d of the LN_x output)
//   dug = dh * ux * sigmoid(ug) * (1 + ug (1 - sigmoid(ug)))
//   dU  = rsx (dux gx - mean(dux gx) - nx mean(dux gx nx)), same for dG.
constexpr int RING = 2;

template <typename ST, int MAXT, int RPG>
__global__ __launch_bounds__(MAXT) void k_gate_bwd_ring(const ST* __restrict__ Z, const ST* __restrict__ dhid,
                                                        const ST* __restrict__ gx, const ST* __restrict__ bx,
                                                        const ST* __restrict__ gg, const ST* __restrict__ bg,
                                                        const float* __restrict__ stats, ST* __restrict__ dZ,
                                                        float* __restrict__ pgate, float* __restrict__ pb1, int B,
                                                        int T, int H, int nb) {
  __shared__ float red8[2 * 16 * 8];
  __shared__ float4 sst[MAX_ROWS_PER_GROUP];
  // the group size is a compile-time constant: the row loop keeps a static trip count
  static_assert(RPG >= MIN_ROWS_PER_GROUP && RPG <= MAX_ROWS_PER_GROUP && (RPG & (RPG - 1)) == 0, "group size");
  constexpr int rpg = RPG;
  constexpr int SZ = (int)sizeof(ST);
  const int t = blockIdx.x, grp = blockIdx.y;
  const int nw = blockDim.x >> 6;
  const long NR = (long)B * T;
  const float invH = 1.0f / (float)H;
  const int craw = threadIdx.x * 4;
  const int c = min(craw, H - 4);
  float cgx[4], cbx[4], cgg[4], cbg[4];
  ldv(gx + c, cgx);
  ldv(bx + c, cbx);
  ldv(gg + c, cgg);
  ldv(bg + c, cbg);
  float agx[4], abx[4], agg[4], abg[4], au[4], ag[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) agx[e] = abx[e] = agg[e] = abg[e] = au[e] = ag[e] = 0.f;

  const int b0 = grp * rpg, bl = min(B, b0 + rpg) - 1;
  // every row access: uniform row offset (scalar) + this thread's column offset
  const __amdgpu_buffer_rsrc_t zrs = row_rsrc(Z, NR * 2 * H * SZ);
  const __amdgpu_buffer_rsrc_t hrs = row_rsrc(dhid, NR * H * SZ);
  const __amdgpu_buffer_rsrc_t drs = row_rsrc(dZ, NR * 2 * H * SZ);
  const uint32_t vu = (uint32_t)(c * SZ), vg = (uint32_t)((H + c) * SZ);
  const uint32_t zrow = (uint32_t)(2 * H * SZ), hrow = (uint32_t)(H * SZ);

  zero_red(red8);
  // the group's inner-LN statistics (mux, rsx, mug, rsg per row) staged in LDS once
  for (int i = threadIdx.x; i < 4 * rpg; i += blockDim.x) {
    const int r = i >> 2, q = i & 3;
    const long row = (long)min(b0 + r, bl) * T + t;
    reinterpret_cast<float*>(sst)[i] = stats[(ST_MUX + q) * NR + row];
  }
  Raw<ST, 4> ru[RING], rg[RING], rd[RING];
  // d hidden of rows past B and of columns past H reads as zero (out-of-range
  // offset), which zeroes every term of theirs
  auto load_row = [&](int slot, int r) {
    const uint32_t row = (uint32_t)(min(b0 + r, bl) * T + t);
    bld4<ST>(zrs, vu, row * zrow, ru[slot]);
    bld4<ST>(zrs, vg, row * zrow, rg[slot]);
    bld4<ST>(hrs, (b0 + r <= bl && craw < H) ? vu : 0x80000000u, row * hrow, rd[slot]);
  };
  // two dropped (out-of-range) stores after each slot's loads, as every row
  // step issues: the compiler's wait counts at the loop head then match the
  // steady state instead of forcing the next rows' loads to complete
  const float zero4[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int p = 0; p < RING; ++p) {
    __builtin_amdgcn_sched_barrier(0);
    load_row(p, p);
    bst4<ST>(drs, 0x80000000u + 64u * p, 0, zero4);  // distinct offsets: not merged as redundant
    bst4<ST>(drs, 0x80000020u + 64u * p, 0, zero4);
    __builtin_amdgcn_sched_barrier(0);
  }
  __syncthreads();

  // RING rows (all ring slots) per step: consume them, refill the slots with
  // rows r + RING .. r + 2 RING - 1 (PREFETCH), one block reduction of the
  // rows' 4 RING sums, store the rows of dZ
  int parity = 0;
  auto pair_step = [&](int r, auto prefetch) {
    float nx[RING][4], ng[RING][4], dnx[RING][4], dng[RING][4], rsx[RING], rsg[RING], sm[4 * RING];
    uint32_t rowk[RING];
    bool validk[RING];
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      validk[k] = b0 + r + k <= bl;
      const float4 sr = sst[r + k];
      const float mux = sr.x, mug = sr.z;
      rsx[k] = sr.y;
      rsg[k] = sr.w;
      float u[4], g[4], dh[4];
      unpack(ru[k], u);
      unpack(rg[k], g);
      unpack(rd[k], dh);
      rowk[k] = (uint32_t)(min(b0 + r + k, bl) * T + t);
      if constexpr (decltype(prefetch)::value) load_row(k, r + k + RING);
      sm[4 * k] = sm[4 * k + 1] = sm[4 * k + 2] = sm[4 * k + 3] = 0.f;
      const float ox = -mux * rsx[k], og = -mug * rsg[k];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        nx[k][e] = u[e] * rsx[k] + ox;
        ng[k][e] = g[e] * rsg[k] + og;
        const float ux = nx[k][e] * cgx[e] + cbx[e];
        const float ug = ng[k][e] * cgg[e] + cbg[e];
        const float sgm = sigmoidf_(ug);
        // dux = dh ug s;  dug = dh ux s (1 + ug (1 - s)) = dh ux (s + ug s (1 - s))
        const float us = ug * sgm;
        const float dux = dh[e] * us;
        const float dug = (dh[e] * ux) * fmaf(us, 1.f - sgm, sgm);
        dnx[k][e] = dux * cgx[e];
        dng[k][e] = dug * cgg[e];
        sm[4 * k] += dnx[k][e];
        sm[4 * k + 1] += dnx[k][e] * nx[k][e];
        sm[4 * k + 2] += dng[k][e];
        sm[4 * k + 3] += dng[k][e] * ng[k][e];
        agx[e] += dux * nx[k][e];
        abx[e] += dux;
        agg[e] += dug * ng[k][e];
        abg[e] += dug;
      }
    }
    static_assert(4 * RING == 8, "one block reduction of the pair's eight sums");
    block_sum8(sm, red8, parity);
    parity ^= 1;
#pragma unroll
    for (int k = 0; k < RING; ++k) {
      // rs (dn - m1 - n m2) = dn rs + (n (-rs m2) - rs m1): two FMAs per element
      const float c1x = -rsx[k] * (sm[4 * k] * invH), c2x = -rsx[k] * (sm[4 * k + 1] * invH);
      const float c1g = -rsg[k] * (sm[4 * k + 2] * invH), c2g = -rsg[k] * (sm[4 * k + 3] * invH);
      float du[4], dg[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        du[e] = fmaf(dnx[k][e], rsx[k], fmaf(nx[k][e], c2x, c1x));
        dg[e] = fmaf(dng[k][e], rsg[k], fmaf(ng[k][e], c2g, c1g));
        // a row past B has all four sums zero, so du = dg = 0 there; columns
        // past H are never stored
        au[e] += du[e];
        ag[e] += dg[e];
      }
      const bool sok = validk[k] && craw < H;
      bst4<ST>(drs, sok ? vu : 0x80000000u, rowk[k] * zrow, du);
      bst4<ST>(drs, sok ? vg : 0x80000000u, rowk[k] * zrow, dg);
    }
  };
  // rpg is a power of two of at least MIN_ROWS_PER_GROUP: the ring slots are consumed together
  static_assert(MIN_ROWS_PER_GROUP % RING == 0, "whole ring steps per group");
#pragma unroll 1
  for (int r0 = 0; r0 < rpg - RING; r0 += RING) pair_step(r0, std::true_type{});
  pair_step(rpg - RING, std::false_type{});
  if (craw < H) {
    const long blk = (long)nb * T * H;
    const long o = ((long)grp * T + t) * H;
    const long o1 = ((long)grp * T + t) * 2 * H;
    stv(pgate + o + c, agx);
    stv(pgate + blk + o + c, abx);
    stv(pgate + 2 * blk + o + c, agg);
    stv(pgate + 3 * blk + o + c, abg);
    stv(pb1 + o1 + c, au);
    stv(pb1 + o1 + H + c, ag);
  }
}

// Backward tail for 16-bit storage, one workgroup (8 waves for the 160 KB LDS
// tier, 4 for the smaller ones) per sample b with the sample staged in LDS
// (at most 160 KB), so the token-mix gathers read LDS instead of 40-byte
// pieces of HBM lines.  Wave w of nw owns the contiguous rows R*w .. R*w+R-1
// (R = ceil(T / nw)) in both row phases.
//   1. x[b] -> LDS by direct 16-byte copies, all in flight together (plain
//      loads when x is not 16-byte aligned);
//   2. norm1 backward per row i: r1 = token_mix(norm0(x)) + x, the mixed term
//      gathered from LDS (column run i of every row) and the residual x[i]
//      read from global memory; dr1 = rstd1 (dn - mean(dn) - n1 mean(dn n1)),
//      dn = d(out1) gamma1.  Each lane writes its dr1 values into the LDS
//      slots its own gather just read: that run of x is needed by row i only,
//      and the slot of dr1[i, c] is the slot of da0 = token_mix(dr1) at
//      [c / S, i S + c % S], so after the phase LDS holds da0 row by row;
//   3. norm0 backward per row j: da0[j] is LDS row j, dr1[j] is gathered from
//      LDS, n0 from x[j] (global, next row prefetched) and the saved
//      statistics; dx = dr1 + rstd0 (dn - mean(dn) - n0 mean(dn n0)),
//      dn = da0 gamma0;
//   4. the waves' column partials of both phases added through LDS in a
//      fixed order and stored.
// The next row's global operands are loaded while the current row is
// computed; row statistics are read once per wave, one row per lane.
// Partials: part[k][b][col], k = 0..3: dgamma0, dbeta0, dgamma1, dbeta1.
// Needs D % 8 == 0 (16-byte rows), S % 4 == 0, T * D * 2 <= 160 KB.
__device__ __forceinline__ void wave_partials_to_lds(const float (&acc)[MAXD / 256][4], float* lds, int wave,
                                                     int lane, int D) {
#pragma unroll
  for (int q = 0; q < MAXD / 256; ++q) {
    const int c = (lane + 64 * q) * 4;
    if (c < D) *reinterpret_cast<float4*>(lds + wave * D + c) = make_float4(acc[q][0], acc[q][1], acc[q][2], acc[q][3]);
  }
}
// out[c] = sum over the nw waves' rows of lds (fixed order), c < D.
__device__ __forceinline__ void sum_wave_rows(const float* lds, float* __restrict__ out, int nw, int D) {
  for (int c = threadIdx.x; c < D; c += blockDim.x) {
    float t = 0.f;
    for (int w = 0; w < nw; ++w) t += lds[w * D + c];
    out[c] = t;
  }
}

template <typename ST, int LDSB>
__global__ __launch_bounds__(tail_threads(LDSB), 2) void k_tail_bwd_lds(const ST* __restrict__ x, const ST* __restrict__ dh1,
                                                       const ST* __restrict__ g0, const ST* __restrict__ be0,
                                                       const ST* __restrict__ g1, const float* __restrict__ stats,
                                                       ST* __restrict__ dx, float* __restrict__ part, int B, int T,
                                                       int D) {
  constexpr int N = 4;
  constexpr int Q = MAXD / (64 * N);
  __shared__ __attribute__((aligned(16))) char sx[LDSB];
  float* const lf = reinterpret_cast<float*>(sx);
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = blockDim.x >> 6;
  const long NR = (long)B * T;
  const long base = (long)b * T * D;
  const long srow = (long)b * T;  // first row of the sample
  const int S = D / T;
  const float invS = 1.0f / (float)S, invD = 1.0f / (float)D;
  const long pblk = (long)B * D;
  const int R = (T + nw - 1) / nw;
  const int r0 = min(wave * R, T), r1 = min(r0 + R, T);  // this wave's rows (none if r0 == T)
  const int i0 = min(r0, T - 1);
  const __amdgpu_buffer_rsrc_t dxs = row_rsrc(dx + srow * D, (long)T * D * (long)sizeof(ST));
  const uint32_t rowb = (uint32_t)D * (uint32_t)sizeof(ST);

  // 1. x[b] -> LDS
  if ((reinterpret_cast<uintptr_t>(x) & 15) == 0) {
    copy_to_lds(x + base, sx, T * D * 2, wave * 64, nw * 64, lane);
  } else {
    for (int j = wave; j < T; j += nw) {
#pragma unroll
      for (int q = 0; q < Q; ++q) {
        const int c = (lane + 64 * q) * N;
        if (c < D)
          *reinterpret_cast<uint2*>(sx + ((long)j * D + c) * 2) = *reinterpret_cast<const uint2*>(x + base + (long)j * D + c);
      }
    }
  }
  // gather sources of this lane's columns: row c/S (same for every row of the sample);
  // the first row's d(out1), x, gathered gamma0 / beta0
  int jq[Q];
  float nmr0[Q], rs0[Q];
  Raw<ST, N> rg1[Q], rgg0[Q], pdh[Q], px[Q], pg0[Q], pb0[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int cc = min((lane + 64 * q) * N, D - N);
    const int j = div_small(cc, invS);
    jq[q] = j;
    rs0[q] = stats[ST_RS0 * NR + srow + j];
    nmr0[q] = -stats[ST_MU0 * NR + srow + j] * rs0[q];
    ldr(g1 + cc, rg1[q]);
    ldr(g0 + cc, rgg0[q]);
    ldr(dh1 + (srow + i0) * D + cc, pdh[q]);
    ldr(x + base + (long)i0 * D + cc, px[q]);
    const int sc = i0 * S + (cc - j * S);
    ldr(g0 + sc, pg0[q]);
    ldr(be0 + sc, pb0[q]);
  }
  // statistics of this wave's rows, lane l holding row r0 + l (vector loads:
  // scalar ones would share the LDS reads' wait counter inside the row loops)
  const int ri = min(r0 + lane, T - 1);
  const float lmu1 = stats[ST_MU1 * NR + srow + ri], lrs1 = stats[ST_RS1 * NR + srow + ri];
  const float lmu0 = stats[ST_MU0 * NR + srow + ri], lrs0 = stats[ST_RS0 * NR + srow + ri];
  wait_vm_all();
  __syncthreads();

  // 2. norm1 backward; dr1 into the LDS slots just gathered from
  float pa1[Q][N], pb1[Q][N];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < N; ++e) pa1[q][e] = pb1[q][e] = 0.f;
  for (int i = r0; i < r1; ++i) {
    const float mu1 = lane_f(lmu1, i - r0), rs1 = lane_f(lrs1, i - r0);
    const int in = min(i + 1, T - 1);
    Raw<ST, N> cdh[Q], cx[Q], cg0[Q], cb0[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int cc = min((lane + 64 * q) * N, D - N);
      cdh[q] = pdh[q];
      cx[q] = px[q];
      cg0[q] = pg0[q];
      cb0[q] = pb0[q];
      ldr(dh1 + (srow + in) * D + cc, pdh[q]);
      ldr(x + base + (long)in * D + cc, px[q]);
      const int scn = in * S + (cc - jq[q] * S);
      ldr(g0 + scn, pg0[q]);
      ldr(be0 + scn, pb0[q]);
    }
    float n1[Q][N], dn[Q][N], gv[Q][N];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const int cc = min(c, D - N);
      const float m = c < D ? 1.f : 0.f;
      const int sc = i * S + (cc - jq[q] * S);
      const uint2 ra = *reinterpret_cast<const uint2*>(sx + ((long)jq[q] * D + sc) * 2);
      float a[N], xi[N], gg0[N], bb0[N], gg1[N];
      a[0] = lo16<ST>(ra.x); a[1] = hi16<ST>(ra.x); a[2] = lo16<ST>(ra.y); a[3] = hi16<ST>(ra.y);
      unpack(cx[q], xi);
      unpack(cdh[q], gv[q]);
      unpack(cg0[q], gg0);
      unpack(cb0[q], bb0);
      unpack(rg1[q], gg1);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float r1v = mixed_residual(a[e], rs0[q], nmr0[q], gg0[e], bb0[e], xi[e]);
        n1[q][e] = (r1v - mu1) * rs1;
        dn[q][e] = m * gv[q][e] * gg1[e];
        s1 += dn[q][e];
        s2 += dn[q][e] * n1[q][e];
      }
    }
    const float m1 = wave_sum_dpp(s1) * invD, m2 = wave_sum_dpp(s2) * invD;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const int cc = min(c, D - N);
      float o[N];
#pragma unroll
      for (int e = 0; e < N; ++e) {
        o[e] = rs1 * (dn[q][e] - m1 - n1[q][e] * m2);
        pa1[q][e] += gv[q][e] * n1[q][e];  // columns past D: accumulated, never stored
        pb1[q][e] += gv[q][e];
      }
      // dr1[i, c] -> the slot of da0[c / S, i S + c % S] (the gather source read above)
      const int sc = i * S + (cc - jq[q] * S);
      if (c < D)
        *reinterpret_cast<uint2*>(sx + ((long)jq[q] * D + sc) * 2) =
            make_uint2(pack16x2<ST>(o[0], o[1]), pack16x2<ST>(o[2], o[3]));
    }
  }
  __syncthreads();  // LDS holds da0 = token_mix(dr1)

  // 3. norm0 backward
  float pa0[Q][N], pb0s[Q][N];
#pragma unroll
  for (int q = 0; q < Q; ++q)
#pragma unroll
    for (int e = 0; e < N; ++e) pa0[q][e] = pb0s[q][e] = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q) ldr(x + base + (long)i0 * D + min((lane + 64 * q) * N, D - N), px[q]);
  for (int j = r0; j < r1; ++j) {
    const float mu = lane_f(lmu0, j - r0), rs = lane_f(lrs0, j - r0);
    const int jn = min(j + 1, T - 1);
    Raw<ST, N> cx[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      cx[q] = px[q];
      ldr(x + base + (long)jn * D + min((lane + 64 * q) * N, D - N), px[q]);
    }
    float n0[Q][N], dn[Q][N], da[Q][N];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const int cc = min(c, D - N);
      const float m = c < D ? 1.f : 0.f;
      const uint2 rd = *reinterpret_cast<const uint2*>(sx + ((long)j * D + cc) * 2);  // da0[j, c]
      da[q][0] = lo16<ST>(rd.x); da[q][1] = hi16<ST>(rd.x); da[q][2] = lo16<ST>(rd.y); da[q][3] = hi16<ST>(rd.y);
      float xv[N], cg0[N];
      unpack(cx[q], xv);
      unpack(rgg0[q], cg0);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        n0[q][e] = (xv[e] - mu) * rs;
        dn[q][e] = m * da[q][e] * cg0[e];
        s1 += dn[q][e];
        s2 += dn[q][e] * n0[q][e];
      }
    }
    const float m1 = wave_sum_dpp(s1) * invD, m2 = wave_sum_dpp(s2) * invD;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      const int cc = min(c, D - N);
      // dr1[j, c], stored at the slot of da0[c / S, j S + c % S]
      const int sc = j * S + (cc - jq[q] * S);
      const uint2 ro = *reinterpret_cast<const uint2*>(sx + ((long)jq[q] * D + sc) * 2);
      float own[N], o[N];
      own[0] = lo16<ST>(ro.x); own[1] = hi16<ST>(ro.x); own[2] = lo16<ST>(ro.y); own[3] = hi16<ST>(ro.y);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        o[e] = own[e] + rs * (dn[q][e] - m1 - n0[q][e] * m2);
        pa0[q][e] += da[q][e] * n0[q][e];  // columns past D: accumulated, never stored
        pb0s[q][e] += da[q][e];
      }
      bst4<ST>(dxs, c < D ? (uint32_t)(c * (int)sizeof(ST)) : 0x80000000u, (uint32_t)j * rowb, o);
    }
  }
  __syncthreads();

  // 4. column partials of both phases (the LDS is free again)
  wave_partials_to_lds(pa0, lf, wave, lane, D);
  __syncthreads();
  sum_wave_rows(lf, part + (long)b * D, nw, D);
  __syncthreads();
  wave_partials_to_lds(pb0s, lf, wave, lane, D);
  __syncthreads();
  sum_wave_rows(lf, part + pblk + (long)b * D, nw, D);
  __syncthreads();
  wave_partials_to_lds(pa1, lf, wave, lane, D);
  __syncthreads();
  sum_wave_rows(lf, part + 2 * pblk + (long)b * D, nw, D);
  __syncthreads();
  wave_partials_to_lds(pb1, lf, wave, lane, D);
  __syncthreads();
  sum_wave_rows(lf, part + 3 * pblk + (long)b * D, nw, D);
}

// norm1 backward:  dr1 = rstd1 * (dn - mean(dn) - n1 * mean(dn * n1)),  dn = d(out1) * gamma1,
// with r1 = token_mix(norm0(x)) + x recomputed through the token-mix gather.
// Partials: dgamma1 (d(out1) * n1), dbeta1 (d(out1)).  Row (b, i) with i = t.
// N > 1 needs S % N == 0 (a chunk's gather source is contiguous).
template <typename ST, int N, int Q>
__global__ __launch_bounds__(256) void k_ln1_bwd(const ST* __restrict__ x, const ST* __restrict__ dh1,
                                                 const ST* __restrict__ g0, const ST* __restrict__ be0,
                                                 const ST* __restrict__ g1, const float* __restrict__ stats,
                                                 ST* __restrict__ dr1, float* __restrict__ part, int B, int T,
                                                 int D, int nb, int rpg) {
  __shared__ float lds[4 * MAXD];
  const int i = blockIdx.x, grp = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long NR = (long)B * T;
  const int S = D / T;
  const float invS = 1.0f / (float)S, invD = 1.0f / (float)D;
  float pg[Q][N], pb[Q][N];
  int src_j[Q], src_c[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = min((lane + 64 * q) * N, D - N);
    const int j = div_small(c, invS);
    src_j[q] = j;
    src_c[q] = i * S + (c - j * S);
#pragma unroll
    for (int e = 0; e < N; ++e) pg[q][e] = pb[q][e] = 0.f;
  }
  const int b_end = min(B, (grp + 1) * rpg);
  for (int b = grp * rpg + wave; b < b_end; b += 4) {
    const long row = (long)b * T + i;
    const long base = (long)b * T * D;
    const float mu1 = stats[ST_MU1 * NR + row], rs1 = stats[ST_RS1 * NR + row];
    Raw<ST, N> ra[Q], rxi[Q];
    Raw<ST, N> rg[Q];
    float mu0[Q], rs0[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = min((lane + 64 * q) * N, D - N);
      ldr(x + base + (long)src_j[q] * D + src_c[q], ra[q]);
      ldr(x + base + (long)i * D + c, rxi[q]);
      ldr(dh1 + row * D + c, rg[q]);
      mu0[q] = stats[ST_MU0 * NR + (long)b * T + src_j[q]];
      rs0[q] = stats[ST_RS0 * NR + (long)b * T + src_j[q]];
    }
    float n1[Q][N], dn[Q][N];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = min((lane + 64 * q) * N, D - N);
      const float m = ((lane + 64 * q) * N < D) ? 1.f : 0.f;
      float a[N], xi[N], gv[N], cg0[N], cb0[N], cg1[N];
      unpack(ra[q], a);
      unpack(rxi[q], xi);
      unpack(rg[q], gv);
      ldv(g0 + src_c[q], cg0);
      ldv(be0 + src_c[q], cb0);
      ldv(g1 + c, cg1);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        const float r1 = mixed_residual(a[e], rs0[q], -mu0[q] * rs0[q], cg0[e], cb0[e], xi[e]);
        n1[q][e] = (r1 - mu1) * rs1;
        dn[q][e] = m * gv[e] * cg1[e];
        s1 += dn[q][e];
        s2 += dn[q][e] * n1[q][e];
      }
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        float gv[N], o[N];
        unpack(rg[q], gv);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          o[e] = rs1 * (dn[q][e] - m1 - n1[q][e] * m2);
          pg[q][e] += gv[e] * n1[q][e];
          pb[q][e] += gv[e];
        }
        stv(dr1 + row * D + c, o);
      }
    }
  }
  const long blk = (long)nb * T * D;
  float* out = part + ((long)grp * T + i) * D;
  combine_waves_store(pg, lds, out + 2 * blk, D);
  combine_waves_store(pb, lds, out + 3 * blk, D);
}

// Token-mix adjoint and norm0 backward, row (b, j) with j = t:
//   da0 = token_mix(dr1)  (a gather: row j, column c reads row c/S, column j*S + c%S)
//   dx = dr1 + rstd0 * (dn - mean(dn) - n0 * mean(dn * n0)),  dn = da0 * gamma0.
// Partials: dgamma0 (da0 * n0), dbeta0 (da0).
template <typename ST, int N, int Q>
__global__ __launch_bounds__(256) void k_ln0_bwd(const ST* __restrict__ x, const ST* __restrict__ dr1,
                                                 const ST* __restrict__ g0, const float* __restrict__ stats,
                                                 ST* __restrict__ dx, float* __restrict__ part, int B, int T, int D,
                                                 int nb, int rpg) {
  __shared__ float lds[4 * MAXD];
  const int j = blockIdx.x, grp = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long NR = (long)B * T;
  const int S = D / T;
  const float invS = 1.0f / (float)S, invD = 1.0f / (float)D;
  float pg[Q][N], pb[Q][N];
  int src_i[Q], src_c[Q];
#pragma unroll
  for (int q = 0; q < Q; ++q) {
    const int c = min((lane + 64 * q) * N, D - N);
    const int ii = div_small(c, invS);
    src_i[q] = ii;
    src_c[q] = j * S + (c - ii * S);
#pragma unroll
    for (int e = 0; e < N; ++e) pg[q][e] = pb[q][e] = 0.f;
  }
  const int b_end = min(B, (grp + 1) * rpg);
  for (int b = grp * rpg + wave; b < b_end; b += 4) {
    const long row = (long)b * T + j;
    const long base = (long)b * T * D;
    const float mu0 = stats[ST_MU0 * NR + row], rs0 = stats[ST_RS0 * NR + row];
    Raw<ST, N> rda[Q], rown[Q];
    Raw<ST, N> rx[Q];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = min((lane + 64 * q) * N, D - N);
      ldr(dr1 + base + (long)src_i[q] * D + src_c[q], rda[q]);
      ldr(x + row * D + c, rx[q]);
      ldr(dr1 + row * D + c, rown[q]);
    }
    float n0[Q][N], dn[Q][N];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = min((lane + 64 * q) * N, D - N);
      const float m = ((lane + 64 * q) * N < D) ? 1.f : 0.f;
      float da[N], xv[N], cg0[N];
      unpack(rda[q], da);
      unpack(rx[q], xv);
      ldv(g0 + c, cg0);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        n0[q][e] = (xv[e] - mu0) * rs0;
        dn[q][e] = m * da[e] * cg0[e];
        s1 += dn[q][e];
        s2 += dn[q][e] * n0[q][e];
      }
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int c = (lane + 64 * q) * N;
      if (c < D) {
        float da[N], own[N], o[N];
        unpack(rda[q], da);
        unpack(rown[q], own);
#pragma unroll
        for (int e = 0; e < N; ++e) {
          o[e] = own[e] + rs0 * (dn[q][e] - m1 - n0[q][e] * m2);
          pg[q][e] += da[e] * n0[q][e];
          pb[q][e] += da[e];
        }
        stv(dx + row * D + c, o);
      }
    }
  }
  const long blk = (long)nb * T * D;
  float* out = part + ((long)grp * T + j) * D;
  combine_waves_store(pg, lds, out, D);
  combine_waves_store(pb, lds, out + blk, D);
}

// ---------------------------------------------------------------------------
// Fixed-order column sums of partial rows: out[c] = sum_p part[p * pstride + c],
// twelve jobs in one flat launch (job k owns blocks blk0 .. blk0 + nblk - 1).
//   * short jobs (P <= 32 rows, many columns): one thread per column sums its
//     P rows in order, eight loads in flight;
//   * tall jobs: a block takes 64 columns with 16 row lanes (one wave per row
//     lane, so each load instruction reads 256 contiguous bytes of a row);
//     row lane r sums rows r, r+16, ... (eight loads in flight), then the 16
//     lane sums are added in order.
struct RedJob {
  const float* part;
  long pstride;
  int P;
  int ncols;
  void* out;
  int blk0;
};
struct RedJobs {
  RedJob j[12];
};
constexpr int RED_SHORT_ROWS = 32;
constexpr int RED_TALL_COLS = 64, RED_TALL_LANES = 16;  // 1024 threads
inline int red_blocks(const RedJob& j) {
  return j.P <= RED_SHORT_ROWS ? (j.ncols + 1023) / 1024 : (j.ncols + RED_TALL_COLS - 1) / RED_TALL_COLS;
}

__device__ __forceinline__ float sum8(const float* p, long stride) {
  float v[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) v[u] = p[(long)u * stride];
  return ((v[0] + v[1]) + (v[2] + v[3])) + ((v[4] + v[5]) + (v[6] + v[7]));
}

template <typename ST>
__global__ __launch_bounds__(1024) void k_finalize(RedJobs jobs) {
  __shared__ float red[RED_TALL_LANES][RED_TALL_COLS + 1];
  int jid = 0;
#pragma unroll
  for (int k = 1; k < 12; ++k)
    if ((int)blockIdx.x >= jobs.j[k].blk0) jid = k;
  const RedJob& job = jobs.j[jid];
  const int b = (int)blockIdx.x - job.blk0;
  if (job.P <= RED_SHORT_ROWS) {
    const long c = (long)b * 1024 + threadIdx.x;
    if (c >= job.ncols) return;
    const float* p = job.part + c;
    float s = 0.f;
    int r = 0;
    for (; r + 8 <= job.P; r += 8) s += sum8(p + (long)r * job.pstride, job.pstride);
    for (; r < job.P; ++r) s += p[(long)r * job.pstride];
    st(reinterpret_cast<ST*>(job.out), c, s);
    return;
  }
  const int cx = threadIdx.x & (RED_TALL_COLS - 1), ry = threadIdx.x / RED_TALL_COLS;
  const long c = (long)b * RED_TALL_COLS + cx;
  float s = 0.f;
  if (c < job.ncols) {
    const float* p = job.part + c;
    constexpr int L = RED_TALL_LANES;
    int r = ry;
    for (; r + 7 * L < job.P; r += 8 * L) s += sum8(p + (long)r * job.pstride, L * job.pstride);
    for (; r < job.P; r += L) s += p[(long)r * job.pstride];
  }
  red[ry][cx] = s;
  __syncthreads();
  if (ry == 0 && c < job.ncols) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < RED_TALL_LANES; ++k) t += red[k][cx];
    st(reinterpret_cast<ST*>(job.out), c, t);
  }
}

// ---------------------------------------------------------------------------
template <typename E>
__global__ __launch_bounds__(256) void k_token_mix(const E* __restrict__ in, E* __restrict__ out, int T, int D) {
  const long row = blockIdx.x;
  const long b = row / T;
  const int i = (int)(row - b * T);
  const int S = D / T;
  for (int c = threadIdx.x; c < D; c += 256) {
    int j, sc;
    tm_source(i, c, S, j, sc);
    out[row * D + c] = in[(b * T + j) * D + sc];
  }
}

template <typename ST>
inline ST* wsp(void* ws, size_t off) {
  return reinterpret_cast<ST*>(reinterpret_cast<char*>(ws) + off);
}

inline unsigned round64(long n) { return (unsigned)((n + 63) / 64 * 64); }

// chunk width of a D-wide row: 4 elements when rows, and (for the token-mix
// gathers) the S-wide runs, are multiples of 4; else 1.
inline bool vec4_rows(const rm_dims& d) { return d.D % 4 == 0 && (d.D / d.T) % 4 == 0; }

template <typename ST>
hipError_t prologue_t(const rm_dims& d, const rm_params& p, const void* x, void* ws, const WsLayout& L,
                      hipStream_t s) {
  prof_begin(KID_PROLOGUE, s);
  if constexpr (sizeof(ST) == 2) {
    if (sample_in_lds(d)) {
      const int tier = lds_tier((long)d.T * d.D * 2);
      auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(d.B), dim3(threads), 0, s, cptr<ST>(x), cptr<ST>(p.ln0_g),
                           cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), cptr<ST>(p.ln1_b), wsp<ST>(ws, L.h1),
                           wsp<float>(ws, L.stats), d.B, d.T, d.D);
      };
      constexpr int T1 = PRO_LDS_BYTES, T2 = PRO_LDS_BYTES / 2, T4 = PRO_LDS_BYTES / 4;
      if (tier == T4) launch(k_prologue_lds<ST, T4>, pro_threads(T4));
      else if (tier == T2) launch(k_prologue_lds<ST, T2>, pro_threads(T2));
      else launch(k_prologue_lds<ST, T1>, pro_threads(T1));
      prof_end(KID_PROLOGUE, s);
      return hipGetLastError();
    }
  }
  if (vec4_rows(d))
    hipLaunchKernelGGL((k_prologue<ST, 4>), dim3(d.B), dim3(512), 0, s, cptr<ST>(x), cptr<ST>(p.ln0_g),
                       cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), cptr<ST>(p.ln1_b), wsp<ST>(ws, L.h1),
                       wsp<float>(ws, L.stats), d.B, d.T, d.D);
  else
    hipLaunchKernelGGL((k_prologue<ST, 1>), dim3(d.B), dim3(512), 0, s, cptr<ST>(x), cptr<ST>(p.ln0_g),
                       cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), cptr<ST>(p.ln1_b), wsp<ST>(ws, L.h1),
                       wsp<float>(ws, L.stats), d.B, d.T, d.D);
  prof_end(KID_PROLOGUE, s);
  return hipGetLastError();
}

template <typename ST, int N, int Q>
void gate_fwd_launch(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  const long NR = (long)d.B * d.T;
  hipLaunchKernelGGL((k_gate_fwd<ST, N, Q>), dim3((unsigned)((NR + 3) / 4)), dim3(256), 0, s, wsp<ST>(ws, L.z),
                     cptr<ST>(p.lnx_g), cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g), cptr<ST>(p.lng_b), wsp<ST>(ws, L.hid),
                     wsp<float>(ws, L.stats), NR, d.k * d.D);
}

template <typename ST>
hipError_t gate_fwd_t(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  const int H = d.k * d.D;
  constexpr int NV = 16 / sizeof(ST);
  prof_begin(KID_GATE_FWD, s);
  if (H % NV == 0) {
    // the smallest instantiated lane-chunk count covering H
    const int q = (H + 64 * NV - 1) / (64 * NV);
    if (q <= 1) gate_fwd_launch<ST, NV, 1>(d, p, ws, L, s);
    else if (q <= 2) gate_fwd_launch<ST, NV, 2>(d, p, ws, L, s);
    else if (q <= 3) gate_fwd_launch<ST, NV, 3>(d, p, ws, L, s);
    else if (q <= 4) gate_fwd_launch<ST, NV, 4>(d, p, ws, L, s);
    else if (q <= 5) gate_fwd_launch<ST, NV, 5>(d, p, ws, L, s);
    else if (q <= 6) gate_fwd_launch<ST, NV, 6>(d, p, ws, L, s);
    else if (q <= 8) gate_fwd_launch<ST, NV, 8>(d, p, ws, L, s);
    else if (q <= 12) gate_fwd_launch<ST, NV, 12>(d, p, ws, L, s);
    else gate_fwd_launch<ST, NV, 15>(d, p, ws, L, s);
  } else {
    gate_fwd_launch<ST, 1, (MAXH + 63) / 64>(d, p, ws, L, s);
  }
  prof_end(KID_GATE_FWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t ln2_fwd_t(const rm_dims& d, const rm_params& p, void* y, void* ws, const WsLayout& L, hipStream_t s) {
  const long NR = (long)d.B * d.T;
  // persistent: as many four-wave blocks as stay resident
  const int rb = d.D % 4 == 0 ? resident_blocks<k_ln2_fwd<ST, 4>>(256) : resident_blocks<k_ln2_fwd<ST, 1>>(256);
  const dim3 grid((unsigned)std::min<long>((NR + 3) / 4, (long)rb * device_cu_count()));
  prof_begin(KID_LN2_FWD, s);
  if (d.D % 4 == 0)
    hipLaunchKernelGGL((k_ln2_fwd<ST, 4>), grid, dim3(256), 0, s, wsp<ST>(ws, L.r2), cptr<ST>(p.ln2_g),
                       cptr<ST>(p.ln2_b), reinterpret_cast<ST*>(y), wsp<float>(ws, L.stats), NR, d.D);
  else
    hipLaunchKernelGGL((k_ln2_fwd<ST, 1>), grid, dim3(256), 0, s, wsp<ST>(ws, L.r2), cptr<ST>(p.ln2_g),
                       cptr<ST>(p.ln2_b), reinterpret_cast<ST*>(y), wsp<float>(ws, L.stats), NR, d.D);
  prof_end(KID_LN2_FWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t ln2_bwd_t(const rm_dims& d, const rm_params& p, const void* dy, void* ws, void* sc, const WsLayout& L,
                     hipStream_t s) {
  const dim3 grid(d.T, L.nb);
  prof_begin(KID_LN2_BWD, s);
  if (d.D % 4 == 0)
    hipLaunchKernelGGL((k_ln2_bwd<ST, 4, MAXD / 256>), grid, dim3(256), 0, s, wsp<ST>(ws, L.r2), cptr<ST>(dy),
                       cptr<ST>(p.ln2_g), wsp<float>(ws, L.stats), wsp<ST>(sc, L.do2), wsp<float>(sc, L.p_ln2), d.B,
                       d.T, d.D, L.nb, L.rpg);
  else
    hipLaunchKernelGGL((k_ln2_bwd<ST, 1, MAXD / 64>), grid, dim3(256), 0, s, wsp<ST>(ws, L.r2), cptr<ST>(dy),
                       cptr<ST>(p.ln2_g), wsp<float>(ws, L.stats), wsp<ST>(sc, L.do2), wsp<float>(sc, L.p_ln2), d.B,
                       d.T, d.D, L.nb, L.rpg);
  prof_end(KID_LN2_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t gate_bwd_t(const rm_dims& d, const rm_params& p, void* ws, void* sc, const WsLayout& L, hipStream_t s) {
  const int H = d.k * d.D;
  constexpr int NV = 16 / sizeof(ST);
  float* pg = wsp<float>(sc, L.p_gate);
  float* pb1 = pg + 4L * L.nb * d.T * H;
  const dim3 grid(d.T, L.nb);
  prof_begin(KID_GATE_BWD, s);
  // 8-byte chunks (4 elements) keep the per-thread partial sums small
  // one workgroup of H/4 threads per row group (up to 640: 10 waves, room for the prefetch ring)
  if (H % 4 == 0 && H <= 2560 && 2L * d.B * d.T * H * (long)sizeof(ST) <= 0x7fffffffL)
  {
    auto ring = [&](auto kernel) {
      hipLaunchKernelGGL(kernel, grid, dim3(round64(H / 4)), 0, s, wsp<ST>(ws, L.z), wsp<ST>(sc, L.dhid),
                         cptr<ST>(p.lnx_g), cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g), cptr<ST>(p.lng_b),
                         wsp<float>(ws, L.stats), wsp<ST>(sc, L.dz), pg, pb1, d.B, d.T, H, L.nb);
    };
    static_assert(MIN_ROWS_PER_GROUP == 16 && MAX_ROWS_PER_GROUP == 128, "one instantiation per group size");
    if (L.rpg == 16) ring(k_gate_bwd_ring<ST, 640, 16>);
    else if (L.rpg == 32) ring(k_gate_bwd_ring<ST, 640, 32>);
    else if (L.rpg == 64) ring(k_gate_bwd_ring<ST, 640, 64>);
    else ring(k_gate_bwd_ring<ST, 640, 128>);
  }
  else if (H % 4 == 0)
    hipLaunchKernelGGL((k_gate_bwd<ST, 4, 1, 1024, 2>), grid, dim3(round64(H / 4)), 0, s, wsp<ST>(ws, L.z),
                       wsp<ST>(sc, L.dhid), cptr<ST>(p.lnx_g), cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g),
                       cptr<ST>(p.lng_b), wsp<float>(ws, L.stats), wsp<ST>(sc, L.dz), pg, pb1, d.B, d.T, H, L.nb, L.rpg);
  else
    hipLaunchKernelGGL((k_gate_bwd<ST, 1, 8, 512, 1>), grid, dim3(round64((H + 7) / 8)), 0, s, wsp<ST>(ws, L.z),
                       wsp<ST>(sc, L.dhid), cptr<ST>(p.lnx_g), cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g),
                       cptr<ST>(p.lng_b), wsp<float>(ws, L.stats), wsp<ST>(sc, L.dz), pg, pb1, d.B, d.T, H, L.nb, L.rpg);
  prof_end(KID_GATE_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t tail_bwd_t(const rm_dims& d, const rm_params& p, const void* x, void* dx, void* ws, void* sc,
                      const WsLayout& L,
                      hipStream_t s) {
  const dim3 grid(d.T, L.nb);
  hipError_t e;
  if constexpr (sizeof(ST) == 2) {
    if (sample_in_lds(d)) {
      prof_begin(KID_TAIL_BWD, s);
      const int tier = lds_tier((long)d.T * d.D * 2);
      auto launch = [&](auto kernel, int threads) {
        hipLaunchKernelGGL(kernel, dim3(d.B), dim3(threads), 0, s, cptr<ST>(x), wsp<ST>(sc, L.dh1),
                           cptr<ST>(p.ln0_g), cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), wsp<float>(ws, L.stats),
                           reinterpret_cast<ST*>(dx), wsp<float>(sc, L.p_tail), d.B, d.T, d.D);
      };
      constexpr int T1 = PRO_LDS_BYTES, T2 = PRO_LDS_BYTES / 2, T4 = PRO_LDS_BYTES / 4;
      if (tier == T4) launch(k_tail_bwd_lds<ST, T4>, tail_threads(T4));
      else if (tier == T2) launch(k_tail_bwd_lds<ST, T2>, tail_threads(T2));
      else launch(k_tail_bwd_lds<ST, T1>, tail_threads(T1));
      prof_end(KID_TAIL_BWD, s);
      return hipGetLastError();
    }
  }
  prof_begin(KID_LN1_BWD, s);
  if (vec4_rows(d))
    hipLaunchKernelGGL((k_ln1_bwd<ST, 4, MAXD / 256>), grid, dim3(256), 0, s, cptr<ST>(x), wsp<ST>(sc, L.dh1),
                       cptr<ST>(p.ln0_g), cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), wsp<float>(ws, L.stats),
                       wsp<ST>(sc, L.dr1), wsp<float>(sc, L.p_tail), d.B, d.T, d.D, L.nb, L.rpg);
  else
    hipLaunchKernelGGL((k_ln1_bwd<ST, 1, MAXD / 64>), grid, dim3(256), 0, s, cptr<ST>(x), wsp<ST>(sc, L.dh1),
                       cptr<ST>(p.ln0_g), cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), wsp<float>(ws, L.stats),
                       wsp<ST>(sc, L.dr1), wsp<float>(sc, L.p_tail), d.B, d.T, d.D, L.nb, L.rpg);
  prof_end(KID_LN1_BWD, s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  prof_begin(KID_LN0_BWD, s);
  if (vec4_rows(d))
    hipLaunchKernelGGL((k_ln0_bwd<ST, 4, MAXD / 256>), grid, dim3(256), 0, s, cptr<ST>(x), wsp<ST>(sc, L.dr1),
                       cptr<ST>(p.ln0_g), wsp<float>(ws, L.stats), reinterpret_cast<ST*>(dx),
                       wsp<float>(sc, L.p_tail), d.B, d.T, d.D, L.nb, L.rpg);
  else
    hipLaunchKernelGGL((k_ln0_bwd<ST, 1, MAXD / 64>), grid, dim3(256), 0, s, cptr<ST>(x), wsp<ST>(sc, L.dr1),
                       cptr<ST>(p.ln0_g), wsp<float>(ws, L.stats), reinterpret_cast<ST*>(dx),
                       wsp<float>(sc, L.p_tail), d.B, d.T, d.D, L.nb, L.rpg);
  prof_end(KID_LN0_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t finalize_t(const rm_dims& d, const rm_grads& g, void* sc, const WsLayout& L, hipStream_t s) {
  const int T = d.T, D = d.D, H = d.k * d.D, nb = L.nb;
  const float* pl = wsp<float>(sc, L.p_ln2);
  const float* pg = wsp<float>(sc, L.p_gate);
  const float* pt = wsp<float>(sc, L.p_tail);
  const long bl = (long)nb * T * D, bg = (long)nb * T * H;
  RedJobs J;
  J.j[0] = {pl + 0 * bl, D, nb * T, D, g.ln2_g, 0};
  J.j[1] = {pl + 1 * bl, D, nb * T, D, g.ln2_b, 0};
  J.j[2] = {pl + 2 * bl, (long)T * D, nb, T * D, g.bout, 0};
  J.j[3] = {pg + 0 * bg, H, nb * T, H, g.lnx_g, 0};
  J.j[4] = {pg + 1 * bg, H, nb * T, H, g.lnx_b, 0};
  J.j[5] = {pg + 2 * bg, H, nb * T, H, g.lng_g, 0};
  J.j[6] = {pg + 3 * bg, H, nb * T, H, g.lng_b, 0};
  J.j[7] = {pg + 4 * bg, (long)T * 2 * H, nb, T * 2 * H, g.b1, 0};
  // tail partials: [4][row groups * T][D], or [4][B][D] when the tail ran one sample per workgroup
  const int pt_rows = sample_in_lds(d) ? d.B : nb * T;
  const long bt = (long)pt_rows * D;
  J.j[8] = {pt + 0 * bt, D, pt_rows, D, g.ln0_g, 0};
  J.j[9] = {pt + 1 * bt, D, pt_rows, D, g.ln0_b, 0};
  J.j[10] = {pt + 2 * bt, D, pt_rows, D, g.ln1_g, 0};
  J.j[11] = {pt + 3 * bt, D, pt_rows, D, g.ln1_b, 0};
  int nblk = 0;
  for (RedJob& j : J.j) {
    j.blk0 = nblk;
    nblk += red_blocks(j);
  }
  prof_begin(KID_FINALIZE, s);
  hipLaunchKernelGGL(k_finalize<ST>, dim3(nblk), dim3(1024), 0, s, J);
  prof_end(KID_FINALIZE, s);
  return hipGetLastError();
}

}  // namespace

#define RM_DISPATCH(fn, ...) \
  ((d.dtype == RM_BF16) ? fn<bf16_t>(__VA_ARGS__) : (d.dtype == RM_F16) ? fn<f16_t>(__VA_ARGS__) : fn<float>(__VA_ARGS__))

hipError_t launch_prologue(const rm_dims& d, const rm_params& p, const void* x, void* ws, const WsLayout& L,
                           hipStream_t s) {
  return RM_DISPATCH(prologue_t, d, p, x, ws, L, s);
}
hipError_t launch_gate_fwd(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(gate_fwd_t, d, p, ws, L, s);
}
hipError_t launch_ln2_fwd(const rm_dims& d, const rm_params& p, void* y, void* ws, const WsLayout& L,
                          hipStream_t s) {
  return RM_DISPATCH(ln2_fwd_t, d, p, y, ws, L, s);
}
hipError_t launch_ln2_bwd(const rm_dims& d, const rm_params& p, const void* dy, void* ws, void* sc, const WsLayout& L,
                          hipStream_t s) {
  return RM_DISPATCH(ln2_bwd_t, d, p, dy, ws, sc, L, s);
}
hipError_t launch_gate_bwd(const rm_dims& d, const rm_params& p, void* ws, void* sc, const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(gate_bwd_t, d, p, ws, sc, L, s);
}
hipError_t launch_tail_bwd(const rm_dims& d, const rm_params& p, const void* x, void* dx, void* ws, void* sc,
                           const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(tail_bwd_t, d, p, x, dx, ws, sc, L, s);
}
hipError_t launch_finalize(const rm_dims& d, const rm_grads& g, void* sc, const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(finalize_t, d, g, sc, L, s);
}
hipError_t launch_token_mix(const rm_dims& d, const void* in, void* out, hipStream_t s) {
  const long rows = (long)d.B * d.T;
  prof_begin(KID_TOKEN_MIX, s);
  if (d.dtype != RM_F32)
    hipLaunchKernelGGL(k_token_mix<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(in), reinterpret_cast<uint16_t*>(out), d.T, d.D);
  else
    hipLaunchKernelGGL(k_token_mix<uint32_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(in), reinterpret_cast<uint32_t*>(out), d.T, d.D);
  prof_end(KID_TOKEN_MIX, s);
  return hipGetLastError();
}

}  // namespace rm
