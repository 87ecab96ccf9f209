// bf16 T-batched GEMM with 256x256 workgroup tiles for gfx950 (CDNA4).
//
// Same contract as the general kernel (GemmArgs; page 1 of "Subgraph-fusion-
// based Mega-kernel Generation", section "Exact computation": one independent
// GEMM per token t), for the common case K % 64 == 0 with 16-byte aligned,
// 8-element-multiple rows.
//
//   * 4 waves (2 x 2), each owning a 128 x 128 output tile: 4 x 4 MFMA
//     v_mfma_f32_32x32x16_bf16 tiles, 256 fp32 accumulators per lane (AGPRs,
//     one wave per SIMD).  Per 16-deep k step a wave reads 8 KB of operand
//     fragments from LDS for 16 MFMAs (64 bytes of LDS per clock per CU at
//     full MFMA rate).
//   * Operand slabs (64 deep in K) are copied global -> LDS with the gfx950
//     16-byte direct loads (no register staging), double buffered: the copy of
//     slab k+1 is issued before the MFMAs of slab k and awaited at the one
//     barrier per slab.  The two stages are separate LDS objects named
//     directly (the K loop is unrolled by two), which lets the compiler see
//     that the copies cannot alias the fragment reads of the other stage.
//   * K-major operands (row = m or n, 128 contiguous bytes of K) live in LDS
//     as 128-byte rows whose 16-byte chunks are XOR-swizzled by (row/2)%8; an
//     MFMA fragment is one 16-byte read per lane.
//   * M/N-major operands (the forward weights and both weight-gradient
//     operands) live in LDS as 64 rows of k, each 256 contiguous m/n values
//     (512 bytes, 16-byte chunks XOR-swizzled by 4*(k%4), so the 4 k-rows x
//     4 chunks one half-wave reads cover all 64 banks); a fragment is built by
//     two ds_read_b64_tr_b16 transposing reads (in each 16-lane group, lane j
//     names row kbase + j/4, columns nbase + 4*(j%4); lane i receives column
//     nbase + i for four consecutive k).  No transposed copy of any operand is
//     ever made.
//   * Rows past M or N are loaded from a clamped valid address and their
//     results discarded; K must be a multiple of 128.
#include "rm_common.h"
#include "rm_internal.h"

#include <type_traits>

namespace rm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));

constexpr int BM = 256, BN = 256, BK = 32;
constexpr int STAGES = 4;
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand slab: 256 x 32 bf16 = 16 KB
typedef __attribute__((address_space(3))) short4_t lds_short4;
typedef __attribute__((address_space(3))) void lds_void;

// K-major slab: 256 rows x 64 bytes (4 chunks of 16 B); chunk swizzled by (row/4)%4
// so the 16 rows of a fragment read hit 16 distinct 4-bank groups.
__device__ __forceinline__ int kswz(int row, int chunk) { return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4); }
// M/N-major slab: 32 k-rows x 512 bytes (32 chunks); chunk swizzled by 4*(k%4).
__device__ __forceinline__ int mswz(int krow, int chunk) { return krow * 512 + ((chunk ^ ((krow & 3) << 2)) << 4); }

// Loop-invariant element offsets of this thread's four 16-byte pieces of a
// slab (32-bit: every operand here is far below 2^31 elements).  Instruction
// i of wave w writes 1 KB of LDS: K-major rows 64w + 16i .. +15 (lane l ->
// row +l/4, physical chunk l%4), M/N-major k-rows 8w + 2i, +1 (lane l -> k-row
// +l/32, physical chunk l%32); each lane fetches the logical chunk that the
// swizzle places there.
template <bool KMAJ>
__device__ __forceinline__ void slab_offsets(uint32_t (&off)[4], long ld, int mn0, int MN, int wave, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (KMAJ) {
      const int row = 64 * wave + 16 * i + (lane >> 2);
      const int chunk = (lane & 3) ^ ((row >> 2) & 3);
      const int mn = min(mn0 + row, MN - 1);
      off[i] = (uint32_t)((long)mn * ld + chunk * 8);
    } else {
      const int krow = 8 * wave + 2 * i + (lane >> 5);
      const int chunk = (lane & 31) ^ ((krow & 3) << 2);
      const int mn = min(mn0 + chunk * 8, MN - 8);
      off[i] = (uint32_t)((long)krow * ld + mn);
    }
  }
}

// One 16-byte direct global -> LDS load per lane: lane l's bytes land at
// LDS address lds + 16*l.  Issued through inline assembly so that the
// compiler's own wait-count bookkeeping ignores it; the pipeline below waits
// for these loads explicitly (vm_barrier) before any LDS read of their data,
// and no other vector-memory instruction is in flight meanwhile.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds_addr) {
  asm volatile("s_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(gptr), "s"(lds_addr) : "memory", "m0");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  // low 32 bits of a flat pointer into the LDS aperture are the LDS address
  return __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(p));
}

// Copy the slab starting at k0 into LDS with 16-byte direct loads.
template <bool KMAJ>
__device__ __forceinline__ void dma_slab(char* lds, const bf16_t* __restrict__ base, const uint32_t (&off)[4], long ld,
                                         int k0, int wave) {
  const bf16_t* b = base + (KMAJ ? (long)k0 : (long)k0 * ld);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int dst = KMAJ ? (64 * wave + 16 * i) * 64 : (8 * wave + 2 * i) * 512;
    dma16(b + off[i], lds_addr(lds + dst));
  }
}

// MFMA fragment (32 rows of m or n, 16 of k at k-step ks) for this lane.
template <bool KMAJ>
__device__ __forceinline__ bf16x8_t read_frag(const char* lds, int row0, int ks, int lane) {
  if constexpr (KMAJ) {
    const int row = row0 + (lane & 31);
    const int chunk = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const bf16x8_t*>(lds + kswz(row, chunk));
  } else {
    const int g = lane >> 4, li = lane & 15;
    const int krow = 16 * ks + 8 * (g >> 1) + (li >> 2);
    const int col = row0 + 16 * (g & 1) + 4 * (li & 3);
    const int off0 = mswz(krow, col >> 3) + (col & 7) * 2;
    const int off1 = mswz(krow + 4, col >> 3) + (col & 7) * 2;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off0));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off1));
    const short8_t v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_bit_cast(bf16x8_t, v);
  }
}

template <bool AK, bool BKM>
__device__ __forceinline__ void read_frags(bf16x8_t (&a)[4], bf16x8_t (&b)[4], const char* a_s, const char* b_s,
                                           int wm, int wn, int ks, int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = read_frag<AK>(a_s, wm * 128 + 32 * i, ks, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) b[j] = read_frag<BKM>(b_s, wn * 128 + 32 * j, ks, lane);
}

// MFMAs over one 32-deep slab (2 k steps x 16 MFMAs).  The fragments of the
// second step are read while the MFMAs of the first issue (one MFMA, one LDS
// read, alternately).
template <bool AK, bool BKM>
__device__ __forceinline__ void slab_mfma(f32x16_t (&acc)[4][4], const char* a_s, const char* b_s, int wm, int wn,
                                          int lane) {
  constexpr int NREAD = (AK ? 4 : 8) + (BKM ? 4 : 8);
  bf16x8_t a0[4], b0[4], a1[4], b1[4];
  read_frags<AK, BKM>(a0, b0, a_s, b_s, wm, wn, 0, lane);
  read_frags<AK, BKM>(a1, b1, a_s, b_s, wm, wn, 1, lane);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0[i], b0[j], acc[i][j], 0, 0, 0);
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1[i], b1[j], acc[i][j], 0, 0, 0);
}

// Wait until at most N of this wave's direct loads are outstanding (gfx9
// s_waitcnt encoding: vmcnt in bits 3:0 and 15:14; expcnt and lgkmcnt left
// at their maxima), then a workgroup barrier.  After it, every wave's copies
// older than the newest N are in LDS.
template <int N>
__device__ __forceinline__ void vm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Directly-loaded copies per slab per wave (A and B pieces).
constexpr int DMA_PER_SLAB = 8;

// One pipeline step: slab k sits in stage s (LDS objects sa, sb); wait for
// it, then start the copy of slab k + 3 into the stage read one step ago
// (sa3, sb3), then run its MFMAs.
template <bool AK, bool BKM>
__device__ __forceinline__ void pipe_step(f32x16_t (&acc)[4][4], const char* sa, const char* sb, char* sa3, char* sb3,
                                          int k, int nk, const bf16_t* A, const bf16_t* B, const GemmArgs& g,
                                          const uint32_t (&offa)[4], const uint32_t (&offb)[4], int wm, int wn,
                                          int wave, int lane) {
  // copies still allowed in flight: those of slabs k+1 and k+2 that exist
  if (k + 2 < nk) vm_barrier<2 * DMA_PER_SLAB>();
  else if (k + 1 < nk) vm_barrier<DMA_PER_SLAB>();
  else vm_barrier<0>();
  if (k + 3 < nk) {
    dma_slab<AK>(sa3, A, offa, g.a_ld, (k + 3) * BK, wave);
    dma_slab<BKM>(sb3, B, offb, g.b_ld, (k + 3) * BK, wave);
  }
  __builtin_amdgcn_sched_barrier(0);
  slab_mfma<AK, BKM>(acc, sa, sb, wm, wn, lane);
}

template <bool AK, bool BKM>
__global__ __launch_bounds__(256, 1) void k_gemm256(GemmArgs g) {
  // four stages, each in LDS objects of their own that are always named
  // directly (the k loop is unrolled by four), so the compiler can tell which
  // direct loads feed which fragment reads
  // stage s = one LDS object holding the A slab then the B slab
  __shared__ __attribute__((aligned(1024))) char s0[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s1[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s2[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char s3[2 * TILE_BYTES];
  char* const a0 = s0;
  char* const b0 = s0 + TILE_BYTES;
  char* const a1 = s1;
  char* const b1 = s1 + TILE_BYTES;
  char* const a2 = s2;
  char* const b2 = s2 + TILE_BYTES;
  char* const a3 = s3;
  char* const b3 = s3 + TILE_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile numbering (workgroup w runs on XCD w % 8): each XCD gets a
  // contiguous range of logical tiles, token-major, then N tile, then M tile.
  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int total = tiles_m * tiles_n * g.batch;
  const int w = blockIdx.x;
  const int xcd = w & 7, q = total >> 3, rem = total & 7;
  const int logical = xcd * q + min(xcd, rem) + (w >> 3);
  const int per_t = tiles_m * tiles_n;
  const int t = logical / per_t;
  const int in_t = logical - t * per_t;
  const int tn = in_t / tiles_m, tm = in_t - tn * tiles_m;
  const int m0 = tm * BM, n0 = tn * BN;

  const bf16_t* A = reinterpret_cast<const bf16_t*>(g.A) + (long)t * g.a_bs;
  const bf16_t* B = reinterpret_cast<const bf16_t*>(g.B) + (long)t * g.b_bs;

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  uint32_t offa[4], offb[4];
  slab_offsets<AK>(offa, g.a_ld, m0, g.M, wave, lane);
  slab_offsets<BKM>(offb, g.b_ld, n0, g.N, wave, lane);
  const int nk = g.K / BK;  // a multiple of 4: K % 128 == 0
  dma_slab<AK>(a0, A, offa, g.a_ld, 0, wave);
  dma_slab<BKM>(b0, B, offb, g.b_ld, 0, wave);
  dma_slab<AK>(a1, A, offa, g.a_ld, BK, wave);
  dma_slab<BKM>(b1, B, offb, g.b_ld, BK, wave);
  dma_slab<AK>(a2, A, offa, g.a_ld, 2 * BK, wave);
  dma_slab<BKM>(b2, B, offb, g.b_ld, 2 * BK, wave);
  for (int k = 0; k < nk; k += 4) {
    pipe_step<AK, BKM>(acc, a0, b0, a3, b3, k, nk, A, B, g, offa, offb, wm, wn, wave, lane);
    pipe_step<AK, BKM>(acc, a1, b1, a0, b0, k + 1, nk, A, B, g, offa, offb, wm, wn, wave, lane);
    pipe_step<AK, BKM>(acc, a2, b2, a1, b1, k + 2, nk, A, B, g, offa, offb, wm, wn, wave, lane);
    pipe_step<AK, BKM>(acc, a3, b3, a2, b2, k + 3, nk, A, B, g, offa, offb, wm, wn, wave, lane);
  }

  // ---- epilogue ------------------------------------------------------
  // Each wave stages its 128 x 128 tile through its own LDS area 32 rows at a
  // time (fp32, rows padded to 136 floats so the two half-waves of an MFMA
  // output write land in disjoint banks), then writes whole 256-byte row
  // segments with 16-byte vector stores, adding bias[t] and the residual.
  // MFMA 32x32 output layout: element v of lane l is (row 8*(v/4) + 4*(l/32) + v%4, column l%32).
  __syncthreads();  // every wave is done reading the operand stages
  constexpr int PITCH = 136;
  float* stage = reinterpret_cast<float*>(wave == 0 ? s0 : wave == 1 ? s1 : wave == 2 ? s2 : s3);
  const int r32 = lane & 31, hl = lane >> 5;
  const bf16_t* bias = reinterpret_cast<const bf16_t*>(g.bias);
  float bv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int col = min(n0 + wn * 128 + 32 * j + r32, g.N - 1);
    bv[j] = bias ? to_f32(bias[(long)t * g.bias_bs + col]) : 0.f;
  }
  const int rsub = lane >> 4;        // write phase: 4 rows per pass
  const int csub = (lane & 15) * 8;  // 8 consecutive columns per lane
  const int col0 = n0 + wn * 128 + csub;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rr = 8 * (v >> 2) + 4 * hl + (v & 3);
        stage[rr * PITCH + 32 * j + r32] = acc[i][j][v] + bv[j];
      }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's staging writes are in LDS
#pragma unroll
    for (int pass = 0; pass < 8; ++pass) {
      const int rr = 4 * pass + rsub;
      const int row = m0 + wm * 128 + 32 * i + rr;
      float vals[8];
      const float4 lo = *reinterpret_cast<const float4*>(stage + rr * PITCH + csub);
      const float4 hi = *reinterpret_cast<const float4*>(stage + rr * PITCH + csub + 4);
      vals[0] = lo.x; vals[1] = lo.y; vals[2] = lo.z; vals[3] = lo.w;
      vals[4] = hi.x; vals[5] = hi.y; vals[6] = hi.z; vals[7] = hi.w;
      if (row < g.M && col0 < g.N) {
        if (g.res) {
          const long ri = (long)t * g.res_bs + (long)row * g.res_ld + col0;
          if (g.res_f32) {
            const float4 a = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.res) + ri);
            const float4 b = *reinterpret_cast<const float4*>(reinterpret_cast<const float*>(g.res) + ri + 4);
            vals[0] += a.x; vals[1] += a.y; vals[2] += a.z; vals[3] += a.w;
            vals[4] += b.x; vals[5] += b.y; vals[6] += b.z; vals[7] += b.w;
          } else {
            const uint4 a = *reinterpret_cast<const uint4*>(reinterpret_cast<const bf16_t*>(g.res) + ri);
            const uint32_t w4[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              vals[2 * e] += __uint_as_float(w4[e] << 16);
              vals[2 * e + 1] += __uint_as_float(w4[e] & 0xffff0000u);
            }
          }
        }
        const long o = (long)t * g.c_bs + (long)row * g.c_ld + col0;
        if (g.c_f32) {
          float* c = reinterpret_cast<float*>(g.C) + o;
          *reinterpret_cast<float4*>(c) = make_float4(vals[0], vals[1], vals[2], vals[3]);
          *reinterpret_cast<float4*>(c + 4) = make_float4(vals[4], vals[5], vals[6], vals[7]);
        } else {
          uint4 pk;
          pk.x = (uint32_t)f32_to_bf16_bits(vals[0]) | ((uint32_t)f32_to_bf16_bits(vals[1]) << 16);
          pk.y = (uint32_t)f32_to_bf16_bits(vals[2]) | ((uint32_t)f32_to_bf16_bits(vals[3]) << 16);
          pk.z = (uint32_t)f32_to_bf16_bits(vals[4]) | ((uint32_t)f32_to_bf16_bits(vals[5]) << 16);
          pk.w = (uint32_t)f32_to_bf16_bits(vals[6]) | ((uint32_t)f32_to_bf16_bits(vals[7]) << 16);
          *reinterpret_cast<uint4*>(reinterpret_cast<bf16_t*>(g.C) + o) = pk;
        }
      }
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // staging reads done before the next block overwrites it
  }
}

template <bool AK, bool BKM>
hipError_t run256(const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.batch;
  hipLaunchKernelGGL((k_gemm256<AK, BKM>), dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

bool gemm256_supported(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g) {
  if (dtype != RM_BF16) return false;
  if (a_kmajor == false && b_kmajor == true) return false;
  if (g.K % (STAGES * BK) != 0) return false;
  const long a_cont = a_kmajor ? g.K : g.M, b_cont = b_kmajor ? g.K : g.N;
  if (a_cont % 8 || b_cont % 8 || g.a_ld % 8 || g.b_ld % 8 || g.a_bs % 8 || g.b_bs % 8) return false;
  if ((reinterpret_cast<uintptr_t>(g.A) & 15) || (reinterpret_cast<uintptr_t>(g.B) & 15)) return false;
  if (!a_kmajor && g.M < 8) return false;
  if (!b_kmajor && g.N < 8) return false;
  // the epilogue writes 8-column vectors
  if (g.N % 8 || g.c_ld % 8 || g.c_bs % 8 || (reinterpret_cast<uintptr_t>(g.C) & 15)) return false;
  if (g.res && (g.res_ld % 8 || g.res_bs % 8 || (reinterpret_cast<uintptr_t>(g.res) & 15))) return false;
  return true;
}

hipError_t launch_gemm256(bool a_kmajor, bool b_kmajor, const GemmArgs& g, hipStream_t s) {
  if (a_kmajor && !b_kmajor) return run256<true, false>(g, s);
  if (a_kmajor && b_kmajor) return run256<true, true>(g, s);
  return run256<false, false>(g, s);
}

}  // namespace rm
