// bf16 / fp16 T-batched GEMM with 256x256 workgroup tiles for gfx950 (CDNA4).
//
// Same contract as the general kernel (GemmArgs; page 1 of "Subgraph-fusion-
// based Mega-kernel Generation", section "Exact computation": one independent
// GEMM per token t), for the common case K % 128 == 0, K >= 256, with 16-byte
// aligned, 8-element-multiple rows.
//
//   * 4 waves (2 x 2), each owning a 128 x 128 output tile: 4 x 4 MFMA
//     v_mfma_f32_32x32x16_bf16 (or _f16) tiles, 256 fp32 accumulators per lane (AGPRs,
//     one wave per SIMD).  Per 16-deep k step a wave reads 8 KB of operand
//     fragments from LDS for 16 MFMAs (64 bytes of LDS per clock per CU at
//     full MFMA rate).
//   * Operand slabs (64 deep in K, 32 KB per operand) are copied global ->
//     LDS with the gfx950 16-byte buffer loads that write LDS directly (no
//     register staging): A through a ring of two stages, B through a ring of
//     three, so two B slabs and one A slab are in flight while a slab is
//     multiplied (the whole 160 KB of LDS).  Each copy goes through a buffer
//     resource that spans exactly the token's operand from the slab's first
//     element on, so an address outside it reads zero instead of faulting.
//     The copies are inline assembly with explicit wait counts, so the
//     compiler neither waits for them at every LDS read nor reorders them.
//   * One barrier per slab, before its last k step: the fragments of k steps
//     2..4 are read during the MFMAs of the step before, then the barrier
//     (next slab landed, this slab fully read); A slab k+2 is copied into the
//     stage just freed between the last k step's MFMAs, B slab k+3 at the
//     starts of the next slab's first three k steps, and the next slab's
//     first fragments are read during the last k step's MFMAs, so every
//     fragment read is issued a k step before its MFMAs.
//   * Persistent: one workgroup per CU walks a range of tiles; the copy
//     stream continues into the next tile, and a tile's results go through
//     LDS (freed operand stages) to whole-cache-line stores while the next
//     tile's copies land.  The bias is the accumulators' starting value (a
//     rank-1 MFMA); a residual is copied into LDS like an operand slab.
//   * K-major operands (row = m or n, 128 contiguous bytes of K: one whole
//     cache line per row and slab) live in LDS as 128-byte rows whose 16-byte
//     chunks are XOR-swizzled by (row/2)%8; an MFMA fragment is one 16-byte
//     read per lane.
//   * M/N-major operands (the forward weights and both weight-gradient
//     operands) live in LDS as 64 rows of k, each 256 contiguous m/n values
//     (512 bytes, 16-byte chunks XOR-swizzled by 4*(k%4), so the 4 k-rows x
//     4 chunks one half-wave reads cover all 64 banks); a fragment is built by
//     two ds_read_b64_tr_b16 transposing reads (in each 16-lane group, lane j
//     names row kbase + j/4, columns nbase + 4*(j%4); lane i receives column
//     nbase + i for four consecutive k).  No transposed copy of any operand is
//     ever made.
//   * Rows past M or N are loaded from a clamped valid address and their
//     results dropped at the store.
#include <atomic>
#include <type_traits>

#include "rm_common.h"
#include "rm_internal.h"

namespace rm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef short short4_t __attribute__((ext_vector_type(4)));
typedef short short8_t __attribute__((ext_vector_type(8)));
typedef uint32_t v2u32 __attribute__((ext_vector_type(2)));
typedef uint32_t v4u32 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) short4_t lds_short4;

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand slab: 256 x 64 bf16 = 32 KB
constexpr int KSTEPS = BK / 16;           // MFMA k steps per slab
// Buffer stores the epilogue issues per tile per wave at least (32 for bf16
// output, 64 for fp32), unconditionally (lanes outside C get an out-of-range
// offset, which the buffer unit drops).
constexpr int EPI_STORES = 32;

// Two fp32 values as a packed pair of the 16-bit storage type ST, round to
// nearest even (one v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32).
template <typename ST>
__device__ __forceinline__ uint32_t pair16(float a, float b) {
  return pack16x2<ST>(a, b);
}

// K-major slab: 256 rows x 128 bytes (8 chunks of 16 B, one cache line per
// row); chunk swizzled by (row/2)%8.  A 16-byte read serves 16 lanes (16
// consecutive rows, one chunk) per LDS cycle: rows 2r and 2r+1 fall in the two
// 128-byte halves of the 256-byte bank space and the swizzle gives the 8 row
// pairs 8 distinct chunks, so the 16 reads hit 16 distinct 4-bank groups.
__device__ __forceinline__ int kswz(int row, int chunk) { return row * 128 + ((chunk ^ ((row >> 1) & 7)) << 4); }
// M/N-major slab: 64 k-rows x 512 bytes (32 chunks); chunk swizzled by 4*(k%4).
__device__ __forceinline__ int mswz(int krow, int chunk) { return krow * 512 + ((chunk ^ ((krow & 3) << 2)) << 4); }

// Loop-invariant byte offsets of this thread's eight 16-byte pieces of a
// slab (32-bit: every operand here spans far less than 4 GB per token).
// Instruction i of wave w writes 1 KB of LDS: K-major rows 64w + 8i .. +7,
// whole 128-byte lines (lane l -> row +l/8, physical chunk l%8), M/N-major
// k-rows 16w + 2i, +1 (lane l -> k-row +l/32, physical chunk l%32); each lane
// fetches the logical chunk that the swizzle places there.
constexpr int DMA_PER_OPERAND = 8;
// B pieces of a slab issued in the last k step of the step that frees its
// stage; the other pieces follow, spread over the starts of the next step's
// first three k steps, so that no k step issues more than 10 copies per wave.
constexpr int B_LATE = 0;
static_assert(B_LATE >= 0 && B_LATE <= DMA_PER_OPERAND, "B pieces per slab");
// first B piece issued in k step ks = 0..3 of the following step (3: none left)
constexpr int b_early_begin(int ks) { return B_LATE + ((DMA_PER_OPERAND - B_LATE) * ks) / 3; }
// Slots of the last k step (after MFMA x = 0..15): the A piece or the late B
// piece issued there, or -1.  A_STRIDE 1: A after MFMAs 0..7, late B after
// 8..; A_STRIDE 2: A after the even MFMAs, late B after the odd ones.
constexpr int A_STRIDE = 2;
static_assert(A_STRIDE == 1 || A_STRIDE == 2, "A slot spacing");
// the waits count DMA_PER_OPERAND B pieces after A's last piece: late B pieces
// may only follow every A piece
static_assert(A_STRIDE == 1 || B_LATE == 0, "late B pieces between A pieces");
constexpr int a_slot_piece(int x) {
  return (x % A_STRIDE == 0 && x / A_STRIDE < DMA_PER_OPERAND) ? x / A_STRIDE : -1;
}
constexpr int b_slot_piece(int x) {
  return A_STRIDE == 1 ? ((x >= DMA_PER_OPERAND && x - DMA_PER_OPERAND < B_LATE) ? x - DMA_PER_OPERAND : -1)
                       : ((x % 2 == 1 && x / 2 < B_LATE) ? x / 2 : -1);
}
constexpr int DMA_PER_SLAB = 2 * DMA_PER_OPERAND;  // per wave, A and B
template <bool KMAJ>
__device__ __forceinline__ void slab_offsets(uint32_t (&off)[DMA_PER_OPERAND], long ld, int mn0, int MN, int wave,
                                             int lane) {
#pragma unroll
  for (int i = 0; i < DMA_PER_OPERAND; ++i) {
    if constexpr (KMAJ) {
      const int row = 64 * wave + 8 * i + (lane >> 3);
      const int chunk = (lane & 7) ^ ((row >> 1) & 7);
      const int mn = min(mn0 + row, MN - 1);
      off[i] = (uint32_t)(((long)mn * ld + chunk * 8) * 2);
    } else {
      const int krow = 16 * wave + 2 * i + (lane >> 5);
      const int chunk = (lane & 31) ^ ((krow & 3) << 2);
      const int mn = min(mn0 + chunk * 8, MN - 8);
      off[i] = (uint32_t)(((long)krow * ld + mn) * 2);
    }
  }
}

// Buffer resource over `bytes` bytes from `base` (gfx9 word 3 with a 32-bit
// data format; a zero format would disable the access).  Offsets at or beyond
// the extent read zero / write nothing.  The extent is a 32-bit byte count.
constexpr int RSRC_WORD3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc32(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, RSRC_WORD3);
}

// One 16-byte buffer load per lane that writes LDS directly: bytes
// [voff, voff + 16) of the resource land at LDS address lds + 16*l for lane l
// (zeros where they lie outside the resource).  Issued through inline
// assembly so that the compiler's own wait-count bookkeeping ignores it; the
// pipeline waits for these loads explicitly (sync_slab) before any LDS read
// of their data.
__device__ __forceinline__ void dma16(uint32_t voff, __amdgpu_buffer_rsrc_t rs, uint32_t lds) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rs), "{m0}"(lds) : "memory");
}

// LDS byte address of a pointer into a __shared__ object.
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) const char*)p);
}

// Copy the slab starting at k0 into LDS with 16-byte direct loads (wave is
// uniform, so the LDS addresses are scalar).  The resource spans the token's
// operand; the slab's offset (k0 elements along a row, or k0 rows) is added
// to each lane's offset, so every piece is range-checked against the operand.
template <bool KMAJ>
__device__ __forceinline__ void dma_slab(char* lds, __amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[DMA_PER_OPERAND],
                                         long ld, int k0, int wave) {
  const uint32_t koff = (uint32_t)(KMAJ ? (long)k0 * 2 : (long)k0 * ld * 2);
#pragma unroll
  for (int i = 0; i < DMA_PER_OPERAND; ++i) {
    const int dst = KMAJ ? (64 * wave + 8 * i) * 128 : (16 * wave + 2 * i) * 512;
    dma16(off[i] + koff, rs, lds_addr(lds + dst));
  }
}

// MFMA fragment (32 rows of m or n, 16 of k at k-step ks) for this lane.
template <bool KMAJ>
__device__ __forceinline__ short8_t read_frag(const char* lds, int row0, int ks, int lane) {
  if constexpr (KMAJ) {
    const int row = row0 + (lane & 31);
    const int chunk = 2 * ks + (lane >> 5);
    return *reinterpret_cast<const short8_t*>(lds + kswz(row, chunk));
  } else {
    const int g = lane >> 4, li = lane & 15;
    const int krow = 16 * ks + 8 * (g >> 1) + (li >> 2);
    const int col = row0 + 16 * (g & 1) + 4 * (li & 3);
    const int off0 = mswz(krow, col >> 3) + (col & 7) * 2;
    const int off1 = mswz(krow + 4, col >> 3) + (col & 7) * 2;
    const short4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off0));
    const short4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4*)(lds + off1));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  }
}

// Operand fragments of one 16-deep k step: 4 of A (m blocks), 4 of B (n blocks).
// Eight 16-bit elements per lane per fragment, bf16 or fp16 by the kernel.
struct Frags {
  short8_t a[4], b[4];
};

template <bool AK, bool BKM>
__device__ __forceinline__ void read_frags(Frags& f, const char* a_s, const char* b_s, int wm, int wn, int ks,
                                           int lane) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f.a[i] = read_frag<AK>(a_s, wm * 128 + 32 * i, ks, lane);
#pragma unroll
  for (int j = 0; j < 4; ++j) f.b[j] = read_frag<BKM>(b_s, wn * 128 + 32 * j, ks, lane);
}

// 16 MFMAs of one k step.  The B fragment is the MFMA's first operand, so
// each 32 x 32 accumulator block holds C transposed: element v of lane l is
// C[m = l%32][n = 8*(v/4) + 4*(l/32) + v%4], four consecutive n per lane.
// ZERO: the tile's first k step starts from zero accumulators.  ST selects
// v_mfma_f32_32x32x16_bf16 or v_mfma_f32_32x32x16_f16 (same operand layout).
template <typename ST, bool ZERO>
__device__ __forceinline__ void mfma16(f32x16_t (&acc)[4][4], const Frags& f) {
  const f32x16_t zero = {};
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (std::is_same<ST, f16_t>::value)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, f.b[j]),
                                                           __builtin_bit_cast(f16x8_t, f.a[i]),
                                                           ZERO ? zero : acc[i][j], 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f.b[j]),
                                                            __builtin_bit_cast(bf16x8_t, f.a[i]),
                                                            ZERO ? zero : acc[i][j], 0, 0, 0);
    }
}

// The bias enters as the accumulators' starting value: one MFMA per block
// with a rank-1 product, first operand = the bias column of the block (k = 0:
// lane l < 32 holds bias[n = l] in element 0, everything else 0), second
// operand = ones (lane l < 32 holds 1.0 in element 0), so that block (i, j)
// starts at bias[n] in every row m; the products are exact in fp32.  This
// replaces a bias load and add in the epilogue.
template <typename ST>
constexpr uint32_t ONE_BITS = std::is_same<ST, f16_t>::value ? 0x3C00u : 0x3F80u;

template <typename ST>
__device__ __forceinline__ void bias_init(f32x16_t (&acc)[4][4], const uint16_t (&bf)[4], uint32_t ones) {
  const f32x16_t zero = {};
  const short8_t one8 = __builtin_bit_cast(short8_t, v4u32{ones, 0u, 0u, 0u});
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const short8_t b8 = __builtin_bit_cast(short8_t, v4u32{(uint32_t)bf[j], 0u, 0u, 0u});
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if constexpr (std::is_same<ST, f16_t>::value)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, b8),
                                                           __builtin_bit_cast(f16x8_t, one8), zero, 0, 0, 0);
      else
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, b8),
                                                            __builtin_bit_cast(bf16x8_t, one8), zero, 0, 0, 0);
    }
  }
}

// Scheduling pattern for 16 MFMAs whose fragments are already in registers,
// issued together with NREAD LDS reads for a later k step: one MFMA, one
// read, alternately, then the remaining MFMAs.
template <int NREAD>
__device__ __forceinline__ void interleave() {
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (k < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
  }
}

// Wait until this wave's LDS reads are done and at most N of its
// vector-memory operations are outstanding (gfx9 s_waitcnt encoding: vmcnt
// in bits 3:0 and 15:14, expcnt 6:4 left at its maximum, lgkmcnt 11:8 = 0),
// then a workgroup barrier.  Vector-memory operations complete in issue
// order, so afterwards every wave's operations older than its newest N are
// done, and no wave still reads LDS data from before the barrier.
template <int N>
__device__ __forceinline__ void sync_slab() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0070);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Raw buffer resource for the epilogue: base and a byte extent of at most
// 2^31 - 1, so that OUT_OF_RANGE lies beyond every extent.
constexpr uint32_t OUT_OF_RANGE = 0x80000000u;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, long bytes) {
  const int n = (int)min(bytes, 0x7fffffffL);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, RSRC_WORD3);
}

// One tile of the persistent schedule: token, first row, first column.
struct Tile {
  int t, m0, n0;
};
__device__ __forceinline__ Tile tile_of(int logical, int tiles_m, int per_t) {
  Tile c;
  c.t = logical / per_t;
  const int in_t = logical - c.t * per_t;
  const int tn = in_t / tiles_m;
  c.m0 = (in_t - tn * tiles_m) * BM;
  c.n0 = tn * BN;
  return c;
}

// Byte extent of one token's operand: from its first element to one past its
// last.  K-major: rows (m or n) of K contiguous elements; M/N-major: K rows of
// MN contiguous elements.
__device__ __forceinline__ uint32_t operand_extent(bool kmajor, long ld, int K, int MN) {
  return (uint32_t)(kmajor ? ((long)(MN - 1) * ld + K) * 2 : ((long)(K - 1) * ld + MN) * 2);
}

// Operand source of one tile: buffer resources over the token's A and B
// operands and this thread's eight slab offsets for each.
struct Src {
  __amdgpu_buffer_rsrc_t A, B;
  uint32_t offa[DMA_PER_OPERAND], offb[DMA_PER_OPERAND];
};
// active = false gives resources of extent 0: every copy through them reads
// nothing and writes zeros (the next tile's copies when there is none).
template <bool AK, bool BKM>
__device__ __forceinline__ void tile_src(Src& s, const GemmArgs& g, const Tile& c, int wave, int lane,
                                         bool active = true) {
  s.A = rsrc32(reinterpret_cast<const char*>(g.A) + (long)c.t * g.a_bs * 2,
               active ? operand_extent(AK, g.a_ld, g.K, g.M) : 0u);
  s.B = rsrc32(reinterpret_cast<const char*>(g.B) + (long)c.t * g.b_bs * 2,
               active ? operand_extent(BKM, g.b_ld, g.K, g.N) : 0u);
  slab_offsets<AK>(s.offa, g.a_ld, c.m0, g.M, wave, lane);
  slab_offsets<BKM>(s.offb, g.b_ld, c.n0, g.N, wave, lane);
}

template <bool KMAJ>
__device__ __forceinline__ void dma_operand(char* stage, __amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[DMA_PER_OPERAND],
                                            long ld, int kslab, int wave) {
  dma_slab<KMAJ>(stage, rs, off, ld, kslab * BK, wave);
}

// Piece i of dma_slab alone (the same source offset and LDS destination).
template <bool KMAJ>
__device__ __forceinline__ void dma_piece(char* stage, __amdgpu_buffer_rsrc_t rs, uint32_t off, uint32_t koff, int i,
                                          int wave) {
  const int dst = KMAJ ? (64 * wave + 8 * i) * 128 : (16 * wave + 2 * i) * 512;
  dma16(off + koff, rs, lds_addr(stage + dst));
}

// Byte offset of a slab along an operand: k0 elements along each row (K-major) or k0 rows.
template <bool KMAJ>
__device__ __forceinline__ uint32_t slab_koff(long ld, int kslab) {
  return (uint32_t)(KMAJ ? (long)kslab * BK * 2 : (long)kslab * BK * ld * 2);
}

// B pieces b_early_begin(ks) .. b_early_begin(ks + 1) - 1 of a slab into its
// stage (k step ks = 0, 1, 2 of the step after the one that issued the slab's
// first pieces), fenced from the surrounding schedule.
template <bool KMAJ, int KS>
__device__ __forceinline__ void early_b(char* stage, __amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[DMA_PER_OPERAND],
                                        uint32_t koff, int wave) {
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = b_early_begin(KS); i < b_early_begin(KS + 1); ++i) dma_piece<KMAJ>(stage, rs, off[i], koff, i, wave);
  __builtin_amdgcn_sched_barrier(0);
}

// Residual of a tile's epilogue, copied into LDS like the operand slabs.
// During the epilogue two stages are free: the B stage and the A stage of the
// tile's last slab (the next tile's B slab 2 and A slab 1 go there only
// afterwards).  Each wave copies the 32 x 128 residual block of its m block i
// into its own 8 KB of one of them (i even: the B stage, i odd: the A stage),
// so a wave reads only data it copied itself and needs no barrier: row r of a
// block is 256 bytes whose 16-byte chunks are XOR-swizzled by r % 16, piece p
// (one copy per lane) holds rows 4p .. 4p+3.
struct ResDma {
  __amdgpu_buffer_rsrc_t rs;          // the token's residual rows
  uint32_t off[4];                    // block 0 source offsets of pieces 0..3 (OUT_OF_RANGE past N);
                                      // piece p + 4 is 16 rows further on, same columns
  uint32_t step;                      // bytes from one block to the next (32 rows)
  char* xb;                           // this wave's 8 KB of the free B stage (blocks 0, 2)
  char* ya;                           // this wave's 8 KB of the free A stage (blocks 1, 3)
};
constexpr int RES_REGION = 8192;      // bytes of one wave's block: 32 rows x 256 bytes

__device__ __forceinline__ void res_offsets(ResDma& r, const GemmArgs& g, const Tile& c, int wm, int wn, int lane) {
  const uint32_t rld = (uint32_t)(g.res_ld * 2);
  r.rs = make_rsrc(reinterpret_cast<const char*>(g.res) + (long)c.t * g.res_bs * 2, (long)g.M * g.res_ld * 2);
  r.step = 32u * rld;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int row = 4 * p + (lane >> 4);
    const int lc = (lane & 15) ^ (row & 15);
    const int m = c.m0 + wm * 128 + row;  // rows past M read zero (offset beyond the extent)
    const int n = c.n0 + wn * 128 + 8 * lc;
    r.off[p] = n < g.N ? (uint32_t)m * rld + (uint32_t)n * 2 : OUT_OF_RANGE;
  }
}

// Piece p of residual block blk into a wave region.
__device__ __forceinline__ void res_piece(const ResDma& r, char* region, int blk, int p) {
  const uint32_t o = r.off[p & 3];
  const uint32_t rows = (uint32_t)blk * r.step + (p >= 4 ? r.step / 2 : 0u);  // 32 rows per block, 16 per half
  dma16(o == OUT_OF_RANGE ? OUT_OF_RANGE : o + rows, r.rs, lds_addr(region + p * 1024));
}

// The last k step of a slab: its 16 MFMAs, with the copies of the freed
// stages (8 A pieces, then the first B_LATE B pieces) issued one after each
// MFMA and the next slab's first-k-step fragments read after MFMAs 8..15.
// Each group is fenced (sched_barrier), so the copies issue in the shadow of
// the MFMAs instead of as a burst while the matrix pipe waits.  There are no
// branches: copies that have no source go through a resource of extent 0.
// RDMA (the last step of a tile with a residual): the slots carry residual
// block 0 (slots 0..7), then block 1 (slots 8..15), instead of the A pieces,
// whose copy follows the epilogue; block 1 after all of block 0 leaves exactly
// DMA_PER_OPERAND copies after block 0 for the epilogue's first wait.
template <typename ST, bool AK, bool BKM, bool RDMA = false>
__device__ __forceinline__ void last_kstep(f32x16_t (&acc)[4][4], const Frags& f1, Frags& f0, const char* na,
                                           const char* nb, char* sa, char* sb, __amdgpu_buffer_rsrc_t rsa,
                                           const uint32_t (&offa)[DMA_PER_OPERAND], uint32_t koffa,
                                           __amdgpu_buffer_rsrc_t rsb, const uint32_t (&offb)[DMA_PER_OPERAND],
                                           uint32_t koffb, int wm, int wn, int wave, int lane, const ResDma* rd) {
  static_assert(!RDMA || B_LATE == 0, "residual slots leave no room for late B pieces");
#pragma unroll
  for (int x = 0; x < 16; ++x) {
    const int i = x >> 2, j = x & 3;
    if constexpr (std::is_same<ST, f16_t>::value)
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, f1.b[j]),
                                                         __builtin_bit_cast(f16x8_t, f1.a[i]), acc[i][j], 0, 0, 0);
    else
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, f1.b[j]),
                                                          __builtin_bit_cast(bf16x8_t, f1.a[i]), acc[i][j], 0, 0, 0);
    if constexpr (RDMA) {
      res_piece(*rd, x < DMA_PER_OPERAND ? rd->xb : rd->ya, x < DMA_PER_OPERAND ? 0 : 1, x % DMA_PER_OPERAND);
    } else {
      if (a_slot_piece(x) >= 0) dma_piece<AK>(sa, rsa, offa[a_slot_piece(x)], koffa, a_slot_piece(x), wave);
      if (b_slot_piece(x) >= 0) dma_piece<BKM>(sb, rsb, offb[b_slot_piece(x)], koffb, b_slot_piece(x), wave);
    }
    if (x >= 8) {
      const int r = x - 8;
      if (r < 4) f0.a[r] = read_frag<AK>(na, wm * 128 + 32 * r, 0, lane);
      else f0.b[r - 4] = read_frag<BKM>(nb, wn * 128 + 32 * (r - 4), 0, lane);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Four 16-bit storage values (two packed words) added to v.
template <typename ST>
__device__ __forceinline__ void add16x4(float (&v)[4], v2u32 w) {
  v[0] += lo16<ST>(w.x);
  v[1] += hi16<ST>(w.x);
  v[2] += lo16<ST>(w.y);
  v[3] += hi16<ST>(w.y);
}

// Tile epilogue: C = acc (+ residual), bf16
// (a bias is already in the accumulators, see bias_init).  Each wave's 32 x
// 128 block i passes through 8 KB of LDS: lane l holds, per (n block j, group
// q), the 4 columns 32j + 8q + 4(l/32) .. + 3 of row l%32 and writes them
// (8 bytes) at row r, logical 16-byte chunk 4j + q of 256-byte rows whose
// chunks are XOR-swizzled by row % 16; it then reads back 16 bytes of a row,
// so each store covers 4 rows x 256 contiguous bytes (whole cache lines),
// with no lane exchanges.  Every store is issued (rows past M or columns past
// N get an out-of-range offset, which the buffer unit drops): EPI_STORES per
// wave.
//   Without a residual, block i uses this wave's part of the free B stage
// (ResDma::xb).  With one (RES), block i's residual is already in that place
// (blocks 0, 2 in xb, 1, 3 in ya, copied by ResDma): the epilogue waits for it
// with an exact count (RES_WAIT: the copies and stores this wave issued after
// it), reads each 8-byte piece, adds it in fp32 and writes the sum over it,
// and after block i's stores copies block i+2 into the same place.
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
constexpr int EPI_STORES_PER_BLOCK = EPI_STORES / 4;
// vector-memory operations issued after residual block i's copy when the epilogue waits for it
constexpr int RES_WAIT[4] = {DMA_PER_OPERAND, EPI_STORES_PER_BLOCK + DMA_PER_OPERAND,
                             EPI_STORES_PER_BLOCK + DMA_PER_OPERAND, EPI_STORES_PER_BLOCK};

template <typename ST, bool RES>
__device__ __forceinline__ void epilogue(const f32x16_t (&acc)[4][4], const GemmArgs& g, const Tile& c, int wm, int wn,
                                         int lane, const ResDma& rd) {
  const int r = lane & 31, h = lane >> 5;
  char* cbase = reinterpret_cast<char*>(g.C) + (long)c.t * g.c_bs * 2;
  const __amdgpu_buffer_rsrc_t crs = make_rsrc(cbase, (long)g.M * g.c_ld * 2);
  const uint32_t cld = (uint32_t)(g.c_ld * 2);
  const int rr0 = lane >> 4, ch = lane & 15;  // read-back: row 4s + rr0, logical chunk ch
  const int ns = c.n0 + wn * 128 + 8 * ch;
  // store s of block i: row m0 + 128 wm + rr0 + (32 i + 4 s), so its offset is this lane's
  // base plus a uniform multiple of the row pitch; rows_left = rows from the lane's first on
  const int m_first = c.m0 + wm * 128 + rr0;
  const int rows_left = ns < g.N ? g.M - m_first : 0;
  const uint32_t off_first = (uint32_t)m_first * cld + (uint32_t)ns * 2;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    __builtin_amdgcn_sched_barrier(0);
    char* stg = (RES && (i & 1)) ? rd.ya : rd.xb;
    if constexpr (RES) {
      if (i == 0) vm_wait<RES_WAIT[0]>();  // i is a constant once the loop is unrolled
      else if (i == 1) vm_wait<RES_WAIT[1]>();
      else if (i == 2) vm_wait<RES_WAIT[2]>();
      else vm_wait<RES_WAIT[3]>();
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // one n block at a time keeps few registers live (the residual kernels are at the limit)
      if constexpr (RES) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v2u32* piece = reinterpret_cast<v2u32*>(stg + r * 256 + (((4 * j + q) ^ (r & 15)) << 4) + 8 * h);
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * q + e];
        if constexpr (RES) add16x4<ST>(v, *piece);
        *piece = v2u32{pair16<ST>(v[0], v[1]), pair16<ST>(v[2], v[3])};
      }
    }
#pragma unroll
    for (int s8 = 0; s8 < 8; ++s8) {
      if (RES && s8 == 4) __builtin_amdgcn_sched_barrier(0);  // four read-backs in flight at a time
      const int rr = 4 * s8 + rr0;
      const v4u32 val = *reinterpret_cast<const v4u32*>(stg + rr * 256 + ((ch ^ (rr & 15)) << 4));
      const int dr = 32 * i + 4 * s8;  // rr - rr0
      const uint32_t co = dr < rows_left ? off_first + (uint32_t)dr * cld : OUT_OF_RANGE;
      __builtin_amdgcn_raw_buffer_store_b128(val, crs, co, 0, 0);
    }
    if constexpr (RES) {
      if (i < 2) {
        // this wave's reads of the place are complete: residual block i+2 into it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int p = 0; p < DMA_PER_OPERAND; ++p) res_piece(rd, stg, i + 2, p);
      }
    }
  }
  __builtin_amdgcn_sched_barrier(0);
}

// Wait counts of the slab steps (see gemm256_body).
constexpr int WAIT_STEADY = DMA_PER_OPERAND;
constexpr int WAIT_AFTER_EPILOGUE = DMA_PER_OPERAND + EPI_STORES;
static_assert(WAIT_AFTER_EPILOGUE <= 63, "vmcnt range");

// Where a slab step's copies come from: this tile's slab (CUR), the next
// tile's (NXT, only when there is a next tile), or nothing.
enum { FROM_CUR = 0, FROM_NXT = 1 };

// One slab step k of a tile with nk slabs.  On entry f0 holds slab k's
// first-k-step fragments (A stage sa, B stage sb).  The second, third and
// fourth k steps' fragments are read while the previous k step's MFMAs
// issue; then this wave waits for its LDS reads and for slab k+1 (stages na,
// nb), leaving at most `wait` newer vector-memory operations in flight (the
// caller's count, see gemm256_body), and the workgroup barrier.  The stages
// just freed receive A slab k+2 (sa) and B slab k+3 (sb): from this tile
// (k+2 < nk, k+3 < nk) or the next one (when there is one).  The next slab's
// first fragments are read during the last k step's MFMAs.
template <typename ST, bool AK, bool BKM, bool ZERO, int SRC_A, int SRC_B, bool BIAS = false, bool RDMA = false>
__device__ __forceinline__ void slab_step(f32x16_t (&acc)[4][4], Frags& f0, Frags& f1, char* sa, char* sb,
                                          const char* na, const char* nb, char* eb, int k, int nk, int wait,
                                          const GemmArgs& g, const Src& cur, const Src& nxt, int wm, int wn, int wave,
                                          int lane, const uint16_t (&bf)[4], uint32_t ones, const ResDma* rd = nullptr) {
  constexpr int NR = (AK ? 4 : 8) + (BKM ? 4 : 8);
  // B slab k+2 (stage eb, freed by the previous step) comes from where A slab k+2 does
  const Src& srca = SRC_A == FROM_CUR ? cur : nxt;
  const uint32_t koffe = slab_koff<BKM>(g.b_ld, SRC_A == FROM_CUR ? k + 2 : k + 2 - nk);
  early_b<BKM, 0>(eb, srca.B, srca.offb, koffe, wave);
  read_frags<AK, BKM>(f1, sa, sb, wm, wn, 1, lane);
  if constexpr (ZERO && BIAS) {
    bias_init<ST>(acc, bf, ones);
    mfma16<ST, false>(acc, f0);
  } else {
    mfma16<ST, ZERO>(acc, f0);
  }
  interleave<NR>();
  __builtin_amdgcn_sched_barrier(0);
  early_b<BKM, 1>(eb, srca.B, srca.offb, koffe, wave);
  read_frags<AK, BKM>(f0, sa, sb, wm, wn, 2, lane);
  mfma16<ST, false>(acc, f1);
  interleave<NR>();
  __builtin_amdgcn_sched_barrier(0);
  early_b<BKM, 2>(eb, srca.B, srca.offb, koffe, wave);
  read_frags<AK, BKM>(f1, sa, sb, wm, wn, 3, lane);
  mfma16<ST, false>(acc, f0);
  interleave<NR>();
  if (wait == WAIT_AFTER_EPILOGUE) sync_slab<WAIT_AFTER_EPILOGUE>();
  else sync_slab<WAIT_STEADY>();
  // copies into the freed stages: A slab k+2 and the first B pieces of slab k+3,
  // from this tile or the next one
  const Src& srcb = SRC_B == FROM_CUR ? cur : nxt;
  const uint32_t koffa = slab_koff<AK>(g.a_ld, SRC_A == FROM_CUR ? k + 2 : k + 2 - nk);
  const uint32_t koffb = slab_koff<BKM>(g.b_ld, SRC_B == FROM_CUR ? k + 3 : k + 3 - nk);
  last_kstep<ST, AK, BKM, RDMA>(acc, f1, f0, na, nb, sa, sb, srca.A, srca.offa, koffa, srcb.B, srcb.offb, koffb, wm,
                                wn, wave, lane, rd);
}

// Bias fragment of a tile for bias_init: lane l < 32 loads bias[n0 + 128 wn +
// 32 j + l] (zero past N, for lanes l >= 32 and without a tile).
__device__ __forceinline__ void load_bias_frag(uint16_t (&bf)[4], const GemmArgs& g, const Tile& c, int wn, int lane,
                                               bool active) {
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<const char*>(g.bias) + (long)c.t * g.bias_bs * 2, active ? (long)g.N * 2 : 0L);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = c.n0 + wn * 128 + 32 * j + lane;
    const uint32_t off = (lane < 32 && n < g.N) ? (uint32_t)n * 2 : OUT_OF_RANGE;
    bf[j] = __builtin_amdgcn_raw_buffer_load_b16(rs, off, 0, 0);
  }
}

// Marks the loaded bias fragment as used here, so that the compiler's wait
// for the load lands at this point (it counts only its own memory operations,
// not the copies, so a wait placed anywhere else could also wait for copies
// still in flight).
__device__ __forceinline__ void settle(uint16_t (&bf)[4]) {
  asm volatile("" : "+v"(bf[0]), "+v"(bf[1]), "+v"(bf[2]), "+v"(bf[3]));
}

// Persistent kernel: one workgroup per CU.  Workgroup w runs on XCD w % 8;
// each XCD owns a contiguous range of logical tiles (token-major, then N
// tile, then M tile) and its workgroups take every (grid/8)-th tile of it, so
// the tiles in flight on one XCD share operands in that XCD's L2.
//
// Pipeline.  Slab index s runs on across tiles (nk, the slabs per tile, is
// even).  A slabs use a ring of 2 LDS stages (s % 2), B slabs a ring of 3
// (rotating at run time): the whole 160 KB of LDS.  Step k, once slab k is
// fully read, copies A slab k+2 and the first B_LATE pieces of B slab k+3
// into the stages it frees; the other B pieces of slab k+3 follow in the
// first three k steps of step k+1, so no k step issues more than ten copies
// per wave.  One A slab and about two B slabs are in flight while a slab is
// multiplied (B, the operand with more misses in L2, runs one slab further
// ahead: a copy-only run of these operand streams delivers 15-20 % more bytes
// per clock with B two slabs ahead than with both one ahead).  The copies of
// the last three steps of a tile come from the next tile (if any).
//
// Wait counts (vector-memory operations complete in issue order; every wave
// issues DMA_PER_OPERAND copies per operand and slab, on every step, also
// when they have no source).  Step k waits for slab k+1, whose last copy is
// A(k+1), issued in step k-1's last k step; after it come the DMA_PER_OPERAND
// pieces of B(k+2) (B_LATE in step k-1, the rest in step k before the wait):
//   * steady state: B(k+2) may stay in flight: WAIT_STEADY = DMA_PER_OPERAND;
//   * a tile's first step (not the first tile): the previous tile's epilogue
//     (EPI_STORES stores, every one issued) lies between B(k+2)'s pieces:
//     WAIT_AFTER_EPILOGUE = DMA_PER_OPERAND + EPI_STORES.
// The first tile's prologue issues A(0) B(0) A(1) B(1) and B(2)'s first
// B_LATE pieces and waits for slab 0 with the last of them in flight; its
// first step issues the rest of B(2) and keeps B(2) in flight.  The kernel
// ends with a wait for every copy.

template <typename ST, bool AK, bool BKM, bool BIAS, bool RES>
__device__ __forceinline__ void gemm256_body(const GemmArgs& g) {
  // A ring: sA + s * TILE_BYTES, s = 0, 1; B ring: sB + r * TILE_BYTES, r = 0, 1, 2
  __shared__ __attribute__((aligned(1024))) char sA[2 * TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB[3 * TILE_BYTES];
  char* const a0 = sA;
  char* const a1 = sA + TILE_BYTES;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform per wave: scalar address arithmetic
  const int wm = wave >> 1, wn = wave & 1;

  const int tiles_m = (g.M + BM - 1) / BM, tiles_n = (g.N + BN - 1) / BN;
  const int per_t = tiles_m * tiles_n;
  const int total = per_t * g.batch;
  const int xcd = blockIdx.x & 7, slot = blockIdx.x >> 3, nslots = gridDim.x >> 3;
  const int q = total >> 3, rem = total & 7;
  const int lo = xcd * q + min(xcd, rem), hi = lo + q + (xcd < rem ? 1 : 0);
  int tile = lo + slot;
  if (tile >= hi) return;

  Tile ct = tile_of(tile, tiles_m, per_t);
  Src cur;
  tile_src<AK, BKM>(cur, g, ct, wave, lane);
  // bias fragments of the current and the next tile (the next one's is loaded a tile ahead)
  uint16_t bias_cur[4] = {0, 0, 0, 0}, bias_nxt[4] = {0, 0, 0, 0};
  const uint32_t ones = lane < 32 ? ONE_BITS<ST> : 0u;
  if constexpr (BIAS) {
    load_bias_frag(bias_cur, g, ct, wn, lane, true);
    settle(bias_cur);  // before any copy is issued
  }
  const int nk = g.K / BK;  // even, at least 4
  // B stage of the slab being multiplied (rotates 0, 1, 2 with the global slab index)
  int rb = 0;
  auto bst = [&](int r) { return sB + r * TILE_BYTES; };
  auto nxt3 = [](int r) { return r == 2 ? 0 : r + 1; };
  dma_operand<AK>(a0, cur.A, cur.offa, g.a_ld, 0, wave);
  dma_operand<BKM>(bst(0), cur.B, cur.offb, g.b_ld, 0, wave);
  dma_operand<AK>(a1, cur.A, cur.offa, g.a_ld, 1, wave);
  dma_operand<BKM>(bst(1), cur.B, cur.offb, g.b_ld, 1, wave);
#pragma unroll
  for (int i = 0; i < B_LATE; ++i) dma_piece<BKM>(bst(2), cur.B, cur.offb[i], slab_koff<BKM>(g.b_ld, 2), i, wave);
  sync_slab<2 * DMA_PER_OPERAND + B_LATE>();
  Frags f0, f1;
  read_frags<AK, BKM>(f0, a0, bst(0), wm, wn, 0, lane);

  f32x16_t acc[4][4];
  bool first = true;
  for (;;) {
    const int next = tile + nslots;
    const bool has_next = next < hi;
    const Tile nt = tile_of(has_next ? next : tile, tiles_m, per_t);
    Src nxt;
    tile_src<AK, BKM>(nxt, g, nt, wave, lane, has_next);  // extent 0 without a next tile
    if constexpr (BIAS) load_bias_frag(bias_nxt, g, nt, wn, lane, has_next);

    // step 0 (accumulators start from zero); for nk == 4 it is also step nk-4
    {
      char* sb = bst(rb);
      const char* nb = bst(nxt3(rb));
      char* eb = bst(nxt3(nxt3(rb)));
      slab_step<ST, AK, BKM, true, FROM_CUR, FROM_CUR, BIAS>(acc, f0, f1, a0, sb, a1, nb, eb, 0, nk,
                                                            (first || RES) ? WAIT_STEADY : WAIT_AFTER_EPILOGUE, g, cur,
                                                            nxt, wm,
                                                            wn, wave, lane, bias_cur, ones);
      rb = nxt3(rb);
    }
    // steps 1 .. nk-4 in pairs (A stages 1, 0): every copy from this tile
    for (int k = 1; k + 1 <= nk - 4; k += 2) {
      {
        char* sb = bst(rb);
        const char* nb = bst(nxt3(rb));
        char* eb = bst(nxt3(nxt3(rb)));
        slab_step<ST, AK, BKM, false, FROM_CUR, FROM_CUR>(acc, f0, f1, a1, sb, a0, nb, eb, k, nk, WAIT_STEADY, g, cur, nxt,
                                                         wm, wn, wave, lane, bias_cur, ones);
        rb = nxt3(rb);
      }
      {
        char* sb = bst(rb);
        const char* nb = bst(nxt3(rb));
        char* eb = bst(nxt3(nxt3(rb)));
        slab_step<ST, AK, BKM, false, FROM_CUR, FROM_CUR>(acc, f0, f1, a0, sb, a1, nb, eb, k + 1, nk, WAIT_STEADY, g, cur,
                                                         nxt, wm, wn, wave, lane, bias_cur, ones);
        rb = nxt3(rb);
      }
    }
    // step nk-3 (A stage 1): A slab nk-1 of this tile, B slab 0 of the next
    {
      char* sb = bst(rb);
      const char* nb = bst(nxt3(rb));
      char* eb = bst(nxt3(nxt3(rb)));
      slab_step<ST, AK, BKM, false, FROM_CUR, FROM_NXT>(acc, f0, f1, a1, sb, a0, nb, eb, nk - 3, nk, WAIT_STEADY, g, cur,
                                                       nxt, wm, wn, wave, lane, bias_cur, ones);
      rb = nxt3(rb);
    }
    // steps nk-2 (A stage 0) and nk-1 (A stage 1): the next tile's A slabs 0, 1 and B slabs 1, 2
    // (with a residual, step nk-1 copies residual blocks 0, 1 instead and A slab 1 follows the
    // epilogue).
    // Without a next tile these copies read nothing (extent 0) and fill freed stages with
    // zeros, and the last step's fragment reads of the next stages are unused: the same code
    // on both paths keeps the accumulators in AGPRs.
    {
      char* sb = bst(rb);
      const char* nb = bst(nxt3(rb));
      char* eb = bst(nxt3(nxt3(rb)));
      slab_step<ST, AK, BKM, false, FROM_NXT, FROM_NXT>(acc, f0, f1, a0, sb, a1, nb, eb, nk - 2, nk, WAIT_STEADY, g, cur,
                                                       nxt, wm, wn, wave, lane, bias_cur, ones);
      rb = nxt3(rb);
    }
    ResDma rdm;
    {
      char* sb = bst(rb);
      const char* nb = bst(nxt3(rb));
      char* eb = bst(nxt3(nxt3(rb)));
      rdm.xb = sb + wave * RES_REGION;  // stage of this tile's last B slab
      rdm.ya = a1 + wave * RES_REGION;  // stage of this tile's last A slab
      if constexpr (RES) res_offsets(rdm, g, ct, wm, wn, lane);
      slab_step<ST, AK, BKM, false, FROM_NXT, FROM_NXT, false, RES>(acc, f0, f1, a1, sb, a0, nb, eb, nk - 1, nk,
                                                                    WAIT_STEADY, g, cur, nxt, wm, wn, wave, lane,
                                                                    bias_cur, ones, &rdm);
      rb = nxt3(rb);
    }

    epilogue<ST, RES>(acc, g, ct, wm, wn, lane, rdm);
    // after the epilogue's stores: the wait leaves them in flight
    if constexpr (BIAS) settle(bias_nxt);
    if constexpr (RES) {
      // the next tile's A slab 1 into the stage residual blocks 1 and 3 leave (this wave's reads done)
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < DMA_PER_OPERAND; ++i)
        dma_piece<AK>(a1, nxt.A, nxt.offa[i], slab_koff<AK>(g.a_ld, 1), i, wave);
    }
    if (!has_next) break;
    tile = next;
    ct = nt;
    cur = nxt;
#pragma unroll
    for (int j = 0; j < 4; ++j) bias_cur[j] = bias_nxt[j];
    first = false;
  }
  // the last tile's empty copies still write LDS: let every copy land before the workgroup ends
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
}


// One kernel symbol per GEMM of the block and storage type, so that profiles
// name them; the epilogue (bias, residual) is fixed per kernel.
#define RM_GEMM256_KERNELS(SFX, ST)                                                                            \
  __global__ __launch_bounds__(256, 1) void gemm_up_##SFX(GemmArgs g) { gemm256_body<ST, true, false, true, false>(g); } \
  __global__ __launch_bounds__(256, 1) void gemm_down_##SFX(GemmArgs g) { gemm256_body<ST, true, false, true, true>(g); } \
  __global__ __launch_bounds__(256, 1) void gemm_dhid_##SFX(GemmArgs g) {                                       \
    gemm256_body<ST, true, true, false, false>(g);                                                                   \
  }                                                                                                                  \
  __global__ __launch_bounds__(256, 1) void gemm_dh1_##SFX(GemmArgs g) { gemm256_body<ST, true, true, false, true>(g); } \
  __global__ __launch_bounds__(256, 1) void gemm_dwout_##SFX(GemmArgs g) {                                      \
    gemm256_body<ST, false, false, false, false>(g);                                                                 \
  }                                                                                                                  \
  __global__ __launch_bounds__(256, 1) void gemm_dw1_##SFX(GemmArgs g) { gemm256_body<ST, false, false, false, false>(g); }
RM_GEMM256_KERNELS(bf16, bf16_t)
RM_GEMM256_KERNELS(f16, f16_t)
#undef RM_GEMM256_KERNELS

typedef void (*Gemm256Kernel)(GemmArgs);

// The kernel of each GEMM of the block with its operand layouts and epilogue.
struct Gemm256Entry {
  int kid;
  bool a_kmajor, b_kmajor, bias, res;
  Gemm256Kernel bf16, f16;
};
const Gemm256Entry kGemm256[] = {
    {KID_GEMM_UP, true, false, true, false, gemm_up_bf16, gemm_up_f16},
    {KID_GEMM_DOWN, true, false, true, true, gemm_down_bf16, gemm_down_f16},
    {KID_GEMM_DHID, true, true, false, false, gemm_dhid_bf16, gemm_dhid_f16},
    {KID_GEMM_DH1, true, true, false, true, gemm_dh1_bf16, gemm_dh1_f16},
    {KID_GEMM_DWOUT, false, false, false, false, gemm_dwout_bf16, gemm_dwout_f16},
    {KID_GEMM_DW1, false, false, false, false, gemm_dw1_bf16, gemm_dw1_f16},
};
const Gemm256Entry* gemm256_entry(bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid) {
  for (const Gemm256Entry& e : kGemm256)
    if (e.kid == kid && e.a_kmajor == a_kmajor && e.b_kmajor == b_kmajor && e.bias == (g.bias != nullptr) &&
        e.res == (g.res != nullptr))
      return &e;
  return nullptr;
}

hipError_t run256(Gemm256Kernel k, const GemmArgs& g, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.batch;
  // one workgroup per CU (its LDS use allows no more), a multiple of 8 (XCDs)
  int grid = device_cu_count() & ~7;
  if (grid < 8) grid = 8;
  const int need = (tiles + 7) & ~7;
  if (grid > need) grid = need;
  hipLaunchKernelGGL(k, dim3(grid), dim3(256), 0, s, g);
  return hipGetLastError();
}

}  // namespace

// Compute units of the current device (cached per device; concurrent first
// calls store the same value).
int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool gemm256_supported(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid) {
  if ((dtype != RM_BF16 && dtype != RM_F16) || g.c_f32) return false;  // 16-bit operands and output
  if (gemm256_entry(a_kmajor, b_kmajor, g, kid) == nullptr) return false;
  if (g.K % (2 * BK) != 0 || g.K < 4 * BK) return false;  // nk even, at least 4
  const long a_cont = a_kmajor ? g.K : g.M, b_cont = b_kmajor ? g.K : g.N;
  if (a_cont % 8 || b_cont % 8 || g.a_ld % 8 || g.b_ld % 8 || g.a_bs % 8 || g.b_bs % 8) return false;
  if ((reinterpret_cast<uintptr_t>(g.A) & 15) || (reinterpret_cast<uintptr_t>(g.B) & 15)) return false;
  if (!a_kmajor && g.M < 8) return false;
  if (!b_kmajor && g.N < 8) return false;
  // per-token operand byte offsets fit the 32-bit copy offsets
  const long a_rows = a_kmajor ? g.M : g.K, b_rows = b_kmajor ? g.N : g.K;
  if (a_rows * g.a_ld * 2 > 0xffffffffL || b_rows * g.b_ld * 2 > 0xffffffffL) return false;
  // the epilogue stores 8 columns per lane pair (the bias is read element by element)
  if (g.N % 8 || g.c_ld % 4 || g.c_bs % 4 || (reinterpret_cast<uintptr_t>(g.C) & 15)) return false;
  if (g.res && (g.res_f32 || g.res_ld % 4 || g.res_bs % 4 || (reinterpret_cast<uintptr_t>(g.res) & 15)))
    return false;  // the residual is bf16
  // per-token byte offsets of C and the residual fit the 31-bit buffer range
  if ((long)g.M * g.c_ld * 2 > 0x7fffffffL) return false;
  if (g.res && (long)g.M * g.res_ld * 2 > 0x7fffffffL) return false;
  return true;
}

hipError_t launch_gemm256(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid, hipStream_t s) {
  const Gemm256Entry* e = gemm256_entry(a_kmajor, b_kmajor, g, kid);
  if (e == nullptr) return hipErrorInvalidValue;  // callers check gemm256_supported first
  return run256(dtype == RM_F16 ? e->f16 : e->bf16, g, s);
}

}  // namespace rm
