// T-batched MFMA GEMM for gfx950 (CDNA4, wave64): the six per-token
// contractions of the RankMixerBlock dense FFN and its backward.
//
// Page 1 of "Subgraph-fusion-based Mega-kernel Generation", section "Exact
// computation": Z[b,t,:] = out1[b,t,:] @ w1[t] + b1[t] and
// out2[b,t,:] = hidden[b,t,:] @ wout[t] + bout[t], one independent GEMM per
// token t.  The backward uses the transposed products of the same operands.
//
// Design
//   * one workgroup = 256 threads = 4 waves (2 x 2), block tile BM x BN,
//     wave tile (BM/2) x (BN/2) built from 32x32 MFMA tiles:
//       bf16: v_mfma_f32_32x32x16_bf16 (8 K-contiguous bf16 per lane per operand)
//       fp16: v_mfma_f32_32x32x16_f16  (the same layout, fp16 operands)
//       fp32: v_mfma_f32_32x32x2f32    (fp32 operands, never a lower precision)
//   * K is staged 128 bytes at a time (64 16-bit / 32 fp32) into LDS rows that
//     are K-contiguous for both operands ([mn][k]); the 16-byte chunks of a
//     row are XOR-swizzled by (row/2)%8 so the MFMA fragment reads (32 rows,
//     same chunk) hit distinct banks;
//   * a K-major global operand is copied in 16-byte vectors; an M/N-major one
//     (forward weights, both weight-gradient operands) is loaded as 4(k) x VW(mn)
//     register blocks and transposed in registers before the LDS write, so no
//     transposed copy of any tensor is ever materialised;
//   * the next K slab is loaded into registers while MFMAs run on the current
//     one (single LDS buffer, two barriers per slab);
//   * workgroups are numbered so that each XCD (8 per MI355X, round-robin
//     dispatch) works through a contiguous run of tiles: the M tiles that
//     share a weight slab, and the tokens whose weights it streams, stay in
//     that XCD's L2;
//   * the epilogue adds bias[t] and a residual and stores fp32 or the storage
//     dtype (round to nearest even).
#include <type_traits>

#include "rm_common.h"
#include "rm_internal.h"

namespace rm {
namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

template <typename ST>
struct Cfg;
template <>
struct Cfg<bf16_t> {
  static constexpr int VW = 8;   // elements per 16-byte vector
  static constexpr int BK = 64;  // K per LDS slab (128 bytes)
};
template <>
struct Cfg<f16_t> : Cfg<bf16_t> {};
template <>
struct Cfg<float> {
  static constexpr int VW = 4;
  static constexpr int BK = 32;
};

constexpr int ROWB = 128;  // LDS bytes per tile row (one K slab), no padding: swizzled

__device__ __forceinline__ int swz(int row, int chunk) { return row * ROWB + ((chunk ^ ((row >> 1) & 7)) << 4); }

// ---------------------------------------------------------------------------
// operand tile loader: R rows (m or n) x BK (k) of one operand
template <typename ST, bool KMAJ, int R, bool VEC>
struct Loader {
  static constexpr int VW = Cfg<ST>::VW, BK = Cfg<ST>::BK;
  static constexpr int KCH = BK / VW;                  // 16-byte chunks per K-major row
  static constexpr int NCH = R * KCH / 256;            // K-major: chunks per thread
  static constexpr int KB = BK / 4;                    // MN-major: 4-row k blocks per slab
  static constexpr int MNB = R / VW;                   // MN-major: VW-wide mn blocks
  static constexpr int NBLK = R * BK / (4 * VW) / 256; // MN-major: blocks per thread
  static constexpr int NREG = KMAJ ? NCH : 4 * NBLK;
  static_assert(KMAJ ? (R * KCH) % 256 == 0 : (R * BK / (4 * VW)) % 256 == 0, "tile/thread mismatch");
  uint4 r[NREG];

  // element (mn, k) of the operand is at base + mn*ld + k (K-major) or base + k*ld + mn (MN-major)
  __device__ __forceinline__ void load(const ST* __restrict__ base, long ld, int mn0, int MN, int k0, int K,
                                       int tid) {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + 256 * i;
        const int row = id / KCH, kc = id % KCH;
        const int mn = mn0 + row, k = k0 + kc * VW;
        if constexpr (VEC) {
          if (mn < MN && k < K)
            r[i] = *reinterpret_cast<const uint4*>(base + (long)mn * ld + k);
          else
            r[i] = make_uint4(0, 0, 0, 0);
        } else {
          ST tmp[VW];
#pragma unroll
          for (int e = 0; e < VW; ++e) {
            if (mn < MN && k + e < K) tmp[e] = base[(long)mn * ld + k + e];
            else tmp[e] = ST{};
          }
          r[i] = *reinterpret_cast<const uint4*>(tmp);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NBLK; ++i) {
        const int id = tid + 256 * i;
        const int kb_lo = id & 3;
        const int mnb = (id >> 2) % MNB;
        const int kb = (id >> 2) / MNB * 4 + kb_lo;
        const int mn = mn0 + mnb * VW;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
          const int k = k0 + kb * 4 + rr;
          if constexpr (VEC) {
            if (k < K && mn < MN)
              r[4 * i + rr] = *reinterpret_cast<const uint4*>(base + (long)k * ld + mn);
            else
              r[4 * i + rr] = make_uint4(0, 0, 0, 0);
          } else {
            ST tmp[VW];
#pragma unroll
            for (int e = 0; e < VW; ++e) {
              if (k < K && mn + e < MN) tmp[e] = base[(long)k * ld + mn + e];
              else tmp[e] = ST{};
            }
            r[4 * i + rr] = *reinterpret_cast<const uint4*>(tmp);
          }
        }
      }
    }
  }

  __device__ __forceinline__ void store(char* __restrict__ lds, int tid) const {
    if constexpr (KMAJ) {
#pragma unroll
      for (int i = 0; i < NCH; ++i) {
        const int id = tid + 256 * i;
        const int row = id / KCH, kc = id % KCH;
        *reinterpret_cast<uint4*>(lds + swz(row, kc)) = r[i];
      }
    } else {
#pragma unroll
      for (int i = 0; i < NBLK; ++i) {
        const int id = tid + 256 * i;
        const int kb_lo = id & 3;
        const int mnb = (id >> 2) % MNB;
        const int kb = (id >> 2) / MNB * 4 + kb_lo;
        const uint4 a = r[4 * i + 0], b = r[4 * i + 1], c = r[4 * i + 2], d = r[4 * i + 3];
        if constexpr (sizeof(ST) == 2) {
          // 4 rows (k) x 8 bf16 (mn) -> 8 vectors of 4 k-consecutive bf16
          const uint32_t aw[4] = {a.x, a.y, a.z, a.w}, bw[4] = {b.x, b.y, b.z, b.w};
          const uint32_t cw[4] = {c.x, c.y, c.z, c.w}, dw[4] = {d.x, d.y, d.z, d.w};
          const int chunk = kb >> 1, inner = (kb & 1) * 8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int w = e >> 1;
            uint2 v;
            if (e & 1) {
              v.x = (aw[w] >> 16) | (bw[w] & 0xffff0000u);
              v.y = (cw[w] >> 16) | (dw[w] & 0xffff0000u);
            } else {
              v.x = (aw[w] & 0xffffu) | (bw[w] << 16);
              v.y = (cw[w] & 0xffffu) | (dw[w] << 16);
            }
            const int row = mnb * 8 + e;
            *reinterpret_cast<uint2*>(lds + swz(row, chunk) + inner) = v;
          }
        } else {
          // 4 rows (k) x 4 fp32 (mn) -> 4 vectors of 4 k-consecutive fp32
          const int chunk = kb;
          *reinterpret_cast<uint4*>(lds + swz(mnb * 4 + 0, chunk)) = make_uint4(a.x, b.x, c.x, d.x);
          *reinterpret_cast<uint4*>(lds + swz(mnb * 4 + 1, chunk)) = make_uint4(a.y, b.y, c.y, d.y);
          *reinterpret_cast<uint4*>(lds + swz(mnb * 4 + 2, chunk)) = make_uint4(a.z, b.z, c.z, d.z);
          *reinterpret_cast<uint4*>(lds + swz(mnb * 4 + 3, chunk)) = make_uint4(a.w, b.w, c.w, d.w);
        }
      }
    }
  }
};

template <typename ST>
__device__ __forceinline__ float ld_any(const void* p, long i, int is_f32) {
  return is_f32 ? reinterpret_cast<const float*>(p)[i] : to_f32(reinterpret_cast<const ST*>(p)[i]);
}

// ---------------------------------------------------------------------------
template <typename ST, bool AK, bool BKM, int BM, int BN, bool VEC>
__global__ __launch_bounds__(256, 2) void k_gemm(GemmArgs g) {
  constexpr int BK = Cfg<ST>::BK;
  constexpr int WTM = BM / 2, WTN = BN / 2;
  constexpr int TM = WTM / 32, TN = WTN / 32;
  __shared__ __attribute__((aligned(16))) char smem[(BM + BN) * ROWB];
  char* As = smem;
  char* Bs = smem + BM * ROWB;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile numbering: workgroup w runs on XCD w % 8; give each XCD a
  // contiguous range of logical tiles (token-major, then N tile, then M tile).
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

  const ST* A = reinterpret_cast<const ST*>(g.A) + (long)t * g.a_bs;
  const ST* B = reinterpret_cast<const ST*>(g.B) + (long)t * g.b_bs;

  Loader<ST, AK, BM, VEC> la;
  Loader<ST, BKM, BN, VEC> lb;

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = (g.K + BK - 1) / BK;
  la.load(A, g.a_ld, m0, g.M, 0, g.K, tid);
  lb.load(B, g.b_ld, n0, g.N, 0, g.K, tid);
  la.store(As, tid);
  lb.store(Bs, tid);
  __syncthreads();

  const int r32 = lane & 31, hl = lane >> 5;
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) {
      la.load(A, g.a_ld, m0, g.M, (kt + 1) * BK, g.K, tid);
      lb.load(B, g.b_ld, n0, g.N, (kt + 1) * BK, g.K, tid);
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = 2 * ks + hl;
      if constexpr (sizeof(ST) == 2) {
        // bf16: v_mfma_f32_32x32x16_bf16; fp16: v_mfma_f32_32x32x16_f16 (same fragment layout)
        typedef std::conditional_t<std::is_same<ST, f16_t>::value, f16x8_t, bf16x8_t> frag_t;
        frag_t a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          a[i] = *reinterpret_cast<const frag_t*>(As + swz(wm * WTM + 32 * i + r32, chunk));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[j] = *reinterpret_cast<const frag_t*>(Bs + swz(wn * WTN + 32 * j + r32, chunk));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (std::is_same<ST, f16_t>::value)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a[i], b[j], acc[i][j], 0, 0, 0);
            else
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
          }
      } else {
        float4 a[TM], b[TN];
#pragma unroll
        for (int i = 0; i < TM; ++i)
          a[i] = *reinterpret_cast<const float4*>(As + swz(wm * WTM + 32 * i + r32, chunk));
#pragma unroll
        for (int j = 0; j < TN; ++j)
          b[j] = *reinterpret_cast<const float4*>(Bs + swz(wn * WTN + 32 * j + r32, chunk));
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].x, b[j].x, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].y, b[j].y, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].z, b[j].z, acc[i][j], 0, 0, 0);
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[i].w, b[j].w, acc[i][j], 0, 0, 0);
          }
      }
    }
    if (kt + 1 < nk) {
      __syncthreads();
      la.store(As, tid);
      lb.store(Bs, tid);
      __syncthreads();
    }
  }

  // epilogue: 32x32 accumulator layout: element v of lane l is
  // (row 8*(v/4) + 4*(l/32) + v%4, column l%32)
  const ST* bias = reinterpret_cast<const ST*>(g.bias);
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int col = n0 + wn * WTN + 32 * j + r32;
      if (col >= g.N) continue;
      const float bv = bias ? to_f32(bias[(long)t * g.bias_bs + col]) : 0.f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int row = m0 + wm * WTM + 32 * i + 8 * (v >> 2) + 4 * hl + (v & 3);
        if (row >= g.M) continue;
        float val = acc[i][j][v] + bv;
        if (g.res) val += ld_any<ST>(g.res, (long)t * g.res_bs + (long)row * g.res_ld + col, g.res_f32);
        const long o = (long)t * g.c_bs + (long)row * g.c_ld + col;
        if (g.c_f32)
          reinterpret_cast<float*>(g.C)[o] = val;
        else
          reinterpret_cast<ST*>(g.C)[o] = from_f32<ST>(val);
      }
    }
  }
}

template <typename ST, bool AK, bool BKM, int BM, int BN>
hipError_t run(const GemmArgs& g, bool vec, hipStream_t s) {
  const int tiles = ((g.M + BM - 1) / BM) * ((g.N + BN - 1) / BN) * g.batch;
  if (vec)
    hipLaunchKernelGGL((k_gemm<ST, AK, BKM, BM, BN, true>), dim3(tiles), dim3(256), 0, s, g);
  else
    hipLaunchKernelGGL((k_gemm<ST, AK, BKM, BM, BN, false>), dim3(tiles), dim3(256), 0, s, g);
  return hipGetLastError();
}

template <typename ST, bool AK, bool BKM>
hipError_t run_shape(const GemmArgs& g, bool vec, hipStream_t s) {
  const long cus = device_cu_count();
  auto tiles = [&](int bm, int bn) { return (long)((g.M + bm - 1) / bm) * ((g.N + bn - 1) / bn) * g.batch; };
  // the larger of M and N gets the 256-wide side of the tile, while that leaves no compute unit idle
  if (g.M >= g.N && tiles(256, 128) >= cus) return run<ST, AK, BKM, 256, 128>(g, vec, s);
  if (g.M < g.N && tiles(128, 256) >= cus) return run<ST, AK, BKM, 128, 256>(g, vec, s);
  // few tiles (small B or few tokens): smaller tiles spread the work over more compute units.  A
  // 64-wide side needs a K-major operand on it (the M/N-major loader covers 128 rows at least).
  if (tiles(128, 128) >= cus) return run<ST, AK, BKM, 128, 128>(g, vec, s);
  if constexpr (AK) {
    if (!BKM || g.M >= g.N) return run<ST, AK, BKM, 64, 128>(g, vec, s);
  }
  if constexpr (BKM) return run<ST, AK, BKM, 128, 64>(g, vec, s);
  return run<ST, AK, BKM, 128, 128>(g, vec, s);
}

template <typename ST>
hipError_t dispatch(bool ak, bool bk, const GemmArgs& g, bool vec, hipStream_t s) {
  if (ak && !bk) return run_shape<ST, true, false>(g, vec, s);   // forward: weights N-major
  if (ak && bk) return run_shape<ST, true, true>(g, vec, s);     // data gradient
  if (!ak && !bk) return run_shape<ST, false, false>(g, vec, s); // weight gradient
  return hipErrorInvalidValue;
}

inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

hipError_t launch_gemm(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid, hipStream_t s) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0 || g.batch <= 0) return hipSuccess;
  const int vw = dtype == RM_F32 ? 4 : 8;
  // 16-byte vector loads need every contiguous extent, stride and batch
  // offset to be a multiple of the vector width and 16-byte aligned bases.
  const long a_cont = a_kmajor ? g.K : g.M, b_cont = b_kmajor ? g.K : g.N;
  const bool vec = (a_cont % vw == 0) && (b_cont % vw == 0) && (g.a_ld % vw == 0) && (g.b_ld % vw == 0) &&
                   (g.a_bs % vw == 0) && (g.b_bs % vw == 0) && aligned16(g.A) && aligned16(g.B);
  prof_begin(kid, s);
  hipError_t e;
  if (gemm256_supported(dtype, a_kmajor, b_kmajor, g, kid))
    e = launch_gemm256(dtype, a_kmajor, b_kmajor, g, kid, s);
  else
    e = dtype == RM_BF16  ? dispatch<bf16_t>(a_kmajor, b_kmajor, g, vec, s)
        : dtype == RM_F16 ? dispatch<f16_t>(a_kmajor, b_kmajor, g, vec, s)
                          : dispatch<float>(a_kmajor, b_kmajor, g, vec, s);
  prof_end(kid, s);
  return e;
}

}  // namespace rm
