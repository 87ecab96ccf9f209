// Small-batch path of the RankMixerBlock forward and backward (page 1 of
// "Subgraph-fusion-based Mega-kernel Generation", section "Exact
// computation"), for B <= 8, D <= 128, H <= 256.  At these sizes each fused
// step of the main path is a few microseconds of launch and memory latency,
// so here a token's whole chain runs in one workgroup with its B rows in LDS:
// one launch for the forward, two for the backward.
//
// Forward, one workgroup per token t (8 waves; wave b owns row (b, t)):
//   1. norm0 statistics of every row of every sample (each workgroup
//      recomputes them: the token-mix gather of row (b, t) reads all rows of
//      sample b);
//   2. out1[b,t] = norm1(token_mix(norm0(x))[b,t] + x[b,t]);
//   3. Z = out1 @ w1[t] + b1[t];  4. hidden = LN_x(U) * silu(LN_gate(G));
//   5. r2 = out1 + hidden @ wout[t] + bout[t];  6. y = norm2(r2).
// The saved state (out1, Z, hidden, r2 and the ten statistics) goes to the
// same workspace regions as in the main path, rounded to the storage type at
// the same points, so either backward can follow either forward.
//
// Backward, one workgroup per token t: norm2 backward, dbout[t], dwout[t],
// d hidden, the gate backward, db1[t], dw1[t], d out1 and the norm1 backward
// -> d r1 (workspace), with per-token partial sums of the LayerNorm affine
// gradients.  Then one workgroup: the token-mix adjoint (the same gather) and
// the norm0 backward -> dx, and every affine gradient summed over the tokens
// in a fixed order.  Every sum runs in a fixed order: results are bitwise
// repeatable.
#include <type_traits>

#include "rm_common.h"
#include "rm_internal.h"

namespace rm {
namespace {

constexpr float EPS_OUTER = 1e-3f;  // norm0, norm1, norm2
constexpr float EPS_INNER = 1e-5f;  // LN_x, LN_gate
constexpr int SB = SMALL_MAX_B, SD = SMALL_MAX_D, SH = SMALL_MAX_H;
constexpr int QD = SD / 64, QH = SH / 64;  // columns per lane
constexpr int FWD_THREADS = 64 * SB;       // one wave per row of the token
// partial sums of a contraction split over FWD_THREADS / D thread groups
constexpr int TMP_FLOATS = FWD_THREADS * SB > SB * SH ? FWD_THREADS * SB : SB * SH;
static_assert(SB * 2 * SH >= FWD_THREADS * SB, "the output projection's partial sums fit the Z area");

struct SmallArgs {
  const void *x, *dy;
  rm_params p;
  rm_grads g;
  void *y, *dx;
  char* ws;  // the forward's saved regions (layout offsets from ws)
  char* sc;  // the backward's scratch (layout offsets from sc)
  WsLayout L;
  int B, T, D, H;
};

// a value rounded to the storage type and read back (the value every later
// step sees)
template <typename ST>
__device__ __forceinline__ float rnd(float v) {
  return to_f32(from_f32<ST>(v));
}

// 8 consecutive storage elements at a 16-byte aligned address, as fp32
__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0], b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
template <typename ST>
__device__ __forceinline__ void ld8(const ST* p, float (&v)[8]) {
  const uint4 q = *reinterpret_cast<const uint4*>(p);
  const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = lo16<ST>(w[i]);
    v[2 * i + 1] = hi16<ST>(w[i]);
  }
}

// p[i], p[i+1] = v0, v1 (storage type, round to nearest even) with one store;
// the caller guarantees p + i is aligned to two elements
template <typename ST>
__device__ __forceinline__ void st2(ST* p, long i, float v0, float v1) {
  if constexpr (std::is_same<ST, float>::value) *reinterpret_cast<float2*>(p + i) = make_float2(v0, v1);
  else *reinterpret_cast<uint32_t*>(p + i) = pack16x2<ST>(v0, v1);
}

// rows r = 0 .. nrows-1 of a weight gradient g (row length len, g + r len + n):
// g[r][n] = sum_k a(k, r) b(k, n) over the token's rows k < B.  One or, for
// 16-bit storage with len even and g aligned to two elements, two consecutive
// columns per thread (one 4-byte store for both instead of two 2-byte ones),
// rows strided over the threads; fixed order k = 0 .. B-1, so either form
// gives the same bits.
template <typename ST, typename FA, typename FB>
__device__ __forceinline__ void weight_grad(ST* g, int nrows, int len, int B, FA a, FB b) {
  const int tid = threadIdx.x;
  const bool pairs = sizeof(ST) == 2 && (len % 2) == 0 && (reinterpret_cast<uintptr_t>(g) % (2 * sizeof(ST))) == 0;
  const int w = pairs ? 2 : 1, ncol = len / w;  // column groups per row
  const int per = FWD_THREADS / ncol;           // rows per pass (ncol <= FWD_THREADS)
  if (tid >= per * ncol) return;
  const int n = (tid % ncol) * w;
  for (int r = tid / ncol; r < nrows; r += per) {
    float s0 = 0.f, s1 = 0.f;
    for (int k = 0; k < B; ++k) {
      const float ak = a(k, r);
      s0 = fmaf(ak, b(k, n), s0);
      if (pairs) s1 = fmaf(ak, b(k, n + 1), s1);
    }
    if (pairs) st2(g, (long)r * len + n, s0, s1);
    else st(g, (long)r * len + n, s0);
  }
}

// mean and rstd of a row held as v[q] at columns lane + 64 q (< n), two passes
template <int Q>
__device__ __forceinline__ void row_stats(const float (&v)[Q], int n, float eps, float& mean, float& rstd) {
  const int lane = threadIdx.x & 63;
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (lane + 64 * q < n) s += v[q];
  mean = wave_sum(s) / (float)n;
  float s2 = 0.f;
#pragma unroll
  for (int q = 0; q < Q; ++q)
    if (lane + 64 * q < n) {
      const float d = v[q] - mean;
      s2 += d * d;
    }
  rstd = rsqrtf(wave_sum(s2) / (float)n + eps);
}

// NB: rows accumulated per output in the contraction loops, a power of two >= B
template <typename ST, int NB>
__global__ __launch_bounds__(FWD_THREADS) void k_small_fwd(SmallArgs a) {
  __shared__ float s_mu0[SB * 64], s_rs0[SB * 64];
  __shared__ float s_h1[SB][SD];      // out1, later r2
  __shared__ float s_z[SB][2 * SH];  // Z, later the output projection's partial sums
  __shared__ float s_hid[SB][SH];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B, T = a.T, D = a.D, H = a.H, S = D / T;
  const long NR = (long)B * T;
  const ST* x = reinterpret_cast<const ST*>(a.x);
  float* stats = reinterpret_cast<float*>(a.ws + a.L.stats);
  const auto P = [&](const void* q) { return reinterpret_cast<const ST*>(q); };

  // 1. norm0 statistics of every row (b, j)
  for (int r = wave; r < B * T; r += SB) {
    float v[QD];
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      v[q] = c < D ? ld(x, (long)r * D + c) : 0.f;
    }
    float mu, rs;
    row_stats(v, D, EPS_OUTER, mu, rs);
    if (lane == 0) {
      s_mu0[r] = mu;
      s_rs0[r] = rs;
      if (t == 0) {
        stats[ST_MU0 * NR + r] = mu;
        stats[ST_RS0 * NR + r] = rs;
      }
    }
  }
  __syncthreads();

  // 2. out1 row (b, t): the token-mix gather, the residual, norm1
  const int b = wave;
  const long row = (long)b * T + t;
  if (b < B) {
    float r1[QD];
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      r1[q] = 0.f;
      if (c < D) {
        int j, sc;
        tm_source(t, c, S, j, sc);  // source row j, column sc of sample b
        const int src = b * T + j;
        r1[q] = mixed_residual(ld(x, (long)src * D + sc), s_rs0[src], -s_mu0[src] * s_rs0[src], ld(P(a.p.ln0_g), sc),
                               ld(P(a.p.ln0_b), sc), ld(x, row * D + c));
      }
    }
    float mu, rs;
    row_stats(r1, D, EPS_OUTER, mu, rs);
    ST* h1 = reinterpret_cast<ST*>(a.ws + a.L.h1);
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) {
        const float h = fmaf(fmaf(r1[q], rs, -mu * rs), ld(P(a.p.ln1_g), c), ld(P(a.p.ln1_b), c));
        st(h1, row * D + c, h);
        s_h1[b][c] = rnd<ST>(h);
      }
    }
    if (lane == 0) {
      stats[ST_MU1 * NR + row] = mu;
      stats[ST_RS1 * NR + row] = rs;
    }
  }
  __syncthreads();

  // 3. Z[b, t, n] = out1[b, t] . w1[t][:, n] + b1[t, n]
  {
    const ST* w1 = P(a.p.w1) + (long)t * D * 2 * H;
    ST* z = reinterpret_cast<ST*>(a.ws + a.L.z);
    for (int n = tid; n < 2 * H; n += FWD_THREADS) {
      float acc[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) acc[k] = 0.f;
      for (int c = 0; c < D; ++c) {
        const float w = ld(w1, (long)c * 2 * H + n);
#pragma unroll
        for (int k = 0; k < NB; ++k) acc[k] = fmaf(s_h1[k][c], w, acc[k]);  // rows past B: unused
      }
      const float bias = ld(P(a.p.b1), (long)t * 2 * H + n);
      for (int k = 0; k < B; ++k) {
        const float v = acc[k] + bias;
        st(z, ((long)k * T + t) * 2 * H + n, v);
        s_z[k][n] = rnd<ST>(v);
      }
    }
  }
  __syncthreads();

  // 4. hidden row (b, t) from the stored Z
  if (b < B) {
    float u[QH], g[QH];
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      const int h = lane + 64 * q;
      u[q] = h < H ? s_z[b][h] : 0.f;
      g[q] = h < H ? s_z[b][H + h] : 0.f;
    }
    float mux, rsx, mug, rsg;
    row_stats(u, H, EPS_INNER, mux, rsx);
    row_stats(g, H, EPS_INNER, mug, rsg);
    ST* hid = reinterpret_cast<ST*>(a.ws + a.L.hid);
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      const int h = lane + 64 * q;
      if (h < H) {
        const float ux = fmaf(fmaf(u[q], rsx, -mux * rsx), ld(P(a.p.lnx_g), h), ld(P(a.p.lnx_b), h));
        const float ug = fmaf(fmaf(g[q], rsg, -mug * rsg), ld(P(a.p.lng_g), h), ld(P(a.p.lng_b), h));
        const float o = ux * (ug * sigmoidf_(ug));
        st(hid, row * H + h, o);
        s_hid[b][h] = rnd<ST>(o);
      }
    }
    if (lane == 0) {
      stats[ST_MUX * NR + row] = mux;
      stats[ST_RSX * NR + row] = rsx;
      stats[ST_MUG * NR + row] = mug;
      stats[ST_RSG * NR + row] = rsg;
    }
  }
  __syncthreads();

  // 5. r2 = (hidden . wout[t] + bout[t]) + out1.  The threads form
  // FWD_THREADS / D groups of D (one column n each); group g sums its slice of
  // the h range (coalesced reads of wout rows) into the Z area, no longer
  // needed, and the slices are added in group order.  r2 replaces out1 in
  // s_h1: each element's residual is read and overwritten by the same thread.
  {
    const int NG = FWD_THREADS / D;
    const ST* wo = P(a.p.wout) + (long)t * H * D;
    float* part = &s_z[0][0];  // [NG][SB][D], NG * D <= FWD_THREADS
    const int n = tid % D, grp = tid / D, hs = (H + NG - 1) / NG;
    if (grp < NG) {
      const int h0 = grp * hs, h1 = min(H, h0 + hs);
      float acc[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) acc[k] = 0.f;
      for (int h = h0; h < h1; ++h) {
        const float w = ld(wo, (long)h * D + n);
#pragma unroll
        for (int k = 0; k < NB; ++k) acc[k] = fmaf(s_hid[k][h], w, acc[k]);
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) part[(grp * SB + k) * D + n] = acc[k];
    }
    __syncthreads();
    ST* r2 = reinterpret_cast<ST*>(a.ws + a.L.r2);
    for (int i = tid; i < B * D; i += FWD_THREADS) {
      const int k = i / D, c = i - k * D;
      float sum = 0.f;
      for (int g = 0; g < NG; ++g) sum += part[(g * SB + k) * D + c];
      const float v = (sum + ld(P(a.p.bout), (long)t * D + c)) + s_h1[k][c];
      st(r2, ((long)k * T + t) * D + c, v);
      s_h1[k][c] = rnd<ST>(v);
    }
  }
  __syncthreads();

  // 6. y = norm2(r2)
  if (b < B) {
    float v[QD];
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      v[q] = c < D ? s_h1[b][c] : 0.f;
    }
    float mu, rs;
    row_stats(v, D, EPS_OUTER, mu, rs);
    ST* y = reinterpret_cast<ST*>(a.y);
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) st(y, row * D + c, (v[q] - mu) * rs * ld(P(a.p.ln2_g), c) + ld(P(a.p.ln2_b), c));
    }
    if (lane == 0) {
      stats[ST_MU2 * NR + row] = mu;
      stats[ST_RS2 * NR + row] = rs;
    }
  }
}

// Column sums over the token's rows b < B of values each wave (row b) holds
// at columns lane + 64 q (< n): through LDS scratch tmp[SB][SH], fixed order
// b = 0 .. B-1; the result goes to out[c] (fp32) or, when `grad` is set, to
// grad[c] rounded to the storage type.
template <typename ST, int Q>
__device__ __forceinline__ void column_sum(const float (&v)[Q], int n, int B, float (*tmp)[SH], float* out, ST* grad) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  __syncthreads();  // tmp is free
  if (wave < B) {
#pragma unroll
    for (int q = 0; q < Q; ++q)
      if (lane + 64 * q < n) tmp[wave][lane + 64 * q] = v[q];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < n; c += blockDim.x) {
    float s = 0.f;
    for (int k = 0; k < B; ++k) s += tmp[k][c];
    if (grad) st(grad, c, s);
    else out[c] = s;
  }
}

template <typename ST, int NB>
__global__ __launch_bounds__(FWD_THREADS) void k_small_bwd_tok(SmallArgs a) {
  __shared__ float s_do2[SB][SD];
  __shared__ float s_hid[SB][SH];   // hidden, later d hidden
  __shared__ float s_z[SB][2 * SH];  // Z, later dZ
  __shared__ float s_h1[SB][SD];
  __shared__ float s_dh1[SB][SD];
  // column-sum scratch ([SB][SH]) and the d out1 partial sums ([NG][SB][D], NG * D <= FWD_THREADS)
  __shared__ float s_tmp_buf[TMP_FLOATS];
  float(*const s_tmp)[SH] = reinterpret_cast<float(*)[SH]>(s_tmp_buf);
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.B, T = a.T, D = a.D, H = a.H, S = D / T;
  const long NR = (long)B * T;
  const auto P = [&](const void* q) { return reinterpret_cast<const ST*>(q); };
  const ST* x = P(a.x);
  const float* stats = reinterpret_cast<const float*>(a.ws + a.L.stats);
  float* p_ln2 = reinterpret_cast<float*>(a.sc + a.L.p_ln2);    // [2][T][D]: dgamma2, dbeta2
  float* p_gate = reinterpret_cast<float*>(a.sc + a.L.p_gate);  // [4][T][H]: dgamma_x, dbeta_x, dgamma_g, dbeta_g
  // [2][T][D]: dgamma1, dbeta1, in the dZ region (dZ stays in LDS here; its
  // B*T*2H storage elements hold 2*T*D floats for every B >= 1, k >= 2)
  float* p_ln1 = reinterpret_cast<float*>(a.sc + a.L.dz);
  const int b = wave;
  const long row = (long)b * T + t;

  // saved state of the token's rows
  for (int i = tid; i < B * 2 * H; i += FWD_THREADS) {
    const int k = i / (2 * H), n = i - k * 2 * H;
    s_z[k][n] = ld(P(a.ws + a.L.z), ((long)k * T + t) * 2 * H + n);
  }
  for (int i = tid; i < B * H; i += FWD_THREADS) {
    const int k = i / H, n = i - k * H;
    s_hid[k][n] = ld(P(a.ws + a.L.hid), ((long)k * T + t) * H + n);
  }
  for (int i = tid; i < B * D; i += FWD_THREADS) {
    const int k = i / D, n = i - k * D;
    s_h1[k][n] = ld(P(a.ws + a.L.h1), ((long)k * T + t) * D + n);
  }

  // 1. norm2 backward: d out2 = rs (dn - mean(dn) - n2 mean(dn n2)), dn = dy gamma2
  float pg[QD], pb[QD], po[QD];
  {
    const ST* dy = P(a.dy);
    const ST* r2 = P(a.ws + a.L.r2);
    const float mu = b < B ? stats[ST_MU2 * NR + row] : 0.f, rs = b < B ? stats[ST_RS2 * NR + row] : 0.f;
    float n2[QD], d[QD], dn[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      const bool ok = b < B && c < D;
      n2[q] = ok ? (ld(r2, row * D + c) - mu) * rs : 0.f;
      d[q] = ok ? ld(dy, row * D + c) : 0.f;
      dn[q] = ok ? d[q] * ld(P(a.p.ln2_g), c) : 0.f;
      s1 += dn[q];
      s2 += dn[q] * n2[q];
    }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      const float o = rs * (dn[q] - m1 - n2[q] * m2);
      pg[q] = d[q] * n2[q];
      pb[q] = d[q];
      po[q] = o;
      if (b < B && c < D) s_do2[b][c] = rnd<ST>(o);
    }
  }
  column_sum<ST, QD>(pg, D, B, s_tmp, p_ln2 + (long)t * D, (ST*)nullptr);
  column_sum<ST, QD>(pb, D, B, s_tmp, p_ln2 + (long)(T + t) * D, (ST*)nullptr);
  column_sum<ST, QD>(po, D, B, s_tmp, nullptr, reinterpret_cast<ST*>(a.g.bout) + (long)t * D);
  __syncthreads();

  // 2. dwout[t][h][n] = sum_b hidden[b,h] d out2[b,n]
  weight_grad(reinterpret_cast<ST*>(a.g.wout) + (long)t * H * D, H, D, B,
              [&](int k, int h) { return s_hid[k][h]; }, [&](int k, int n) { return s_do2[k][n]; });
  // 3. d hidden[b,h] = d out2[b] . wout[t][h], one thread per h, into s_tmp
  // until every thread has read hidden
  {
    const ST* wo = P(a.p.wout) + (long)t * H * D;
    for (int h = tid; h < H; h += FWD_THREADS) {
      float acc[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) acc[k] = 0.f;
      for (int n = 0; n < D; ++n) {
        const float w = ld(wo, (long)h * D + n);
#pragma unroll
        for (int k = 0; k < NB; ++k) acc[k] = fmaf(s_do2[k][n], w, acc[k]);
      }
      for (int k = 0; k < B; ++k) s_tmp[k][h] = rnd<ST>(acc[k]);
    }
  }
  __syncthreads();
  for (int i = tid; i < B * H; i += FWD_THREADS) {
    const int k = i / H, h = i - k * H;
    s_hid[k][h] = s_tmp[k][h];
  }
  __syncthreads();

  // 4. gate / SiLU / inner LayerNorm backward of row (b, t) -> dZ (into s_z)
  {
    float ax[QH], bx[QH], ag[QH], bg[QH], au[QH], agv[QH];
    const float mux = b < B ? stats[ST_MUX * NR + row] : 0.f, rsx = b < B ? stats[ST_RSX * NR + row] : 0.f;
    const float mug = b < B ? stats[ST_MUG * NR + row] : 0.f, rsg = b < B ? stats[ST_RSG * NR + row] : 0.f;
    float nx[QH], ng[QH], dnx[QH], dng[QH];
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      const int h = lane + 64 * q;
      const bool ok = b < B && h < H;
      const float u = ok ? s_z[b][h] : 0.f, g = ok ? s_z[b][H + h] : 0.f, dh = ok ? s_hid[b][h] : 0.f;
      const float cgx = ok ? ld(P(a.p.lnx_g), h) : 0.f, cbx = ok ? ld(P(a.p.lnx_b), h) : 0.f;
      const float cgg = ok ? ld(P(a.p.lng_g), h) : 0.f, cbg = ok ? ld(P(a.p.lng_b), h) : 0.f;
      nx[q] = fmaf(u, rsx, -mux * rsx);
      ng[q] = fmaf(g, rsg, -mug * rsg);
      const float ux = nx[q] * cgx + cbx, ug = ng[q] * cgg + cbg;
      const float sg = sigmoidf_(ug), us = ug * sg;
      const float dux = dh * us;
      const float dug = (dh * ux) * fmaf(us, 1.f - sg, sg);
      dnx[q] = dux * cgx;
      dng[q] = dug * cgg;
      s[0] += dnx[q];
      s[1] += dnx[q] * nx[q];
      s[2] += dng[q];
      s[3] += dng[q] * ng[q];
      ax[q] = dux * nx[q];
      bx[q] = dux;
      ag[q] = dug * ng[q];
      bg[q] = dug;
    }
    const float m1 = wave_sum(s[0]) / (float)H, m2 = wave_sum(s[1]) / (float)H;
    const float m3 = wave_sum(s[2]) / (float)H, m4 = wave_sum(s[3]) / (float)H;
#pragma unroll
    for (int q = 0; q < QH; ++q) {
      const int h = lane + 64 * q;
      au[q] = rsx * (dnx[q] - m1 - nx[q] * m2);
      agv[q] = rsg * (dng[q] - m3 - ng[q] * m4);
      if (b < B && h < H) {
        s_z[b][h] = rnd<ST>(au[q]);
        s_z[b][H + h] = rnd<ST>(agv[q]);
      }
    }
    column_sum<ST, QH>(ax, H, B, s_tmp, p_gate + (long)t * H, (ST*)nullptr);
    column_sum<ST, QH>(bx, H, B, s_tmp, p_gate + (long)(T + t) * H, (ST*)nullptr);
    column_sum<ST, QH>(ag, H, B, s_tmp, p_gate + (long)(2 * T + t) * H, (ST*)nullptr);
    column_sum<ST, QH>(bg, H, B, s_tmp, p_gate + (long)(3 * T + t) * H, (ST*)nullptr);
    ST* db1 = reinterpret_cast<ST*>(a.g.b1) + (long)t * 2 * H;
    column_sum<ST, QH>(au, H, B, s_tmp, nullptr, db1);
    column_sum<ST, QH>(agv, H, B, s_tmp, nullptr, db1 + H);
  }
  __syncthreads();

  // 5. dw1[t][c][n] = sum_b out1[b,c] dZ[b,n]
  static_assert(2 * SH <= FWD_THREADS && SD <= FWD_THREADS, "one pass covers every column of a weight gradient");
  weight_grad(reinterpret_cast<ST*>(a.g.w1) + (long)t * D * 2 * H, D, 2 * H, B,
              [&](int k, int c) { return s_h1[k][c]; }, [&](int k, int n) { return s_z[k][n]; });
  // 6. d out1[b,c] = dZ[b] . w1[t][c] + d out2[b,c].  The threads form
  // FWD_THREADS / D groups of D (one column c each); group g sums its slice
  // of the n range into s_tmp (free here) and the slices are added in group
  // order.
  {
    const int NG = FWD_THREADS / D;
    const ST* w1 = P(a.p.w1) + (long)t * D * 2 * H;
    float* part = s_tmp_buf;  // [NG][SB][D], NG * D <= FWD_THREADS
    const int c = tid % D, grp = tid / D, ns = (2 * H + NG - 1) / NG;
    // loads of 8 consecutive elements when every slice boundary and the row
    // length are multiples of 8 (each load then stays inside its slice) and
    // the rows start 16-byte aligned
    const bool vec8 = (ns % 8) == 0 && ((2 * H) % 8) == 0 && ((2 * H * (int)sizeof(ST)) % 16) == 0 &&
                      (reinterpret_cast<uintptr_t>(w1) & 15) == 0;
    if (grp < NG) {
      const int n0 = grp * ns, n1 = min(2 * H, n0 + ns);
      float acc[NB];
#pragma unroll
      for (int k = 0; k < NB; ++k) acc[k] = 0.f;
      const ST* wr = w1 + (long)c * 2 * H;
      if (vec8) {
        for (int n = n0; n < n1; n += 8) {
          float w[8];
          ld8(wr + n, w);
#pragma unroll
          for (int e = 0; e < 8; ++e)
#pragma unroll
            for (int k = 0; k < NB; ++k) acc[k] = fmaf(s_z[k][n + e], w[e], acc[k]);
        }
      } else {
        for (int n = n0; n < n1; ++n) {
          const float w = ld(wr, n);
#pragma unroll
          for (int k = 0; k < NB; ++k) acc[k] = fmaf(s_z[k][n], w, acc[k]);
        }
      }
#pragma unroll
      for (int k = 0; k < NB; ++k) part[(grp * SB + k) * D + c] = acc[k];
    }
    __syncthreads();
    for (int i = tid; i < B * D; i += FWD_THREADS) {
      const int k = i / D, cc = i - k * D;
      float sum = 0.f;
      for (int g = 0; g < NG; ++g) sum += part[(g * SB + k) * D + cc];
      s_dh1[k][cc] = rnd<ST>(sum + s_do2[k][cc]);
    }
  }
  __syncthreads();

  // 7. norm1 backward of row (b, t): r1 recomputed through the token-mix gather -> d r1
  {
    const float mu1 = b < B ? stats[ST_MU1 * NR + row] : 0.f, rs1 = b < B ? stats[ST_RS1 * NR + row] : 0.f;
    float n1[QD], dh[QD], dn[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      const bool ok = b < B && c < D;
      n1[q] = dh[q] = dn[q] = 0.f;
      if (ok) {
        int j, sc;
        tm_source(t, c, S, j, sc);
        const long src = (long)b * T + j;
        const float rs0 = stats[ST_RS0 * NR + src], mu0 = stats[ST_MU0 * NR + src];
        const float r1 = mixed_residual(ld(x, src * D + sc), rs0, -mu0 * rs0, ld(P(a.p.ln0_g), sc),
                                        ld(P(a.p.ln0_b), sc), ld(x, row * D + c));
        n1[q] = (r1 - mu1) * rs1;
        dh[q] = s_dh1[b][c];
        dn[q] = dh[q] * ld(P(a.p.ln1_g), c);
      }
      s1 += dn[q];
      s2 += dn[q] * n1[q];
    }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
    ST* dr1 = reinterpret_cast<ST*>(a.sc + a.L.dr1);
    float pa[QD];
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (b < B && c < D) st(dr1, row * D + c, rs1 * (dn[q] - m1 - n1[q] * m2));
      pa[q] = dh[q] * n1[q];
    }
    column_sum<ST, QD>(pa, D, B, s_tmp, p_ln1 + (long)t * D, (ST*)nullptr);
    column_sum<ST, QD>(dh, D, B, s_tmp, p_ln1 + (long)(T + t) * D, (ST*)nullptr);
  }
}

constexpr int FIN_THREADS = 1024;

// The token-mix adjoint and the norm0 backward of every row, and the affine
// gradients summed over the tokens (one workgroup).
template <typename ST>
__global__ __launch_bounds__(FIN_THREADS) void k_small_bwd_fin(SmallArgs a) {
  __shared__ float s_part[FIN_THREADS / 64][SD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, nw = FIN_THREADS / 64;
  const int B = a.B, T = a.T, D = a.D, H = a.H, S = D / T;
  const long NR = (long)B * T;
  const auto P = [&](const void* q) { return reinterpret_cast<const ST*>(q); };
  const ST* x = P(a.x);
  const ST* dr1 = P(a.sc + a.L.dr1);
  const float* stats = reinterpret_cast<const float*>(a.ws + a.L.stats);
  ST* dx = reinterpret_cast<ST*>(a.dx);

  // norm0 backward: dx[r] = d r1[r] + rs0 (dn - mean(dn) - n0 mean(dn n0)),
  // dn = da0 gamma0, da0 = token_mix(d r1) (the involution's own gather)
  float pa[QD], pb[QD];
#pragma unroll
  for (int q = 0; q < QD; ++q) pa[q] = pb[q] = 0.f;
  for (int r = wave; r < B * T; r += nw) {
    const int b = r / T, j = r - b * T;
    const float mu = stats[ST_MU0 * NR + r], rs = stats[ST_RS0 * NR + r];
    float n0[QD], da[QD], dn[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      n0[q] = da[q] = dn[q] = 0.f;
      if (c < D) {
        int i, sc;
        tm_source(j, c, S, i, sc);
        da[q] = ld(dr1, ((long)b * T + i) * D + sc);
        n0[q] = (ld(x, (long)r * D + c) - mu) * rs;
        dn[q] = da[q] * ld(P(a.p.ln0_g), c);
      }
      s1 += dn[q];
      s2 += dn[q] * n0[q];
    }
    const float m1 = wave_sum(s1) / (float)D, m2 = wave_sum(s2) / (float)D;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) st(dx, (long)r * D + c, ld(dr1, (long)r * D + c) + rs * (dn[q] - m1 - n0[q] * m2));
      pa[q] += da[q] * n0[q];
      pb[q] += da[q];
    }
  }
  // the waves' column partials added in wave order
  for (int pass = 0; pass < 2; ++pass) {
    __syncthreads();
#pragma unroll
    for (int q = 0; q < QD; ++q)
      if (lane + 64 * q < D) s_part[wave][lane + 64 * q] = pass == 0 ? pa[q] : pb[q];
    __syncthreads();
    ST* out = reinterpret_cast<ST*>(pass == 0 ? a.g.ln0_g : a.g.ln0_b);
    for (int c = tid; c < D; c += FIN_THREADS) {
      float s = 0.f;
      for (int w = 0; w < nw; ++w) s += s_part[w][c];
      st(out, c, s);
    }
  }

  // per-token partials summed over t in order
  const float* p_ln2 = reinterpret_cast<const float*>(a.sc + a.L.p_ln2);
  const float* p_gate = reinterpret_cast<const float*>(a.sc + a.L.p_gate);
  const float* p_ln1 = reinterpret_cast<const float*>(a.sc + a.L.dz);
  // every (job, column) pair on its own thread; the token rows are loaded
  // eight at a time before they are added in order
  const int ncol = 4 * D + 4 * H;
  for (int i = tid; i < ncol; i += FIN_THREADS) {
    // jobs 0-3: dgamma2, dbeta2, dgamma1, dbeta1 (D columns); 4-7: dgamma_x,
    // dbeta_x, dgamma_g, dbeta_g (H columns); partials [job][T][columns]
    const int k = i < 4 * D ? i / D : 4 + (i - 4 * D) / H;
    const int c = i < 4 * D ? i - k * D : (i - 4 * D) - (k - 4) * H;
    const long stride = k < 4 ? D : H;
    const float* pp = (k < 2 ? p_ln2 + (long)k * T * D
                             : k < 4 ? p_ln1 + (long)(k - 2) * T * D : p_gate + (long)(k - 4) * T * H) + c;
    void* outp = k == 0 ? a.g.ln2_g : k == 1 ? a.g.ln2_b : k == 2 ? a.g.ln1_g : k == 3 ? a.g.ln1_b
               : k == 4 ? a.g.lnx_g : k == 5 ? a.g.lnx_b : k == 6 ? a.g.lng_g : a.g.lng_b;
    float s = 0.f;
    int t = 0;
    for (; t + 8 <= T; t += 8) {
      float v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = pp[(long)(t + u) * stride];
#pragma unroll
      for (int u = 0; u < 8; ++u) s += v[u];
    }
    for (; t < T; ++t) s += pp[(long)t * stride];
    st(reinterpret_cast<ST*>(outp), c, s);
  }
}

// the kernel instance for the batch: rows accumulated = B rounded up to 1, 2, 4 or 8
template <typename ST>
void launch_fwd_rows(const SmallArgs& a, hipStream_t s) {
  if (a.B <= 1) hipLaunchKernelGGL((k_small_fwd<ST, 1>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else if (a.B <= 2) hipLaunchKernelGGL((k_small_fwd<ST, 2>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else if (a.B <= 4) hipLaunchKernelGGL((k_small_fwd<ST, 4>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else hipLaunchKernelGGL((k_small_fwd<ST, SB>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
}
template <typename ST>
void launch_bwd_rows(const SmallArgs& a, hipStream_t s) {
  if (a.B <= 1) hipLaunchKernelGGL((k_small_bwd_tok<ST, 1>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else if (a.B <= 2) hipLaunchKernelGGL((k_small_bwd_tok<ST, 2>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else if (a.B <= 4) hipLaunchKernelGGL((k_small_bwd_tok<ST, 4>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
  else hipLaunchKernelGGL((k_small_bwd_tok<ST, SB>), dim3(a.T), dim3(FWD_THREADS), 0, s, a);
}

template <typename ST>
hipError_t small_fwd_t(const SmallArgs& a, hipStream_t s) {
  prof_begin(KID_SMALL_FWD, s);
  launch_fwd_rows<ST>(a, s);
  prof_end(KID_SMALL_FWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t small_bwd_t(const SmallArgs& a, hipStream_t s) {
  prof_begin(KID_SMALL_BWD, s);
  launch_bwd_rows<ST>(a, s);
  prof_end(KID_SMALL_BWD, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  prof_begin(KID_SMALL_FIN, s);
  hipLaunchKernelGGL(k_small_bwd_fin<ST>, dim3(1), dim3(FIN_THREADS), 0, s, a);
  prof_end(KID_SMALL_FIN, s);
  return hipGetLastError();
}

SmallArgs small_args(const rm_dims& d, const rm_params& p, const void* x, void* ws, const WsLayout& L) {
  SmallArgs a{};
  a.x = x;
  a.p = p;
  a.ws = reinterpret_cast<char*>(ws);
  a.L = L;
  a.B = d.B;
  a.T = d.T;
  a.D = d.D;
  a.H = d.k * d.D;
  return a;
}

}  // namespace

bool small_supported(const rm_dims& d) {
  return dims_valid(d) && d.B <= SMALL_MAX_B && d.D <= SMALL_MAX_D && d.k * d.D <= SMALL_MAX_H;
}

hipError_t launch_small_fwd(const rm_dims& d, const rm_params& p, const void* x, void* y, void* ws,
                            const WsLayout& L, hipStream_t s) {
  SmallArgs a = small_args(d, p, x, ws, L);
  a.y = y;
  if (d.dtype == RM_BF16) return small_fwd_t<bf16_t>(a, s);
  if (d.dtype == RM_F16) return small_fwd_t<f16_t>(a, s);
  return small_fwd_t<float>(a, s);
}

hipError_t launch_small_bwd(const rm_dims& d, const rm_params& p, const void* x, const void* dy, void* ws, void* sc,
                            const WsLayout& L, void* dx, const rm_grads& g, hipStream_t s) {
  SmallArgs a = small_args(d, p, x, ws, L);
  a.sc = reinterpret_cast<char*>(sc);
  a.dy = dy;
  a.dx = dx;
  a.g = g;
  if (d.dtype == RM_BF16) return small_bwd_t<bf16_t>(a, s);
  if (d.dtype == RM_F16) return small_bwd_t<f16_t>(a, s);
  return small_bwd_t<float>(a, s);
}

}  // namespace rm
