// Row-wise kernels of the RankMixerBlock (LayerNorms, token mixing, gating,
// and their backward), for gfx950 wave64.  All of them are HBM-bandwidth
// bound: each reads and writes its rows once and keeps statistics in fp32.
//
// Page 1 of "Subgraph-fusion-based Mega-kernel Generation", section "Exact
// computation", defines what they compute: outer LayerNorms (eps 1e-3),
// token mixing (swap the two T axes of a [B,T,T,D/T] view), the residual
// adds, and the gated inner LayerNorms (eps 1e-5) of the dense subgraph.
#include "rm_common.h"
#include "rm_internal.h"

namespace rm {

namespace {

constexpr float EPS_OUTER = 1e-3f;
constexpr float EPS_INNER = 1e-5f;
constexpr int QD = 1280 / 64;   // columns per lane when one wave owns a D-wide row (D <= 1280)
constexpr int QH = 3840 / 256;  // columns per thread when 256 threads own an H-wide row (H <= 3840)
constexpr int QG = 4096 / 512;  // columns per thread when 512 threads own an H-wide row

template <typename ST>
__host__ __device__ __forceinline__ const ST* cptr(const void* p) { return reinterpret_cast<const ST*>(p); }

// ---------------------------------------------------------------------------
// Forward prologue, one workgroup per sample b:
//   a0 = norm0(x[b]);  r1 = token_mix(a0) + x[b];  out1 = norm1(r1).
// The token-mixed a0 is never stored: row i of token_mix(a0) gathers column
// block i of every token j, recomputed from x and norm0's statistics.
template <typename ST>
__global__ __launch_bounds__(256) void k_prologue(const ST* __restrict__ x, const ST* __restrict__ g0,
                                                  const ST* __restrict__ be0, const ST* __restrict__ g1,
                                                  const ST* __restrict__ be1, ST* __restrict__ h1,
                                                  float* __restrict__ stats, int B, int T, int D) {
  __shared__ float s_mu0[64], s_rs0[64];
  const int b = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long N = (long)B * T;
  const long base = (long)b * T * D;
  const int S = D / T;
  const float invD = 1.0f / (float)D;

  for (int j = wave; j < T; j += 4) {
    float v[QD];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      v[q] = (c < D) ? ld(x, base + (long)j * D + c) : 0.f;
      s += v[q];
    }
    const float mean = wave_sum(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      const float dd = (c < D) ? v[q] - mean : 0.f;
      s2 += dd * dd;
    }
    const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
    if (lane == 0) {
      s_mu0[j] = mean;
      s_rs0[j] = rstd;
      stats[ST_MU0 * N + (long)b * T + j] = mean;
      stats[ST_RS0 * N + (long)b * T + j] = rstd;
    }
  }
  __syncthreads();

  for (int i = wave; i < T; i += 4) {
    float r[QD];
    float s = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      float v = 0.f;
      if (c < D) {
        int j, sc;
        tm_source(i, c, S, j, sc);
        const float a0 = (ld(x, base + (long)j * D + sc) - s_mu0[j]) * s_rs0[j] * ld(g0, sc) + ld(be0, sc);
        v = a0 + ld(x, base + (long)i * D + c);
      }
      r[q] = v;
      s += v;
    }
    const float mean = wave_sum(s) * invD;
    float s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      const float dd = (c < D) ? r[q] - mean : 0.f;
      s2 += dd * dd;
    }
    const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) st(h1, base + (long)i * D + c, (r[q] - mean) * rstd * ld(g1, c) + ld(be1, c));
    }
    if (lane == 0) {
      stats[ST_MU1 * N + (long)b * T + i] = mean;
      stats[ST_RS1 * N + (long)b * T + i] = rstd;
    }
  }
}

// ---------------------------------------------------------------------------
// hidden = LN_x(U) * silu(LN_gate(G)) for one row of Z per workgroup.
// The statistics are taken from the stored (rounded) Z so that the backward,
// which re-reads Z, sees the same normalised values.
template <typename ST>
__global__ __launch_bounds__(256) void k_gate_fwd(const ST* __restrict__ Z, const ST* __restrict__ gx,
                                                  const ST* __restrict__ bx, const ST* __restrict__ gg,
                                                  const ST* __restrict__ bg, ST* __restrict__ hid,
                                                  float* __restrict__ stats, long N, int H) {
  __shared__ float red[8];
  const long row = blockIdx.x;
  const int tid = threadIdx.x;
  const ST* z = Z + row * 2 * H;
  const float invH = 1.0f / (float)H;
  float u[QH], g[QH];
  float s[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < QH; ++q) {
    const int h = tid + 256 * q;
    u[q] = (h < H) ? ld(z, h) : 0.f;
    g[q] = (h < H) ? ld(z, H + h) : 0.f;
    s[0] += u[q];
    s[1] += g[q];
  }
  block_sum256(s, red);
  const float mu_u = s[0] * invH, mu_g = s[1] * invH;
  float s2[2] = {0.f, 0.f};
#pragma unroll
  for (int q = 0; q < QH; ++q) {
    const int h = tid + 256 * q;
    if (h < H) {
      const float du = u[q] - mu_u, dg = g[q] - mu_g;
      s2[0] += du * du;
      s2[1] += dg * dg;
    }
  }
  block_sum256(s2, red);
  const float rs_u = rsqrtf(s2[0] * invH + EPS_INNER);
  const float rs_g = rsqrtf(s2[1] * invH + EPS_INNER);
#pragma unroll
  for (int q = 0; q < QH; ++q) {
    const int h = tid + 256 * q;
    if (h < H) {
      const float ux = (u[q] - mu_u) * rs_u * ld(gx, h) + ld(bx, h);
      const float ug = (g[q] - mu_g) * rs_g * ld(gg, h) + ld(bg, h);
      st(hid, row * H + h, ux * (ug * sigmoidf_(ug)));
    }
  }
  if (tid == 0) {
    stats[ST_MUX * N + row] = mu_u;
    stats[ST_RSX * N + row] = rs_u;
    stats[ST_MUG * N + row] = mu_g;
    stats[ST_RSG * N + row] = rs_g;
  }
}

// ---------------------------------------------------------------------------
// y = norm2(r2), r2 = out1 + out2 kept in fp32.  One wave per row.
template <typename ST>
__global__ __launch_bounds__(256) void k_ln2_fwd(const float* __restrict__ r2, const ST* __restrict__ g2,
                                                 const ST* __restrict__ be2, ST* __restrict__ y,
                                                 float* __restrict__ stats, long N, int D) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long row = (long)blockIdx.x * 4 + wave;
  if (row >= N) return;
  const float invD = 1.0f / (float)D;
  const float* r = r2 + row * D;
  float v[QD];
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < QD; ++q) {
    const int c = lane + 64 * q;
    v[q] = (c < D) ? r[c] : 0.f;
    s += v[q];
  }
  const float mean = wave_sum(s) * invD;
  float s2 = 0.f;
#pragma unroll
  for (int q = 0; q < QD; ++q) {
    const int c = lane + 64 * q;
    const float dd = (c < D) ? v[q] - mean : 0.f;
    s2 += dd * dd;
  }
  const float rstd = rsqrtf(wave_sum(s2) * invD + EPS_OUTER);
#pragma unroll
  for (int q = 0; q < QD; ++q) {
    const int c = lane + 64 * q;
    if (c < D) st(y, row * D + c, (v[q] - mean) * rstd * ld(g2, c) + ld(be2, c));
  }
  if (lane == 0) {
    stats[ST_MU2 * N + row] = mean;
    stats[ST_RS2 * N + row] = rstd;
  }
}

// Adds the four waves' per-column partials (lane-owned columns lane + 64*q)
// in a fixed order through LDS (4 x D floats) and writes them to out[0, D).
__device__ __forceinline__ void combine_waves_store(const float (&acc)[QD], float* lds, float* __restrict__ out,
                                                    int D) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int q = 0; q < QD; ++q) {
    const int c = lane + 64 * q;
    if (c < D) lds[wave * D + c] = acc[q];
  }
  __syncthreads();
  for (int c = threadIdx.x; c < D; c += 256)
    out[c] = (lds[c] + lds[D + c]) + (lds[2 * D + c] + lds[3 * D + c]);
  __syncthreads();
}

// ---------------------------------------------------------------------------
// norm2 backward for the rows (b, t), b in one group of ROWS_PER_GROUP, t fixed:
//   do2 = rstd2 * (dn - mean(dn) - n2 * mean(dn * n2)),  dn = dy * gamma2.
// Per-group partial sums: dgamma2 += dy * n2, dbeta2 += dy, dbout[t] += do2.
template <typename ST>
__global__ __launch_bounds__(256) void k_ln2_bwd(const float* __restrict__ r2, const ST* __restrict__ dy,
                                                 const ST* __restrict__ g2, const float* __restrict__ stats,
                                                 ST* __restrict__ do2, float* __restrict__ part, int B,
                                                 int T, int D, int nb) {
  __shared__ float lds[4 * 1280];
  const int t = blockIdx.x, grp = blockIdx.y;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long N = (long)B * T;
  const float invD = 1.0f / (float)D;
  float pg[QD], pb[QD], po[QD];
#pragma unroll
  for (int q = 0; q < QD; ++q) pg[q] = pb[q] = po[q] = 0.f;
  const int b_end = min(B, (grp + 1) * ROWS_PER_GROUP);
  for (int b = grp * ROWS_PER_GROUP + wave; b < b_end; b += 4) {
    const long row = (long)b * T + t;
    const float mu = stats[ST_MU2 * N + row], rs = stats[ST_RS2 * N + row];
    float n2[QD], dn[QD], dyv[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) {
        n2[q] = (r2[row * D + c] - mu) * rs;
        dyv[q] = ld(dy, row * D + c);
        dn[q] = dyv[q] * ld(g2, c);
      } else {
        n2[q] = dn[q] = dyv[q] = 0.f;
      }
      s1 += dn[q];
      s2 += dn[q] * n2[q];
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) {
        const float v = rs * (dn[q] - m1 - n2[q] * m2);
        st(do2, row * D + c, v);
        pg[q] += dyv[q] * n2[q];
        pb[q] += dyv[q];
        po[q] += v;
      }
    }
  }
  // partial layout: [3][nb][T][D]
  const long blk = (long)nb * T * D;
  float* out = part + ((long)grp * T + t) * D;
  combine_waves_store(pg, lds, out + 0 * blk, D);
  combine_waves_store(pb, lds, out + 1 * blk, D);
  combine_waves_store(po, lds, out + 2 * blk, D);
}

// ---------------------------------------------------------------------------
// Backward of hidden = LN_x(U) * silu(LN_gate(G)) for the rows (b, t) of one
// group, t fixed.  512 threads; thread h owns columns h, h+512, ...
//   ux = LN_x(U), ug = LN_gate(G), s = sigmoid(ug)
//   d ux = dh * ug * s,  d ug = dh * ux * s * (1 + ug * (1 - s))
//   dU = rstd_x * (dnx - mean(dnx) - nx * mean(dnx * nx)),  dnx = d ux * gamma_x   (same for G)
// Per-group partials: dgamma_x, dbeta_x, dgamma_g, dbeta_g and db1[t] (= sum of dZ).
template <typename ST>
__global__ __launch_bounds__(512) void k_gate_bwd(const ST* __restrict__ Z, const ST* __restrict__ dhid,
                                                  const ST* __restrict__ gx, const ST* __restrict__ bx,
                                                  const ST* __restrict__ gg, const ST* __restrict__ bg,
                                                  const float* __restrict__ stats, ST* __restrict__ dZ,
                                                  float* __restrict__ pgate, float* __restrict__ pb1,
                                                  int B, int T, int H, int nb) {
  __shared__ float red[32];
  const int t = blockIdx.x, grp = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long N = (long)B * T;
  const float invH = 1.0f / (float)H;
  float agx[QG], abx[QG], agg[QG], abg[QG], au[QG], ag[QG];
  float cgx[QG], cbx[QG], cgg[QG], cbg[QG];
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    agx[q] = abx[q] = agg[q] = abg[q] = au[q] = ag[q] = 0.f;
    const int h = tid + 512 * q;
    cgx[q] = (h < H) ? ld(gx, h) : 0.f;
    cbx[q] = (h < H) ? ld(bx, h) : 0.f;
    cgg[q] = (h < H) ? ld(gg, h) : 0.f;
    cbg[q] = (h < H) ? ld(bg, h) : 0.f;
  }
  const int b_end = min(B, (grp + 1) * ROWS_PER_GROUP);
  for (int b = grp * ROWS_PER_GROUP; b < b_end; ++b) {
    const long row = (long)b * T + t;
    const float mux = stats[ST_MUX * N + row], rsx = stats[ST_RSX * N + row];
    const float mug = stats[ST_MUG * N + row], rsg = stats[ST_RSG * N + row];
    const ST* z = Z + row * 2 * H;
    float nx[QG], ng[QG], dnx[QG], dng[QG];
    float s[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int h = tid + 512 * q;
      if (h < H) {
        nx[q] = (ld(z, h) - mux) * rsx;
        ng[q] = (ld(z, H + h) - mug) * rsg;
        const float dh = ld(dhid, row * H + h);
        const float ux = nx[q] * cgx[q] + cbx[q];
        const float ug = ng[q] * cgg[q] + cbg[q];
        const float sg = sigmoidf_(ug);
        const float dux = dh * ug * sg;
        const float dug = dh * ux * sg * (1.f + ug * (1.f - sg));
        agx[q] += dux * nx[q];
        abx[q] += dux;
        agg[q] += dug * ng[q];
        abg[q] += dug;
        dnx[q] = dux * cgx[q];
        dng[q] = dug * cgg[q];
      } else {
        nx[q] = ng[q] = dnx[q] = dng[q] = 0.f;
      }
      s[0] += dnx[q];
      s[1] += dnx[q] * nx[q];
      s[2] += dng[q];
      s[3] += dng[q] * ng[q];
    }
    // block reduction over 8 waves, fixed order
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float w = wave_sum(s[i]);
      if (lane == 0) red[i * 8 + wave] = w;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float* r = red + i * 8;
      s[i] = ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
    }
    __syncthreads();
    const float m1 = s[0] * invH, m2 = s[1] * invH, m3 = s[2] * invH, m4 = s[3] * invH;
#pragma unroll
    for (int q = 0; q < QG; ++q) {
      const int h = tid + 512 * q;
      if (h < H) {
        const float du = rsx * (dnx[q] - m1 - nx[q] * m2);
        const float dg = rsg * (dng[q] - m3 - ng[q] * m4);
        st(dZ, row * 2 * H + h, du);
        st(dZ, row * 2 * H + H + h, dg);
        au[q] += du;
        ag[q] += dg;
      }
    }
  }
  // partial layouts: pgate [4][nb][T][H], pb1 [nb][T][2H]
  const long blk = (long)nb * T * H;
  const long o = ((long)grp * T + t) * H;
  const long o1 = ((long)grp * T + t) * 2 * H;
#pragma unroll
  for (int q = 0; q < QG; ++q) {
    const int h = tid + 512 * q;
    if (h < H) {
      pgate[0 * blk + o + h] = agx[q];
      pgate[1 * blk + o + h] = abx[q];
      pgate[2 * blk + o + h] = agg[q];
      pgate[3 * blk + o + h] = abg[q];
      pb1[o1 + h] = au[q];
      pb1[o1 + H + h] = ag[q];
    }
  }
}

// ---------------------------------------------------------------------------
// Backward tail, one workgroup per sample b:
//   phase 1 (rows i): dr1 = norm1 backward of d(out1), with r1 recomputed from x
//                     through the token-mix gather and norm0's statistics;
//   phase 2 (rows j): da0 = token_mix(dr1) (the permutation is its own adjoint,
//                     applied as a gather, never as a copy);
//                     dx = dr1 + norm0 backward of da0.
// Per-sample partials: dgamma1, dbeta1, dgamma0, dbeta0.
template <typename ST>
__global__ __launch_bounds__(256) void k_tail_bwd(const ST* __restrict__ x, const float* __restrict__ dh1,
                                                  const ST* __restrict__ g0, const ST* __restrict__ be0,
                                                  const ST* __restrict__ g1, const float* __restrict__ stats,
                                                  float* __restrict__ dr1, ST* __restrict__ dx,
                                                  float* __restrict__ ptail, int B, int T, int D) {
  __shared__ float s_mu0[64], s_rs0[64];
  __shared__ float lds[4 * 1280];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const long N = (long)B * T;
  const long base = (long)b * T * D;
  const int S = D / T;
  const float invD = 1.0f / (float)D;
  for (int j = tid; j < T; j += 256) {
    s_mu0[j] = stats[ST_MU0 * N + (long)b * T + j];
    s_rs0[j] = stats[ST_RS0 * N + (long)b * T + j];
  }
  __syncthreads();

  float pg1[QD], pb1[QD], pg0[QD], pb0[QD];
#pragma unroll
  for (int q = 0; q < QD; ++q) pg1[q] = pb1[q] = pg0[q] = pb0[q] = 0.f;

  for (int i = wave; i < T; i += 4) {
    const float mu1 = stats[ST_MU1 * N + (long)b * T + i], rs1 = stats[ST_RS1 * N + (long)b * T + i];
    float n1[QD], dn[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) {
        int j, sc;
        tm_source(i, c, S, j, sc);
        const float a0 = (ld(x, base + (long)j * D + sc) - s_mu0[j]) * s_rs0[j] * ld(g0, sc) + ld(be0, sc);
        const float r1 = a0 + ld(x, base + (long)i * D + c);
        n1[q] = (r1 - mu1) * rs1;
        const float g = dh1[base + (long)i * D + c];
        dn[q] = g * ld(g1, c);
        pg1[q] += g * n1[q];
        pb1[q] += g;
      } else {
        n1[q] = dn[q] = 0.f;
      }
      s1 += dn[q];
      s2 += dn[q] * n1[q];
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) dr1[base + (long)i * D + c] = rs1 * (dn[q] - m1 - n1[q] * m2);
    }
  }
  __threadfence();
  __syncthreads();

  for (int j = wave; j < T; j += 4) {
    const float mu0 = s_mu0[j], rs0 = s_rs0[j];
    float n0[QD], dn[QD];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) {
        int i, sc;
        tm_source(j, c, S, i, sc);
        const float da0 = dr1[base + (long)i * D + sc];
        n0[q] = (ld(x, base + (long)j * D + c) - mu0) * rs0;
        dn[q] = da0 * ld(g0, c);
        pg0[q] += da0 * n0[q];
        pb0[q] += da0;
      } else {
        n0[q] = dn[q] = 0.f;
      }
      s1 += dn[q];
      s2 += dn[q] * n0[q];
    }
    const float m1 = wave_sum(s1) * invD, m2 = wave_sum(s2) * invD;
#pragma unroll
    for (int q = 0; q < QD; ++q) {
      const int c = lane + 64 * q;
      if (c < D) st(dx, base + (long)j * D + c, dr1[base + (long)j * D + c] + rs0 * (dn[q] - m1 - n0[q] * m2));
    }
  }

  // partial layout: [4][B][D]: dgamma0, dbeta0, dgamma1, dbeta1
  const long blk = (long)B * D;
  float* out = ptail + (long)b * D;
  combine_waves_store(pg0, lds, out + 0 * blk, D);
  combine_waves_store(pb0, lds, out + 1 * blk, D);
  combine_waves_store(pg1, lds, out + 2 * blk, D);
  combine_waves_store(pb1, lds, out + 3 * blk, D);
}

// ---------------------------------------------------------------------------
// Fixed-order column sums of partial rows: out[c] = sum_p part[p * pstride + c].
struct RedJob {
  const float* part;
  long pstride;
  int P;
  int ncols;
  void* out;
};
struct RedJobs {
  RedJob j[12];
};

template <typename ST>
__global__ __launch_bounds__(256) void k_finalize(RedJobs jobs) {
  const RedJob job = jobs.j[blockIdx.y];
  const long c = (long)blockIdx.x * 256 + threadIdx.x;
  if (c >= job.ncols) return;
  float total = 0.f;
  for (int p0 = 0; p0 < job.P; p0 += 16) {
    float s = 0.f;
    const int p1 = min(job.P, p0 + 16);
    for (int p = p0; p < p1; ++p) s += job.part[(long)p * job.pstride + c];
    total += s;
  }
  st(reinterpret_cast<ST*>(job.out), c, total);
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

template <typename ST>
hipError_t prologue_t(const rm_dims& d, const rm_params& p, const void* x, void* ws, const WsLayout& L,
                      hipStream_t s) {
  prof_begin(KID_PROLOGUE, s);
  hipLaunchKernelGGL(k_prologue<ST>, dim3(d.B), dim3(256), 0, s, cptr<ST>(x), cptr<ST>(p.ln0_g),
                     cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), cptr<ST>(p.ln1_b), wsp<ST>(ws, L.h1),
                     wsp<float>(ws, L.stats), d.B, d.T, d.D);
  prof_end(KID_PROLOGUE, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t gate_fwd_t(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  const long N = (long)d.B * d.T;
  prof_begin(KID_GATE_FWD, s);
  hipLaunchKernelGGL(k_gate_fwd<ST>, dim3((unsigned)N), dim3(256), 0, s, wsp<ST>(ws, L.z), cptr<ST>(p.lnx_g),
                     cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g), cptr<ST>(p.lng_b), wsp<ST>(ws, L.hid),
                     wsp<float>(ws, L.stats), N, d.k * d.D);
  prof_end(KID_GATE_FWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t ln2_fwd_t(const rm_dims& d, const rm_params& p, void* y, void* ws, const WsLayout& L, hipStream_t s) {
  const long N = (long)d.B * d.T;
  prof_begin(KID_LN2_FWD, s);
  hipLaunchKernelGGL(k_ln2_fwd<ST>, dim3((unsigned)((N + 3) / 4)), dim3(256), 0, s, wsp<float>(ws, L.r2),
                     cptr<ST>(p.ln2_g), cptr<ST>(p.ln2_b), reinterpret_cast<ST*>(y), wsp<float>(ws, L.stats), N,
                     d.D);
  prof_end(KID_LN2_FWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t ln2_bwd_t(const rm_dims& d, const rm_params& p, const void* dy, void* ws, const WsLayout& L,
                     hipStream_t s) {
  prof_begin(KID_LN2_BWD, s);
  hipLaunchKernelGGL(k_ln2_bwd<ST>, dim3(d.T, L.nb), dim3(256), 0, s, wsp<float>(ws, L.r2), cptr<ST>(dy),
                     cptr<ST>(p.ln2_g), wsp<float>(ws, L.stats), wsp<ST>(ws, L.do2), wsp<float>(ws, L.p_ln2),
                     d.B, d.T, d.D, L.nb);
  prof_end(KID_LN2_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t gate_bwd_t(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  const int H = d.k * d.D;
  float* pg = wsp<float>(ws, L.p_gate);
  float* pb1 = pg + 4L * L.nb * d.T * H;
  prof_begin(KID_GATE_BWD, s);
  hipLaunchKernelGGL(k_gate_bwd<ST>, dim3(d.T, L.nb), dim3(512), 0, s, wsp<ST>(ws, L.z), wsp<ST>(ws, L.dhid),
                     cptr<ST>(p.lnx_g), cptr<ST>(p.lnx_b), cptr<ST>(p.lng_g), cptr<ST>(p.lng_b),
                     wsp<float>(ws, L.stats), wsp<ST>(ws, L.dz), pg, pb1, d.B, d.T, H, L.nb);
  prof_end(KID_GATE_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t tail_bwd_t(const rm_dims& d, const rm_params& p, const void* x, void* dx, void* ws, const WsLayout& L,
                      hipStream_t s) {
  prof_begin(KID_TAIL_BWD, s);
  hipLaunchKernelGGL(k_tail_bwd<ST>, dim3(d.B), dim3(256), 0, s, cptr<ST>(x), wsp<float>(ws, L.dh1),
                     cptr<ST>(p.ln0_g), cptr<ST>(p.ln0_b), cptr<ST>(p.ln1_g), wsp<float>(ws, L.stats),
                     wsp<float>(ws, L.dr1), reinterpret_cast<ST*>(dx), wsp<float>(ws, L.p_tail), d.B, d.T, d.D);
  prof_end(KID_TAIL_BWD, s);
  return hipGetLastError();
}

template <typename ST>
hipError_t finalize_t(const rm_dims& d, const rm_grads& g, void* ws, const WsLayout& L, hipStream_t s) {
  const int T = d.T, D = d.D, H = d.k * d.D, nb = L.nb;
  const float* pl = wsp<float>(ws, L.p_ln2);
  const float* pg = wsp<float>(ws, L.p_gate);
  const float* pt = wsp<float>(ws, L.p_tail);
  const long bl = (long)nb * T * D, bg = (long)nb * T * H, bt = (long)d.B * D;
  RedJobs J;
  J.j[0] = {pl + 0 * bl, D, nb * T, D, g.ln2_g};
  J.j[1] = {pl + 1 * bl, D, nb * T, D, g.ln2_b};
  J.j[2] = {pl + 2 * bl, (long)T * D, nb, T * D, g.bout};
  J.j[3] = {pg + 0 * bg, H, nb * T, H, g.lnx_g};
  J.j[4] = {pg + 1 * bg, H, nb * T, H, g.lnx_b};
  J.j[5] = {pg + 2 * bg, H, nb * T, H, g.lng_g};
  J.j[6] = {pg + 3 * bg, H, nb * T, H, g.lng_b};
  J.j[7] = {pg + 4 * bg, (long)T * 2 * H, nb, T * 2 * H, g.b1};
  J.j[8] = {pt + 0 * bt, D, d.B, D, g.ln0_g};
  J.j[9] = {pt + 1 * bt, D, d.B, D, g.ln0_b};
  J.j[10] = {pt + 2 * bt, D, d.B, D, g.ln1_g};
  J.j[11] = {pt + 3 * bt, D, d.B, D, g.ln1_b};
  const int maxc = T * 2 * H;
  prof_begin(KID_FINALIZE, s);
  hipLaunchKernelGGL(k_finalize<ST>, dim3((maxc + 255) / 256, 12), dim3(256), 0, s, J);
  prof_end(KID_FINALIZE, s);
  return hipGetLastError();
}

}  // namespace

#define RM_DISPATCH(fn, ...) \
  ((d.dtype == RM_BF16) ? fn<bf16_t>(__VA_ARGS__) : fn<float>(__VA_ARGS__))

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
hipError_t launch_ln2_bwd(const rm_dims& d, const rm_params& p, const void* dy, void* ws, const WsLayout& L,
                          hipStream_t s) {
  return RM_DISPATCH(ln2_bwd_t, d, p, dy, ws, L, s);
}
hipError_t launch_gate_bwd(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(gate_bwd_t, d, p, ws, L, s);
}
hipError_t launch_tail_bwd(const rm_dims& d, const rm_params& p, const void* x, void* dx, void* ws,
                           const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(tail_bwd_t, d, p, x, dx, ws, L, s);
}
hipError_t launch_finalize(const rm_dims& d, const rm_grads& g, void* ws, const WsLayout& L, hipStream_t s) {
  return RM_DISPATCH(finalize_t, d, g, ws, L, s);
}
hipError_t launch_token_mix(const rm_dims& d, const void* in, void* out, hipStream_t s) {
  const long rows = (long)d.B * d.T;
  prof_begin(KID_TOKEN_MIX, s);
  if (d.dtype == RM_BF16)
    hipLaunchKernelGGL(k_token_mix<uint16_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const uint16_t*>(in), reinterpret_cast<uint16_t*>(out), d.T, d.D);
  else
    hipLaunchKernelGGL(k_token_mix<uint32_t>, dim3((unsigned)rows), dim3(256), 0, s,
                       reinterpret_cast<const uint32_t*>(in), reinterpret_cast<uint32_t*>(out), d.T, d.D);
  prof_end(KID_TOKEN_MIX, s);
  return hipGetLastError();
}

}  // namespace rm
