// Internal host-side declarations: workspace layout, kernel ids, launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "rmblock.h"

namespace rm {

// Rows (b) per workgroup in the per-token row-group kernels of the backward:
// 128, halved (down to 16) while the T x ceil(B / rows) workgroups of those
// kernels would number fewer than 512 (two per compute unit), so that small
// batches still spread over the chip.  Always a power of two.
constexpr int MAX_ROWS_PER_GROUP = 128;
constexpr int MIN_ROWS_PER_GROUP = 16;
inline int rows_per_group(int B, int T) {
  int r = MAX_ROWS_PER_GROUP;
  while (r > MIN_ROWS_PER_GROUP && (long)T * ((B + r - 1) / r) < 512) r >>= 1;
  return r;
}

enum KernelId {
  KID_PROLOGUE = 0,   // norm0 -> token mix -> +x -> norm1
  KID_GEMM_UP,        // Z = out1 @ w1[t] + b1[t]
  KID_GATE_FWD,       // LN_x(U) * silu(LN_gate(G))
  KID_GEMM_DOWN,      // out1 + hidden @ wout[t] + bout[t]
  KID_LN2_FWD,        // norm2
  KID_LN2_BWD,        // norm2 backward (+ dbout, dgamma2, dbeta2 partials)
  KID_GEMM_DHID,      // d hidden = d(out2) @ wout[t]^T
  KID_GATE_BWD,       // gate / SiLU / inner LayerNorm backward -> dZ
  KID_GEMM_DWOUT,     // dwout[t] = hidden^T @ d(out2)
  KID_GEMM_DW1,       // dw1[t] = out1^T @ dZ
  KID_GEMM_DH1,       // d(out1) = dZ @ w1[t]^T + d(out2)
  KID_LN1_BWD,        // norm1 backward (r1 recomputed through the token-mix gather)
  KID_LN0_BWD,        // token-mix adjoint (gather) + norm0 backward -> dx
  KID_FINALIZE,       // fixed-order sums of parameter-gradient partials
  KID_TOKEN_MIX,      // stand-alone token permutation
  KID_TAIL_BWD,       // norm1 + token-mix adjoint + norm0 backward, one sample per workgroup
  KID_SMALL_FWD,      // small-batch forward: one workgroup per token
  KID_SMALL_BWD,      // small-batch backward up to d r1: one workgroup per token
  KID_SMALL_FIN,      // small-batch norm0 backward and affine-gradient sums: one workgroup
  KID_COUNT
};

extern const char* const kKernelNames[KID_COUNT];

// Workspace layout.  The regions the forward saves for the backward come
// first, at byte offsets from the workspace's start; the backward's scratch
// follows at scratch_off, its regions at byte offsets from the scratch start
// (so the scratch may also live elsewhere: rm_block_bwd_static).
struct WsLayout {
  size_t h1, z, hid, r2, stats;            // saved by the forward: offsets from the workspace start
  size_t do2, dhid, dz, dh1, dr1;          // backward scratch: offsets from the scratch start
  size_t p_ln2, p_gate, p_tail;            // backward partial sums (fp32): offsets from the scratch start
  size_t scratch_off, scratch_bytes;       // where the scratch starts in the workspace, its size
  size_t total;                            // scratch_off + scratch_bytes
  int rpg;                                 // rows per group: rows_per_group(B, T)
  int nb;                                  // row groups per token: ceil(B / rpg)
};

bool dims_valid(const rm_dims& d);

// One 16-bit (bf16 or fp16) sample (T x D) fits the 160 KB LDS of a workgroup, rows are whole
// 16-byte pieces (D % 8 == 0) and 4-element chunks have contiguous token-mix
// sources: the prologue and the backward tail then run one sample per
// workgroup, staged in LDS by direct copies (which also need a 16-byte
// aligned x).
constexpr long SAMPLE_LDS_BYTES = 64L * 1280 * 2;
inline bool sample_in_lds(const rm_dims& d) {
  return (d.dtype == RM_BF16 || d.dtype == RM_F16) && d.D % 8 == 0 && (d.D / d.T) % 4 == 0 &&
         (long)d.T * d.D * 2 <= SAMPLE_LDS_BYTES;
}
WsLayout ws_layout(const rm_dims& d);

// stats block: 10 arrays of B*T floats in this order
enum { ST_MU0 = 0, ST_RS0, ST_MU1, ST_RS1, ST_MUX, ST_RSX, ST_MUG, ST_RSG, ST_MU2, ST_RS2, ST_COUNT };

// instrumentation hooks (no-ops unless enabled)
void prof_begin(int kid, hipStream_t s);
void prof_end(int kid, hipStream_t s);

// ---------------------------------------------------------------------------
// GEMM over T independent problems (one per token t):  C_t = A_t (MxK) . B_t (KxN)
// A K-major: element (m,k) at A + t*a_bs + m*a_ld + k;  M-major: at A + t*a_bs + k*a_ld + m
// B K-major: element (k,n) at B + t*b_bs + n*b_ld + k;  N-major: at B + t*b_bs + k*b_ld + n
// epilogue: v = acc (+ bias[t*bias_bs + n]) (+ res[t*res_bs + m*res_ld + n]);
//           C[t*c_bs + m*c_ld + n] = v  (storage dtype, or fp32 when c_f32)
struct GemmArgs {
  int M, N, K, batch;
  const void* A; long a_bs, a_ld;
  const void* B; long b_bs, b_ld;
  void* C; long c_bs, c_ld; int c_f32;
  const void* bias; long bias_bs;
  const void* res; long res_bs, res_ld; int res_f32;
};

hipError_t launch_gemm(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid,
                       hipStream_t s);
// 256x256-tile bf16 / fp16 kernel (direct-to-LDS loads, transposing LDS reads): shapes it takes
// Compute units of the current device (cached per device).
int device_cu_count();
bool gemm256_supported(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid);
hipError_t launch_gemm256(int dtype, bool a_kmajor, bool b_kmajor, const GemmArgs& g, int kid, hipStream_t s);

// ---------------------------------------------------------------------------
// row kernels
hipError_t launch_prologue(const rm_dims& d, const rm_params& p, const void* x, void* ws,
                           const WsLayout& L, hipStream_t s);
hipError_t launch_gate_fwd(const rm_dims& d, const rm_params& p, void* ws, const WsLayout& L,
                           hipStream_t s);
hipError_t launch_ln2_fwd(const rm_dims& d, const rm_params& p, void* y, void* ws,
                          const WsLayout& L, hipStream_t s);
// Backward launchers: ws holds the forward's saved regions, sc the scratch.
hipError_t launch_ln2_bwd(const rm_dims& d, const rm_params& p, const void* dy, void* ws, void* sc,
                          const WsLayout& L, hipStream_t s);
hipError_t launch_gate_bwd(const rm_dims& d, const rm_params& p, void* ws, void* sc, const WsLayout& L,
                           hipStream_t s);
hipError_t launch_tail_bwd(const rm_dims& d, const rm_params& p, const void* x, void* dx, void* ws, void* sc,
                           const WsLayout& L, hipStream_t s);
hipError_t launch_finalize(const rm_dims& d, const rm_grads& g, void* sc, const WsLayout& L,
                           hipStream_t s);
hipError_t launch_token_mix(const rm_dims& d, const void* in, void* out, hipStream_t s);

// ---------------------------------------------------------------------------
// small-batch path: the whole forward in one launch, the backward in two.
// A token's contractions run on one CU, so the path pays off only while they
// are small: measured 4.5x faster than the main path at B8 T8 D64 k2 and 1.6x
// at B4 T16 D128 k2.
constexpr int SMALL_MAX_B = 8, SMALL_MAX_D = 128, SMALL_MAX_H = 256;
bool small_supported(const rm_dims& d);
hipError_t launch_small_fwd(const rm_dims& d, const rm_params& p, const void* x, void* y, void* ws,
                            const WsLayout& L, hipStream_t s);
hipError_t launch_small_bwd(const rm_dims& d, const rm_params& p, const void* x, const void* dy, void* ws, void* sc,
                            const WsLayout& L, void* dx, const rm_grads& g, hipStream_t s);

}  // namespace rm
