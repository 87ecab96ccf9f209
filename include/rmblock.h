/*
 * rmblock.h -- C ABI of the MI355X (gfx950) RankMixerBlock forward + backward.
 *
 * The operation is the block defined on the page "Subgraph-fusion-based
 * Mega-kernel Generation" (page 1):
 *   section "Exact computation":
 *     out1 = norm1(token_mixer(norm0(x)) + x)
 *     out2 = dense_ffn_v2(out1):  Z[b,t,:] = out1[b,t,:] @ w1[t] + b1[t];
 *            (U, G) = the two H-wide halves of Z (U first);
 *            hidden = LN_x(U) * silu(LN_gate(G));
 *            out2[b,t,:] = hidden[b,t,:] @ wout[t] + bout[t]
 *     y    = norm2(out1 + out2)
 *   outer LayerNorms norm0/1/2: eps 1e-3, D-element gamma/beta;
 *   inner LayerNorms norm_x / norm_gate: eps 1e-5, H-element gamma/beta shared by all tokens;
 *   token mixing: view [B,T,D] as [B,T,T,D/T], swap the two T axes, view back;
 *   section "Workload and interfaces": shapes, the same-shape upstream gradient,
 *     differentiation of the complete block;
 *   section "Public checks and instructor coverage": the dimension envelope
 *     1<=B<=1024, 8<=T<=64, 64<=D<=1280, D%T==0, k in {2,3}, H = k*D.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, contiguous, in the storage dtype of
 *     rm_dims.dtype (fp32, bf16 or fp16).  Device pointers only; the caller owns
 *     every buffer.  The library never allocates, frees or synchronises
 *     (except the instrumentation calls rm_prof_*, which say so).
 *   - `stream` is a hipStream_t (0 = the null stream) of the current device.
 *     Work is enqueued on it; results are valid once the caller syncs it.
 *   - Apart from the instrumentation records (rm_prof_*), the library keeps
 *     no state between calls: everything a call does is fixed by its
 *     arguments, so calls on distinct streams with distinct workspaces may run
 *     from several threads at once.
 *   - Validation (dims, dtype, null pointers, alignment, workspace size) runs
 *     on the host before anything is enqueued; on failure nothing is launched
 *     and the status says why.  RM_E_HIP means a launch failed.
 *   - Arithmetic: storage dtype (fp32, bf16 or fp16) for inputs, parameters,
 *     outputs, gradients and every saved or intermediate tensor; fp32
 *     accumulation and statistics; round to nearest even on every store.  Results are bitwise repeatable for
 *     identical inputs (fixed-order reductions, no floating-point atomics).
 */
#ifndef RMBLOCK_H
#define RMBLOCK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RM_ABI_VERSION 2

/* Storage dtypes.  Besides the bf16 production workload, the page's section
 * "Run the benchmark" runs the block with fp32 and fp16 storage; every
 * storage dtype computes in fp32 inside the kernels. */
typedef enum { RM_F32 = 0, RM_BF16 = 1, RM_F16 = 2 } rm_dtype;

typedef enum {
  RM_OK = 0,
  RM_E_DIMS = 1,       /* outside the envelope, D % T != 0, or k not in {2,3} */
  RM_E_NULL = 2,       /* a required pointer is NULL                           */
  RM_E_ALIGN = 3,      /* a pointer is not aligned to its element size         */
  RM_E_WORKSPACE = 4,  /* ws_bytes < rm_workspace_bytes(dims)                  */
  RM_E_DTYPE = 5,      /* dtype is not RM_F32, RM_BF16 or RM_F16               */
  RM_E_HIP = 6,        /* a HIP launch or runtime call failed                  */
  RM_E_ARG = 7,        /* any other invalid argument                            */
  RM_E_SCRATCH = 8     /* rm_block_bwd_static: scratch beyond its static buffer */
} rm_status;

/* Kernel-set choice, per call (rm_dims.flags).  By default (0) shapes with
 * B <= 8, D <= 128 and H <= 256 run the same computation (page 1, "Exact
 * computation") as one launch for the forward (one workgroup per token, its
 * rows in LDS) and two for the backward, instead of one launch per fused
 * step; every other shape takes the main kernels.  RM_FLAG_MAIN_KERNELS sends
 * the call through the main kernels whatever the shape.  Both kernel sets save
 * the same state in ws, so either backward may follow either forward.  Any
 * other bit set: RM_E_ARG. */
#define RM_FLAG_MAIN_KERNELS 1

/* Block dimensions.  H = k*D.  dtype is an rm_dtype value; flags holds RM_FLAG_* bits. */
typedef struct {
  int32_t B, T, D, k;
  int32_t dtype;
  int32_t flags;
} rm_dims;

/* Parameters (device pointers, storage dtype):
 *   w1 [T,D,2H]   b1 [T,2H]   wout [T,H,D]   bout [T,D]
 *   lnx_g, lnx_b, lng_g, lng_b : [H]   (norm_x, norm_gate)
 *   ln0_g ... ln2_b            : [D]   (norm0, norm1, norm2)          */
typedef struct {
  const void *w1, *b1, *wout, *bout;
  const void *lnx_g, *lnx_b, *lng_g, *lng_b;
  const void *ln0_g, *ln0_b, *ln1_g, *ln1_b, *ln2_g, *ln2_b;
} rm_params;

/* Parameter gradients, same shapes and dtype as rm_params.  Overwritten, never
 * accumulated (the pages reset gradients to None before every iteration). */
typedef struct {
  void *w1, *b1, *wout, *bout;
  void *lnx_g, *lnx_b, *lng_g, *lng_b;
  void *ln0_g, *ln0_b, *ln1_g, *ln1_b, *ln2_g, *ln2_b;
} rm_grads;

/* Bytes of device workspace rm_block_fwd / rm_block_bwd need for these dims
 * (256-byte aligned regions).  Returns 0 if the dims are invalid. */
size_t rm_workspace_bytes(const rm_dims* dims);

/* Forward.  x, y: [B,T,D].  ws: at least rm_workspace_bytes(dims) bytes,
 * 256-byte aligned; the forward writes into it everything the backward needs
 * (out1, Z, hidden, out1+out2 and the per-row LayerNorm mean/rstd).
 * x, the parameters and ws must stay unchanged until rm_block_bwd is done. */
rm_status rm_block_fwd(const rm_dims* dims, const rm_params* p, const void* x, void* y,
                       void* ws, size_t ws_bytes, void* stream);

/* Backward of the whole block for the upstream gradient dy [B,T,D].
 * Writes dx [B,T,D] and every gradient in g.  Reads what rm_block_fwd saved in
 * ws (left intact) and uses the rest of ws as scratch, so it may be called
 * again with the same ws.  Calls on one ws must not overlap in time. */
rm_status rm_block_bwd(const rm_dims* dims, const rm_params* p, const void* x, const void* dy,
                       void* ws, size_t ws_bytes, void* dx, const rm_grads* g, void* stream);

/* Backward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same computation and results as rm_block_bwd, with the backward's scratch
 * (d out2, d hidden, dZ, d out1, d r1, gradient partials) in a static device
 * array of RM_STATIC_SCRATCH_BYTES that the library holds on each GPU it runs
 * on until the process ends, instead of in the caller's workspace.
 *   - ws needs to hold only the regions the forward saves: ws_bytes >= offset
 *     + bytes of region RM_WS_STATS (rm_ws_region), the start of a workspace
 *     that rm_block_fwd filled (a full rm_workspace_bytes() one is fine).
 *   - Shapes whose scratch exceeds RM_STATIC_SCRATCH_BYTES get RM_E_SCRATCH
 *     and nothing is launched (the small workloads of the pages fit; the
 *     production shape B1024 T64 D1280 needs rm_block_bwd).
 *   - Allocates nothing (no hipMalloc, hipFree or allocating library call;
 *     the instrumentation rm_prof_* must be off).
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's contents (nothing in it needs to start at zero): calls that
 *     overlap in time on one GPU race and give undefined results. */
#define RM_STATIC_SCRATCH_BYTES (256u << 20)
rm_status rm_block_bwd_static(const rm_dims* dims, const rm_params* p, const void* x, const void* dy,
                              void* ws, size_t ws_bytes, void* dx, const rm_grads* g, void* stream);

/* Token mixing alone (page 1, "Exact computation", token mixing paragraph):
 * out[b,i,j*S+s] = in[b,j,i*S+s], S = D/T.  A pure permutation of element bits
 * (no arithmetic), through the same device index function the block uses.
 * in and out must not alias. */
rm_status rm_token_mix(const rm_dims* dims, const void* in, void* out, void* stream);

/* Layout of ws: regions saved by the forward (for inspection by tests).
 * region ids: see RM_WS_* below.  Writes the region's byte offset and size. */
enum {
  RM_WS_H1 = 0,     /* out1 [B,T,D] storage dtype                         */
  RM_WS_Z = 1,      /* Z [B,T,2H] storage dtype                           */
  RM_WS_HID = 2,    /* hidden [B,T,H] storage dtype                       */
  RM_WS_R2 = 3,     /* out1 + out2 [B,T,D] storage dtype                  */
  RM_WS_STATS = 4,  /* 10 x [B*T] fp32: mean,rstd of norm0, norm1, norm_x, norm_gate, norm2 */
  RM_WS_NREGIONS = 5
};
rm_status rm_ws_region(const rm_dims* dims, int region, size_t* offset, size_t* bytes);

const char* rm_status_string(int status);
int rm_abi_version(void);

/* Instrumentation.  While enabled, every kernel launched by rm_block_fwd /
 * rm_block_bwd is bracketed by two hipEvents recorded on the caller's stream
 * (creating events as needed: this mode allocates).  Open brackets are kept
 * per stream, so calls on several streams from several threads pair their
 * events correctly.  rm_prof_collect synchronises those events, adds their
 * elapsed times per kernel id into ms[id] and launches[id] (arrays of
 * rm_prof_kernels() entries) and releases the pending records. */
rm_status rm_prof_enable(int on);
int rm_prof_kernels(void);
const char* rm_prof_name(int id);
rm_status rm_prof_collect(double* ms, int64_t* launches, int n);

#ifdef __cplusplus
}
#endif
#endif /* RMBLOCK_H */
