// C ABI of the RankMixerBlock library: host-side validation, workspace
// layout and the launch sequence of the forward and backward passes.
//
// Forward (page 1 of "Subgraph-fusion-based Mega-kernel Generation",
// section "Exact computation", in the page's order):
//   prologue   norm0 -> token mix -> + x -> norm1            => out1, stats
//   gemm up    Z = out1 @ w1[t] + b1[t]                       => Z
//   gate fwd   hidden = LN_x(U) * silu(LN_gate(G))            => hidden, stats
//   gemm down  r2 = out1 + hidden @ wout[t] + bout[t]         => r2
//   ln2 fwd    y = norm2(r2)                                  => y, stats
// Backward (the same steps in reverse):
//   ln2 bwd    d(out2) = norm2 backward of dy                 (+ dgamma2, dbeta2, dbout partials)
//   gemm dhid  d hidden = d(out2) @ wout[t]^T
//   gate bwd   dZ = gate / SiLU / inner-LayerNorm backward    (+ inner affine, db1 partials)
//   gemm dwout dwout[t] = hidden^T @ d(out2)
//   gemm dw1   dw1[t] = out1^T @ dZ
//   gemm dh1   d(out1) = dZ @ w1[t]^T + d(out2)
//   ln1 bwd    norm1 backward (r1 recomputed via the token-mix gather) => dr1 (+ dgamma1, dbeta1)
//   ln0 bwd    token-mix adjoint as a gather, norm0 backward, + dr1   => dx (+ dgamma0, dbeta0)
//   finalize   fixed-order sums of every partial              => parameter gradients
#include <atomic>
#include <mutex>
#include <vector>

#include "rm_internal.h"

namespace rm {

const char* const kKernelNames[KID_COUNT] = {
    "prologue", "gemm_up", "gate_fwd", "gemm_down", "ln2_fwd", "ln2_bwd", "gemm_dhid",
    "gate_bwd", "gemm_dwout", "gemm_dw1", "gemm_dh1", "ln1_bwd", "ln0_bwd", "finalize", "token_mix",
    "tail_bwd", "small_fwd", "small_bwd", "small_fin"};

bool dims_valid(const rm_dims& d) {
  if (d.dtype != RM_F32 && d.dtype != RM_BF16 && d.dtype != RM_F16) return false;
  if (d.B < 1 || d.B > 1024) return false;
  if (d.T < 8 || d.T > 64) return false;
  if (d.D < 64 || d.D > 1280) return false;
  if (d.D % d.T != 0) return false;
  if (d.k != 2 && d.k != 3) return false;
  return true;
}

static size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

WsLayout ws_layout(const rm_dims& d) {
  WsLayout L{};
  const size_t N = (size_t)d.B * d.T, D = d.D, H = (size_t)d.k * d.D, T = d.T;
  const size_t sz = d.dtype == RM_F32 ? 4 : 2;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    off = align256(off);
    const size_t r = off;
    off += bytes;
    return r;
  };
  L.rpg = rows_per_group(d.B, d.T);
  L.nb = (d.B + L.rpg - 1) / L.rpg;
  const size_t nb = L.nb;
  L.h1 = take(N * D * sz);
  L.z = take(N * 2 * H * sz);
  L.hid = take(N * H * sz);
  L.r2 = take(N * D * sz);
  L.stats = take(ST_COUNT * N * 4);
  // the backward's scratch: offsets from its own (256-byte aligned) start
  L.scratch_off = align256(off);
  off = 0;
  L.do2 = take(N * D * sz);
  L.dhid = take(N * H * sz);
  L.dz = take(N * 2 * H * sz);
  L.dh1 = take(N * D * sz);
  L.dr1 = take(N * D * sz);
  L.p_ln2 = take(3 * nb * T * D * 4);
  L.p_gate = take((4 * nb * T * H + nb * T * 2 * H) * 4);
  // tail partials per (row group, token), or per sample when the tail runs one sample per workgroup
  L.p_tail = take(4 * (sample_in_lds(d) ? (size_t)d.B : nb * T) * D * 4);
  L.scratch_bytes = align256(off);
  L.total = L.scratch_off + L.scratch_bytes;
  return L;
}

// ---------------------------------------------------------------------------
// instrumentation
namespace {
struct ProfRec {
  int kid;
  hipEvent_t a, b;
};
struct OpenRec {
  hipStream_t s;
  int kid;
  hipEvent_t a;
};
std::mutex g_mu;
bool g_prof = false;
std::vector<ProfRec> g_recs;
std::vector<hipEvent_t> g_pool;
std::vector<OpenRec> g_open;  // brackets begun and not yet ended, per stream

hipEvent_t get_event() {
  if (!g_pool.empty()) {
    hipEvent_t e = g_pool.back();
    g_pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void prof_begin(int kid, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_prof) return;
  hipEvent_t a = get_event();
  if (!a) return;
  if (hipEventRecord(a, s) != hipSuccess) {
    g_pool.push_back(a);
    return;
  }
  g_open.push_back({s, kid, a});
}

void prof_end(int kid, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_mu);
  if (!g_prof) return;
  // the latest bracket this stream opened for this kernel
  for (size_t i = g_open.size(); i-- > 0;) {
    if (g_open[i].s != s || g_open[i].kid != kid) continue;
    const hipEvent_t a = g_open[i].a;
    g_open.erase(g_open.begin() + (long)i);
    hipEvent_t b = get_event();
    if (b && hipEventRecord(b, s) == hipSuccess) {
      g_recs.push_back({kid, a, b});
    } else {
      g_pool.push_back(a);
      if (b) g_pool.push_back(b);
    }
    return;
  }
}

}  // namespace rm

using namespace rm;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// need_saved_only: the workspace has to hold the forward's saved regions only
// (rm_block_bwd_static), not the backward's scratch as well.
rm_status check_common(const rm_dims* dims, const rm_params* p, const void* ws, size_t ws_bytes,
                       bool need_saved_only = false) {
  if (!dims || !p) return RM_E_NULL;
  if (dims->dtype != RM_F32 && dims->dtype != RM_BF16 && dims->dtype != RM_F16) return RM_E_DTYPE;
  if (!dims_valid(*dims)) return RM_E_DIMS;
  if (dims->flags & ~RM_FLAG_MAIN_KERNELS) return RM_E_ARG;
  const void* ptrs[] = {p->w1, p->b1, p->wout, p->bout, p->lnx_g, p->lnx_b, p->lng_g,
                        p->lng_b, p->ln0_g, p->ln0_b, p->ln1_g, p->ln1_b, p->ln2_g, p->ln2_b};
  const size_t es = dims->dtype == RM_F32 ? 4 : 2;
  for (const void* q : ptrs) {
    if (!q) return RM_E_NULL;
    if (!aligned(q, es)) return RM_E_ALIGN;
  }
  if (!ws) return RM_E_NULL;
  if (!aligned(ws, 256)) return RM_E_ALIGN;
  const WsLayout L = ws_layout(*dims);
  const size_t saved_end = L.stats + (size_t)ST_COUNT * dims->B * dims->T * 4;  // end of the last saved region
  if (ws_bytes < (need_saved_only ? saved_end : L.total)) return RM_E_WORKSPACE;
  return RM_OK;
}

rm_status hip_status(hipError_t e) { return e == hipSuccess ? RM_OK : RM_E_HIP; }

// The small-batch kernels run this call: its shape fits them and the caller did not ask for the main kernels.
bool use_small(const rm_dims& d) { return !(d.flags & RM_FLAG_MAIN_KERNELS) && small_supported(d); }

// Scratch of rm_block_bwd_static: the backward's scratch regions (d out2,
// d hidden, dZ, d out1, d r1 and the parameter-gradient partials) for shapes
// whose scratch fits.  One array per GPU the library runs on, held until the
// process ends.  In host code `scratch` is a stand-in, not a device address:
// host code uses only the per-device address that static_scratch() obtains.
__device__ __align__(256) char scratch[RM_STATIC_SCRATCH_BYTES];

// Per-device address of `scratch`, looked up once per device (with that
// device current) and kept.
std::atomic<void*> g_scratch_ptr[64];
std::mutex g_scratch_mu;

rm_status static_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return RM_E_HIP;
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (!ptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    ptr = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (!ptr) {
      if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return RM_E_HIP;
      g_scratch_ptr[dev].store(ptr, std::memory_order_release);
    }
  }
  *out = ptr;
  return RM_OK;
}

// Checks of the backward's arguments other than the workspace size.
rm_status check_bwd_args(const rm_dims* dims, const void* x, const void* dy, void* dx, const rm_grads* g) {
  if (!x || !dy || !dx || !g) return RM_E_NULL;
  const size_t es = dims->dtype == RM_F32 ? 4 : 2;
  if (!aligned(x, es) || !aligned(dy, es) || !aligned(dx, es)) return RM_E_ALIGN;
  const void* gptrs[] = {g->w1, g->b1, g->wout, g->bout, g->lnx_g, g->lnx_b, g->lng_g,
                         g->lng_b, g->ln0_g, g->ln0_b, g->ln1_g, g->ln1_b, g->ln2_g, g->ln2_b};
  for (const void* q : gptrs) {
    if (!q) return RM_E_NULL;
    if (!aligned(q, es)) return RM_E_ALIGN;
  }
  return RM_OK;
}

// The backward's launch sequence: the forward's saved regions in ws, the
// scratch regions (layout offsets from the scratch start) at sc.
rm_status backward(const rm_dims& d, const rm_params* p, const void* x, const void* dy, void* ws, void* sc,
                   void* dx, const rm_grads* g, hipStream_t s) {
  const WsLayout L = ws_layout(d);
  char* w = reinterpret_cast<char*>(ws);
  char* c = reinterpret_cast<char*>(sc);
  const long T = d.T, D = d.D, H = (long)d.k * d.D;
  hipError_t e;
  if (use_small(d)) return hip_status(launch_small_bwd(d, *p, x, dy, ws, sc, L, dx, *g, s));

  if ((e = launch_ln2_bwd(d, *p, dy, ws, sc, L, s)) != hipSuccess) return hip_status(e);

  GemmArgs a{};
  a.M = d.B; a.N = H; a.K = D; a.batch = T;
  a.A = c + L.do2; a.a_bs = D; a.a_ld = T * D;
  a.B = p->wout; a.b_bs = H * D; a.b_ld = D;
  a.C = c + L.dhid; a.c_bs = H; a.c_ld = T * H; a.c_f32 = 0;
  if ((e = launch_gemm(d.dtype, true, true, a, KID_GEMM_DHID, s)) != hipSuccess) return hip_status(e);

  if ((e = launch_gate_bwd(d, *p, ws, sc, L, s)) != hipSuccess) return hip_status(e);

  GemmArgs wo{};
  wo.M = H; wo.N = D; wo.K = d.B; wo.batch = T;
  wo.A = w + L.hid; wo.a_bs = H; wo.a_ld = T * H;
  wo.B = c + L.do2; wo.b_bs = D; wo.b_ld = T * D;
  wo.C = g->wout; wo.c_bs = H * D; wo.c_ld = D; wo.c_f32 = 0;
  if ((e = launch_gemm(d.dtype, false, false, wo, KID_GEMM_DWOUT, s)) != hipSuccess) return hip_status(e);

  GemmArgs w1g{};
  w1g.M = D; w1g.N = 2 * H; w1g.K = d.B; w1g.batch = T;
  w1g.A = w + L.h1; w1g.a_bs = D; w1g.a_ld = T * D;
  w1g.B = c + L.dz; w1g.b_bs = 2 * H; w1g.b_ld = T * 2 * H;
  w1g.C = g->w1; w1g.c_bs = D * 2 * H; w1g.c_ld = 2 * H; w1g.c_f32 = 0;
  if ((e = launch_gemm(d.dtype, false, false, w1g, KID_GEMM_DW1, s)) != hipSuccess) return hip_status(e);

  GemmArgs dh{};
  dh.M = d.B; dh.N = D; dh.K = 2 * H; dh.batch = T;
  dh.A = c + L.dz; dh.a_bs = 2 * H; dh.a_ld = T * 2 * H;
  dh.B = p->w1; dh.b_bs = D * 2 * H; dh.b_ld = 2 * H;
  dh.C = c + L.dh1; dh.c_bs = D; dh.c_ld = T * D; dh.c_f32 = d.dtype == RM_F32;
  dh.res = c + L.do2; dh.res_bs = D; dh.res_ld = T * D; dh.res_f32 = 0;
  if ((e = launch_gemm(d.dtype, true, true, dh, KID_GEMM_DH1, s)) != hipSuccess) return hip_status(e);

  if ((e = launch_tail_bwd(d, *p, x, dx, ws, sc, L, s)) != hipSuccess) return hip_status(e);
  if ((e = launch_finalize(d, *g, sc, L, s)) != hipSuccess) return hip_status(e);
  return RM_OK;
}

}  // namespace

extern "C" {

int rm_abi_version(void) { return RM_ABI_VERSION; }

const char* rm_status_string(int s) {
  switch (s) {
    case RM_OK: return "ok";
    case RM_E_DIMS: return "dimensions outside 1<=B<=1024, 8<=T<=64, 64<=D<=1280, D%T==0, k in {2,3}";
    case RM_E_NULL: return "a required pointer is NULL";
    case RM_E_ALIGN: return "a pointer is misaligned (elements: element size; workspace: 256 bytes)";
    case RM_E_WORKSPACE: return "workspace smaller than rm_workspace_bytes()";
    case RM_E_DTYPE: return "dtype must be RM_F32, RM_BF16 or RM_F16";
    case RM_E_HIP: return "HIP launch or runtime error";
    case RM_E_ARG: return "invalid argument";
    case RM_E_SCRATCH:
      return "backward scratch larger than RM_STATIC_SCRATCH_BYTES (rm_block_bwd_static); use rm_block_bwd with a "
             "workspace of rm_workspace_bytes()";
    default: return "unknown status";
  }
}

size_t rm_workspace_bytes(const rm_dims* dims) {
  if (!dims || !dims_valid(*dims)) return 0;
  return ws_layout(*dims).total;
}

rm_status rm_ws_region(const rm_dims* dims, int region, size_t* offset, size_t* bytes) {
  if (!dims || !offset || !bytes) return RM_E_NULL;
  if (dims->dtype != RM_F32 && dims->dtype != RM_BF16 && dims->dtype != RM_F16) return RM_E_DTYPE;
  if (!dims_valid(*dims)) return RM_E_DIMS;
  const WsLayout L = ws_layout(*dims);
  const size_t N = (size_t)dims->B * dims->T, D = dims->D, H = (size_t)dims->k * dims->D;
  const size_t sz = dims->dtype == RM_F32 ? 4 : 2;
  switch (region) {
    case RM_WS_H1: *offset = L.h1; *bytes = N * D * sz; return RM_OK;
    case RM_WS_Z: *offset = L.z; *bytes = N * 2 * H * sz; return RM_OK;
    case RM_WS_HID: *offset = L.hid; *bytes = N * H * sz; return RM_OK;
    case RM_WS_R2: *offset = L.r2; *bytes = N * D * sz; return RM_OK;
    case RM_WS_STATS: *offset = L.stats; *bytes = ST_COUNT * N * 4; return RM_OK;
    default: return RM_E_ARG;
  }
}

rm_status rm_block_fwd(const rm_dims* dims, const rm_params* p, const void* x, void* y, void* ws,
                       size_t ws_bytes, void* stream) {
  rm_status st = check_common(dims, p, ws, ws_bytes);
  if (st != RM_OK) return st;
  if (!x || !y) return RM_E_NULL;
  const size_t es = dims->dtype == RM_F32 ? 4 : 2;
  if (!aligned(x, es) || !aligned(y, es)) return RM_E_ALIGN;
  const rm_dims d = *dims;
  const WsLayout L = ws_layout(d);
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  char* w = reinterpret_cast<char*>(ws);
  const long T = d.T, D = d.D, H = (long)d.k * d.D;
  hipError_t e;
  if (use_small(d)) return hip_status(launch_small_fwd(d, *p, x, y, ws, L, s));

  if ((e = launch_prologue(d, *p, x, ws, L, s)) != hipSuccess) return hip_status(e);

  GemmArgs up{};
  up.M = d.B; up.N = 2 * H; up.K = D; up.batch = T;
  up.A = w + L.h1; up.a_bs = D; up.a_ld = T * D;
  up.B = p->w1; up.b_bs = D * 2 * H; up.b_ld = 2 * H;
  up.C = w + L.z; up.c_bs = 2 * H; up.c_ld = T * 2 * H; up.c_f32 = 0;
  up.bias = p->b1; up.bias_bs = 2 * H;
  if ((e = launch_gemm(d.dtype, true, false, up, KID_GEMM_UP, s)) != hipSuccess) return hip_status(e);

  if ((e = launch_gate_fwd(d, *p, ws, L, s)) != hipSuccess) return hip_status(e);

  GemmArgs dn{};
  dn.M = d.B; dn.N = D; dn.K = H; dn.batch = T;
  dn.A = w + L.hid; dn.a_bs = H; dn.a_ld = T * H;
  dn.B = p->wout; dn.b_bs = H * D; dn.b_ld = D;
  dn.C = w + L.r2; dn.c_bs = D; dn.c_ld = T * D; dn.c_f32 = d.dtype == RM_F32;
  dn.bias = p->bout; dn.bias_bs = D;
  dn.res = w + L.h1; dn.res_bs = D; dn.res_ld = T * D; dn.res_f32 = 0;
  if ((e = launch_gemm(d.dtype, true, false, dn, KID_GEMM_DOWN, s)) != hipSuccess) return hip_status(e);

  if ((e = launch_ln2_fwd(d, *p, y, ws, L, s)) != hipSuccess) return hip_status(e);
  return RM_OK;
}



rm_status rm_block_bwd(const rm_dims* dims, const rm_params* p, const void* x, const void* dy, void* ws,
                       size_t ws_bytes, void* dx, const rm_grads* g, void* stream) {
  rm_status st = check_common(dims, p, ws, ws_bytes);
  if (st != RM_OK) return st;
  if ((st = check_bwd_args(dims, x, dy, dx, g)) != RM_OK) return st;
  const WsLayout L = ws_layout(*dims);
  return backward(*dims, p, x, dy, ws, reinterpret_cast<char*>(ws) + L.scratch_off, dx, g,
                  reinterpret_cast<hipStream_t>(stream));
}

rm_status rm_block_bwd_static(const rm_dims* dims, const rm_params* p, const void* x, const void* dy, void* ws,
                              size_t ws_bytes, void* dx, const rm_grads* g, void* stream) {
  rm_status st = check_common(dims, p, ws, ws_bytes, true);
  if (st != RM_OK) return st;
  if ((st = check_bwd_args(dims, x, dy, dx, g)) != RM_OK) return st;
  const WsLayout L = ws_layout(*dims);
  if (L.scratch_bytes > RM_STATIC_SCRATCH_BYTES) return RM_E_SCRATCH;
  void* sc = nullptr;
  if ((st = static_scratch(&sc)) != RM_OK) return st;
  return backward(*dims, p, x, dy, ws, sc, dx, g, reinterpret_cast<hipStream_t>(stream));
}

rm_status rm_token_mix(const rm_dims* dims, const void* in, void* out, void* stream) {
  if (!dims) return RM_E_NULL;
  if (dims->dtype != RM_F32 && dims->dtype != RM_BF16 && dims->dtype != RM_F16) return RM_E_DTYPE;
  if (!dims_valid(*dims)) return RM_E_DIMS;
  if (!in || !out) return RM_E_NULL;
  const size_t es = dims->dtype == RM_F32 ? 4 : 2;
  if (!aligned(in, es) || !aligned(out, es)) return RM_E_ALIGN;
  if (in == out || (dims->flags & ~RM_FLAG_MAIN_KERNELS)) return RM_E_ARG;
  return hip_status(launch_token_mix(*dims, in, out, reinterpret_cast<hipStream_t>(stream)));
}

rm_status rm_prof_enable(int on) {
  std::lock_guard<std::mutex> lk(g_mu);
  g_prof = on != 0;
  return RM_OK;
}

int rm_prof_kernels(void) { return KID_COUNT; }

const char* rm_prof_name(int id) { return (id >= 0 && id < KID_COUNT) ? kKernelNames[id] : nullptr; }

rm_status rm_prof_collect(double* ms, int64_t* launches, int n) {
  if (!ms || !launches) return RM_E_NULL;
  if (n < KID_COUNT) return RM_E_ARG;
  std::lock_guard<std::mutex> lk(g_mu);
  rm_status st = RM_OK;
  for (const ProfRec& r : g_recs) {
    float f = 0.f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&f, r.a, r.b) != hipSuccess) st = RM_E_HIP;
    ms[r.kid] += f;
    launches[r.kid] += 1;
    g_pool.push_back(r.a);
    g_pool.push_back(r.b);
  }
  g_recs.clear();
  return st;
}

}  // extern "C"
