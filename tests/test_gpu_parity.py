"""GPU parity: the HIP path through the C ABI against the float64 oracle.

Metric per tensor: max |gpu - oracle| / max |oracle|; bound 1e-4 for fp32
storage and 3e-2 for bf16 storage (fp32 accumulation in both).  Every output
must be finite.  Token mixing is compared bit for bit.
"""
import numpy as np
import pytest

import oracle
from rankmixer_inputs import WORKLOADS, as_f64, make_case, make_custom
from oracle_chunked import oracle_by_chunks
from rm_gpu import FULL_SIZE_REPORT, GRAD_KEYS, TOL, DeviceCase, compare, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import transformer_block_norm0_amd as rb
    rb.library()  # raises if the HIP library is not built: no fallback


def oracle_results(case):
    x, p, dy = as_f64(case)
    y, cache = oracle.forward(x, p)
    g = oracle.backward(dy, cache, p)
    g["y"] = y
    return g, cache


# ---------------------------------------------------------------------------
# token mixing, bit exact

@pytest.mark.parametrize("shape", [(1, 8, 64), (2, 64, 64), (3, 13, 65), (5, 8, 1280), (4, 16, 128),
                                   (7, 40, 1000)])
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_token_mix_bit_exact(shape, dtype):
    import torch
    import transformer_block_norm0_amd as rb
    B, T, D = shape
    say(f"token_mix {shape} {dtype}")
    rng = np.random.default_rng(B * 1000 + T + D)
    if dtype == "bf16":
        bits = rng.integers(0, 1 << 16, size=(B, T, D), dtype=np.uint16)
        bits.flat[:4] = [0x8000, 0x7FC1, 0xFF81, 0x7F80]   # -0.0, NaN payloads, +inf
        inp = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    elif dtype == "f16":
        bits = rng.integers(0, 1 << 16, size=(B, T, D), dtype=np.uint16)
        bits.flat[:4] = [0x8000, 0x7E01, 0xFE01, 0x7C00]   # -0.0, NaN payloads, +inf
        inp = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.float16)
    else:
        bits = rng.integers(0, 1 << 32, size=(B, T, D), dtype=np.uint32)
        bits.flat[:4] = [0x80000000, 0x7FC00001, 0xFF800123, 0x7F800000]
        inp = torch.from_numpy(bits.view(np.int32)).cuda().view(torch.float32)
    out = torch.empty_like(inp)
    rb.token_mix(rb.dims(B, T, D, 2, dtype), inp, out)
    torch.cuda.synchronize()
    iview = torch.int32 if dtype == "f32" else torch.int16
    got = out.view(iview).cpu().numpy().view(bits.dtype)
    S = D // T
    want = bits.reshape(B, T, T, S).swapaxes(1, 2).reshape(B, T, D)
    assert np.array_equal(got, want)


# ---------------------------------------------------------------------------
# full parity at sizes the oracle finishes in seconds

SMALL = [
    ("B8_T8_D64_k2_f32", None),
    ("B4_T16_D128_k2_f32_public", None),
    ("B4_T16_D128_k2_bf16_public", None),
    ("B256_T16_D256_k3_f32", None),
    ("B4_T16_D128_k2_f16_public", None),
    ("B256_T16_D256_k3_f16_lnrand", None),
]
EDGE = [  # (B, T, D, k): B=1 minimum dims; S=1; odd D (unaligned bf16 rows); S=160 and H=3840;
    # ragged tiles; the small-batch envelope's maximum (B*T = 512 rows, D = 128, H = 256); an
    # 80 KB 16-bit sample (the middle LDS tier of the sample-in-LDS prologue and tail)
    (1, 8, 64, 2), (2, 64, 64, 3), (3, 13, 65, 3), (5, 8, 1280, 3), (67, 16, 256, 2), (130, 8, 96, 3),
    (8, 64, 128, 2), (6, 32, 1280, 2)]


def check_case(case, intermediates=True, kernels="auto"):
    label = f"{case['name']} ({kernels} kernels)"
    say(f"case {label}: gpu fwd+bwd")
    dc = DeviceCase(case, kernels=kernels)
    dc.run()
    got = dc.results()
    say(f"case {label}: oracle")
    ref, cache = oracle_results(case)
    tol = TOL[case["dtype"]]
    if intermediates:
        d = case["dims"]
        h1 = dc.ws_region(0, (d.B, d.T, d.D), f32=False)
        compare({"h1": h1}, {"h1": cache["h1"]}, ["h1"], tol, label + " out1")
    keys = ["y"] + list(GRAD_KEYS)
    d = case["dims"]
    if d.S == 1:
        # With D/T == 1 every column of dbeta0 sums one norm1-backward row, which
        # is zero exactly: the max-normalised metric has no scale.  Check the
        # vanishing value against the summation bound tol * sum_rows |da0| instead.
        keys.remove("dln0_b")
        scale = dbeta0_summand_scale(case, cache)
        assert np.max(np.abs(ref["dln0_b"])) <= 1e-12 * scale
        err = float(np.max(np.abs(got["dln0_b"]))) / scale
        say(f"{label}: dln0_b (exact zero) |gpu|/sum|da0| = {err:.2e}")
        assert err <= tol
    compare(got, ref, keys, tol, label)
    assert got["y"].shape == case["x"].shape
    return dc


def dbeta0_summand_scale(case, cache):
    """max over columns of sum over rows of |da0|, da0 = token_mix(dr1), from the oracle's steps."""
    x, p, dy = as_f64(case)
    dr2, _, _ = oracle.mixer_epilogue_backward(dy, cache, p)
    dh1_ffn, _ = oracle.dense_ffn_backward(dr2, cache, p)
    c = cache["pro"]
    dr1, _, _ = oracle.layer_norm_backward(dr2 + dh1_ffn, c["n1"], c["rstd1"], p["ln1_g"])
    return float(np.max(np.abs(oracle.token_mix(dr1)).sum(axis=(0, 1))))


# ---------------------------------------------------------------------------
# the two kernel sets: shapes inside B <= 8, D <= 128, H <= 256 take the
# small-batch kernels by default; rm_dims.flags = RM_FLAG_MAIN_KERNELS ("main")
# sends a call through the main kernels.  "small" below names the default on
# such a shape.

def small_shape(B, D, k):
    return B <= 8 and D <= 128 and k * D <= 256


def kernel_flag(which):
    return "main" if which == "main" else "auto"


SMALL_RUNS = [(n, ks) for n, _ in SMALL for ks in ("main", "small")
              if ks == "main" or small_shape(WORKLOADS[n].dims.B, WORKLOADS[n].dims.D, WORKLOADS[n].dims.k)]
EDGE_RUNS = [(sh, ks) for sh in EDGE for ks in ("main", "small") if ks == "main" or small_shape(sh[0], sh[2], sh[3])]


@pytest.mark.parametrize("name,kernels", SMALL_RUNS)
def test_parity_small_workloads(name, kernels):
    check_case(make_case(WORKLOADS[name]), kernels=kernel_flag(kernels))


@pytest.mark.parametrize("shape,kernels", EDGE_RUNS)
@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_parity_edge_shapes(shape, kernels, dtype):
    B, T, D, k = shape
    check_case(make_custom(B, T, D, k, dtype, seed=B * 31 + T * 7 + D + k, ln_affine="random"),
               kernels=kernel_flag(kernels))


@pytest.mark.parametrize("fwd_set,bwd_set", [("small", "main"), ("main", "small")])
@pytest.mark.parametrize("name", ["B4_T16_D128_k2_bf16_public", "B8_T8_D64_k2_f32", "B4_T16_D128_k2_f16_public"])
def test_small_and_main_paths_interchange(name, fwd_set, bwd_set):
    """Both kernel sets save the same state in the workspace: either backward follows either forward."""
    import torch
    case = make_case(WORKLOADS[name])
    dc = DeviceCase(case)
    dc.fwd(kernels=kernel_flag(fwd_set))
    dc.bwd(kernels=kernel_flag(bwd_set))
    torch.cuda.synchronize()
    got = dc.results()
    ref, _ = oracle_results(case)
    compare(got, ref, ["y"] + list(GRAD_KEYS), TOL[case["dtype"]], f"{name} fwd {fwd_set} bwd {bwd_set}")


@pytest.mark.parametrize("shape,kernels", [((8, 64, 128, 2), "small"), ((8, 64, 128, 2), "main"),
                                            ((1, 8, 64, 2), "small"), ((3, 13, 65, 3), "small"),
                                            ((3, 13, 65, 3), "main"), ((67, 16, 256, 2), "main")])
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_writes_stay_inside_buffers(shape, kernels, dtype):
    """The workspace and every output live inside larger buffers with guard bytes on both sides:
    after fwd+bwd the guards are unchanged and the results still match the oracle."""
    import torch
    B, T, D, k = shape
    case = make_custom(B, T, D, k, dtype, seed=B * 17 + T + D + k, ln_affine="random")
    dc = DeviceCase(case, kernels=kernel_flag(kernels))
    G = 4096  # guard bytes on each side (a multiple of 256: the workspace stays 256-byte aligned)
    guards = []

    def guarded(t):
        nbytes = t.numel() * t.element_size()
        buf = torch.full((nbytes + 2 * G,), 0xA5, dtype=torch.uint8, device=t.device)
        guards.append(buf)
        return buf[G:G + nbytes].view(t.dtype).view(t.shape)

    dc.ws = guarded(dc.ws)
    dc.y, dc.dx = guarded(dc.y), guarded(dc.dx)
    dc.grads = {n: guarded(g) for n, g in dc.grads.items()}
    dc.run()
    for buf in guards:
        head, tail = buf[:G].cpu().numpy(), buf[-G:].cpu().numpy()
        assert np.all(head == 0xA5) and np.all(tail == 0xA5)
    ref, _ = oracle_results(case)
    compare(dc.results(), ref, ["y"] + list(GRAD_KEYS), TOL[case["dtype"]], f"{case['name']} guarded {kernels}")


def test_small_path_bitwise_repeatable():
    """Two fwd+bwd runs of the small-batch kernels on identical inputs give identical bits."""
    case = make_case(WORKLOADS["B4_T16_D128_k2_bf16_public"])
    a = DeviceCase(case)
    a.run()
    b = DeviceCase(case)
    b.run()
    ra, rb_ = a.raw_bits(), b.raw_bits()
    for k in ra:
        assert np.array_equal(ra[k], rb_[k]), k


def test_bitwise_repeatable():
    """Two fwd+bwd runs on identical inputs give identical bits (no atomics)."""
    case = make_custom(67, 16, 256, 2, "bf16", seed=3, ln_affine="random")
    dc = DeviceCase(case)
    dc.run()
    a = dc.raw_bits()
    dc.run()
    b = dc.raw_bits()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("shape", [(67, 16, 256, 2), (5, 8, 1280, 3)])
def test_misaligned_io_same_bits(shape):
    """Element-aligned (not 16-byte aligned) x, dy, y, dx give the same bits as aligned buffers:
    the kernels that stage a sample in LDS by 16-byte copies take their plain-load path."""
    B, T, D, k = shape
    say(f"misaligned io {shape} bf16")
    case = make_custom(B, T, D, k, "bf16", seed=5, ln_affine="random")
    a = DeviceCase(case)
    a.run()
    ra = a.raw_bits()
    m = DeviceCase(case)
    m.misalign()
    m.run()
    rm = m.raw_bits()
    for key in ra:
        assert np.array_equal(ra[key], rm[key]), key


def test_backward_repeatable_on_same_workspace():
    """The backward leaves the forward's saved state intact: a second call agrees bitwise."""
    import torch
    case = make_custom(5, 8, 1280, 3, "f32", seed=9)
    dc = DeviceCase(case)
    dc.run()
    a = dc.raw_bits()
    dc.bwd()
    torch.cuda.synchronize()
    b = dc.raw_bits()
    for k in a:
        assert np.array_equal(a[k], b[k]), k


# ---------------------------------------------------------------------------
# full-size workloads: the oracle checks sampled outputs exactly

def sampled_check(name, samples=(0, -1), tokens=(0, -1)):
    w = WORKLOADS[name]
    case = make_case(w)
    d = case["dims"]
    tol = TOL[case["dtype"]]
    say(f"case {name}: gpu fwd+bwd (full size)")
    dc = DeviceCase(case)
    dc.run()
    got = dc.results()
    x, p, dy = as_f64(case)
    # (1) whole samples: y[b] and dx[b] depend only on x[b], dy[b] and the parameters
    bs = sorted({s % d.B for s in samples})
    say(f"case {name}: oracle on samples {bs}")
    y_s, cache_s = oracle.forward(x[bs], p)
    g_s = oracle.backward(dy[bs], cache_s, p)
    compare({"y": got["y"][bs], "dx": got["dx"][bs]}, {"y": y_s, "dx": g_s["dx"]}, ["y", "dx"], tol,
            f"{name} samples {bs}")
    # (2) whole tokens: the per-token weight gradients need every sample at that token only
    ts = sorted({t % d.T for t in tokens})
    say(f"case {name}: oracle on tokens {ts}")
    h1, _ = oracle.mixer_prologue(x, p)
    sub = dict(p)
    for n in ("w1", "b1", "wout", "bout"):
        sub[n] = p[n][ts]
    h1_t = h1[:, ts, :]
    out2, c_ffn = oracle.dense_ffn(h1_t, sub)
    y_t, c_epi = oracle.mixer_epilogue(h1_t, out2, sub)
    cache = {"ffn": c_ffn, "epi": c_epi}
    dr2, _, _ = oracle.mixer_epilogue_backward(dy[:, ts, :], cache, sub)
    _, g_t = oracle.dense_ffn_backward(dr2, cache, sub)
    compare({"y": got["y"][:, ts, :], "dw1": got["dw1"][ts], "db1": got["db1"][ts],
             "dwout": got["dwout"][ts], "dbout": got["dbout"][ts]},
            {"y": y_t, "dw1": g_t["dw1"], "db1": g_t["db1"], "dwout": g_t["dwout"], "dbout": g_t["dbout"]},
            ["y", "dw1", "db1", "dwout", "dbout"], tol, f"{name} tokens {ts}")
    # (3) closed form at any size: dbeta2 = sum of dy over every row
    compare({"dln2_b": got["dln2_b"]}, {"dln2_b": dy.sum(axis=(0, 1))}, ["dln2_b"], tol, f"{name} dbeta2")
    for k, v in got.items():
        assert np.all(np.isfinite(v)), k


def full_check(case, chunk=64):
    """y and all 15 gradients against the unchanged oracle over every sample
    (run on chunks of samples, parameter gradients added in float64)."""
    d = case["dims"]
    name = case["name"]
    tol = TOL[case["dtype"]]
    assert d.S != 1   # dbeta0 would vanish exactly (check_case handles that case)
    say(f"case {name}: gpu fwd+bwd (full size)")
    dc = DeviceCase(case)
    dc.run()
    got = dc.results()
    del dc
    x, p, dy = as_f64(case)
    num = {"y": 0.0, "dx": 0.0}
    den = {"y": 0.0, "dx": 0.0}

    def visit(b0, b1, y_c, dx_c):
        say(f"case {name}: oracle on samples {b0}..{b1 - 1}")
        for key, ref in (("y", y_c), ("dx", dx_c)):
            g = got[key][b0:b1]
            assert np.all(np.isfinite(g)), key
            num[key] = max(num[key], float(np.max(np.abs(g - ref))))
            den[key] = max(den[key], float(np.max(np.abs(ref))))

    sums = oracle_by_chunks(x, p, dy, chunk, visit)
    errs = {k: num[k] / max(den[k], 1e-30) for k in num}
    errs.update(compare(got, sums, [k for k in GRAD_KEYS if k != "dx"], tol, f"{name} parameter gradients"))
    say(f"{name} all outputs: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    FULL_SIZE_REPORT.append((f"{name} [{case['dtype']}, tol {tol:g}]", errs))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{name}: over tolerance {tol}: {bad}"
    return errs


def test_full_size_B1024_T32_D512_k2_bf16():
    """Small enough for the complete oracle: every output and gradient compared."""
    check_case(make_case(WORKLOADS["B1024_T32_D512_k2_bf16_lnrand"]), intermediates=False)


@pytest.mark.timeout(900)
def test_full_size_B1024_T64_D1280_k2_bf16():
    """The production workload: y and all 15 gradients over every sample."""
    full_check(make_case(WORKLOADS["B1024_T64_D1280_k2_bf16"]))


@pytest.mark.timeout(900)
def test_full_size_B999_T40_D1000_k3_f32():
    """Ragged fp32 workload (D/T = 25, no dimension a multiple of the tiles): every output."""
    full_check(make_case(WORKLOADS["B999_T40_D1000_k3_f32_lnrand"]))


@pytest.mark.timeout(900)
@pytest.mark.parametrize("shape,dtype", [((1024, 40, 1000, 3), "bf16"), ((512, 16, 640, 3), "bf16"),
                                         ((384, 8, 384, 3), "bf16"), ((384, 8, 384, 3), "f16"),
                                         ((300, 8, 384, 3), "bf16")])
def test_tile_tails_16bit(shape, dtype):
    """16-bit shapes whose GEMMs take the 256x256-tile kernels with partial tiles:
    (1024,40,1000,3): both weight-gradient GEMMs with M and N tails (232/112, 184/232);
    (512,16,640,3) and (384,8,384,3): N tails of 128 on the down, d-hidden, dwout and d-out1
    GEMMs, M tails of 128 on the weight-gradient GEMMs, and (384,...) M tails of 128 on the
    row-major GEMMs; (300,8,384,3): M tails of 44 rows (not a multiple of 32) on those."""
    B, T, D, k = shape
    full_check(make_custom(B, T, D, k, dtype, seed=B + T + D + k + 11, ln_affine="random"))


def test_full_size_B1024_T64_D1280_k2_f16_sampled():
    """fp16 storage (page 1, "Run the benchmark": the --dtype float16 run) at the production shape."""
    sampled_check("B1024_T64_D1280_k2_f16", samples=(0, 300, -1), tokens=(0, 41, -1))


def test_full_size_envelope_maximum_sampled():
    """B, T, D and k all at the maximum of page 1's envelope ("Public checks and instructor
    coverage"): H = 3840 takes the general gate backward, random LayerNorm affines."""
    sampled_check("B1024_T64_D1280_k3_bf16_lnrand", samples=(0, 777, -1), tokens=(0, 29, -1))


@pytest.mark.parametrize("name", ["B4_T16_D128_k2_bf16_public", "B8_T8_D64_k2_f32", "B4_T16_D128_k2_f16_public"])
def test_graph_replay_matches_eager(name):
    """fwd+bwd captured once into a HIP graph: every replay, with eager work and
    cleared outputs and workspace in between, gives the eager run's bits."""
    import torch
    say(f"graph replay {name}")
    dc = DeviceCase(make_case(WORKLOADS[name]))
    dc.run()
    ref = dc.raw_bits()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        dc.fwd(side)
        dc.bwd(side)
    side.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        dc.fwd(side)
        dc.bwd(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in [dc.y, dc.dx, dc.ws] + list(dc.grads.values()):
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = dc.raw_bits()
        for k in ref:
            assert np.array_equal(ref[k], got[k]), (rep, k)
        dc.run()  # eager work between replays
    del g
