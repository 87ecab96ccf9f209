"""Pins of the float64 oracle to facts other than itself (CPU only).

Each test names what fixes the expected value: the pages' worked example,
a textbook / library routine (PyTorch float64 LayerNorm, SiLU, autograd),
brute-force index loops on tiny inputs, closed forms, invariants, or central
finite differences.  A plausible slip in the oracle (a dropped term, a wrong
sign or index, a transposed operand, the wrong residual) fails at least one.
"""
import os

import numpy as np
import pytest

import oracle
from rankmixer_inputs import Dims, as_f64, make_custom

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rand_params(dims: Dims, rng, ln_random=True):
    T, D, H = dims.T, dims.D, dims.H
    p = {
        "w1": rng.standard_normal((T, D, 2 * H)) / np.sqrt(D),
        "b1": rng.standard_normal((T, 2 * H)) * 0.3,
        "wout": rng.standard_normal((T, H, D)) / np.sqrt(H),
        "bout": rng.standard_normal((T, D)) * 0.3,
    }
    for ln, n in (("ln0", D), ("ln1", D), ("ln2", D), ("lnx", H), ("lng", H)):
        if ln_random:
            p[ln + "_g"] = rng.uniform(0.5, 1.5, n)
            p[ln + "_b"] = rng.uniform(-0.3, 0.3, n)
        else:
            p[ln + "_g"] = np.ones(n)
            p[ln + "_b"] = np.zeros(n)
    return p


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = [int(v) for v in vals]
    return out


# ---------------------------------------------------------------------------
# token mixing

def test_token_mix_worked_example():
    """Page 1, "Exact computation": [[0,1,2,3],[4,5,6,7]] -> [[0,1,4,5],[2,3,6,7]]."""
    g = read_golden("token_mix_example.txt")
    shape = tuple(g["shape"])
    a = np.array(g["input"], dtype=np.float64).reshape(shape)
    want = np.array(g["expected"], dtype=np.float64).reshape(shape)
    assert np.array_equal(oracle.token_mix(a), want)


@pytest.mark.parametrize("B,T,D", [(1, 2, 4), (2, 4, 16), (1, 8, 64), (3, 5, 15), (2, 8, 8)])
def test_token_mix_brute_force_index_map(B, T, D):
    """Element-by-element loops: out[b,i,j*S+s] = in[b,j,i*S+s]."""
    S = D // T
    a = np.arange(B * T * D, dtype=np.float64).reshape(B, T, D)
    want = np.empty_like(a)
    for b in range(B):
        for i in range(T):
            for j in range(T):
                for s in range(S):
                    want[b, i, j * S + s] = a[b, j, i * S + s]
    assert np.array_equal(oracle.token_mix(a), want)


def test_token_mix_involution_adjoint_and_per_sample_multiset():
    rng = np.random.default_rng(0)
    a = rng.standard_normal((3, 8, 64))
    c = rng.standard_normal((3, 8, 64))
    m = oracle.token_mix(a)
    assert np.array_equal(oracle.token_mix(m), a)
    assert np.isclose(np.sum(m * c), np.sum(a * oracle.token_mix(c)), rtol=1e-13)
    for b in range(3):
        assert np.array_equal(np.sort(m[b].ravel()), np.sort(a[b].ravel()))
    # S == 1 (T == D): a plain transpose of each sample's T x T matrix
    sq = rng.standard_normal((2, 16, 16))
    assert np.array_equal(oracle.token_mix(sq), sq.transpose(0, 2, 1))


# ---------------------------------------------------------------------------
# LayerNorm

@pytest.mark.parametrize("eps", [oracle.EPS_OUTER, oracle.EPS_INNER])
def test_layer_norm_matches_torch_float64(eps):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    z = rng.standard_normal((5, 7, 96)) * 0.2 + 0.5
    g, b = rng.uniform(0.5, 1.5, 96), rng.uniform(-0.2, 0.2, 96)
    out, n, mu, rstd = oracle.layer_norm(z, g, b, eps)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(z), (96,), torch.from_numpy(g),
                                         torch.from_numpy(b), eps).numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)


def test_layer_norm_invariants():
    rng = np.random.default_rng(2)
    eps = 1e-3
    z = rng.standard_normal((4, 64)) * rng.uniform(0.01, 3.0, (4, 1)) + 2.0
    out, n, mu, rstd = oracle.layer_norm(z, np.ones(64), np.zeros(64), eps)
    var = z.var(axis=-1)
    np.testing.assert_allclose(n.mean(axis=-1), 0.0, atol=1e-14)
    np.testing.assert_allclose((n ** 2).mean(axis=-1), var / (var + eps), rtol=1e-12)
    np.testing.assert_array_equal(out, n)                      # unit affine is the identity
    const = np.full((2, 32), 3.25)
    beta = rng.standard_normal(32)
    out_c, *_ = oracle.layer_norm(const, rng.standard_normal(32), beta, eps)
    np.testing.assert_allclose(out_c, np.broadcast_to(beta, (2, 32)), atol=1e-15)


def test_layer_norm_backward_finite_differences_and_shift_invariance():
    rng = np.random.default_rng(3)
    z = rng.standard_normal((3, 40))
    g, b = rng.uniform(0.5, 1.5, 40), rng.uniform(-1, 1, 40)
    dout = rng.standard_normal((3, 40))
    _, n, _, rstd = oracle.layer_norm(z, g, b, 1e-3)
    dz, dg, db = oracle.layer_norm_backward(dout, n, rstd, g)
    np.testing.assert_allclose(dz.sum(axis=-1), 0.0, atol=1e-12)
    h = 1e-6

    def L(z_, g_, b_):
        return np.sum(dout * oracle.layer_norm(z_, g_, b_, 1e-3)[0])
    for arr, grad in ((z, dz), (g, dg), (b, db)):
        v = rng.standard_normal(arr.shape)
        args_p = [z, g, b]
        args_m = [z, g, b]
        idx = [id(z), id(g), id(b)].index(id(arr))
        args_p = list(args_p); args_m = list(args_m)
        args_p[idx] = arr + h * v
        args_m[idx] = arr - h * v
        fd = (L(*args_p) - L(*args_m)) / (2 * h)
        assert np.isclose(fd, np.sum(grad * v), rtol=1e-7, atol=1e-9)


# ---------------------------------------------------------------------------
# SiLU

def test_silu_matches_torch_and_special_values():
    torch = pytest.importorskip("torch")
    v = np.linspace(-30, 30, 1001)
    ref = torch.nn.functional.silu(torch.from_numpy(v)).numpy()
    np.testing.assert_allclose(oracle.silu(v), ref, rtol=1e-13, atol=1e-300)
    assert oracle.silu(np.array(0.0)) == 0.0
    h = 1e-6
    d0 = (oracle.silu(np.array(h)) - oracle.silu(np.array(-h))) / (2 * h)
    assert abs(d0 - 0.5) < 1e-10


# ---------------------------------------------------------------------------
# forward composition, brute force on tiny inputs

def brute_forward(x, p):
    """The page's four block lines and dense subgraph with explicit Python loops.

    Shares only the LayerNorm row helper (itself pinned above against PyTorch).
    """
    B, T, D = x.shape
    H = p["wout"].shape[1]
    S = D // T

    def ln_row(v, g, b, eps):
        mu = sum(v) / len(v)
        var = sum((e - mu) ** 2 for e in v) / len(v)
        return [((e - mu) / np.sqrt(var + eps)) * gg + bb for e, gg, bb in zip(v, g, b)]

    y = np.zeros_like(x)
    for b in range(B):
        a0 = [ln_row(list(x[b, j]), p["ln0_g"], p["ln0_b"], 1e-3) for j in range(T)]
        h1 = []
        for i in range(T):
            r1 = [a0[c // S][i * S + c % S] + x[b, i, c] for c in range(D)]
            h1.append(ln_row(r1, p["ln1_g"], p["ln1_b"], 1e-3))
        for t in range(T):
            Z = [sum(h1[t][d] * p["w1"][t, d, n] for d in range(D)) + p["b1"][t, n]
                 for n in range(2 * H)]
            ux = ln_row(Z[:H], p["lnx_g"], p["lnx_b"], 1e-5)
            ug = ln_row(Z[H:], p["lng_g"], p["lng_b"], 1e-5)
            hid = [u * (g / (1 + np.exp(-g))) for u, g in zip(ux, ug)]
            o2 = [sum(hid[h] * p["wout"][t, h, n] for h in range(H)) + p["bout"][t, n]
                  for n in range(D)]
            y[b, t] = ln_row([h1[t][n] + o2[n] for n in range(D)], p["ln2_g"], p["ln2_b"], 1e-3)
    return y


@pytest.mark.parametrize("B,T,D,k", [(1, 2, 4, 2), (2, 4, 8, 3)])
def test_forward_brute_force_loops(B, T, D, k):
    rng = np.random.default_rng(4)
    dims = Dims(B, T, D, k)
    p = rand_params(dims, rng)
    x = rng.standard_normal((B, T, D))
    y, _ = oracle.forward(x, p)
    np.testing.assert_allclose(y, brute_forward(x, p), rtol=1e-11, atol=1e-11)


def test_forward_special_case_zero_ffn_weights():
    """w1 = 0, b1 = 0 and beta_x = 0 make hidden = 0, so y = norm2(out1 + bout)."""
    rng = np.random.default_rng(5)
    dims = Dims(2, 4, 16, 2)
    p = rand_params(dims, rng)
    p["w1"][:] = 0.0
    p["b1"][:] = 0.0
    p["lnx_b"][:] = 0.0
    x = rng.standard_normal((2, 4, 16))
    y, _ = oracle.forward(x, p)
    # out1 written without the oracle's prologue: loops for token mixing, torch for LayerNorm
    torch = pytest.importorskip("torch")
    ln = lambda v, g, b: torch.nn.functional.layer_norm(
        torch.from_numpy(v), (v.shape[-1],), torch.from_numpy(g), torch.from_numpy(b), 1e-3).numpy()
    a0 = ln(x, p["ln0_g"], p["ln0_b"])
    S = 4
    m = np.empty_like(a0)
    for b in range(2):
        for i in range(4):
            for c in range(16):
                m[b, i, c] = a0[b, c // S, i * S + c % S]
    out1 = ln(m + x, p["ln1_g"], p["ln1_b"])
    want = ln(out1 + p["bout"][None], p["ln2_g"], p["ln2_b"])
    np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)


def test_forward_zero_norm0_affine_reduces_prologue():
    """gamma0 = beta0 = 0 removes the token-mixing branch: out1 = norm1(x)."""
    rng = np.random.default_rng(6)
    dims = Dims(2, 4, 16, 2)
    p = rand_params(dims, rng)
    p["ln0_g"][:] = 0.0
    p["ln0_b"][:] = 0.0
    x = rng.standard_normal((2, 4, 16))
    h1, _ = oracle.mixer_prologue(x, p)
    torch = pytest.importorskip("torch")
    want = torch.nn.functional.layer_norm(torch.from_numpy(x), (16,), torch.from_numpy(p["ln1_g"]),
                                          torch.from_numpy(p["ln1_b"]), 1e-3).numpy()
    np.testing.assert_allclose(h1, want, rtol=1e-12, atol=1e-12)


def test_per_token_locality_and_per_sample_independence():
    rng = np.random.default_rng(7)
    dims = Dims(3, 4, 16, 2)
    p = rand_params(dims, rng)
    x = rng.standard_normal((3, 4, 16))
    dy = rng.standard_normal((3, 4, 16))
    y, g = oracle.forward_backward(x, p, dy)
    # perturbing token 2's FFN weights changes only y[:, 2, :]
    q = {k: v.copy() for k, v in p.items()}
    q["w1"][2] += 0.1 * rng.standard_normal(q["w1"][2].shape)
    q["wout"][2] += 0.1 * rng.standard_normal(q["wout"][2].shape)
    y2, _ = oracle.forward(x, q)
    changed = np.abs(y2 - y).max(axis=(0, 2)) > 0
    assert list(changed) == [False, False, True, False]
    # permuting the batch permutes y and dx and leaves parameter grads unchanged
    perm = np.array([2, 0, 1])
    yp, gp = oracle.forward_backward(x[perm], p, dy[perm])
    np.testing.assert_allclose(yp, y[perm], rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(gp["dx"], g["dx"][perm], rtol=1e-12, atol=1e-12)
    for name in oracle.GRAD_NAMES[1:]:
        np.testing.assert_allclose(gp[name], g[name], rtol=1e-10, atol=1e-10)


# ---------------------------------------------------------------------------
# backward

def _loss(x, p, dy):
    return float(np.sum(dy * oracle.forward(x, p)[0]))


@pytest.mark.parametrize("B,T,D,k", [(1, 2, 4, 2), (2, 4, 16, 2), (2, 8, 64, 3)])
def test_backward_central_finite_differences(B, T, D, k):
    """All 15 gradient tensors against fp64 central differences of <dy, y>."""
    rng = np.random.default_rng(100 + B * T + D)
    dims = Dims(B, T, D, k)
    p = rand_params(dims, rng)
    x = rng.standard_normal((B, T, D))
    dy = rng.standard_normal((B, T, D))
    _, g = oracle.forward_backward(x, p, dy)
    h = 1e-6
    for gname in oracle.GRAD_NAMES:
        name = gname[1:]
        base = x if name == "x" else p[name]
        v = rng.standard_normal(base.shape)

        def shifted(s):
            if name == "x":
                return _loss(x + s * v, p, dy)
            q = dict(p)
            q[name] = p[name] + s * v
            return _loss(x, q, dy)
        fd = (shifted(h) - shifted(-h)) / (2 * h)
        an = float(np.sum(g[gname] * v))
        assert np.isclose(fd, an, rtol=2e-6, atol=1e-8), (gname, fd, an)
        # one spot element as well
        idx = tuple(int(rng.integers(0, s)) for s in base.shape)
        e = np.zeros(base.shape)
        e[idx] = 1.0
        v = e

        def shifted_e(s):
            if name == "x":
                return _loss(x + s * e, p, dy)
            q = dict(p)
            q[name] = p[name] + s * e
            return _loss(x, q, dy)
        fd_e = (shifted_e(h) - shifted_e(-h)) / (2 * h)
        assert np.isclose(fd_e, g[gname][idx], rtol=2e-5, atol=1e-8), (gname, idx, fd_e, g[gname][idx])


def test_backward_matches_torch_autograd_float64():
    """An independent PyTorch composition differentiated by autograd (library routine)."""
    torch = pytest.importorskip("torch")
    F = torch.nn.functional
    rng = np.random.default_rng(8)
    dims = Dims(3, 8, 64, 3)
    B, T, D, H = dims.B, dims.T, dims.D, dims.H
    p = rand_params(dims, rng)
    x = rng.standard_normal((B, T, D))
    dy = rng.standard_normal((B, T, D))
    _, g = oracle.forward_backward(x, p, dy)
    tp = {k: torch.tensor(v, requires_grad=True) for k, v in p.items()}
    tx = torch.tensor(x, requires_grad=True)
    a0 = F.layer_norm(tx, (D,), tp["ln0_g"], tp["ln0_b"], 1e-3)
    m = a0.reshape(B, T, T, D // T).transpose(1, 2).reshape(B, T, D)
    out1 = F.layer_norm(m + tx, (D,), tp["ln1_g"], tp["ln1_b"], 1e-3)
    Z = torch.einsum("btd,tdn->btn", out1, tp["w1"]) + tp["b1"]
    U, G = Z.split(H, dim=-1)
    hid = F.layer_norm(U, (H,), tp["lnx_g"], tp["lnx_b"], 1e-5) * F.silu(
        F.layer_norm(G, (H,), tp["lng_g"], tp["lng_b"], 1e-5))
    out2 = torch.einsum("bth,thd->btd", hid, tp["wout"]) + tp["bout"]
    y = F.layer_norm(out1 + out2, (D,), tp["ln2_g"], tp["ln2_b"], 1e-3)
    y.backward(torch.tensor(dy))
    np.testing.assert_allclose(g["dx"], tx.grad.numpy(), rtol=1e-9, atol=1e-11)
    for name in oracle.GRAD_NAMES[1:]:
        np.testing.assert_allclose(g[name], tp[name[1:]].grad.numpy(), rtol=1e-9, atol=1e-11,
                                   err_msg=name)


def test_backward_zero_gamma2_special_case():
    """gamma2 = 0 blocks every path except norm2's affine: only dgamma2, dbeta2 survive."""
    rng = np.random.default_rng(9)
    dims = Dims(2, 4, 16, 2)
    p = rand_params(dims, rng)
    p["ln2_g"][:] = 0.0
    x = rng.standard_normal((2, 4, 16))
    dy = rng.standard_normal((2, 4, 16))
    _, cache = oracle.forward(x, p)
    g = oracle.backward(dy, cache, p)
    n2 = cache["epi"]["n2"]
    for name in oracle.GRAD_NAMES:
        if name == "dln2_g":
            np.testing.assert_allclose(g[name], (dy * n2).sum(axis=(0, 1)), rtol=1e-13)
        elif name == "dln2_b":
            np.testing.assert_allclose(g[name], dy.sum(axis=(0, 1)), rtol=1e-13)
        else:
            assert np.all(g[name] == 0.0), name


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
def test_generated_case_runs_and_is_finite(dtype):
    case = make_custom(2, 8, 64, 2, dtype, seed=11)
    x, p, dy = as_f64(case)
    y, g = oracle.forward_backward(x, p, dy)
    assert y.shape == x.shape
    assert np.all(np.isfinite(y))
    for name in oracle.GRAD_NAMES:
        assert np.all(np.isfinite(g[name])), name


def test_f16_storage_rounding():
    """fp16 storage: exactly representable values round-trip; a value halfway
    between two fp16 neighbours goes to the even one; overflow gives inf."""
    from rankmixer_inputs import storage_to_f64, to_storage
    exact = np.array([0.0, -0.0, 1.0, -2.5, 65504.0, 2.0 ** -24, 1.0 + 2.0 ** -10])
    bits = to_storage(exact, "f16")
    assert bits.dtype == np.uint16
    np.testing.assert_array_equal(storage_to_f64(bits, "f16"), exact)
    assert bits[1] == 0x8000 and bits[2] == 0x3C00 and bits[4] == 0x7BFF and bits[5] == 0x0001
    # 1 + 2^-11 lies halfway between 1 (even mantissa) and 1 + 2^-10: rounds to 1
    # 1 + 3*2^-11 lies halfway between 1 + 2^-10 (odd) and 1 + 2^-9 (even): rounds up
    half = to_storage(np.array([1.0 + 2.0 ** -11, 1.0 + 3 * 2.0 ** -11]), "f16")
    np.testing.assert_array_equal(storage_to_f64(half, "f16"), [1.0, 1.0 + 2.0 ** -9])
    assert storage_to_f64(to_storage(np.array([70000.0]), "f16"), "f16")[0] == np.inf


def test_chunked_oracle_equals_whole_batch():
    """The chunked run the large-workload parity tests use gives the whole-batch
    oracle's outputs: y and dx chunk by chunk, parameter gradients as sums."""
    import sys
    sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
    from oracle_chunked import oracle_by_chunks
    case = make_custom(11, 8, 64, 3, "f32", seed=21, ln_affine="random")
    x, p, dy = as_f64(case)
    y, g = oracle.forward_backward(x, p, dy)
    seen = []

    def visit(b0, b1, y_c, dx_c):
        seen.append((b0, b1))
        np.testing.assert_allclose(y_c, y[b0:b1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(dx_c, g["dx"][b0:b1], rtol=0, atol=1e-12)

    sums = oracle_by_chunks(x, p, dy, 4, visit)
    assert seen == [(0, 4), (4, 8), (8, 11)]
    assert set(sums) == set(g) - {"dx"}
    for k, v in sums.items():
        scale = max(1.0, float(np.max(np.abs(g[k]))))
        np.testing.assert_allclose(v, g[k], rtol=0, atol=1e-12 * scale, err_msg=k)
