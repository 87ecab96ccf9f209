"""Float64 CPU oracle of the RankMixerBlock forward and backward pass.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import or call this module.  It shares no code with the
HIP path (transformer_block_norm0_amd/) and imports nothing from it.

Everything is float64 NumPy.  Inputs are the storage-dtype values (bf16 or
fp32) decoded to float64; no intermediate is rounded.

What it follows: "Subgraph-fusion-based Mega-kernel Generation" (page 1),
  * "Workload and interfaces": shapes of w1[T,D,2H], b1[T,2H], wout[T,H,D],
    bout[T,D], inner LayerNorm affines of H elements, outer ones of D elements,
    a same-shape upstream gradient, and the whole block is differentiated;
  * "Exact computation": the four-line block composition, outer LayerNorm with
    eps 1e-3, token mixing (reshape to [B,T,T,D/T], swap the two T axes,
    reshape back), and the dense subgraph (per-token up-projection, split into
    U and G, LN_x(U) * silu(LN_gate(G)), per-token down-projection) with inner
    PyTorch LayerNorm eps 1e-5.

Readings taken where the page leaves a step open:
  * the LayerNorm formula's flattened parentheses are read as the textbook
    form (z - mean) / sqrt(biased variance + eps), eps inside the root;
  * "NezhaLayerNorm" (the outer norms) is that same formula with eps 1e-3;
  * U is the first H columns of Z and G the last H;
  * silu(v) = v * sigmoid(v);
  * the residual into norm2 is the rebound out1, i.e. the output of norm1;
  * the two inner LayerNorm affines are shared by all T tokens.

The backward is derived by hand from the forward (chain rule, step by step in
reverse order); tests pin it to central finite differences and to PyTorch's
autograd in float64.
"""
from __future__ import annotations

import numpy as np

EPS_OUTER = 1e-3   # norm0, norm1, norm2 ("Exact computation")
EPS_INNER = 1e-5   # norm_x, norm_gate ("Exact computation")

GRAD_NAMES = ("dx", "dw1", "db1", "dwout", "dbout",
              "dlnx_g", "dlnx_b", "dlng_g", "dlng_b",
              "dln0_g", "dln0_b", "dln1_g", "dln1_b", "dln2_g", "dln2_b")


# ---------------------------------------------------------------------------
# building blocks

def layer_norm(z, gamma, beta, eps):
    """LayerNorm over the last axis: ((z - mean) / sqrt(mean((z - mean)^2) + eps)) * gamma + beta.

    Page 1, "Exact computation", the LN(z) line of the dense subgraph.
    Returns (out, n, mean, rstd) with n the normalised value before the affine.
    """
    mean = z.mean(axis=-1, keepdims=True)
    var = ((z - mean) ** 2).mean(axis=-1, keepdims=True)
    rstd = 1.0 / np.sqrt(var + eps)
    n = (z - mean) * rstd
    return n * gamma + beta, n, mean[..., 0], rstd[..., 0]


def layer_norm_backward(dout, n, rstd, gamma):
    """Gradient of layer_norm given the upstream gradient `dout`.

    With n = (z - mean) * rstd and out = n * gamma + beta:
      dgamma = sum over rows of dout * n,  dbeta = sum over rows of dout,
      dn = dout * gamma,
      dz = rstd * (dn - mean(dn) - n * mean(dn * n))   (means over the row).
    Returns (dz, dgamma, dbeta); the parameter grads sum over every leading axis.
    """
    lead = tuple(range(dout.ndim - 1))
    dgamma = (dout * n).sum(axis=lead)
    dbeta = dout.sum(axis=lead)
    dn = dout * gamma
    dz = rstd[..., None] * (dn - dn.mean(axis=-1, keepdims=True)
                            - n * (dn * n).mean(axis=-1, keepdims=True))
    return dz, dgamma, dbeta


def token_mix(a):
    """reshape [B,T,D] -> [B,T,T,D/T], swap the two T axes, reshape back.

    Page 1, "Exact computation" (token mixing paragraph and its [1,2,4] example).
    The map is a permutation that is its own inverse and its own transpose.
    """
    B, T, D = a.shape
    if D % T:
        raise ValueError("token mixing needs D % T == 0")
    return a.reshape(B, T, T, D // T).swapaxes(1, 2).reshape(B, T, D)


def sigmoid(v):
    return 1.0 / (1.0 + np.exp(-v))


def silu(v):
    """silu(v) = v * sigmoid(v)."""
    return v * sigmoid(v)


# ---------------------------------------------------------------------------
# forward, in the page's order

def mixer_prologue(x, p):
    """out1 = norm1(token_mixer(norm0(x)) + x).  Page 1, "Exact computation", lines 1-2."""
    a0, n0, mu0, rstd0 = layer_norm(x, p["ln0_g"], p["ln0_b"], EPS_OUTER)
    m = token_mix(a0)
    r1 = m + x
    h1, n1, mu1, rstd1 = layer_norm(r1, p["ln1_g"], p["ln1_b"], EPS_OUTER)
    cache = {"n0": n0, "mu0": mu0, "rstd0": rstd0, "n1": n1, "mu1": mu1, "rstd1": rstd1}
    return h1, cache


def dense_ffn(h1, p):
    """dense_ffn_v2_compute: page 1, "Exact computation", the dense subgraph.

    Z[b,t,:] = h1[b,t,:] @ w1[t] + b1[t];  (U, G) = halves of Z;
    hidden = LN_x(U) * silu(LN_gate(G));  out[b,t,:] = hidden[b,t,:] @ wout[t] + bout[t].
    Works for any number of tokens as long as the per-token parameters match.
    """
    H = p["wout"].shape[1]
    ht = np.ascontiguousarray(h1.transpose(1, 0, 2))            # [T,B,D]
    Z = np.matmul(ht, p["w1"]) + p["b1"][:, None, :]             # [T,B,2H]
    U, G = Z[..., :H], Z[..., H:]
    ux, nx, mux, rstdx = layer_norm(U, p["lnx_g"], p["lnx_b"], EPS_INNER)
    ug, ng, mug, rstdg = layer_norm(G, p["lng_g"], p["lng_b"], EPS_INNER)
    hidden = ux * silu(ug)
    out = np.matmul(hidden, p["wout"]) + p["bout"][:, None, :]   # [T,B,D]
    cache = {"ht": ht, "nx": nx, "rstdx": rstdx, "mux": mux, "ux": ux,
             "ng": ng, "rstdg": rstdg, "mug": mug, "ug": ug, "hidden": hidden, "Z": Z}
    return np.ascontiguousarray(out.transpose(1, 0, 2)), cache


def mixer_epilogue(h1, out2, p):
    """output = norm2(out1 + out2).  Page 1, "Exact computation", line 4."""
    r2 = h1 + out2
    y, n2, mu2, rstd2 = layer_norm(r2, p["ln2_g"], p["ln2_b"], EPS_OUTER)
    return y, {"n2": n2, "mu2": mu2, "rstd2": rstd2}


def forward(x, p):
    """Whole block forward.  Returns (y, cache)."""
    h1, c_pro = mixer_prologue(x, p)
    out2, c_ffn = dense_ffn(h1, p)
    y, c_epi = mixer_epilogue(h1, out2, p)
    return y, {"pro": c_pro, "ffn": c_ffn, "epi": c_epi, "h1": h1, "out2": out2}


# ---------------------------------------------------------------------------
# backward, the same steps in reverse

def mixer_epilogue_backward(dy, cache, p):
    """Through norm2: returns (dr2, dln2_g, dln2_b); dr2 flows to both out1 and out2."""
    c = cache["epi"]
    return layer_norm_backward(dy, c["n2"], c["rstd2"], p["ln2_g"])


def dense_ffn_backward(dout, cache, p):
    """Gradient of dense_ffn for upstream `dout` [B,T,D].

    Returns (dh1, grads) with grads holding dw1, db1, dwout, dbout and the four
    inner LayerNorm affine grads.
    """
    c = cache["ffn"]
    dot = np.ascontiguousarray(dout.transpose(1, 0, 2))          # [T,B,D]
    g = {}
    g["dbout"] = dot.sum(axis=1)
    g["dwout"] = np.matmul(c["hidden"].transpose(0, 2, 1), dot)
    dhid = np.matmul(dot, p["wout"].transpose(0, 2, 1))          # [T,B,H]
    sg = sigmoid(c["ug"])
    dux = dhid * (c["ug"] * sg)                                   # d LN_x(U)
    dug = dhid * c["ux"] * sg * (1.0 + c["ug"] * (1.0 - sg))     # d LN_gate(G), silu'
    dU, g["dlnx_g"], g["dlnx_b"] = layer_norm_backward(dux, c["nx"], c["rstdx"], p["lnx_g"])
    dG, g["dlng_g"], g["dlng_b"] = layer_norm_backward(dug, c["ng"], c["rstdg"], p["lng_g"])
    dZ = np.concatenate([dU, dG], axis=-1)                        # [T,B,2H]
    g["db1"] = dZ.sum(axis=1)
    g["dw1"] = np.matmul(c["ht"].transpose(0, 2, 1), dZ)
    dht = np.matmul(dZ, p["w1"].transpose(0, 2, 1))              # [T,B,D]
    return np.ascontiguousarray(dht.transpose(1, 0, 2)), g


def mixer_prologue_backward(dh1, cache, p):
    """Through norm1, the residual, token mixing and norm0.  Returns (dx, grads)."""
    c = cache["pro"]
    g = {}
    dr1, g["dln1_g"], g["dln1_b"] = layer_norm_backward(dh1, c["n1"], c["rstd1"], p["ln1_g"])
    da0 = token_mix(dr1)             # adjoint of the token permutation is itself
    dx0, g["dln0_g"], g["dln0_b"] = layer_norm_backward(da0, c["n0"], c["rstd0"], p["ln0_g"])
    return dr1 + dx0, g


def backward(dy, cache, p):
    """Whole block backward for upstream gradient dy.  Returns a dict of GRAD_NAMES."""
    dr2, dg2, db2 = mixer_epilogue_backward(dy, cache, p)
    dh1_ffn, g_ffn = dense_ffn_backward(dr2, cache, p)
    dh1 = dr2 + dh1_ffn              # out1 feeds both the FFN and the norm2 residual
    dx, g_pro = mixer_prologue_backward(dh1, cache, p)
    grads = {"dx": dx, "dln2_g": dg2, "dln2_b": db2}
    grads.update(g_ffn)
    grads.update(g_pro)
    return grads


def forward_backward(x, p, dy):
    y, cache = forward(x, p)
    return y, backward(dy, cache, p)
