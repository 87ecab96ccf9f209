"""Seeded synthetic inputs for the RankMixerBlock forward+backward workload.

This module only draws random numbers and rounds them to the storage dtype.
It holds none of the block's arithmetic, so both the float64 oracle and the
HIP path can take their inputs from here without sharing any of the method.

What it follows ("Subgraph-fusion-based Mega-kernel Generation", page 1):
  * section "Workload and interfaces": parameter shapes w1[T,D,2H], b1[T,2H],
    wout[T,H,D], bout[T,D], two H-element inner LayerNorm affines, three
    D-element outer LayerNorm affines, input and upstream gradient [B,T,D];
  * section "Exact computation", last paragraph: the he-uniform initializer
    (fan_in is the product of all but the last dimension, values uniform in
    +-sqrt(6/fan_in)) for weights and biases, LayerNorm gamma=1 / beta=0,
    input drawn after the model, upstream gradient from its own generator
    seeded with seed+1000;
  * section "Public checks and instructor coverage": the dimension envelope
    1<=B<=1024, 8<=T<=64, 64<=D<=1280, D%T==0, k in {2,3}.

The pages' own random streams (torch's CPU and CUDA generators) cannot be
reproduced without their runner, so NumPy's PCG64 stands in with a fixed draw
order: w1, b1, wout, bout, then (only when random LayerNorm affines are asked
for) gamma/beta of norm0, norm1, norm2, norm_x, norm_gate, then x; dy comes
from PCG64(seed + 1000).  Values are drawn in float64 and rounded once to the
storage dtype (round-to-nearest-even); bf16 and fp16 are carried as uint16 bit
patterns.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np

PARAM_NAMES = (
    "w1", "b1", "wout", "bout",
    "lnx_g", "lnx_b", "lng_g", "lng_b",
    "ln0_g", "ln0_b", "ln1_g", "ln1_b", "ln2_g", "ln2_b",
)

DTYPES = ("f32", "bf16", "f16")


@dataclasses.dataclass(frozen=True)
class Dims:
    B: int
    T: int
    D: int
    k: int

    @property
    def H(self) -> int:
        return self.k * self.D

    @property
    def S(self) -> int:
        return self.D // self.T


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: shape, storage dtype, seed, LayerNorm affine mode."""
    name: str
    dims: Dims
    dtype: str            # "f32", "bf16" or "f16"
    seed: int
    ln_affine: str        # "unit" (gamma=1, beta=0) or "random" (U[0.5,1.5] / U[-0.1,0.1])


def _w(name, B, T, D, k, dtype, seed, ln):
    return Workload(name, Dims(B, T, D, k), dtype, seed, ln)


# The workloads this repository measures and tests.  Names state sizes and dtype.
WORKLOADS = {w.name: w for w in (
    _w("B8_T8_D64_k2_f32", 8, 8, 64, 2, "f32", 1, "unit"),
    _w("B256_T16_D256_k3_f32", 256, 16, 256, 3, "f32", 2, "unit"),
    _w("B1024_T32_D512_k2_bf16_lnrand", 1024, 32, 512, 2, "bf16", 3, "random"),
    _w("B1024_T64_D1280_k2_bf16", 1024, 64, 1280, 2, "bf16", 4, "unit"),
    _w("B999_T40_D1000_k3_f32_lnrand", 999, 40, 1000, 3, "f32", 5, "random"),
    # the pages' public check shape and seed (page 1, "Public checks and instructor coverage")
    _w("B4_T16_D128_k2_f32_public", 4, 16, 128, 2, "f32", 7101, "unit"),
    _w("B4_T16_D128_k2_bf16_public", 4, 16, 128, 2, "bf16", 7101, "unit"),
    # fp16 storage (page 1, "Run the benchmark": the --dtype float16 run)
    _w("B4_T16_D128_k2_f16_public", 4, 16, 128, 2, "f16", 7101, "unit"),
    _w("B256_T16_D256_k3_f16_lnrand", 256, 16, 256, 3, "f16", 8, "random"),
    _w("B1024_T64_D1280_k2_f16", 1024, 64, 1280, 2, "f16", 6, "unit"),
    # every dimension at the envelope's maximum (H = 3840)
    _w("B1024_T64_D1280_k3_bf16_lnrand", 1024, 64, 1280, 3, "bf16", 9, "random"),
)}

PRODUCTION = "B1024_T64_D1280_k2_bf16"


def in_envelope(d: Dims) -> bool:
    """The pages' held-out dimension envelope (page 1, "Public checks and instructor coverage")."""
    return (1 <= d.B <= 1024 and 8 <= d.T <= 64 and 64 <= d.D <= 1280
            and d.D % d.T == 0 and d.k in (2, 3))


# ---------------------------------------------------------------------------
# storage rounding (bf16 and fp16 as uint16 bit patterns)

def f64_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (through float32, both round-to-nearest-even)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def to_storage(a64: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(a64, dtype=np.float32)
    if dtype == "bf16":
        return f64_to_bf16_bits(a64)
    if dtype == "f16":
        # float64 -> float16 directly, round-to-nearest-even (beyond the range: inf)
        with np.errstate(over="ignore"):
            h = np.asarray(a64, dtype=np.float64).astype(np.float16)
        return np.ascontiguousarray(h.view(np.uint16))
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f64(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(a, dtype=np.float64)
    if dtype == "bf16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "f16":
        return np.ascontiguousarray(a, dtype=np.uint16).view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# draws

def _he_uniform(rng: np.random.Generator, shape) -> np.ndarray:
    fan_in = int(np.prod(shape[:-1]))
    bound = np.sqrt(6.0 / fan_in)
    return rng.uniform(-bound, bound, size=shape)


def make_params(dims: Dims, dtype: str, seed: int, ln_affine: str = "unit",
                rng: np.random.Generator | None = None) -> dict:
    """Parameters in storage form, drawn in the fixed order stated in the module doc."""
    if rng is None:
        rng = np.random.Generator(np.random.PCG64(seed))
    T, D, H = dims.T, dims.D, dims.H
    p = {}
    p["w1"] = to_storage(_he_uniform(rng, (T, D, 2 * H)), dtype)
    p["b1"] = to_storage(_he_uniform(rng, (T, 2 * H)), dtype)
    p["wout"] = to_storage(_he_uniform(rng, (T, H, D)), dtype)
    p["bout"] = to_storage(_he_uniform(rng, (T, D)), dtype)
    widths = {"ln0": D, "ln1": D, "ln2": D, "lnx": H, "lng": H}
    for ln in ("ln0", "ln1", "ln2", "lnx", "lng"):
        n = widths[ln]
        if ln_affine == "unit":
            g, b = np.ones(n), np.zeros(n)
        elif ln_affine == "random":
            g = rng.uniform(0.5, 1.5, size=n)
            b = rng.uniform(-0.1, 0.1, size=n)
        else:
            raise ValueError(f"unknown ln_affine {ln_affine!r}")
        p[ln + "_g"] = to_storage(g, dtype)
        p[ln + "_b"] = to_storage(b, dtype)
    return p


def make_case(w: Workload | str, batch: int | None = None) -> dict:
    """Full seeded case: {'params', 'x', 'dy', 'dims', 'dtype'} in storage form.

    `batch` optionally draws only the first `batch` samples of x and dy (the
    parameters are identical to the full workload's; x and dy rows are a prefix
    of the full draw because samples are drawn in order).
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    dims = w.dims
    rng = np.random.Generator(np.random.PCG64(w.seed))
    params = make_params(dims, w.dtype, w.seed, w.ln_affine, rng=rng)
    B = dims.B if batch is None else batch
    shape = (B, dims.T, dims.D)
    x = to_storage(rng.standard_normal(size=shape), w.dtype)
    rng_dy = np.random.Generator(np.random.PCG64(w.seed + 1000))
    dy = to_storage(rng_dy.standard_normal(size=shape), w.dtype)
    return {"params": params, "x": x, "dy": dy,
            "dims": Dims(B, dims.T, dims.D, dims.k), "dtype": w.dtype, "name": w.name}


def make_custom(B, T, D, k, dtype, seed, ln_affine="unit") -> dict:
    """A case of arbitrary shape (edge shapes of the envelope, tiny oracle shapes)."""
    w = Workload(f"B{B}_T{T}_D{D}_k{k}_{dtype}_s{seed}", Dims(B, T, D, k), dtype, seed, ln_affine)
    return make_case(w)


def as_f64(case: dict) -> tuple[np.ndarray, dict, np.ndarray]:
    """(x, params, dy) of a case decoded to float64 (what the oracle consumes)."""
    dt = case["dtype"]
    p = {k: storage_to_f64(v, dt) for k, v in case["params"].items()}
    return storage_to_f64(case["x"], dt), p, storage_to_f64(case["dy"], dt)


def digest(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()[:16]
