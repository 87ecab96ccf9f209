"""Helpers of the GPU tests: move a seeded case to the device, run the HIP
path through the C ABI, bring results back as float64, compare with the
oracle under the stated metric."""
from __future__ import annotations

import sys

import numpy as np

from rankmixer_inputs import PARAM_NAMES, storage_to_f64

# max |gpu - oracle| / max |oracle| per tensor (fp32 storage / 16-bit storage)
TOL = {"f32": 1e-4, "bf16": 3e-2, "f16": 3e-2}
TORCH16 = {"bf16": "bfloat16", "f16": "float16"}

GRAD_KEYS = ("dx",) + tuple("d" + n for n in PARAM_NAMES)


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_torch(a: np.ndarray, dtype: str, device="cuda"):
    import torch
    if dtype in TORCH16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(getattr(torch, TORCH16[dtype]))
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def from_torch(t, dtype: str) -> np.ndarray:
    import torch
    if dtype in TORCH16:
        return storage_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16), dtype)
    return t.cpu().numpy().astype(np.float64)


class DeviceCase:
    """A case's tensors on the device plus output buffers and the workspace."""

    def __init__(self, case: dict, device="cuda", kernels="auto"):
        import torch
        import transformer_block_norm0_amd as rb
        self.case = case
        self.dtype = case["dtype"]
        d = case["dims"]
        self.cd = rb.dims(d.B, d.T, d.D, d.k, self.dtype, kernels)
        self.params = {n: to_torch(v, self.dtype, device) for n, v in case["params"].items()}
        self.x = to_torch(case["x"], self.dtype, device)
        self.dy = to_torch(case["dy"], self.dtype, device)
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.grads = {n: torch.empty_like(v) for n, v in self.params.items()}
        self.ws = rb.alloc_workspace(self.cd, device)

    def misalign(self):
        """Move x, dy, y and dx to buffers that start 2 bytes past a 16-byte boundary
        (element-aligned only, as the interface allows)."""
        import torch
        for name in ("x", "dy", "y", "dx"):
            t = getattr(self, name)
            buf = torch.empty(t.numel() + 8, dtype=t.dtype, device=t.device)
            v = buf[1:1 + t.numel()].view(t.shape)
            v.copy_(t)
            assert v.data_ptr() % 16 != 0
            setattr(self, name, v)

    def _dims(self, kernels):
        import transformer_block_norm0_amd as rb
        if kernels is None:
            return self.cd
        c = self.cd
        return rb.dims(c.B, c.T, c.D, c.k, self.dtype, kernels)

    def fwd(self, stream=None, kernels=None):
        """rm_block_fwd; kernels ("auto" / "main") overrides the case's kernel set for this call."""
        import transformer_block_norm0_amd as rb
        rb.block_fwd(self._dims(kernels), self.params, self.x, self.y, self.ws, stream=stream)

    def bwd(self, stream=None, kernels=None):
        import transformer_block_norm0_amd as rb
        rb.block_bwd(self._dims(kernels), self.params, self.x, self.dy, self.ws, self.dx, self.grads, stream=stream)

    def run(self):
        import torch
        self.fwd()
        self.bwd()
        torch.cuda.synchronize()

    def results(self) -> dict:
        out = {"y": from_torch(self.y, self.dtype), "dx": from_torch(self.dx, self.dtype)}
        for n, t in self.grads.items():
            out["d" + n] = from_torch(t, self.dtype)
        return out

    def raw_bits(self) -> dict:
        """Exact bit patterns of every output (for determinism checks)."""
        import torch
        view = torch.int16 if self.dtype in TORCH16 else torch.int32
        out = {"y": self.y.view(view).cpu().numpy(), "dx": self.dx.view(view).cpu().numpy()}
        for n, t in self.grads.items():
            out["d" + n] = t.view(view).cpu().numpy()
        return out

    def ws_region(self, region: int, shape, f32: bool) -> np.ndarray:
        import torch
        import transformer_block_norm0_amd as rb
        off, nbytes = rb.ws_region(self.cd, region)
        raw = self.ws[off:off + nbytes]
        if f32:
            return raw.view(torch.float32).cpu().numpy().astype(np.float64).reshape(shape)
        if self.dtype in TORCH16:
            return storage_to_f64(raw.view(torch.int16).cpu().numpy().view(np.uint16), self.dtype).reshape(shape)
        return raw.view(torch.float32).cpu().numpy().astype(np.float64).reshape(shape)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    assert got.shape == ref.shape, (got.shape, ref.shape)
    den = max(float(np.max(np.abs(ref))), 1e-30)
    return float(np.max(np.abs(got - ref))) / den


# (label, {tensor: error}) of every full-size comparison, printed in pytest's terminal summary
FULL_SIZE_REPORT: list = []


def compare(got: dict, ref: dict, keys, tol: float, label: str) -> dict:
    errs = {}
    for k in keys:
        g, r = got[k], ref[k]
        assert np.all(np.isfinite(g)), f"{label}: {k} has non-finite values"
        errs[k] = rel_err(g, r)
    say(f"{label}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()))
    bad = {k: v for k, v in errs.items() if not v <= tol}
    assert not bad, f"{label}: over tolerance {tol}: {bad}"
    return errs
