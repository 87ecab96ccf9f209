"""MI355X (gfx950) RankMixerBlock forward + backward behind a C ABI (librmblock.so).

The package holds the HIP sources (csrc/), the hipcc build step (build.py)
and a ctypes binding (rmblock.py).  Importing it does not load the library;
the first call does, and raises if it has not been built.
"""
from .rmblock import (PARAM_NAMES, RM_BF16, RM_F32, RmError, alloc_workspace, block_bwd, block_bwd_static, block_fwd, dims,
                      kernel_names, library, param_shapes, prof_collect, prof_enable, token_mix,
                      workspace_bytes, ws_region)

__all__ = ["PARAM_NAMES", "RM_BF16", "RM_F32", "RmError", "alloc_workspace", "block_bwd", "block_bwd_static", "block_fwd", "dims",
           "kernel_names", "library", "param_shapes", "prof_collect", "prof_enable", "token_mix",
           "workspace_bytes", "ws_region"]
