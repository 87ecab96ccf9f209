"""Float64 CPU oracle of the RankMixerBlock (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg use it;
the product path never imports it.
"""
from .rankmixer import (EPS_INNER, EPS_OUTER, GRAD_NAMES, backward, dense_ffn,
                        dense_ffn_backward, forward, forward_backward, layer_norm,
                        layer_norm_backward, mixer_epilogue, mixer_epilogue_backward,
                        mixer_prologue, mixer_prologue_backward, sigmoid, silu, token_mix)

__all__ = ["EPS_INNER", "EPS_OUTER", "GRAD_NAMES", "backward", "dense_ffn",
           "dense_ffn_backward", "forward", "forward_backward", "layer_norm",
           "layer_norm_backward", "mixer_epilogue", "mixer_epilogue_backward",
           "mixer_prologue", "mixer_prologue_backward", "sigmoid", "silu", "token_mix"]
