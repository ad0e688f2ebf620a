"""MI355X-native Sparsely-Gated Mixture-of-Experts layer forward.

The computation lives in libmoe.so (hand-written HIP for gfx950 behind the C
ABI of include/moe.h).  This package holds the ctypes binding, a small helper
that allocates outputs and workspace with torch, and the seeded synthetic
workloads.  Importing it loads the library and fails loudly when it has not
been built.
"""
from __future__ import annotations

from . import workloads
from ._lib import (EXPORTS, MOE_ERR_HIP, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED,
                   MOE_ERR_WORKSPACE, MOE_OK, N_LOSSES, MoeConfig, MoeDiag, MoEError,
                   MoeWeights, load_library, make_config, make_diag, make_weights,
                   moe_aux_loss, moe_combine, moe_dispatch, moe_expert_ffn, moe_forward,
                   moe_gate, moe_gate_hier, moe_last_error, moe_profile_collect,
                   moe_profile_enable, moe_profile_entry, moe_router_bias_update,
                   moe_shared_ffn, moe_status_string, moe_workspace_size)

load_library()


class MoELayer:
    """Holds one configuration, its weights (torch device tensors, see
    workloads.make_inputs) and a workspace; ``forward`` runs the whole layer
    through moe_forward on the current stream."""

    def __init__(self, cfg, weights: dict, device="cuda"):
        import torch
        self.cfg = cfg
        self.c = make_config(cfg)
        self.device = device
        self.weights = weights
        self.w = make_weights(weights["w_gate"], weights.get("b_gate"), weights.get("w_noise"),
                              weights.get("w_gate2"), weights.get("w_noise2"), weights["w1"],
                              weights.get("b1"), weights.get("w3"), weights["w2"],
                              weights.get("b2"), weights.get("ws1"), weights.get("ws3"),
                              weights.get("ws2"))
        size = moe_workspace_size(self.c)
        if size == 0:
            raise MoEError(MOE_ERR_INVALID_ARG, moe_last_error())
        self.ws = torch.empty(size, dtype=torch.uint8, device=device)

    def forward(self, x, noise=None, noise2=None, y=None, losses=None, diag: dict | None = None):
        import torch
        if y is None:
            y = torch.empty((self.c.T, self.c.d_model), dtype=torch.float32, device=self.device)
        if losses is None:
            losses = torch.empty(N_LOSSES, dtype=torch.float32, device=self.device)
        dg = make_diag(**diag) if diag else None
        moe_forward(self.c, self.w, x, noise, noise2, y, losses, dg, self.ws)
        return y, losses


__all__ = ["workloads", "EXPORTS", "MoELayer", "MoEError", "MoeConfig", "MoeWeights", "MoeDiag",
           "make_config", "make_weights", "make_diag", "moe_workspace_size", "moe_gate",
           "moe_gate_hier", "moe_dispatch", "moe_expert_ffn", "moe_shared_ffn", "moe_combine",
           "moe_aux_loss", "moe_router_bias_update", "moe_forward", "N_LOSSES", "moe_status_string", "moe_last_error", "moe_profile_enable",
           "moe_profile_collect", "moe_profile_entry", "MOE_OK", "MOE_ERR_INVALID_ARG",
           "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]
