"""MI355X-native Sparsely-Gated Mixture-of-Experts layer: forward and backward.

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
                   MoeGrads, MoeWeights, load_library, make_config, make_diag, make_grads,
                   make_weights, moe_aux_loss, moe_backward, moe_backward_workspace_size,
                   moe_combine, moe_dispatch, moe_expert_ffn, moe_expert_split_rows,
                   moe_gate_k_splits, moe_expert_cu_split,
                   moe_backward_saved, moe_fp8_weight_bytes, moe_forward,
                   moe_forward_train, moe_pack_fp8_weights,
                   moe_gate, moe_gate_hier, moe_gate_static, moe_last_error, moe_profile_collect,
                   moe_probe_hbm_read, moe_probe_mfma, moe_profile_enable,
                   moe_profile_entry,
                   moe_router_bias_update,
                   moe_shared_ffn, moe_status_string, moe_workspace_size)

load_library()

MOE_F32, MOE_BF16, MOE_FP8 = 0, 1, 2


def pack_fp8(w, stream=None):
    """Pack a [n, N, K] (or [N, K]) bf16 / fp32 device tensor of expert
    weights into the library's FP8 E4M3 layout (uint8 tensor)."""
    import torch
    w3 = w if w.dim() == 3 else w.unsqueeze(0)
    n, N, K = w3.shape
    size = moe_fp8_weight_bytes(n, N, K)
    if size == 0:
        raise MoEError(MOE_ERR_UNSUPPORTED, f"cannot pack a [{n}, {N}, {K}] matrix as FP8")
    out = torch.empty(size, dtype=torch.uint8, device=w.device)
    src = w3.contiguous()
    moe_pack_fp8_weights(n, N, K, MOE_BF16 if src.dtype == torch.bfloat16 else MOE_F32, src, out,
                         stream)
    return out


class MoELayer:
    """Holds one configuration, its weights (torch device tensors, see
    workloads.make_inputs) and a workspace; ``forward`` runs the whole layer
    through moe_forward on the current stream."""

    def __init__(self, cfg, weights: dict, device="cuda"):
        import torch
        self.cfg = cfg
        self.c = make_config(cfg)
        self.device = device
        if int(cfg.expert_dtype) == MOE_FP8:
            # FP8 experts: pack bf16 / fp32 weights once (already packed
            # uint8 buffers pass through).
            weights = dict(weights)
            for name in ("w1", "w3", "w2"):
                t = weights.get(name)
                if t is not None and t.dtype != torch.uint8:
                    weights[name] = pack_fp8(t)
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

    # gradient name -> weight it belongs to
    _GRAD_OF = dict(dw_gate="w_gate", db_gate="b_gate", dw_noise="w_noise", dw1="w1",
                    db1="b1", dw3="w3", dw2="w2", db2="b2", dws1="ws1", dws3="ws3", dws2="ws2",
                    dw_gate2="w_gate2", dw_noise2="w_noise2")

    def _bwd_ws(self):
        import torch
        if getattr(self, "ws_bwd", None) is None:
            size = moe_backward_workspace_size(self.c)
            if size == 0:
                raise MoEError(MOE_ERR_UNSUPPORTED, "the backward pass does not cover this "
                               "configuration (bf16 or fp32 experts, sizes multiples of 64)")
            self.ws_bwd = torch.empty(size, dtype=torch.uint8, device=self.device)
        return self.ws_bwd

    def forward_train(self, x, noise=None, noise2=None, y=None, losses=None):
        """The forward through moe_forward_train: y and losses as ``forward``,
        with the intermediates kept for ``backward(..., saved=True)``."""
        import torch
        if y is None:
            y = torch.empty((self.c.T, self.c.d_model), dtype=torch.float32, device=self.device)
        if losses is None:
            losses = torch.empty(N_LOSSES, dtype=torch.float32, device=self.device)
        moe_forward_train(self.c, self.w, x, noise, noise2, y, losses, self._bwd_ws())
        return y, losses

    def backward(self, x, dy, dlosses=None, noise=None, noise2=None, saved=False):
        """Gradients of sum <dy, y> + sum dlosses * losses (dlosses: 5 values,
        default zeros); returns a dict of fp32 tensors (dx and one per present
        weight; no db_gate for the sigmoid gate).  saved=False: moe_backward
        (recomputes the forward); saved=True: moe_backward_saved, after a
        ``forward_train`` on the same inputs."""
        import torch
        ws = self._bwd_ws()
        if dlosses is None:
            dlosses = torch.zeros(N_LOSSES, dtype=torch.float32, device=self.device)
        grads = {"dx": torch.empty((self.c.T, self.c.d_model), dtype=torch.float32,
                                   device=self.device)}
        for g, wname in self._GRAD_OF.items():
            t = self.weights.get(wname)
            if t is None or (g == "db_gate" and int(self.cfg.gate) == 2):
                continue
            grads[g] = torch.empty(t.shape, dtype=torch.float32, device=self.device)
        call = moe_backward_saved if saved else moe_backward
        call(self.c, self.w, x, noise, noise2, dy, dlosses, make_grads(**grads), ws)
        return grads

__all__ = ["workloads", "EXPORTS", "MoELayer", "pack_fp8", "moe_fp8_weight_bytes",
           "moe_pack_fp8_weights", "MOE_F32", "MOE_BF16", "MOE_FP8", "MoEError", "MoeConfig",
           "MoeWeights", "MoeDiag", "MoeGrads", "make_config", "make_weights", "make_diag",
           "make_grads", "moe_workspace_size", "moe_gate", "moe_gate_hier", "moe_dispatch",
           "moe_expert_ffn", "moe_shared_ffn", "moe_combine", "moe_aux_loss",
           "moe_router_bias_update", "moe_forward", "moe_backward_workspace_size",
           "moe_backward", "moe_forward_train", "moe_backward_saved", "N_LOSSES", "moe_status_string", "moe_last_error",
           "moe_probe_mfma", "moe_probe_hbm_read", "moe_profile_enable", "moe_profile_collect", "moe_profile_entry",
           "MOE_OK",
           "MOE_ERR_INVALID_ARG", "MOE_ERR_UNSUPPORTED", "MOE_ERR_WORKSPACE", "MOE_ERR_HIP"]
