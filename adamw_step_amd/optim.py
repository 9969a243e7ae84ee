"""torch.optim front end of the packed-AdamW step.

Follows the reference's execution contract (project page, Execution contract
table): contiguous parameters and dense gradients on one device (FP32, or
bfloat16/float16 with the update still in FP32),
one parameter group, one global step, ordinary PyTorch forward and backward
around it.  Every update is one pa_step_list launch over all parameters
(see include/pa.h); this module only holds the state tensors and marshals
arguments.

Modes: "e4" (one uint32 word per parameter: E4M11 first moment, E4M12 RMS),
"fp16" (the same word with binary16 lanes) and "fp32" (two FP32 moments).
The blockwise 8-bit mode writes BF16 parameters to a separate buffer and
needs 2048-multiple tensors, so it is driven through pa_step directly.
"""
from __future__ import annotations

import torch

from . import PA_FP32, PA_PACKED_E4, PA_PACKED_FP16, StepList, pa_state_bytes

_MODES = {"e4": PA_PACKED_E4, "fp16": PA_PACKED_FP16, "fp32": PA_FP32}


class PackedAdamW(torch.optim.Optimizer):
    """AdamW with decoupled weight decay whose moments persist in packed form.

    Arguments keep their usual AdamW meaning (TurboAdam package page, API
    section: lr, betas, eps, weight_decay).  ``count_nonfinite`` keeps a
    device counter of elements whose new parameter or moment was not finite
    (the optimizer non-finite count of the reference's smoke check); read it
    with ``nonfinite_count()``.
    """

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                 mode="e4", count_nonfinite=True):
        if mode not in _MODES:
            raise ValueError(f"mode must be one of {sorted(_MODES)}")
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults)
        if len(self.param_groups) != 1:
            raise ValueError("PackedAdamW takes one parameter group (one lr, one step for all)")
        self.mode = mode
        self._mode = _MODES[mode]
        self.step_count = 0
        self._prepared = None
        self._prepared_key = None
        plist = self.param_groups[0]["params"]
        if not plist:
            raise ValueError("no parameters")
        dev, dt = plist[0].device, plist[0].dtype
        if dt not in (torch.float32, torch.bfloat16, torch.float16):
            raise TypeError("parameters must be float32, bfloat16 or float16")
        for p in plist:
            if p.dtype != dt or not p.is_cuda or not p.is_contiguous() or p.device != dev:
                raise TypeError("parameters must be contiguous tensors of one dtype on one GPU")
            self._init_state(p)
        self._nonfinite = torch.zeros(1, dtype=torch.int64, device=dev) if count_nonfinite else None

    def _init_state(self, p):
        st = self.state[p]
        if self._mode == PA_FP32:
            st["exp_avg"] = torch.zeros(p.numel(), dtype=torch.float32, device=p.device)
            st["exp_avg_sq"] = torch.zeros(p.numel(), dtype=torch.float32, device=p.device)
        else:
            st["words"] = torch.zeros(p.numel(), dtype=torch.int32, device=p.device)

    def _state_of(self, p):
        st = self.state[p]
        return (st["exp_avg"], st["exp_avg_sq"]) if self._mode == PA_FP32 else st["words"]

    def state_bytes(self):
        """Persistent optimizer-state bytes (the ledger): 4 per parameter packed, 8 for FP32."""
        return sum(pa_state_bytes(self._mode, p.numel()) for p in self.param_groups[0]["params"])

    def nonfinite_count(self):
        return 0 if self._nonfinite is None else int(self._nonfinite.item())

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        group = self.param_groups[0]
        params = group["params"]
        grads = []
        for p in params:
            g = p.grad
            if g is None:
                raise RuntimeError("every parameter needs a dense gradient on every update")
            if g.is_sparse:
                raise RuntimeError("sparse gradients are not supported")
            if not g.is_contiguous():
                g = g.contiguous()
            grads.append(g)
        states = [self._state_of(p) for p in params]
        key = tuple(g.data_ptr() for g in grads) + tuple(p.data_ptr() for p in params)
        if self._prepared is None or key != self._prepared_key:
            self._prepared = StepList(self._mode, params, grads, states)
            self._prepared_key = key
        self.step_count += 1
        beta1, beta2 = group["betas"]
        hyper = dict(lr=group["lr"], beta1=beta1, beta2=beta2, eps=group["eps"],
                     weight_decay=group["weight_decay"])
        if self._nonfinite is not None:
            hyper["nonfinite"] = self._nonfinite
        self._prepared.step(hyper, self.step_count)
        return loss

    def state_dict(self):
        sd = super().state_dict()
        sd["packed"] = {"mode": self.mode, "step": self.step_count}
        return sd

    def load_state_dict(self, state_dict):
        """Restore a checkpoint.  The packed words are put back bit for bit:
        torch's loader would convert non-float state to the parameters'
        dtype, which would turn the words into float values."""
        meta = state_dict.get("packed", {})
        if meta.get("mode", self.mode) != self.mode:
            raise ValueError(f"checkpoint holds mode {meta.get('mode')}, optimizer uses {self.mode}")
        words, rest = {}, {}
        for idx, st in state_dict["state"].items():
            st = dict(st)
            if "words" in st:
                words[idx] = st.pop("words")
            rest[idx] = st
        base = {k: v for k, v in state_dict.items() if k not in ("packed", "state")}
        base["state"] = rest
        super().load_state_dict(base)
        params = self.param_groups[0]["params"]
        for idx, w in words.items():
            p = params[idx]
            if w.numel() != p.numel():
                raise ValueError("checkpoint words do not match the parameter sizes")
            self.state[p]["words"] = w.to(device=p.device, dtype=torch.int32).contiguous().clone()
        for p in params:
            st = self.state[p]
            for k, v in st.items():
                if torch.is_tensor(v) and not v.is_contiguous():
                    st[k] = v.contiguous()
        self.step_count = int(meta.get("step", 0))
        self._prepared = None
