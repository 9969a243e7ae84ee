"""torch.optim front end of the packed-AdamW step.

Follows the reference's execution contract (project page, Execution contract
table): contiguous parameters and dense gradients on one device (FP32, or
bfloat16/float16 with the update still in FP32), one global step, ordinary
PyTorch forward and backward around it.  Parameter groups (the TurboAdam
page's API takes "parameters or parameter groups") each carry their own
lr, betas, eps and weight decay; every update is one pa_step_list launch
per group (see include/pa.h), all groups sharing the step number, the
non-finite counter and one gradient pre-pass over every gradient.  This
module only holds the state tensors and marshals arguments.

Modes: "e4" (one uint32 word per parameter: E4M11 first moment, E4M12 RMS),
"fp16" (the same word with binary16 lanes) and "fp32" (two FP32 moments).
TurboAdam (UState + 1Q compressed state) has its own class below.
The blockwise 8-bit mode writes BF16 parameters to a separate buffer and
needs 2048-multiple tensors, so it is driven through pa_step directly.
"""
from __future__ import annotations

import torch

from . import PA_FP32, PA_PACKED_E4, PA_PACKED_FP16, GradStats, StepList, pa_state_bytes

_MODES = {"e4": PA_PACKED_E4, "fp16": PA_PACKED_FP16, "fp32": PA_FP32}


def _check_group_params(opt, group):
    """Every parameter of the optimizer: contiguous, on one GPU, one dtype
    (float32, bfloat16 or float16)."""
    for p in group["params"]:
        if opt._dtype is None:
            if p.dtype not in (torch.float32, torch.bfloat16, torch.float16):
                raise TypeError("parameters must be float32, bfloat16 or float16")
            opt._dtype, opt._device = p.dtype, p.device
        if p.dtype != opt._dtype or not p.is_cuda or not p.is_contiguous() or p.device != opt._device:
            raise TypeError("parameters must be contiguous tensors of one dtype on one GPU")


def _add_group(opt, param_group, init):
    """torch's add_param_group, then the checks and the state of the new
    parameters; a group that fails the checks is taken back out."""
    torch.optim.Optimizer.add_param_group(opt, param_group)
    group = opt.param_groups[-1]
    try:
        opt._check_group(group)
        _check_group_params(opt, group)
    except Exception:
        opt.param_groups.pop()
        raise
    for p in group["params"]:
        init(p)
    opt._prepared = {}


def _cached_list(cache, gi, params, grads, build):
    """The cached step list of group gi: built again when the parameters
    change, pointed at the new gradients when only those moved (torch
    allocates fresh ones after zero_grad(set_to_none=True))."""
    pkey = tuple(p.data_ptr() for p in params)
    gkey = tuple(g.data_ptr() for g in grads)
    cached = cache.get(gi)
    if cached is None or cached[0] != pkey:
        cached = [pkey, gkey, build()]
        cache[gi] = cached
    elif cached[1] != gkey:
        cached[2].set_grads(grads)
        cached[1] = gkey
    return cached[2]


def _grads_of(params):
    grads = []
    for p in params:
        g = p.grad
        if g is None:
            raise RuntimeError("every parameter needs a dense gradient on every update")
        if g.is_sparse:
            raise RuntimeError("sparse gradients are not supported")
        grads.append(g if g.is_contiguous() else g.contiguous())
    return grads


class PackedAdamW(torch.optim.Optimizer):
    """AdamW with decoupled weight decay whose moments persist in packed form.

    Arguments keep their usual AdamW meaning (TurboAdam package page, API
    section: lr, betas, eps, weight_decay), per parameter group.  ``count_nonfinite`` keeps a
    device counter of elements whose new parameter or moment was not finite
    (the optimizer non-finite count of the reference's smoke check); read it
    with ``nonfinite_count()``.

    ``max_grad_norm`` clips the global gradient norm and ``skip_nonfinite``
    skips an update whose gradients hold NaN or Inf.  Either one adds the
    gradient pre-pass (pa_grad_stats_list) before the update; its clip
    coefficient and non-finite count reach the update on the device, with
    no host synchronisation.  A skipped update does not count as a step:
    the pre-pass count is copied to pinned host memory and checked at the
    next ``step()`` (by then long finished), which then reuses the step
    number.  ``last_grad_norm()`` reads the norm of the latest pre-pass.
    """

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0,
                 mode="e4", count_nonfinite=True, max_grad_norm=None, skip_nonfinite=False):
        if mode not in _MODES:
            raise ValueError(f"mode must be one of {sorted(_MODES)}")
        self.mode = mode
        self._mode = _MODES[mode]
        self._dtype = self._device = None
        self._prepared = {}                 # group index -> (pointer key, StepList)
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults)
        if not any(g["params"] for g in self.param_groups):
            raise ValueError("no parameters")
        self.step_count = 0
        dev = self._device
        self._nonfinite = torch.zeros(1, dtype=torch.int64, device=dev) if count_nonfinite else None
        if max_grad_norm is not None and not (float(max_grad_norm) > 0.0):
            raise ValueError("max_grad_norm must be positive")
        self.max_grad_norm = None if max_grad_norm is None else float(max_grad_norm)
        self.skip_nonfinite = bool(skip_nonfinite)
        self.skipped_steps = 0
        self._stats = None
        self._stats_key = None
        if self.max_grad_norm is not None or self.skip_nonfinite:
            self._sumsq = torch.zeros(1, dtype=torch.float64, device=dev)
            self._grad_bad = torch.zeros(1, dtype=torch.int64, device=dev)
            self._clip = torch.ones(1, dtype=torch.float32, device=dev)
            self._bad_host = torch.zeros(1, dtype=torch.int64, pin_memory=True)
            self._bad_event = torch.cuda.Event()
            self._pending = False

    def add_param_group(self, param_group):
        _add_group(self, param_group, self._init_state)

    def _check_group(self, group):
        pass

    def _params(self):
        return [p for g in self.param_groups for p in g["params"]]

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
        return sum(pa_state_bytes(self._mode, p.numel()) for p in self._params())

    def nonfinite_count(self):
        return 0 if self._nonfinite is None else int(self._nonfinite.item())

    def last_grad_norm(self):
        """Global L2 norm of the gradients seen by the latest pre-pass (None without one)."""
        if self._stats is None:
            return None
        return float(self._sumsq.item()) ** 0.5

    def _reconcile(self):
        # A pre-pass whose count was nonzero skipped its update on the device.
        if self._stats is not None and self.skip_nonfinite and self._pending:
            self._bad_event.synchronize()
            if int(self._bad_host.item()) != 0:
                self.step_count -= 1
                self.skipped_steps += 1
            self._pending = False

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        work, all_grads = [], []
        for gi, group in enumerate(self.param_groups):
            if not group["params"]:
                continue
            grads = _grads_of(group["params"])
            work.append((gi, group, grads))
            all_grads += grads
        self._reconcile()
        self.step_count += 1
        common = {}
        if self._nonfinite is not None:
            common["nonfinite"] = self._nonfinite
        if self.max_grad_norm is not None or self.skip_nonfinite:
            gkey = tuple(g.data_ptr() for g in all_grads)
            if self._stats is None or len(gkey) != len(self._stats_key):
                self._stats = GradStats(all_grads)
            elif gkey != self._stats_key:       # fresh gradient tensors: same list, new pointers
                self._stats.set_grads(all_grads)
            self._stats_key = gkey
            self._stats.run(self._sumsq, self._grad_bad,
                            self._clip if self.max_grad_norm is not None else None,
                            max_norm=self.max_grad_norm or 0.0)
            if self.max_grad_norm is not None:
                common["grad_scale"] = self._clip
            if self.skip_nonfinite:
                common["skip_if_nonzero"] = self._grad_bad
                self._bad_host.copy_(self._grad_bad, non_blocking=True)
                self._bad_event.record()
                self._pending = True
        for gi, group, grads in work:
            params = group["params"]
            sl = _cached_list(self._prepared, gi, params, grads,
                              lambda: StepList(self._mode, params, grads, [self._state_of(p) for p in params]))
            beta1, beta2 = group["betas"]
            hyper = dict(lr=group["lr"], beta1=beta1, beta2=beta2, eps=group["eps"],
                         weight_decay=group["weight_decay"], **common)
            sl.step(hyper, self.step_count)
        return loss

    def state_dict(self):
        self._reconcile()
        sd = super().state_dict()
        sd["packed"] = {"mode": self.mode, "step": self.step_count}
        return sd

    _RAW_STATE = {"words": torch.int32, "exp_avg": torch.float32, "exp_avg_sq": torch.float32}

    def load_state_dict(self, state_dict):
        """Restore a checkpoint.  The state tensors are put back bit for bit
        in their own dtypes: torch's loader would convert floating-point
        state to the parameters' dtype (bfloat16 moments for bfloat16
        parameters) and non-float state to float values."""
        meta = state_dict.get("packed", {})
        if meta.get("mode", self.mode) != self.mode:
            raise ValueError(f"checkpoint holds mode {meta.get('mode')}, optimizer uses {self.mode}")
        raw, rest = {}, {}
        for idx, st in state_dict["state"].items():
            st = dict(st)
            raw[idx] = {k: st.pop(k) for k in self._RAW_STATE if k in st}
            rest[idx] = st
        base = {k: v for k, v in state_dict.items() if k not in ("packed", "state")}
        base["state"] = rest
        super().load_state_dict(base)
        params = self._params()
        for idx, tensors in raw.items():
            p = params[idx]
            for k, t in tensors.items():
                if t.numel() != p.numel() or t.dtype != self._RAW_STATE[k]:
                    raise ValueError(f"checkpoint {k} does not match the parameter size or its dtype")
                self.state[p][k] = t.to(device=p.device).contiguous().clone()
        for p in params:
            st = self.state[p]
            for k, v in st.items():
                if torch.is_tensor(v) and not v.is_contiguous():
                    st[k] = v.contiguous()
        self.step_count = int(meta.get("step", 0))
        self._prepared = {}
        if self._stats is not None:
            self._pending = False


class TurboAdam(torch.optim.Optimizer):
    """AdamW whose moments persist as TurboAdam state: UState for the first
    moment, 1Q for the second (TurboAdam package page, API and "How it
    works"), every update one pa_turbo_step_list launch plus the scale
    rotation, with the page's defaults.

    Arguments follow the page's API: lr, betas, eps, weight_decay,
    block_size (a power of two from 32 to 1024), v_bits (2, 3, 4, 6 or 8),
    compress_m, compress_v, min_m_compress_elements and
    min_v_compress_elements (a tensor below the threshold keeps that
    moment in FP32), m_block_size (a power of two dividing block_size),
    m_step_factor and rounding_seed.  The default layout (128, 4 bits, 64)
    runs the tuned kernel at every index width, every other layout the
    general kernel.  The page's validation of beta1^2 < beta2 with UState on
    is kept, per parameter group.  Parameter groups carry their own lr,
    betas, eps and weight decay (one launch each); the layout, thresholds,
    scale factor and seed are the optimizer's.  Contiguous tensors of one
    dtype on one GPU: float32, bfloat16 or float16 (the page's tests run all
    three; the update runs in FP32 and only the new parameter is rounded
    back), with gradients of the same dtype.  Tensors are numbered across
    the groups in order; the number keys their random draws.
    ``count_nonfinite``, ``nonfinite_count()`` and ``state_bytes()`` as for
    PackedAdamW.
    """

    def __init__(self, params, lr=1e-3, betas=(0.9, 0.999), eps=1e-8, weight_decay=0.0, block_size=128, v_bits=4,
                 compress_m=True, compress_v=True, min_m_compress_elements=4096, min_v_compress_elements=4096,
                 m_block_size=64, m_step_factor=1.1, rounding_seed=0x12345678, count_nonfinite=True):
        from . import TurboList, TurboState, turbo_layout_ok
        if not turbo_layout_ok(v_bits, block_size, m_block_size):
            raise ValueError("v_bits must be 2, 3, 4, 6 or 8, block_size a power of two from 32 to 1024 and "
                             "m_block_size a power of two dividing block_size")
        self.v_bits, self.m_step_factor, self.seed = v_bits, float(m_step_factor), int(rounding_seed)
        self.block_size, self.m_block_size = int(block_size), int(m_block_size)
        self._compress = (bool(compress_m), bool(compress_v), int(min_m_compress_elements),
                          int(min_v_compress_elements))
        self._TurboList, self._TurboState = TurboList, TurboState
        self._dtype = self._device = None
        self._states = []
        self._prepared = {}                 # group index -> (pointer key, TurboList)
        defaults = dict(lr=lr, betas=betas, eps=eps, weight_decay=weight_decay)
        super().__init__(params, defaults)
        if not self._states:
            raise ValueError("no parameters")
        self.step_count = 0
        self._nonfinite = torch.zeros(1, dtype=torch.int64, device=self._device) if count_nonfinite else None

    def add_param_group(self, param_group):
        _add_group(self, param_group, self._init_state)

    def _check_group(self, group):
        beta1, beta2 = group["betas"]
        if self._compress[0] and not beta1 ** 2 < beta2:
            raise ValueError("UState needs beta1**2 < beta2")

    def _init_state(self, p):
        cm, cv, min_m, min_v = self._compress
        n = p.numel()
        st = self._TurboState(n, p.device, compress_m=cm and n >= min_m, compress_v=cv and n >= min_v,
                              v_bits=self.v_bits, tensor_id=len(self._states), block_size=self.block_size,
                              m_block_size=self.m_block_size)
        self._states.append(st)
        self.state[p]["turbo"] = st

    def state_bytes(self):
        """Persistent optimizer-state bytes: codes, means, indices, endpoints,
        per-tensor scales, and the FP32 moments of uncompressed tensors."""
        return sum(st.nbytes() for st in self._states)

    def nonfinite_count(self):
        return 0 if self._nonfinite is None else int(self._nonfinite.item())

    @torch.no_grad()
    def step(self, closure=None):
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        work = [(gi, group, _grads_of(group["params"])) for gi, group in enumerate(self.param_groups)
                if group["params"]]
        self.step_count += 1
        for gi, group, grads in work:
            params = group["params"]
            tl = _cached_list(self._prepared, gi, params, grads, lambda: self._TurboList(
                params, grads, [self.state[p]["turbo"] for p in params], v_bits=self.v_bits,
                m_step_factor=self.m_step_factor, seed=self.seed, block_size=self.block_size,
                m_block_size=self.m_block_size))
            beta1, beta2 = group["betas"]
            hyper = dict(lr=group["lr"], beta1=beta1, beta2=beta2, eps=group["eps"],
                         weight_decay=group["weight_decay"])
            if self._nonfinite is not None:
                hyper["nonfinite"] = self._nonfinite
            tl.step(hyper, self.step_count)
        return loss

    def state_dict(self):
        """Hyperparameters and, per parameter, the raw state tensors (codes,
        means, indices, endpoints, scales or FP32 moments) and the step."""
        groups = [{k: v for k, v in g.items() if k != "params"} for g in self.param_groups]
        state = {}
        for i, st in enumerate(self._states):
            state[i] = {name: t.detach().clone() for name, t in (
                ("m_codes", st.m_codes), ("m_means", st.m_means), ("scalars", st.scalars), ("m_fp32", st.m_fp32),
                ("v_index", st.v_index), ("v_ends", st.v_ends), ("v_fp32", st.v_fp32)) if t is not None}
        return {"state": state, "param_groups": groups,
                "turbo": {"step": self.step_count, "v_bits": self.v_bits, "seed": self.seed,
                          "m_step_factor": self.m_step_factor, "block_size": self.block_size,
                          "m_block_size": self.m_block_size}}

    def load_state_dict(self, state_dict):
        """Restore a checkpoint written by state_dict(), bit for bit."""
        meta = state_dict["turbo"]
        if meta["v_bits"] != self.v_bits or meta["seed"] != self.seed:
            raise ValueError("checkpoint was written with another v_bits or rounding seed")
        if (meta.get("block_size", 128), meta.get("m_block_size", 64)) != (self.block_size, self.m_block_size):
            raise ValueError("checkpoint was written with another block_size or m_block_size")
        if len(state_dict["param_groups"]) != len(self.param_groups) or len(state_dict["state"]) != len(self._states):
            raise ValueError("checkpoint has another number of parameter groups or tensors")
        for g, saved in zip(self.param_groups, state_dict["param_groups"]):
            for k, v in saved.items():
                g[k] = v
        for i, st in enumerate(self._states):
            saved = state_dict["state"][i]
            for name in ("m_codes", "m_means", "scalars", "m_fp32", "v_index", "v_ends", "v_fp32"):
                t = getattr(st, name)
                if (t is None) != (name not in saved):
                    raise ValueError(f"checkpoint tensor {i} has a different state layout")
                if t is not None:
                    src = saved[name]
                    if src.numel() != t.numel() or src.dtype != t.dtype:
                        raise ValueError(f"checkpoint tensor {i}: {name} differs in size or type")
                    t.copy_(src.to(t.device))
        self.step_count = int(meta["step"])
        self.m_step_factor = float(meta["m_step_factor"])
        self._prepared = {}
