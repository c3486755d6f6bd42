"""Device-buffer helpers over the C ABI: allocate the tensors one layer call
needs and invoke the library.  Allocation and argument marshalling only."""
from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def torch_dtype(name: str):
    return torch.bfloat16 if name == "bf16" else torch.float32


def to_device(a: np.ndarray, dtype, device="cuda") -> torch.Tensor:
    """Copy a host array to the device in `dtype` (bf16-exact values stay exact)."""
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dtype)


class PtbShard:
    """Holds the inputs, parameters, outputs and workspaces of one shard."""

    def __init__(self, cfg, inputs: dict, device="cuda"):
        self.cfg = cfg
        self.dims = B.dims_from(cfg)
        dt = torch_dtype(cfg.dtype)
        self.dt = dt
        self.x = to_device(inputs["x"], dt, device)
        self.gamma = to_device(inputs["gamma"], torch.float32, device)
        self.beta = to_device(inputs["beta"], torch.float32, device)
        self.w_in = to_device(inputs["w_in"], dt, device)
        self.w_out = to_device(inputs["w_out"], dt, device)
        self.dy = to_device(inputs["dy"], dt, device)
        self.y = torch.empty_like(self.x)
        self.dx = torch.empty_like(self.x)
        self.dgamma = torch.empty_like(self.gamma)
        self.dbeta = torch.empty_like(self.beta)
        self.dw_in = torch.empty_like(self.w_in)
        self.dw_out = torch.empty_like(self.w_out)
        self.saved = torch.empty(B.ptb_saved_bytes(self.dims), dtype=torch.uint8, device=device)
        self.scratch = torch.empty(B.ptb_scratch_bytes(self.dims), dtype=torch.uint8, device=device)

    def forward(self, stream=None, use_scratch=True):
        B.ptb_forward(self.dims, self.x, self.gamma, self.beta, self.w_in, self.w_out, self.y,
                      self.saved, self.scratch if use_scratch else None, stream)

    def backward(self, stream=None):
        B.ptb_backward(self.dims, self.x, self.gamma, self.w_in, self.w_out, self.saved, self.dy,
                       self.dx, self.dgamma, self.dbeta, self.dw_in, self.dw_out, self.scratch,
                       stream)

    def forward_stage(self, stage, stream=None):
        B.ptb_forward_stage(self.dims, stage, self.x, self.gamma, self.beta, self.w_in,
                            self.w_out, self.y, self.saved, self.scratch, stream)

    def backward_stage(self, stage, stream=None):
        B.ptb_backward_stage(self.dims, stage, self.x, self.gamma, self.w_in, self.w_out,
                             self.saved, self.dy, self.dx, self.dgamma, self.dbeta, self.dw_in,
                             self.dw_out, self.scratch, stream)

    def outputs(self) -> dict:
        """Host fp64 copies of every output."""
        f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        return dict(y=f(self.y), dx=f(self.dx), dgamma=f(self.dgamma), dbeta=f(self.dbeta),
                    dw_in=f(self.dw_in), dw_out=f(self.dw_out))


class SerialShard(PtbShard):
    """The serial pre-LN block on the same inputs and weights as a PtbShard,
    plus the second LayerNorm's (gamma2, beta2)."""

    def __init__(self, cfg, inputs: dict, gamma2, beta2, device="cuda"):
        super().__init__(cfg, inputs, device)
        self.gamma2 = to_device(gamma2, torch.float32, device)
        self.beta2 = to_device(beta2, torch.float32, device)
        self.dgamma2 = torch.empty_like(self.gamma2)
        self.dbeta2 = torch.empty_like(self.beta2)
        self.saved = torch.empty(B.ptb_serial_saved_bytes(self.dims), dtype=torch.uint8,
                                 device=device)
        self.scratch = torch.empty(B.ptb_serial_scratch_bytes(self.dims), dtype=torch.uint8,
                                   device=device)

    def forward(self, stream=None, use_scratch=True):
        B.ptb_serial_forward(self.dims, self.x, self.gamma, self.beta, self.gamma2, self.beta2,
                             self.w_in, self.w_out, self.y, self.saved,
                             self.scratch if use_scratch else None, stream)

    def backward(self, stream=None):
        B.ptb_serial_backward(self.dims, self.x, self.gamma, self.gamma2, self.w_in, self.w_out,
                              self.saved, self.dy, self.dx, self.dgamma, self.dbeta, self.dgamma2,
                              self.dbeta2, self.dw_in, self.dw_out, self.scratch, stream)

    def forward_stage(self, stage, stream=None):
        raise NotImplementedError("the serial block runs as whole forward / backward calls")

    backward_stage = forward_stage

    def outputs(self) -> dict:
        out = super().outputs()
        f = lambda t: t.detach().float().cpu().numpy().astype(np.float64)
        out.update(dgamma2=f(self.dgamma2), dbeta2=f(self.dbeta2))
        return out


class LambState:
    """Device copies of per-tensor (w, g, m, v) plus the scratch of one step.

    grad_dtype: one name for every tensor, or a list with one name per tensor.
    bf16_copy: also keep a bf16 copy of each w that the step refreshes."""

    def __init__(self, tensors: list, grad_dtype="bf16", weight_decay=0.01, device="cuda",
                 bf16_copy=False):
        gdts = grad_dtype if isinstance(grad_dtype, (list, tuple)) else [grad_dtype] * len(tensors)
        self.params = []
        for t, gd in zip(tensors, gdts):
            p = dict(w=to_device(t["w"], torch.float32, device),
                     g=to_device(t["g"], torch_dtype(gd), device),
                     m=to_device(t["m"], torch.float32, device),
                     v=to_device(t["v"], torch.float32, device),
                     weight_decay=t.get("weight_decay", weight_decay))
            if bf16_copy:
                p["w_bf16"] = torch.empty(p["w"].shape, dtype=torch.bfloat16, device=device)
            self.params.append(p)
        self.desc = B.lamb_tensors(self.params)
        self.scratch = torch.empty(B.lamb_scratch_bytes(self.desc), dtype=torch.uint8,
                                   device=device)
        self.ratios = torch.empty(len(tensors), dtype=torch.float32, device=device)

    def step(self, step, lr, beta1, beta2, eps, stream=None):
        B.lamb_step(self.desc, lr, beta1, beta2, eps, step, self.ratios, self.scratch, stream)

    def set_grads(self, grads: list):
        for p, g in zip(self.params, grads):
            p["g"].copy_(torch.from_numpy(np.ascontiguousarray(g, dtype=np.float32)).to(p["g"].dtype))


def shard_bounds(n: int, n_shards: int, align: int = 8) -> list:
    """Contiguous element ranges of n over n_shards ranks, every start a
    multiple of `align` (16-byte aligned fp32 and bf16 views); the last
    ranks may be shorter or empty."""
    per = -(-n // n_shards)
    per = -(-per // align) * align
    return [(min(n, r * per), min(n, (r + 1) * per)) for r in range(n_shards)]


class ShardedLamb:
    """ZeRO-2 sharded LAMB over a list of LAMB parameter dicts (w, g, m, v,
    optional w_bf16, weight_decay; e.g. LambState.params): rank r owns
    range r of every tensor (views into the same device tensors).  Each
    rank's shard step is lamb_shard_norms, a sum of the per-rank norms (the
    data-parallel all-reduce), then lamb_shard_apply."""

    def __init__(self, all_params: list, n_shards: int):
        self.ranks = []
        nt = len(all_params)
        device = all_params[0]["w"].device
        for r in range(n_shards):
            params = []
            for p in all_params:
                a, b = shard_bounds(p["w"].numel(), n_shards)[r]
                # element ranges of the flattened (contiguous) tensors
                q = {k: p[k].view(-1)[a:b] for k in ("w", "g", "m", "v")}
                if p.get("w_bf16") is not None:
                    q["w_bf16"] = p["w_bf16"].view(-1)[a:b]
                q["weight_decay"] = p["weight_decay"]
                params.append(q)
            # ranks with an empty range of some tensor pass that tensor with
            # n = 0 nowhere: such a rank keeps only its non-empty tensors
            keep = [i for i, q in enumerate(params) if q["w"].numel() > 0]
            desc = B.lamb_tensors([params[i] for i in keep]) if keep else None
            scratch = (torch.empty(B.lamb_scratch_bytes(desc), dtype=torch.uint8, device=device)
                       if keep else None)
            self.ranks.append(dict(keep=keep, desc=desc, scratch=scratch, params=params,
                                   norms=torch.zeros(2 * nt, dtype=torch.float64, device=device)))
        self.ratios = torch.empty(nt, dtype=torch.float32, device=device)

    def norms(self, rank, step, beta1, beta2, eps, stream=None):
        """This rank's first half; returns its fp64 [2 n_tensors] norms."""
        R = self.ranks[rank]
        R["norms"].zero_()
        if R["keep"]:
            part = torch.empty(2 * len(R["keep"]), dtype=torch.float64, device=R["norms"].device)
            B.lamb_shard_norms(R["desc"], beta1, beta2, eps, step, part, R["scratch"], stream)
            idx = torch.tensor([[2 * i, 2 * i + 1] for i in R["keep"]],
                               device=part.device).reshape(-1)
            R["norms"].index_copy_(0, idx, part)
        return R["norms"]

    def apply(self, rank, total, step, lr, beta1, beta2, eps, stream=None):
        """This rank's second half with the norms summed over all ranks."""
        R = self.ranks[rank]
        if not R["keep"]:
            return
        idx = torch.tensor([[2 * i, 2 * i + 1] for i in R["keep"]], device=total.device).reshape(-1)
        sub = total.index_select(0, idx).contiguous()
        ratios = torch.empty(len(R["keep"]), dtype=torch.float32, device=total.device)
        B.lamb_shard_apply(R["desc"], lr, beta1, beta2, eps, step, sub, ratios, R["scratch"],
                           stream)
        self.ratios.index_copy_(0, torch.tensor(R["keep"], device=total.device), ratios)

    def step(self, step, lr, beta1, beta2, eps, stream=None):
        """All ranks on this one device in turn; the sum stands in for the
        all-reduce between the halves."""
        total = None
        for r in range(len(self.ranks)):
            n = self.norms(r, step, beta1, beta2, eps, stream).clone()
            total = n if total is None else total + n
        for r in range(len(self.ranks)):
            self.apply(r, total, step, lr, beta1, beta2, eps, stream)
