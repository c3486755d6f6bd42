"""ctypes binding of libptb.so.  Argument marshalling only: every step of the
computation runs in the library's HIP kernels.  The functions carry the C
names (include/ptb.h, include/ptb_ops.h) and take torch tensors for device
buffers; the stream is torch's current stream unless one is given.

If the library cannot be loaded every call raises RuntimeError: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libptb.so")

PTB_F32, PTB_BF16 = 0, 1
STATUS = {0: "PTB_OK", -1: "PTB_ERR_INVALID_ARG", -2: "PTB_ERR_UNSUPPORTED",
          -3: "PTB_ERR_WORKSPACE", -4: "PTB_ERR_HIP"}
EXPORTED = ("ptb_saved_bytes", "ptb_scratch_bytes", "ptb_forward", "ptb_backward",
            "lamb_scratch_bytes", "lamb_step", "ptb_status_string",
            "ptb_forward_stage", "ptb_backward_stage",
            "ptb_layernorm_forward", "ptb_gemm_workspace_bytes", "ptb_gemm", "ptb_swa_forward",
            "ptb_swa_backward", "ptb_serial_saved_bytes", "ptb_serial_scratch_bytes",
            "ptb_serial_forward", "ptb_serial_backward", "lamb_shard_norms", "lamb_shard_apply",
            "ptb_layernorm_scratch_bytes", "ptb_layernorm_backward",
            "lamb_noalloc_max_scratch_bytes", "lamb_step_noalloc")
FWD_STAGES = ("layernorm", "gemm_in", "attention", "gemm_out")
BWD_STAGES = ("gemm_dcat", "gemm_dw_out", "attention", "gemm_dw_in", "gemm_dxn", "layernorm")


class PtbDims(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq", ctypes.c_int32), ("hidden", ctypes.c_int32),
                ("n_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("ffn", ctypes.c_int32), ("window", ctypes.c_int32),
                ("add_residual", ctypes.c_int32), ("ln_eps", ctypes.c_float),
                ("dtype", ctypes.c_int32)]


class LambTensor(ctypes.Structure):
    _fields_ = [("w", ctypes.c_void_p), ("g", ctypes.c_void_p), ("m", ctypes.c_void_p),
                ("v", ctypes.c_void_p), ("w_bf16", ctypes.c_void_p), ("n", ctypes.c_int64),
                ("weight_decay", ctypes.c_float), ("grad_dtype", ctypes.c_int32)]


class PtbError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {STATUS.get(status, status)}")
        self.status = status


_lib = None


def lib():
    """The loaded library (raises RuntimeError when it is missing)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with "
                               "`python -m transformer_block_lamb_amd.build`")
        L = ctypes.CDLL(_LIB_PATH)
        vp, sz, i32, i64, f32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
        pd = ctypes.POINTER(PtbDims)
        pl = ctypes.POINTER(LambTensor)
        sig = {
            "ptb_saved_bytes": (sz, [pd]),
            "ptb_scratch_bytes": (sz, [pd]),
            "ptb_forward": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz, vp]),
            "ptb_backward": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp, vp, vp,
                                            vp, sz, vp]),
            "ptb_forward_stage": (ctypes.c_int, [pd, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz,
                                                 vp]),
            "ptb_backward_stage": (ctypes.c_int, [pd, i32, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp,
                                                  vp, vp, vp, sz, vp]),
            "lamb_scratch_bytes": (sz, [pl, i32]),
            "lamb_step": (ctypes.c_int, [pl, i32, f32, f32, f32, f32, i64, vp, vp, sz, vp]),
            "lamb_noalloc_max_scratch_bytes": (sz, []),
            "lamb_step_noalloc": (ctypes.c_int, [pl, i32, f32, f32, f32, f32, i64, vp, vp]),
            "lamb_shard_norms": (ctypes.c_int, [pl, i32, f32, f32, f32, i64, vp, vp, sz, vp]),
            "lamb_shard_apply": (ctypes.c_int, [pl, i32, f32, f32, f32, f32, i64, vp, vp, vp, sz,
                                                vp]),
            "ptb_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "ptb_layernorm_forward": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, f32, vp, vp, vp,
                                                     vp]),
            "ptb_layernorm_scratch_bytes": (sz, [i32, i32]),
            "ptb_layernorm_backward": (ctypes.c_int, [i32, i32, i32, vp, vp, vp, vp, vp, vp, vp,
                                                      vp, vp, vp, sz, vp]),
            "ptb_gemm_workspace_bytes": (ctypes.c_size_t, []),
            "ptb_gemm": (ctypes.c_int, [i32, i32, i32, i32, i32, i32, vp, i64, vp, i64, vp, i64,
                                        i32, vp, ctypes.c_size_t, vp]),
            "ptb_swa_forward": (ctypes.c_int, [pd, vp, vp, i64, vp, vp]),
            "ptb_swa_backward": (ctypes.c_int, [pd, vp, vp, i64, vp, vp, vp, vp, vp]),
            "ptb_serial_saved_bytes": (sz, [pd]),
            "ptb_serial_scratch_bytes": (sz, [pd]),
            "ptb_serial_forward": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                                  sz, vp]),
            "ptb_serial_backward": (ctypes.c_int, [pd, vp, vp, vp, vp, vp, vp, sz, vp, vp, vp, vp,
                                                   vp, vp, vp, vp, vp, sz, vp]),
        }
        for name, (res, args) in sig.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _lib = L
    return _lib


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _nbytes(t):
    return t.numel() * t.element_size()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str):
    if status != 0:
        raise PtbError(status, where)


def make_dims(batch, seq, hidden, n_heads, head_dim, ffn, window, add_residual=1, ln_eps=1e-5,
              dtype=PTB_BF16) -> PtbDims:
    return PtbDims(batch, seq, hidden, n_heads, head_dim, ffn, window, add_residual, ln_eps, dtype)


def dims_from(cfg) -> PtbDims:
    """PtbDims from any object with the layer's dimension attributes."""
    dt = PTB_BF16 if getattr(cfg, "dtype", "bf16") in ("bf16", PTB_BF16) else PTB_F32
    return make_dims(cfg.batch, cfg.seq, cfg.hidden, cfg.n_heads, cfg.head_dim, cfg.ffn,
                     cfg.window, cfg.add_residual, cfg.ln_eps, dt)


# ------------------------------------------------------------------ block
def ptb_saved_bytes(dims: PtbDims) -> int:
    return lib().ptb_saved_bytes(ctypes.byref(dims))


def ptb_scratch_bytes(dims: PtbDims) -> int:
    return lib().ptb_scratch_bytes(ctypes.byref(dims))


def _opt_nbytes(t):
    return 0 if t is None else _nbytes(t)


def ptb_forward(dims, x, ln_gamma, ln_beta, w_in, w_out, y, saved, scratch, stream=None):
    """scratch: the ptb_scratch_bytes buffer (also used by ptb_backward), or
    None for whole-tile GEMM schedules."""
    _check(lib().ptb_forward(ctypes.byref(dims), _ptr(x), _ptr(ln_gamma), _ptr(ln_beta),
                             _ptr(w_in), _ptr(w_out), _ptr(y), _ptr(saved), _nbytes(saved),
                             _ptr(scratch), _opt_nbytes(scratch), _stream(stream)),
           "ptb_forward")


def ptb_backward(dims, x, ln_gamma, w_in, w_out, saved, dy, dx, d_ln_gamma, d_ln_beta, dw_in,
                 dw_out, scratch, stream=None):
    _check(lib().ptb_backward(ctypes.byref(dims), _ptr(x), _ptr(ln_gamma), _ptr(w_in),
                              _ptr(w_out), _ptr(saved), saved.numel() * saved.element_size(),
                              _ptr(dy), _ptr(dx), _ptr(d_ln_gamma), _ptr(d_ln_beta),
                              _ptr(dw_in), _ptr(dw_out), _ptr(scratch),
                              scratch.numel() * scratch.element_size(), _stream(stream)),
           "ptb_backward")


def ptb_forward_stage(dims, stage, x, ln_gamma, ln_beta, w_in, w_out, y, saved, scratch,
                      stream=None):
    _check(lib().ptb_forward_stage(ctypes.byref(dims), stage, _ptr(x), _ptr(ln_gamma),
                                   _ptr(ln_beta), _ptr(w_in), _ptr(w_out), _ptr(y), _ptr(saved),
                                   _nbytes(saved), _ptr(scratch), _opt_nbytes(scratch),
                                   _stream(stream)),
           f"ptb_forward_stage({stage})")


def ptb_backward_stage(dims, stage, x, ln_gamma, w_in, w_out, saved, dy, dx, d_ln_gamma,
                       d_ln_beta, dw_in, dw_out, scratch, stream=None):
    _check(lib().ptb_backward_stage(ctypes.byref(dims), stage, _ptr(x), _ptr(ln_gamma),
                                    _ptr(w_in), _ptr(w_out), _ptr(saved),
                                    saved.numel() * saved.element_size(), _ptr(dy), _ptr(dx),
                                    _ptr(d_ln_gamma), _ptr(d_ln_beta), _ptr(dw_in), _ptr(dw_out),
                                    _ptr(scratch), scratch.numel() * scratch.element_size(),
                                    _stream(stream)),
           f"ptb_backward_stage({stage})")


# ------------------------------------------------------------------ LAMB
def lamb_tensors(params) -> ctypes.Array:
    """params: list of dicts with torch tensors w, g, m, v, optional w_bf16
    (receives the bf16 copy of the new w) and optional weight_decay."""
    arr = (LambTensor * len(params))()
    for i, p in enumerate(params):
        gdt = PTB_BF16 if p["g"].dtype == torch.bfloat16 else PTB_F32
        arr[i] = LambTensor(_ptr(p["w"]), _ptr(p["g"]), _ptr(p["m"]), _ptr(p["v"]),
                            _ptr(p.get("w_bf16")), p["w"].numel(), p.get("weight_decay", 0.0),
                            gdt)
    return arr


def lamb_scratch_bytes(tensors) -> int:
    return lib().lamb_scratch_bytes(tensors, len(tensors))


def lamb_step(tensors, lr, beta1, beta2, eps, step, ratios_out, scratch, stream=None):
    _check(lib().lamb_step(tensors, len(tensors), lr, beta1, beta2, eps, step,
                           _ptr(ratios_out), _ptr(scratch),
                           scratch.numel() * scratch.element_size(), _stream(stream)),
           "lamb_step")


def lamb_noalloc_max_scratch_bytes() -> int:
    return int(lib().lamb_noalloc_max_scratch_bytes())


def lamb_step_noalloc(tensors, lr, beta1, beta2, eps, step, ratios_out, stream=None):
    """lamb_step with the library's static per-device scratch (no buffer)."""
    _check(lib().lamb_step_noalloc(tensors, len(tensors), lr, beta1, beta2, eps, step,
                                   _ptr(ratios_out), _stream(stream)),
           "lamb_step_noalloc")


def lamb_shard_norms(tensors, beta1, beta2, eps, step, norms_out, scratch, stream=None):
    """First half of the sharded step: m, v of the shard updated; norms_out
    (fp64 [2 n]) receives the shard's sums of w^2 and u^2 per tensor."""
    _check(lib().lamb_shard_norms(tensors, len(tensors), beta1, beta2, eps, step,
                                  _ptr(norms_out), _ptr(scratch),
                                  scratch.numel() * scratch.element_size(), _stream(stream)),
           "lamb_shard_norms")


def lamb_shard_apply(tensors, lr, beta1, beta2, eps, step, norms, ratios_out, scratch,
                     stream=None):
    """Second half: w of the shard updated from the norms summed over shards."""
    _check(lib().lamb_shard_apply(tensors, len(tensors), lr, beta1, beta2, eps, step,
                                  _ptr(norms), _ptr(ratios_out), _ptr(scratch),
                                  scratch.numel() * scratch.element_size(), _stream(stream)),
           "lamb_shard_apply")


def ptb_status_string(status: int) -> str:
    return lib().ptb_status_string(status).decode()


# ------------------------------------------------------------------ components
def ptb_layernorm_forward(dtype, rows, width, x, gamma, beta, eps, xn, mean, rstd, stream=None):
    _check(lib().ptb_layernorm_forward(dtype, rows, width, _ptr(x), _ptr(gamma), _ptr(beta), eps,
                                       _ptr(xn), _ptr(mean), _ptr(rstd), _stream(stream)),
           "ptb_layernorm_forward")


def ptb_layernorm_scratch_bytes(rows, width) -> int:
    return int(lib().ptb_layernorm_scratch_bytes(rows, width))


def ptb_layernorm_backward(dtype, rows, width, x, gamma, mean, rstd, dxn, dy, dx, dgamma, dbeta,
                           scratch, stream=None):
    _check(lib().ptb_layernorm_backward(dtype, rows, width, _ptr(x), _ptr(gamma), _ptr(mean),
                                        _ptr(rstd), _ptr(dxn), _ptr(dy), _ptr(dx), _ptr(dgamma),
                                        _ptr(dbeta), _ptr(scratch), _nbytes(scratch),
                                        _stream(stream)),
           "ptb_layernorm_backward")


def ptb_gemm_workspace_bytes():
    return int(lib().ptb_gemm_workspace_bytes())


def ptb_gemm(dtype, a_layout, b_layout, M, N, K, a, lda, b, ldb, c, ldc, c_f32=0,
             workspace=None, stream=None):
    ws_bytes = 0 if workspace is None else _nbytes(workspace)
    _check(lib().ptb_gemm(dtype, a_layout, b_layout, M, N, K, _ptr(a), lda, _ptr(b), ldb,
                          _ptr(c), ldc, c_f32, _ptr(workspace), ws_bytes, _stream(stream)),
           "ptb_gemm")


def ptb_swa_forward(dims, qkv, o, ldo, lse, stream=None):
    _check(lib().ptb_swa_forward(ctypes.byref(dims), _ptr(qkv), _ptr(o), ldo, _ptr(lse),
                                 _stream(stream)), "ptb_swa_forward")


def ptb_swa_backward(dims, qkv, o, ldo, d_o, lse, dqkv, dvec, stream=None):
    _check(lib().ptb_swa_backward(ctypes.byref(dims), _ptr(qkv), _ptr(o), ldo, _ptr(d_o),
                                  _ptr(lse), _ptr(dqkv), _ptr(dvec), _stream(stream)),
           "ptb_swa_backward")


def ptb_serial_saved_bytes(dims: PtbDims) -> int:
    return int(lib().ptb_serial_saved_bytes(ctypes.byref(dims)))


def ptb_serial_scratch_bytes(dims: PtbDims) -> int:
    return int(lib().ptb_serial_scratch_bytes(ctypes.byref(dims)))


def ptb_serial_forward(dims, x, ln1_gamma, ln1_beta, ln2_gamma, ln2_beta, w_in, w_out, y, saved,
                       scratch, stream=None):
    _check(lib().ptb_serial_forward(ctypes.byref(dims), _ptr(x), _ptr(ln1_gamma), _ptr(ln1_beta),
                                    _ptr(ln2_gamma), _ptr(ln2_beta), _ptr(w_in), _ptr(w_out),
                                    _ptr(y), _ptr(saved), _nbytes(saved), _ptr(scratch),
                                    _opt_nbytes(scratch), _stream(stream)),
           "ptb_serial_forward")


def ptb_serial_backward(dims, x, ln1_gamma, ln2_gamma, w_in, w_out, saved, dy, dx, d_ln1_gamma,
                        d_ln1_beta, d_ln2_gamma, d_ln2_beta, dw_in, dw_out, scratch, stream=None):
    _check(lib().ptb_serial_backward(ctypes.byref(dims), _ptr(x), _ptr(ln1_gamma), _ptr(ln2_gamma),
                                     _ptr(w_in), _ptr(w_out), _ptr(saved), _nbytes(saved), _ptr(dy),
                                     _ptr(dx), _ptr(d_ln1_gamma), _ptr(d_ln1_beta),
                                     _ptr(d_ln2_gamma), _ptr(d_ln2_beta), _ptr(dw_in), _ptr(dw_out),
                                     _ptr(scratch), _nbytes(scratch), _stream(stream)),
           "ptb_serial_backward")
