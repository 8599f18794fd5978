"""Python binding of the fused LM-head log-prob HIP library (MI355X / gfx950).

Thin ctypes layer over ``include/lmhead_logprob.h``: functions with the same names as the C entry
points, which only marshal torch tensors to device pointers and raise on a non-OK status, plus a
``torch.autograd.Function`` wrapper.  Every step of the computation runs in the HIP kernels;
there is no fallback: if the library is not built, importing works but any call raises.

PyTorch provides device memory and the current stream, nothing else.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "liblmhead_logprob.so")

LMH_OK = 0
LMH_ERR_INVALID_ARG = 1
LMH_ERR_UNSUPPORTED = 2
LMH_ERR_WORKSPACE_TOO_SMALL = 3
LMH_ERR_HIP = 4

# Entry points declared in include/lmhead_logprob.h, with their ctypes signatures.
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t
_F = ctypes.c_float
_INT = ctypes.c_int
_SIGNATURES = {
    "lmhead_logprob_fwd_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "lmhead_logprob_fwd_workspace_size_min": (_SZ, [_I64, _I64, _I64]),
    "lmhead_logprob_fwd": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "lmhead_logprob_fwd_partials": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _SZ, _P]),
    "lmhead_logprob_fwd_finalize": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _SZ, _P]),
    "lmhead_logprob_bwd_workspace_size": (_SZ, [_I64, _I64, _I64]),
    "lmhead_logprob_bwd_workspace_size_step": (_SZ, [_I64, _I64, _I64, _I64]),
    "lmhead_logprob_bwd": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P, _INT, _P, _SZ, _P]),
    "lmhead_logprob_fwd_ex": (_INT, [_P, _P, _P, _I64, _I64, _I64, _F, _P, _P, _P, _P, _P, _SZ, _P]),
    "lmhead_logprob_fwd_partials_ex": (_INT, [_P, _P, _P, _I64, _I64, _I64, _F, _I64, _I64, _INT, _P, _SZ, _P]),
    "lmhead_logprob_fwd_finalize_ex": (_INT, [_P, _I64, _I64, _I64, _P, _P, _P, _P, _P, _SZ, _P]),
    "lmhead_logprob_bwd_ex": (_INT, [_P, _P, _P, _I64, _I64, _I64, _F, _I64, _P, _P, _P, _P, _P, _P, _INT, _P, _SZ,
                                     _P]),
    "lmhead_logprob_fwd_noalloc": (_INT, [_P, _P, _P, _I64, _I64, _I64, _P, _P, _P, _P]),
    "lmhead_status_string": (ctypes.c_char_p, [_INT]),
}

# Size of the allocation-free forward's built-in scratch array (LMH_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 * 1024 * 1024

_lib = None


class LmheadError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status} ({lmhead_status_string(status)})")


def lib() -> ctypes.CDLL:
    """The loaded HIP library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"HIP library not built: {LIB_PATH} is missing "
                               "(run `python -c 'import __graft_entry__ as g; g.build()'` at the repo root)")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(l, name)
            fn.restype = res
            fn.argtypes = args
        _lib = l
    return _lib


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != LMH_OK:
        raise LmheadError(status, where)


def _check_tensor(t: Optional[torch.Tensor], name: str, dtype, numel: Optional[int] = None) -> None:
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if numel is not None and t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")


# ---------------------------------------------------------------------------------------------
# the C entry points, same names
# ---------------------------------------------------------------------------------------------

def lmhead_status_string(status: int) -> str:
    return lib().lmhead_status_string(int(status)).decode()


def lmhead_logprob_fwd_workspace_size(T: int, H: int, V: int) -> int:
    return int(lib().lmhead_logprob_fwd_workspace_size(T, H, V))


def lmhead_logprob_fwd_workspace_size_min(T: int, H: int, V: int) -> int:
    return int(lib().lmhead_logprob_fwd_workspace_size_min(T, H, V))


def lmhead_logprob_bwd_workspace_size(T: int, H: int, V: int) -> int:
    return int(lib().lmhead_logprob_bwd_workspace_size(T, H, V))


def lmhead_logprob_bwd_workspace_size_step(T: int, H: int, V: int, step: int) -> int:
    return int(lib().lmhead_logprob_bwd_workspace_size_step(T, H, V, step))


def _dims(hidden: torch.Tensor, weight: torch.Tensor):
    if hidden.dim() != 2 or weight.dim() != 2 or hidden.shape[1] != weight.shape[1]:
        raise ValueError(f"hidden [T,H] and weight [V,H] expected, got {tuple(hidden.shape)} and {tuple(weight.shape)}")
    return hidden.shape[0], hidden.shape[1], weight.shape[0]


def lmhead_logprob_fwd(hidden, weight, labels, logprob, entropy=None, lse=None, workspace=None, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((logprob, "logprob"), (entropy, "entropy"), (lse, "lse")):
        _check_tensor(t, n, torch.float32, T)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lmhead_logprob_fwd(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, _ptr(logprob), _ptr(entropy),
                                    _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)), "lmhead_logprob_fwd")


def lmhead_logprob_fwd_partials(hidden, weight, labels, workspace, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib().lmhead_logprob_fwd_partials(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, _ptr(workspace),
                                             ws_bytes, _stream(stream)), "lmhead_logprob_fwd_partials")


def lmhead_logprob_fwd_finalize(labels, T, H, V, logprob, entropy=None, lse=None, workspace=None, stream=None) -> None:
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((logprob, "logprob"), (entropy, "entropy"), (lse, "lse")):
        _check_tensor(t, n, torch.float32, T)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lmhead_logprob_fwd_finalize(_ptr(labels), T, H, V, _ptr(logprob), _ptr(entropy), _ptr(lse),
                                             _ptr(workspace), ws_bytes, _stream(stream)), "lmhead_logprob_fwd_finalize")


def lmhead_logprob_bwd(hidden, weight, labels, grad_logprob, lse, grad_hidden=None, grad_weight=None,
                       accumulate_grad_weight: bool = False, workspace=None, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    _check_tensor(grad_logprob, "grad_logprob", torch.float32, T)
    _check_tensor(lse, "lse", torch.float32, T)
    _check_tensor(grad_hidden, "grad_hidden", torch.float32, T * H)
    _check_tensor(grad_weight, "grad_weight", torch.float32, V * H)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().lmhead_logprob_bwd(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, _ptr(grad_logprob), _ptr(lse),
                                    _ptr(grad_hidden), _ptr(grad_weight), int(bool(accumulate_grad_weight)),
                                    _ptr(workspace), ws_bytes, _stream(stream)), "lmhead_logprob_bwd")


def lmhead_logprob_fwd_noalloc(hidden, weight, labels, logprob, entropy=None, lse=None, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((logprob, "logprob"), (entropy, "entropy"), (lse, "lse")):
        _check_tensor(t, n, torch.float32, T)
    _check(lib().lmhead_logprob_fwd_noalloc(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, _ptr(logprob),
                                            _ptr(entropy), _ptr(lse), _stream(stream)), "lmhead_logprob_fwd_noalloc")


def _nbytes(workspace) -> int:
    return 0 if workspace is None else workspace.numel() * workspace.element_size()


def lmhead_logprob_fwd_ex(hidden, weight, labels, temperature: float, logprob, entropy=None, lse=None, sum_p2=None,
                          workspace=None, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((logprob, "logprob"), (entropy, "entropy"), (lse, "lse"), (sum_p2, "sum_p2")):
        _check_tensor(t, n, torch.float32, T)
    _check(lib().lmhead_logprob_fwd_ex(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, float(temperature),
                                       _ptr(logprob), _ptr(entropy), _ptr(lse), _ptr(sum_p2), _ptr(workspace),
                                       _nbytes(workspace), _stream(stream)), "lmhead_logprob_fwd_ex")


def lmhead_logprob_fwd_partials_ex(hidden, weight, labels, temperature: float, vocab_start: int, vocab_total: int,
                                   want_sum_p2: bool, workspace, stream=None) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    _check(lib().lmhead_logprob_fwd_partials_ex(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, float(temperature),
                                                int(vocab_start), int(vocab_total), int(bool(want_sum_p2)),
                                                _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "lmhead_logprob_fwd_partials_ex")


def lmhead_logprob_fwd_finalize_ex(labels, T, H, V, logprob, entropy=None, lse=None, sum_p2=None, workspace=None,
                                   stream=None) -> None:
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((logprob, "logprob"), (entropy, "entropy"), (lse, "lse"), (sum_p2, "sum_p2")):
        _check_tensor(t, n, torch.float32, T)
    _check(lib().lmhead_logprob_fwd_finalize_ex(_ptr(labels), T, H, V, _ptr(logprob), _ptr(entropy), _ptr(lse),
                                                _ptr(sum_p2), _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "lmhead_logprob_fwd_finalize_ex")


def lmhead_logprob_bwd_ex(hidden, weight, labels, temperature: float, grad_logprob, lse, grad_entropy=None,
                          entropy=None, grad_hidden=None, grad_weight=None, accumulate_grad_weight: bool = False,
                          workspace=None, stream=None, vocab_start: int = 0) -> None:
    T, H, V = _dims(hidden, weight)
    _check_tensor(hidden, "hidden", torch.bfloat16)
    _check_tensor(weight, "weight", torch.bfloat16)
    _check_tensor(labels, "labels", torch.int32, T)
    for t, n in ((grad_logprob, "grad_logprob"), (lse, "lse"), (grad_entropy, "grad_entropy"), (entropy, "entropy")):
        _check_tensor(t, n, torch.float32, T)
    _check_tensor(grad_hidden, "grad_hidden", torch.float32, T * H)
    _check_tensor(grad_weight, "grad_weight", torch.float32, V * H)
    _check(lib().lmhead_logprob_bwd_ex(_ptr(hidden), _ptr(weight), _ptr(labels), T, H, V, float(temperature),
                                       int(vocab_start), _ptr(grad_logprob), _ptr(lse), _ptr(grad_entropy),
                                       _ptr(entropy), _ptr(grad_hidden), _ptr(grad_weight),
                                       int(bool(accumulate_grad_weight)),
                                       _ptr(workspace), _nbytes(workspace), _stream(stream)), "lmhead_logprob_bwd_ex")


# ---------------------------------------------------------------------------------------------
# allocation helpers and the autograd wrapper
# ---------------------------------------------------------------------------------------------

def _workspace(nbytes: int, device) -> torch.Tensor:
    # torch's caching allocator returns 256-byte (or better) aligned blocks
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)


def forward(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor, entropy: bool = False,
            want_lse: bool = False, stream=None, temperature: float = 1.0, sum_p2: bool = False):
    """Allocate outputs and workspace with torch and run lmhead_logprob_fwd (lmhead_logprob_fwd_ex
    when a temperature or sum_p2 is asked for).

    Returns (logprob [T] fp32, entropy [T] fp32 or None, lse [T] fp32 or None), plus sum_p2 [T]
    as a fourth element when sum_p2 is true."""
    T, H, V = _dims(hidden, weight)
    dev = hidden.device
    lp = torch.empty(T, dtype=torch.float32, device=dev)
    ent = torch.empty(T, dtype=torch.float32, device=dev) if entropy else None
    lse = torch.empty(T, dtype=torch.float32, device=dev) if want_lse else None
    p2 = torch.empty(T, dtype=torch.float32, device=dev) if sum_p2 else None
    ws = _workspace(lmhead_logprob_fwd_workspace_size(T, H, V), dev)
    if temperature == 1.0 and not sum_p2:
        lmhead_logprob_fwd(hidden, weight, labels, lp, ent, lse, ws, stream)
    else:
        lmhead_logprob_fwd_ex(hidden, weight, labels, temperature, lp, ent, lse, p2, ws, stream)
    return (lp, ent, lse, p2) if sum_p2 else (lp, ent, lse)


def backward(hidden, weight, labels, grad_logprob, lse, need_hidden=True, need_weight=True, stream=None,
             temperature: float = 1.0, grad_entropy=None, entropy=None, vocab_start: int = 0):
    """Allocate gradients and workspace with torch and run lmhead_logprob_bwd (overwrite mode;
    lmhead_logprob_bwd_ex when a temperature, an entropy gradient or a vocabulary shard is given)."""
    T, H, V = _dims(hidden, weight)
    dev = hidden.device
    gh = torch.empty((T, H), dtype=torch.float32, device=dev) if need_hidden else None
    # an empty batch contributes nothing: the library leaves the buffers untouched for T == 0
    alloc = torch.zeros if T == 0 else torch.empty
    gw = alloc((V, H), dtype=torch.float32, device=dev) if need_weight else None
    ws = _workspace(lmhead_logprob_bwd_workspace_size(T, H, V), dev)
    if temperature == 1.0 and grad_entropy is None and vocab_start == 0:
        lmhead_logprob_bwd(hidden, weight, labels, grad_logprob, lse, gh, gw, False, ws, stream)
    else:
        lmhead_logprob_bwd_ex(hidden, weight, labels, temperature, grad_logprob, lse, grad_entropy, entropy, gh, gw,
                              False, ws, stream, vocab_start)
    return gh, gw


class _FusedLogprob(torch.autograd.Function):
    @staticmethod
    def forward(ctx, hidden, weight, labels, want_entropy, temperature):
        # hidden arrives in the caller's dtype; the projection takes it in the weight's dtype, and
        # the gradient goes back in the caller's dtype with no rounding to bf16 on the way
        h = hidden.to(weight.dtype).contiguous()
        lp, ent, lse = forward(h, weight, labels, entropy=want_entropy, want_lse=True, temperature=temperature)
        ctx.save_for_backward(h, weight, labels, lse, ent)
        ctx.temperature = temperature
        ctx.hidden_dtype = hidden.dtype
        ctx.set_materialize_grads(False)
        return lp, ent

    @staticmethod
    def backward(ctx, grad_lp, grad_ent):
        hidden, weight, labels, lse, ent = ctx.saved_tensors
        T = hidden.shape[0]
        if grad_lp is None:
            g = torch.zeros(T, dtype=torch.float32, device=hidden.device)
        else:
            g = grad_lp.contiguous().to(torch.float32)
        ge = None if grad_ent is None else grad_ent.contiguous().to(torch.float32)
        gh, gw = backward(hidden, weight, labels, g, lse, ctx.needs_input_grad[0], ctx.needs_input_grad[1],
                          temperature=ctx.temperature, grad_entropy=ge, entropy=ent if ge is not None else None)
        if gh is not None:
            gh = gh.to(ctx.hidden_dtype)
        if gw is not None:
            gw = gw.to(weight.dtype)
        return gh, gw, None, None, None


def logprob(hidden: torch.Tensor, weight: torch.Tensor, labels: torch.Tensor, entropy: bool = False,
            temperature: float = 1.0):
    """Fused LM-head log-prob with autograd.

    hidden [..., H] (any float dtype; cast to weight's dtype before the projection, and the fp32
    gradient returned in hidden's dtype, as the pages' adapter does), weight [V, H] bf16, labels
    [...] integer.  Leading dimensions are flattened to token rows.  Labels outside [0, V) of any
    integer width follow the out-of-range rule (they are mapped to -1 before the int32 conversion,
    so a wide label never wraps onto a vocabulary id).  The logits are divided by the fp32
    temperature before the softmax.  Returns (logprob [...], entropy [...] or None), fp32; both
    are differentiable (the entropy's gradient is -p (log p + entropy) per logit)."""
    if weight.dtype != torch.bfloat16:
        raise ValueError("weight must be bf16")
    if labels.dtype.is_floating_point or labels.dtype.is_complex or labels.dtype == torch.bool:
        raise ValueError(f"labels must be an integer tensor, got {labels.dtype}")
    lead = hidden.shape[:-1]
    h2 = hidden.reshape(-1, hidden.shape[-1])
    V = weight.shape[0]
    y = labels.reshape(-1)
    y = torch.where((y >= 0) & (y < V), y, torch.full_like(y, -1)).to(torch.int32).contiguous()
    lp, ent = _FusedLogprob.apply(h2, weight.contiguous(), y, entropy, float(temperature))
    return lp.reshape(lead), (ent.reshape(lead) if ent is not None else None)
