"""ctypes binding over librlk.so (C ABI declared in include/rlk.h).

Argument marshalling only: dtype/device/stride checks, output allocation
through torch, and the call with raw device pointers on torch's current
stream.  Every step of the computation runs in the HIP kernels; a missing or
unloadable library raises RlkError -- there is no fallback.
"""

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

_STATUS = {0: "RLK_OK", 1: "RLK_ERR_INVALID_ARG", 2: "RLK_ERR_UNSUPPORTED", 3: "RLK_ERR_LAUNCH"}


class RlkError(RuntimeError):
    """Raised when the library is missing or a call returns a non-zero status."""

    def __init__(self, msg, status=None):
        super().__init__(msg)
        self.status = status


def library_path():
    return os.path.join(_HERE, "librlk.so")


def load_library():
    """Load librlk.so once and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RlkError(f"HIP library not built: {path} (run python -m invariant_logprob_amd.build)")
    lib = ctypes.CDLL(path)
    vp, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
    lib.rlk_logp_selected.argtypes = [vp, i64, vp, vp, i64, i64, vp, vp, vp]
    lib.rlk_logp_selected.restype = ctypes.c_int
    lib.rlk_logp_entropy.argtypes = [vp, i64, vp, vp, i64, i64, vp, vp, vp, vp]
    lib.rlk_logp_entropy.restype = ctypes.c_int
    lib.rlk_log_softmax.argtypes = [vp, i64, vp, vp, i64, i64, vp, i64, vp]
    lib.rlk_log_softmax.restype = ctypes.c_int
    f32 = ctypes.c_float
    lib.rlk_token_losses.argtypes = [vp, vp, vp, vp, vp, i64, f32, f32, f32, vp, vp, vp, vp, vp]
    lib.rlk_token_losses.restype = ctypes.c_int
    lib.rlk_linear_logp_workspace_size.argtypes = [i64, i64, i64]
    lib.rlk_linear_logp_workspace_size.restype = sz
    lib.rlk_linear_logp.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, vp, vp, vp, sz, vp]
    lib.rlk_linear_logp.restype = ctypes.c_int
    lib.rlk_linear_logp_noalloc.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, vp, vp, vp]
    lib.rlk_linear_logp_noalloc.restype = ctypes.c_int
    lib.rlk_logp_backward.argtypes = [vp, i64, vp, i64, vp, i64, i64, vp, vp, vp, vp, i64, i64, vp,
                                      i64, vp]
    lib.rlk_logp_backward.restype = ctypes.c_int
    lib.rlk_linear_logp_with_logits.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, vp, vp,
                                                vp, i64, vp, sz, vp]
    lib.rlk_linear_logp_with_logits.restype = ctypes.c_int
    lib.rlk_logp_backward_f32.argtypes = [vp, i64, vp, vp, vp, vp, i64, i64, vp, i64, vp]
    lib.rlk_logp_backward_f32.restype = ctypes.c_int
    lib.rlk_linear_logp_param_grads_workspace_size.argtypes = [i64, i64, i64]
    lib.rlk_linear_logp_param_grads_workspace_size.restype = sz
    lib.rlk_linear_logp_param_grads.argtypes = [vp, i64, vp, i64, vp, vp, vp, vp, i64, i64, i64, vp,
                                                i64, vp, i64, vp, sz, vp]
    lib.rlk_linear_logp_param_grads.restype = ctypes.c_int
    lib.rlk_linear_logp_param_grads_from_logits.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, vp,
                                                            vp, i64, i64, i64, vp, i64, vp, i64,
                                                            vp, sz, vp]
    lib.rlk_linear_logp_param_grads_from_logits.restype = ctypes.c_int
    lib.rlk_status_string.argtypes = [ctypes.c_int]
    lib.rlk_status_string.restype = ctypes.c_char_p
    lib.rlk_build_info.argtypes = []
    lib.rlk_build_info.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def build_info():
    return load_library().rlk_build_info().decode()


def _raise(status, fn):
    if status != 0:
        raise RlkError(f"{fn} failed: {_STATUS.get(status, status)}", status)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _device_of(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")
    return t.device


def _matrix(t, name, dtype, read=True):
    _device_of(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D, got shape {tuple(t.shape)}")
    if t.shape[1] > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} must have unit stride along its last dimension")
    if t.shape[0] > 1:
        ld = t.stride(0)
    else:
        # a single row: any leading dimension the library accepts will do
        # (a multiple of 8 bf16 or 4 fp32 elements, 16 bytes)
        mult = 16 // t.element_size()
        ld = (t.shape[1] + mult - 1) // mult * mult
    # The library reads input rows in whole aligned groups up to ld, the last
    # row included, so the storage must hold all of it.
    if read and t.numel() > 0:
        end = (t.storage_offset() + (t.shape[0] - 1) * ld + ld) * t.element_size()
        if end > t.untyped_storage().nbytes():
            raise ValueError(f"{name}: the storage must hold {ld} elements in every row, the last "
                             f"one included (pad the rows to a multiple of 8 elements)")
    return ld


def _rows(t, name, n, dtype):
    _device_of(t, name)
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != 1 or t.shape[0] != n:
        raise ValueError(f"{name} must have shape ({n},), got {tuple(t.shape)}")
    if n > 1 and t.stride(0) != 1:
        raise ValueError(f"{name} must be contiguous")


def _mask(mask, n):
    if mask is None:
        return None
    if mask.dtype == torch.bool:
        mask = mask.view(torch.uint8)
    _rows(mask, "mask", n, torch.uint8)
    return mask


def _workspace(workspace, need, dev):
    """The caller's workspace, or a new one: a contiguous GPU buffer of at
    least `need` bytes on `dev`.  Returns (tensor, bytes)."""
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _device_of(workspace, "workspace")
    if workspace.device != dev:
        raise ValueError(f"workspace must be on {dev}, got {workspace.device}")
    if not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    nbytes = workspace.numel() * workspace.element_size()
    if nbytes < need:
        raise ValueError(f"workspace too small: need {need} bytes, got {nbytes}")
    return workspace, nbytes


def _same_device(*ts):
    devs = {t.device for t in ts if t is not None}
    if len(devs) > 1:
        raise ValueError(f"all tensors must be on one device, got {sorted(map(str, devs))}")
    return devs.pop()


def logp_selected(logits, targets, mask=None, *, logp=None, lse=None):
    """Selected-token logprob from bf16 logits [N, V] (rows may be strided).

    Returns (logp, lse), both float32 [N]; inactive rows get 0.
    """
    lib = load_library()
    ld = _matrix(logits, "logits", torch.bfloat16)
    n, v = logits.shape
    _rows(targets, "targets", n, torch.int64)
    mask = _mask(mask, n)
    dev = _same_device(logits, targets, mask)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    _rows(logp, "logp", n, torch.float32)
    _rows(lse, "lse", n, torch.float32)
    if n == 0:
        return logp, lse
    with torch.cuda.device(dev):
        st = lib.rlk_logp_selected(_ptr(logits), ld, _ptr(targets), _ptr(mask), n, v, _ptr(logp),
                                   _ptr(lse), _stream(dev))
    _raise(st, "rlk_logp_selected")
    return logp, lse


def logp_entropy(logits, targets, mask=None, *, logp=None, lse=None, entropy=None):
    """Selected-token logprob plus per-row entropy from bf16 logits [N, V],
    one pass.  Returns (logp, lse, entropy), float32 [N]."""
    lib = load_library()
    ld = _matrix(logits, "logits", torch.bfloat16)
    n, v = logits.shape
    _rows(targets, "targets", n, torch.int64)
    mask = _mask(mask, n)
    dev = _same_device(logits, targets, mask)
    logp = torch.empty(n, dtype=torch.float32, device=dev) if logp is None else logp
    lse = torch.empty(n, dtype=torch.float32, device=dev) if lse is None else lse
    entropy = torch.empty(n, dtype=torch.float32, device=dev) if entropy is None else entropy
    for t, nm in ((logp, "logp"), (lse, "lse"), (entropy, "entropy")):
        _rows(t, nm, n, torch.float32)
    if n == 0:
        return logp, lse, entropy
    with torch.cuda.device(dev):
        st = lib.rlk_logp_entropy(_ptr(logits), ld, _ptr(targets), _ptr(mask), n, v, _ptr(logp),
                                  _ptr(lse), _ptr(entropy), _stream(dev))
    _raise(st, "rlk_logp_entropy")
    return logp, lse, entropy


def log_softmax(logits, lse, mask=None, *, out=None):
    """Dense log-softmax rows x - lse from bf16 logits [N, V] and the
    forward's lse: float32 [N, V]; inactive rows are zero."""
    lib = load_library()
    ld = _matrix(logits, "logits", torch.bfloat16)
    n, v = logits.shape
    _rows(lse, "lse", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(logits, lse, mask)
    out, ldo = _grad_out(out, n, v, dev)
    if n == 0:
        return out
    with torch.cuda.device(dev):
        st = lib.rlk_log_softmax(_ptr(logits), ld, _ptr(mask), _ptr(lse), n, v, _ptr(out), ldo,
                                 _stream(dev))
    _raise(st, "rlk_log_softmax")
    return out


def token_losses(logp, logp_old, advantages, mask=None, logp_ref=None, eps_lo=0.2, eps_hi=0.2,
                 beta=0.0):
    """Per-token GRPO/PPO terms from fp32 [N] logprobs: returns a dict of
    float32 [N] tensors ratio, loss, kl, grad (d loss / d logp)."""
    lib = load_library()
    n = logp.shape[0] if logp.dim() == 1 else -1
    for t, nm in ((logp, "logp"), (logp_old, "logp_old"), (advantages, "advantages")):
        _rows(t, nm, n, torch.float32)
    if logp_ref is not None:
        _rows(logp_ref, "logp_ref", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(logp, logp_old, advantages, logp_ref, mask)
    out = {k: torch.empty(n, dtype=torch.float32, device=dev) for k in ("ratio", "loss", "kl", "grad")}
    if n == 0:
        return out
    with torch.cuda.device(dev):
        st = lib.rlk_token_losses(_ptr(logp), _ptr(logp_old), _ptr(logp_ref), _ptr(advantages),
                                  _ptr(mask), n, float(eps_lo), float(eps_hi), float(beta),
                                  _ptr(out["ratio"]), _ptr(out["loss"]), _ptr(out["kl"]),
                                  _ptr(out["grad"]), _stream(dev))
    _raise(st, "rlk_token_losses")
    return out


def linear_logp_workspace_size(n, v, h):
    return int(load_library().rlk_linear_logp_workspace_size(n, v, h))


def linear_logp(hidden, weight, targets, mask=None, *, workspace=None, logp=None, lse=None):
    """Fused lm_head + selected logprob: hidden bf16 [N, H], weight bf16
    [V, H] (nn.Linear layout).  Returns (logp, lse), float32 [N]."""
    lib = load_library()
    ldh = _matrix(hidden, "hidden", torch.bfloat16)
    ldw = _matrix(weight, "weight", torch.bfloat16)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h != h2:
        raise ValueError(f"hidden has H={h} but weight has H={h2}")
    _rows(targets, "targets", n, torch.int64)
    mask = _mask(mask, n)
    dev = _same_device(hidden, weight, targets, mask)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    _rows(logp, "logp", n, torch.float32)
    _rows(lse, "lse", n, torch.float32)
    if n == 0:
        return logp, lse
    workspace, ws_bytes = _workspace(workspace, linear_logp_workspace_size(n, v, h), dev)
    with torch.cuda.device(dev):
        st = lib.rlk_linear_logp(_ptr(hidden), ldh, _ptr(weight), ldw, _ptr(targets), _ptr(mask), n,
                                 v, h, _ptr(logp), _ptr(lse), _ptr(workspace), ws_bytes,
                                 _stream(dev))
    _raise(st, "rlk_linear_logp")
    return logp, lse


def linear_logp_noalloc(hidden, weight, targets, mask=None, *, logp=None, lse=None):
    """linear_logp through rlk_linear_logp_noalloc: no workspace, the library's
    own 32 MiB per-GPU array holds the partials (for callers that cannot
    allocate; pass logp and lse to allocate nothing here either).  Calls that
    overlap in time on one GPU race on that array.  Returns (logp, lse)."""
    lib = load_library()
    ldh = _matrix(hidden, "hidden", torch.bfloat16)
    ldw = _matrix(weight, "weight", torch.bfloat16)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h != h2:
        raise ValueError(f"hidden has H={h} but weight has H={h2}")
    _rows(targets, "targets", n, torch.int64)
    mask = _mask(mask, n)
    dev = _same_device(hidden, weight, targets, mask)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    _rows(logp, "logp", n, torch.float32)
    _rows(lse, "lse", n, torch.float32)
    if n == 0:
        return logp, lse
    with torch.cuda.device(dev):
        st = lib.rlk_linear_logp_noalloc(_ptr(hidden), ldh, _ptr(weight), ldw, _ptr(targets),
                                         _ptr(mask), n, v, h, _ptr(logp), _ptr(lse), _stream(dev))
    _raise(st, "rlk_linear_logp_noalloc")
    return logp, lse


def linear_logp_with_logits(hidden, weight, targets, mask=None, *, workspace=None, logp=None,
                            lse=None, logits=None):
    """The fused forward that also keeps its fp32 logits z = hidden . weight^T
    (every row, masked or not), for a backward without the second
    projection: logp_backward(logits, ...).  Returns (logp, lse, logits);
    logp and lse are bit-identical to linear_logp's."""
    lib = load_library()
    ldh = _matrix(hidden, "hidden", torch.bfloat16)
    ldw = _matrix(weight, "weight", torch.bfloat16)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h != h2:
        raise ValueError(f"hidden has H={h} but weight has H={h2}")
    _rows(targets, "targets", n, torch.int64)
    mask = _mask(mask, n)
    dev = _same_device(hidden, weight, targets, mask)
    if logp is None:
        logp = torch.empty(n, dtype=torch.float32, device=dev)
    if lse is None:
        lse = torch.empty(n, dtype=torch.float32, device=dev)
    _rows(logp, "logp", n, torch.float32)
    _rows(lse, "lse", n, torch.float32)
    logits, ldz = _grad_out(logits, n, v, dev, "logits")
    if n == 0:
        return logp, lse, logits
    workspace, ws_bytes = _workspace(workspace, linear_logp_workspace_size(n, v, h), dev)
    with torch.cuda.device(dev):
        st = lib.rlk_linear_logp_with_logits(
            _ptr(hidden), ldh, _ptr(weight), ldw, _ptr(targets), _ptr(mask), n, v, h, _ptr(logp),
            _ptr(lse), _ptr(logits), ldz, _ptr(workspace), ws_bytes, _stream(dev))
    _raise(st, "rlk_linear_logp_with_logits")
    return logp, lse, logits


def _grad_out(out, n, v, dev, name="out"):
    if out is None:
        ldg = (v + 3) // 4 * 4
        buf = torch.empty((n, ldg), dtype=torch.float32, device=dev)
        return buf[:, :v], ldg
    ldg = _matrix(out, name, torch.float32, read=False)
    if tuple(out.shape) != (n, v):
        raise ValueError(f"{name} must have shape ({n}, {v})")
    return out, ldg


def logp_backward(logits, targets, lse, grad_logp, mask=None, *, out=None):
    """d(sum_i g_i logp_i)/d logits: float32 [N, V].  From bf16 logits [N, V],
    or from the fp32 logits linear_logp_with_logits keeps (then the result is
    bit-identical to linear_logp_backward's, and `out` may be `logits` itself
    to compute in place)."""
    lib = load_library()
    if isinstance(logits, torch.Tensor) and logits.dtype == torch.float32:
        return _logp_backward_f32(lib, logits, targets, lse, grad_logp, mask, out)
    ld = _matrix(logits, "logits", torch.bfloat16)
    n, v = logits.shape
    _rows(targets, "targets", n, torch.int64)
    _rows(lse, "lse", n, torch.float32)
    _rows(grad_logp, "grad_logp", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(logits, targets, lse, grad_logp, mask)
    out, ldg = _grad_out(out, n, v, dev)
    if n == 0:
        return out
    with torch.cuda.device(dev):
        st = lib.rlk_logp_backward(_ptr(logits), ld, None, 0, None, 0, 0, _ptr(targets), _ptr(mask),
                                   _ptr(lse), _ptr(grad_logp), n, v, _ptr(out), ldg, _stream(dev))
    _raise(st, "rlk_logp_backward")
    return out


def _logp_backward_f32(lib, logits, targets, lse, grad_logp, mask, out):
    ld = _matrix(logits, "logits", torch.float32)
    n, v = logits.shape
    _rows(targets, "targets", n, torch.int64)
    _rows(lse, "lse", n, torch.float32)
    _rows(grad_logp, "grad_logp", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(logits, targets, lse, grad_logp, mask)
    out, ldg = _grad_out(out, n, v, dev)
    if n == 0:
        return out
    with torch.cuda.device(dev):
        st = lib.rlk_logp_backward_f32(_ptr(logits), ld, _ptr(targets), _ptr(mask), _ptr(lse),
                                       _ptr(grad_logp), n, v, _ptr(out), ldg, _stream(dev))
    _raise(st, "rlk_logp_backward_f32")
    return out


def linear_logp_backward(hidden, weight, targets, lse, grad_logp, mask=None, *, out=None):
    """Gradient with respect to the logits z = hidden . weight^T, recomputed
    with the forward's tiles: float32 [N, V]."""
    lib = load_library()
    ldh = _matrix(hidden, "hidden", torch.bfloat16)
    ldw = _matrix(weight, "weight", torch.bfloat16)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h != h2:
        raise ValueError(f"hidden has H={h} but weight has H={h2}")
    _rows(targets, "targets", n, torch.int64)
    _rows(lse, "lse", n, torch.float32)
    _rows(grad_logp, "grad_logp", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(hidden, weight, targets, lse, grad_logp, mask)
    out, ldg = _grad_out(out, n, v, dev)
    if n == 0:
        return out
    with torch.cuda.device(dev):
        st = lib.rlk_logp_backward(None, 0, _ptr(hidden), ldh, _ptr(weight), ldw, h, _ptr(targets),
                                   _ptr(mask), _ptr(lse), _ptr(grad_logp), n, v, _ptr(out), ldg,
                                   _stream(dev))
    _raise(st, "rlk_logp_backward")
    return out


def linear_logp_param_grads_workspace_size(n, v, h):
    return int(load_library().rlk_linear_logp_param_grads_workspace_size(n, v, h))


def _param_out(out, rows, cols, dev, name):
    if out is None:
        return torch.empty((rows, cols), dtype=torch.float32, device=dev), cols
    ld = _matrix(out, name, torch.float32, read=False)
    if tuple(out.shape) != (rows, cols):
        raise ValueError(f"{name} must have shape ({rows}, {cols})")
    return out, ld


def linear_logp_param_grads(hidden, weight, targets, lse, grad_logp, mask=None, *,
                            want_hidden=True, want_weight=True, grad_hidden=None,
                            grad_weight=None, workspace=None, logits=None):
    """Gradients of sum_i g_i logp_i with respect to hidden [N, H] and weight
    [V, H] of the fused path: returns (grad_hidden, grad_weight), float32,
    each None when not requested.  `logits`: the fp32 [N, V] logits
    linear_logp_with_logits kept, used instead of recomputing them (the
    gradients are bit-identical)."""
    lib = load_library()
    if not (want_hidden or want_weight):
        raise ValueError("request at least one of grad_hidden / grad_weight")
    ldh = _matrix(hidden, "hidden", torch.bfloat16)
    ldw = _matrix(weight, "weight", torch.bfloat16)
    n, h = hidden.shape
    v, h2 = weight.shape
    if h != h2:
        raise ValueError(f"hidden has H={h} but weight has H={h2}")
    _rows(targets, "targets", n, torch.int64)
    _rows(lse, "lse", n, torch.float32)
    _rows(grad_logp, "grad_logp", n, torch.float32)
    mask = _mask(mask, n)
    dev = _same_device(hidden, weight, targets, lse, grad_logp, mask, logits)
    ldz = 0
    if logits is not None:
        ldz = _matrix(logits, "logits", torch.float32)
        if tuple(logits.shape) != (n, v):
            raise ValueError(f"logits must have shape ({n}, {v})")
    gh = gw = None
    ld_gh = ld_gw = 0
    if want_hidden:
        gh, ld_gh = _param_out(grad_hidden, n, h, dev, "grad_hidden")
    if want_weight:
        gw, ld_gw = _param_out(grad_weight, v, h, dev, "grad_weight")
    workspace, ws_bytes = _workspace(workspace, linear_logp_param_grads_workspace_size(n, v, h),
                                     dev)
    with torch.cuda.device(dev):
        if logits is None:
            st = lib.rlk_linear_logp_param_grads(
                _ptr(hidden), ldh, _ptr(weight), ldw, _ptr(targets), _ptr(mask), _ptr(lse),
                _ptr(grad_logp), n, v, h, _ptr(gh), ld_gh, _ptr(gw), ld_gw, _ptr(workspace),
                ws_bytes, _stream(dev))
            _raise(st, "rlk_linear_logp_param_grads")
        else:
            st = lib.rlk_linear_logp_param_grads_from_logits(
                _ptr(logits), ldz, _ptr(hidden), ldh, _ptr(weight), ldw, _ptr(targets),
                _ptr(mask), _ptr(lse), _ptr(grad_logp), n, v, h, _ptr(gh), ld_gh, _ptr(gw), ld_gw,
                _ptr(workspace), ws_bytes, _stream(dev))
            _raise(st, "rlk_linear_logp_param_grads_from_logits")
    return gh, gw


class SelectedLogprob(torch.autograd.Function):
    """Autograd wrapper: forward through rlk_logp_selected, backward through
    rlk_logp_backward with the saved lse."""

    @staticmethod
    def forward(ctx, logits, targets, mask=None):
        logp, lse = logp_selected(logits, targets, mask)
        ctx.save_for_backward(logits, targets, lse, mask if mask is not None else torch.empty(0))
        ctx.has_mask = mask is not None
        return logp

    @staticmethod
    def backward(ctx, grad):
        logits, targets, lse, mask = ctx.saved_tensors
        g = grad.contiguous().to(torch.float32)
        d = logp_backward(logits, targets, lse, g, mask if ctx.has_mask else None)
        return d, None, None


class LinearLogprob(torch.autograd.Function):
    """Autograd wrapper of the fused path: forward through rlk_linear_logp,
    backward through rlk_linear_logp_param_grads with the saved lse.  With
    keep_logits=True the forward keeps its fp32 logits (N x V x 4 bytes,
    held until backward) and the backward forms the gradients from them
    instead of recomputing them; the gradients are bit-identical.  The
    gradients are float32; autograd casts them to the inputs' dtype."""

    @staticmethod
    def forward(ctx, hidden, weight, targets, mask=None, keep_logits=False):
        if keep_logits:
            logp, lse, logits = linear_logp_with_logits(hidden, weight, targets, mask)
        else:
            logp, lse = linear_logp(hidden, weight, targets, mask)
            logits = torch.empty(0)
        ctx.save_for_backward(hidden, weight, targets, lse,
                              mask if mask is not None else torch.empty(0), logits)
        ctx.has_mask = mask is not None
        ctx.keep_logits = bool(keep_logits)
        return logp

    @staticmethod
    def backward(ctx, grad):
        hidden, weight, targets, lse, mask, logits = ctx.saved_tensors
        g = grad.contiguous().to(torch.float32)
        gh, gw = linear_logp_param_grads(hidden, weight, targets, lse, g,
                                         mask if ctx.has_mask else None,
                                         want_hidden=ctx.needs_input_grad[0],
                                         want_weight=ctx.needs_input_grad[1],
                                         logits=logits if ctx.keep_logits else None)
        return gh, gw, None, None, None
