"""Python binding of libitl.so: the invariant token-logprob library (MI355X).

Thin ctypes marshalling over the C ABI declared in include/itl.h: every
function checks tensor dtypes, devices and contiguity, allocates outputs and
workspace with torch (PyTorch supplies device memory and the current stream
only) and calls the library; every step of the computation runs in the
library's HIP kernels. There is no fallback: if libitl.so is missing, importing
this package fails.

Entry points (same names as the C ABI without the ``itl_`` prefix):

* ``lmhead_logprob(H, W, tokens) -> (logprob, lse)``
* ``group_advantage(rewards, group_offsets) -> advantages``
* ``reinforce_zero_loss(logprob, rollout_logprob, advantages, resp_offsets) -> (resp_loss, loss, coef)``
* ``reinforce_zero_backward(H, W, tokens, lse, coef) -> (dH, dW)``
* ``mismatch_stats(logprob, rollout_logprob, same_weights_logprob=None) -> stats``
* ``quantize_rows_fp8(X) -> (Xq, scale)``,
  ``lmhead_logprob_fp8(Hq, h_scale, Wq, w_scale, tokens) -> (logprob, lse)``
* ``quantize_rows_mxfp4(X) -> (Xq4, scale_codes)``,
  ``lmhead_logprob_mxfp4(Hq, h_scale, Wq4, w_scale_codes, tokens) -> (logprob, lse)``
* ``check_inputs(tokens, vocab, resp_offsets=None)``, ``build_info()``
"""

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libitl.so")

ITL_OK = 0
ITL_BF16 = 0
ITL_F32 = 1

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_i32 = ctypes.c_int32
_size = ctypes.c_size_t


class ItlError(RuntimeError):
    """A non-OK status from the library."""

    def __init__(self, status, message):
        super().__init__(message)
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run `python -m invariant_token_logprobs_lm_amd.build` "
            "(there is no fallback implementation)"
        )
    lib = ctypes.CDLL(LIB_PATH)
    sig = {
        "itl_lmhead_logprob_workspace_bytes": (_size, [_i64, _i64]),
        "itl_lmhead_logprob": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p,
                                              _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
        "itl_lmhead_logprob_noalloc": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64, _i64,
                                                      _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
        "itl_lmhead_logprob_keep_logits": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64, _i64,
                                                          _c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64,
                                                          _c_void_p, _size, _c_void_p]),
        "itl_group_advantage": (ctypes.c_int, [_c_void_p, _c_void_p, _i32, _i32, _c_void_p, _c_void_p]),
        "itl_reinforce_zero_loss_workspace_bytes": (_size, [_i64, _i32]),
        "itl_reinforce_zero_loss": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i32, _i64,
                                                   _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
        "itl_reinforce_zero_backward_workspace_bytes": (_size, [_i64, _i64, _i64, ctypes.c_int]),
        "itl_reinforce_zero_backward": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64, _i64,
                                                       _c_void_p, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                       _c_void_p, _size, _c_void_p]),
        "itl_reinforce_zero_backward_from_logits": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64,
                                                                   _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p,
                                                                   _i64, _c_void_p, _c_void_p, _c_void_p, _size,
                                                                   _c_void_p]),
        "itl_quantize_rows_fp8": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _c_void_p, _c_void_p,
                                                 _c_void_p]),
        "itl_lmhead_logprob_fp8": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64,
                                                  _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
        "itl_quantize_rows_mxfp4": (ctypes.c_int, [_c_void_p, ctypes.c_int, _i64, _i64, _c_void_p, _c_void_p,
                                                   _c_void_p]),
        "itl_lmhead_logprob_mxfp4": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _c_void_p, _i64, _i64, _i64,
                                                    _c_void_p, _c_void_p, _c_void_p, _c_void_p, _size, _c_void_p]),
        "itl_mismatch_stats_workspace_bytes": (_size, [_i64]),
        "itl_mismatch_stats": (ctypes.c_int, [_c_void_p, _c_void_p, _c_void_p, _i64, _c_void_p, _c_void_p, _size,
                                              _c_void_p]),
        "itl_check_inputs": (ctypes.c_int, [_c_void_p, _i64, _i64, _c_void_p, _i32, _c_void_p]),
        "itl_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "itl_last_error": (ctypes.c_char_p, []),
        "itl_build_info": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()

EXPORTS = (
    "itl_lmhead_logprob_workspace_bytes",
    "itl_lmhead_logprob",
    "itl_lmhead_logprob_noalloc",
    "itl_lmhead_logprob_keep_logits",
    "itl_group_advantage",
    "itl_reinforce_zero_loss_workspace_bytes",
    "itl_reinforce_zero_loss",
    "itl_reinforce_zero_backward_workspace_bytes",
    "itl_reinforce_zero_backward",
    "itl_reinforce_zero_backward_from_logits",
    "itl_quantize_rows_fp8",
    "itl_lmhead_logprob_fp8",
    "itl_quantize_rows_mxfp4",
    "itl_lmhead_logprob_mxfp4",
    "itl_mismatch_stats_workspace_bytes",
    "itl_mismatch_stats",
    "itl_check_inputs",
    "itl_status_string",
    "itl_last_error",
    "itl_build_info",
)


def build_info():
    return lib.itl_build_info().decode()


def _check(status):
    if status != ITL_OK:
        msg = lib.itl_status_string(status).decode()
        detail = lib.itl_last_error().decode()
        raise ItlError(status, f"{msg}: {detail}" if detail else msg)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _need(t, name, dtypes, device=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} has dtype {t.dtype}; expected one of {dtypes}")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a HIP device, got {t.device}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


_HEAD_DTYPES = {torch.bfloat16: ITL_BF16, torch.float32: ITL_F32}


def lmhead_workspace_bytes(n_tok, vocab):
    return int(lib.itl_lmhead_logprob_workspace_bytes(n_tok, vocab))


def lmhead_logprob(H, W, tokens, *, logprob=None, lse=None, workspace=None, want_lse=True):
    """Sampled-token logprob and log-normaliser of every row of H.

    H [n_tok, d] and W [vocab, d] (bf16 or fp32, same dtype), tokens int32
    [n_tok]. Returns (logprob fp32 [n_tok], lse fp32 [n_tok] or None).
    """
    _need(H, "H", tuple(_HEAD_DTYPES), ndim=2)
    _need(W, "W", (H.dtype,), device=H.device, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=H.device, ndim=1)
    n_tok, d = H.shape
    vocab = W.shape[0]
    if W.shape[1] != d or tokens.shape[0] != n_tok:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)}, W {tuple(W.shape)}, tokens {tuple(tokens.shape)}")
    if logprob is None:
        logprob = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    if lse is None and want_lse:
        lse = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    for name, t in (("logprob", logprob), ("lse", lse)):
        if t is not None:
            _need(t, name, (torch.float32,), device=H.device, ndim=1)
            if t.shape[0] != n_tok:
                raise ValueError(f"{name} must have {n_tok} elements")
    need = lmhead_workspace_bytes(n_tok, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    _need(workspace, "workspace", (torch.uint8,), device=H.device)
    _check(lib.itl_lmhead_logprob(_ptr(H), _ptr(W), _HEAD_DTYPES[H.dtype], n_tok, d, vocab, _ptr(tokens),
                                  _ptr(logprob), _ptr(lse), _ptr(workspace), workspace.numel(),
                                  _stream(H.device)))
    return logprob, lse


def lmhead_logprob_noalloc(H, W, tokens, *, logprob=None, lse=None, want_lse=True):
    """lmhead_logprob without a workspace (the library's static per-GPU
    scratch; at most 16,368 tokens for large vocabularies). Same bits."""
    _need(H, "H", tuple(_HEAD_DTYPES), ndim=2)
    _need(W, "W", (H.dtype,), device=H.device, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=H.device, ndim=1)
    n_tok, d = H.shape
    vocab = W.shape[0]
    if W.shape[1] != d or tokens.shape[0] != n_tok:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)}, W {tuple(W.shape)}, tokens {tuple(tokens.shape)}")
    if logprob is None:
        logprob = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    if lse is None and want_lse:
        lse = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    for name, t in (("logprob", logprob), ("lse", lse)):
        if t is not None:
            _need(t, name, (torch.float32,), device=H.device, ndim=1)
            if t.shape[0] != n_tok:
                raise ValueError(f"{name} must have {n_tok} elements")
    _check(lib.itl_lmhead_logprob_noalloc(_ptr(H), _ptr(W), _HEAD_DTYPES[H.dtype], n_tok, d, vocab, _ptr(tokens),
                                          _ptr(logprob), _ptr(lse), _stream(H.device)))
    return logprob, lse


def lmhead_logprob_keep_logits(H, W, tokens, *, logits=None, logprob=None, lse=None, workspace=None):
    """lmhead_logprob (same bits) that also returns the logits z [n_tok, ld]
    fp32 (ld = vocab rounded up to a multiple of 4 when allocated here; a
    caller's buffer may have any ld >= vocab that is a multiple of 4).
    Returns (logprob, lse, logits)."""
    _need(H, "H", tuple(_HEAD_DTYPES), ndim=2)
    _need(W, "W", (H.dtype,), device=H.device, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=H.device, ndim=1)
    n_tok, d = H.shape
    vocab = W.shape[0]
    if W.shape[1] != d or tokens.shape[0] != n_tok:
        raise ValueError(f"shape mismatch: H {tuple(H.shape)}, W {tuple(W.shape)}, tokens {tuple(tokens.shape)}")
    if logits is None:
        logits = torch.empty((n_tok, (vocab + 3) // 4 * 4), dtype=torch.float32, device=H.device)
    _need(logits, "logits", (torch.float32,), device=H.device, ndim=2)
    if logits.shape[0] != n_tok:
        raise ValueError(f"logits must have {n_tok} rows")
    if logprob is None:
        logprob = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    if lse is None:
        lse = torch.empty(n_tok, dtype=torch.float32, device=H.device)
    for name, t in (("logprob", logprob), ("lse", lse)):
        _need(t, name, (torch.float32,), device=H.device, ndim=1)
        if t.shape[0] != n_tok:
            raise ValueError(f"{name} must have {n_tok} elements")
    need = lmhead_workspace_bytes(n_tok, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=H.device)
    _need(workspace, "workspace", (torch.uint8,), device=H.device)
    _check(lib.itl_lmhead_logprob_keep_logits(_ptr(H), _ptr(W), _HEAD_DTYPES[H.dtype], n_tok, d, vocab, _ptr(tokens),
                                              _ptr(logprob), _ptr(lse), _ptr(logits), logits.shape[1],
                                              _ptr(workspace), workspace.numel(), _stream(H.device)))
    return logprob, lse, logits


def group_advantage(rewards, group_offsets, *, advantages=None):
    """advantages[i] = rewards[i] - mean reward of i's group (fp32)."""
    _need(rewards, "rewards", (torch.float32,), ndim=1)
    _need(group_offsets, "group_offsets", (torch.int32,), device=rewards.device, ndim=1)
    n_resp = rewards.shape[0]
    n_groups = group_offsets.shape[0] - 1
    if n_groups < 0:
        raise ValueError("group_offsets needs at least one element")
    if advantages is None:
        advantages = torch.empty_like(rewards)
    _need(advantages, "advantages", (torch.float32,), device=rewards.device, ndim=1)
    _check(lib.itl_group_advantage(_ptr(rewards), _ptr(group_offsets), n_groups, n_resp, _ptr(advantages),
                                   _stream(rewards.device)))
    return advantages


def loss_workspace_bytes(n_tok, n_resp):
    return int(lib.itl_reinforce_zero_loss_workspace_bytes(n_tok, n_resp))


def reinforce_zero_loss(logprob, rollout_logprob, advantages, resp_offsets, *, want_coef=True, workspace=None):
    """(resp_loss fp32 [N], loss fp32 [1], coef fp32 [n_tok] or None)."""
    _need(logprob, "logprob", (torch.float32,), ndim=1)
    dev = logprob.device
    _need(rollout_logprob, "rollout_logprob", (torch.float32,), device=dev, ndim=1)
    _need(advantages, "advantages", (torch.float32,), device=dev, ndim=1)
    _need(resp_offsets, "resp_offsets", (torch.int64,), device=dev, ndim=1)
    n_tok = logprob.shape[0]
    n_resp = advantages.shape[0]
    if rollout_logprob.shape[0] != n_tok or resp_offsets.shape[0] != n_resp + 1:
        raise ValueError("shape mismatch between logprobs, advantages and resp_offsets")
    resp_loss = torch.empty(n_resp, dtype=torch.float32, device=dev)
    loss = torch.empty(1, dtype=torch.float32, device=dev)
    coef = torch.empty(n_tok, dtype=torch.float32, device=dev) if want_coef else None
    need = loss_workspace_bytes(n_tok, n_resp)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_reinforce_zero_loss(_ptr(logprob), _ptr(rollout_logprob), _ptr(advantages), _ptr(resp_offsets),
                                       n_resp, n_tok, _ptr(resp_loss), _ptr(loss), _ptr(coef), _ptr(workspace),
                                       workspace.numel(), _stream(dev)))
    return resp_loss, loss, coef


def backward_workspace_bytes(n_tok, d, vocab, dtype=torch.bfloat16):
    return int(lib.itl_reinforce_zero_backward_workspace_bytes(n_tok, d, vocab, _HEAD_DTYPES[dtype]))


def reinforce_zero_backward(H, W, tokens, lse, coef, *, dH=None, dW=None, workspace=None):
    """(dH fp32 [n_tok, d], dW fp32 [vocab, d]) of the REINFORCE Zero loss."""
    _need(H, "H", tuple(_HEAD_DTYPES), ndim=2)
    dev = H.device
    _need(W, "W", (H.dtype,), device=dev, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=dev, ndim=1)
    _need(lse, "lse", (torch.float32,), device=dev, ndim=1)
    _need(coef, "coef", (torch.float32,), device=dev, ndim=1)
    n_tok, d = H.shape
    vocab = W.shape[0]
    if W.shape[1] != d or tokens.shape[0] != n_tok or lse.shape[0] != n_tok or coef.shape[0] != n_tok:
        raise ValueError("shape mismatch between H, W, tokens, lse and coef")
    if dH is None:
        dH = torch.empty((n_tok, d), dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty((vocab, d), dtype=torch.float32, device=dev)
    _need(dH, "dH", (torch.float32,), device=dev, ndim=2)
    _need(dW, "dW", (torch.float32,), device=dev, ndim=2)
    need = backward_workspace_bytes(n_tok, d, vocab, H.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_reinforce_zero_backward(_ptr(H), _ptr(W), _HEAD_DTYPES[H.dtype], n_tok, d, vocab, _ptr(tokens),
                                           _ptr(lse), _ptr(coef), _ptr(dH), _ptr(dW), _ptr(workspace),
                                           workspace.numel(), _stream(dev)))
    return dH, dW


def reinforce_zero_backward_from_logits(H, W, tokens, lse, coef, logits, *, dH=None, dW=None, workspace=None):
    """reinforce_zero_backward (same bits) with the dlogits formed from the
    logits kept by lmhead_logprob_keep_logits ([n_tok, ld] fp32)."""
    _need(H, "H", tuple(_HEAD_DTYPES), ndim=2)
    dev = H.device
    _need(W, "W", (H.dtype,), device=dev, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=dev, ndim=1)
    _need(lse, "lse", (torch.float32,), device=dev, ndim=1)
    _need(coef, "coef", (torch.float32,), device=dev, ndim=1)
    _need(logits, "logits", (torch.float32,), device=dev, ndim=2)
    n_tok, d = H.shape
    vocab = W.shape[0]
    if (W.shape[1] != d or tokens.shape[0] != n_tok or lse.shape[0] != n_tok or coef.shape[0] != n_tok
            or logits.shape[0] != n_tok):
        raise ValueError("shape mismatch between H, W, tokens, lse, coef and logits")
    if dH is None:
        dH = torch.empty((n_tok, d), dtype=torch.float32, device=dev)
    if dW is None:
        dW = torch.empty((vocab, d), dtype=torch.float32, device=dev)
    _need(dH, "dH", (torch.float32,), device=dev, ndim=2)
    _need(dW, "dW", (torch.float32,), device=dev, ndim=2)
    need = backward_workspace_bytes(n_tok, d, vocab, H.dtype)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_reinforce_zero_backward_from_logits(_ptr(H), _ptr(W), _HEAD_DTYPES[H.dtype], n_tok, d, vocab,
                                                       _ptr(tokens), _ptr(lse), _ptr(coef), _ptr(logits),
                                                       logits.shape[1], _ptr(dH), _ptr(dW), _ptr(workspace),
                                                       workspace.numel(), _stream(dev)))
    return dH, dW


def quantize_rows_fp8(X, *, Xq=None, scale=None):
    """Per-row E4M3 codes (uint8 [n, d]) and fp32 scales [n] of a bf16 or
    fp32 matrix [n, d] (d a multiple of 128)."""
    _need(X, "X", tuple(_HEAD_DTYPES), ndim=2)
    n, d = X.shape
    if Xq is None:
        Xq = torch.empty((n, d), dtype=torch.uint8, device=X.device)
    if scale is None:
        scale = torch.empty(n, dtype=torch.float32, device=X.device)
    _need(Xq, "Xq", (torch.uint8,), device=X.device, ndim=2)
    _need(scale, "scale", (torch.float32,), device=X.device, ndim=1)
    if tuple(Xq.shape) != (n, d) or scale.shape[0] != n:
        raise ValueError("Xq must be [n, d] and scale [n]")
    _check(lib.itl_quantize_rows_fp8(_ptr(X), _HEAD_DTYPES[X.dtype], n, d, _ptr(Xq), _ptr(scale), _stream(X.device)))
    return Xq, scale


def lmhead_logprob_fp8(Hq, h_scale, Wq, w_scale, tokens, *, logprob=None, lse=None, workspace=None, want_lse=True):
    """Sampled-token logprob and lse from an E4M3 head with per-row scales
    (as written by quantize_rows_fp8)."""
    _need(Hq, "Hq", (torch.uint8,), ndim=2)
    dev = Hq.device
    _need(h_scale, "h_scale", (torch.float32,), device=dev, ndim=1)
    _need(Wq, "Wq", (torch.uint8,), device=dev, ndim=2)
    _need(w_scale, "w_scale", (torch.float32,), device=dev, ndim=1)
    _need(tokens, "tokens", (torch.int32,), device=dev, ndim=1)
    n_tok, d = Hq.shape
    vocab = Wq.shape[0]
    if Wq.shape[1] != d or h_scale.shape[0] != n_tok or w_scale.shape[0] != vocab or tokens.shape[0] != n_tok:
        raise ValueError("shape mismatch between Hq, h_scale, Wq, w_scale and tokens")
    if logprob is None:
        logprob = torch.empty(n_tok, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(n_tok, dtype=torch.float32, device=dev)
    need = lmhead_workspace_bytes(n_tok, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_lmhead_logprob_fp8(_ptr(Hq), _ptr(h_scale), _ptr(Wq), _ptr(w_scale), n_tok, d, vocab,
                                      _ptr(tokens), _ptr(logprob), _ptr(lse), _ptr(workspace), workspace.numel(),
                                      _stream(dev)))
    return logprob, lse


def quantize_rows_mxfp4(X, *, Xq=None, scale_codes=None):
    """MXFP4 of a bf16 or fp32 matrix [n, d] (d a multiple of 128): packed
    E2M1 codes uint8 [n, d / 2] and E8M0 scale codes uint8 [n, d / 32]."""
    _need(X, "X", tuple(_HEAD_DTYPES), ndim=2)
    n, d = X.shape
    if Xq is None:
        Xq = torch.empty((n, d // 2), dtype=torch.uint8, device=X.device)
    if scale_codes is None:
        scale_codes = torch.empty((n, d // 32), dtype=torch.uint8, device=X.device)
    _need(Xq, "Xq", (torch.uint8,), device=X.device, ndim=2)
    _need(scale_codes, "scale_codes", (torch.uint8,), device=X.device, ndim=2)
    if tuple(Xq.shape) != (n, d // 2) or tuple(scale_codes.shape) != (n, d // 32):
        raise ValueError("Xq must be [n, d/2] and scale_codes [n, d/32]")
    _check(lib.itl_quantize_rows_mxfp4(_ptr(X), _HEAD_DTYPES[X.dtype], n, d, _ptr(Xq), _ptr(scale_codes),
                                       _stream(X.device)))
    return Xq, scale_codes


def lmhead_logprob_mxfp4(Hq, h_scale, Wq4, w_scale_codes, tokens, *, logprob=None, lse=None, workspace=None,
                         want_lse=True):
    """Sampled-token logprob and lse from an MXFP4 head against E4M3 token
    rows (quantize_rows_mxfp4 / quantize_rows_fp8)."""
    _need(Hq, "Hq", (torch.uint8,), ndim=2)
    dev = Hq.device
    _need(h_scale, "h_scale", (torch.float32,), device=dev, ndim=1)
    _need(Wq4, "Wq4", (torch.uint8,), device=dev, ndim=2)
    _need(w_scale_codes, "w_scale_codes", (torch.uint8,), device=dev, ndim=2)
    _need(tokens, "tokens", (torch.int32,), device=dev, ndim=1)
    n_tok, d = Hq.shape
    vocab = Wq4.shape[0]
    if (Wq4.shape[1] * 2 != d or tuple(w_scale_codes.shape) != (vocab, d // 32) or h_scale.shape[0] != n_tok
            or tokens.shape[0] != n_tok):
        raise ValueError("shape mismatch between Hq, h_scale, Wq4, w_scale_codes and tokens")
    if logprob is None:
        logprob = torch.empty(n_tok, dtype=torch.float32, device=dev)
    if lse is None and want_lse:
        lse = torch.empty(n_tok, dtype=torch.float32, device=dev)
    need = lmhead_workspace_bytes(n_tok, vocab)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_lmhead_logprob_mxfp4(_ptr(Hq), _ptr(h_scale), _ptr(Wq4), _ptr(w_scale_codes), n_tok, d, vocab,
                                        _ptr(tokens), _ptr(logprob), _ptr(lse), _ptr(workspace), workspace.numel(),
                                        _stream(dev)))
    return logprob, lse


# Field order of itl_mismatch_stats' output (the itl_stat enum of include/itl.h).
STAT_FIELDS = (
    "n_tok",
    "kl_k1",
    "kl_k2",
    "kl_k3",
    "weight_mean",
    "weight_max",
    "weight_min",
    "deviation_max",
    "deviation_median",
    "deviation_peak_over_median",
    "lag_abs_mean",
    "lag_abs_max",
    "lag_kl_k3",
    "kernel_abs_mean",
    "kernel_abs_max",
    "kernel_kl_k3",
    "kernel_nonzero",
)


def mismatch_stats_workspace_bytes(n_tok):
    return int(lib.itl_mismatch_stats_workspace_bytes(n_tok))


def mismatch_stats(logprob, rollout_logprob, same_weights_logprob=None, *, stats=None, workspace=None):
    """Mismatch diagnostics of one batch: fp64 device tensor [len(STAT_FIELDS)]
    in STAT_FIELDS order (use ``stats_dict`` to read it on the host)."""
    _need(logprob, "logprob", (torch.float32,), ndim=1)
    dev = logprob.device
    _need(rollout_logprob, "rollout_logprob", (torch.float32,), device=dev, ndim=1)
    n_tok = logprob.shape[0]
    if rollout_logprob.shape[0] != n_tok:
        raise ValueError("logprob and rollout_logprob differ in length")
    if same_weights_logprob is not None:
        _need(same_weights_logprob, "same_weights_logprob", (torch.float32,), device=dev, ndim=1)
        if same_weights_logprob.shape[0] != n_tok:
            raise ValueError("same_weights_logprob differs in length")
    if stats is None:
        stats = torch.empty(len(STAT_FIELDS), dtype=torch.float64, device=dev)
    _need(stats, "stats", (torch.float64,), device=dev, ndim=1)
    if stats.shape[0] < len(STAT_FIELDS):
        raise ValueError(f"stats needs {len(STAT_FIELDS)} elements")
    need = mismatch_stats_workspace_bytes(n_tok)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", (torch.uint8,), device=dev)
    _check(lib.itl_mismatch_stats(_ptr(logprob), _ptr(rollout_logprob), _ptr(same_weights_logprob), n_tok,
                                  _ptr(stats), _ptr(workspace), workspace.numel(), _stream(dev)))
    return stats


def stats_dict(stats):
    """Host dict of a mismatch_stats result (synchronises on the copy)."""
    vals = stats.cpu().tolist()
    return {k: vals[i] for i, k in enumerate(STAT_FIELDS)}


def check_inputs(tokens, vocab, resp_offsets=None):
    """Validate device-resident token ids and offsets (synchronises)."""
    _need(tokens, "tokens", (torch.int32,), ndim=1)
    n_resp = 0
    if resp_offsets is not None:
        _need(resp_offsets, "resp_offsets", (torch.int64,), device=tokens.device, ndim=1)
        n_resp = resp_offsets.shape[0] - 1
    _check(lib.itl_check_inputs(_ptr(tokens), tokens.shape[0], vocab, _ptr(resp_offsets), n_resp,
                                _stream(tokens.device)))
