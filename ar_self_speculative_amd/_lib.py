"""ctypes binding of libtidar (include/tidar.h).

Argument marshalling only: every step of the hot path runs in the HIP
library. Tensors are torch tensors on the GPU; the binding checks dtype,
device and contiguity, passes raw pointers and the current HIP stream, and
raises on a non-zero status. There is no fallback: if the library is missing
the import fails.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtidar.so")

TIDAR_OK = 0
TIDAR_E_INVALID = -1
TIDAR_E_UNSUPPORTED = -2
TIDAR_E_WORKSPACE = -3
TIDAR_E_CAPACITY = -4
TIDAR_E_HIP = -5
DTYPE_F32 = 0
DTYPE_BF16 = 1

DEV_CACHE_LEN_RANGE = 1
DEV_ACCEPT_RANGE = 2
DEV_CAPACITY = 4
DEV_NONFINITE_ROW = 8
DEV_DRAFT_RANGE = 16
DEV_TARGET_RANGE = 32

EXPORTS = (
    "tidar_status_string", "tidar_last_error", "tidar_version",
    "tidar_attn_workspace_bytes", "tidar_attn_step", "tidar_kv_commit",
    "tidar_reject_workspace_bytes", "tidar_reject_sample", "tidar_reject_sample_trust",
    "tidar_reject_sample_noalloc", "tidar_reject_noalloc_max_bytes",
    "tidar_logprob_workspace_bytes", "tidar_token_logprobs",
    # measurement kernels (include/tidar_ceilings.h)
    "tidar_ceiling_hbm_read", "tidar_ceiling_mfma_bf16", "tidar_ceiling_exp_f32", "tidar_ceiling_fma_f32",
    "tidar_ceiling_lds_read_b128", "tidar_ceiling_lds_read_tr16", "tidar_ceiling_empty", "tidar_attn_stamps",
)


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("k", ctypes.c_int32), ("num_blocks", ctypes.c_int32), ("block_len", ctypes.c_int32),
        ("cache_capacity", ctypes.c_int32), ("max_cache_len", ctypes.c_int32),
        ("sm_scale", ctypes.c_float), ("dtype", ctypes.c_int32), ("num_splits", ctypes.c_int32),
    ]


class TidarError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


def load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python ar_self_speculative_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    lib.tidar_status_string.restype = ctypes.c_char_p
    lib.tidar_status_string.argtypes = [ctypes.c_int]
    lib.tidar_last_error.restype = ctypes.c_char_p
    lib.tidar_last_error.argtypes = []
    lib.tidar_version.restype = ctypes.c_int
    lib.tidar_attn_workspace_bytes.restype = sz
    lib.tidar_attn_workspace_bytes.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.tidar_attn_step.restype = ctypes.c_int
    lib.tidar_attn_step.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tidar_kv_commit.restype = ctypes.c_int
    lib.tidar_kv_commit.argtypes = [i32] * 9 + [vp] * 8 + [vp]
    lib.tidar_reject_workspace_bytes.restype = sz
    lib.tidar_reject_workspace_bytes.argtypes = [i32, i32, i32]
    lib.tidar_reject_sample.restype = ctypes.c_int
    lib.tidar_reject_sample.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, sz, vp]
    lib.tidar_logprob_workspace_bytes.restype = sz
    lib.tidar_logprob_workspace_bytes.argtypes = [i32, i32]
    lib.tidar_token_logprobs.restype = ctypes.c_int
    lib.tidar_token_logprobs.argtypes = [i32, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.tidar_reject_sample_trust.restype = ctypes.c_int
    lib.tidar_reject_sample_trust.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                              vp, vp, vp, vp, vp, sz, vp]
    lib.tidar_reject_sample_noalloc.restype = ctypes.c_int
    lib.tidar_reject_sample_noalloc.argtypes = [i32, i32, i32, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                                vp, vp, vp, vp, vp]
    lib.tidar_reject_noalloc_max_bytes.restype = sz
    lib.tidar_reject_noalloc_max_bytes.argtypes = []
    lib.tidar_ceiling_hbm_read.restype = ctypes.c_int
    lib.tidar_ceiling_hbm_read.argtypes = [vp, sz, ctypes.c_int, vp, vp]
    for name in ("tidar_ceiling_mfma_bf16", "tidar_ceiling_exp_f32", "tidar_ceiling_fma_f32",
                 "tidar_ceiling_lds_read_b128", "tidar_ceiling_lds_read_tr16"):
        getattr(lib, name).restype = ctypes.c_int
        getattr(lib, name).argtypes = [ctypes.c_int, ctypes.c_int, vp, vp]
    lib.tidar_ceiling_empty.restype = ctypes.c_int
    lib.tidar_ceiling_empty.argtypes = [ctypes.c_int, vp]
    lib.tidar_attn_stamps.restype = ctypes.c_int
    lib.tidar_attn_stamps.argtypes = [vp, ctypes.c_int]
    return lib


_lib = load()


def _status_name(s: int) -> str:
    return _lib.tidar_status_string(s).decode()


def last_error() -> str:
    return _lib.tidar_last_error().decode()


def _check(status: int):
    if status != TIDAR_OK:
        raise TidarError(status, last_error())


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _dev(t, dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


_TORCH_DT = {DTYPE_F32: torch.float32, DTYPE_BF16: torch.bfloat16}


def make_attn_desc(*, batch, num_q_heads, num_kv_heads, head_dim, k, num_blocks, block_len,
                   cache_capacity, max_cache_len, sm_scale, dtype, num_splits=0) -> AttnDesc:
    return AttnDesc(batch, num_q_heads, num_kv_heads, head_dim, k, num_blocks, block_len,
                    cache_capacity, max_cache_len, float(sm_scale), dtype, num_splits)


def attn_workspace_bytes(desc: AttnDesc) -> int:
    return int(_lib.tidar_attn_workspace_bytes(ctypes.byref(desc)))


def attn_workspace(desc: AttnDesc, device="cuda"):
    """A workspace tensor for ``desc`` (None when none is needed)."""
    n = attn_workspace_bytes(desc)
    if n == 0:
        return None
    return torch.zeros(n, dtype=torch.uint8, device=device)


def attn_step(desc: AttnDesc, q, k_step, v_step, k_cache, v_cache, cache_len, out, lse=None,
              dev_status=None, workspace=None, stream=None):
    """tidar_attn_step on torch tensors (shapes and layouts as in include/tidar.h)."""
    dt = _TORCH_DT.get(desc.dtype)
    for name, t in (("q", q), ("k_step", k_step), ("v_step", v_step), ("k_cache", k_cache),
                    ("v_cache", v_cache), ("out", out)):
        _dev(t, dt, name)
    _dev(cache_len, torch.int32, "cache_len")
    _dev(lse, torch.float32, "lse", allow_none=True)
    _dev(dev_status, torch.int32, "dev_status", allow_none=True)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(_lib.tidar_attn_step(ctypes.byref(desc), _ptr(q), _ptr(k_step), _ptr(v_step), _ptr(k_cache),
                                _ptr(v_cache), _ptr(cache_len), _ptr(out), _ptr(lse), _ptr(dev_status),
                                _ptr(workspace), ws_bytes, _stream(stream)))


def kv_commit(*, num_layers, batch, num_kv_heads, head_dim, k, step_rows, cache_capacity,
              max_cache_len, dtype, k_step, v_step, k_cache, v_cache, accept_len, cache_len_in,
              cache_len_out, dev_status=None, stream=None):
    dt = _TORCH_DT.get(dtype)
    for name, t in (("k_step", k_step), ("v_step", v_step), ("k_cache", k_cache), ("v_cache", v_cache)):
        _dev(t, dt, name)
    for name, t in (("accept_len", accept_len), ("cache_len_in", cache_len_in),
                    ("cache_len_out", cache_len_out)):
        _dev(t, torch.int32, name)
    _dev(dev_status, torch.int32, "dev_status", allow_none=True)
    _check(_lib.tidar_kv_commit(num_layers, batch, num_kv_heads, head_dim, k, step_rows,
                                cache_capacity, max_cache_len, dtype, _ptr(k_step), _ptr(v_step),
                                _ptr(k_cache), _ptr(v_cache), _ptr(accept_len), _ptr(cache_len_in),
                                _ptr(cache_len_out), _ptr(dev_status), _stream(stream)))


def reject_workspace_bytes(batch: int, k: int, vocab: int) -> int:
    return int(_lib.tidar_reject_workspace_bytes(batch, k, vocab))


def reject_sample(*, ar_logits, diff_logits, drafts, uniforms, accept_len, next_token, ratio=None,
                  dev_status=None, workspace, temperature: float = 1.0, trust_ar: float = 1.0, stream=None):
    B, kp1, V = ar_logits.shape
    k = kp1 - 1
    _dev(ar_logits, torch.float32, "ar_logits")
    _dev(diff_logits, torch.float32, "diff_logits", allow_none=(k == 0))
    _dev(drafts, torch.int32, "drafts", allow_none=(k == 0))
    _dev(uniforms, torch.float32, "uniforms")
    _dev(accept_len, torch.int32, "accept_len")
    _dev(next_token, torch.int32, "next_token")
    _dev(ratio, torch.float32, "ratio", allow_none=True)
    _dev(dev_status, torch.int32, "dev_status", allow_none=True)
    _dev(workspace, None, "workspace")
    args = (_ptr(accept_len), _ptr(next_token), _ptr(ratio), _ptr(dev_status), _ptr(workspace),
            workspace.numel() * workspace.element_size(), _stream(stream))
    if trust_ar == 1.0:
        _check(_lib.tidar_reject_sample(B, k, V, _ptr(ar_logits), _ptr(diff_logits), _ptr(drafts),
                                        _ptr(uniforms), float(temperature), *args))
    else:
        _check(_lib.tidar_reject_sample_trust(B, k, V, _ptr(ar_logits), _ptr(diff_logits), _ptr(drafts),
                                              _ptr(uniforms), float(temperature), float(trust_ar), *args))


def reject_sample_noalloc(*, ar_logits, diff_logits, drafts, uniforms, accept_len, next_token, ratio=None,
                          dev_status=None, temperature: float = 1.0, trust_ar: float = 1.0, stream=None):
    """tidar_reject_sample_noalloc: the sampler on the library's static scratch (no workspace)."""
    B, kp1, V = ar_logits.shape
    k = kp1 - 1
    _dev(ar_logits, torch.float32, "ar_logits")
    _dev(diff_logits, torch.float32, "diff_logits", allow_none=(k == 0))
    _dev(drafts, torch.int32, "drafts", allow_none=(k == 0))
    _dev(uniforms, torch.float32, "uniforms")
    _dev(accept_len, torch.int32, "accept_len")
    _dev(next_token, torch.int32, "next_token")
    _dev(ratio, torch.float32, "ratio", allow_none=True)
    _dev(dev_status, torch.int32, "dev_status", allow_none=True)
    _check(_lib.tidar_reject_sample_noalloc(B, k, V, _ptr(ar_logits), _ptr(diff_logits), _ptr(drafts),
                                            _ptr(uniforms), float(temperature), float(trust_ar), _ptr(accept_len),
                                            _ptr(next_token), _ptr(ratio), _ptr(dev_status), _stream(stream)))


def logprob_workspace_bytes(rows: int, vocab: int) -> int:
    return int(_lib.tidar_logprob_workspace_bytes(rows, vocab))


def token_logprobs(*, logits, targets, logprobs, workspace, dev_status=None, stream=None):
    """Likelihood mode: logprobs[..] = log softmax(logits[.., :])[targets[..]] (one launch pair)."""
    V = logits.shape[-1]
    rows = targets.numel()
    _dev(logits, torch.float32, "logits")
    _dev(targets, torch.int32, "targets")
    _dev(logprobs, torch.float32, "logprobs")
    _dev(dev_status, torch.int32, "dev_status", allow_none=True)
    _dev(workspace, None, "workspace")
    if logits.numel() != rows * V or logprobs.numel() != rows:
        raise ValueError("logits must hold targets.numel() rows of V logits, logprobs one value per row")
    _check(_lib.tidar_token_logprobs(rows, V, _ptr(logits), _ptr(targets), _ptr(logprobs), _ptr(dev_status),
                                     _ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))


def ceiling(name: str, *args, stream=None):
    """Enqueue one measurement kernel of include/tidar_ceilings.h:
    ceiling("hbm_read", src_tensor, grid, sink), ceiling("mfma_bf16", grid, iters, sink),
    ceiling("exp_f32" | "fma_f32" | "lds_read_b128" | "lds_read_tr16", grid, iters, sink),
    ceiling("empty", grid)."""
    st = _stream(stream)
    if name == "hbm_read":
        src, grid, sink = args
        _dev(src, None, "src")
        rc = _lib.tidar_ceiling_hbm_read(_ptr(src), src.numel() * src.element_size(), int(grid), _ptr(sink), st)
    elif name == "empty":
        rc = _lib.tidar_ceiling_empty(int(args[0]), st)
    else:
        grid, iters, sink = args
        rc = getattr(_lib, "tidar_ceiling_" + name)(int(grid), int(iters), _ptr(sink), st)
    if rc != 0:
        raise RuntimeError(f"tidar_ceiling_{name} returned {rc}")


def attn_stamps(max_workgroups: int):
    """The per-workgroup records of the last attention launch made with
    TIDAR_ATTN_STAMPS=1 (include/tidar_ceilings.h): a [max_workgroups, 8]
    uint64 numpy array."""
    import numpy as np
    out = np.zeros((max_workgroups, 8), dtype=np.uint64)
    rc = _lib.tidar_attn_stamps(out.ctypes.data, int(max_workgroups))
    if rc != 0:
        raise RuntimeError(f"tidar_attn_stamps returned {rc}")
    return out
