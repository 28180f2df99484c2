"""ctypes binding of libpxa.so (include/pxa.h).

Argument marshalling only: every step of the method runs in the HIP kernels
of libpxa.so.  Functions keep the C names; tensor arguments may be torch
tensors (device, dtype and contiguity are checked) or raw integer addresses
(used by host-only tests of the validation paths).  A non-zero return code
raises PxaError.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass
from typing import Optional

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpxa.so")

PXA_OK = 0
PXA_EINVAL = -1
PXA_EUNSUPPORTED = -2
PXA_ENULL = -3
PXA_EALIGN = -4
PXA_EWORKSPACE = -5
PXA_EHIP = -6
ERROR_NAMES = {0: "PXA_OK", -1: "PXA_EINVAL", -2: "PXA_EUNSUPPORTED", -3: "PXA_ENULL",
               -4: "PXA_EALIGN", -5: "PXA_EWORKSPACE", -6: "PXA_EHIP"}


class PxaError(RuntimeError):
    def __init__(self, code: int, where: str, detail: str = ""):
        self.code = code
        super().__init__(f"{where}: {ERROR_NAMES.get(code, code)} ({detail})")


class pxa_config(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("seq_len", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block", ctypes.c_int32), ("num_proxies", ctypes.c_int32),
                ("gamma", ctypes.c_float), ("softmax_scale", ctypes.c_float)]


PXA_BUDGET_DYNAMIC = 0
PXA_BUDGET_FIXED = 1
PXA_BUDGET_RATIO = 2
PXA_MAX_PROBE_BLOCKS = 64
PXA_MAX_FUSED_SEQS = 64


class pxa_options(ctypes.Structure):
    _fields_ = [("budget_mode", ctypes.c_int32), ("last_blocks", ctypes.c_int32),
                ("fixed_blocks", ctypes.c_int32), ("ratio", ctypes.c_float),
                ("score_stride", ctypes.c_int32), ("skip_threshold", ctypes.c_float)]


class pxa_workspace_layout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_size_t) for n in
                ("qbar", "kbar", "qexp", "kexp", "scores", "masses", "k_h", "row_ptr", "col_idx",
                 "row_order", "budget_ws", "select_ws", "total")]


_P = ctypes.c_void_p
_CFG = ctypes.POINTER(pxa_config)
_OPT = ctypes.POINTER(pxa_options)
_SIGNATURES = {
    "pxa_abi_version": (ctypes.c_int, []),
    "pxa_strerror": (ctypes.c_char_p, [ctypes.c_int]),
    "pxa_last_hip_error": (ctypes.c_char_p, []),
    "pxa_validate_config": (ctypes.c_int, [_CFG]),
    "pxa_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "pxa_get_workspace_layout": (ctypes.c_int, [_CFG, ctypes.POINTER(pxa_workspace_layout)]),
    "pxa_budget_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "pxa_select_workspace_bytes": (ctypes.c_size_t, [_CFG]),
    "pxa_max_col_entries": (ctypes.c_size_t, [_CFG]),
    "pxa_prefill": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_proxy_pool": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P]),
    "pxa_proxy_score": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P]),
    "pxa_budget_estimate": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_block_select": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_sparse_prefill": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pxa_dense_prefill": (ctypes.c_int, [_CFG, _P, _P, _P, _P, _P]),
    "pxa_validate_options": (ctypes.c_int, [_CFG, _OPT]),
    "pxa_proxy_score_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P, _P]),
    "pxa_sparse_prefill_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P, _P, _P, _P]),
    "pxa_prefill_batch": (ctypes.c_int, [_CFG, _OPT, ctypes.c_int32, ctypes.POINTER(ctypes.c_int32),
                                         _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_dense_prefill_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P]),
    "pxa_workspace_bytes_ex": (ctypes.c_size_t, [_CFG, _OPT]),
    "pxa_get_workspace_layout_ex": (ctypes.c_int, [_CFG, _OPT, ctypes.POINTER(pxa_workspace_layout)]),
    "pxa_budget_workspace_bytes_ex": (ctypes.c_size_t, [_CFG, _OPT]),
    "pxa_prefill_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_prefill_noalloc": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P]),
    "pxa_budget_estimate_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_block_select_ex": (ctypes.c_int, [_CFG, _OPT, _P, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]),
    "pxa_batch_workspace_bytes": (ctypes.c_size_t, [_CFG, _OPT, ctypes.c_int32,
                                                    ctypes.POINTER(ctypes.c_int32)]),
    "pxa_get_batch_workspace_layout": (ctypes.c_int, [_CFG, _OPT, ctypes.c_int32,
                                                      ctypes.POINTER(ctypes.c_int32),
                                                      ctypes.POINTER(pxa_workspace_layout)]),
}

_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpxa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m block_sparse_long_proxy_amd.build` "
            "(there is no fallback implementation)")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


@dataclass(frozen=True)
class Config:
    num_heads: int
    num_kv_heads: int
    seq_len: int
    head_dim: int
    num_proxies: int
    gamma: float
    softmax_scale: float = 0.0   # <= 0: 1/sqrt(head_dim)
    block: int = 128

    def c(self) -> pxa_config:
        return pxa_config(self.num_heads, self.num_kv_heads, self.seq_len, self.head_dim,
                          self.block, self.num_proxies, self.gamma, self.softmax_scale)

    @property
    def nb(self) -> int:
        """Blocks: ceil(N / B); the last one is partial when B does not divide N."""
        return -(-self.seq_len // self.block)

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclass(frozen=True)
class Options:
    """Method variants (include/pxa.h, pxa_options).  Options() is the default:
    the dynamic budget probed on the last query block, every query scored."""
    budget_mode: int = PXA_BUDGET_DYNAMIC
    last_blocks: int = 1
    fixed_blocks: int = 0
    ratio: float = 0.0
    score_stride: int = 1
    skip_threshold: float = 0.0

    @staticmethod
    def dynamic(last_blocks: int = 1, score_stride: int = 1, skip_threshold: float = 0.0) -> "Options":
        return Options(PXA_BUDGET_DYNAMIC, last_blocks=last_blocks, score_stride=score_stride,
                       skip_threshold=skip_threshold)

    @staticmethod
    def fixed(blocks: int, score_stride: int = 1, skip_threshold: float = 0.0) -> "Options":
        return Options(PXA_BUDGET_FIXED, fixed_blocks=blocks, score_stride=score_stride,
                       skip_threshold=skip_threshold)

    @staticmethod
    def ratio_of(r: float, score_stride: int = 1, skip_threshold: float = 0.0) -> "Options":
        return Options(PXA_BUDGET_RATIO, ratio=r, score_stride=score_stride,
                       skip_threshold=skip_threshold)

    def c(self) -> pxa_options:
        return pxa_options(self.budget_mode, self.last_blocks, self.fixed_blocks, self.ratio,
                           self.score_stride, self.skip_threshold)


def _bref(opts: Optional[Options]):
    return None if opts is None else ctypes.byref(opts.c())


def _check(rc: int, where: str) -> None:
    if rc != PXA_OK:
        lib = load_library()
        detail = lib.pxa_strerror(rc).decode()
        if rc == PXA_EHIP:
            detail += ": " + lib.pxa_last_hip_error().decode()
        raise PxaError(rc, where, detail)


def _ptr(x, dtype=None, name="tensor"):
    """Address of a torch tensor (checked) or a raw integer address."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    import torch
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor or an int address")
    if x.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {x.device})")
    if dtype is not None and x.dtype != dtype:
        raise ValueError(f"{name}: dtype {x.dtype}, expected {dtype}")
    if not x.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _dt(kind):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32, "i32": torch.int32,
            "u8": torch.uint8}[kind]


def _tp(x, kind, name):
    return _ptr(x, None if isinstance(x, int) or x is None else _dt(kind), name)


def _needs(cfg: Config, tokens: Optional[int] = None) -> dict:
    """Elements each array argument must hold for cfg (tokens: the total of a batch)."""
    H, Hkv, G, d, nb = cfg.num_heads, cfg.num_kv_heads, cfg.num_proxies, cfg.head_dim, cfg.nb
    N = cfg.seq_len if tokens is None else tokens
    return dict(q=H * N * d, o=H * N * d, k=Hkv * N * d, v=Hkv * N * d, qbar=G * N * d,
                kbar=G * N * d, qexp=G * nb, kexp=G * nb, scores=G * nb * nb, k_h=H, masses=H * nb, row_ptr=H * nb + 1,
                row_order=H * nb, col_idx=H * nb * (nb + 1) // 2)


def _check_sizes(cfg: Config, tokens: Optional[int] = None, ws=None, ws_bytes=None, **arrays):
    """Refuse torch tensors smaller than the call reads or writes (the kernels
    trust the sizes the configuration implies; raw int addresses are the
    caller's responsibility).  Skipped for an invalid configuration, which the
    library itself reports."""
    import torch
    if load_library().pxa_validate_config(ctypes.byref(cfg.c())) != PXA_OK:
        return
    need = _needs(cfg, tokens)
    for name, x in arrays.items():
        if isinstance(x, torch.Tensor) and x.numel() < need[name]:
            raise ValueError(f"{name}: {x.numel()} elements, the configuration needs {need[name]}")
    if isinstance(ws, torch.Tensor) and ws_bytes is not None:
        if ws_bytes > ws.numel() * ws.element_size():
            raise ValueError(f"ws_bytes {ws_bytes} exceeds the workspace tensor "
                             f"({ws.numel() * ws.element_size()} bytes)")


# ---------------------------------------------------------------- queries
def pxa_abi_version() -> int:
    return load_library().pxa_abi_version()


def pxa_strerror(code: int) -> str:
    return load_library().pxa_strerror(code).decode()


def pxa_validate_config(cfg: Config) -> int:
    return load_library().pxa_validate_config(ctypes.byref(cfg.c()))


def pxa_workspace_bytes(cfg: Config) -> int:
    return load_library().pxa_workspace_bytes(ctypes.byref(cfg.c()))


def pxa_get_workspace_layout(cfg: Config) -> pxa_workspace_layout:
    out = pxa_workspace_layout()
    _check(load_library().pxa_get_workspace_layout(ctypes.byref(cfg.c()), ctypes.byref(out)),
           "pxa_get_workspace_layout")
    return out


def pxa_budget_workspace_bytes(cfg: Config) -> int:
    return load_library().pxa_budget_workspace_bytes(ctypes.byref(cfg.c()))


def pxa_select_workspace_bytes(cfg: Config) -> int:
    return load_library().pxa_select_workspace_bytes(ctypes.byref(cfg.c()))


def pxa_max_col_entries(cfg: Config) -> int:
    return load_library().pxa_max_col_entries(ctypes.byref(cfg.c()))


# ---------------------------------------------------------------- compute calls
def _nbytes(ws, ws_bytes):
    if ws_bytes is not None:
        return ws_bytes
    return ws.numel() * ws.element_size()


def pxa_prefill(cfg: Config, q, k, v, o, ws, ws_bytes=None, stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, o=o, ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_prefill(
        ctypes.byref(cfg.c()), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"), _tp(v, "bf16", "v"),
        _tp(o, "bf16", "o"), _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes), _stream(stream)),
        "pxa_prefill")


def pxa_proxy_pool(cfg: Config, q, k, qbar, kbar, qexp, kexp, stream=None) -> None:
    """qbar, kbar: float16 [G, N, d]; qexp, kexp: int32 [G, nb] (block exponents)."""
    _check_sizes(cfg, q=q, k=k, qbar=qbar, kbar=kbar, qexp=qexp, kexp=kexp)
    _check(load_library().pxa_proxy_pool(
        ctypes.byref(cfg.c()), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(qbar, "f16", "qbar"), _tp(kbar, "f16", "kbar"), _tp(qexp, "i32", "qexp"),
        _tp(kexp, "i32", "kexp"), _stream(stream)), "pxa_proxy_pool")


def pxa_proxy_score(cfg: Config, qbar, kbar, qexp, kexp, scores, stream=None) -> None:
    _check_sizes(cfg, qbar=qbar, kbar=kbar, qexp=qexp, kexp=kexp, scores=scores)
    _check(load_library().pxa_proxy_score(
        ctypes.byref(cfg.c()), _tp(qbar, "f16", "qbar"), _tp(kbar, "f16", "kbar"),
        _tp(qexp, "i32", "qexp"), _tp(kexp, "i32", "kexp"), _tp(scores, "f32", "scores"),
        _stream(stream)), "pxa_proxy_score")


def pxa_budget_estimate(cfg: Config, q, k, scores, k_h, masses, ws, ws_bytes=None,
                        stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, scores=scores, k_h=k_h, masses=masses,
                 ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_budget_estimate(
        ctypes.byref(cfg.c()), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(scores, "f32", "scores"), _tp(k_h, "i32", "k_h"), _tp(masses, "f32", "masses"),
        _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes), _stream(stream)), "pxa_budget_estimate")


def pxa_block_select(cfg: Config, scores, k_h, row_ptr, col_idx, ws, ws_bytes=None,
                     stream=None, row_order=None) -> None:
    _check_sizes(cfg, scores=scores, k_h=k_h, row_ptr=row_ptr, col_idx=col_idx,
                 row_order=row_order, ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_block_select(
        ctypes.byref(cfg.c()), _tp(scores, "f32", "scores"), _tp(k_h, "i32", "k_h"),
        _tp(row_ptr, "i32", "row_ptr"), _tp(col_idx, "i32", "col_idx"),
        _tp(row_order, "i32", "row_order"), _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes),
        _stream(stream)), "pxa_block_select")


def pxa_sparse_prefill(cfg: Config, q, k, v, row_ptr, col_idx, o, stream=None,
                       row_order=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, row_ptr=row_ptr, row_order=row_order, o=o)
    _check(load_library().pxa_sparse_prefill(
        ctypes.byref(cfg.c()), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"), _tp(v, "bf16", "v"),
        _tp(row_ptr, "i32", "row_ptr"), _tp(col_idx, "i32", "col_idx"),
        _tp(row_order, "i32", "row_order"), _tp(o, "bf16", "o"), _stream(stream)),
        "pxa_sparse_prefill")


def pxa_dense_prefill(cfg: Config, q, k, v, o, stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, o=o)
    _check(load_library().pxa_dense_prefill(
        ctypes.byref(cfg.c()), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"), _tp(v, "bf16", "v"),
        _tp(o, "bf16", "o"), _stream(stream)), "pxa_dense_prefill")


# ---------------------------------------------------------------- method variants
def pxa_proxy_score_ex(cfg: Config, opts: Optional[Options], qbar, kbar, qexp, kexp, scores,
                       stream=None) -> None:
    _check_sizes(cfg, qbar=qbar, kbar=kbar, qexp=qexp, kexp=kexp, scores=scores)
    _check(load_library().pxa_proxy_score_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(qbar, "f16", "qbar"), _tp(kbar, "f16", "kbar"),
        _tp(qexp, "i32", "qexp"), _tp(kexp, "i32", "kexp"), _tp(scores, "f32", "scores"),
        _stream(stream)), "pxa_proxy_score_ex")


def pxa_validate_options(cfg: Config, opts: Optional[Options]) -> int:
    return load_library().pxa_validate_options(ctypes.byref(cfg.c()), _bref(opts))


def pxa_workspace_bytes_ex(cfg: Config, opts: Optional[Options]) -> int:
    return load_library().pxa_workspace_bytes_ex(ctypes.byref(cfg.c()), _bref(opts))


def pxa_get_workspace_layout_ex(cfg: Config, opts: Optional[Options]) -> pxa_workspace_layout:
    out = pxa_workspace_layout()
    _check(load_library().pxa_get_workspace_layout_ex(ctypes.byref(cfg.c()), _bref(opts),
                                                      ctypes.byref(out)),
           "pxa_get_workspace_layout_ex")
    return out


def pxa_budget_workspace_bytes_ex(cfg: Config, opts: Optional[Options]) -> int:
    return load_library().pxa_budget_workspace_bytes_ex(ctypes.byref(cfg.c()), _bref(opts))


def pxa_prefill_ex(cfg: Config, opts: Optional[Options], q, k, v, o, ws, ws_bytes=None,
                   stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, o=o, ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_prefill_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(v, "bf16", "v"), _tp(o, "bf16", "o"), _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes),
        _stream(stream)), "pxa_prefill_ex")


PXA_NOALLOC_SCRATCH_BYTES = 64 << 20


def pxa_prefill_noalloc(cfg: Config, opts: Optional[Options], q, k, v, o, stream=None) -> None:
    """The whole method in the library's static scratch array (no workspace,
    no allocation); configurations needing more than PXA_NOALLOC_SCRATCH_BYTES
    raise PXA_EWORKSPACE.  Overlapping calls on one GPU race."""
    _check_sizes(cfg, q=q, k=k, v=v, o=o)
    _check(load_library().pxa_prefill_noalloc(
        ctypes.byref(cfg.c()), _bref(opts), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(v, "bf16", "v"), _tp(o, "bf16", "o"), _stream(stream)), "pxa_prefill_noalloc")


def pxa_budget_estimate_ex(cfg: Config, opts: Optional[Options], q, k, scores, k_h, masses, ws,
                           ws_bytes=None, stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, scores=scores, k_h=k_h, masses=masses,
                 ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_budget_estimate_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(scores, "f32", "scores"), _tp(k_h, "i32", "k_h"), _tp(masses, "f32", "masses"),
        _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes) if ws is not None else 0, _stream(stream)),
        "pxa_budget_estimate_ex")


def pxa_block_select_ex(cfg: Config, opts: Optional[Options], scores, k_h, row_ptr, col_idx, ws,
                        ws_bytes=None, stream=None, row_order=None) -> None:
    _check_sizes(cfg, scores=scores, k_h=k_h, row_ptr=row_ptr, col_idx=col_idx,
                 row_order=row_order, ws=ws, ws_bytes=ws_bytes)
    _check(load_library().pxa_block_select_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(scores, "f32", "scores"), _tp(k_h, "i32", "k_h"),
        _tp(row_ptr, "i32", "row_ptr"), _tp(col_idx, "i32", "col_idx"),
        _tp(row_order, "i32", "row_order"), _tp(ws, "u8", "ws"), _nbytes(ws, ws_bytes),
        _stream(stream)), "pxa_block_select_ex")


def pxa_sparse_prefill_ex(cfg: Config, opts: Optional[Options], q, k, v, row_ptr, col_idx, o,
                          stream=None, row_order=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, row_ptr=row_ptr, row_order=row_order, o=o)
    _check(load_library().pxa_sparse_prefill_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(v, "bf16", "v"), _tp(row_ptr, "i32", "row_ptr"), _tp(col_idx, "i32", "col_idx"),
        _tp(row_order, "i32", "row_order"), _tp(o, "bf16", "o"), _stream(stream)),
        "pxa_sparse_prefill_ex")


def pxa_dense_prefill_ex(cfg: Config, opts: Optional[Options], q, k, v, o, stream=None) -> None:
    _check_sizes(cfg, q=q, k=k, v=v, o=o)
    _check(load_library().pxa_dense_prefill_ex(
        ctypes.byref(cfg.c()), _bref(opts), _tp(q, "bf16", "q"), _tp(k, "bf16", "k"),
        _tp(v, "bf16", "v"), _tp(o, "bf16", "o"), _stream(stream)), "pxa_dense_prefill_ex")


def _lens(seq_lens):
    n = len(seq_lens)
    return n, ((ctypes.c_int32 * max(n, 1))(*[int(x) for x in seq_lens]) if n else None)


def pxa_batch_workspace_bytes(cfg: Config, opts: Optional[Options], seq_lens) -> int:
    n, arr = _lens(seq_lens)
    return load_library().pxa_batch_workspace_bytes(ctypes.byref(cfg.c()), _bref(opts), n, arr)


def pxa_get_batch_workspace_layout(cfg: Config, opts: Optional[Options],
                                   seq_lens) -> pxa_workspace_layout:
    n, arr = _lens(seq_lens)
    out = pxa_workspace_layout()
    _check(load_library().pxa_get_batch_workspace_layout(ctypes.byref(cfg.c()), _bref(opts), n,
                                                         arr, ctypes.byref(out)),
           "pxa_get_batch_workspace_layout")
    return out


def pxa_prefill_batch(cfg: Config, opts: Optional[Options], seq_lens, q, k, v, o, ws,
                      ws_bytes=None, stream=None) -> None:
    """seq_lens: host list of per-sequence token counts; q/k/v/o: the per-sequence
    [heads][N_s][d] blocks stored one after another (flat bf16 tensors are fine).
    Fused when ws holds pxa_batch_workspace_bytes, else one sequence at a time."""
    _check_sizes(cfg, tokens=sum(int(x) for x in seq_lens), q=q, k=k, v=v, o=o, ws=ws,
                 ws_bytes=ws_bytes)
    n, arr = _lens(seq_lens)
    _check(load_library().pxa_prefill_batch(
        ctypes.byref(cfg.c()), _bref(opts), n, arr, _tp(q, "bf16", "q"),
        _tp(k, "bf16", "k"), _tp(v, "bf16", "v"), _tp(o, "bf16", "o"), _tp(ws, "u8", "ws"),
        _nbytes(ws, ws_bytes), _stream(stream)), "pxa_prefill_batch")
