"""Python binding of the FastOCR decode-step attention library (gfx950 HIP).

Thin marshalling over the C ABI in include/fastocr.h: every function named
``fastocr_*`` here calls the C function of the same name with raw device
pointers taken from torch tensors.  PyTorch provides device memory and
streams only; every step of the attention path runs in the library's HIP
kernels.  The shared library is loaded on first use and a missing library is
an error, never a fallback.

Before handing pointers to the library the binding checks every tensor's
device, dtype, contiguity and shape against the handle's configuration, so a
kernel never sees a buffer smaller than its grid assumes.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Dict, List, Optional, Sequence

from . import _abi
from ._abi import (DTYPE_BF16, DTYPE_F32, ERR_HIP, ERR_INVALID_ARG, ERR_OOM, ERR_SCRATCH, ERR_STATE,  # noqa: F401
                   FLAG_INDEX_CLAMPED, FLAG_LENS_CLAMPED, KC_NAMES, MODE_FULL, MODE_PRUNED,
                   OK, STATIC_SCRATCH_MIB)


class FastOCRError(RuntimeError):
    def __init__(self, fn: str, code: int):
        lib = _abi.load()
        msg = lib.fastocr_error_string(code).decode()
        super().__init__(f"{fn} failed: {msg} ({code})")
        self.code = code


def _check(fn: str, code: int) -> None:
    if code != OK:
        raise FastOCRError(fn, code)


def lib():
    return _abi.load()


@dataclass
class Config:
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    batch: int
    max_seq_len: int
    max_img_tokens: int
    tau: float
    num_focal: int = 1
    warmup_steps: int = 1
    dtype: str = "bf16"  # "bf16" | "f32"
    mode: str = "pruned"  # "pruned" | "full"
    sm_scale: float = 0.0
    min_img_tokens: int = 0
    max_text_tokens: int = 0
    reprofile_every: int = 0  # R > 0: re-pick the focal layers after every R pruned steps

    def to_c(self) -> _abi.Config:
        return _abi.Config(
            tau=float(self.tau), sm_scale=float(self.sm_scale), num_layers=self.num_layers,
            num_q_heads=self.num_q_heads, num_kv_heads=self.num_kv_heads, head_dim=self.head_dim,
            batch=self.batch, max_seq_len=self.max_seq_len, max_img_tokens=self.max_img_tokens,
            min_img_tokens=self.min_img_tokens, max_text_tokens=self.max_text_tokens,
            dtype=DTYPE_BF16 if self.dtype == "bf16" else DTYPE_F32,
            num_focal=self.num_focal, warmup_steps=self.warmup_steps,
            mode=MODE_FULL if self.mode == "full" else MODE_PRUNED,
            reprofile_every=self.reprofile_every)


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------


def _torch():
    import torch
    return torch


def _dev_ptr(t, dtype, shape, name: str, align: int = 16) -> int:
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.data_ptr() % align:
        raise ValueError(f"{name} must be {align}-byte aligned")
    return t.data_ptr()


def _stream_ptr(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream)


# ---------------------------------------------------------------------------
# the C ABI, one function per entry point
# ---------------------------------------------------------------------------


class Handle:
    """Owns a ``fastocr_handle*``; remembers the config for shape checks."""

    def __init__(self, ptr: int, cfg: Config, stream):
        self.ptr = ctypes.c_void_p(ptr)
        self.cfg = cfg
        self.stream = stream
        t = _torch()
        self.io_dtype = t.bfloat16 if cfg.dtype == "bf16" else t.float32

    def __del__(self):
        try:
            if getattr(self, "ptr", None) is not None and self.ptr.value:
                _abi.load().fastocr_destroy(self.ptr)
                self.ptr = ctypes.c_void_p(0)
        except Exception:  # interpreter shutdown: ctypes may already be gone
            pass


def fastocr_create(cfg: Config, stream=None) -> Handle:
    c = cfg.to_c()
    out = ctypes.c_void_p(0)
    _check("fastocr_create", lib().fastocr_create(ctypes.byref(c), ctypes.c_void_p(_stream_ptr(stream)),
                                                  ctypes.byref(out)))
    return Handle(out.value, cfg, stream)


def fastocr_create_static(cfg: Config, stream=None) -> Handle:
    """fastocr_create without device allocation: the scratch lives in the
    library's static array (at most one live static handle per GPU)."""
    c = cfg.to_c()
    out = ctypes.c_void_p(0)
    _check("fastocr_create_static", lib().fastocr_create_static(
        ctypes.byref(c), ctypes.c_void_p(_stream_ptr(stream)), ctypes.byref(out)))
    return Handle(out.value, cfg, stream)


def fastocr_attend(h: Handle, layer: int, q, k_cache, v_cache, lens, out) -> None:
    c = h.cfg
    t = _torch()
    qs = (c.batch, c.num_q_heads, c.head_dim)
    ks = (c.batch, c.num_kv_heads, c.max_seq_len, c.head_dim)
    args = (
        _dev_ptr(q, h.io_dtype, qs, "q"),
        _dev_ptr(k_cache, h.io_dtype, ks, "k_cache"),
        _dev_ptr(v_cache, h.io_dtype, ks, "v_cache"),
        _dev_ptr(lens, t.int32, (c.batch, 2), "lens", 4),
        _dev_ptr(out, h.io_dtype, qs, "out"),
    )
    _check("fastocr_attend", lib().fastocr_attend(h.ptr, int(layer), *args))


def fastocr_attend_append(h: Handle, layer: int, q, k_new, v_new, k_cache, v_cache, lens, out) -> None:
    c = h.cfg
    t = _torch()
    qs = (c.batch, c.num_q_heads, c.head_dim)
    ns = (c.batch, c.num_kv_heads, c.head_dim)
    ks = (c.batch, c.num_kv_heads, c.max_seq_len, c.head_dim)
    args = (
        _dev_ptr(q, h.io_dtype, qs, "q"),
        _dev_ptr(k_new, h.io_dtype, ns, "k_new"),
        _dev_ptr(v_new, h.io_dtype, ns, "v_new"),
        _dev_ptr(k_cache, h.io_dtype, ks, "k_cache"),
        _dev_ptr(v_cache, h.io_dtype, ks, "v_cache"),
        _dev_ptr(lens, t.int32, (c.batch, 2), "lens", 4),
        _dev_ptr(out, h.io_dtype, qs, "out"),
    )
    _check("fastocr_attend_append", lib().fastocr_attend_append(h.ptr, int(layer), *args))


def fastocr_profile_warmup(h: Handle) -> List[int]:
    arr = (ctypes.c_int32 * h.cfg.num_focal)()
    _check("fastocr_profile_warmup", lib().fastocr_profile_warmup(h.ptr, arr))
    return list(arr)


def fastocr_get_focal_layers(h: Handle) -> List[int]:
    arr = (ctypes.c_int32 * h.cfg.num_focal)()
    _check("fastocr_get_focal_layers", lib().fastocr_get_focal_layers(h.ptr, arr))
    return list(arr)


def fastocr_destroy(h: Handle) -> None:
    if h.ptr.value:
        code = lib().fastocr_destroy(h.ptr)
        h.ptr = ctypes.c_void_p(0)
        _check("fastocr_destroy", code)


def fastocr_get_status(h: Handle) -> int:
    v = ctypes.c_int32(0)
    _check("fastocr_get_status", lib().fastocr_get_status(h.ptr, ctypes.byref(v)))
    return v.value


def fastocr_get_info(h: Handle) -> Dict[str, int]:
    info = _abi.Info()
    _check("fastocr_get_info", lib().fastocr_get_info(h.ptr, ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _abi.Info._fields_}


def fastocr_plan_launch(cfg: Config, num_cu: int = 256) -> Dict[str, int]:
    """The launch plan fastocr_create would choose for cfg (host only)."""
    c = cfg.to_c()
    info = _abi.Info()
    _check("fastocr_plan_launch", lib().fastocr_plan_launch(ctypes.byref(c), int(num_cu), ctypes.byref(info)))
    return {f: getattr(info, f) for f, _ in _abi.Info._fields_}


def fastocr_get_selection(h: Handle, idx, cnt) -> None:
    t = _torch()
    info = fastocr_get_info(h)
    _check("fastocr_get_selection", lib().fastocr_get_selection(
        h.ptr, _dev_ptr(idx, t.int32, (h.cfg.batch, info["k_max"]), "idx", 4),
        _dev_ptr(cnt, t.int32, (h.cfg.batch,), "cnt", 4)))


def fastocr_set_selection(h: Handle, idx, cnt) -> None:
    t = _torch()
    info = fastocr_get_info(h)
    _check("fastocr_set_selection", lib().fastocr_set_selection(
        h.ptr, _dev_ptr(idx, t.int32, (h.cfg.batch, info["k_max"]), "idx", 4),
        _dev_ptr(cnt, t.int32, (h.cfg.batch,), "cnt", 4)))


def fastocr_get_scores(h: Handle, scores) -> None:
    t = _torch()
    _check("fastocr_get_scores", lib().fastocr_get_scores(
        h.ptr, _dev_ptr(scores, t.float32, (h.cfg.batch, h.cfg.max_img_tokens), "scores", 4)))


def fastocr_get_layer_ratios(h: Handle) -> List[float]:
    arr = (ctypes.c_double * h.cfg.num_layers)()
    _check("fastocr_get_layer_ratios", lib().fastocr_get_layer_ratios(h.ptr, arr))
    return list(arr)


def fastocr_set_focal_layers(h: Handle, layers: Sequence[int]) -> None:
    arr = (ctypes.c_int32 * len(layers))(*[int(x) for x in layers])
    _check("fastocr_set_focal_layers", lib().fastocr_set_focal_layers(h.ptr, arr, len(layers)))


def fastocr_set_timing(h: Handle, enable: bool) -> None:
    _check("fastocr_set_timing", lib().fastocr_set_timing(h.ptr, 1 if enable else 0))


def fastocr_get_timing(h: Handle) -> Dict[str, Dict[str, float]]:
    tm = _abi.Timing()
    _check("fastocr_get_timing", lib().fastocr_get_timing(h.ptr, ctypes.byref(tm)))
    return {name: {"total_ms": tm.total_ms[i], "launches": int(tm.launches[i]), "timed": int(tm.timed[i])}
            for i, name in enumerate(KC_NAMES)}


def fastocr_reset_timing(h: Handle) -> None:
    _check("fastocr_reset_timing", lib().fastocr_reset_timing(h.ptr))


def fastocr_select_topk(scores, lens, tau: float, idx_out, cnt_out, stream=None) -> None:
    t = _torch()
    B, stride = scores.shape
    k_stride = idx_out.shape[1]
    _check("fastocr_select_topk", lib().fastocr_select_topk(
        _dev_ptr(scores, t.float32, (B, stride), "scores", 4), int(stride),
        _dev_ptr(lens, t.int32, (B, 2), "lens", 4), int(B), float(tau),
        _dev_ptr(idx_out, t.int32, (B, k_stride), "idx_out", 4), int(k_stride),
        _dev_ptr(cnt_out, t.int32, (B,), "cnt_out", 4), ctypes.c_void_p(_stream_ptr(stream))))


def fastocr_state_bytes(h: Handle) -> int:
    n = ctypes.c_int64(0)
    _check("fastocr_state_bytes", lib().fastocr_state_bytes(h.ptr, ctypes.byref(n)))
    return n.value


def fastocr_save_state(h: Handle) -> bytes:
    """The handle's decode state at a step boundary, as bytes."""
    n = fastocr_state_bytes(h)
    buf = ctypes.create_string_buffer(n)
    _check("fastocr_save_state", lib().fastocr_save_state(h.ptr, buf, n))
    return buf.raw


def fastocr_load_state(h: Handle, blob: bytes) -> None:
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    _check("fastocr_load_state", lib().fastocr_load_state(h.ptr, buf, len(blob)))


def fastocr_image_first_map(spans: Sequence[Sequence[int]], rows: int):
    """(n_img, map): the image-first row permutation of one sequence (host)."""
    flat = [int(x) for sp in spans for x in sp]
    arr = (ctypes.c_int32 * max(len(flat), 1))(*flat)
    out = (ctypes.c_int32 * max(int(rows), 1))()
    n = int(lib().fastocr_image_first_map(arr, len(spans), int(rows), out))
    _check("fastocr_image_first_map", min(n, 0))
    return n, list(out)[:int(rows)]


def fastocr_pack_rows(src, dst, row_map, rows, status=None, stream=None) -> None:
    """dst[b, h, i] = src[b, h, row_map[b, i]] for i < rows[b] (device tensors)."""
    t = _torch()
    B, Hkv, S, d = src.shape
    dtype = {t.bfloat16: DTYPE_BF16, t.float32: DTYPE_F32}.get(src.dtype)
    if dtype is None:
        raise ValueError(f"src must be bfloat16 or float32, got {src.dtype}")
    _check("fastocr_pack_rows", lib().fastocr_pack_rows(
        _dev_ptr(src, src.dtype, (B, Hkv, S, d), "src"), _dev_ptr(dst, src.dtype, (B, Hkv, S, d), "dst"),
        _dev_ptr(row_map, t.int32, (B, S), "row_map", 4), _dev_ptr(rows, t.int32, (B,), "rows", 4),
        int(B), int(Hkv), int(S), int(d), dtype,
        ctypes.c_void_p(0 if status is None else _dev_ptr(status, t.int32, (1,), "status", 4)),
        ctypes.c_void_p(_stream_ptr(stream))))


def fastocr_probe_read(buf, nbytes: int, workgroups: int, sink, stream=None) -> None:
    """Read `nbytes` of the device tensor `buf` (from its start) with a
    stream-read kernel; sink: device int32 tensor of 64 entries."""
    t = _torch()
    if not isinstance(buf, t.Tensor) or buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    if nbytes > buf.numel() * buf.element_size() or buf.data_ptr() % 16:
        raise ValueError("nbytes exceeds buf, or buf is not 16-byte aligned")
    _check("fastocr_probe_read", lib().fastocr_probe_read(
        ctypes.c_void_p(buf.data_ptr()), int(nbytes), int(workgroups),
        ctypes.c_void_p(_dev_ptr(sink, t.int32, (64,), "sink", 4)), ctypes.c_void_p(_stream_ptr(stream))))


def fastocr_kept_count(tau: float, n_img: int) -> int:
    return int(lib().fastocr_kept_count(float(tau), int(n_img)))


def fastocr_choose_focal_layers(ratios: Sequence[float], num_focal: int) -> List[int]:
    r = (ctypes.c_double * len(ratios))(*[float(x) for x in ratios])
    out = (ctypes.c_int32 * num_focal)()
    _check("fastocr_choose_focal_layers",
           lib().fastocr_choose_focal_layers(r, len(ratios), int(num_focal), out))
    return list(out)


def fastocr_error_string(code: int) -> str:
    return lib().fastocr_error_string(int(code)).decode()
