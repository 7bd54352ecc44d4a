"""Python binding of libkd.so: argument marshalling only.

The functions here have the names of the C ABI in include/kd.h and do no
arithmetic of the decode step; every step runs in the HIP library. Torch is
used only for device memory and streams: device buffers are passed as
``tensor.data_ptr()``, streams as ``torch.cuda.Stream.cuda_stream``.

If libkd.so has not been built, importing this module still works, but every
call raises. Nothing here falls back to a CPU path.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkd.so")

KD_OK = 0
KD_ERR_INVALID_ARG = -1
KD_ERR_UNSUPPORTED = -2
KD_ERR_NO_DEVICE = -3
KD_ERR_OOM = -4
KD_ERR_HIP = -5
KD_ERR_LAUNCH = -6
KD_ERR_SCRATCH = -7

KD_STATUS_TOKEN_RANGE = 0x1
KD_STATUS_POS_OVERFLOW = 0x2
KD_STATUS_SYNC_TIMEOUT = 0x4
KD_STATUS_NAN = 0x8
KD_STATUS_CANCELLED = 0x10

KD_CTRL_CANCEL = 1
KD_CTRL_WAIT_LIMIT_US = 2

KD_DTYPE_F32 = 0
KD_DTYPE_BF16 = 1
KD_DTYPE_FP8_E4M3 = 2
KD_DTYPE_INT8 = 3

EXPORTS = (
    "kd_init",
    "kd_kv_layout",
    "kd_step",
    "kd_step_noalloc",
    "kd_prefill",
    "kd_generate",
    "kd_control",
    "kd_device_status",
    "kd_destroy",
    "kd_strerror",
    "kd_get_info",
    "kd_trace",
    "kd_stream_read",
)


class KDError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__(f"{what}: {strerror(code)} ({code})")
        self.code = code


class kd_config(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("ffn_dim", ctypes.c_int32),
        ("vocab", ctypes.c_int32),
        ("max_seq", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("norm_eps", ctypes.c_float),
        ("rope_base", ctypes.c_float),
        ("weight_dtype", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32),
        ("prefill_chunk", ctypes.c_int32),
    ]


_LAYER_TENSORS = ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")
_LAYER_SCALES = (("wq", "s_wq"), ("wk", "s_wk"), ("wv", "s_wv"), ("wo", "s_wo"), ("w_gate", "s_gate"), ("w_up", "s_up"),
                 ("w_down", "s_down"))


class kd_layer_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in _LAYER_TENSORS] + [(s, ctypes.c_void_p) for _, s in _LAYER_SCALES]


class kd_weights(ctypes.Structure):
    _fields_ = [
        ("embed", ctypes.c_void_p),
        ("layers", ctypes.POINTER(kd_layer_weights)),
        ("final_norm", ctypes.c_void_p),
        ("lm_head", ctypes.c_void_p),
        ("s_lm_head", ctypes.c_void_p),
    ]


_lib = None


def library() -> ctypes.CDLL:
    """Load libkd.so from the package directory (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} not built; run `python -m bandwidth_bound_transformer_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        lib.kd_init.argtypes = [ctypes.POINTER(kd_config), ctypes.POINTER(kd_weights), ctypes.POINTER(ctypes.c_void_p)]
        lib.kd_init.restype = ctypes.c_int
        lib.kd_kv_layout.argtypes = [ctypes.POINTER(kd_config), ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
        lib.kd_kv_layout.restype = ctypes.c_int
        lib.kd_step.argtypes = [ctypes.c_void_p] * 6
        lib.kd_step.restype = ctypes.c_int
        lib.kd_step_noalloc.argtypes = [ctypes.c_void_p] * 6
        lib.kd_step_noalloc.restype = ctypes.c_int
        lib.kd_prefill.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 5
        lib.kd_prefill.restype = ctypes.c_int
        lib.kd_generate.argtypes = [ctypes.c_void_p, ctypes.c_int32] + [ctypes.c_void_p] * 7
        lib.kd_generate.restype = ctypes.c_int
        lib.kd_control.argtypes = [ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64]
        lib.kd_control.restype = ctypes.c_int
        lib.kd_device_status.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int]
        lib.kd_device_status.restype = ctypes.c_int
        lib.kd_destroy.argtypes = [ctypes.c_void_p]
        lib.kd_destroy.restype = None
        lib.kd_strerror.argtypes = [ctypes.c_int]
        lib.kd_strerror.restype = ctypes.c_char_p
        lib.kd_get_info.argtypes = [ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)]
        lib.kd_get_info.restype = ctypes.c_int
        lib.kd_trace.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64)]
        lib.kd_trace.restype = ctypes.c_int
        lib.kd_stream_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        lib.kd_stream_read.restype = ctypes.c_int
        _lib = lib
    return _lib


def strerror(code: int) -> str:
    return library().kd_strerror(int(code)).decode()


def _check(code: int, what: str) -> None:
    if code != KD_OK:
        raise KDError(code, what)


def make_config(shape, batch: int = 1, max_seq: int = 1, prefill_chunk: int = 0) -> kd_config:
    """kd_config of a ``workloads.ModelShape``."""
    dt = {"f32": KD_DTYPE_F32, "bf16": KD_DTYPE_BF16, "fp8": KD_DTYPE_FP8_E4M3, "int8": KD_DTYPE_INT8}
    return kd_config(
        shape.n_layers, shape.d_model, shape.n_q_heads, shape.n_kv_heads, shape.head_dim, shape.ffn_dim,
        shape.vocab, max_seq, batch, shape.norm_eps, shape.rope_base, dt[shape.weight_dtype], dt[shape.kv_dtype],
        prefill_chunk,
    )


def _host_ptr(a: np.ndarray) -> int:
    if not a.flags["C_CONTIGUOUS"]:
        raise ValueError("weight arrays must be C-contiguous")
    return a.ctypes.data


def kd_kv_layout(cfg: kd_config):
    """(bytes, element strides[6]) of the caller-owned KV cache."""
    nbytes = ctypes.c_size_t()
    strides = (ctypes.c_size_t * 6)()
    _check(library().kd_kv_layout(ctypes.byref(cfg), ctypes.byref(nbytes), strides), "kd_kv_layout")
    return nbytes.value, tuple(strides)


def _tensor_ptrs(t):
    """(data pointer, row-scale pointer or None): an fp8 or int8 matrix carries codes and scales."""
    if hasattr(t, "codes"):
        return _host_ptr(t.codes), _host_ptr(t.scale)
    return _host_ptr(t), None


def kd_init(cfg: kd_config, weights: dict) -> int:
    """Pack ``weights`` (dict from ``workloads.make_weights``) onto the current device; returns a handle."""
    scale_of = dict(_LAYER_SCALES)
    layers = (kd_layer_weights * cfg.n_layers)()
    for i, lw in enumerate(weights["layers"]):
        for n in _LAYER_TENSORS:
            data, scale = _tensor_ptrs(lw[n])
            setattr(layers[i], n, data)
            if scale is not None:
                setattr(layers[i], scale_of[n], scale)
    lm, lm_scale = _tensor_ptrs(weights["lm_head"])
    w = kd_weights(_host_ptr(weights["embed"]), layers, _host_ptr(weights["final_norm"]), lm, lm_scale)
    h = ctypes.c_void_p()
    _check(library().kd_init(ctypes.byref(cfg), ctypes.byref(w), ctypes.byref(h)), "kd_init")
    return h.value


def _dev_ptr(t) -> int | None:
    if t is None:
        return None
    if hasattr(t, "data_ptr"):
        return t.data_ptr()
    return int(t)


def kd_step(handle: int, tokens, positions, kv, logits=None, stream=None) -> None:
    """Enqueue one decode step (device buffers as torch tensors or raw pointers)."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(
        library().kd_step(handle, _dev_ptr(tokens), _dev_ptr(positions), _dev_ptr(kv), _dev_ptr(logits), s),
        "kd_step",
    )


def kd_step_noalloc(handle: int, tokens, positions, kv, logits=None, stream=None) -> None:
    """kd_step with the library's static scratch instead of the handle's exchange memory."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(
        library().kd_step_noalloc(handle, _dev_ptr(tokens), _dev_ptr(positions), _dev_ptr(kv), _dev_ptr(logits), s),
        "kd_step_noalloc",
    )


def kd_prefill(handle: int, prompt, n: int, tokens, positions, kv, logits=None, stream=None) -> None:
    """Enqueue the prompt (device int32[n]) on the matrix cores; tokens[0] receives the next token."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(
        library().kd_prefill(handle, _dev_ptr(prompt), int(n), _dev_ptr(tokens), _dev_ptr(positions), _dev_ptr(kv),
                             _dev_ptr(logits), s),
        "kd_prefill",
    )


def kd_generate(handle: int, n_steps: int, tokens, positions, kv, out_tokens=None, logits=None, progress=None,
                stream=None) -> None:
    """Enqueue n_steps greedy decode steps in one call (device buffers as torch tensors or raw pointers)."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(
        library().kd_generate(handle, int(n_steps), _dev_ptr(tokens), _dev_ptr(positions), _dev_ptr(kv),
                              _dev_ptr(out_tokens), _dev_ptr(logits), _dev_ptr(progress), s),
        "kd_generate",
    )


def kd_control(handle: int, op: int, value: int) -> None:
    _check(library().kd_control(handle, int(op), int(value)), "kd_control")


def kd_device_status(handle: int, clear: bool = False) -> int:
    bits = ctypes.c_uint32()
    _check(library().kd_device_status(handle, ctypes.byref(bits), int(bool(clear))), "kd_device_status")
    return bits.value


def kd_destroy(handle: int | None) -> None:
    library().kd_destroy(handle)


def kd_strerror(code: int) -> str:
    return strerror(code)


def kd_get_info(handle: int) -> dict:
    info = (ctypes.c_int64 * 8)()
    _check(library().kd_get_info(handle, info), "kd_get_info")
    return {
        "workgroups": info[0],
        "threads": info[1],
        "packed_weight_bytes": info[2],
        "lds_bytes": info[3],
        "ring_packets": info[4],
        "kernels_per_step": info[5],
        "split_k": [(info[6] >> (8 * i)) & 0xFF for i in range(4)],
        "attention_chunk": info[7],
    }


def kd_trace(handle: int, dev_buf=None, words: int = 0) -> int:
    """Turn step tracing on (device buffer of uint64 words) or off (None); returns the per-workgroup stride."""
    stride = ctypes.c_int64()
    _check(library().kd_trace(handle, _dev_ptr(dev_buf), int(words), ctypes.byref(stride)), "kd_trace")
    return stride.value


def kd_stream_read(buf, nbytes: int, stream=None) -> None:
    """Enqueue one plain read of nbytes of the device buffer (measurement of the HBM read rate)."""
    s = stream.cuda_stream if hasattr(stream, "cuda_stream") else stream
    _check(library().kd_stream_read(_dev_ptr(buf), int(nbytes), s), "kd_stream_read")


class Decoder:
    """A handle plus the device buffers one session needs (torch for memory and streams only)."""

    def __init__(self, shape, weights: dict, max_seq: int, batch: int = 1, device: str = "cuda:0", prefill_chunk: int = 0):
        import torch

        self.torch = torch
        self.device = torch.device(device)
        self.shape = shape
        self.cfg = make_config(shape, batch, max_seq, prefill_chunk)
        with torch.cuda.device(self.device):
            self.handle = kd_init(self.cfg, weights)
        nbytes, self.kv_strides = kd_kv_layout(self.cfg)
        kv_dtype = torch.bfloat16 if shape.kv_dtype == "bf16" else torch.float32
        elems = nbytes // (2 if shape.kv_dtype == "bf16" else 4)
        self.kv = torch.zeros(elems, dtype=kv_dtype, device=self.device)
        self.s_alloc = self.kv_strides[3] // shape.head_dim
        self.tokens = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.positions = torch.zeros(batch, dtype=torch.int32, device=self.device)
        self.logits = torch.zeros(batch, shape.vocab, dtype=torch.float32, device=self.device)

    def kv_view(self):
        """The cache as [L][2][B][Hkv][S][hd] (a view of the flat buffer)."""
        m = self.shape
        return self.kv.view(m.n_layers, 2, self.cfg.batch, m.n_kv_heads, self.s_alloc, m.head_dim)

    def step(self, write_logits: bool = True, stream=None) -> None:
        kd_step(self.handle, self.tokens, self.positions, self.kv, self.logits if write_logits else None,
                stream if stream is not None else self.torch.cuda.current_stream(self.device))

    def prefill(self, prompt, write_logits: bool = True, stream=None) -> None:
        """Run ``prompt`` (a device int32 tensor) from positions[0] on; tokens[0] gets the next token."""
        kd_prefill(self.handle, prompt, prompt.numel(), self.tokens, self.positions, self.kv,
                   self.logits if write_logits else None,
                   stream if stream is not None else self.torch.cuda.current_stream(self.device))

    def generate(self, n_steps: int, out_tokens=None, logits=None, progress=None, stream=None) -> None:
        kd_generate(self.handle, n_steps, self.tokens, self.positions, self.kv, out_tokens, logits, progress,
                    stream if stream is not None else self.torch.cuda.current_stream(self.device))

    def control(self, op: int, value: int) -> None:
        kd_control(self.handle, op, value)

    def status(self, clear: bool = False) -> int:
        return kd_device_status(self.handle, clear)

    def close(self) -> None:
        if getattr(self, "handle", None):
            kd_destroy(self.handle)
            self.handle = None

    def __del__(self):  # pragma: no cover - best effort
        try:
            self.close()
        except Exception:
            pass
