"""ctypes binding of libmk.so (include/mk.h): argument marshalling only.

Every step of the decode path runs in the HIP kernels behind the C ABI;
PyTorch only provides device memory and the stream handle.  Importing this
module does not touch a GPU; creating an Engine does.  A missing library is
an error, never a fallback.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmk.so")
HEADER = os.path.join(os.path.dirname(PKG), "include", "mk.h")

MK_OK = 0
MK_E_INVAL = -1
MK_E_RANGE = -2
MK_E_HIP = -3
MK_E_STATE = -4
MK_E_TIMEOUT = -5
MK_E_TOKEN = -6
MK_E_NOMEM = -7
MK_E_UNSUPPORTED = -8
MK_E_DEVICE = -9
MK_E_TOOBIG = -10

TRACE_STAMPS = 20  # stamps per (workgroup, stage) trace record

MODE_MEGA = 0
MODE_MULTI = 1
MODE_GRAPH = 2
MODE_CONV = 3
MODE_CONV_GRAPH = 4
MODES = {"mega": MODE_MEGA, "multi": MODE_MULTI, "graph": MODE_GRAPH, "conv": MODE_CONV,
         "conv-graph": MODE_CONV_GRAPH}


class MkConfig(ctypes.Structure):
    _fields_ = [
        ("n_layers", ctypes.c_int32), ("hidden", ctypes.c_int32), ("n_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("ffn", ctypes.c_int32),
        ("vocab", ctypes.c_int32), ("max_seq", ctypes.c_int32), ("batch", ctypes.c_int32),
        ("rms_eps", ctypes.c_float), ("rope_theta", ctypes.c_double), ("tie_embeddings", ctypes.c_int32),
        ("exec_mode", ctypes.c_int32), ("attn_chunks", ctypes.c_int32), ("num_wgs", ctypes.c_int32),
        ("watchdog_ms", ctypes.c_int32), ("trace", ctypes.c_int32), ("partial_input", ctypes.c_int32),
        ("prefill", ctypes.c_int32), ("reserved", ctypes.c_int32 * 4),
    ]


class MkLayerWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("attn_norm", "wq", "wk", "wv", "wo", "ffn_norm", "w_gate", "w_up", "w_down")]


class MkWeights(ctypes.Structure):
    _fields_ = [("embed", ctypes.c_void_p), ("final_norm", ctypes.c_void_p), ("lm_head", ctypes.c_void_p),
                ("layers", ctypes.POINTER(MkLayerWeights))]


class MkKv(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p)]


class MkStatus(ctypes.Structure):
    _fields_ = [("code", ctypes.c_int32), ("stage", ctypes.c_int32), ("wg", ctypes.c_int32),
                ("detail", ctypes.c_uint32)]


class MkPlanInfo(ctypes.Structure):
    _fields_ = [("num_wgs", ctypes.c_int32), ("num_stages", ctypes.c_int32), ("num_tasks", ctypes.c_int32),
                ("attn_chunks", ctypes.c_int32), ("weight_bytes", ctypes.c_int64),
                ("workspace_bytes", ctypes.c_int64), ("lds_bytes", ctypes.c_int32),
                ("ring_units", ctypes.c_int32), ("reserved", ctypes.c_int32 * 4)]


class MkError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {error_string(code)} ({code})" if what else f"{error_string(code)} ({code})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libmk.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: run `python -m persistent_megakernel_cu_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.mk_load.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkWeights), ctypes.POINTER(ctypes.c_void_p)]
        L.mk_load.restype = ctypes.c_int
        L.mk_decode_step.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(MkKv),
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mk_decode_step.restype = ctypes.c_int
        L.mk_decode_steps.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.POINTER(MkKv), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mk_decode_steps.restype = ctypes.c_int
        L.mk_reset.argtypes = [ctypes.c_void_p]
        L.mk_reset.restype = ctypes.c_int
        L.mk_free.argtypes = [ctypes.c_void_p]
        L.mk_free.restype = None
        L.mk_status.argtypes = [ctypes.c_void_p, ctypes.POINTER(MkStatus)]
        L.mk_status.restype = ctypes.c_int
        L.mk_error_string.argtypes = [ctypes.c_int]
        L.mk_error_string.restype = ctypes.c_char_p
        L.mk_plan_describe.argtypes = [ctypes.POINTER(MkConfig), ctypes.c_int32, ctypes.POINTER(MkPlanInfo)]
        L.mk_plan_describe.restype = ctypes.c_int
        L.mk_trace_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.POINTER(ctypes.c_int64),
                                    ctypes.POINTER(ctypes.c_int32)]
        L.mk_trace_copy.restype = ctypes.c_int
        L.mk_conv_workspace_size.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(ctypes.c_size_t)]
        L.mk_conv_workspace_size.restype = ctypes.c_int
        L.mk_conv_decode_step.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkWeights), ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.POINTER(MkKv), ctypes.c_void_p, ctypes.c_void_p,
                                          ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.mk_conv_decode_step.restype = ctypes.c_int
        L.mk_conv_decode_step_static.argtypes = [ctypes.POINTER(MkConfig), ctypes.POINTER(MkWeights),
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.POINTER(MkKv),
                                                 ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mk_conv_decode_step_static.restype = ctypes.c_int
        L.mk_w2a8_pack.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        L.mk_w2a8_pack.restype = ctypes.c_int
        L.mk_w2a8_quantize.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p]
        L.mk_w2a8_quantize.restype = ctypes.c_int
        L.mk_w2a8_gemv.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.mk_w2a8_gemv.restype = ctypes.c_int
        L.mk_w2a8_linear.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p]
        L.mk_w2a8_linear.restype = ctypes.c_int
        _lib = L
    return _lib


def header_functions() -> list[str]:
    """Names of the functions include/mk.h declares."""
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_\s\*]*?\b(mk_[a-z0-9_]+)\s*\(", text, re.M)))


def error_string(code: int) -> str:
    return lib().mk_error_string(int(code)).decode()


def make_config(shape, max_seq: int, batch: int = 1, mode: str | int = "mega", attn_chunks: int = 0,
                num_wgs: int = 0, watchdog_ms: int = 0, trace: bool = False, partial_input: bool = False,
                prefill: bool = False) -> MkConfig:
    c = MkConfig()
    c.n_layers, c.hidden, c.n_heads = shape.n_layers, shape.hidden, shape.n_heads
    c.n_kv_heads, c.head_dim, c.ffn, c.vocab = shape.n_kv_heads, shape.head_dim, shape.ffn, shape.vocab
    c.max_seq, c.batch = max_seq, batch
    c.rms_eps, c.rope_theta = shape.rms_eps, shape.rope_theta
    c.tie_embeddings = 1 if shape.tie_embeddings else 0
    c.exec_mode = MODES[mode] if isinstance(mode, str) else int(mode)
    c.attn_chunks, c.num_wgs, c.watchdog_ms = attn_chunks, num_wgs, watchdog_ms
    c.trace = 1 if trace else 0
    c.partial_input = 1 if partial_input else 0
    c.prefill = 1 if prefill else 0
    return c


def plan_describe(shape, max_seq: int, num_wgs: int = 256, **kw) -> MkPlanInfo:
    """Build and validate the task tape on the host (no GPU needed)."""
    info = MkPlanInfo()
    rc = lib().mk_plan_describe(ctypes.byref(make_config(shape, max_seq, **kw)), num_wgs, ctypes.byref(info))
    if rc != MK_OK:
        raise MkError(rc, "mk_plan_describe")
    return info


def weights_struct(shape, weights: dict):
    """(MkWeights, layer array) pointing at the device tensors of ``weights``;
    keep both (and the tensors) alive while the library may read them."""
    layers = (MkLayerWeights * max(1, shape.n_layers))()
    for l in range(shape.n_layers):
        for f in MkLayerWeights._fields_:
            setattr(layers[l], f[0], weights[f"layers.{l}.{f[0]}"].data_ptr())
    w = MkWeights()
    w.embed = weights["embed"].data_ptr()
    w.final_norm = weights["final_norm"].data_ptr()
    w.lm_head = weights["lm_head"].data_ptr() if not shape.tie_embeddings else None
    w.layers = layers
    return w, layers


def _stream_handle(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else stream


def conv_workspace_size(shape, max_seq: int, batch: int = 1) -> int:
    """Bytes of the conventional path's workspace (mk_conv_workspace_size; no GPU needed)."""
    n = ctypes.c_size_t()
    rc = lib().mk_conv_workspace_size(ctypes.byref(make_config(shape, max_seq, batch)), ctypes.byref(n))
    if rc != MK_OK:
        raise MkError(rc, "mk_conv_workspace_size")
    return n.value


def conv_decode_step(shape, weights: dict, max_seq: int, token, d_pos, kcache, vcache, logits, out_token,
                     workspace, batch: int = 1, stream=None) -> None:
    """One conventional step through mk_conv_decode_step (stateless; d_pos is a
    device int32 tensor, workspace a device buffer of conv_workspace_size bytes)."""
    cfg = make_config(shape, max_seq, batch)
    w, layers = weights_struct(shape, weights)
    kv = MkKv()
    kv.k, kv.v = kcache.data_ptr(), vcache.data_ptr()
    rc = lib().mk_conv_decode_step(ctypes.byref(cfg), ctypes.byref(w), token.data_ptr(), d_pos.data_ptr(),
                                   ctypes.byref(kv), logits.data_ptr(), out_token.data_ptr(), workspace.data_ptr(),
                                   workspace.numel() * workspace.element_size(),
                                   ctypes.c_void_p(_stream_handle(stream)))
    del layers
    if rc != MK_OK:
        raise MkError(rc, "mk_conv_decode_step")


def conv_decode_step_static(shape, weights: dict, max_seq: int, token, d_pos, kcache, vcache, logits, out_token,
                            batch: int = 1, stream=None) -> None:
    """One conventional step through mk_conv_decode_step_static (the library's
    fixed per-GPU scratch instead of a caller workspace)."""
    cfg = make_config(shape, max_seq, batch)
    w, layers = weights_struct(shape, weights)
    kv = MkKv()
    kv.k, kv.v = kcache.data_ptr(), vcache.data_ptr()
    rc = lib().mk_conv_decode_step_static(ctypes.byref(cfg), ctypes.byref(w), token.data_ptr(), d_pos.data_ptr(),
                                          ctypes.byref(kv), logits.data_ptr(), out_token.data_ptr(),
                                          ctypes.c_void_p(_stream_handle(stream)))
    del layers
    if rc != MK_OK:
        raise MkError(rc, "mk_conv_decode_step_static")


def w2a8_pack(codes):
    """Host packing of ternary codes (numpy int8 [rows][cols]) into the
    [rows][cols / 16] uint32 layout of mk_w2a8_pack."""
    import numpy as np

    codes = np.ascontiguousarray(codes, dtype=np.int8)
    rows, cols = codes.shape
    out = np.zeros((rows, cols // 16), dtype=np.uint32)
    rc = lib().mk_w2a8_pack(codes.ctypes.data, rows, cols, out.ctypes.data)
    if rc != MK_OK:
        raise MkError(rc, "mk_w2a8_pack")
    return out


def w2a8_quantize(x, xq, scale, stream=None) -> None:
    """mk_w2a8_quantize on device tensors: x float32 [cols] -> xq int8 [cols], scale float32 [1]."""
    rc = lib().mk_w2a8_quantize(ctypes.c_void_p(x.data_ptr()), x.numel(), ctypes.c_void_p(xq.data_ptr()),
                                ctypes.c_void_p(scale.data_ptr()), ctypes.c_void_p(_stream_handle(stream)))
    if rc != MK_OK:
        raise MkError(rc, "mk_w2a8_quantize")


def w2a8_gemv(packed, gamma, rows: int, cols: int, xq, scale, y, stream=None) -> None:
    """mk_w2a8_gemv on device tensors (packed uint32/int32 [rows][cols/16])."""
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    rc = lib().mk_w2a8_gemv(ptr(packed), ptr(gamma), rows, cols, ptr(xq), ptr(scale), ptr(y),
                            ctypes.c_void_p(_stream_handle(stream)))
    if rc != MK_OK:
        raise MkError(rc, "mk_w2a8_gemv")


def w2a8_linear(packed, gamma, rows: int, cols: int, x, y, stream=None) -> None:
    """mk_w2a8_linear on device tensors: y = W2A8 product of the float32 input x, one launch."""
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t is not None else 0)
    rc = lib().mk_w2a8_linear(ptr(packed), ptr(gamma), rows, cols, ptr(x), ptr(y),
                              ctypes.c_void_p(_stream_handle(stream)))
    if rc != MK_OK:
        raise MkError(rc, "mk_w2a8_linear")


class Engine:
    """One mk_handle: weights loaded once, then one decode step per call.

    ``weights`` maps tensor names (see synth_inputs.weight_shapes) to device
    tensors holding bf16 bit patterns (int16/uint16/bfloat16 dtype).  The
    library reads the embedding in place, and the LM head too (the embedding
    when tied, else ``lm_head``) whenever the hidden size needs no row padding
    (include/mk.h, mk_weights); the engine keeps a reference to the whole dict
    so that no borrowed buffer is freed while the handle lives.
    """

    def __init__(self, shape, weights: dict, max_seq: int, mode: str = "mega", batch: int = 1,
                 attn_chunks: int = 0, num_wgs: int = 0, watchdog_ms: int = 0, trace: bool = False,
                 partial_input: bool = False, prefill: bool = False):
        self.shape = shape
        self.max_seq = max_seq
        self.batch = batch
        self.prefill = prefill
        self.cfg = make_config(shape, max_seq, batch, mode, attn_chunks, num_wgs, watchdog_ms, trace, partial_input,
                               prefill)
        w, layers = weights_struct(shape, weights)
        self._weights = dict(weights)
        h = ctypes.c_void_p()
        rc = lib().mk_load(ctypes.byref(self.cfg), ctypes.byref(w), ctypes.byref(h))
        if rc != MK_OK:
            raise MkError(rc, "mk_load")
        self._h = h
        self._kv = MkKv()

    def decode_step(self, token, pos: int, kcache, vcache, logits, out_token, stream=None) -> None:
        """Enqueue one step on ``stream`` (a torch.cuda.Stream or raw handle; default: current)."""
        stream = _stream_handle(stream)
        self._kv.k = kcache.data_ptr()
        self._kv.v = vcache.data_ptr()
        rc = lib().mk_decode_step(self._h, token.data_ptr(), int(pos), ctypes.byref(self._kv), logits.data_ptr(),
                                  out_token.data_ptr(), ctypes.c_void_p(stream))
        if rc != MK_OK:
            raise MkError(rc, "mk_decode_step")

    def decode_steps(self, token, pos: int, n_steps: int, kcache, vcache, out_tokens, out_logits=None,
                     stream=None) -> None:
        """Enqueue n_steps greedy steps (mk_decode_steps): token [batch] feeds the first,
        out_tokens [n_steps][batch] receives every step's token, out_logits
        [n_steps][batch][vocab] every step's logits (or None)."""
        stream = _stream_handle(stream)
        self._kv.k = kcache.data_ptr()
        self._kv.v = vcache.data_ptr()
        rc = lib().mk_decode_steps(self._h, token.data_ptr(), int(pos), int(n_steps), ctypes.byref(self._kv),
                                   out_logits.data_ptr() if out_logits is not None else None,
                                   out_tokens.data_ptr(), ctypes.c_void_p(stream))
        if rc != MK_OK:
            raise MkError(rc, "mk_decode_steps")

    def trace(self):
        """Stamps of the latest step as (numpy uint64 [wg][stage][4], clock kHz)."""
        import numpy as np
        info = MkPlanInfo()
        rc = lib().mk_plan_describe(ctypes.byref(self.cfg), self.cfg.num_wgs or 256, ctypes.byref(info))
        if rc != MK_OK:
            raise MkError(rc, "mk_plan_describe")
        cap = TRACE_STAMPS * 4096 * info.num_stages
        buf = np.zeros(cap, dtype=np.uint64)
        n = ctypes.c_int64()
        khz = ctypes.c_int32()
        rc = lib().mk_trace_copy(self._h, buf.ctypes.data, cap, ctypes.byref(n), ctypes.byref(khz))
        if rc != MK_OK:
            raise MkError(rc, "mk_trace_copy")
        return buf[: n.value].reshape(-1, info.num_stages, TRACE_STAMPS), khz.value

    def status(self) -> MkStatus:
        s = MkStatus()
        lib().mk_status(self._h, ctypes.byref(s))
        return s

    def reset(self) -> None:
        rc = lib().mk_reset(self._h)
        if rc != MK_OK:
            raise MkError(rc, "mk_reset")

    def close(self) -> None:
        if getattr(self, "_h", None):
            lib().mk_free(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def to_device(weights_np: dict, device="cuda") -> dict:
    """Copy uint16 bf16 bit arrays to device int16 tensors (bit-identical)."""
    import torch
    out = {}
    for k, a in weights_np.items():
        out[k] = torch.from_numpy(a.view("int16")).to(device)
    return out
