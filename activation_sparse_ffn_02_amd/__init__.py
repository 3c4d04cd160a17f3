"""Python binding of libasf.so, the gfx950 activation-sparse FFN decode library.

Argument marshalling only: every step of the path (predictor, threshold,
compaction, gathered FC1/FC2, reduction, create-time layout) runs in the HIP
kernels behind the C ABI of ``include/asf.h``.  PyTorch supplies device
memory (the layer's storage and the outputs) and the current stream.

The library must be built (``python -m activation_sparse_ffn_02_amd.build``);
importing this module raises ImportError when ``libasf.so`` is missing.  There
is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libasf.so")

if not os.path.exists(LIB_PATH):
    raise ImportError("libasf.so is not built (run: python -m activation_sparse_ffn_02_amd.build)")

_lib = ctypes.CDLL(LIB_PATH)

F32, F16 = 0, 1
ASF_OK = 0
# kernels of a decode step in launch order (asf_kernel_id)
KERNEL_NAMES = ("pred_l1", "score", "score_fc1", "fc1", "fc2", "list")
STATUS_NAMES = {0: "ASF_OK", 1: "ASF_ERR_ARG", 2: "ASF_ERR_SHAPE", 3: "ASF_ERR_ALIGN",
                4: "ASF_ERR_STORAGE", 5: "ASF_ERR_UNSUPPORTED", 6: "ASF_ERR_HIP"}


class LayerDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32),
                ("pred_hidden", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("gated", ctypes.c_int32), ("wtype", ctypes.c_int32),
                ("threshold", ctypes.c_float)]


class LayerWeights(ctypes.Structure):
    _fields_ = [("w_up", ctypes.c_void_p), ("w_gate", ctypes.c_void_p), ("b1", ctypes.c_void_p),
                ("w_down", ctypes.c_void_p), ("b2", ctypes.c_void_p), ("p1", ctypes.c_void_p),
                ("c1", ctypes.c_void_p), ("p2", ctypes.c_void_p), ("c2", ctypes.c_void_p)]


_vp, _i32 = ctypes.c_void_p, ctypes.c_int32
_lib.asf_layer_storage_bytes.argtypes = [ctypes.POINTER(LayerDesc)]
_lib.asf_layer_storage_bytes.restype = ctypes.c_size_t
_lib.asf_create_layer.argtypes = [ctypes.POINTER(LayerDesc), ctypes.POINTER(LayerWeights), _vp,
                                  _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]
_lib.asf_create_layer.restype = ctypes.c_int
_lib.asf_destroy_layer.argtypes = [_vp]
_lib.asf_destroy_layer.restype = None
_lib.asf_predict.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp]
_lib.asf_predict.restype = ctypes.c_int
_lib.asf_sparse_ffn.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.asf_sparse_ffn.restype = ctypes.c_int
_lib.asf_decode_step.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.asf_decode_step.restype = ctypes.c_int
_lib.asf_exact_ffn.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp, _vp]
_lib.asf_exact_ffn.restype = ctypes.c_int
_lib.asf_profile_activations.argtypes = [_vp, _vp, _i32, _vp, _vp]
_lib.asf_profile_activations.restype = ctypes.c_int
_lib.asf_hot_first_table.argtypes = [_vp, _i32, _vp, _vp]
_lib.asf_hot_first_table.restype = ctypes.c_int
_lib.asf_stack_decode.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _i32, _i32, _vp, _vp, _vp]
_lib.asf_stack_decode.restype = ctypes.c_int
_lib.asf_stack_decode_lookahead.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _i32, _vp, _vp, _vp]
_lib.asf_stack_decode_lookahead.restype = ctypes.c_int
_lib.asf_dense_ffn_ref.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp]
_lib.asf_dense_ffn_ref.restype = ctypes.c_int
_lib.asf_layer_set_trace.argtypes = [_vp, ctypes.POINTER(ctypes.c_void_p), _i32]
_lib.asf_layer_set_trace.restype = ctypes.c_int
_lib.asf_status_string.argtypes = [ctypes.c_int]
_lib.asf_status_string.restype = ctypes.c_char_p
_lib.asf_version.argtypes = []
_lib.asf_version.restype = ctypes.c_char_p


class AsfError(RuntimeError):
    def __init__(self, code: int, what: str):
        super().__init__("%s: %s (%s)" % (what, _lib.asf_status_string(code).decode(),
                                           STATUS_NAMES.get(code, code)))
        self.code = code


def _check(code: int, what: str) -> None:
    if code != ASF_OK:
        raise AsfError(code, what)


def version() -> str:
    return _lib.asf_version().decode()


def library():
    """The loaded ctypes library (for direct C-ABI calls)."""
    return _lib


def _wtype(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.float32:
        return F32
    raise TypeError("weights must be float16 or float32, got %s" % t.dtype)


def _dev_ptr(t: Optional[torch.Tensor], dtype=None, name: str = "") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def make_desc(d_model: int, d_ffn: int, pred_hidden: int, max_batch: int = 1,
              gated: bool = False, wtype: int = F16, threshold: float = 0.0) -> LayerDesc:
    return LayerDesc(int(d_model), int(d_ffn), int(pred_hidden), int(max_batch), int(bool(gated)),
                     int(wtype), float(threshold))


def storage_bytes(d_model: int, d_ffn: int, pred_hidden: int, max_batch: int = 1,
                  gated: bool = False, wtype: int = F16) -> int:
    desc = make_desc(d_model, d_ffn, pred_hidden, max_batch, gated, wtype)
    return int(_lib.asf_layer_storage_bytes(ctypes.byref(desc)))


class Layer:
    """One FFN layer resident in device storage owned by this object.

    Weights are given in their original nn.Linear layouts (device tensors):
    w_up/w_gate [f][d], w_down [d][f], p1 [H][d], p2 [f][H]; biases float32.
    ``neuron_table`` (int32 [f], slot -> original id, hot neurons first) sets
    the stored order; None keeps the original order.
    """

    def __init__(self, w_up, w_down, p1, p2, *, w_gate=None, b1=None, b2=None, c1=None,
                 c2=None, neuron_table=None, max_batch: int = 1, threshold: float = 0.0,
                 stream=None, storage: Optional[torch.Tensor] = None):
        f, d = w_up.shape
        H = p1.shape[0]
        wt = _wtype(w_up)
        tdt = w_up.dtype
        self.d_model, self.d_ffn, self.pred_hidden, self.max_batch = d, f, H, max_batch
        self.gated = w_gate is not None
        self.device = w_up.device
        self.desc = make_desc(d, f, H, max_batch, self.gated, wt, threshold)
        nbytes = int(_lib.asf_layer_storage_bytes(ctypes.byref(self.desc)))
        if nbytes == 0:
            raise AsfError(2, "asf_layer_storage_bytes")
        if storage is None:
            storage = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.storage = storage
        w = LayerWeights(_dev_ptr(w_up, tdt, "w_up"), _dev_ptr(w_gate, tdt, "w_gate"),
                         _dev_ptr(b1, torch.float32, "b1"), _dev_ptr(w_down, tdt, "w_down"),
                         _dev_ptr(b2, torch.float32, "b2"), _dev_ptr(p1, tdt, "p1"),
                         _dev_ptr(c1, torch.float32, "c1"), _dev_ptr(p2, tdt, "p2"),
                         _dev_ptr(c2, torch.float32, "c2"))
        handle = _vp()
        _check(_lib.asf_create_layer(ctypes.byref(self.desc), ctypes.byref(w),
                                     _dev_ptr(neuron_table, torch.int32, "neuron_table"),
                                     storage.data_ptr(), storage.numel(), _stream(stream),
                                     ctypes.byref(handle)), "asf_create_layer")
        self._h = handle.value

    # ------------------------------------------------------------------ helpers
    def _x(self, x: torch.Tensor) -> torch.Tensor:
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.shape[-1] != self.d_model:
            raise ValueError("x must be [B][%d]" % self.d_model)
        return x

    def _out(self, out, B):
        if out is None:
            out = torch.empty((B, self.d_model), dtype=torch.float32, device=self.device)
        return out

    @property
    def handle(self) -> int:
        return self._h

    # ------------------------------------------------------------------ calls
    def predict(self, x, active=None, n_active=None, token_masks=None, stream=None,
                want_list: bool = True):
        """Returns (active ids [f] int32, n_active [1] int32); entries past
        n_active are unspecified."""
        x = self._x(x)
        B = x.shape[0]
        if want_list and active is None:
            active = torch.empty(self.d_ffn, dtype=torch.int32, device=self.device)
        if want_list and n_active is None:
            n_active = torch.empty(1, dtype=torch.int32, device=self.device)
        _check(_lib.asf_predict(self._h, _dev_ptr(x, torch.float32, "x"), B,
                                _dev_ptr(active, torch.int32, "active"),
                                _dev_ptr(n_active, torch.int32, "n_active"),
                                _dev_ptr(token_masks, torch.int64, "token_masks"), _stream(stream)),
               "asf_predict")
        return active, n_active

    def sparse_ffn(self, x, active=None, n_active=None, residual=None, out=None, stream=None):
        x = self._x(x)
        B = x.shape[0]
        out = self._out(out, B)
        _check(_lib.asf_sparse_ffn(self._h, _dev_ptr(x, torch.float32, "x"), B,
                                   _dev_ptr(active, torch.int32, "active"),
                                   _dev_ptr(n_active, torch.int32, "n_active"),
                                   _dev_ptr(residual, torch.float32, "residual"),
                                   _dev_ptr(out, torch.float32, "out"), _stream(stream)),
               "asf_sparse_ffn")
        return out

    def decode_step(self, x, residual=None, out=None, active=None, n_active=None, stream=None):
        x = self._x(x)
        B = x.shape[0]
        out = self._out(out, B)
        _check(_lib.asf_decode_step(self._h, _dev_ptr(x, torch.float32, "x"), B,
                                    _dev_ptr(residual, torch.float32, "residual"),
                                    _dev_ptr(out, torch.float32, "out"),
                                    _dev_ptr(active, torch.int32, "active"),
                                    _dev_ptr(n_active, torch.int32, "n_active"), _stream(stream)),
               "asf_decode_step")
        return out

    def decode_step_raw(self, x_ptr: int, B: int, y_ptr: int, stream_handle: int,
                        residual_ptr: Optional[int] = None) -> None:
        """decode_step on raw device pointers and a raw stream handle (no
        tensor checks), for launch-bound loops."""
        rc = _lib.asf_decode_step(self._h, x_ptr, B, residual_ptr, y_ptr, None, None,
                                  stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_decode_step")

    def sparse_ffn_raw(self, x_ptr: int, B: int, active_ptr: int, n_active_ptr: int, y_ptr: int,
                       stream_handle: int) -> None:
        """sparse_ffn over a caller id list on raw device pointers and a raw
        stream handle (no tensor checks), for launch-bound loops."""
        rc = _lib.asf_sparse_ffn(self._h, x_ptr, B, active_ptr, n_active_ptr, None, y_ptr,
                                 stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_sparse_ffn")

    def exact_ffn(self, x, residual=None, out=None, active=None, n_active=None, stream=None):
        """asf_exact_ffn: one token through the FFN over its true active set
        (every pre-activation computed, no predictor)."""
        x = self._x(x)
        B = x.shape[0]
        out = self._out(out, B)
        _check(_lib.asf_exact_ffn(self._h, _dev_ptr(x, torch.float32, "x"), B,
                                  _dev_ptr(residual, torch.float32, "residual"),
                                  _dev_ptr(out, torch.float32, "out"),
                                  _dev_ptr(active, torch.int32, "active"),
                                  _dev_ptr(n_active, torch.int32, "n_active"), _stream(stream)),
               "asf_exact_ffn")
        return out

    def exact_ffn_raw(self, x_ptr: int, y_ptr: int, stream_handle: int) -> None:
        """exact_ffn of one token on raw device pointers and a raw stream handle."""
        rc = _lib.asf_exact_ffn(self._h, x_ptr, 1, None, y_ptr, None, None, stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_exact_ffn")

    def profile_activations(self, x, counts=None, stream=None):
        """asf_profile_activations: add each token's true active set (by
        original id) into `counts` (uint32 viewed as int32 [d_ffn]; zeros when
        not given); returns counts."""
        x = self._x(x)
        if counts is None:
            counts = torch.zeros(self.d_ffn, dtype=torch.int32, device=x.device)
        _check(_lib.asf_profile_activations(self._h, _dev_ptr(x, torch.float32, "x"), x.shape[0],
                                            _dev_ptr(counts, torch.int32, "counts"),
                                            _stream(stream)),
               "asf_profile_activations")
        return counts

    def dense_ffn_ref(self, x, residual=None, out=None, stream=None):
        x = self._x(x)
        B = x.shape[0]
        out = self._out(out, B)
        _check(_lib.asf_dense_ffn_ref(self._h, _dev_ptr(x, torch.float32, "x"), B,
                                      _dev_ptr(residual, torch.float32, "residual"),
                                      _dev_ptr(out, torch.float32, "out"), _stream(stream)),
               "asf_dense_ffn_ref")
        return out

    def set_trace(self, events=None, n: int = 0):
        """Record HIP events (ctypes array of 2*n hipEvent_t) around each of
        the first n kernels of every later call; None turns tracing off."""
        _check(_lib.asf_layer_set_trace(self._h, events, int(n) if events is not None else 0),
               "asf_layer_set_trace")

    def close(self):
        if getattr(self, "_h", None):
            _lib.asf_destroy_layer(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Stack:
    """Layers run one after another in one call (asf_stack_decode):
    x_{l+1} = FFN_l(x_l), plus x_l when ``residual``.  Holds references to the
    layers; every layer must have the same d_model."""

    def __init__(self, layers, residual: bool = False):
        self.layers = list(layers)
        if not self.layers:
            raise ValueError("empty stack")
        self.d_model = self.layers[0].d_model
        self.device = self.layers[0].device
        self.residual = 1 if residual else 0
        self._arr = (_vp * len(self.layers))(*[l.handle for l in self.layers])
        self._work = {}

    def _work_for(self, B):
        w = self._work.get(B)
        if w is None:
            w = torch.empty((B, self.d_model), dtype=torch.float32, device=self.device)
            self._work[B] = w
        return w

    def decode(self, x, out=None, work=None, stream=None):
        if x.dim() == 1:
            x = x.unsqueeze(0)
        B = x.shape[0]
        if out is None:
            out = torch.empty((B, self.d_model), dtype=torch.float32, device=self.device)
        if work is None:
            work = self._work_for(B)
        _check(_lib.asf_stack_decode(self._arr, len(self.layers), _dev_ptr(x, torch.float32, "x"),
                                     B, self.residual, _dev_ptr(out, torch.float32, "out"),
                                     _dev_ptr(work, torch.float32, "work"), _stream(stream)),
               "asf_stack_decode")
        return out

    def decode_lookahead(self, x, out=None, work=None, stream=None):
        """asf_stack_decode_lookahead: one token, layer l+1's set predicted
        from layer l's input, in the same launches as layer l's FFN."""
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if out is None:
            out = torch.empty((1, self.d_model), dtype=torch.float32, device=self.device)
        if work is None:
            work = self._work_for(1)
        _check(_lib.asf_stack_decode_lookahead(self._arr, len(self.layers),
                                               _dev_ptr(x, torch.float32, "x"), self.residual,
                                               _dev_ptr(out, torch.float32, "out"),
                                               _dev_ptr(work, torch.float32, "work"),
                                               _stream(stream)),
               "asf_stack_decode_lookahead")
        return out

    def decode_lookahead_raw(self, x_ptr: int, y_ptr: int, work_ptr: int,
                             stream_handle: int) -> None:
        rc = _lib.asf_stack_decode_lookahead(self._arr, len(self.layers), x_ptr, self.residual,
                                             y_ptr, work_ptr, stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_stack_decode_lookahead")

    def decode_raw(self, x_ptr: int, B: int, y_ptr: int, work_ptr: int,
                   stream_handle: int) -> None:
        """decode on raw device pointers and a raw stream handle."""
        rc = _lib.asf_stack_decode(self._arr, len(self.layers), x_ptr, B, self.residual, y_ptr,
                                   work_ptr, stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_stack_decode")


def hot_first_table(counts, stream=None):
    """asf_hot_first_table: int32 [d_ffn] table (slot -> original id), most
    frequently active first, ties by smaller id, from device counts."""
    f = counts.numel()
    table = torch.empty(f, dtype=torch.int32, device=counts.device)
    _check(_lib.asf_hot_first_table(_dev_ptr(counts, torch.int32, "counts"), f,
                                    _dev_ptr(table, torch.int32, "table"), _stream(stream)),
           "asf_hot_first_table")
    return table


def layer_from_numpy(L, device="cuda", max_batch: int = 1, threshold: float = 0.0,
                     use_table: bool = True, stream=None) -> Layer:
    """Upload a host-side layer (workload.Layer-like object with numpy arrays)
    and create it.  The uploaded originals are dropped after creation."""
    def up(a):
        return None if a is None else torch.from_numpy(a).to(device)
    lay = Layer(up(L.w_up), up(L.w_down), up(L.p1), up(L.p2), w_gate=up(L.w_gate), b1=up(L.b1),
                b2=up(L.b2), c1=up(L.c1), c2=up(L.c2),
                neuron_table=up(L.perm) if use_table else None, max_batch=max_batch,
                threshold=threshold, stream=stream)
    return lay
