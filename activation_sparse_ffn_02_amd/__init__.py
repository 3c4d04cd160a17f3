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
_lib.asf_stack_decode_static.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _i32, _i32, _vp, _vp]
_lib.asf_stack_decode_static.restype = ctypes.c_int
_lib.asf_stack_decode_lookahead.argtypes = [ctypes.POINTER(_vp), _i32, _vp, _i32, _vp, _vp, _vp]
_lib.asf_stack_decode_lookahead.restype = ctypes.c_int
_lib.asf_dense_ffn_ref.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp]
_lib.asf_dense_ffn_ref.restype = ctypes.c_int
class HeadDesc(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("n_heads", ctypes.c_int32),
                ("pred_hidden", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("threshold", ctypes.c_float)]


class HeadWeights(ctypes.Structure):
    _fields_ = [("q1", ctypes.c_void_p), ("c1", ctypes.c_void_p), ("q2", ctypes.c_void_p),
                ("c2", ctypes.c_void_p)]


_lib.asf_head_predictor_storage_bytes.argtypes = [ctypes.POINTER(HeadDesc)]
_lib.asf_head_predictor_storage_bytes.restype = ctypes.c_size_t
_lib.asf_create_head_predictor.argtypes = [ctypes.POINTER(HeadDesc), ctypes.POINTER(HeadWeights),
                                           _vp, ctypes.c_size_t, _vp, ctypes.POINTER(_vp)]
_lib.asf_create_head_predictor.restype = ctypes.c_int
_lib.asf_destroy_head_predictor.argtypes = [_vp]
_lib.asf_destroy_head_predictor.restype = None
_lib.asf_predict_heads.argtypes = [_vp, _vp, _i32, _vp, _vp, _vp, _vp]
_lib.asf_predict_heads.restype = ctypes.c_int
_lib.asf_step_launches.argtypes = [_vp, _i32]
_lib.asf_step_launches.restype = _i32
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


def _arg(t: Optional[torch.Tensor], name: str, dtype=None, shape=None,
         min_numel=None) -> Optional[int]:
    """Check a tensor argument's dtype, shape (exact, or at least
    ``min_numel`` elements) and contiguity, and return its data pointer
    (None for None).  The C ABI takes bare pointers, so a short buffer would
    be read or written out of bounds on the device: a mismatch raises
    ValueError (TypeError for a wrong dtype) here instead.  Where the tensor
    lives is checked by ``_on_device`` once every argument has passed."""
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s must have shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if min_numel is not None and t.numel() < min_numel:
        raise ValueError("%s must hold at least %d elements, got %d" % (name, min_numel, t.numel()))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t.data_ptr()


def _on_device(device, **tensors) -> None:
    """Every given tensor (None skipped) is a GPU tensor on ``device`` (on
    the same device as the others when ``device`` is None)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError("%s must be a device tensor" % name)
        if device is None:
            device = t.device
        elif t.device != torch.device(device):
            raise ValueError("%s is on %s, expected %s" % (name, t.device, device))


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


def _tokens(x, d_model: int, max_b: int) -> torch.Tensor:
    """x as [B][d_model] float32 (a 1-D x is one token), B in 1 .. max_b."""
    if not isinstance(x, torch.Tensor):
        raise TypeError("x must be a torch.Tensor")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2 or x.shape[1] != d_model:
        raise ValueError("x must be [B][%d], got %s" % (d_model, tuple(x.shape)))
    if not 1 <= x.shape[0] <= max_b:
        raise ValueError("batch %d outside 1 .. %d" % (x.shape[0], max_b))
    _arg(x, "x", torch.float32)
    return x


class Layer:
    """One FFN layer resident in device storage owned by this object.

    Weights are given in their original nn.Linear layouts (device tensors):
    w_up/w_gate [f][d], w_down [d][f], p1 [H][d], p2 [f][H]; biases float32.
    ``neuron_table`` (int32 [f], slot -> original id, hot neurons first) sets
    the stored order; None keeps the original order.  Every tensor argument
    of every call is checked (dtype, shape, device) before the C call.
    """

    def __init__(self, w_up, w_down, p1, p2, *, w_gate=None, b1=None, b2=None, c1=None,
                 c2=None, neuron_table=None, max_batch: int = 1, threshold: float = 0.0,
                 stream=None, storage: Optional[torch.Tensor] = None):
        if not isinstance(w_up, torch.Tensor) or w_up.dim() != 2:
            raise ValueError("w_up must be a [d_ffn][d_model] tensor")
        if not isinstance(p1, torch.Tensor) or p1.dim() != 2:
            raise ValueError("p1 must be a [pred_hidden][d_model] tensor")
        f, d = w_up.shape
        H = p1.shape[0]
        wt = _wtype(w_up)
        tdt = w_up.dtype
        self.d_model, self.d_ffn, self.pred_hidden, self.max_batch = d, f, H, max_batch
        self.gated = w_gate is not None
        self.device = w_up.device
        w = LayerWeights(_arg(w_up, "w_up", tdt, (f, d)), _arg(w_gate, "w_gate", tdt, (f, d)),
                         _arg(b1, "b1", torch.float32, (f,)), _arg(w_down, "w_down", tdt, (d, f)),
                         _arg(b2, "b2", torch.float32, (d,)), _arg(p1, "p1", tdt, (H, d)),
                         _arg(c1, "c1", torch.float32, (H,)), _arg(p2, "p2", tdt, (f, H)),
                         _arg(c2, "c2", torch.float32, (f,)))
        table = _arg(neuron_table, "neuron_table", torch.int32, (f,))
        self.desc = make_desc(d, f, H, max_batch, self.gated, wt, threshold)
        nbytes = int(_lib.asf_layer_storage_bytes(ctypes.byref(self.desc)))
        if nbytes == 0:
            raise AsfError(2, "asf_layer_storage_bytes")
        _arg(storage, "storage", torch.uint8, min_numel=nbytes)
        _on_device(None, w_up=w_up, w_gate=w_gate, b1=b1, w_down=w_down, b2=b2, p1=p1, c1=c1,
                   p2=p2, c2=c2, neuron_table=neuron_table, storage=storage)
        if storage is None:
            storage = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.storage = storage
        handle = _vp()
        _check(_lib.asf_create_layer(ctypes.byref(self.desc), ctypes.byref(w),
                                     table, storage.data_ptr(), storage.numel(), _stream(stream),
                                     ctypes.byref(handle)), "asf_create_layer")
        self._h = handle.value

    # ------------------------------------------------------------------ helpers
    def _vec(self, t, name, B):
        """A [B][d_model] float32 operand (residual, out)."""
        return _arg(t, name, torch.float32, (B, self.d_model))

    def _new_out(self, out, B):
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
        n_active are unspecified.  ``token_masks``: int64 [B][ceil(f/64)]."""
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        _arg(active, "active", torch.int32, min_numel=self.d_ffn)
        _arg(n_active, "n_active", torch.int32, min_numel=1)
        pm = _arg(token_masks, "token_masks", torch.int64, min_numel=B * ((self.d_ffn + 63) // 64))
        _on_device(self.device, x=x, active=active, n_active=n_active, token_masks=token_masks)
        if want_list and active is None:
            active = torch.empty(self.d_ffn, dtype=torch.int32, device=self.device)
        if want_list and n_active is None:
            n_active = torch.empty(1, dtype=torch.int32, device=self.device)
        pa, pn = _arg(active, "active"), _arg(n_active, "n_active")
        _check(_lib.asf_predict(self._h, x.data_ptr(), B, pa, pn, pm, _stream(stream)),
               "asf_predict")
        return active, n_active

    def sparse_ffn(self, x, active=None, n_active=None, residual=None, out=None, stream=None):
        """FFN over a neuron set.  ``active``: a 1-D int32 list of at most
        d_ffn original ids on the device, or None for the layer's last
        prediction.  ``n_active``: a device int32 count, or None for all of
        ``active``.  A device count is not read back here: it must not
        exceed ``active.numel()`` (the library reads that many ids, at most
        d_ffn)."""
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        if active is not None:
            _arg(active, "active", torch.int32)
            if active.dim() != 1 or active.numel() > self.d_ffn:
                raise ValueError("active must be a 1-D list of at most %d ids" % self.d_ffn)
        elif n_active is not None:
            raise ValueError("n_active without active")
        pr, po = self._vec(residual, "residual", B), self._vec(out, "out", B)
        _arg(n_active, "n_active", torch.int32, min_numel=1)
        _on_device(self.device, x=x, active=active, n_active=n_active, residual=residual, out=out)
        out = self._new_out(out, B)
        if active is not None and n_active is None:
            n_active = torch.full((1,), active.numel(), dtype=torch.int32, device=self.device)
        _check(_lib.asf_sparse_ffn(self._h, x.data_ptr(), B, _arg(active, "active"),
                                   _arg(n_active, "n_active"), pr, out.data_ptr(),
                                   _stream(stream)),
               "asf_sparse_ffn")
        return out

    def decode_step(self, x, residual=None, out=None, active=None, n_active=None, stream=None):
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        pr = self._vec(residual, "residual", B)
        self._vec(out, "out", B)
        pa = _arg(active, "active", torch.int32, min_numel=self.d_ffn)
        pn = _arg(n_active, "n_active", torch.int32, min_numel=1)
        _on_device(self.device, x=x, residual=residual, out=out, active=active, n_active=n_active)
        out = self._new_out(out, B)
        _check(_lib.asf_decode_step(self._h, x.data_ptr(), B, pr, out.data_ptr(), pa, pn,
                                    _stream(stream)),
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
        x = _tokens(x, self.d_model, 1)
        pr = self._vec(residual, "residual", 1)
        self._vec(out, "out", 1)
        pa = _arg(active, "active", torch.int32, min_numel=self.d_ffn)
        pn = _arg(n_active, "n_active", torch.int32, min_numel=1)
        _on_device(self.device, x=x, residual=residual, out=out, active=active, n_active=n_active)
        out = self._new_out(out, 1)
        _check(_lib.asf_exact_ffn(self._h, x.data_ptr(), 1, pr, out.data_ptr(), pa, pn,
                                  _stream(stream)),
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
        if not isinstance(x, torch.Tensor):
            raise TypeError("x must be a torch.Tensor")
        if x.dim() == 1:
            x = x.unsqueeze(0)
        if x.dim() != 2 or x.shape[1] != self.d_model:
            raise ValueError("x must be [n][%d], got %s" % (self.d_model, tuple(x.shape)))
        px = _arg(x, "x", torch.float32)
        _arg(counts, "counts", torch.int32, (self.d_ffn,))
        _on_device(self.device, x=x, counts=counts)
        if counts is None:
            counts = torch.zeros(self.d_ffn, dtype=torch.int32, device=self.device)
        _check(_lib.asf_profile_activations(self._h, px, x.shape[0], counts.data_ptr(),
                                            _stream(stream)),
               "asf_profile_activations")
        return counts

    def dense_ffn_ref(self, x, residual=None, out=None, stream=None):
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        pr = self._vec(residual, "residual", B)
        self._vec(out, "out", B)
        _on_device(self.device, x=x, residual=residual, out=out)
        out = self._new_out(out, B)
        _check(_lib.asf_dense_ffn_ref(self._h, x.data_ptr(), B, pr, out.data_ptr(),
                                      _stream(stream)),
               "asf_dense_ffn_ref")
        return out

    def step_launches(self, B: int = 1) -> int:
        """Kernel launches of one decode step for B tokens (list left out)."""
        return int(_lib.asf_step_launches(self._h, int(B)))

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
    layers; every layer must have the same d_model and device."""

    def __init__(self, layers, residual: bool = False):
        self.layers = list(layers)
        if not self.layers:
            raise ValueError("empty stack")
        self.d_model = self.layers[0].d_model
        self.device = self.layers[0].device
        for l in self.layers:
            if l.d_model != self.d_model or l.device != self.device:
                raise ValueError("every layer of a stack needs the same d_model and device")
        self.max_batch = min(l.max_batch for l in self.layers)
        self.residual = 1 if residual else 0
        self._arr = (_vp * len(self.layers))(*[l.handle for l in self.layers])
        self._work = {}

    def _work_for(self, B):
        w = self._work.get(B)
        if w is None:
            w = torch.empty((B, self.d_model), dtype=torch.float32, device=self.device)
            self._work[B] = w
        return w

    def _args(self, x, out, work, max_b):
        """x, out, work as [B][d_model] float32 on the stack's device."""
        x = _tokens(x, self.d_model, max_b)
        B = x.shape[0]
        shape = (B, self.d_model)
        _arg(out, "out", torch.float32, shape)
        _arg(work, "work", torch.float32, shape)
        _on_device(self.device, x=x, out=out, work=work)
        if out is None:
            out = torch.empty(shape, dtype=torch.float32, device=self.device)
        if work is None:
            work = self._work_for(B)
        return x, out, work

    def decode(self, x, out=None, work=None, stream=None):
        x, out, work = self._args(x, out, work, self.max_batch)
        _check(_lib.asf_stack_decode(self._arr, len(self.layers), x.data_ptr(), x.shape[0],
                                     self.residual, out.data_ptr(), work.data_ptr(),
                                     _stream(stream)),
               "asf_stack_decode")
        return out

    def decode_static(self, x, out, stream=None):
        """asf_stack_decode_static: as decode, with the buffer between layers
        in the library's static device array (the call allocates nothing;
        ``out`` is required for the same reason).  Calls that overlap on one
        GPU share that array and must be ordered by the caller."""
        if out is None:
            raise ValueError("decode_static needs out (it allocates nothing)")
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        _arg(out, "out", torch.float32, (B, self.d_model))
        _on_device(self.device, x=x, out=out)
        _check(_lib.asf_stack_decode_static(self._arr, len(self.layers), x.data_ptr(), B,
                                            self.residual, out.data_ptr(), _stream(stream)),
               "asf_stack_decode_static")
        return out

    def decode_lookahead(self, x, out=None, work=None, stream=None):
        """asf_stack_decode_lookahead: one token, layer l+1's set predicted
        from layer l's input, in the same launches as layer l's FFN."""
        x, out, work = self._args(x, out, work, 1)
        _check(_lib.asf_stack_decode_lookahead(self._arr, len(self.layers), x.data_ptr(),
                                               self.residual, out.data_ptr(), work.data_ptr(),
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


class HeadPredictor:
    """Attention-head predictor (asf_create_head_predictor): q1 [H][d],
    q2 [heads][H] device tensors (float16 or float32), c1 [H] and c2 [heads]
    float32 or None.  ``predict`` gives each token's selected heads."""

    def __init__(self, q1, q2, *, c1=None, c2=None, max_batch: int = 1,
                 threshold: float = 0.0, stream=None, storage: Optional[torch.Tensor] = None):
        if not isinstance(q1, torch.Tensor) or q1.dim() != 2:
            raise ValueError("q1 must be a [pred_hidden][d_model] tensor")
        if not isinstance(q2, torch.Tensor) or q2.dim() != 2:
            raise ValueError("q2 must be a [n_heads][pred_hidden] tensor")
        H, d = q1.shape
        nh = q2.shape[0]
        wt = _wtype(q1)
        self.d_model, self.n_heads, self.pred_hidden, self.max_batch = d, nh, H, max_batch
        self.words = (nh + 63) // 64
        self.device = q1.device
        w = HeadWeights(_arg(q1, "q1", q1.dtype, (H, d)), _arg(c1, "c1", torch.float32, (H,)),
                        _arg(q2, "q2", q1.dtype, (nh, H)), _arg(c2, "c2", torch.float32, (nh,)))
        self.desc = HeadDesc(d, nh, H, int(max_batch), wt, float(threshold))
        nbytes = int(_lib.asf_head_predictor_storage_bytes(ctypes.byref(self.desc)))
        if nbytes == 0:
            raise AsfError(2, "asf_head_predictor_storage_bytes")
        _arg(storage, "storage", torch.uint8, min_numel=nbytes)
        _on_device(None, q1=q1, c1=c1, q2=q2, c2=c2, storage=storage)
        if storage is None:
            storage = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.storage = storage
        handle = _vp()
        _check(_lib.asf_create_head_predictor(ctypes.byref(self.desc), ctypes.byref(w),
                                              storage.data_ptr(), storage.numel(),
                                              _stream(stream), ctypes.byref(handle)),
               "asf_create_head_predictor")
        self._h = handle.value

    @property
    def handle(self) -> int:
        return self._h

    def predict(self, x, masks=None, heads=None, counts=None, stream=None):
        """Returns (masks int64 [B][ceil(heads/64)], heads int32 [B][n_heads]
        (row b's first counts[b] entries are token b's heads, ascending),
        counts int32 [B]); outputs not given are allocated."""
        x = _tokens(x, self.d_model, self.max_batch)
        B = x.shape[0]
        _arg(masks, "masks", torch.int64, (B, self.words))
        _arg(heads, "heads", torch.int32, (B, self.n_heads))
        _arg(counts, "counts", torch.int32, (B,))
        _on_device(self.device, x=x, masks=masks, heads=heads, counts=counts)
        if masks is None:
            masks = torch.zeros((B, self.words), dtype=torch.int64, device=self.device)
        if heads is None:
            heads = torch.full((B, self.n_heads), -1, dtype=torch.int32, device=self.device)
        if counts is None:
            counts = torch.zeros(B, dtype=torch.int32, device=self.device)
        _check(_lib.asf_predict_heads(self._h, x.data_ptr(), B, masks.data_ptr(),
                                      heads.data_ptr(), counts.data_ptr(), _stream(stream)),
               "asf_predict_heads")
        return masks, heads, counts

    def predict_raw(self, x_ptr: int, B: int, masks_ptr, heads_ptr, counts_ptr,
                    stream_handle: int) -> None:
        """predict on raw device pointers (None skips an output)."""
        rc = _lib.asf_predict_heads(self._h, x_ptr, B, masks_ptr, heads_ptr, counts_ptr,
                                    stream_handle)
        if rc != ASF_OK:
            raise AsfError(rc, "asf_predict_heads")

    def close(self):
        if getattr(self, "_h", None):
            _lib.asf_destroy_head_predictor(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def head_predictor_from_numpy(P, device="cuda", max_batch: int = 1, threshold: float = 0.0,
                              stream=None) -> HeadPredictor:
    """Upload a host-side head predictor (workload.HeadPredictor-like) and create it."""
    def up(a):
        return None if a is None else torch.from_numpy(a).to(device)
    return HeadPredictor(up(P.q1), up(P.q2), c1=up(P.c1), c2=up(P.c2), max_batch=max_batch,
                         threshold=threshold, stream=stream)


def hot_first_table(counts, stream=None):
    """asf_hot_first_table: int32 [d_ffn] table (slot -> original id), most
    frequently active first, ties by smaller id, from device counts."""
    if not isinstance(counts, torch.Tensor) or counts.dim() != 1:
        raise ValueError("counts must be a 1-D int32 device tensor")
    f = counts.numel()
    pc = _arg(counts, "counts", torch.int32)
    _on_device(None, counts=counts)
    table = torch.empty(f, dtype=torch.int32, device=counts.device)
    _check(_lib.asf_hot_first_table(pc, f, table.data_ptr(), _stream(stream)),
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
