"""Thin ctypes binding of ``libmlp.so`` (C ABI in ``include/mlp.h``).

Argument marshalling only: torch tensors in, their device pointers and the
current HIP stream out to the library; every step of the path runs in the
library's HIP kernels.  PyTorch provides device memory (the workspace and the
tensors) and streams.  There is no fallback: if the shared library is missing
the import of this module fails.
"""
from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmlp.so")

MLP_OK, MLP_ERR_ARG, MLP_ERR_SHAPE, MLP_ERR_WORKSPACE, MLP_ERR_HIP, MLP_ERR_STATE, MLP_ERR_GUARD = range(7)
DEBUG_SYNC, DEBUG_GUARDS = 1, 2
MLP_F32, MLP_BF16 = 0, 1
STATE_ACT, STATE_MASK, STATE_DLOGITS, STATE_LOGITS = range(4)
OPT_SGD, OPT_ADAM, OPT_LAPROP = range(3)
OPTIMIZERS = {"sgd": OPT_SGD, "adam": OPT_ADAM, "laprop": OPT_LAPROP}

# Every entry point include/mlp.h declares: name -> (restype, argtypes).
_c = ctypes
SIGNATURES = {
    "mlp_abi_version": (_c.c_int32, []),
    "mlp_workspace_bytes": (_c.c_size_t, [_c.c_void_p]),
    "mlp_create": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.POINTER(_c.c_void_p)]),
    "mlp_destroy": (None, [_c.c_void_p]),
    "mlp_set_params": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_void_p]),
    "mlp_read_params": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_void_p]),
    "mlp_forward_probs": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p]),
    "mlp_forward": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                               _c.POINTER(_c.c_float)]),
    "mlp_train_step": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_float,
                                  _c.POINTER(_c.c_float)]),
    "mlp_train_step_async": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_float,
                                        _c.c_void_p]),
    "mlp_train_steps": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_void_p, _c.c_void_p, _c.c_float,
                                   _c.c_void_p]),
    "mlp_train_step_static": (_c.c_int, [_c.c_void_p, _c.POINTER(_c.c_void_p), _c.c_void_p, _c.c_void_p,
                                         _c.c_float, _c.c_void_p]),
    "mlp_grads": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.POINTER(_c.c_void_p),
                             _c.c_void_p, _c.POINTER(_c.c_float)]),
    "mlp_read_state": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_int32, _c.c_void_p]),
    "mlp_optimizer_bytes": (_c.c_size_t, [_c.c_void_p, _c.c_int32]),
    "mlp_checkpoint_bytes": (_c.c_size_t, [_c.c_void_p, _c.c_int32]),
    "mlp_save_checkpoint": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t, _c.c_int32]),
    "mlp_checkpoint_info": (_c.c_int, [_c.c_void_p, _c.c_size_t, _c.POINTER(_c.c_int32),
                                       _c.POINTER(_c.c_int32), _c.POINTER(_c.c_int32),
                                       _c.POINTER(_c.c_int64)]),
    "mlp_load_checkpoint": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_size_t]),
    "mlp_tune": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int32]),
    "mlp_set_optimizer": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_float, _c.c_float, _c.c_float,
                                     _c.c_void_p, _c.c_size_t]),
    "mlp_profile_enable": (_c.c_int, [_c.c_void_p, _c.c_int32]),
    "mlp_set_debug": (_c.c_int, [_c.c_void_p, _c.c_int32]),
    "mlp_profile_reset": (_c.c_int, [_c.c_void_p]),
    "mlp_profile_slots": (_c.c_int32, [_c.c_void_p]),
    "mlp_profile_read": (_c.c_int, [_c.c_void_p, _c.c_int32, _c.c_char_p, _c.c_size_t,
                                    _c.POINTER(_c.c_double), _c.POINTER(_c.c_int64),
                                    _c.POINTER(_c.c_double), _c.POINTER(_c.c_double)]),
    "mlp_status_string": (_c.c_char_p, [_c.c_int]),
    "mlp_last_error": (_c.c_char_p, [_c.c_void_p]),
}


STATIC_SCRATCH_BYTES = 64 << 20   # MLP_STATIC_SCRATCH_BYTES


def train_step_static(dims: Sequence[int], batch: int, weights: Sequence, x, labels, lr: float,
                      loss_dev=None, stream=None):
    """mlp_train_step_static: one float32 SGD step on the caller's weights
    (updated in place) with every intermediate in the library's static
    device buffer; enqueue only.  Tensors are contiguous float32 CUDA
    tensors; the stream defaults to torch's current one."""
    import torch
    dev = x.device
    st = stream if stream is not None else torch.cuda.current_stream(dev)
    cfg = make_config(dims, batch, MLP_F32, st.cuda_stream)
    arr = (ctypes.c_void_p * len(weights))(*[w.data_ptr() for w in weights])
    rc = lib().mlp_train_step_static(ctypes.byref(cfg), arr, ctypes.c_void_p(x.data_ptr()),
                                     ctypes.c_void_p(labels.data_ptr()), float(lr),
                                     ctypes.c_void_p(_ptr(loss_dev)))
    if rc != MLP_OK:
        raise MlpError(rc, lib().mlp_last_error(None).decode())


def checkpoint_info(buf: bytes) -> dict:
    """Header of a checkpoint held in host memory (no GPU work)."""
    n = ctypes.c_int32()
    dims = (ctypes.c_int32 * 17)()
    opt = ctypes.c_int32()
    step = ctypes.c_int64()
    cbuf = ctypes.create_string_buffer(bytes(buf), len(buf))
    st = lib().mlp_checkpoint_info(cbuf, len(buf), ctypes.byref(n), dims, ctypes.byref(opt), ctypes.byref(step))
    if st != MLP_OK:
        raise MlpError(st, lib().mlp_last_error(None).decode())
    return {"n_layers": n.value, "dims": list(dims[:n.value + 1]), "optimizer": opt.value, "step": step.value}


class MlpConfig(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32),
                ("dims", ctypes.POINTER(ctypes.c_int32)),
                ("batch", ctypes.c_int32),
                ("precision", ctypes.c_int32),
                ("stream", ctypes.c_void_p)]


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m mlp_gemm_softmax_amd.build`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_LIB: Optional[ctypes.CDLL] = None


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        _LIB = load_library()
    return _LIB


class MlpError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{lib().mlp_status_string(status).decode()}: {msg}")
        self.status = status


def make_config(dims: Sequence[int], batch: int, precision: int = MLP_F32, stream: int = 0):
    arr = (ctypes.c_int32 * len(dims))(*dims)
    cfg = MlpConfig(len(dims) - 1, arr, batch, precision, ctypes.c_void_p(stream))
    cfg._dims_keepalive = arr
    return cfg


def workspace_bytes(dims: Sequence[int], batch: int, precision: int = MLP_F32) -> int:
    cfg = make_config(dims, batch, precision)
    return int(lib().mlp_workspace_bytes(ctypes.byref(cfg)))


def _ptr(t) -> int:
    return 0 if t is None else int(t.data_ptr())


def debug_flags_from_env(value: str | None = None) -> int:
    """Debug modes named by the MLP_DEBUG environment variable (or `value`):
    a comma-separated list of ``sync`` (a wait after every launch) and
    ``guards`` (workspace guard bands checked after every call); empty or
    unset means none.  The library reads no environment itself: as the
    README's environment variables are resolved into a session's
    configuration at creation, this binding resolves MLP_DEBUG when it
    creates a session."""
    if value is None:
        value = os.environ.get("MLP_DEBUG", "")
    names = {"sync": DEBUG_SYNC, "guards": DEBUG_GUARDS}
    flags = 0
    for part in value.replace(" ", "").split(","):
        if not part:
            continue
        if part not in names:
            raise ValueError(f"MLP_DEBUG: unknown mode {part!r} (known: sync, guards)")
        flags |= names[part]
    return flags


class Mlp:
    """One static-shape MLP on one GPU: weights and scratch in a torch-owned
    workspace, steps enqueued on the given (default: current) torch stream.
    The debug modes MLP_DEBUG names are set on every new session."""

    def __init__(self, dims: Sequence[int], batch: int, precision: str = "f32",
                 device: str = "cuda", stream=None):
        import torch
        self.torch = torch
        self.dims = tuple(int(d) for d in dims)
        self.batch = int(batch)
        self.precision = precision
        self.device = torch.device(device)
        self.stream = stream if stream is not None else torch.cuda.current_stream(self.device)
        prec = MLP_BF16 if precision == "bf16" else MLP_F32
        self._cfg = make_config(self.dims, self.batch, prec, self.stream.cuda_stream)
        L = lib()
        nbytes = int(L.mlp_workspace_bytes(ctypes.byref(self._cfg)))
        if nbytes == 0:
            raise MlpError(MLP_ERR_SHAPE, L.mlp_last_error(None).decode())
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        handle = ctypes.c_void_p()
        st = L.mlp_create(ctypes.byref(self._cfg), ctypes.c_void_p(self.workspace.data_ptr()),
                          nbytes, ctypes.byref(handle))
        if st != MLP_OK:
            raise MlpError(st, L.mlp_last_error(None).decode())
        self._h = handle
        self._loss = ctypes.c_float(0.0)
        flags = debug_flags_from_env()
        if flags:
            self.set_debug(flags)

    # -- plumbing -------------------------------------------------------------
    def _handoff(self):
        """Order the caller's current stream after the work just enqueued on
        the session's stream, so tensors it filled can be used there."""
        cur = self.torch.cuda.current_stream(self.device)
        if cur != self.stream:
            cur.wait_stream(self.stream)

    def _check(self, st: int):
        if st != MLP_OK:
            raise MlpError(st, lib().mlp_last_error(self._h).decode())

    def close(self):
        if getattr(self, "_h", None):
            lib().mlp_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def n_layers(self) -> int:
        return len(self.dims) - 1

    def _dev_f32(self, t, shape):
        torch = self.torch
        if t.dtype != torch.float32 or t.device.type != "cuda" or not t.is_contiguous():
            raise ValueError("expected a contiguous float32 CUDA tensor")
        if tuple(t.shape) != tuple(shape):
            raise ValueError(f"expected shape {tuple(shape)}, got {tuple(t.shape)}")
        return t

    # -- entry points -----------------------------------------------------------
    def set_params(self, weights: Sequence):
        for l, w in enumerate(weights):
            self._dev_f32(w, (self.dims[l], self.dims[l + 1]))
            self._check(lib().mlp_set_params(self._h, l, ctypes.c_void_p(w.data_ptr())))

    def set_optimizer(self, rule: str = "sgd", beta1: float = 0.9, beta2: float = 0.999,
                      eps: float = 1e-8):
        """Update rule of later training steps; Adam/LaProp state (moments and a
        gradient buffer) lives in a torch-owned device buffer kept here."""
        opt = OPTIMIZERS[rule]
        state, nbytes = None, 0
        if opt != OPT_SGD:
            nbytes = int(lib().mlp_optimizer_bytes(ctypes.byref(self._cfg), opt))
            if nbytes == 0:
                raise MlpError(MLP_ERR_ARG, "no optimizer state size for this configuration")
            state = self.torch.empty(nbytes, dtype=self.torch.uint8, device=self.device)
        ptr = ctypes.c_void_p(state.data_ptr()) if state is not None else None
        self._check(lib().mlp_set_optimizer(self._h, opt, float(beta1), float(beta2), float(eps), ptr, nbytes))
        self.opt_state = state

    def checkpoint_bytes(self, with_optimizer: bool = True) -> int:
        return int(lib().mlp_checkpoint_bytes(self._h, 1 if with_optimizer else 0))

    def save_checkpoint(self, with_optimizer: bool = True, out=None):
        """Weights (and Adam/LaProp moments) as checkpoint bytes in host
        memory; with `out` (a contiguous uint8 CPU tensor, e.g. pinned, of at
        least checkpoint_bytes()) they are written there and `out` returned."""
        n = self.checkpoint_bytes(with_optimizer)
        if out is not None:
            if out.device.type != "cpu" or out.dtype != self.torch.uint8 or not out.is_contiguous() \
                    or out.numel() < n:
                raise ValueError(f"out must be a contiguous uint8 CPU tensor of at least {n} bytes")
            self._check(lib().mlp_save_checkpoint(self._h, ctypes.c_void_p(out.data_ptr()), n,
                                                  1 if with_optimizer else 0))
            return out
        buf = ctypes.create_string_buffer(n)
        self._check(lib().mlp_save_checkpoint(self._h, buf, n, 1 if with_optimizer else 0))
        return buf.raw

    def load_checkpoint(self, data):
        """Restore from checkpoint bytes, or from a contiguous uint8 CPU tensor."""
        if hasattr(data, "data_ptr"):
            if data.device.type != "cpu" or data.dtype != self.torch.uint8 or not data.is_contiguous():
                raise ValueError("expected checkpoint bytes or a contiguous uint8 CPU tensor")
            self._check(lib().mlp_load_checkpoint(self._h, ctypes.c_void_p(data.data_ptr()), data.numel()))
            return
        buf = ctypes.create_string_buffer(bytes(data), len(data))
        self._check(lib().mlp_load_checkpoint(self._h, buf, len(data)))

    def read_params(self) -> List:
        out = []
        for l in range(self.n_layers):
            t = self.torch.empty((self.dims[l], self.dims[l + 1]), dtype=self.torch.float32,
                                 device=self.device)
            self._check(lib().mlp_read_params(self._h, l, ctypes.c_void_p(t.data_ptr())))
            out.append(t)
        self._handoff()
        return out

    def forward(self, x, labels=None, want_loss: bool = True):
        B, C = self.batch, self.dims[-1]
        self._dev_f32(x, (B, self.dims[0]))
        if labels is not None:
            self._dev_f32(labels, (B, C))
        logits = self.torch.empty((B, C), dtype=self.torch.float32, device=self.device)
        loss_p = ctypes.byref(self._loss) if (labels is not None and want_loss) else None
        self._check(lib().mlp_forward(self._h, ctypes.c_void_p(x.data_ptr()),
                                      ctypes.c_void_p(logits.data_ptr()),
                                      ctypes.c_void_p(_ptr(labels)), loss_p))
        self._handoff()
        return logits, (self._loss.value if loss_p is not None else None)

    def tune(self, x, labels, repeats: int = 3):
        """Choose tile shapes and K splits by timing them on this batch."""
        self._dev_f32(x, (self.batch, self.dims[0]))
        self._dev_f32(labels, (self.batch, self.dims[-1]))
        self._check(lib().mlp_tune(self._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(labels.data_ptr()),
                                   int(repeats)))

    def forward_probs(self, x, probs=None):
        """Class probabilities of batch x (softmax of the logits); enqueue only."""
        B, C = self.batch, self.dims[-1]
        self._dev_f32(x, (B, self.dims[0]))
        if probs is None:
            probs = self.torch.empty((B, C), dtype=self.torch.float32, device=self.device)
        self._dev_f32(probs, (B, C))
        self._check(lib().mlp_forward_probs(self._h, ctypes.c_void_p(x.data_ptr()),
                                            ctypes.c_void_p(probs.data_ptr())))
        self._handoff()
        return probs

    def forward_async(self, x, logits):
        """Logits of batch x into the given device buffer; enqueue only."""
        self._check(lib().mlp_forward(self._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(logits.data_ptr()),
                                      None, None))

    def train_step(self, x, labels, lr: float) -> float:
        self._dev_f32(x, (self.batch, self.dims[0]))
        self._dev_f32(labels, (self.batch, self.dims[-1]))
        self._check(lib().mlp_train_step(self._h, ctypes.c_void_p(x.data_ptr()),
                                         ctypes.c_void_p(labels.data_ptr()), float(lr),
                                         ctypes.byref(self._loss)))
        return self._loss.value

    def train_step_async(self, x, labels, lr: float, loss_dev=None):
        self._check(lib().mlp_train_step_async(self._h, ctypes.c_void_p(x.data_ptr()),
                                               ctypes.c_void_p(labels.data_ptr()), float(lr),
                                               ctypes.c_void_p(_ptr(loss_dev))))

    def train_steps(self, x, labels, lr: float, loss_dev=None):
        """len(x) training steps on the batches x[s], labels[s]; enqueue
        only.  loss_dev: device float32 [n] or None."""
        n = int(x.shape[0]) if x.dim() == 3 else 0
        self._dev_f32(x, (n, self.batch, self.dims[0]))
        self._dev_f32(labels, (n, self.batch, self.dims[-1]))
        if loss_dev is not None:
            self._dev_f32(loss_dev, (n,))
        self._check(lib().mlp_train_steps(self._h, n, ctypes.c_void_p(x.data_ptr()),
                                          ctypes.c_void_p(labels.data_ptr()), float(lr),
                                          ctypes.c_void_p(_ptr(loss_dev))))

    def grads(self, x, labels):
        """(loss, [dW_l], dlogits) without an update."""
        torch = self.torch
        self._dev_f32(x, (self.batch, self.dims[0]))
        self._dev_f32(labels, (self.batch, self.dims[-1]))
        dws = [torch.empty((self.dims[l], self.dims[l + 1]), dtype=torch.float32, device=self.device)
               for l in range(self.n_layers)]
        arr = (ctypes.c_void_p * self.n_layers)(*[d.data_ptr() for d in dws])
        dl = torch.empty((self.batch, self.dims[-1]), dtype=torch.float32, device=self.device)
        self._check(lib().mlp_grads(self._h, ctypes.c_void_p(x.data_ptr()),
                                    ctypes.c_void_p(labels.data_ptr()), arr,
                                    ctypes.c_void_p(dl.data_ptr()), ctypes.byref(self._loss)))
        self._handoff()
        return self._loss.value, dws, dl

    def read_state(self, which: int, layer: int = 0):
        torch = self.torch
        if which in (STATE_ACT, STATE_MASK):
            shape = (self.batch, self.dims[layer])
            dtype = torch.float32 if which == STATE_ACT else torch.uint8
        else:
            shape = (self.batch, self.dims[-1])
            dtype = torch.float32
        t = torch.empty(shape, dtype=dtype, device=self.device)
        self._check(lib().mlp_read_state(self._h, which, layer, ctypes.c_void_p(t.data_ptr())))
        self._handoff()
        return t

    # -- debug modes ---------------------------------------------------------
    def set_debug(self, flags: int):
        """OR of DEBUG_SYNC (wait after every launch, name the failing one)
        and DEBUG_GUARDS (check the workspace's guard bands after every call
        that runs kernels); 0 turns both off."""
        self._check(lib().mlp_set_debug(self._h, int(flags)))

    # -- per-launch timing -----------------------------------------------------
    def profile(self, enable: bool = True):
        self._check(lib().mlp_profile_enable(self._h, 1 if enable else 0))

    def profile_reset(self):
        self._check(lib().mlp_profile_reset(self._h))

    def profile_read(self):
        L = lib()
        rows = []
        name = ctypes.create_string_buffer(128)
        for i in range(L.mlp_profile_slots(self._h)):
            ms, n, fl, by = ctypes.c_double(), ctypes.c_int64(), ctypes.c_double(), ctypes.c_double()
            self._check(L.mlp_profile_read(self._h, i, name, 128, ctypes.byref(ms), ctypes.byref(n),
                                           ctypes.byref(fl), ctypes.byref(by)))
            rows.append({"slot": i, "name": name.value.decode(), "total_ms": ms.value,
                         "launches": n.value, "flops": fl.value, "bytes": by.value})
        return rows

