"""MI355X-native compiled training step of a ReLU MLP (matmul -> ReLU ->
matmul -> softmax cross-entropy -> backward -> SGD).

The step runs in hand-written HIP kernels for gfx950 behind the C ABI in
``include/mlp.h`` (``libmlp.so``); ``mlp_gemm_softmax_amd.binding`` marshals
torch tensors into that ABI.  The binding is imported lazily so that the
seeded input generator (``synth``) works without the shared library.
"""
import importlib

__all__ = ["synth", "binding"]


def __getattr__(name):
    if name in ("binding", "synth", "build"):
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
