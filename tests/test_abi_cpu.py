"""Host-only checks of the C ABI: libmlp.so loads, exports every entry point
include/mlp.h declares, and rejects bad arguments in preflight (before any
HIP call, so these run without a GPU)."""
import ctypes
import os
import re

import pytest

from mlp_gemm_softmax_amd import binding
from mlp_gemm_softmax_amd.synth import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mlp.h")


def _lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libmlp.so not built (run __graft_entry__.build())")
    return binding.lib()


def declared_entry_points():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mlp_[a-z_]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_entry_points() == sorted(binding.SIGNATURES)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_entry_points():
        assert hasattr(lib, name), name
    assert lib.mlp_abi_version() == 1


def test_status_strings():
    lib = _lib()
    names = [lib.mlp_status_string(i).decode() for i in range(8)]
    assert names == ["MLP_OK", "MLP_ERR_ARG", "MLP_ERR_SHAPE", "MLP_ERR_WORKSPACE",
                     "MLP_ERR_HIP", "MLP_ERR_STATE", "MLP_ERR_GUARD", "MLP_ERR_UNKNOWN"]


def _cfg(dims, batch, precision=binding.MLP_F32):
    return binding.make_config(dims, batch, precision)


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_workspace_bytes_for_workloads(name):
    lib = _lib()
    w = WORKLOADS[name]
    prec = binding.MLP_BF16 if w.precision == "bf16" else binding.MLP_F32
    n = lib.mlp_workspace_bytes(ctypes.byref(_cfg(w.dims, w.batch, prec)))
    assert n > 0 and n % 256 == 0
    # at least the float32 weights, activations and logits
    weights = sum(4 * w.dims[i] * w.dims[i + 1] for i in range(len(w.dims) - 1))
    assert n >= weights + 4 * w.batch * w.dims[-1]


@pytest.mark.parametrize("dims,batch,prec", [
    ((), 4, 0),                       # no layers
    ((10,), 4, 0),
    ((10, 0, 3), 4, 0),               # zero width
    ((10, 5, 3), 0, 0),               # zero batch
    ((10, 5, 3), 4, 7),               # bad precision
    ((10, 1 << 21, 3), 4, 0),         # width beyond the limit
    (tuple([4] * 18), 4, 0),          # 17 layers > 16
    ((1 << 20, 1 << 20), 1, 0),       # 2^40-element weight
])
def test_invalid_configs_need_no_workspace(dims, batch, prec):
    lib = _lib()
    if len(dims) == 0:
        cfg = binding.MlpConfig(0, None, batch, prec, None)
    else:
        cfg = _cfg(dims, batch, prec)
    assert lib.mlp_workspace_bytes(ctypes.byref(cfg)) == 0
    h = ctypes.c_void_p()
    st = lib.mlp_create(ctypes.byref(cfg), ctypes.c_void_p(4096), 1 << 30, ctypes.byref(h))
    assert st in (binding.MLP_ERR_ARG, binding.MLP_ERR_SHAPE)
    assert not h.value
    assert lib.mlp_last_error(None).decode() != ""


def test_null_config_and_out():
    lib = _lib()
    h = ctypes.c_void_p()
    assert lib.mlp_workspace_bytes(None) == 0
    assert lib.mlp_create(None, ctypes.c_void_p(256), 1 << 20, ctypes.byref(h)) == binding.MLP_ERR_ARG
    cfg = _cfg((8, 4, 2), 2)
    assert lib.mlp_create(ctypes.byref(cfg), ctypes.c_void_p(256), 1 << 20, None) == binding.MLP_ERR_ARG


@pytest.mark.parametrize("ptr,delta", [(0, 0), (256 + 16, 0), (256, -256)])
def test_workspace_preflight(ptr, delta):
    """Null, misaligned or short workspaces fail before any device work."""
    lib = _lib()
    cfg = _cfg((784, 128, 10), 32)
    need = lib.mlp_workspace_bytes(ctypes.byref(cfg))
    h = ctypes.c_void_p()
    st = lib.mlp_create(ctypes.byref(cfg), ctypes.c_void_p(ptr), need + delta, ctypes.byref(h))
    assert st == binding.MLP_ERR_WORKSPACE
    assert "workspace" in lib.mlp_last_error(None).decode()


def _static_call(lib, dims, batch, prec=binding.MLP_F32, weights=True, x=4096, labels=4096, lr=0.1, loss=None):
    cfg = _cfg(dims, batch, prec)
    arr = (ctypes.c_void_p * (len(dims) - 1))(*([4096] * (len(dims) - 1))) if weights else None
    return lib.mlp_train_step_static(ctypes.byref(cfg), arr, ctypes.c_void_p(x), ctypes.c_void_p(labels),
                                     lr, ctypes.c_void_p(loss) if loss else None)


def test_static_step_preflight():
    """The allocation-free step rejects, before touching the GPU: bf16
    configurations, missing or misaligned pointers, a non-finite lr, and
    configurations whose scratch exceeds the static buffer."""
    lib = _lib()
    assert lib.mlp_train_step_static(None, None, None, None, 0.1, None) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 32, prec=binding.MLP_BF16) == binding.MLP_ERR_ARG
    assert "float32" in lib.mlp_last_error(None).decode()
    assert _static_call(lib, (784, 128, 10), 32, weights=False) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 32, x=4100) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 32, labels=0) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 32, lr=float("nan")) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 32, loss=4098) == binding.MLP_ERR_ARG
    assert _static_call(lib, (784, 128, 10), 0) == binding.MLP_ERR_SHAPE
    w = WORKLOADS["wide_f32"]
    assert _static_call(lib, w.dims, w.batch) == binding.MLP_ERR_WORKSPACE
    msg = lib.mlp_last_error(None).decode()
    assert "static buffer" in msg and str(binding.STATIC_SCRATCH_BYTES) in msg


def test_null_context_calls():
    lib = _lib()
    assert lib.mlp_set_params(None, 0, None) == binding.MLP_ERR_ARG
    assert lib.mlp_read_params(None, 0, None) == binding.MLP_ERR_ARG
    assert lib.mlp_forward(None, None, None, None, None) == binding.MLP_ERR_ARG
    assert lib.mlp_train_step(None, None, None, 0.1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_train_step_async(None, None, None, 0.1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_train_steps(None, 1, None, None, 0.1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_grads(None, None, None, None, None, None) == binding.MLP_ERR_ARG
    assert lib.mlp_read_state(None, 0, 1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_profile_enable(None, 1) == binding.MLP_ERR_ARG
    assert lib.mlp_set_debug(None, binding.DEBUG_SYNC) == binding.MLP_ERR_ARG
    assert lib.mlp_profile_slots(None) == 0
    lib.mlp_destroy(None)


# ------------------------------------------------------------- checkpoints --
# A checkpoint written here by hand from the format include/mlp.h documents
# (no GPU): the host-side check accepts it and rejects every damaged copy.

import struct

import numpy as np

from tests import ckpt_format


def _checkpoint(dims, opt=0, step=0, betas=(0.0, 0.0, 0.0), seed=0):
    rng = np.random.default_rng(seed)
    Ws = [rng.standard_normal((dims[l], dims[l + 1])).astype("<f4") for l in range(len(dims) - 1)]
    m = [np.abs(w) for w in Ws] if opt else None
    v = [w * w for w in Ws] if opt else None
    return ckpt_format.build(dims, Ws, m, v, opt=opt, step=step, betas=betas)


def test_checkpoint_info_reads_the_documented_format():
    _lib()
    buf = _checkpoint((5, 3, 2), opt=binding.OPT_ADAM, step=7, betas=(0.9, 0.999, 1e-8))
    info = binding.checkpoint_info(buf)
    assert info == {"n_layers": 2, "dims": [5, 3, 2], "optimizer": binding.OPT_ADAM, "step": 7}
    assert binding.checkpoint_info(_checkpoint((4, 4)))["optimizer"] == binding.OPT_SGD


def test_checkpoint_checksum_pins():
    """The format's checksum, pinned outside its own code: byte-wise FNV-1a-64
    against the published test vectors, and the four-lane fold on short
    payloads written out by hand (word i into lane i mod 4, a 4-byte tail
    zero-extended, then FNV-1a over the lanes' bytes)."""
    assert ckpt_format.fnv1a(b"") == 0xcbf29ce484222325
    assert ckpt_format.fnv1a(b"a") == 0xaf63dc4c8601ec8c
    assert ckpt_format.fnv1a(b"foobar") == 0x85944171f73967e8
    B, P, M = 0xcbf29ce484222325, 0x100000001b3, (1 << 64) - 1

    def fold(lanes):
        r = B
        for x in lanes:
            for k in range(8):
                r = ((r ^ ((x >> (8 * k)) & 0xFF)) * P) & M
        return r

    assert ckpt_format.checksum(b"") == fold([B, B, B, B])
    payload = bytes(range(1, 13))                       # 12 bytes: one word and a 4-byte tail
    w0 = int.from_bytes(payload[:8], "little")
    w1 = int.from_bytes(payload[8:] + b"\0\0\0\0", "little")
    assert ckpt_format.checksum(payload) == fold([((B ^ w0) * P) & M, ((B ^ w1) * P) & M, B, B])
    payload = bytes((7 * i + 3) & 0xFF for i in range(40))   # five words: lane 0 takes words 0 and 4
    w = [int.from_bytes(payload[8 * i:8 * i + 8], "little") for i in range(5)]
    lane0 = (((((B ^ w[0]) * P) & M) ^ w[4]) * P) & M
    assert ckpt_format.checksum(payload) == fold([lane0] + [((B ^ w[i]) * P) & M for i in (1, 2, 3)])
    # one flipped bit anywhere changes it
    base = ckpt_format.checksum(payload)
    for i in (0, 17, 39):
        bad = bytearray(payload)
        bad[i] ^= 0x10
        assert ckpt_format.checksum(bytes(bad)) != base


def _damaged():
    good = _checkpoint((6, 4, 3))
    yield "truncated header", good[:100]
    yield "truncated payload", good[:-4]
    yield "magic", b"X" + good[1:]
    yield "version 1 (another checksum)", good[:8] + struct.pack("<I", 1) + good[12:]
    yield "version 3", good[:8] + struct.pack("<I", 3) + good[12:]
    yield "layers", good[:12] + struct.pack("<I", 0) + good[16:]
    yield "rule", good[:20] + struct.pack("<I", 9) + good[24:]
    yield "width", good[:24] + struct.pack("<i", -1) + good[28:]
    yield "payload size", good[:120] + struct.pack("<Q", 8) + good[128:]
    flipped = bytearray(good)
    flipped[200] ^= 1
    yield "payload bit", bytes(flipped)


def test_checkpoint_info_survives_random_damage():
    """Seeded mutations of a valid checkpoint -- truncations, random bytes in
    the header and payload, random lengths and whole random buffers -- come
    back as MLP_OK (checksum and fields still consistent) or MLP_ERR_ARG,
    never anything else; under the host sanitizers (test_sanitizers_cpu.py)
    this also checks that the parser reads only the bytes it was given."""
    _lib()
    rng = np.random.default_rng([20, 26])
    good = _checkpoint((6, 4, 3), opt=binding.OPT_ADAM, step=3, betas=(0.9, 0.99, 1e-7))
    ok = 0
    for it in range(600):
        kind = it % 4
        b = bytearray(good)
        if kind == 0:
            b = b[: int(rng.integers(0, len(b)))]
        elif kind == 1:
            for _ in range(int(rng.integers(1, 6))):
                b[int(rng.integers(0, 136))] = int(rng.integers(0, 256))
        elif kind == 2:
            for _ in range(int(rng.integers(1, 6))):
                b[int(rng.integers(0, len(b)))] = int(rng.integers(0, 256))
        else:
            b = bytearray(rng.integers(0, 256, int(rng.integers(0, 400))).astype(np.uint8).tobytes())
            if len(b) >= 8 and rng.random() < 0.5:
                b[:8] = b"MLPCKPT1"
        try:
            binding.checkpoint_info(bytes(b))
            ok += 1
        except binding.MlpError as e:
            assert e.status == binding.MLP_ERR_ARG
    assert ok < 600


@pytest.mark.parametrize("what,buf", list(_damaged()))
def test_checkpoint_info_rejects_damage(what, buf):
    _lib()
    with pytest.raises(binding.MlpError) as ei:
        binding.checkpoint_info(buf)
    assert ei.value.status == binding.MLP_ERR_ARG, what


@pytest.mark.parametrize("value,flags", [("", 0), ("sync", binding.DEBUG_SYNC), ("guards", binding.DEBUG_GUARDS),
                                         ("sync,guards", binding.DEBUG_SYNC | binding.DEBUG_GUARDS),
                                         (" guards , sync ", binding.DEBUG_SYNC | binding.DEBUG_GUARDS)])
def test_debug_flags_from_env(value, flags):
    assert binding.debug_flags_from_env(value) == flags


def test_debug_flags_from_env_rejects_unknown_modes():
    with pytest.raises(ValueError):
        binding.debug_flags_from_env("sync,verbose")
