"""The checkpoint format that include/mlp.h documents, written out in Python
for the tests: a 136-byte little-endian header (magic "MLPCKPT1", version 1,
layer count, writer precision, update rule, 17 widths, beta1, beta2, eps,
two reserved words, step count, payload size, FNV-1a-64 checksum of the
payload), then every W_l as float32 [dims[l], dims[l+1]] row-major, then,
with an adaptive rule's state, every m_l and every v_l in the same shapes.
Independent of the library: the tests build checkpoints with it and decode
the library's checkpoints with it."""
import struct

import numpy as np

HEADER = struct.Struct("<8s4I17i3f2Iq2Q")
assert HEADER.size == 136


def fnv1a(data: bytes) -> int:
    """FNV-1a, 64-bit: offset basis 14695981039346656037, prime 1099511628211."""
    h = 1469598103934665603
    for b in data:
        h ^= b
        h = (h * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return h


def build(dims, Ws, m=None, v=None, opt=0, step=0, betas=(0.0, 0.0, 0.0), precision=0):
    """Checkpoint bytes of weights Ws (and moments m, v when given)."""
    parts = [np.ascontiguousarray(w, dtype="<f4") for w in Ws]
    if m is not None:
        parts += [np.ascontiguousarray(a, dtype="<f4") for a in m]
        parts += [np.ascontiguousarray(a, dtype="<f4") for a in v]
    payload = b"".join(p.tobytes() for p in parts)
    d = list(dims) + [0] * (17 - len(dims))
    head = HEADER.pack(b"MLPCKPT1", 1, len(dims) - 1, precision, opt, *d, *betas, 0, 0, step,
                       len(payload), fnv1a(payload))
    return head + payload


def parse(buf: bytes) -> dict:
    """Header fields and the payload's tensors of checkpoint bytes."""
    f = HEADER.unpack_from(buf, 0)
    magic, version, L, precision, opt = f[:5]
    dims = list(f[5:5 + L + 1])
    beta1, beta2, eps = f[22:25]
    reserved = f[25:27]
    step, nbytes, checksum = f[27:30]
    payload = buf[HEADER.size:]
    out = {"magic": magic, "version": version, "n_layers": L, "precision": precision, "optimizer": opt,
           "dims": dims, "unused_dims": list(f[5 + L + 1:22]), "betas": (beta1, beta2, eps),
           "reserved": reserved, "step": step, "payload_bytes": nbytes, "checksum": checksum,
           "payload_checksum": fnv1a(payload), "payload_len": len(payload)}
    off = 0
    tensors = []
    for _ in range(3 if opt else 1):
        for l in range(L):
            n = dims[l] * dims[l + 1]
            tensors.append(np.frombuffer(payload, dtype="<f4", count=n, offset=off).reshape(dims[l], dims[l + 1]))
            off += 4 * n
    out["W"] = tensors[:L]
    if opt:
        out["m"] = tensors[L:2 * L]
        out["v"] = tensors[2 * L:]
    out["trailing"] = len(payload) - off
    return out
