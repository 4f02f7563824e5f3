"""The checkpoint format that include/mlp.h documents, written out in Python
for the tests: a 136-byte little-endian header (magic "MLPCKPT1", version 2,
layer count, writer precision, update rule, 17 widths, beta1, beta2, eps,
two reserved words, step count, payload size, checksum of the payload),
then every W_l as float32 [dims[l], dims[l+1]] row-major, then, with an
adaptive rule's state, every m_l and every v_l in the same shapes.
Independent of the library: the tests build checkpoints with it and decode
the library's checkpoints with it."""
import struct

import numpy as np

HEADER = struct.Struct("<8s4I17i3f2Iq2Q")
assert HEADER.size == 136
VERSION = 2

FNV_BASIS = 0xcbf29ce484222325      # FNV-1a, 64-bit offset basis
FNV_PRIME = 0x100000001b3
MASK = (1 << 64) - 1


def fnv1a(data: bytes) -> int:
    """Byte-wise FNV-1a, 64-bit (Fowler, Noll and Vo)."""
    h = FNV_BASIS
    for b in data:
        h = ((h ^ b) * FNV_PRIME) & MASK
    return h


def checksum(payload: bytes) -> int:
    """The payload checksum of format version 2: little-endian 64-bit words
    (a last 4-byte remainder zero-extended), word i folded into lane i mod 4
    by h = (h ^ word) * prime from the FNV basis, then byte-wise FNV-1a over
    the four lanes' 32 little-endian bytes."""
    data = bytes(payload)
    data += b"\0" * (-len(data) % 8)
    words = np.frombuffer(data, dtype="<u8")
    full = len(words) // 4
    lanes = np.full(4, FNV_BASIS, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for row in words[:4 * full].reshape(full, 4):
            lanes = (lanes ^ row) * np.uint64(FNV_PRIME)
    lanes = [int(x) for x in lanes]
    for i in range(4 * full, len(words)):
        lanes[i % 4] = ((lanes[i % 4] ^ int(words[i])) * FNV_PRIME) & MASK
    return fnv1a(b"".join(x.to_bytes(8, "little") for x in lanes))


def build(dims, Ws, m=None, v=None, opt=0, step=0, betas=(0.0, 0.0, 0.0), precision=0):
    """Checkpoint bytes of weights Ws (and moments m, v when given)."""
    parts = [np.ascontiguousarray(w, dtype="<f4") for w in Ws]
    if m is not None:
        parts += [np.ascontiguousarray(a, dtype="<f4") for a in m]
        parts += [np.ascontiguousarray(a, dtype="<f4") for a in v]
    payload = b"".join(p.tobytes() for p in parts)
    d = list(dims) + [0] * (17 - len(dims))
    head = HEADER.pack(b"MLPCKPT1", VERSION, len(dims) - 1, precision, opt, *d, *betas, 0, 0, step,
                       len(payload), checksum(payload))
    return head + payload


def parse(buf: bytes) -> dict:
    """Header fields and the payload's tensors of checkpoint bytes."""
    f = HEADER.unpack_from(buf, 0)
    magic, version, L, precision, opt = f[:5]
    dims = list(f[5:5 + L + 1])
    beta1, beta2, eps = f[22:25]
    reserved = f[25:27]
    step, nbytes, stored_sum = f[27:30]
    payload = buf[HEADER.size:]
    out = {"magic": magic, "version": version, "n_layers": L, "precision": precision, "optimizer": opt,
           "dims": dims, "unused_dims": list(f[5 + L + 1:22]), "betas": (beta1, beta2, eps),
           "reserved": reserved, "step": step, "payload_bytes": nbytes, "checksum": stored_sum,
           "payload_checksum": checksum(payload), "payload_len": len(payload)}
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
