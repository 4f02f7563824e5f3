"""Helpers for the GPU parity tests: run the HIP path through the C ABI and
compare it with the float64 oracle on the same seeded inputs.

Gates (strict f32 / bf16 fast path):
  loss       |L_gpu - L_ref| / |L_ref|              <= 1e-5 / 2e-2
  gradients  max|dW_gpu - dW_ref| <= tol * max|dW_ref|, per tensor (also dlogits)
  update     max|dW'_gpu - dW'_ref| <= tol * max|dW'_ref| + ulp(max|W|),  dW' = W' - W_old
  weights    max|W'_gpu - W'_ref| <= tol * max|W'_ref|
  masks      identical outside the rounding band of the oracle (inside it either
             value is a correct ReLU derivative and the oracle follows the GPU's);
             and, layer by layer, identical to the sign of the exact product of
             the GPU's own operands outside that product's float32 summation bound
"""
from __future__ import annotations

import numpy as np

from oracle import mlp_oracle

TOL = {"f32": 1e-5, "bf16": 2e-2}
GRAD_TOL = {"f32": 1e-4, "bf16": 2e-2}
# Fraction of a layer's hidden units whose mask bit may differ from the
# oracle's inside its rounding band.  Every such bit is a valid ReLU choice
# (the band is a worst-case bound), so the cap is a regression guard, set
# from measurement: on one MI355X the wide workload differs in 1 and 6 of
# 16.8M units per layer in float32 (3.6e-7) and in 12858 and 17816 with
# bf16 operands (7.7e-4, 1.06e-3); the small and ragged cases stay below
# 1.4e-3.  The caps sit at about 4x the largest of these (bf16) and well
# above them (f32, where a dozen units of a small layer are already 1e-4).
MAX_ADOPTED = {"f32": 1e-4, "bf16": 5e-3}

# Per-layer mask counts of every check, printed at the end of the test run
# (tests/conftest.py): label, layer, units, units in the oracle's band, bits
# adopted from the GPU there, bits differing outside it, units in the
# self-consistency band, bits differing there, bits differing outside it.
MASK_REPORT = []


def to_dev(arrs, dev):
    import torch
    return [torch.from_numpy(np.ascontiguousarray(a)).to(dev) for a in arrs]


def gpu_grads(net, x, t):
    """(loss, dW list, dlogits, masks) from mlp_grads + mlp_read_state."""
    from mlp_gemm_softmax_amd import binding
    loss, dws, dl = net.grads(x, t)
    masks = [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, net.n_layers)]
    return loss, [d.cpu().numpy() for d in dws], dl.cpu().numpy(), masks


def gpu_train(net, x, t, lr):
    from mlp_gemm_softmax_amd import binding
    loss = net.train_step(x, t, lr)
    masks = [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, net.n_layers)]
    return loss, [w.cpu().numpy() for w in net.read_params()], masks


def oracle_step(x, t, Ws, lr, dims, precision, masks):
    return mlp_oracle.train_step(x, t, Ws, lr, kink_choice=masks, precision=precision)


def gpu_acts(net):
    """The GPU's hidden activations a_1..a_{L-1} (float32; bf16 ones widened)."""
    from mlp_gemm_softmax_amd import binding
    return [net.read_state(binding.STATE_ACT, l).cpu().numpy() for l in range(1, net.n_layers)]


def rne_bf16(v):
    """float32 -> bfloat16 -> float32, round to nearest, ties to even
    (integer form: add 0x7fff plus the lowest kept bit, drop 16 bits)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def check_masks(ref, B, dims, precision, label="", limit_band=True, self_counts=None):
    """limit_band=False drops the cap on band adoptions (weights that left an
    integer lattice put many pre-activations next to 0 on purpose).
    self_counts: per-layer (in band, differing in band, differing outside)
    of ``check_mask_self_consistency``, for the report."""
    fwd = ref["fwd"]
    if len(dims) <= 2:
        return
    for l, (ad, out, ib) in enumerate(zip(fwd["adopted"], fwd["outside"], fwd["in_band"]), start=1):
        sc = self_counts[l - 1] if self_counts else (None, None, None)
        MASK_REPORT.append((label, l, B * dims[l], ib, ad, out) + tuple(sc))
        assert out == 0, f"{label} layer {l}: {out} mask bits differ outside the rounding band"
        frac = ad / float(B * dims[l])
        if limit_band:
            # a fraction cap, with a floor of two bits: a layer of a few dozen
            # units cannot adopt a fraction below one bit's share
            assert ad <= max(MAX_ADOPTED[precision] * B * dims[l], 2), \
                f"{label} layer {l}: {ad} band bits differ ({frac:.2e})"


def check_mask_self_consistency(x, Ws, masks, acts, precision, label=""):
    """Each hidden layer's mask against its own operands: the GPU forms
    z_l from x (layer 1) or its own a_{l-1}, and the operand copy of W_l
    (bf16-rounded in bf16 mode, as are x and the activations it stores), so
    its mask must equal [z > 0] of the exact product of those operands
    wherever |z| exceeds the float32 summation bound gamma_K (|a| @ |W|),
    gamma_K = K u / (1 - K u), u = 2^-23 (one ulp per operation, whatever the
    matrix cores' rounding).  Returns per layer (units in that band, bits
    differing inside it, bits differing outside it); asserts the last is 0."""
    bf16 = precision == "bf16"
    out = []
    a = np.asarray(x, np.float32)
    for l in range(1, len(Ws)):
        W = np.asarray(Ws[l - 1], np.float32)
        aop = (rne_bf16(a) if bf16 else a).astype(np.float64)
        Wop = (rne_bf16(W) if bf16 else W).astype(np.float64)
        K = W.shape[0]
        u = 2.0 ** -23
        g = K * u / (1.0 - K * u)
        z = aop @ Wop
        band = g * (np.abs(aop) @ np.abs(Wop))
        m = np.asarray(masks[l - 1]).astype(bool)
        in_band = np.abs(z) <= band
        differ = m != (z > 0)
        counts = (int(np.count_nonzero(in_band)), int(np.count_nonzero(differ & in_band)),
                  int(np.count_nonzero(differ & ~in_band)))
        assert counts[2] == 0, (f"{label} layer {l}: {counts[2]} mask bits disagree with the sign of the "
                                f"GPU's own operands' product outside its summation bound")
        out.append(counts)
        a = np.asarray(acts[l - 1], np.float32)
    return out


def rel_max(a, ref):
    a = np.asarray(a, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    err = np.max(np.abs(a - ref)) if a.size else 0.0
    return err, scale


def check_grads(loss, dws, dlogits, ref, precision, label=""):
    tol = TOL[precision]
    gtol = GRAD_TOL[precision]
    rel = abs(loss - ref["loss"]) / max(abs(ref["loss"]), 1e-30)
    assert rel <= tol, f"{label} loss {loss!r} vs {ref['loss']!r}: rel {rel:.3e} > {tol}"
    err, scale = rel_max(dlogits, ref["dlogits"])
    assert err <= gtol * scale, f"{label} dlogits: {err:.3e} > {gtol} * {scale:.3e}"
    for l, (g, r) in enumerate(zip(dws, ref["dW"])):
        err, scale = rel_max(g, r)
        assert err <= gtol * scale + 1e-30, f"{label} dW{l}: {err:.3e} > {gtol} * {scale:.3e}"


def check_update(loss, W_new, W_old, ref, precision, label=""):
    tol = TOL[precision]
    gtol = GRAD_TOL[precision]
    rel = abs(loss - ref["loss"]) / max(abs(ref["loss"]), 1e-30)
    assert rel <= tol, f"{label} loss {loss!r} vs {ref['loss']!r}: rel {rel:.3e} > {tol}"
    for l, (g, r, w0) in enumerate(zip(W_new, ref["W_new"], W_old)):
        w0 = np.asarray(w0, np.float64)
        err, scale = rel_max(g, r)
        assert err <= gtol * scale + 1e-30, f"{label} W'{l}: {err:.3e} > {gtol} * {scale:.3e}"
        d_gpu = np.asarray(g, np.float64) - w0
        d_ref = r - w0
        ulp = float(np.spacing(np.float32(max(np.max(np.abs(r)), np.max(np.abs(w0))))))
        err, scale = rel_max(d_gpu, d_ref)
        assert err <= gtol * scale + ulp, f"{label} dW'{l}: {err:.3e} > {gtol} * {scale:.3e} + {ulp:.1e}"


def check_fused_update_matches_grads(W_new, W_old, dws, lr):
    """The fused SGD epilogue equals fl32(W - fl32(lr*dW)) of the stored
    gradient (same kernel, same accumulation order) up to the rounding that
    separates a fused multiply-add from two rounded operations:
    |W'_gpu - fl32(W - fl32(lr*dW))| <= ulp(lr*dW)/2 + ulp(max(|W'_gpu|, |expect|))."""
    for l, (g, w0, dw) in enumerate(zip(W_new, W_old, dws)):
        step = (np.float32(lr) * np.float32(dw)).astype(np.float32)
        expect = (np.float32(w0) - step).astype(np.float32)
        bound = 0.5 * np.spacing(np.abs(step)).astype(np.float64) + \
            np.spacing(np.maximum(np.abs(expect), np.abs(g)).astype(np.float32)).astype(np.float64)
        bad = np.abs(g.astype(np.float64) - expect) > bound
        assert not np.any(bad), f"W'{l}: {int(bad.sum())} elements beyond the fma/two-rounding bound"


def _exact_everywhere(x, t, Ws, bf16):
    """True if every partial sum of the step is an integer (times 1/B for the
    backward) below 2^23, so that float32 arithmetic in any order is exact;
    with bf16 operands also every GEMM operand must fit 8 significant bits."""
    B = x.shape[0]
    r = mlp_oracle.train_step(x, t, Ws, 0.0)
    a = r["fwd"]["a"]
    G = r["G"]
    lim = 2.0 ** 23
    for l, W in enumerate(Ws):
        Wa = np.abs(np.asarray(W, np.float64))
        if np.max(np.abs(a[l]) @ Wa) >= lim:
            return False
        Gl = np.abs(G[l + 1]) * B
        if np.max(np.abs(a[l]).T @ Gl) >= lim:
            return False
        if l > 0 and np.max(Gl @ Wa.T) >= lim:
            return False
        if bf16:
            if np.max(np.abs(a[l])) > 256 or np.max(Wa) > 256 or np.max(Gl) > 256:
                return False
            if not np.all(Gl == np.round(Gl)):
                return False
    return True


def loss_sum_bound(rowloss):
    """Largest error of a float32 sum of the (integer) row losses in any order,
    before the exact division by B = 2^k: zero while every partial sum stays
    below 2^24, else the classical bound (B - 1) * 2^-24 * sum |l_b|."""
    s = float(np.sum(np.abs(np.asarray(rowloss, np.float64))))
    if s < 2.0 ** 24:
        return 0.0
    return (len(rowloss) - 1) * 2.0 ** -24 * s


def integer_problem(dims, B, seed, xmax=2, wmax=2, gap=50, bf16=False):
    """Integer-valued x and weights for which every product, partial sum,
    softmax and row loss of the step is exact in float32 (and in bf16
    operands; the mean of the row losses is exact only while their sum stays
    below 2^24, see loss_sum_bound):
    the last layer's column 0 beats every other column by gap * sum(a) >= 110
    per row, so softmax is exactly one-hot in float32 and dlogits =
    (e_0 - t)/B.  B must be a power of two."""
    assert B & (B - 1) == 0
    rng = np.random.default_rng([seed, 99])
    for _ in range(200):
        x = rng.integers(0, xmax + 1, (B, dims[0])).astype(np.float32)
        Ws = [rng.integers(-wmax, wmax + 1, (dims[l], dims[l + 1])).astype(np.float32)
              for l in range(len(dims) - 1)]
        WL = Ws[-1]
        WL[:, 0] = WL[:, 1:].max(axis=1) + gap if WL.shape[1] > 1 else gap
        a = x.astype(np.float64)
        for W in Ws[:-1]:
            a = np.maximum(a @ W, 0)
        if not np.all(a.sum(axis=1) * gap >= 110):
            continue
        ids = rng.integers(0, dims[-1], B)
        t = np.zeros((B, dims[-1]), np.float32)
        t[np.arange(B), ids] = 1.0
        if _exact_everywhere(x, t, Ws, bf16):
            return x, t, Ws
    raise RuntimeError("no exactly representable integer problem found")


# ------------------------------------------------ Adam / LaProp update gate --

def _f32_update_rounding(W, step):
    """A few float32 roundings of the update arithmetic and of W itself."""
    return 16 * 2.0 ** -24 * np.abs(step) + np.spacing(np.abs(W).astype(np.float32)).astype(np.float64)


class AdaptiveBound:
    """Per-element bound on |W_gpu - W_ref| along a trajectory of Adam or
    LaProp steps, derived from the update rule: every stored gradient may
    differ from the oracle's by at most dg (the gradient gate of the step),
    the bias-corrected moments are weighted means of the past gradients
    (weights summing to 1), so the first moment moves by at most
    max dg and the root of the second by at most max dg (Minkowski); the
    step lr * m_hat / (sqrt(v_hat) + eps) then moves by at most
    lr * (dm / (s' + eps) + |m_hat| ds / ((s' + eps)(s + eps))), s' = max(s -
    ds, 0); LaProp's momentum averages g / (s_i + eps) instead.  Errors add
    up over steps; float32 rounding of the update and of W is added per
    step.  Every quantity is the oracle's."""

    def __init__(self, rule, lr, b1, b2, eps, shapes):
        self.rule, self.lr, self.b1, self.b2, self.eps = rule, lr, b1, b2, eps
        self.t = 0
        self.gs, self.dgs = [], []
        self.acc = [np.zeros(s) for s in shapes]

    def step(self, g_ref, dg, W_new_ref, W_old_ref):
        self.t += 1
        t, b1, b2, eps = self.t, self.b1, self.b2, self.eps
        self.gs.append([np.asarray(g, np.float64) for g in g_ref])
        self.dgs.append(list(dg))
        c1, c2 = 1 - b1 ** t, 1 - b2 ** t
        out = []
        for l in range(len(self.acc)):
            w1 = [(1 - b1) * b1 ** (t - i) / c1 for i in range(1, t + 1)]
            u = [(1 - b2) * b2 ** (t - i) / c2 for i in range(1, t + 1)]
            gs = [self.gs[i][l] for i in range(t)]
            dgs = [self.dgs[i][l] for i in range(t)]
            vhat = sum(ui * g * g for ui, g in zip(u, gs))
            s = np.sqrt(vhat)
            ds = max(dgs)
            sp = np.maximum(s - ds, 0.0)
            if self.rule == "adam":
                mhat = sum(wi * g for wi, g in zip(w1, gs))
                dm = max(dgs)
                d = self.lr * (dm / (sp + eps) + np.abs(mhat) * ds / ((sp + eps) * (s + eps)))
            else:
                dm = 0.0
                for i in range(t):
                    ui = [(1 - b2) * b2 ** (i + 1 - k) / (1 - b2 ** (i + 1)) for k in range(1, i + 2)]
                    vi = sum(a * self.gs[k][l] ** 2 for a, k in zip(ui, range(i + 1)))
                    si = np.sqrt(vi)
                    dsi = max(self.dgs[k][l] for k in range(i + 1))
                    spi = np.maximum(si - dsi, 0.0)
                    dq = dgs[i] / (spi + eps) + np.abs(gs[i]) * dsi / ((spi + eps) * (si + eps))
                    dm = dm + w1[i] * dq
                d = self.lr * dm
            step_ref = np.asarray(W_new_ref[l], np.float64) - np.asarray(W_old_ref[l], np.float64)
            self.acc[l] = self.acc[l] + d + _f32_update_rounding(W_new_ref[l], step_ref)
            out.append(self.acc[l])
        return out


def check_adaptive(W_gpu, W_ref, bounds, label=""):
    for l, (g, r, b) in enumerate(zip(W_gpu, W_ref, bounds)):
        err = np.abs(np.asarray(g, np.float64) - np.asarray(r, np.float64))
        bad = err > b
        assert not np.any(bad), (f"{label} W{l}: {int(bad.sum())} elements beyond the derived bound; "
                                 f"worst excess {np.max(err - b):.3e}")
