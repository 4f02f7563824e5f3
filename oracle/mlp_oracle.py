"""Float64 CPU oracle for one training step of the ReLU MLP.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may use it.  It shares no code with the
HIP implementation (no kernels, headers, helpers or constants).

What it computes is the plain definition of the step in the Meganeura README
("Example" section): ``h = relu(matmul(x, w1))``, ``logits = matmul(h, w2)``,
``loss = cross_entropy_loss(logits, labels)``, with the gradient the
framework's autodiff derives ("Example": autodiff happens inside
``build_session``) and a plain SGD update (README "Contents": SGD is one of
the optimizers a session can carry).  The arXiv abstract of "Meganeura:
Portable GPU Training and Inference through Vulkan and Metal" fixes the
evaluation protocol this oracle serves: a strict-f32 contract and a validated
fast-path contract, with forward and backward gated separately.

Notation (weights are [in, out], ``out = in @ W``, as in the README example):

    a_0 = x                                  [B, d_0]
    z_l = a_{l-1} W_l,  l = 1..L             [B, d_l]
    m_l = [z_l > 0],    a_l = z_l * m_l      l = 1..L-1 (ReLU, ReLU'(0) = 0)
    mu_b  = max_c z_L[b,c]
    lse_b = mu_b + log sum_c exp(z_L[b,c] - mu_b)
    s_b   = sum_c t[b,c]
    l_b   = s_b * lse_b - sum_c t[b,c] z_L[b,c]
    loss  = (1/B) sum_b l_b
    G_L   = (exp(z_L - lse) * s - t) / B     (dloss/dlogits)
    dW_l  = a_{l-1}^T G_l
    G_{l-1} = (G_l W_l^T) * m_{l-1}          (old W_l)
    W_l  <- W_l - lr * dW_l                  (after every dW_l is formed)

Readings where the pages are silent (each is also listed in the design
notes): no bias; dense labels with any non-negative rows (s_b = 1 for the
one-hot rows the workloads use, which gives (softmax - onehot)/B); mean over
the batch; the row max is subtracted before exponentiating; ReLU'(0) = 0;
SGD without momentum or decay; the loss returned is the one at the
pre-update weights.  Adam and LaProp, which the README names without
defining, follow their published algorithms (see ``adam`` and ``laprop``).

Every input is upcast to float64 first; nothing here rounds to float32 or
bfloat16, so the same oracle serves both contracts.

ReLU kinks.  Where |z| is within the rounding-error bound of a float32 (or
bfloat16-operand) evaluation, the sign of z -- and so the mask bit -- is not
determined by the inputs at working precision, and both mask values give a
correct derivative.  ``forward`` accepts an optional ``kink_choice`` per
hidden layer; the choice is honoured only inside that band (|z_l| <= e_l,
``mask_band``) and the function reports how many bits it took from the choice
and how many bits outside the band disagree with it.
"""
from __future__ import annotations

import math
from typing import Dict, List, Optional, Sequence

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# --------------------------------------------------------------------------
# Rounding-error bands for the mask tie-break.
#
# Rounding model of an evaluation at working precision (not of the oracle,
# which is float64):
#   * every float32 addition or multiplication of a dot product returns the
#     exact result times (1 + d), |d| <= U_ACC = 2^-23, one unit in the last
#     place: this holds for round-to-nearest and for truncation alike, since
#     the rounding inside a matrix-core accumulation is not specified;
#   * a bfloat16 operand is the float32 value times (1 + d), |d| <= U_BF16 =
#     2^-8, the unit roundoff of round-to-nearest-even to 8 significant bits;
#   * no underflow.
# Then (Higham, "Accuracy and Stability of Numerical Algorithms", 2nd ed.,
# section 3.1) a K-term dot product evaluated in any order is off by at most
# gamma_K * sum_k |a_k w_k|, gamma_K = K u / (1 - K u).
# --------------------------------------------------------------------------

U_ACC = 2.0 ** -23
U_BF16 = 2.0 ** -8


def gamma(k: int, u: float) -> float:
    """Higham's gamma_k = k u / (1 - k u): relative bound on a k-term
    floating-point dot product's error, in units of sum |a_i b_i|."""
    ku = k * u
    if ku >= 1.0:
        return math.inf
    return ku / (1.0 - ku)


def layer_error_factors(K: int, precision: str):
    """(c_own, c_in) of one layer z = a @ W with K = rows of W (the layer's
    input width):

        |z~ - z| <= c_own * (|a| @ |W|) + c_in * (|a~ - a| @ |W|)

    where a~ is the evaluation's own (already perturbed) input.  Float32:
    the dot product of a~ and W is off by gamma_K (|a~| @ |W|) <= gamma_K
    (|a| + |a~ - a|) @ |W|, and the input error adds (|a~ - a| @ |W|), so
    c_own = gamma_K, c_in = 1 + gamma_K.  bfloat16 operands: a^ = a~(1+s),
    W^ = W(1+t) with |s|, |t| <= U_BF16, so a^ W^ - a W = a W((1+s)(1+t) - 1)
    + (a~ - a) W (1+s)(1+t), and the float32 sum of the exact bf16 products
    adds gamma_K (1+U_BF16)^2 (|a| + |a~ - a|) @ |W|:
    c_own = 2 U_BF16 + U_BF16^2 + gamma_K (1+U_BF16)^2,
    c_in = (1+U_BF16)^2 (1+gamma_K)."""
    g = gamma(K, U_ACC)
    ub = U_BF16 if precision == "bf16" else 0.0
    return 2.0 * ub + ub * ub + g * (1.0 + ub) ** 2, (1.0 + ub) ** 2 * (1.0 + g)


def mask_band(a, W, err_in, precision: str):
    """Band e_l of one hidden layer: the elementwise bound

        e_l = c_own (|a| @ |W|) + c_in (err_in @ |W|)  >=  |z~_l - z_l|

    (``layer_error_factors``), with err_in the elementwise bound on
    |a~_{l-1} - a_{l-1}| (None for the input x, which both sides hold
    exactly).  Outside |z_l| <= e_l the evaluation's sign of z_l equals the
    exact one.  ``forward`` hands e_l on to the next layer where
    z_l > -e_l and 0 elsewhere: ReLU is 1-Lipschitz, and where z_l <= -e_l
    both sides give 0."""
    a = _f64(a)
    W = _f64(W)
    c_own, c_in = layer_error_factors(W.shape[0], precision)
    absW = np.abs(W)
    e = c_own * (np.abs(a) @ absW)
    if err_in is not None:
        e = e + c_in * (_f64(err_in) @ absW)
    return e


# --------------------------------------------------------------------------
# Forward: matmul -> ReLU -> ... -> matmul  (README "Example").
# --------------------------------------------------------------------------

def forward(x, weights: Sequence, kink_choice: Optional[Sequence] = None,
            precision: str = "f32") -> Dict:
    """Forward pass in float64.

    Returns a dict with ``a`` (a_0..a_{L-1}), ``z`` (z_1..z_L), ``m``
    (m_1..m_{L-1}, bool), ``logits`` (= z_L), and, when ``kink_choice`` is
    given, per hidden layer ``band`` (e_l of ``mask_band`` for an evaluation
    in ``precision``), ``in_band`` (units with |z_l| <= e_l), ``adopted``
    (bits taken from the choice inside the band, where it differs from
    [z_l > 0]) and ``outside`` (bits of the choice that differ from
    [z_l > 0] outside the band)."""
    W = [_f64(w) for w in weights]
    L = len(W)
    a = [_f64(x)]
    zs, ms, adopted, outside, bands, in_bands = [], [], [], [], [], []
    err = None
    for l in range(1, L + 1):
        z = a[-1] @ W[l - 1]
        zs.append(z)
        if l == L:
            break
        m = z > 0.0
        if kink_choice is not None:
            band = mask_band(a[-1], W[l - 1], err, precision)
            choice = np.asarray(kink_choice[l - 1]).astype(bool)
            in_band = np.abs(z) <= band
            differ = choice != m
            adopted.append(int(np.count_nonzero(differ & in_band)))
            outside.append(int(np.count_nonzero(differ & ~in_band)))
            in_bands.append(int(np.count_nonzero(in_band)))
            bands.append(band)
            m = np.where(in_band, choice, m)
            err = np.where(z > -band, band, 0.0)
        ms.append(m)
        a.append(z * m)
    out = {"a": a, "z": zs, "m": ms, "logits": zs[-1]}
    if kink_choice is not None:
        out["adopted"] = adopted
        out["outside"] = outside
        out["in_band"] = in_bands
        out["band"] = bands
    return out


# --------------------------------------------------------------------------
# Softmax cross-entropy against dense labels (README "Example":
# cross_entropy_loss(logits, labels) with labels of the logits' shape).
# --------------------------------------------------------------------------

def softmax_xent(logits, labels) -> Dict:
    """Mean softmax cross-entropy and its gradient w.r.t. the logits.

    Per row: mu = max z, lse = mu + log sum exp(z - mu), s = sum t,
    loss_b = s*lse - sum t*z; loss = mean_b loss_b; dlogits = (p*s - t)/B
    with p = exp(z - lse)."""
    z = _f64(logits)
    t = _f64(labels)
    B = z.shape[0]
    mu = z.max(axis=1, keepdims=True)
    ssum = np.exp(z - mu).sum(axis=1, keepdims=True)
    lse = mu + np.log(ssum)
    s = t.sum(axis=1, keepdims=True)
    rowloss = (s * lse)[:, 0] - (t * z).sum(axis=1)
    p = np.exp(z - lse)
    dlogits = (p * s - t) / B
    return {"loss": float(rowloss.mean()), "rowloss": rowloss,
            "dlogits": dlogits, "lse": lse[:, 0], "p": p}


def probabilities(logits) -> np.ndarray:
    """Class probabilities of each row for inference (the deployed forward of
    the README's train-to-deploy flow): the softmax that the loss above
    normalises with, p[b,c] = exp(z[b,c] - lse_b), lse_b = mu_b +
    log sum_c exp(z[b,c] - mu_b), mu_b = max_c z[b,c] (row max subtracted
    before exponentiating, as for the loss)."""
    z = _f64(logits)
    mu = z.max(axis=1, keepdims=True)
    lse = mu + np.log(np.exp(z - mu).sum(axis=1, keepdims=True))
    return np.exp(z - lse)


def forward_probabilities(x, weights: Sequence, kink_choice: Optional[Sequence] = None,
                          precision: str = "f32") -> Dict:
    """The forward pass followed by ``probabilities`` of its logits."""
    fwd = forward(x, weights, kink_choice=kink_choice, precision=precision)
    return {"fwd": fwd, "probs": probabilities(fwd["logits"])}


# --------------------------------------------------------------------------
# Backward (the derivative the README's autodiff produces for this graph).
# --------------------------------------------------------------------------

def backward(fwd: Dict, dlogits, weights: Sequence) -> Dict:
    """Gradients of the mean loss w.r.t. every W_l, at the given weights.

    dW_l = a_{l-1}^T G_l; G_{l-1} = (G_l W_l^T) * m_{l-1}."""
    W = [_f64(w) for w in weights]
    L = len(W)
    G = _f64(dlogits)
    dW = [None] * L
    Gs = [None] * (L + 1)
    Gs[L] = G
    for l in range(L, 0, -1):
        dW[l - 1] = fwd["a"][l - 1].T @ G
        if l > 1:
            G = (G @ W[l - 1].T) * fwd["m"][l - 2]
            Gs[l - 1] = G
    return {"dW": dW, "G": Gs}


def sgd(weights: Sequence, grads: Sequence, lr: float) -> List[np.ndarray]:
    """Plain SGD: W_l - lr * dW_l for every layer."""
    return [_f64(w) - float(lr) * _f64(g) for w, g in zip(weights, grads)]


def adam(weights: Sequence, grads: Sequence, m: Sequence, v: Sequence, t: int, lr: float,
         beta1: float, beta2: float, eps: float) -> Dict:
    """Adam, step t >= 1 (Kingma and Ba, "Adam: A Method for Stochastic
    Optimization", Algorithm 1; the pages name Adam among the optimizers a
    session can carry, README "Contents", without restating it).  Per element:

        m <- beta1 m + (1 - beta1) g
        v <- beta2 v + (1 - beta2) g^2
        W <- W - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)

    Returns {"W_new", "m", "v"} (float64 lists); m = v = 0 before step 1."""
    assert t >= 1
    c1 = 1.0 - float(beta1) ** t
    c2 = 1.0 - float(beta2) ** t
    W_new, m_new, v_new = [], [], []
    for w, g, m0, v0 in zip(weights, grads, m, v):
        g = _f64(g)
        m1 = beta1 * _f64(m0) + (1.0 - beta1) * g
        v1 = beta2 * _f64(v0) + (1.0 - beta2) * g * g
        W_new.append(_f64(w) - float(lr) * (m1 / c1) / (np.sqrt(v1 / c2) + eps))
        m_new.append(m1)
        v_new.append(v1)
    return {"W_new": W_new, "m": m_new, "v": v_new}


def laprop(weights: Sequence, grads: Sequence, m: Sequence, v: Sequence, t: int, lr: float,
           beta1: float, beta2: float, eps: float) -> Dict:
    """LaProp, step t >= 1 (Ziyin, Wang and Ueda, "LaProp: Separating Momentum
    and Adaptivity in Adam", Algorithm 1; named beside Adam in the README
    "Contents").  The gradient is divided by the bias-corrected root mean
    square before it enters the momentum:

        v <- beta2 v + (1 - beta2) g^2
        m <- beta1 m + (1 - beta1) g / (sqrt(v / (1 - beta2^t)) + eps)
        W <- W - lr * m / (1 - beta1^t)

    Returns {"W_new", "m", "v"} (float64 lists); m = v = 0 before step 1."""
    assert t >= 1
    c1 = 1.0 - float(beta1) ** t
    c2 = 1.0 - float(beta2) ** t
    W_new, m_new, v_new = [], [], []
    for w, g, m0, v0 in zip(weights, grads, m, v):
        g = _f64(g)
        v1 = beta2 * _f64(v0) + (1.0 - beta2) * g * g
        m1 = beta1 * _f64(m0) + (1.0 - beta1) * g / (np.sqrt(v1 / c2) + eps)
        W_new.append(_f64(w) - float(lr) * m1 / c1)
        m_new.append(m1)
        v_new.append(v1)
    return {"W_new": W_new, "m": m_new, "v": v_new}


OPTIMIZERS = {"adam": adam, "laprop": laprop}


# --------------------------------------------------------------------------
# One whole training step.
# --------------------------------------------------------------------------

def train_step(x, labels, weights: Sequence, lr: float,
               kink_choice: Optional[Sequence] = None, precision: str = "f32") -> Dict:
    """Forward, mean softmax-CE, backward and SGD for one batch.

    Returns loss (at the pre-update weights), dlogits, dW (per layer),
    W_new (per layer), and the forward dict under "fwd"."""
    fwd = forward(x, weights, kink_choice, precision)
    ce = softmax_xent(fwd["logits"], labels)
    bwd = backward(fwd, ce["dlogits"], weights)
    W_new = sgd(weights, bwd["dW"], lr)
    return {"loss": ce["loss"], "rowloss": ce["rowloss"],
            "dlogits": ce["dlogits"], "dW": bwd["dW"], "G": bwd["G"],
            "W_new": W_new, "fwd": fwd}

