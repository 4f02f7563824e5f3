"""Pins for the float64 oracle: values it must reproduce that do not come from
the oracle itself -- a hand-derived step, closed forms, invariants, central
finite differences, brute-force loops and a library special case -- plus
planted mistakes (mutants of the oracle) that at least one pin must catch."""
import math

import numpy as np
import pytest

from oracle import mlp_oracle as O
from mlp_gemm_softmax_amd import synth

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------- helpers --

def _rng(seed):
    return np.random.default_rng([1234, seed])


def _tiny_mlp(seed, dims=(6, 4, 3), B=2, soft=False, kink_guard=1e-3):
    """Random tiny MLP whose hidden pre-activations stay away from 0."""
    for attempt in range(1000):
        r = _rng(seed * 1000 + attempt)
        Ws = [r.uniform(-1, 1, (dims[i], dims[i + 1])) for i in range(len(dims) - 1)]
        x = r.standard_normal((B, dims[0]))
        if soft:
            t = r.uniform(0.1, 1.0, (B, dims[-1]))
        else:
            t = np.eye(dims[-1])[r.integers(0, dims[-1], B)]
        fwd = O.forward(x, Ws)
        if all(np.min(np.abs(z)) > kink_guard for z in fwd["z"][:-1]):
            return x, t, Ws
    raise RuntimeError("no kink-free draw")


def _fd_grads(step_fn, x, t, Ws, h=1e-6):
    """Central finite differences of the mean loss w.r.t. every weight."""
    out = []
    for l, W in enumerate(Ws):
        g = np.zeros_like(W)
        for idx in np.ndindex(W.shape):
            Wp = [w.copy() for w in Ws]
            Wm = [w.copy() for w in Ws]
            Wp[l][idx] += h
            Wm[l][idx] -= h
            g[idx] = (step_fn(x, t, Wp, 0.0)["loss"] - step_fn(x, t, Wm, 0.0)["loss"]) / (2 * h)
        out.append(g)
    return out


def _fd_max_rel(step_fn, x, t, Ws):
    res = step_fn(x, t, Ws, 0.0)
    fd = _fd_grads(step_fn, x, t, Ws)
    worst = 0.0
    for g_an, g_fd in zip(res["dW"], fd):
        scale = max(np.max(np.abs(g_fd)), 1e-12)
        worst = max(worst, np.max(np.abs(g_an - g_fd)) / scale)
    return worst


def _pins_pass(step_fn, golden):
    """Run the pins that a mutant could slip past; True if all hold."""
    try:
        g = golden("hand_worked_step.txt")
        x = np.array(g["x"]).reshape(1, 2)
        Ws = [np.array(g["W1"]).reshape(2, 2), np.array(g["W2"]).reshape(2, 2)]
        t = np.array(g["labels"]).reshape(1, 2)
        r = step_fn(x, t, Ws, g["lr"][0])
        ok = abs(r["loss"] - g["loss"][0]) < 1e-12
        ok &= np.allclose(r["dW"][0].ravel(), g["dW1"], atol=1e-12)
        ok &= np.allclose(r["dW"][1].ravel(), g["dW2"], atol=1e-12)
        ok &= np.allclose(r["W_new"][0].ravel(), g["W1_new"], atol=1e-12)
        ok &= np.allclose(r["W_new"][1].ravel(), g["W2_new"], atol=1e-12)
        for soft in (False, True):
            x, t, Ws = _tiny_mlp(3, soft=soft)
            ok &= _fd_max_rel(step_fn, x, t, Ws) < 1e-6
        return bool(ok)
    except Exception:
        return False


# ------------------------------------------------------------------- pins --

def test_hand_worked_step(golden):
    """Every quantity of a 2->2->2 step derived by hand (tests/golden)."""
    g = golden("hand_worked_step.txt")
    x = np.array(g["x"]).reshape(1, 2)
    Ws = [np.array(g["W1"]).reshape(2, 2), np.array(g["W2"]).reshape(2, 2)]
    t = np.array(g["labels"]).reshape(1, 2)
    r = O.train_step(x, t, Ws, g["lr"][0])
    np.testing.assert_allclose(r["fwd"]["z"][0].ravel(), g["z1"], atol=1e-14)
    np.testing.assert_array_equal(r["fwd"]["m"][0].ravel().astype(float), g["mask1"])
    np.testing.assert_allclose(r["fwd"]["logits"].ravel(), g["logits"], atol=1e-14)
    assert abs(r["loss"] - g["loss"][0]) < 1e-14
    np.testing.assert_allclose(r["dlogits"].ravel(), g["dlogits"], atol=1e-15)
    np.testing.assert_allclose(r["dW"][1].ravel(), g["dW2"], atol=1e-14)
    np.testing.assert_allclose(r["dW"][0].ravel(), g["dW1"], atol=1e-14)
    np.testing.assert_allclose(r["W_new"][0].ravel(), g["W1_new"], atol=1e-14)
    np.testing.assert_allclose(r["W_new"][1].ravel(), g["W2_new"], atol=1e-14)


@pytest.mark.parametrize("dims,B,key", [((784, 128, 10), 32, "log_C10"),
                                        ((64, 32, 1000), 5, "log_C1000"),
                                        ((16, 8, 4096), 3, "log_C4096")])
def test_zero_weights(golden, dims, B, key):
    """P1: zero weights -> loss = ln C, dlogits = (1/C - t)/B, all dW = 0,
    an SGD step leaves W unchanged."""
    C = dims[-1]
    x, t, _ = synth.make_batch(B, dims[0], C, "uniform01", seed=5)
    Ws = [np.zeros((dims[i], dims[i + 1])) for i in range(len(dims) - 1)]
    r = O.train_step(x, t, Ws, 0.1)
    assert abs(r["loss"] - golden("closed_forms.txt")[key][0]) < 1e-13
    np.testing.assert_allclose(r["dlogits"], (1.0 / C - t) / B, atol=1e-16)
    for dw, w_new in zip(r["dW"], r["W_new"]):
        assert np.all(dw == 0.0)
        assert np.all(w_new == 0.0)


def test_ce_closed_form_row(golden):
    """P3: z = (0, ln2, ln3), one-hot on index 2: p = (1/6,1/3,1/2), loss ln 2."""
    g = golden("closed_forms.txt")
    z = np.array([g["row_z"]])
    t = np.array([[0.0, 0.0, 1.0]])
    r = O.softmax_xent(z, t)
    assert abs(r["loss"] - g["row_loss"][0]) < 1e-15
    np.testing.assert_allclose(r["dlogits"][0], g["row_dlogits"], atol=1e-15)


def test_ce_soft_label_fixed_point():
    """P3: labels equal to softmax(z) give zero gradient; the loss is the
    entropy of the row."""
    r = _rng(2)
    z = r.standard_normal((4, 7))
    p = np.exp(z) / np.exp(z).sum(1, keepdims=True)
    out = O.softmax_xent(z, p)
    assert np.max(np.abs(out["dlogits"])) < 1e-16
    ent = -(p * np.log(p)).sum(1).mean()
    assert abs(out["loss"] - ent) < 1e-14


def test_ce_unnormalised_labels_scale():
    """Dense labels scaled by k scale the loss by k and the label part of the
    gradient accordingly: loss(k t) = k loss(t)."""
    r = _rng(9)
    z = r.standard_normal((3, 5))
    t = np.eye(5)[[1, 4, 0]]
    a = O.softmax_xent(z, t)
    b = O.softmax_xent(z, 2.5 * t)
    assert abs(b["loss"] - 2.5 * a["loss"]) < 1e-13
    np.testing.assert_allclose(b["dlogits"], 2.5 * a["dlogits"], atol=1e-15)


def test_dlogit_rows_sum_to_zero():
    """P2: each dlogits row sums to 0 for rows whose labels sum to 1."""
    for C in (10, 1000, 4096):
        x, t, _ = synth.make_batch(16, 8, C, "normal", seed=C)
        z = _rng(C).standard_normal((16, C)) * 3
        d = O.softmax_xent(z, t)["dlogits"]
        assert np.max(np.abs(d.sum(1))) < 1e-15


def test_ce_shift_invariance_and_overflow():
    """P4: adding a per-row constant (up to 1000) changes neither the loss
    nor dlogits, and produces no inf/NaN."""
    r = _rng(4)
    z = r.standard_normal((6, 9))
    t = np.eye(9)[r.integers(0, 9, 6)]
    base = O.softmax_xent(z, t)
    for c in (1.0, -50.0, 1000.0):
        shifted = O.softmax_xent(z + c * np.arange(1, 7)[:, None], t)
        assert np.isfinite(shifted["loss"])
        assert abs(shifted["loss"] - base["loss"]) < 1e-10
        np.testing.assert_allclose(shifted["dlogits"], base["dlogits"], atol=1e-14)


def _probs_pins_pass(fn, golden):
    """Pins of the inference probabilities: the closed-form row, a batch whose
    rows differ (catches a softmax over the wrong axis), rows summing to 1,
    shift invariance without overflow, and agreement with the p that the
    loss routine normalises with."""
    g = golden("closed_forms.txt")
    ok = True
    with np.errstate(all="ignore"):
        # z = (0, ln2, ln3): e^z = (1, 2, 3), p = (1/6, 1/3, 1/2)
        p = fn(np.array([g["row_z"]]))
        ok &= p.shape == (1, 3) and np.allclose(p[0], [1 / 6, 1 / 3, 1 / 2], rtol=0, atol=1e-15)
        # two rows: (0, ln2, ln3) and (ln3, 0, 0) -> (3/5, 1/5, 1/5)
        z2 = np.array([g["row_z"], [g["row_z"][2], 0.0, 0.0]])
        p2 = fn(z2)
        ok &= np.allclose(p2, [[1 / 6, 1 / 3, 1 / 2], [3 / 5, 1 / 5, 1 / 5]], rtol=0, atol=1e-15)
        r = _rng(31)
        z = r.standard_normal((8, 1000)) * 4
        p = fn(z)
        ok &= bool(np.all(p >= 0)) and np.max(np.abs(p.sum(1) - 1)) < 1e-13
        # z + 1000 is rounded to ulp(1000)/2 ~ 6e-14, which moves p by at most twice that
        shifted = fn(z + 1000.0)
        ok &= bool(np.all(np.isfinite(shifted))) and np.allclose(shifted, p, rtol=0, atol=1e-12)
        t = np.eye(1000)[r.integers(0, 1000, 8)]
        ok &= np.allclose(p, O.softmax_xent(z, t)["p"], rtol=0, atol=1e-15)
    return bool(ok)


def test_probabilities_pins(golden):
    assert _probs_pins_pass(O.probabilities, golden)


@pytest.mark.parametrize("kind", ["no_shift", "batch_axis", "no_exp", "unnormalised"])
def test_probabilities_pins_reject_planted_mistakes(golden, kind):
    def mutant(z):
        z = np.asarray(z, dtype=np.float64)
        if kind == "no_shift":
            return np.exp(z) / np.exp(z).sum(1, keepdims=True)
        if kind == "batch_axis":
            mu = z.max(0, keepdims=True)
            return np.exp(z - mu) / np.exp(z - mu).sum(0, keepdims=True)
        if kind == "no_exp":
            return z / z.sum(1, keepdims=True)
        return np.exp(z - z.max(1, keepdims=True))
    assert not _probs_pins_pass(mutant, golden)


def test_forward_probabilities_composes_forward_and_softmax():
    r = _rng(12)
    x = r.random((5, 6))
    Ws = [r.standard_normal((6, 4)), r.standard_normal((4, 3))]
    out = O.forward_probabilities(x, Ws)
    np.testing.assert_array_equal(out["probs"], O.probabilities(O.forward(x, Ws)["logits"]))


@pytest.mark.parametrize("soft", [False, True])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_finite_differences_tiny_mlp(seed, soft):
    """P5: central differences (h = 1e-6) on B=2, 6->4->3 agree with every
    one of the 36 analytic weight gradients to 1e-6 relative."""
    x, t, Ws = _tiny_mlp(seed, soft=soft)
    assert _fd_max_rel(O.train_step, x, t, Ws) < 1e-6


def test_finite_differences_three_layers():
    """P5 on a 3-weight-layer net (5->4->3->6, B=3): the G recursion through
    two masks."""
    x, t, Ws = _tiny_mlp(7, dims=(5, 4, 3, 6), B=3)
    assert _fd_max_rel(O.train_step, x, t, Ws) < 1e-6


def test_dlogits_finite_differences():
    """The loss derivative w.r.t. the logits themselves (dense labels)."""
    r = _rng(11)
    z = r.standard_normal((3, 4))
    t = r.uniform(0, 1, (3, 4))
    d = O.softmax_xent(z, t)["dlogits"]
    h = 1e-6
    for idx in np.ndindex(z.shape):
        zp, zm = z.copy(), z.copy()
        zp[idx] += h
        zm[idx] -= h
        fd = (O.softmax_xent(zp, t)["loss"] - O.softmax_xent(zm, t)["loss"]) / (2 * h)
        assert abs(fd - d[idx]) < 1e-8


def _loop_matmul(a, b):
    n, k = a.shape
    k2, m = b.shape
    assert k == k2
    c = np.zeros((n, m))
    for i in range(n):
        for j in range(m):
            s = 0.0
            for p in range(k):
                s += a[i, p] * b[p, j]
            c[i, j] = s
    return c


def test_brute_force_loops():
    """P6: forward and backward equal triple-loop products written out
    element by element (covers the NN, NT and TN products of the step)."""
    x, t, Ws = _tiny_mlp(5, dims=(5, 7, 3), B=4)
    r = O.train_step(x, t, Ws, 0.25)
    z1 = _loop_matmul(x, Ws[0])
    a1 = np.where(z1 > 0, z1, 0.0)
    z2 = _loop_matmul(a1, Ws[1])
    np.testing.assert_allclose(r["fwd"]["logits"], z2, rtol=1e-13, atol=1e-14)
    G2 = r["dlogits"]
    np.testing.assert_allclose(r["dW"][1], _loop_matmul(a1.T.copy(), G2), rtol=1e-12, atol=1e-15)
    G1 = _loop_matmul(G2, Ws[1].T.copy()) * (z1 > 0)
    np.testing.assert_allclose(r["dW"][0], _loop_matmul(x.T.copy(), G1), rtol=1e-12, atol=1e-15)
    for w, dw, wn in zip(Ws, r["dW"], r["W_new"]):
        np.testing.assert_array_equal(wn, w - 0.25 * dw)


def test_torch_cpu_autograd_special_case():
    """P6: torch's CPU float64 autograd with F.cross_entropy (probability
    targets) is a library special case of the same step."""
    torch = pytest.importorskip("torch")
    x, t, Ws = _tiny_mlp(8, dims=(12, 9, 5), B=6)
    r = O.train_step(x, t, Ws, 0.0)
    xt = torch.tensor(x)
    wt = [torch.tensor(w, requires_grad=True) for w in Ws]
    h = torch.relu(xt @ wt[0])
    logits = h @ wt[1]
    loss = torch.nn.functional.cross_entropy(logits, torch.tensor(t), reduction="mean")
    loss.backward()
    assert abs(loss.item() - r["loss"]) < 1e-13
    for w, dw in zip(wt, r["dW"]):
        np.testing.assert_allclose(w.grad.numpy(), dw, rtol=1e-11, atol=1e-14)


def test_sgd_descends():
    """P10 (sanity): on the README's MLP at batch 32, ten SGD steps at lr 0.1
    on one fixed batch bring the loss well below its starting value (x in
    [0,1) over 784 inputs makes lr 0.1 oscillate, so the fall is not
    monotone)."""
    w = synth.WORKLOADS["mnist_b32"]
    Ws = synth.workload_weights(w)
    x, t, _ = synth.workload_batch(w)
    losses = []
    for _ in range(10):
        r = O.train_step(x, t, Ws, w.lr)
        losses.append(r["loss"])
        Ws = r["W_new"]
    assert losses[-1] < 0.6 * losses[0]


def test_kink_tiebreak_only_inside_band():
    """The mask tie-break honours a choice only where |z| lies inside the
    rounding band, and counts disagreements outside it."""
    r = _rng(21)
    x = r.standard_normal((8, 16))
    Ws = [r.uniform(-1, 1, (16, 12)), r.uniform(-1, 1, (12, 3))]
    base = O.forward(x, Ws)
    z = base["z"][0]
    flipped = ~base["m"][0]
    betas = O.kink_betas((16, 12, 3), "f32")
    out = O.forward(x, Ws, kink_choice=[flipped], kink_beta=betas)
    band = betas[0] * (np.abs(x) @ np.abs(Ws[0]))
    assert out["adopted"][0] == int(np.count_nonzero(np.abs(z) <= band))
    assert out["outside"][0] == int(np.count_nonzero(np.abs(z) > band))
    np.testing.assert_array_equal(out["m"][0], base["m"][0])  # nothing in band here
    # Force one element into the band: the choice is then taken there.
    Ws2 = [w.copy() for w in Ws]
    Ws2[0][:, 0] *= 0.0
    out2 = O.forward(x, Ws2, kink_choice=[np.ones_like(flipped)], kink_beta=betas)
    assert np.all(out2["m"][0][:, 0])
    assert out2["adopted"][0] == 8


def test_gamma_bound():
    u = 2.0 ** -24
    assert O.gamma(1, u) == pytest.approx(u, rel=1e-6)
    assert O.gamma(4096, u) == pytest.approx(4096 * u / (1 - 4096 * u))
    assert O.gamma(2 ** 25, u) == math.inf


# ---------------------------------------------------------------- mutants --
# Each mutant plants one plausible mistake in a copy of the oracle; the pins
# above must reject every one of them.

def _mutant(kind):
    def step(x, t, Ws, lr):
        fwd = O.forward(x, Ws)
        if kind == "relu_inverted":
            fwd["m"] = [~m for m in fwd["m"]]
            fwd["a"] = [fwd["a"][0]] + [z * m for z, m in zip(fwd["z"][:-1], fwd["m"])]
            fwd["logits"] = fwd["a"][-1] @ np.asarray(Ws[-1], float)
        ce = O.softmax_xent(fwd["logits"], t)
        d = ce["dlogits"]
        loss = ce["loss"]
        if kind == "no_mean":
            d = d * x.shape[0]
        if kind == "no_label_sum":
            z = fwd["logits"]
            p = np.exp(z - ce["lse"][:, None])
            d = (p - t) / x.shape[0]
        if kind == "sign":
            d = -d
        W64 = [np.asarray(w, float) for w in Ws]
        L = len(W64)
        G = d
        dW = [None] * L
        for l in range(L, 0, -1):
            dW[l - 1] = fwd["a"][l - 1].T @ G
            if l > 1:
                if kind == "no_mask":
                    G = G @ W64[l - 1].T
                elif kind == "updated_weights":
                    G = (G @ (W64[l - 1] - lr * dW[l - 1]).T) * fwd["m"][l - 2]
                else:
                    G = (G @ W64[l - 1].T) * fwd["m"][l - 2]
        step_sign = -1.0 if kind != "sgd_sign" else 1.0
        W_new = [w + step_sign * lr * g for w, g in zip(W64, dW)]
        return {"loss": loss, "dW": dW, "W_new": W_new}
    return step


def test_pins_accept_the_oracle(golden):
    assert _pins_pass(O.train_step, golden)


@pytest.mark.parametrize("kind", ["relu_inverted", "no_mean", "no_label_sum", "sign",
                                  "no_mask", "updated_weights", "sgd_sign"])
def test_pins_reject_planted_mistakes(golden, kind):
    assert not _pins_pass(_mutant(kind), golden)


# ------------------------------------------------------ Adam / LaProp pins --
# Closed forms derived by hand from the published update rules (scalar
# sequences run through the oracle's per-element arithmetic as 1x1 layers),
# plus scale invariance; mutants of each rule must fail at least one pin.

def _run_opt(fn, gs, lr=0.1, b1=0.9, b2=0.999, eps=1e-8, w0=0.5):
    """W after each step of a scalar gradient sequence (float64)."""
    W = [np.array([[w0]])]
    m = [np.zeros((1, 1))]
    v = [np.zeros((1, 1))]
    out = []
    for t, g in enumerate(gs, start=1):
        r = fn(W, [np.array([[g]])], m, v, t, lr, b1, b2, eps)
        W, m, v = r["W_new"], r["m"], r["v"]
        out.append(float(W[0][0, 0]))
    return out


def _opt_pins_pass(fn, name):
    lr, b1, b2 = 0.1, 0.9, 0.999
    ok = True
    # first step, any gradient: bias-corrected moments are g and g^2, so the
    # step is lr * g / (|g| + eps) for both rules
    for g, eps in ((0.3, 1e-8), (-2.0, 0.5), (1e-9, 1e-8)):
        w1 = _run_opt(fn, [g], lr, b1, b2, eps)[0]
        ok &= abs((0.5 - w1) - lr * g / (abs(g) + eps)) < 1e-14
    # constant gradient: the bias corrections cancel the (1 - beta^t) growth
    # of both moments at every step
    ws = _run_opt(fn, [0.7] * 5, lr, b1, b2, 0.25)
    steps = np.diff([0.5] + ws)
    ok &= np.allclose(steps, -lr * 0.7 / 0.95, rtol=0, atol=1e-13)
    # +1 then -1 (eps = 0): v_hat_2 = 1 and m_hat_2 = -(1 - b1)/(1 + b1), so the
    # second step moves W up by lr (1 - b1)/(1 + b1) for both rules
    ws = _run_opt(fn, [1.0, -1.0], lr, b1, b2, 0.0)
    ok &= abs((ws[1] - ws[0]) - lr * (1 - b1) / (1 + b1)) < 1e-14
    # 2 then 1 (eps = 0): v_hat_2 = (4 b2 + 1)/(1 + b2);
    #   Adam:   m_hat_2 = (2 b1 + 1)/(1 + b1),   step = -lr m_hat_2 / sqrt(v_hat_2)
    #   LaProp: m_1 = 1 - b1, m_2 = b1 (1 - b1) + (1 - b1)/sqrt(v_hat_2),
    #           step = -lr m_2 / (1 - b1^2) = -lr (b1 + 1/sqrt(v_hat_2)) / (1 + b1)
    ws = _run_opt(fn, [2.0, 1.0], lr, b1, b2, 0.0)
    vh = (4 * b2 + 1) / (1 + b2)
    if name == "adam":
        want = -lr * (2 * b1 + 1) / (1 + b1) / math.sqrt(vh)
    else:
        want = -lr * (b1 + 1 / math.sqrt(vh)) / (1 + b1)
    ok &= abs((ws[1] - ws[0]) - want) < 1e-14
    # eps = 0: multiplying every gradient by c > 0 leaves every step unchanged
    r = _rng(77)
    gs = r.standard_normal(6)
    a = _run_opt(fn, list(gs), lr, b1, b2, 0.0)
    b = _run_opt(fn, list(37.0 * gs), lr, b1, b2, 0.0)
    ok &= np.allclose(a, b, rtol=0, atol=1e-13)
    return bool(ok)


@pytest.mark.parametrize("name", ["adam", "laprop"])
def test_optimizer_pins(name):
    assert _opt_pins_pass(O.OPTIMIZERS[name], name)


def test_optimizers_on_matrices_match_elementwise_rule():
    """The layer-wise update is the scalar rule applied to every element
    (checked against the scalar runs above on a 3x4 matrix, two steps)."""
    r = _rng(5)
    W = [r.standard_normal((3, 4))]
    g1, g2 = r.standard_normal((3, 4)), r.standard_normal((3, 4))
    for name, fn in O.OPTIMIZERS.items():
        z = [np.zeros((3, 4))]
        s1 = fn(W, [g1], z, z, 1, 0.01, 0.9, 0.99, 1e-3)
        s2 = fn(s1["W_new"], [g2], s1["m"], s1["v"], 2, 0.01, 0.9, 0.99, 1e-3)
        for idx in np.ndindex(3, 4):
            ws = _run_opt(fn, [g1[idx], g2[idx]], 0.01, 0.9, 0.99, 1e-3, w0=W[0][idx])
            assert abs(s2["W_new"][0][idx] - ws[1]) < 1e-14, (name, idx)


def _opt_mutant(name, kind):
    def fn(weights, grads, m, v, t, lr, b1, b2, eps):
        c1 = 1.0 - b1 ** t
        c2 = 1.0 - b2 ** t
        if kind == "no_bias_correction":
            c1 = c2 = 1.0
        if kind == "betas_swapped":
            b1, b2 = b2, b1
            c1, c2 = 1.0 - b1 ** t, 1.0 - b2 ** t
        W_new, m_new, v_new = [], [], []
        for w, g, m0, v0 in zip(weights, grads, m, v):
            g = np.asarray(g, float)
            if kind == "no_square":
                v1 = b2 * np.asarray(v0) + (1 - b2) * np.abs(g)
            else:
                v1 = b2 * np.asarray(v0) + (1 - b2) * g * g
            root = np.sqrt(v1 / c2) if kind != "no_sqrt" else v1 / c2
            if name == "adam":
                m1 = b1 * np.asarray(m0) + (1 - b1) * g
                W_new.append(np.asarray(w) - lr * (m1 / c1) / (root + eps))
            else:
                m1 = b1 * np.asarray(m0) + (1 - b1) * g / (root + eps)
                W_new.append(np.asarray(w) - lr * m1 / c1)
            m_new.append(m1)
            v_new.append(v1)
        return {"W_new": W_new, "m": m_new, "v": v_new}
    return fn


@pytest.mark.parametrize("name", ["adam", "laprop"])
@pytest.mark.parametrize("kind", ["no_bias_correction", "betas_swapped", "no_square", "no_sqrt"])
def test_optimizer_pins_reject_planted_mistakes(name, kind):
    assert _opt_pins_pass(_opt_mutant(name, "none"), name)   # the harness itself is faithful
    assert not _opt_pins_pass(_opt_mutant(name, kind), name)


def test_adam_and_laprop_differ():
    """The two rules part ways as soon as the gradient scale changes."""
    a = _run_opt(O.adam, [2.0, 1.0], eps=0.0)
    b = _run_opt(O.laprop, [2.0, 1.0], eps=0.0)
    assert abs(a[1] - b[1]) > 1e-3
