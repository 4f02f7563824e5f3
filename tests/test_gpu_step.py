"""GPU parity of the HIP training step against the float64 oracle, through
the C ABI (libmlp.so via the ctypes binding)."""
import ctypes
import math

import numpy as np
import pytest

from mlp_gemm_softmax_amd import synth
from oracle import mlp_oracle
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def make_net(dims, B, precision, Ws, dev):
    from mlp_gemm_softmax_amd import binding
    net = binding.Mlp(dims, B, precision, device=str(dev))
    net.set_params(P.to_dev(Ws, dev))
    return net


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


# --------------------------------------------------------------- exactness --

EXACT_CASES = [
    # dims, B, precision
    # dims, B, precision, operand range
    ((200, 300, 36), 64, "f32", 2),          # ragged tiles, split-K in dW
    ((96, 160, 130, 40), 128, "f32", 1),     # three layers, two masks
    ((784, 128, 16), 32, "f32", 2),          # the README MLP's widths, 32x128 tiles
    ((256, 520, 64), 8, "f32", 2),           # skinny-batch kernels, ragged columns
    ((1024, 1100, 260), 16, "f32", 1),       # skinny-batch with K splits
    ((64, 100, 1040), 8, "f32", 1),          # skinny dX + dW with its columns split, ragged rows and split
    ((320, 2080, 40), 512, "f32", 1),        # tiled NN with split-K, ragged N
    ((2080, 1040, 40), 512, "f32", 1),       # tiled TN and NT with split-K, ragged tiles
    ((64, 32, 8), 8, "f32", 2),              # fused output layer with skinny kernels, tail on its own
    ((512, 2048, 16), 1024, "f32", 1),       # fused output layer with tiled GEMMs, tail on its own
    ((1024, 2048, 1040), 2048, "f32", 1),    # f32 256x256 tiles: K splits, split logits into the loss, ragged N
    ((2056, 4096, 1024), 2048, "f32", 1),    # f32 256x256 tiles in all three layouts, ragged K and M
    ((200, 300, 36), 64, "bf16", 1),
    ((120, 136, 24), 256, "bf16", 1),
    ((256, 4096, 40), 2048, "bf16", 1),      # 256-wide bf16 tiles, no split (forward)
    ((2056, 4096, 1024), 2048, "bf16", 1),   # 256-wide bf16 tiles in all three layouts, ragged K and M, 4-way K split
    ((2056, 2048, 1024), 2048, "bf16", 1),   # 256-wide bf16 tiles, 2- and 4-way K splits
]


def _check_exact_loss(loss, ref, B):
    """The mean loss: bitwise while the row-loss sum is representable, else
    within the summation bound of that sum (the division by B = 2^k is exact)."""
    bound = P.loss_sum_bound(ref["rowloss"]) / B
    if bound == 0.0:
        assert np.float32(loss) == np.float32(ref["loss"])
    else:
        assert abs(float(loss) - ref["loss"]) <= bound + float(np.spacing(np.float32(ref["loss"])))


@pytest.mark.parametrize("dims,B,precision,vmax", EXACT_CASES)
def test_exact_integer_step_is_bitwise(torch_dev, dims, B, precision, vmax):
    """P7: integer operands make every product, sum, softmax, row loss and
    update exact, so the GPU must equal the float32-rounded oracle bit for
    bit, whatever its tiling, split-K or summation order (the mean loss too,
    while the row losses sum below 2^24)."""
    torch, dev = torch_dev
    _announce(f"exact dims={dims} B={B} {precision}")
    x, t, Ws = P.integer_problem(dims, B, seed=len(dims) * 1000 + B, xmax=vmax, wmax=vmax,
                                 bf16=precision == "bf16")
    lr = 0.0625
    ref = mlp_oracle.train_step(x, t, Ws, lr)
    net = make_net(dims, B, precision, Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    loss, dws, dl, masks = P.gpu_grads(net, xd, td)
    logits, _ = net.forward(xd)
    _check_exact_loss(loss, ref, B)
    np.testing.assert_array_equal(logits.cpu().numpy(), ref["fwd"]["logits"].astype(np.float32))
    np.testing.assert_array_equal(dl, ref["dlogits"].astype(np.float32))
    for m_gpu, m_ref in zip(masks, ref["fwd"]["m"]):
        np.testing.assert_array_equal(m_gpu.astype(bool), m_ref)
    for g, r in zip(dws, ref["dW"]):
        np.testing.assert_array_equal(g, r.astype(np.float32))
    loss2, W_new, _ = P.gpu_train(net, xd, td, lr)
    _check_exact_loss(loss2, ref, B)
    for g, r in zip(W_new, ref["W_new"]):
        np.testing.assert_array_equal(g, r.astype(np.float32))
    net.close()


# ------------------------------------------------------ workload parity ----

def _workload_parity(torch_dev, name, steps_to_check=(0,)):
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    prec = w.precision
    Ws = synth.workload_weights(w)
    _announce(f"workload {name} dims={w.dims} B={w.batch} {prec}")
    net = make_net(w.dims, w.batch, prec, Ws, dev)
    x, t, _ = synth.workload_batch(w, 0)
    xd, td = P.to_dev([x, t], dev)
    # gradients, no update
    loss, dws, dl, masks = P.gpu_grads(net, xd, td)
    sc = P.check_mask_self_consistency(x, Ws, masks, P.gpu_acts(net), prec, name)
    ref = P.oracle_step(x, t, Ws, w.lr, w.dims, prec, masks)
    P.check_masks(ref, w.batch, w.dims, prec, name, self_counts=sc)
    P.check_grads(loss, dws, dl, ref, prec, name)
    # fused update from the same weights
    loss2, W_new, masks2 = P.gpu_train(net, xd, td, w.lr)
    P.check_mask_self_consistency(x, Ws, masks2, P.gpu_acts(net), prec, name)
    ref2 = P.oracle_step(x, t, Ws, w.lr, w.dims, prec, masks2)
    P.check_update(loss2, W_new, Ws, ref2, prec, name)
    P.check_fused_update_matches_grads(W_new, Ws, dws, w.lr)
    net.close()


def test_parity_mnist_b32(torch_dev):
    _workload_parity(torch_dev, "mnist_b32")


def test_parity_mnist_b1024(torch_dev):
    _workload_parity(torch_dev, "mnist_b1024")


def test_parity_wide_f32(torch_dev):
    _workload_parity(torch_dev, "wide_f32")


def test_parity_wide_bf16(torch_dev):
    _workload_parity(torch_dev, "wide_bf16")


def test_parity_skinny_b8(torch_dev):
    _workload_parity(torch_dev, "skinny_b8")


def test_parity_skinny_b8_tp8_shard(torch_dev):
    """One GPU's share of the skinny workload under 8-way tensor parallelism
    (the per-GPU kernels at their real shapes)."""
    _workload_parity(torch_dev, "skinny_b8_tp8_shard")


# ------------------------------------------------- multi-step trajectories --

def _oracle_trajectory(w, Ws, steps):
    """Oracle states W_s (rounded to float32 after every step, so that each
    one is a valid GPU input) and the oracle's loss at each step."""
    states, losses = [], []
    cur = [np.asarray(a, np.float32) for a in Ws]
    for s in range(steps):
        states.append(cur)
        x, t, _ = synth.workload_batch(w, s)
        r = mlp_oracle.train_step(x, t, cur, w.lr)
        losses.append(r["loss"])
        cur = [a.astype(np.float32) for a in r["W_new"]]
    return states, losses


@pytest.mark.parametrize("name,checked", [("mnist_b32", range(10)),
                                          ("mnist_b1024", (0, 1, 49, 99))])
def test_oracle_forced_steps(torch_dev, name, checked):
    """Multi-step parity: at each checked step s the GPU starts from the
    oracle's own (float32-rounded) state W_s and must reproduce the oracle's
    step s at the strict gates."""
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    states, _ = _oracle_trajectory(w, synth.workload_weights(w), max(checked) + 1)
    net = make_net(w.dims, w.batch, "f32", states[0], dev)
    for s in checked:
        _announce(f"{name} forced step {s}")
        net.set_params(P.to_dev(states[s], dev))
        x, t, _ = synth.workload_batch(w, s)
        xd, td = P.to_dev([x, t], dev)
        loss, W_new, masks = P.gpu_train(net, xd, td, w.lr)
        ref = P.oracle_step(x, t, states[s], w.lr, w.dims, "f32", masks)
        P.check_masks(ref, w.batch, w.dims, "f32", f"{name}@{s}")
        P.check_update(loss, W_new, states[s], ref, "f32", f"{name}@{s}")
    net.close()


@pytest.mark.parametrize("name,steps,tol", [("mnist_b32", 10, 1e-3), ("mnist_b1024", 100, 1e-2)])
def test_free_running_loss_curve(torch_dev, name, steps, tol):
    """The GPU's own trajectory (its updated weights feed the next step)
    tracks the oracle's loss curve.  Not bit-reproducible across
    implementations, so the gate is a loose relative bound per step."""
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    Ws = synth.workload_weights(w)
    _, ref_losses = _oracle_trajectory(w, Ws, steps)
    net = make_net(w.dims, w.batch, "f32", Ws, dev)
    batches = [P.to_dev(synth.workload_batch(w, s)[:2], dev) for s in range(steps)]
    losses = [net.train_step(b[0], b[1], w.lr) for b in batches]
    for s, (g, r) in enumerate(zip(losses, ref_losses)):
        assert abs(g - r) <= tol * abs(r), f"step {s}: {g} vs {r}"
    net.close()


# --------------------------------------------------------- ragged / edges --

EDGE_CASES = [
    ((33, 70, 17, 10), 37, "f32"),
    ((100, 31, 7), 5, "f32"),        # small batch, widths not multiples of 4
    ((64, 260, 36), 12, "f32"),      # skinny kernels, ragged columns
    ((1, 1, 1), 1, "f32"),           # one class: loss 0
    ((5, 3), 3, "f32"),              # no hidden layer
    ((128, 10), 300, "f32"),
    ((784, 128, 10), 7, "f32"),
    ((4100, 64, 8), 16, "f32"),      # skinny, many K splits
    ((2052, 36, 20), 3, "f32"),      # skinny, batch <= 4, ragged last K chunk, one column group
    ((8, 1028, 12), 16, "f32"),      # skinny, K shorter than one wave's rows, 4-column last group
    ((33, 70, 17, 10), 37, "bf16"),
    ((100, 31, 7), 5, "bf16"),
    ((72, 200, 1000), 48, "bf16"),
    ((1 << 20, 8), 2, "f32"),        # a 2^20-wide input: long K splits in the skinny forward
    ((16, 16), 1 << 17, "f32"),      # 2^17 rows: long dW reduction, wide grids
    ((64, 64), 1 << 17, "bf16"),
]


@pytest.mark.parametrize("dims,B,precision", EDGE_CASES)
def test_edge_shapes(torch_dev, dims, B, precision):
    torch, dev = torch_dev
    _announce(f"edge dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=sum(dims) + B)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=B, step=len(dims))
    lr = 0.05
    net = make_net(dims, B, precision, Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    loss, dws, dl, masks = P.gpu_grads(net, xd, td)
    sc = P.check_mask_self_consistency(x, Ws, masks, P.gpu_acts(net), precision, str(dims))
    ref = P.oracle_step(x, t, Ws, lr, dims, precision, masks)
    P.check_masks(ref, B, dims, precision, str(dims), self_counts=sc)
    if dims[-1] == 1:
        assert loss == 0.0 and np.all(dl == 0.0)
    P.check_grads(loss, dws, dl, ref, precision, str(dims))
    loss2, W_new, masks2 = P.gpu_train(net, xd, td, lr)
    ref2 = P.oracle_step(x, t, Ws, lr, dims, precision, masks2)
    P.check_update(loss2, W_new, Ws, ref2, precision, str(dims))
    net.close()


def _sweep_cases():
    """Seeded draws of small shapes from the widths kernels treat specially
    (1, odd, one less or more than a tile edge, the MNIST widths, a skinny
    multiple of 4) and batches from 1 to 40: every kernel family meets ragged
    edges at several of its branch points."""
    rng = np.random.default_rng([2026, 12])
    widths = [1, 4, 7, 8, 10, 16, 31, 33, 64, 100, 128, 260]
    batches = [1, 2, 3, 7, 8, 12, 16, 17, 33, 40]
    cases = []
    for k in range(40):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice(batches))
        precision = "bf16" if k % 4 == 3 else "f32"
        cases.append((dims, B, precision))
    return cases


def _sweep_cases_medium():
    """Seeded medium shapes: tiled, split-K and large-tile plans with ragged
    tiles, the fused output layer, and skinny batches with K splits."""
    rng = np.random.default_rng([2026, 13])
    widths = [12, 36, 96, 200, 300, 520, 784, 1000, 1040, 2056]
    batches = [5, 8, 16, 64, 128, 300, 512, 1024]
    cases = []
    for k in range(24):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice(batches))
        precision = "bf16" if k % 3 == 2 else "f32"
        cases.append((dims, B, precision))
    return cases


@pytest.mark.parametrize("dims,B,precision", _sweep_cases() + _sweep_cases_medium())
def test_shape_sweep(torch_dev, dims, B, precision):
    """Gradients and the update against the oracle at the contract's gates on
    seeded small shapes (the edge-shape checks, drawn rather than listed)."""
    test_edge_shapes(torch_dev, dims, B, precision)


@pytest.mark.parametrize("dims,B,precision", [((784, 128, 10), 32, "f32"),
                                              ((1024, 4096, 4096, 1000), 4096, "f32"),
                                              ((1024, 4096, 4096, 1000), 4096, "bf16")])
def test_zero_weights_loss_is_log_classes(torch_dev, dims, B, precision):
    """P1 on the GPU: zero weights give loss = ln C, dlogits = (1/C - t)/B,
    zero gradients, and an unchanged W after a step."""
    torch, dev = torch_dev
    _announce(f"zero weights dims={dims} B={B} {precision}")
    Ws = [np.zeros((dims[l], dims[l + 1]), np.float32) for l in range(len(dims) - 1)]
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=3)
    net = make_net(dims, B, precision, Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    loss, dws, dl, _ = P.gpu_grads(net, xd, td)
    C = dims[-1]
    assert abs(loss - math.log(C)) <= 1e-6 * math.log(C)
    np.testing.assert_allclose(dl, (1.0 / C - t) / B, rtol=1e-6, atol=1e-12)
    assert np.max(np.abs(dl.astype(np.float64).sum(1))) <= 2 * C * 2.0 ** -24 / B
    for d in dws:
        assert np.all(d == 0)
    net.train_step(xd, td, 0.1)
    for w in net.read_params():
        assert torch.all(w == 0)
    net.close()


# -------------------------------------------------------------- invariants --

@pytest.mark.parametrize("name", ["mnist_b1024", "wide_f32", "wide_bf16", "skinny_b8"])
def test_determinism(torch_dev, name):
    """P9: two steps from the same state are bitwise identical (fixed-order
    reductions, integer tickets, no float atomics)."""
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    Ws = synth.workload_weights(w)
    x, t, _ = synth.workload_batch(w, 0)
    xd, td = P.to_dev([x, t], dev)
    out = []
    for rep in range(2):
        _announce(f"determinism {name} rep {rep}")
        net = make_net(w.dims, w.batch, w.precision, Ws, dev)
        loss, dws, dl, _ = P.gpu_grads(net, xd, td)
        loss2 = net.train_step(xd, td, w.lr)
        W_new = [a.cpu().numpy() for a in net.read_params()]
        out.append((loss, dws, dl, loss2, W_new))
        net.close()
    a, b = out
    assert a[0] == b[0] and a[3] == b[3]
    for u, v in zip(a[1] + [a[2]] + a[4], b[1] + [b[2]] + b[4]):
        assert np.array_equal(u, v)


def test_fused_splitk_loss_matches_forward(torch_dev):
    """A bf16 logits product split over K hands its partial sums to the loss
    kernel, which adds them in split order: the logits it stores equal, bit
    for bit, those of a forward without labels (split-K epilogue launch), and
    the loss and dlogits pass the oracle gates."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (1024, 2048, 1000), 2048    # logits product 2048 x 1000, K = 2048: 32 tiles, 4 splits
    _announce(f"fused split-K loss dims={dims} B={B}")
    Ws = synth.make_weights(dims, "kaiming", seed=21)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=22)
    net = make_net(dims, B, "bf16", Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    plain, _ = net.forward(xd)
    net.profile(True)
    loss, dws, dl, masks = P.gpu_grads(net, xd, td)
    names = [r["name"] for r in net.profile_read()]
    i = names.index("mfma_bf16_nn_partials_l1")
    assert names[i + 1] == "splitk_sum_softmax_xent", names
    fused = net.read_state(binding.STATE_LOGITS)
    assert torch.equal(plain, fused)
    fl, floss = net.forward(xd, td)
    assert torch.equal(fl, plain) and floss == loss
    ref = P.oracle_step(x, t, Ws, 0.0, dims, "bf16", masks)
    P.check_grads(loss, dws, dl, ref, "bf16", "fused split-K loss")
    net.close()


@pytest.mark.parametrize("dims,B", [((256, 520, 64), 8), ((96, 160, 132, 40), 5), ((1024, 1100, 260), 16),
                                    ((4096, 11008, 4096), 8)])
def test_skinny_step_loss_equals_forward_loss(torch_dev, dims, B):
    """In skinny sessions the softmax-CE launch of a step leaves the mean of
    the row losses to the fused dX + dW launch after it, which must give the
    bits of the forward's loss (there the softmax-CE launch takes the mean
    itself): through mlp_grads, mlp_train_step, a device loss and a run of
    steps."""
    torch, dev = torch_dev
    _announce(f"skinny deferred mean dims={dims} B={B}")
    Ws = synth.make_weights(dims, "glorot", seed=B + 31)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=B + 32)
    net = make_net(dims, B, "f32", Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    names = []
    net.profile(True)
    _, floss = net.forward(xd, td)
    gloss, _, _ = net.grads(xd, td)
    names = [r["name"] for r in net.profile_read()]
    net.profile(False)
    assert "softmax_xent" in names and any(n.startswith("skinny_nt_") for n in names), names
    assert np.float32(gloss) == np.float32(floss)
    sloss = net.train_step(xd, td, 0.05)
    assert np.float32(sloss) == np.float32(floss)
    # the updated weights give a new forward loss; the next step's device loss matches it
    _, floss2 = net.forward(xd, td)
    ld = torch.full((2,), float("nan"), dtype=torch.float32, device=dev)
    net.train_step_async(xd, td, 0.05, ld[0:1])
    torch.cuda.synchronize()
    assert np.float32(ld[0].item()) == np.float32(floss2)
    if (B * dims[0]) % 4 == 0 and (B * dims[-1]) % 4 == 0:
        _, floss3 = net.forward(xd, td)
        net.train_steps(torch.stack([xd, xd]), torch.stack([td, td]), 0.05, ld)
        torch.cuda.synchronize()
        assert np.float32(ld[0].item()) == np.float32(floss3)
    net.close()


@pytest.mark.parametrize("dims,B,precision", [((96, 160, 40), 64, "f32"),      # tiled kernels
                                              ((784, 128, 10), 32, "f32"),      # fused output layer
                                              ((256, 520, 64), 8, "f32"),       # skinny kernels
                                              ((200, 300, 36), 64, "bf16"),
                                              ((1024, 2048, 1040), 2048, "f32"),  # 256x256 tiles, split logits
                                              ((5, 3), 3, "f32")])             # no hidden layer
def test_nan_input_reaches_the_loss(torch_dev, dims, B, precision):
    """A NaN in x is not masked: the ReLU keeps it (a = z * [z > 0] is NaN for
    a NaN z), so the row's logits and the loss are NaN and the calls return
    MLP_OK; the other rows' logits stay finite."""
    torch, dev = torch_dev
    _announce(f"nan input dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=71)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=72)
    x[0, 0] = np.nan
    net = make_net(dims, B, precision, Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    logits, floss = net.forward(xd, td)
    lg = logits.cpu().numpy()
    assert np.all(np.isnan(lg[0])) and np.all(np.isfinite(lg[1:]))
    assert np.isnan(floss)
    probs = net.forward_probs(xd).cpu().numpy()
    assert np.all(np.isnan(probs[0])) and np.all(np.isfinite(probs[1:]))
    assert np.isnan(net.train_step(xd, td, 0.05))
    net.close()


def test_dlogits_rows_sum_to_zero(torch_dev):
    """P2 on the GPU: row sums of dlogits vanish to float32 rounding.

    The kernel forms e_c = exp(z_c - max), S = sum_c e_c (float32, any
    order: off by at most (C-1)u sum e, u = 2^-24, all terms positive),
    p_c = e_c / S (correctly rounded: no fast-math), then (p_c s - t_c)/B
    with s = 1 exactly for one-hot rows.  sum_c e_c/S = 1 within (C-1)u;
    rounding the C quotients adds at most u (they sum to ~1); p - 1 on the
    label's column rounds by at most u (exact when p >= 1/2, Sterbenz); the
    other columns subtract 0; B = 512 makes 1/B exact.  So every row sums to
    within (C+1)u/B of 0, under the 2Cu/B asserted here."""
    torch, dev = torch_dev
    w = synth.WORKLOADS["wide_f32"]
    dims, B = (256, 512, 1000), 512
    Ws = synth.make_weights(dims, "kaiming", seed=4)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=5)
    net = make_net(dims, B, "f32", Ws, dev)
    _, _, dl, _ = P.gpu_grads(net, *P.to_dev([x, t], dev))
    C = dims[-1]
    assert np.max(np.abs(dl.astype(np.float64).sum(1))) <= 2 * C * 2.0 ** -24 / B
    del w
    net.close()


def test_softmax_shift_and_overflow(torch_dev):
    """P4 on the GPU: logits of size ~1000 (large weights) give finite loss
    and dlogits matching the oracle."""
    torch, dev = torch_dev
    dims, B = (16, 24, 10), 8
    Ws = [a * 300 for a in synth.make_weights(dims, "glorot", seed=6)]
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=7)
    net = make_net(dims, B, "f32", Ws, dev)
    loss, dws, dl, masks = P.gpu_grads(net, *P.to_dev([x, t], dev))
    ref = P.oracle_step(x, t, Ws, 0.1, dims, "f32", masks)
    assert np.isfinite(loss) and np.all(np.isfinite(dl))
    P.check_grads(loss, dws, dl, ref, "f32", "overflow")
    net.close()


def test_dense_soft_labels(torch_dev):
    """Labels are dense rows; non-one-hot rows follow the same definition."""
    torch, dev = torch_dev
    dims, B = (40, 52, 12), 20
    Ws = synth.make_weights(dims, "glorot", seed=8)
    x, _, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=9)
    t = np.random.default_rng(10).uniform(0, 1, (B, dims[-1])).astype(np.float32)
    net = make_net(dims, B, "f32", Ws, dev)
    loss, dws, dl, masks = P.gpu_grads(net, *P.to_dev([x, t], dev))
    ref = P.oracle_step(x, t, Ws, 0.1, dims, "f32", masks)
    P.check_grads(loss, dws, dl, ref, "f32", "soft labels")
    net.close()


# ------------------------------------------------------------ error paths --

def test_errors_leave_state_unchanged(torch_dev):
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (16, 8, 4), 4
    Ws = synth.make_weights(dims, "glorot", seed=11)
    net = binding.Mlp(dims, B, "f32", device=str(dev))
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=12)
    xd, td = P.to_dev([x, t], dev)
    with pytest.raises(binding.MlpError) as e:       # weights never set
        net.train_step(xd, td, 0.1)
    assert e.value.status == binding.MLP_ERR_STATE
    net.set_params(P.to_dev(Ws, dev))
    for bad_lr in (float("nan"), float("inf")):
        with pytest.raises(binding.MlpError) as e:
            net.train_step(xd, td, bad_lr)
        assert e.value.status == binding.MLP_ERR_ARG
    with pytest.raises(binding.MlpError) as e:
        net.read_state(binding.STATE_MASK, 0)
    assert e.value.status == binding.MLP_ERR_ARG
    lib = binding.lib()
    misaligned = ctypes.c_void_p(xd.data_ptr() + 4)
    assert lib.mlp_train_step(net._h, misaligned, ctypes_ptr(td), 0.1, None) == binding.MLP_ERR_ARG
    for g, w in zip(net.read_params(), Ws):
        np.testing.assert_array_equal(g.cpu().numpy(), w)
    net.close()


def ctypes_ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def test_profile_slots(torch_dev):
    torch, dev = torch_dev
    w = synth.WORKLOADS["mnist_b32"]
    net = make_net(w.dims, w.batch, "f32", synth.workload_weights(w), dev)
    xd, td = P.to_dev(synth.workload_batch(w)[:2], dev)
    net.profile(True)
    for _ in range(3):
        net.train_step(xd, td, w.lr)
    rows = net.profile_read()
    # 784->128->10: the hidden forward GEMM with the fused output layer's head
    # (logits, CE, dX) riding along, then dW + SGD of the first layer with the
    # output layer's dW + SGD and mean loss riding along
    assert [r["name"] for r in rows] == ["mfma_f32_nn_relu_mask_l0+head_logits_xent_dx_l1",
                                         "mfma_f32_tn_sgd_l0+tail_dw_sgd_loss_l1"]
    assert all(r["launches"] == 3 and r["total_ms"] > 0 for r in rows)
    assert rows[0]["flops"] == 2 * 32 * 784 * 128 + 4 * 32 * 128 * 10   # forward + logits and dX
    net.close()
    # without the fused output layer (C > 32): one slot per launch, in order
    dims, B = (16, 8, 40), 64
    rng = np.random.default_rng(5)
    Ws = [(rng.standard_normal((dims[l], dims[l + 1])) * 0.3).astype(np.float32) for l in range(2)]
    net = make_net(dims, B, "f32", Ws, dev)
    x = rng.standard_normal((B, dims[0])).astype(np.float32)
    t = np.eye(dims[-1], dtype=np.float32)[rng.integers(0, dims[-1], B)]
    xd, td = P.to_dev([x, t], dev)
    net.profile(True)
    net.train_step(xd, td, 0.1)
    names = [r["name"] for r in net.profile_read()]
    assert names == ["mfma_f32_nn_relu_mask_l0", "mfma_f32_nn_store_l1", "softmax_xent",
                     "mfma_f32_nt_mask_l1", "mfma_f32_tn_sgd_l1", "mfma_f32_tn_sgd_l0"], names
    # forward passes (without and with a loss) are sequences of their own
    net.profile_reset()
    net.forward(xd)
    torch.cuda.synchronize()    # a forward without a loss returns once enqueued
    rows = net.profile_read()
    assert [r["name"] for r in rows] == ["mfma_f32_nn_relu_mask_l0", "mfma_f32_nn_store_l1"]
    assert all(r["launches"] == 1 for r in rows)
    net.forward(xd, td)
    assert [r["name"] for r in net.profile_read()] == ["mfma_f32_nn_relu_mask_l0", "mfma_f32_nn_store_l1",
                                                       "softmax_xent"]
    net.close()


@pytest.mark.parametrize("name", ["mnist_b1024", "skinny_b8"])
def test_graph_replay_matches_eager(torch_dev, name):
    """A8: a captured training step (HIP graph via torch.cuda.graph) replays
    bit for bit like the eager steps: the step enqueues only kernels (no
    memsets, no host synchronisation) and every reduction has a fixed order.
    Eager work and synchronisations run between the replays."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    _announce(f"graph replay {name}")
    Ws = synth.workload_weights(w)
    x, t, _ = synth.workload_batch(w)
    xd, td = P.to_dev([x, t], dev)
    eager = make_net(w.dims, w.batch, "f32", Ws, dev)
    s = torch.cuda.Stream(device=dev)
    graphed = binding.Mlp(w.dims, w.batch, "f32", device=str(dev), stream=s)
    graphed.set_params(P.to_dev(Ws, dev))
    loss_e = torch.zeros(1, dtype=torch.float32, device=dev)
    loss_g = torch.zeros(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        graphed.train_step_async(xd, td, w.lr, loss_g)
    torch.cuda.synchronize()
    for step in range(3):
        eager.train_step_async(xd, td, w.lr, loss_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert loss_g.item() == loss_e.item(), f"step {step}: loss {loss_g.item()} vs {loss_e.item()}"
        for l, (a, b) in enumerate(zip(graphed.read_params(), eager.read_params())):
            assert torch.equal(a, b), f"step {step}: W{l} differs"
        torch.cuda.synchronize()
    eager.close()
    graphed.close()


# ------------------------------------------------------------ Adam / LaProp --

ADAPTIVE_CASES = [
    # dims, B, precision, integer operands (exact first-step gradients)
    ((200, 300, 36), 64, "f32", True),        # tiled GEMMs with split-K
    ((784, 128, 10), 1024, "f32", False),     # fused output layer: head in the forward, tail in dW
    ((64, 32, 8), 8, "f32", True),            # skinny kernels with the fused output layer
    ((256, 520, 64), 8, "f32", False),        # skinny kernels, ragged columns
    ((64, 100, 1040), 8, "f32", True),        # skinny dX + dW pass with its columns split
    ((33, 70, 17, 10), 37, "f32", False),     # three layers, widths not multiples of 4
    ((120, 136, 24), 256, "bf16", True),      # bf16 operands: the update refreshes the bf16 copy
    ((1024, 2048, 1000), 2048, "bf16", False),  # large bf16 tiles, split-K logits into the loss
    ((1024, 2048, 1000), 2048, "f32", False),   # large f32 tiles
]


def _adaptive_sweep():
    """Seeded shapes for the adaptive rules (both contracts, every plan family)."""
    rng = np.random.default_rng([2026, 15])
    widths = [4, 12, 31, 64, 100, 260, 520, 1040]
    cases = []
    for k in range(8):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice([3, 8, 16, 40, 128, 512]))
        cases.append((dims, B, "bf16" if k % 4 == 3 else "f32", False))
    return cases


@pytest.mark.parametrize("rule", ["adam", "laprop"])
@pytest.mark.parametrize("dims,B,precision,exact", ADAPTIVE_CASES + _adaptive_sweep())
def test_adaptive_update_parity(torch_dev, rule, dims, B, precision, exact):
    """Three Adam / LaProp steps against the oracle's rule applied to the
    oracle's own gradients.  Before each step the GPU gradients (same
    kernels, no update) pass the gradient gate; the weights after each step
    must lie within the bound derived from that gate and the update rule."""
    _adaptive_parity(torch_dev, rule, dims, B, precision, exact)


def test_adaptive_update_parity_skinny_full_size(torch_dev):
    """The same three Adam steps on the skinny workload's full shapes
    (4096 -> 11008 -> 4096, batch 8): the fused dX + dW pass and the first
    layer's streaming update carrying W, m and v."""
    # each Adam step moves every weight by about lr, and 11008 hidden units
    # add those moves up: lr 1e-5 keeps three steps' loss well away from 0
    _adaptive_parity(torch_dev, "adam", (4096, 11008, 4096), 8, "f32", False, lr=1e-5)


def _adaptive_parity(torch_dev, rule, dims, B, precision, exact, lr=1e-3):
    torch, dev = torch_dev
    _announce(f"{rule} dims={dims} B={B} {precision}")
    # small enough that three steps keep the loss away from 0 (the loss gate
    # is relative, and a near-zero loss is a difference of near-equal terms)
    b1, b2, eps = 0.9, 0.999, 1e-8
    if exact:
        x, t, Ws = P.integer_problem(dims, B, seed=sum(dims), bf16=precision == "bf16")
    else:
        Ws = synth.make_weights(dims, "glorot", seed=sum(dims) + B)
        x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=B, step=1)
    net = make_net(dims, B, precision, Ws, dev)
    net.set_optimizer(rule, b1, b2, eps)
    xd, td = P.to_dev([x, t], dev)
    W_ref = [np.asarray(w, np.float64) for w in Ws]
    m = [np.zeros_like(w) for w in W_ref]
    v = [np.zeros_like(w) for w in W_ref]
    bound = P.AdaptiveBound(rule, lr, b1, b2, eps, [w.shape for w in W_ref])
    for step in range(1, 4):
        W_now = [w.cpu().numpy() for w in net.read_params()]
        loss_g, dws, dl, masks = P.gpu_grads(net, xd, td)
        ref = mlp_oracle.train_step(x, t, W_now, 0.0, kink_choice=masks,
                                    precision=precision)
        # after one step from an integer problem many pre-activations sit
        # next to 0 (they were exactly 0): no cap on band adoptions there
        P.check_masks(ref, B, dims, precision, f"{rule} step {step}", limit_band=not exact)
        P.check_grads(loss_g, dws, dl, ref, precision, f"{rule} step {step}")
        # the trajectory's own oracle gradients (at the oracle's weights)
        rt = mlp_oracle.train_step(x, t, W_ref, 0.0, kink_choice=masks,
                                   precision=precision)
        dg = [P.GRAD_TOL[precision] * float(np.max(np.abs(g))) for g in rt["dW"]]
        if exact and step == 1:
            for a, r in zip(dws, rt["dW"]):
                assert np.array_equal(np.asarray(a, np.float64), r)
            dg = [0.0] * len(dg)
        upd = mlp_oracle.OPTIMIZERS[rule](W_ref, rt["dW"], m, v, step, lr, b1, b2, eps)
        loss = net.train_step(xd, td, lr)
        assert loss == loss_g    # the loss of a step is the one of its gradients
        W_gpu = [w.cpu().numpy() for w in net.read_params()]
        bnd = bound.step(rt["dW"], dg, upd["W_new"], W_ref)
        P.check_adaptive(W_gpu, upd["W_new"], bnd, f"{rule} {dims} step {step}")
        W_ref, m, v = upd["W_new"], upd["m"], upd["v"]
    net.close()


def test_adaptive_then_sgd_matches_fresh_sgd(torch_dev):
    """Switching back to SGD gives exactly the plain SGD step (same kernels
    and order) from the same weights."""
    torch, dev = torch_dev
    dims, B = (96, 160, 130, 40), 128
    Ws = synth.make_weights(dims, "glorot", seed=8)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=9)
    xd, td = P.to_dev([x, t], dev)
    a = make_net(dims, B, "f32", Ws, dev)
    a.set_optimizer("adam")
    a.train_step(xd, td, 0.01)
    W_mid = [w.clone() for w in a.read_params()]
    a.set_optimizer("sgd")
    a.train_step(xd, td, 0.05)
    b = make_net(dims, B, "f32", [w.cpu().numpy() for w in W_mid], dev)
    b.train_step(xd, td, 0.05)
    for u, w in zip(a.read_params(), b.read_params()):
        assert torch.equal(u, w)
    a.close()
    b.close()


def test_adaptive_profile_slots_and_errors(torch_dev):
    """With Adam every dW launch applies the rule (no extra launch); bad
    arguments are refused before anything is enqueued, and an Adam step
    refuses stream capture."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (16, 8, 40), 64
    rng = np.random.default_rng(5)
    Ws = [(rng.standard_normal((dims[l], dims[l + 1])) * 0.3).astype(np.float32) for l in range(2)]
    net = make_net(dims, B, "f32", Ws, dev)
    x = rng.standard_normal((B, dims[0])).astype(np.float32)
    t = np.eye(dims[-1], dtype=np.float32)[rng.integers(0, dims[-1], B)]
    xd, td = P.to_dev([x, t], dev)
    L = binding.lib()
    for args in [(binding.OPT_ADAM, 1.0, 0.999, 1e-8), (binding.OPT_ADAM, 0.9, -0.1, 1e-8),
                 (binding.OPT_LAPROP, 0.9, 0.999, 0.0), (7, 0.9, 0.999, 1e-8)]:
        st = L.mlp_set_optimizer(net._h, args[0], args[1], args[2], args[3], None, 0)
        assert st == binding.MLP_ERR_ARG, args
    st = L.mlp_set_optimizer(net._h, binding.OPT_ADAM, 0.9, 0.999, 1e-8, None, 0)
    assert st == binding.MLP_ERR_WORKSPACE
    net.set_optimizer("adam")
    net.profile(True)
    net.train_step(xd, td, 0.01)
    names = [r["name"] for r in net.profile_read()]
    assert names == ["mfma_f32_nn_relu_mask_l0", "mfma_f32_nn_store_l1", "softmax_xent",
                     "mfma_f32_nt_mask_l1", "mfma_f32_tn_adam_l1", "mfma_f32_tn_adam_l0"], names
    net.profile(False)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        snet = binding.Mlp(dims, B, "f32", device=str(dev), stream=side)
        snet.set_params(P.to_dev(Ws, dev))
        snet.set_optimizer("adam")
        torch.cuda.synchronize()
        # the refused step leaves the capture empty, which torch reports
        with pytest.warns(UserWarning, match="empty"):
            with torch.cuda.graph(g, stream=side):
                with pytest.raises(binding.MlpError) as ei:
                    snet.train_step_async(xd, td, 0.01)
        assert ei.value.status == binding.MLP_ERR_ARG
    snet.close()
    net.close()


# ------------------------------------------------------------- checkpoints --

def _ckpt_sweep():
    """Seeded shapes and rules (SGD included) for the checkpoint round trip."""
    rng = np.random.default_rng([2026, 18])
    widths = [4, 12, 33, 64, 100, 260, 1040]
    rules = ["sgd", "adam", "laprop"]
    cases = []
    for k in range(9):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice([2, 8, 16, 64, 256]))
        cases.append((dims, B, "bf16" if k % 3 == 2 else "f32", rules[k % 3]))
    return cases


@pytest.mark.parametrize("dims,B,precision,rule", [((96, 160, 130, 40), 128, "f32", "adam"),
                                                   ((256, 520, 64), 8, "f32", "laprop"),
                                                   ((120, 136, 24), 256, "bf16", "adam")] + _ckpt_sweep())
def test_checkpoint_resumes_training_bit_for_bit(torch_dev, dims, B, precision, rule):
    """Save after two steps (weights, moments, step count), restore into a
    fresh session and continue: the next steps equal those of the session
    that kept going."""
    torch, dev = torch_dev
    _announce(f"checkpoint resume dims={dims} B={B} {precision} {rule}")
    Ws = synth.make_weights(dims, "glorot", seed=31)
    xd, td = P.to_dev(synth.make_batch(B, dims[0], dims[-1], "normal", seed=32)[:2], dev)
    a = make_net(dims, B, precision, Ws, dev)
    a.set_optimizer(rule, 0.9, 0.99, 1e-7)
    for _ in range(2):
        a.train_step(xd, td, 1e-3)
    ck = a.save_checkpoint()
    for _ in range(2):
        a.train_step(xd, td, 1e-3)
    b = binding_net(dims, B, precision, dev)
    b.set_optimizer(rule, 0.9, 0.99, 1e-7)
    b.load_checkpoint(ck)
    for _ in range(2):
        b.train_step(xd, td, 1e-3)
    for u, w in zip(a.read_params(), b.read_params()):
        assert torch.equal(u, w)
    a.close()
    b.close()


def binding_net(dims, B, precision, dev):
    from mlp_gemm_softmax_amd import binding
    return binding.Mlp(dims, B, precision, device=str(dev))


def test_checkpoint_reloads_into_a_forward_session(torch_dev):
    """A bf16 training session's checkpoint (with Adam moments) loads into a
    fresh float32 session without an optimizer: the same masters, and the
    same logits as a session given those masters directly."""
    torch, dev = torch_dev
    dims, B = (120, 136, 24), 256
    Ws = synth.make_weights(dims, "glorot", seed=41)
    xd, td = P.to_dev(synth.make_batch(B, dims[0], dims[-1], "normal", seed=42)[:2], dev)
    a = make_net(dims, B, "bf16", Ws, dev)
    a.set_optimizer("adam")
    a.train_step(xd, td, 1e-3)
    ck = a.save_checkpoint()
    from mlp_gemm_softmax_amd import binding
    assert binding.checkpoint_info(ck)["step"] == 1
    masters = a.read_params()
    inf = binding_net(dims, B, "f32", dev)
    inf.load_checkpoint(ck)
    for u, w in zip(inf.read_params(), masters):
        assert torch.equal(u, w)
    ref = binding_net(dims, B, "f32", dev)
    ref.set_params([w.clone() for w in masters])
    l1, _ = inf.forward(xd)
    l2, _ = ref.forward(xd)
    assert torch.equal(l1, l2)
    for n in (a, inf, ref):
        n.close()


def test_checkpoint_preflight_changes_nothing(torch_dev):
    """Restores that fail their checks leave the session's weights as they
    were: another shape, a rule the checkpoint does not carry, a damaged
    payload."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (48, 40, 12), 32
    src = make_net(dims, B, "f32", synth.make_weights(dims, "glorot", seed=51), dev)
    ck = src.save_checkpoint()
    other = make_net((48, 44, 12), B, "f32", synth.make_weights((48, 44, 12), "glorot", seed=52), dev)
    before = [w.clone() for w in other.read_params()]
    with pytest.raises(binding.MlpError) as ei:
        other.load_checkpoint(ck)
    assert ei.value.status == binding.MLP_ERR_SHAPE
    same = make_net(dims, B, "f32", synth.make_weights(dims, "glorot", seed=53), dev)
    same.set_optimizer("adam")
    before_same = [w.clone() for w in same.read_params()]
    with pytest.raises(binding.MlpError) as ei:
        same.load_checkpoint(ck)            # no Adam state in an SGD checkpoint
    assert ei.value.status == binding.MLP_ERR_ARG
    bad = bytearray(ck)
    bad[-1] ^= 0x40
    same.set_optimizer("sgd")
    with pytest.raises(binding.MlpError) as ei:
        same.load_checkpoint(bytes(bad))
    assert ei.value.status == binding.MLP_ERR_ARG
    for u, w in zip(other.read_params(), before):
        assert torch.equal(u, w)
    for u, w in zip(same.read_params(), before_same):
        assert torch.equal(u, w)
    same.load_checkpoint(ck)                # the intact one restores
    for u, w in zip(same.read_params(), src.read_params()):
        assert torch.equal(u, w)
    for n in (src, other, same):
        n.close()


def _f32(v):
    return float(np.float32(v))


def test_checkpoint_payload_decodes_from_the_documented_layout(torch_dev):
    """A checkpoint the library writes, decoded in Python from the layout
    include/mlp.h documents (tests/ckpt_format.py): header fields, the
    checksum, W_l at their logical [in, out] shapes bit for bit equal to
    mlp_read_params, and the Adam moments of one step from exact gradients
    equal to the oracle's m = (1-b1) g, v = (1-b2) g^2 within the float32
    roundings of that arithmetic (4 units of 2^-24, relative)."""
    from mlp_gemm_softmax_amd import binding
    from tests import ckpt_format
    torch, dev = torch_dev
    dims, B = (48, 40, 12), 64
    x, t, Ws = P.integer_problem(dims, B, seed=71)
    b1, b2, eps = 0.9, 0.99, 1e-7
    net = make_net(dims, B, "f32", Ws, dev)
    net.set_optimizer("adam", b1, b2, eps)
    xd, td = P.to_dev([x, t], dev)
    _, dws, _, _ = P.gpu_grads(net, xd, td)
    ref = mlp_oracle.train_step(x, t, Ws, 0.0)
    for a, r in zip(dws, ref["dW"]):
        assert np.array_equal(a, r.astype(np.float32))      # exact gradients
    net.train_step(xd, td, 1e-3)
    ck = net.save_checkpoint(with_optimizer=True)
    h = ckpt_format.parse(ck)
    n_w = sum(a * b for a, b in zip(dims[:-1], dims[1:]))
    assert h["magic"] == b"MLPCKPT1" and h["version"] == ckpt_format.VERSION and h["n_layers"] == 2
    assert h["dims"] == list(dims) and h["unused_dims"] == [0] * (17 - len(dims))
    assert h["precision"] == binding.MLP_F32 and h["optimizer"] == binding.OPT_ADAM
    assert h["betas"] == (_f32(b1), _f32(b2), _f32(eps)) and h["reserved"] == (0, 0)
    assert h["step"] == 1
    assert h["payload_bytes"] == h["payload_len"] == 3 * 4 * n_w and h["trailing"] == 0
    assert h["checksum"] == h["payload_checksum"]
    for w_ck, w_dev in zip(h["W"], net.read_params()):
        assert w_ck.shape == tuple(w_dev.shape)
        assert np.array_equal(w_ck, w_dev.cpu().numpy())
    zeros = [np.zeros(w.shape) for w in Ws]
    upd = mlp_oracle.adam(Ws, ref["dW"], zeros, zeros, 1, 1e-3, _f32(b1), _f32(b2), _f32(eps))
    u = 2.0 ** -24
    for l in range(2):
        for got, want in ((h["m"][l], upd["m"][l]), (h["v"][l], upd["v"][l])):
            err = np.abs(got.astype(np.float64) - want)
            assert np.all(err <= 4 * u * np.abs(want)), f"layer {l}: moments off the documented layout"
    # without the rule's state: the weights only
    h2 = ckpt_format.parse(net.save_checkpoint(with_optimizer=False))
    assert h2["optimizer"] == binding.OPT_SGD and h2["payload_len"] == 4 * n_w and h2["trailing"] == 0
    for a, b in zip(h2["W"], h["W"]):
        assert np.array_equal(a, b)
    net.close()


def test_hand_built_checkpoint_restores_weights_and_moments(torch_dev):
    """A checkpoint written in Python from the documented layout loads into
    a session: the weights come back bit for bit (SGD session: weights only;
    Adam session: with its moments and step count), and the next Adam step
    from them equals the oracle's rule at t = step + 1 from the same moments
    within the float32 roundings of the update.  The moments share the sign
    of the (exact) gradient, so no cancellation enlarges those roundings."""
    from mlp_gemm_softmax_amd import binding
    from tests import ckpt_format
    torch, dev = torch_dev
    dims, B = (48, 40, 12), 64
    x, t, Ws = P.integer_problem(dims, B, seed=72)
    g = mlp_oracle.train_step(x, t, Ws, 0.0)["dW"]
    rng = np.random.default_rng([73, 1])
    sign = [np.where(gl >= 0, 1.0, -1.0) for gl in g]
    m0 = [(sg * rng.uniform(0.01, 0.5, sg.shape)).astype(np.float32) for sg in sign]
    v0 = [rng.uniform(0.5, 2.0, w.shape).astype(np.float32) for w in Ws]
    b1, b2, eps = _f32(0.9), _f32(0.99), _f32(1e-7)
    ck = ckpt_format.build(dims, Ws, m0, v0, opt=binding.OPT_ADAM, step=7, betas=(b1, b2, eps))
    assert binding.checkpoint_info(ck) == {"n_layers": 2, "dims": list(dims),
                                           "optimizer": binding.OPT_ADAM, "step": 7}
    sgd = binding_net(dims, B, "f32", dev)
    sgd.load_checkpoint(ck)
    for got, w in zip(sgd.read_params(), Ws):
        assert np.array_equal(got.cpu().numpy(), w)
    net = binding_net(dims, B, "f32", dev)
    net.set_optimizer("adam", b1, b2, eps)
    net.load_checkpoint(ck)
    for got, w in zip(net.read_params(), Ws):
        assert np.array_equal(got.cpu().numpy(), w)
    xd, td = P.to_dev([x, t], dev)
    _, dws, _, _ = P.gpu_grads(net, xd, td)
    for a, r in zip(dws, g):
        assert np.array_equal(a, r.astype(np.float32))
    lr = 1e-3
    net.train_step(xd, td, lr)
    upd = mlp_oracle.adam(Ws, g, m0, v0, 8, lr, b1, b2, eps)
    for l, (got, want, w0) in enumerate(zip(net.read_params(), upd["W_new"], Ws)):
        step = want - np.asarray(w0, np.float64)
        bound = P._f32_update_rounding(want, step)
        err = np.abs(got.cpu().numpy().astype(np.float64) - want)
        assert np.all(err <= bound), f"layer {l}: {int((err > bound).sum())} weights off the restored rule"
        # and the restored moments matter: from zero moments the step differs
        fresh = mlp_oracle.adam([w0], [g[l]], [np.zeros_like(w0)], [np.zeros_like(w0)], 1, lr, b1, b2, eps)
        assert np.max(np.abs(fresh["W_new"][0] - want)) > 100 * np.max(bound)
    ck2 = ckpt_format.parse(net.save_checkpoint(with_optimizer=True))
    assert ck2["step"] == 8
    sgd.close()
    net.close()


# ---------------------------------------------------------------- inference --

@pytest.mark.parametrize("name", ["mnist_b1024", "wide_f32", "wide_bf16", "skinny_b8"])
def test_forward_logits_parity(torch_dev, name):
    """Forward only (the inference path): logits of the workload's batch
    against the oracle's forward, per-tensor gate as for the gradients, with
    the GPU's ReLU choices adopted inside the rounding band only."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    _announce(f"forward parity {name}")
    Ws = synth.workload_weights(w)
    x, t, _ = synth.workload_batch(w, 0)
    net = make_net(w.dims, w.batch, w.precision, Ws, dev)
    xd, = P.to_dev([x], dev)
    logits = torch.empty((w.batch, w.dims[-1]), dtype=torch.float32, device=dev)
    net.forward_async(xd, logits)
    torch.cuda.synchronize()
    masks = [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, net.n_layers)]
    sc = P.check_mask_self_consistency(x, Ws, masks, P.gpu_acts(net), w.precision, name)
    ref = mlp_oracle.forward(x, Ws, kink_choice=masks, precision=w.precision)
    P.check_masks({"fwd": ref}, w.batch, w.dims, w.precision, "forward " + name, self_counts=sc)
    err, scale = P.rel_max(logits.cpu().numpy(), ref["logits"])
    gtol = P.GRAD_TOL[w.precision]
    assert err <= gtol * scale, f"{name} logits: {err:.3e} > {gtol} * {scale:.3e}"
    net.close()


# ------------------------------------------------- bf16 rounding (exactly) --

def _rne_bf16(v):
    """float32 -> bfloat16 -> float32, round to nearest, ties to even
    (integer form: add 0x7fff plus the lowest kept bit, drop 16 bits)."""
    u = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def _rounding_values(n, seed):
    """Positive normal float32 values whose dropped 16 bits sit below, at and
    above the halfway point, with even and odd kept mantissas."""
    rng = np.random.default_rng(seed)
    lows = np.array([0x0000, 0x0001, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    hi = (rng.integers(0x3E00, 0x4200, n).astype(np.uint32) & 0xFFFE) | (np.arange(n, dtype=np.uint32) & 1)
    return ((hi << 16) | lows[np.arange(n) % len(lows)]).view(np.float32)


def test_bf16_rounding_is_nearest_even(torch_dev):
    """A7 precision conversions, bit for bit: the cast of x, the bf16 copy of
    W and the activation written by the ReLU epilogue all round to nearest
    even.  Each net is built so that the stored activation is exactly one
    rounded value: a1 = rne(x0) * 1, a1 = 1 * rne(w), and a1 = rne(1 + d) with
    1 + d exact in float32 (d a bfloat16 value); the products and their
    float32 sums are exact, so any other rounding shows."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    B, H = 64, 64
    dims = (8, H, 8)
    W2 = np.zeros((H, 8), dtype=np.float32)

    def act(x, W1):
        net = make_net(dims, B, "bf16", [W1, W2], dev)
        xd, = P.to_dev([x], dev)
        logits = torch.empty((B, 8), dtype=torch.float32, device=dev)
        net.forward_async(xd, logits)
        a = net.read_state(binding.STATE_ACT, 1).cpu().numpy()
        net.close()
        return a

    # the cast of x: x[b][0] = v_b, W1[0][:] = 1
    v = _rounding_values(B, 1)
    x = np.zeros((B, 8), dtype=np.float32)
    x[:, 0] = v
    W1 = np.zeros((8, H), dtype=np.float32)
    W1[0, :] = 1.0
    a = act(x, W1)
    assert np.array_equal(a, np.repeat(_rne_bf16(v)[:, None], H, axis=1)), "cast of x"
    # the bf16 copy of W: x[b][0] = 1, W1[0][c] = w_c
    w = _rounding_values(H, 2)
    x = np.zeros((B, 8), dtype=np.float32)
    x[:, 0] = 1.0
    W1 = np.zeros((8, H), dtype=np.float32)
    W1[0, :] = w
    a = act(x, W1)
    assert np.array_equal(a, np.repeat(_rne_bf16(w)[None, :], B, axis=0)), "bf16 copy of W"
    # the epilogue: x[b][0] = x[b][1] = 1, W1[0][c] = 1, W1[1][c] = d_c with
    # d_c = m * 2^-9 .. m * 2^-12 (bf16-exact), so 1 + d_c falls below, on
    # and above the halfway points between bfloat16 neighbours of 1
    m = np.arange(H, dtype=np.float32)
    d = (m % 16) * np.float32(2.0) ** -(9 + (m // 16))
    x = np.zeros((B, 8), dtype=np.float32)
    x[:, 0] = 1.0
    x[:, 1] = 1.0
    W1 = np.zeros((8, H), dtype=np.float32)
    W1[0, :] = 1.0
    W1[1, :] = d
    assert np.array_equal(_rne_bf16(d), d)
    a = act(x, W1)
    want = _rne_bf16(np.float32(1.0) + d)
    assert np.array_equal(a, np.repeat(want[None, :], B, axis=0)), "ReLU epilogue rounding"
    # the cases include ties that truncation would get wrong
    assert np.any(want != (np.float32(1.0) + d).view(np.uint32).__and__(0xFFFF0000).view(np.float32))


# ------------------------------------------------------ class probabilities --

PROBS_CASES = [
    # (dims, B, precision): the workloads' shapes and edges of both paths
    ((784, 128, 10), 1024, "f32"),      # logits tile normalises in its epilogue
    ((784, 128, 10), 32, "f32"),
    ((33, 70, 17, 10), 37, "f32"),      # three layers, widths not multiples of 4
    ((128, 10), 300, "f32"),            # no hidden layer
    ((1, 1, 1), 1, "f32"),              # one class: p = 1
    ((784, 128, 20), 64, "f32"),        # C > 16: row-softmax launch
    ((64, 260, 36), 12, "f32"),         # skinny kernels
    ((1024, 512, 1000), 512, "f32"),    # wide rows
    ((72, 200, 1000), 48, "bf16"),      # bf16 operands
    ((1024, 2048, 1000), 2048, "bf16"),  # large bf16 tiles with split-K logits
    ((64, 4096), 8, "f32"),             # few wide rows: a workgroup per row
    ((16, 9000), 3, "f32"),             # rows wider than the registers hold: streamed
    ((40, 600), 700, "f32"),            # many rows of 600 classes: a wavefront per row
]


def _probs_sweep():
    """Seeded shapes for class probabilities (epilogue-normalised and
    row-softmax paths, narrow and wide class counts)."""
    rng = np.random.default_rng([2026, 16])
    widths = [1, 7, 10, 16, 33, 100, 300, 1000, 4100]
    cases = []
    for k in range(10):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths[:-1])) for _ in range(L)) + (int(rng.choice(widths)),)
        B = int(rng.choice([1, 5, 8, 32, 100, 1024]))
        cases.append((dims, B, "bf16" if k % 4 == 3 else "f32"))
    return cases


@pytest.mark.parametrize("dims,B,precision", PROBS_CASES + _probs_sweep())
def test_forward_probs_parity(torch_dev, dims, B, precision):
    """Inference probabilities against the oracle's softmax of its forward
    logits.  With every logit within delta = tol * max|z_ref| of the oracle
    (the forward gate), each probability is within a factor e^(+-2 delta) of
    the oracle's, so |dp| <= (e^(2 delta) - 1) max p_ref, plus the float32
    rounding of the normalisation ((C + 4) units of 2^-24).  Rows sum to 1
    within that rounding; two calls agree bitwise."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"forward probs {dims} B={B} {precision}")
    rng = np.random.default_rng([7, len(dims), B])
    Ws = [rng.uniform(-1, 1, (a, b)).astype(np.float32) * np.float32(math.sqrt(6.0 / (a + b)))
          for a, b in zip(dims[:-1], dims[1:])]
    x = rng.standard_normal((B, dims[0])).astype(np.float32)
    net = make_net(dims, B, precision, Ws, dev)
    xd, = P.to_dev([x], dev)
    net.profile(True)
    net.profile_reset()
    probs = net.forward_probs(xd)
    again = net.forward_probs(xd)
    torch.cuda.synchronize()
    names = [r["name"] for r in net.profile_read()]
    net.profile(False)
    masks = [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, net.n_layers)]
    ref = mlp_oracle.forward_probabilities(x, Ws, kink_choice=masks,
                                           precision=precision)
    P.check_masks({"fwd": ref["fwd"]}, B, dims, precision, "probs")
    p = probs.cpu().numpy()
    assert np.array_equal(p, again.cpu().numpy()), "two calls differ"
    C = dims[-1]
    delta = P.GRAD_TOL[precision] * float(np.max(np.abs(ref["fwd"]["logits"])))
    rnd = (C + 4) * 2.0 ** -24
    bound = math.expm1(2 * delta) * float(np.max(ref["probs"])) + rnd
    err = float(np.max(np.abs(p - ref["probs"])))
    assert err <= bound, f"probs: {err:.3e} > {bound:.3e}"
    assert np.all(p >= 0)
    assert float(np.max(np.abs(p.astype(np.float64).sum(1) - 1.0))) <= 2 * rnd
    # the last launch of the sequence is the normalising one; the README
    # MLP's 10 classes normalise inside the logits product
    assert names[-1].endswith("softmax_l" + str(len(dims) - 2)) or names[-1] == "softmax_probs", names
    if dims == (784, 128, 10):
        assert names[-1] == "mfma_f32_nn_softmax_l1", names
    net.close()


def test_forward_probs_argument_errors(torch_dev):
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (784, 128, 10), 32
    Ws = synth.workload_weights(synth.WORKLOADS["mnist_b32"])
    net = make_net(dims, B, "f32", Ws, dev)
    x = torch.zeros((B, dims[0]), dtype=torch.float32, device=dev)
    buf = torch.zeros(B * dims[-1] + 4, dtype=torch.float32, device=dev)
    L = binding.lib()
    st = L.mlp_forward_probs(net._h, ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(buf.data_ptr() + 4))
    assert st == binding.MLP_ERR_ARG
    st = L.mlp_forward_probs(net._h, ctypes.c_void_p(x.data_ptr()), None)
    assert st == binding.MLP_ERR_ARG
    st = L.mlp_forward_probs(net._h, None, ctypes.c_void_p(buf.data_ptr()))
    assert st == binding.MLP_ERR_ARG
    # the context still works
    p = net.forward_probs(x)
    torch.cuda.synchronize()
    assert abs(float(p.sum().item()) - B) < 1e-4
    net.close()


# ------------------------------------------------------------------- tuning --

@pytest.mark.parametrize("dims,B,precision", [((200, 300, 36), 64, "f32"),
                                              ((320, 2080, 40), 512, "f32"),
                                              ((1024, 2048, 1000), 2048, "bf16"),
                                              ((784, 128, 10), 1024, "f32"),
                                              # the head is not fused at creation (32 x 32 tiles) but a
                                              # candidate (32 x 16, 16 waves) fuses it: 128 row blocks
                                              ((784, 128, 10), 4096, "f32"),
                                              ((512, 2048, 1040), 8, "f32")])   # skinny: K and column splits
def test_tuned_plans_keep_parity(torch_dev, dims, B, precision):
    """After mlp_tune the weights are unchanged, and the step with the chosen
    plans still passes the oracle's gates and is repeatable bit for bit."""
    torch, dev = torch_dev
    _announce(f"tune dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=61)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=62)
    net = make_net(dims, B, precision, Ws, dev)
    xd, td = P.to_dev([x, t], dev)
    before = [w.clone() for w in net.read_params()]
    net.tune(xd, td, 2)
    for u, w in zip(net.read_params(), before):
        assert torch.equal(u, w)
    loss, dws, dl, masks = P.gpu_grads(net, xd, td)
    loss_b, dws_b, dl_b, _ = P.gpu_grads(net, xd, td)
    assert loss == loss_b and all(np.array_equal(a, b) for a, b in zip(dws, dws_b))
    ref = P.oracle_step(x, t, Ws, 0.05, dims, precision, masks)
    P.check_masks(ref, B, dims, precision, "tuned")
    P.check_grads(loss, dws, dl, ref, precision, "tuned")
    loss2, W_new, masks2 = P.gpu_train(net, xd, td, 0.05)
    ref2 = P.oracle_step(x, t, Ws, 0.05, dims, precision, masks2)
    P.check_update(loss2, W_new, Ws, ref2, precision, "tuned")
    net.close()


# ------------------------------------------------------------ runs of steps --

STEPS_CASES = [
    # dims, B, precision, optimizer, steps
    ((4096, 11008, 4096), 8, "f32", "sgd", 3),   # the skinny batch-8 workload: fused first-layer passes
    ((256, 520, 64), 8, "f32", "sgd", 4),        # ragged last column group
    ((1024, 1100, 260), 6, "f32", "sgd", 3),     # forward K splits (partials and tickets), 6 of 8 rows
    ((4100, 64, 8), 3, "f32", "sgd", 3),         # many K splits, batch <= 4
    ((64, 32, 8), 8, "f32", "sgd", 3),           # fused output layer with L = 2: its tail goes first
    ((96, 160, 132, 40), 8, "f32", "sgd", 3),    # three layers: dX + dW pass of the middle layer
    ((64, 12), 5, "f32", "sgd", 3),              # one layer: the fused launch makes the next logits
    ((1024, 1100, 260), 16, "f32", "sgd", 2),    # 16 rows: not fused, one step after another
    ((200, 300, 36), 64, "f32", "sgd", 2),       # tiled kernels: not fused
    ((200, 300, 36), 64, "bf16", "sgd", 2),
    ((256, 520, 64), 8, "f32", "adam", 3),       # adaptive rule: not fused
]


def _steps_sweep():
    """Seeded skinny shapes for runs of steps (widths multiples of 4, at most 8
    rows: the first-layer update fused with the next forward)."""
    rng = np.random.default_rng([2026, 14])
    widths = [4, 8, 12, 36, 64, 100, 260, 516, 1028, 2052]
    cases = []
    for _ in range(16):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8]))
        cases.append((dims, B, "f32", "sgd", 3))
    return cases


@pytest.mark.parametrize("dims,B,precision,opt,steps", STEPS_CASES + _steps_sweep())
def test_train_steps_match_single_steps(torch_dev, dims, B, precision, opt, steps):
    """mlp_train_steps over n batches equals n mlp_train_step_async calls on
    the same batches, bit for bit: weights, per-step losses, and the last
    step's activations and masks (in the skinny sessions the first layer's
    update and the next step's first forward share one launch)."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"train_steps dims={dims} B={B} {precision} {opt} n={steps}")
    Ws = synth.make_weights(dims, "glorot", seed=sum(dims) + B)
    xs, ts = [], []
    for s in range(steps):
        x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=B + 7, step=s)
        xs.append(x)
        ts.append(t)
    xd, td = P.to_dev([np.stack(xs), np.stack(ts)], dev)
    lr = 0.05 if opt == "sgd" else 1e-3
    out = []
    for mode in ("run", "single"):
        net = make_net(dims, B, precision, Ws, dev)
        if opt != "sgd":
            net.set_optimizer(opt, 0.9, 0.999, 1e-8)
        losses = torch.full((steps,), float("nan"), dtype=torch.float32, device=dev)
        if mode == "run":
            net.train_steps(xd, td, lr, losses)
        else:
            for s in range(steps):
                net.train_step_async(xd[s], td[s], lr, losses[s:s + 1])
        torch.cuda.synchronize()
        state = [net.read_state(binding.STATE_ACT, l).cpu().numpy() for l in range(1, len(dims) - 1)]
        state += [net.read_state(binding.STATE_MASK, l).cpu().numpy() for l in range(1, len(dims) - 1)]
        out.append((losses.cpu().numpy(), [w.cpu().numpy() for w in net.read_params()], state))
        net.close()
    (la, wa, sa), (lb, wb, sb) = out
    assert np.all(np.isfinite(la))
    assert np.array_equal(la.view(np.uint32), lb.view(np.uint32)), (la, lb)
    for l, (u, v) in enumerate(zip(wa, wb)):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32)), f"W_{l} differs"
    for u, v in zip(sa, sb):
        assert np.array_equal(u, v)


def test_train_steps_follow_the_oracle(torch_dev):
    """A fused run's per-step losses track the oracle's own trajectory over
    the same batches (free-running: each implementation feeds its updated
    weights to the next step), and its first loss is the oracle's at the
    strict loss gate."""
    torch, dev = torch_dev
    dims, B, steps, lr = (256, 520, 64), 8, 4, 0.05
    Ws = synth.make_weights(dims, "glorot", seed=11)
    batches = [synth.make_batch(B, dims[0], dims[-1], "normal", seed=12, step=s)[:2] for s in range(steps)]
    ref, cur = [], [np.asarray(a, np.float32) for a in Ws]
    for x, t in batches:
        r = mlp_oracle.train_step(x, t, cur, lr)
        ref.append(r["loss"])
        cur = [a.astype(np.float32) for a in r["W_new"]]
    xd, td = P.to_dev([np.stack([b[0] for b in batches]), np.stack([b[1] for b in batches])], dev)
    net = make_net(dims, B, "f32", Ws, dev)
    losses = torch.zeros(steps, dtype=torch.float32, device=dev)
    net.train_steps(xd, td, lr, losses)
    got = losses.cpu().numpy()
    net.close()
    assert abs(got[0] - ref[0]) <= 1e-5 * abs(ref[0])
    for s in range(steps):
        assert abs(got[s] - ref[s]) <= 1e-4 * abs(ref[s]), (s, got[s], ref[s])


def test_train_steps_argument_errors(torch_dev):
    """Preflight of mlp_train_steps: nothing is enqueued and the weights stay."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    dims, B = (64, 32, 8), 8
    Ws = synth.make_weights(dims, "glorot", seed=3)
    net = make_net(dims, B, "f32", Ws, dev)
    x = torch.zeros((2, B, dims[0]), dtype=torch.float32, device=dev)
    t = torch.zeros((2, B, dims[-1]), dtype=torch.float32, device=dev)
    lib = binding.lib()
    h = net._h
    assert lib.mlp_train_steps(h, 0, ctypes_ptr(x), ctypes_ptr(t), 0.1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_train_steps(h, 2, None, ctypes_ptr(t), 0.1, None) == binding.MLP_ERR_ARG
    assert lib.mlp_train_steps(h, 2, ctypes_ptr(x), ctypes_ptr(t), float("nan"), None) == binding.MLP_ERR_ARG
    torch.cuda.synchronize()
    for a, b in zip(net.read_params(), Ws):
        assert np.array_equal(a.cpu().numpy(), b)
    net.close()


def test_train_steps_graph_replay_matches_eager(torch_dev):
    """A run of steps on the batch-8 4096-11008-4096 net (the merged
    first-layer launches included) captured into a HIP graph replays bit for
    bit like the same run enqueued eagerly, with eager work and
    synchronisations between the replays."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    w = synth.WORKLOADS["skinny_b8"]
    _announce("graph replay of a run of skinny_b8 steps")
    Ws = synth.workload_weights(w)
    n = 3
    bs = [synth.workload_batch(w, s)[:2] for s in range(n)]
    xd, td = P.to_dev([np.stack([b[0] for b in bs]), np.stack([b[1] for b in bs])], dev)
    eager = make_net(w.dims, w.batch, "f32", Ws, dev)
    s = torch.cuda.Stream(device=dev)
    graphed = binding.Mlp(w.dims, w.batch, "f32", device=str(dev), stream=s)
    graphed.set_params(P.to_dev(Ws, dev))
    loss_e = torch.zeros(n, dtype=torch.float32, device=dev)
    loss_g = torch.zeros(n, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        graphed.train_steps(xd, td, w.lr, loss_g)
    torch.cuda.synchronize()
    for rep in range(3):
        eager.train_steps(xd, td, w.lr, loss_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss_e), f"replay {rep}: losses {loss_g.tolist()} vs {loss_e.tolist()}"
        for l, (a, b) in enumerate(zip(graphed.read_params(), eager.read_params())):
            assert torch.equal(a, b), f"replay {rep}: W{l} differs"
    eager.close()
    graphed.close()


@pytest.mark.parametrize("dims,B", [((1024, 1100, 260), 8), ((4096, 11008, 4096), 8)])
def test_train_steps_after_tuning_match_single_steps(torch_dev, dims, B):
    """After mlp_tune (which may change the first forward's K split, and so
    the merged first-layer launch's), a run of steps from given weights is
    bitwise the same session's single steps from the same weights."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"train_steps after tune dims={dims} B={B}")
    Ws = synth.make_weights(dims, "glorot", seed=71)
    steps, lr = 3, 0.05
    bs = [synth.make_batch(B, dims[0], dims[-1], "normal", seed=72, step=s)[:2] for s in range(steps)]
    xd, td = P.to_dev([np.stack([b[0] for b in bs]), np.stack([b[1] for b in bs])], dev)
    net = make_net(dims, B, "f32", Ws, dev)
    net.tune(xd[0], td[0], 2)
    out = []
    for mode in ("run", "single"):
        net.set_params(P.to_dev(Ws, dev))
        losses = torch.full((steps,), float("nan"), dtype=torch.float32, device=dev)
        if mode == "run":
            net.train_steps(xd, td, lr, losses)
        else:
            for s in range(steps):
                net.train_step_async(xd[s], td[s], lr, losses[s:s + 1])
        torch.cuda.synchronize()
        acts = [net.read_state(binding.STATE_ACT, l).cpu().numpy() for l in range(1, len(dims) - 1)]
        out.append((losses.cpu().numpy(), [w.cpu().numpy() for w in net.read_params()], acts))
    net.close()
    (la, wa, aa), (lb, wb, ab) = out
    assert np.all(np.isfinite(la)) and np.array_equal(la.view(np.uint32), lb.view(np.uint32))
    for u, v in zip(wa + aa, wb + ab):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))
