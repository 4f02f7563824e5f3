"""Debug modes through the C ABI: the serial mode (a wait after every launch)
and the workspace guard bands.  A session with both modes on must give the
same bits as one without them, on shapes that reach every kernel family,
and the guard check must pass there (no kernel writes past the end of a
workspace buffer).  A band the caller overwrites from the host must be
reported, naming the buffer it follows."""
import numpy as np
import pytest

from mlp_gemm_softmax_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _announce(msg):
    print(f"\n[case] {msg}", flush=True)


def _net(dims, B, precision, Ws, dev, flags):
    from mlp_gemm_softmax_amd import binding
    net = binding.Mlp(dims, B, precision, device=str(dev))
    net.set_params(P.to_dev(Ws, dev))
    net.set_debug(flags)
    return net


def _bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32) if a.dtype == np.float32 else a


DEBUG_CASES = [
    # dims, B, precision
    ((200, 300, 36), 64, "f32"),          # tiled kernels, split-K in dW
    ((96, 160, 130, 40), 128, "f32"),     # three layers
    ((320, 2080, 40), 512, "f32"),        # tiled NN with split-K, ragged N
    ((512, 2048, 16), 1024, "f32"),       # fused output layer with tiled GEMMs
    ((1024, 2048, 1040), 2048, "f32"),    # 256x256 f32 tiles, K splits
    ((256, 520, 64), 8, "f32"),           # skinny kernels, ragged column group
    ((1024, 1100, 260), 16, "f32"),       # skinny forward K splits (partials, counters)
    ((64, 100, 1040), 8, "f32"),          # skinny dX + dW with its columns split
    ((64, 32, 8), 8, "f32"),              # fused output layer with skinny kernels
    ((4096, 11008, 4096), 8, "f32"),      # the skinny batch-8 workload
    ((33, 70, 17, 10), 37, "f32"),        # widths not multiples of 4
    ((100, 31, 7), 5, "f32"),
    ((1, 1, 1), 1, "f32"),
    ((5, 3), 3, "f32"),                   # no hidden layer
    ((2052, 36, 20), 3, "f32"),
    ((200, 300, 36), 64, "bf16"),
    ((33, 70, 17, 10), 37, "bf16"),       # bf16 with ragged widths (byte-sized tails)
    ((2056, 4096, 1024), 2048, "bf16"),   # 256-wide bf16 tiles in all three layouts
]


@pytest.mark.parametrize("dims,B,precision", DEBUG_CASES)
def test_debug_modes_change_no_bits_and_guards_hold(torch_dev, dims, B, precision):
    """Forward, probabilities, gradients, two steps and (for batches of at
    most 8 float32 rows) a fused run of three steps, each with the serial mode and
    the guard check on, equal the same calls without them bit for bit; every
    call's guard check passes."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"debug dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=sum(dims) + 3 * B)
    batches = [synth.make_batch(B, dims[0], dims[-1], "normal", seed=B + 11, step=s)[:2] for s in range(3)]
    xs = P.to_dev([np.stack([b[0] for b in batches]), np.stack([b[1] for b in batches])], dev)
    (x, t), (x1, t1) = P.to_dev(batches[0], dev), P.to_dev(batches[1], dev)
    # a run of steps needs every batch 16-byte aligned inside the stacked arrays
    run = precision == "f32" and B <= 8 and (B * dims[0]) % 4 == 0 and (B * dims[-1]) % 4 == 0
    lr = 0.05
    out = []
    for flags in (0, binding.DEBUG_SYNC | binding.DEBUG_GUARDS):
        net = _net(dims, B, precision, Ws, dev, flags)
        r = []
        logits, loss_f = net.forward(x, t)
        r += [logits.cpu().numpy(), np.float32(loss_f)]
        r.append(net.forward_probs(x).cpu().numpy())
        loss_g, dws, dl = net.grads(x, t)
        r += [np.float32(loss_g), dl.cpu().numpy()] + [d.cpu().numpy() for d in dws]
        r.append(np.float32(net.train_step(x, t, lr)))
        r.append(np.float32(net.train_step(x1, t1, lr)))
        if run:
            losses = torch.zeros(3, dtype=torch.float32, device=dev)
            net.train_steps(xs[0], xs[1], lr, losses)
            torch.cuda.synchronize()
            r.append(losses.cpu().numpy())
        r += [w.cpu().numpy() for w in net.read_params()]
        out.append(r)
        net.close()
    plain, debug = out
    assert len(plain) == len(debug)
    for i, (a, b) in enumerate(zip(plain, debug)):
        assert np.array_equal(_bits(a), _bits(b)), f"result {i} differs with the debug modes on"


def _ends(net):
    """Byte offsets inside the first and the last guard band: just past the
    end of W_0 (the workspace starts with the float32 weights) and the
    workspace's last byte (the band after the loss slot)."""
    return net.dims[0] * net.dims[1] * 4, net.workspace.numel() - 1


@pytest.mark.parametrize("dims,B,precision", [((96, 160, 40), 64, "f32"),
                                              ((256, 520, 64), 8, "f32"),
                                              ((33, 70, 17, 10), 37, "bf16")])
def test_overwritten_guard_is_reported(torch_dev, dims, B, precision):
    """A byte of a guard band changed by the caller (the only way to force
    the condition without a faulty kernel) makes the next call that runs
    kernels fail with MLP_ERR_GUARD naming the buffer before the band; the
    context is then poisoned until every layer is set again, after which the
    bands hold again and steps equal those of a fresh session."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"guard dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=5)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=6)
    xd, td = P.to_dev([x, t], dev)
    Wd = P.to_dev(Ws, dev)
    net = _net(dims, B, precision, Ws, dev, binding.DEBUG_GUARDS)
    net.train_step(xd, td, 0.05)
    for off, name, call in [(_ends(net)[0], "W0", lambda: net.train_step(xd, td, 0.05)),
                            (_ends(net)[1], "loss", lambda: net.forward(xd, td))]:
        before = int(net.workspace[off].item())
        assert before == 0xA5
        net.workspace[off] = 0x5A
        with pytest.raises(binding.MlpError) as ei:
            call()
        assert ei.value.status == binding.MLP_ERR_GUARD
        msg = str(ei.value)
        assert f"after {name} " in msg and "0x5a" in msg, msg
        assert int(net.workspace[off].item()) == 0xA5      # the band was rewritten
        with pytest.raises(binding.MlpError) as ei:
            net.train_step(xd, td, 0.05)
        assert ei.value.status == binding.MLP_ERR_STATE
        net.set_params(Wd)
    # after the reset the checks pass and the session computes what a fresh one does
    loss = net.train_step(xd, td, 0.05)
    W_after = [w.cpu().numpy() for w in net.read_params()]
    fresh = _net(dims, B, precision, Ws, dev, 0)
    loss_ref = fresh.train_step(xd, td, 0.05)
    assert np.float32(loss) == np.float32(loss_ref)
    for a, b in zip(W_after, fresh.read_params()):
        assert np.array_equal(_bits(a), _bits(b.cpu().numpy()))
    # with the modes off a changed band goes unnoticed by design
    net.set_debug(0)
    net.workspace[_ends(net)[1]] = 0
    net.train_step(xd, td, 0.05)
    net.close()
    fresh.close()


def test_debug_flags_are_checked(torch_dev):
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    net = binding.Mlp((8, 4, 2), 2, "f32", device=str(dev))
    for bad in (4, 8, -1):
        with pytest.raises(binding.MlpError) as ei:
            net.set_debug(bad)
        assert ei.value.status == binding.MLP_ERR_ARG
    net.set_debug(binding.DEBUG_SYNC)
    net.set_debug(0)
    net.close()


@pytest.mark.parametrize("dims,B,precision", [((200, 300, 36), 64, "f32"),
                                              ((320, 2080, 40), 512, "f32"),
                                              ((1024, 2048, 1000), 2048, "bf16"),
                                              ((784, 128, 10), 4096, "f32"),
                                              ((512, 2048, 1040), 8, "f32")])
def test_tuning_candidates_stay_inside_their_buffers(torch_dev, dims, B, precision):
    """mlp_tune times other tile shapes and K splits than the ones planned at
    creation; with the guard check on, none of them writes past a buffer
    (split-K partials and counters included), and the tuned steps keep the
    bands intact."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"tune guards dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=61)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=62)
    xd, td = P.to_dev([x, t], dev)
    net = _net(dims, B, precision, Ws, dev, binding.DEBUG_GUARDS)
    net.tune(xd, td, 1)
    net.grads(xd, td)
    net.train_step(xd, td, 0.05)
    net.close()


@pytest.mark.parametrize("dims,B,precision,rule", [((256, 520, 64), 8, "f32", "adam"),
                                                   ((200, 300, 36), 64, "f32", "laprop"),
                                                   ((2056, 4096, 1024), 2048, "bf16", "adam")])
def test_debug_modes_with_adaptive_rules(torch_dev, dims, B, precision, rule):
    """Adam / LaProp steps (the moments live in caller memory, outside the
    workspace) keep the guard bands intact and give the bits of the same
    steps without the debug modes."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _announce(f"debug {rule} dims={dims} B={B} {precision}")
    Ws = synth.make_weights(dims, "glorot", seed=sum(dims) + 7)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=B + 13)
    xd, td = P.to_dev([x, t], dev)
    out = []
    for flags in (0, binding.DEBUG_SYNC | binding.DEBUG_GUARDS):
        net = _net(dims, B, precision, Ws, dev, flags)
        net.set_optimizer(rule, 0.9, 0.999, 1e-8)
        losses = [np.float32(net.train_step(xd, td, 1e-3)) for _ in range(3)]
        out.append((losses, [w.cpu().numpy() for w in net.read_params()]))
        net.close()
    (la, wa), (lb, wb) = out
    assert np.array_equal(np.array(la, np.float32).view(np.uint32), np.array(lb, np.float32).view(np.uint32))
    for u, v in zip(wa, wb):
        assert np.array_equal(_bits(u), _bits(v))


def test_debug_modes_from_the_environment(torch_dev, monkeypatch):
    """MLP_DEBUG=guards turns the guard check on for every new session."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    monkeypatch.setenv("MLP_DEBUG", "guards")
    dims, B = (96, 160, 40), 64
    Ws = synth.make_weights(dims, "glorot", seed=9)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=10)
    xd, td = P.to_dev([x, t], dev)
    net = binding.Mlp(dims, B, "f32", device=str(dev))
    net.set_params(P.to_dev(Ws, dev))
    net.train_step(xd, td, 0.05)
    net.workspace[net.workspace.numel() - 1] = 0
    with pytest.raises(binding.MlpError) as ei:
        net.train_step(xd, td, 0.05)
    assert ei.value.status == binding.MLP_ERR_GUARD
    net.close()
