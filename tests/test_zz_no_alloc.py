"""The allocation-free training step (mlp_train_step_static) against the
workspace entry point it varies (mlp_create + mlp_train_step_async): the same
kernels and plans, so losses and updated weights must agree bit for bit,
over consecutive calls whose configurations shrink and change (each change
re-plans inside the same static buffer and clears its counters)."""
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


# (dims, batch): a tiled product with split-K, the README MLP at batch 1024
# (fused output layer), the same MLP at a smaller batch, a skinny batch
SEQUENCE = [((320, 2080, 40), 512), ((784, 128, 10), 1024), ((784, 128, 10), 256), ((256, 520, 64), 8)]


def _run_pair(torch, dev, dims, B, seed, steps=2, lr=0.05):
    from mlp_gemm_softmax_amd import binding
    print(f"\n[case] static step dims={dims} B={B}", flush=True)
    Ws = synth.make_weights(dims, "glorot", seed=seed)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=seed + 1)
    xd, td = P.to_dev([x, t], dev)
    ref = binding.Mlp(dims, B, "f32", device=str(dev))
    ref.set_params(P.to_dev(Ws, dev))
    weights = P.to_dev(Ws, dev)
    loss_ref = torch.zeros(1, dtype=torch.float32, device=dev)
    loss_st = torch.zeros(1, dtype=torch.float32, device=dev)
    for _ in range(steps):
        ref.train_step_async(xd, td, lr, loss_ref)
        binding.train_step_static(dims, B, weights, xd, td, lr, loss_st)
        torch.cuda.synchronize()
        assert torch.equal(loss_ref, loss_st), f"{dims} B={B}: loss {loss_st.item()} vs {loss_ref.item()}"
        for l, (a, b) in enumerate(zip(ref.read_params(), weights)):
            assert torch.equal(a, b), f"{dims} B={B}: W{l} differs"
    assert np.isfinite(loss_st.item()) and loss_st.item() > 0
    ref.close()


def test_static_step_matches_workspace_step(torch_dev):
    torch, dev = torch_dev
    for i, (dims, B) in enumerate(SEQUENCE):
        _run_pair(torch, dev, dims, B, seed=300 + i)


def test_static_step_seeded_sequence(torch_dev):
    """Twelve seeded configurations in a row (widths 4-1040, batches 1-512),
    each re-planned in the same static buffer: every one matches the
    workspace step bit for bit."""
    torch, dev = torch_dev
    rng = np.random.default_rng([2026, 17])
    widths = [4, 10, 31, 64, 100, 260, 520, 1040]
    for i in range(12):
        L = int(rng.integers(1, 4))
        dims = tuple(int(rng.choice(widths)) for _ in range(L + 1))
        B = int(rng.choice([1, 3, 8, 16, 64, 512]))
        _run_pair(torch, dev, dims, B, seed=500 + i)


def test_static_step_after_a_larger_one_and_errors(torch_dev):
    """A larger configuration, then a smaller one (the second call re-plans
    in the buffer the first one filled); a configuration beyond the buffer
    is refused and the next call still runs."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    _run_pair(torch, dev, (784, 128, 10), 2048, seed=400, steps=1)
    w = synth.WORKLOADS["wide_f32"]
    xs = torch.zeros((w.batch, w.dims[0]), dtype=torch.float32, device=dev)
    ts = torch.zeros((w.batch, w.dims[-1]), dtype=torch.float32, device=dev)
    ws = [torch.zeros((a, b), dtype=torch.float32, device=dev) for a, b in zip(w.dims[:-1], w.dims[1:])]
    with pytest.raises(binding.MlpError) as ei:
        binding.train_step_static(w.dims, w.batch, ws, xs, ts, 0.01)
    assert ei.value.status == binding.MLP_ERR_WORKSPACE
    _run_pair(torch, dev, (784, 128, 10), 32, seed=401, steps=2)


@pytest.mark.parametrize("name", ["mnist_b1024", "skinny_b8"])
def test_static_step_under_graph_capture(torch_dev, name):
    """The use the call is for: a step captured into a HIP graph
    (torch.cuda.graph) after one warm-up call has built the plan for this
    configuration and stream, replayed three times with eager work and
    synchronisations between the replays; every replay equals a workspace
    step bit for bit."""
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    w = synth.WORKLOADS[name]
    print(f"\n[case] static step under capture {name}", flush=True)
    Ws = synth.workload_weights(w)
    x, t, _ = synth.workload_batch(w)
    xd, td = P.to_dev([x, t], dev)
    eager = binding.Mlp(w.dims, w.batch, "f32", device=str(dev))
    eager.set_params(P.to_dev(Ws, dev))
    s = torch.cuda.Stream(device=dev)
    warm = P.to_dev(Ws, dev)          # a throw-away copy: the warm-up trains it
    weights = P.to_dev(Ws, dev)
    loss_e = torch.zeros(1, dtype=torch.float32, device=dev)
    loss_g = torch.zeros(1, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    binding.train_step_static(w.dims, w.batch, warm, xd, td, w.lr, loss_g, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        binding.train_step_static(w.dims, w.batch, weights, xd, td, w.lr, loss_g, stream=s)
    torch.cuda.synchronize()
    for step in range(3):
        eager.train_step_async(xd, td, w.lr, loss_e)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(loss_g, loss_e), f"step {step}: loss {loss_g.item()} vs {loss_e.item()}"
        for l, (a, b) in enumerate(zip(eager.read_params(), weights)):
            assert torch.equal(a, b), f"step {step}: W{l} differs"
    eager.close()
