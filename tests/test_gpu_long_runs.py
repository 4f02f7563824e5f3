"""Long runs through the C ABI: the same seeded training run repeated gives
the same bits after thousands of steps (losses of every step and the final
weights), on the launch-bound, skinny and wide workloads; for the skinny
workload the runs of steps (mlp_train_steps, first-layer update fused with
the next forward) reach the same bits as single steps.  This catches a
reduction whose order or a ticket whose reset varies only now and then."""
import numpy as np
import pytest

from mlp_gemm_softmax_amd import synth

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


def _run(torch, dev, w, steps, mode):
    from mlp_gemm_softmax_amd import binding
    net = binding.Mlp(w.dims, w.batch, w.precision, device=str(dev))
    net.set_params([torch.from_numpy(a).to(dev) for a in synth.workload_weights(w)])
    nb = min(w.steps if w.fresh_batch else 1, 8)
    bs = [synth.workload_batch(w, s)[:2] for s in range(nb)]
    xs = torch.from_numpy(np.stack([b[0] for b in bs])).to(dev)
    ts = torch.from_numpy(np.stack([b[1] for b in bs])).to(dev)
    losses = torch.zeros(steps, dtype=torch.float32, device=dev)
    if mode == "single":
        for s in range(steps):
            net.train_step_async(xs[s % nb], ts[s % nb], w.lr, losses[s:s + 1])
    else:
        idx = torch.tensor([s % nb for s in range(steps)], device=dev)
        X, T = xs[idx].contiguous(), ts[idx].contiguous()
        for s0 in range(0, steps, 50):
            net.train_steps(X[s0:s0 + 50], T[s0:s0 + 50], w.lr, losses[s0:s0 + 50])
    torch.cuda.synchronize()
    W = [p.cpu().numpy() for p in net.read_params()]
    net.close()
    return losses.cpu().numpy(), W


@pytest.mark.parametrize("name,steps,modes", [("mnist_b32", 3000, ("single", "single")),
                                              ("mnist_b1024", 3000, ("single", "single")),
                                              ("skinny_b8", 1000, ("single", "single", "run")),
                                              ("wide_bf16", 200, ("single", "single")),
                                              ("wide_f32", 40, ("single", "single"))])
def test_long_runs_are_bitwise_repeatable(torch_dev, name, steps, modes):
    torch, dev = torch_dev
    print(f"\n[case] long run {name} steps={steps} modes={modes}", flush=True)
    w = synth.WORKLOADS[name]
    l0, W0 = _run(torch, dev, w, steps, modes[0])
    assert np.all(np.isfinite(l0))
    for m in modes[1:]:
        l, W = _run(torch, dev, w, steps, m)
        assert np.array_equal(l.view(np.uint32), l0.view(np.uint32)), f"{name} {m}: losses differ"
        for i, (a, b) in enumerate(zip(W, W0)):
            assert np.array_equal(a.view(np.uint32), b.view(np.uint32)), f"{name} {m}: W_{i} differs"
