"""The C ABI from a C program (tests/abi_c_step.c, built next to libmlp.so
by the package's build step): device memory from hipMalloc, no Python or
PyTorch in that process.  Its gradients, losses and updated weights must be
the bits the Python binding gets from the same library on the same inputs
(the binding's results are the ones the oracle tests check)."""
import os
import subprocess

import numpy as np
import pytest

from mlp_gemm_softmax_amd import synth
from tests import parity as P

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CLIENT = os.path.join(ROOT, "mlp_gemm_softmax_amd", "c_client_step")


@pytest.fixture(scope="module")
def torch_dev():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch, torch.device("cuda:0")


@pytest.mark.parametrize("dims,B", [((96, 160, 40), 64),      # tiled kernels
                                    ((784, 128, 10), 32),     # fused output layer
                                    ((256, 520, 64), 8),      # skinny kernels
                                    ((64, 12), 5)])           # one layer
def test_c_client_matches_the_binding(torch_dev, tmp_path, dims, B):
    if not os.path.exists(CLIENT):
        pytest.skip("C client not built (python -m mlp_gemm_softmax_amd.build)")
    from mlp_gemm_softmax_amd import binding
    torch, dev = torch_dev
    print(f"\n[case] C client dims={dims} B={B}", flush=True)
    Ws = synth.make_weights(dims, "glorot", seed=B + 41)
    x, t, _ = synth.make_batch(B, dims[0], dims[-1], "uniform01", seed=B + 42)
    lr = 0.05
    x.astype(np.float32).tofile(tmp_path / "x.f32")
    t.astype(np.float32).tofile(tmp_path / "labels.f32")
    for l, W in enumerate(Ws):
        W.astype(np.float32).tofile(tmp_path / f"w{l}.f32")
    res = subprocess.run([CLIENT, str(tmp_path), str(B), repr(lr), *map(str, dims)],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    words = res.stdout.split()
    loss_g, loss_s = np.float32(words[1]), np.float32(words[3])

    net = binding.Mlp(dims, B, "f32", device=str(dev))
    net.set_params(P.to_dev(Ws, dev))
    xd, td = P.to_dev([x, t], dev)
    pg, pdw, _ = net.grads(xd, td)
    ps = net.train_step(xd, td, lr)
    pw = [w.cpu().numpy() for w in net.read_params()]
    net.close()
    assert loss_g == np.float32(pg) and loss_s == np.float32(ps)
    for l, W in enumerate(Ws):
        cdw = np.fromfile(tmp_path / f"dw{l}.f32", dtype=np.float32).reshape(W.shape)
        cw = np.fromfile(tmp_path / f"w{l}_out.f32", dtype=np.float32).reshape(W.shape)
        assert np.array_equal(cdw.view(np.uint32), pdw[l].cpu().numpy().view(np.uint32)), f"dW_{l}"
        assert np.array_equal(cw.view(np.uint32), pw[l].view(np.uint32)), f"W_{l}"
