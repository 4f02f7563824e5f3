"""Two sessions on two streams at once: each context owns its workspace
(counters, partial sums, row losses), so steps of two sessions that run
concurrently on the GPU give the bits each gives alone."""
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


def _session(torch, dev, dims, B, precision, seed, stream):
    from mlp_gemm_softmax_amd import binding
    Ws = synth.make_weights(dims, "glorot", seed=seed)
    with torch.cuda.stream(stream):
        net = binding.Mlp(dims, B, precision, device=str(dev), stream=stream)
        net.set_params(P.to_dev(Ws, dev))
    xs, ts = [], []
    for s in range(4):
        x, t, _ = synth.make_batch(B, dims[0], dims[-1], "normal", seed=seed, step=s)
        xs.append(x)
        ts.append(t)
    xd, td = P.to_dev([np.stack(xs), np.stack(ts)], dev)
    return net, xd, td


PAIRS = [(((200, 300, 36), 64, "f32"), ((256, 520, 64), 8, "f32")),        # tiled + skinny (split-K counters in both)
         (((1024, 2048, 1040), 2048, "f32"), ((784, 128, 10), 1024, "f32")),  # 256x256 tiles + fused head
         (((2056, 2048, 1024), 2048, "bf16"), ((1024, 1100, 260), 16, "f32"))]


@pytest.mark.parametrize("a,b", PAIRS)
def test_concurrent_sessions_match_separate_runs(torch_dev, a, b):
    torch, dev = torch_dev
    print(f"\n[case] concurrent sessions {a} | {b}", flush=True)
    out = {}
    for mode in ("alone", "together"):
        sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
        na, xa, ta = _session(torch, dev, *a, seed=3, stream=sa)
        nb, xb, tb = _session(torch, dev, *b, seed=4, stream=sb)
        la = torch.zeros(4, dtype=torch.float32, device=dev)
        lb = torch.zeros(4, dtype=torch.float32, device=dev)
        torch.cuda.synchronize()
        if mode == "alone":
            for s in range(4):
                na.train_step_async(xa[s], ta[s], 0.05, la[s:s + 1])
            torch.cuda.synchronize()
            for s in range(4):
                nb.train_step_async(xb[s], tb[s], 0.05, lb[s:s + 1])
        else:
            for s in range(4):      # interleaved launches; the streams run them concurrently
                na.train_step_async(xa[s], ta[s], 0.05, la[s:s + 1])
                nb.train_step_async(xb[s], tb[s], 0.05, lb[s:s + 1])
        torch.cuda.synchronize()
        out[mode] = (la.cpu().numpy(), lb.cpu().numpy(),
                     [w.cpu().numpy() for w in na.read_params()], [w.cpu().numpy() for w in nb.read_params()])
        na.close()
        nb.close()
    A, T = out["alone"], out["together"]
    for u, v in zip(A[:2], T[:2]):
        assert np.array_equal(u.view(np.uint32), v.view(np.uint32))
    for ws_a, ws_t in zip(A[2:], T[2:]):
        for u, v in zip(ws_a, ws_t):
            assert np.array_equal(u.view(np.uint32), v.view(np.uint32))
