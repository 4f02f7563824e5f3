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


def test_sessions_on_host_threads(torch_dev):
    """Two host threads, each creating and driving its own session on its own
    stream (ctypes releases the interpreter lock during the library calls, so
    creation, planning and launches overlap on the host): the results equal
    those of the same sessions run one after the other."""
    import threading
    torch, dev = torch_dev
    print("\n[case] sessions on two host threads", flush=True)
    cases = [((200, 300, 36), 64, "f32", 5), ((256, 520, 64), 8, "f32", 6)]

    def drive(case, res, idx):
        dims, B, precision, seed = case
        s = torch.cuda.Stream()
        net, xd, td = _session(torch, dev, dims, B, precision, seed, s)
        torch.cuda.default_stream(dev).synchronize()   # the batches were copied on the default stream
        with torch.cuda.stream(s):
            losses = torch.zeros(40, dtype=torch.float32, device=dev)
            for k in range(40):
                net.train_step_async(xd[k % 4], td[k % 4], 0.05, losses[k:k + 1])
        s.synchronize()
        res[idx] = (losses.cpu().numpy(), [w.cpu().numpy() for w in net.read_params()])
        net.close()

    seq = [None, None]
    for i, c in enumerate(cases):
        drive(c, seq, i)
    par = [None, None]
    threads = [threading.Thread(target=drive, args=(c, par, i)) for i, c in enumerate(cases)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=120)
    assert all(r is not None for r in par)
    for (la, wa), (lb, wb) in zip(seq, par):
        assert np.array_equal(la.view(np.uint32), lb.view(np.uint32))
        for u, v in zip(wa, wb):
            assert np.array_equal(u.view(np.uint32), v.view(np.uint32))
