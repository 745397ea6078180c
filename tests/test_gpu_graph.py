"""The GEMV entry points inside a captured HIP graph and on a non-default stream. A call only
enqueues kernels on the stream it is given (no allocation, no memset, no host synchronisation), so
a graph captured around it replays it: every replay, with the program's own eager work and
synchronisations in between, gives the bits of the eager call; so does a call on a side stream."""
import numpy as np
import pytest

import oracle
import synth
from gpu_cases import PN3T, PN4T, quantized
from test_gpu_pn import assert_within, dev_bytes

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_quantized_weight_pn3t_amd as pn
    return pn, torch, torch.device("cuda:0")


def setup(pn, torch, dev):
    """Four calls of a decode step: pn3t at one token (8-word pieces), pn4t at three tokens
    (4-word pieces), pn3t with x rotated in slices of 256 at one token (under capture rotated
    into a temporary), and a pn3t and a pn4t matrix that share x in one pn_gemv_group launch."""
    calls = []
    for typ, N, nb, M, seed, B in [(PN3T, 300, 64, 1, 12000, None), (PN4T, 77, 96, 3, 12001, None),
                                   (PN3T, 129, 16, 1, 12002, 256)]:
        G = oracle.PARAMS[typ][1]
        K = nb * G
        _, W = quantized(typ, N, K, seed)
        x = synth.activations(seed + 50, M, K)
        calls.append(dict(typ=typ, N=N, K=K, M=M, B=B, W=W, x=x, Wd=dev_bytes(torch, dev, W),
                          xd=torch.from_numpy(np.ascontiguousarray(x)).to(dev),
                          yd=torch.zeros((M, N), dtype=torch.float32, device=dev)))
    K = 5120
    x = synth.activations(12060, 1, K)
    parts = []
    for typ, N, seed in [(PN3T, 300, 12061), (PN4T, 130, 12062)]:
        _, W = quantized(typ, N, K, seed)
        parts.append(dict(typ=typ, N=N, W=W, Wd=dev_bytes(torch, dev, W),
                          yd=torch.zeros((1, N), dtype=torch.float32, device=dev)))
    calls.append(dict(group=parts, K=K, M=1, B=None, x=x,
                      xd=torch.from_numpy(np.ascontiguousarray(x)).to(dev),
                      yd=torch.zeros((1, 1), dtype=torch.float32, device=dev)))
    return calls


def outputs(c):
    return [p["yd"] for p in c["group"]] if "group" in c else [c["yd"]]


def launch(pn, c, stream):
    if "group" in c:
        pn.gemv_group([(p["typ"], p["Wd"], p["N"], p["yd"]) for p in c["group"]], c["K"], c["xd"],
                      stream=stream)
    elif c["B"] is None:
        pn.gemv(c["typ"], c["Wd"], c["N"], c["K"], c["xd"], c["yd"], stream=stream)
    else:
        pn.gemv_hadamard(c["typ"], c["Wd"], c["N"], c["K"], c["xd"], c["B"], c["yd"], stream=stream)


def test_graph_replays_give_eager_bits(env):
    pn, torch, dev = env
    calls = setup(pn, torch, dev)
    s = torch.cuda.Stream()
    # eager, on the side stream (also the first call of each kernel, outside any capture)
    with torch.cuda.stream(s):
        for c in calls:
            launch(pn, c, s)
    s.synchronize()
    eager = [[y.clone() for y in outputs(c)] for c in calls]
    for c in calls:
        for p in c.get("group", [c] if c["B"] is None else []):
            y_ref, bound = oracle.gemv(p["typ"], p["W"], p["N"], c["K"], c["x"])
            assert_within(p["yd"].cpu().numpy(), y_ref, bound)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in calls:
            launch(pn, c, s)
    for rep in range(4):
        for c in calls:
            for y in outputs(c):
                y.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for c, e in zip(calls, eager):
            for y, ye in zip(outputs(c), e):
                assert torch.equal(y.view(torch.int32), ye.view(torch.int32)), f"replay {rep}"
    # the default stream gives the same bits as the side stream
    for c in calls:
        for y in outputs(c):
            y.zero_()
        launch(pn, c, torch.cuda.current_stream())
    torch.cuda.synchronize()
    for c, e in zip(calls, eager):
        for y, ye in zip(outputs(c), e):
            assert torch.equal(y.view(torch.int32), ye.view(torch.int32))
