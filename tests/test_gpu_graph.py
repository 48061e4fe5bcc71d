"""The entry points under HIP graph capture (the benchmark replays its
launches from graphs).  Each graph holds one call of every kind; it is
replayed several times with the program's own eager work and
synchronisations in between (the outputs overwritten by a fill kernel, other
launches on the stream), and every replay must give the eager call's result
bit for bit (the kernels are deterministic: no atomics decide an order of
additions, no memsets are recorded).  The eager results themselves are
checked against the oracle elsewhere; here the oracle's quantizer supplies
the packed weights."""
import numpy as np
import pytest

import oracle
from group_wise_affine_aq_amd import inputs
from gpu_util import bits_to_dev, packed_to_dev, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def aq():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import group_wise_affine_aq_amd as mod
    mod.load_library()
    return mod


def _calls(aq):
    """(name, output tensor, callable writing it) for one call of each kind."""
    import torch
    N, K, G, bits = 300, 1024, 64, 4
    w = inputs.weights(N, K, seed=90, key=(90,))
    c, s, b = packed_to_dev(*oracle.quantize(w, G, bits))
    calls = []
    for M, xdt in ((1, "f16"), (4, "bf16"), (40, "bf16"), (300, "f16")):
        x = bits_to_dev(inputs.activations(M, K, xdt, seed=90, key=(M,)), xdt)
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
        calls.append((f"quantized_matmul M{M}", y,
                      lambda x=x, y=y: aq.aq_quantized_matmul(x, c, s, b, G, bits, y=y)))
    E, T, topk = 6, 20, 3
    ce, se, be = (np.stack(a) for a in zip(*[
        oracle.quantize(inputs.weights(N, K, seed=91, key=(e,)), G, bits) for e in range(E)]))
    dce, dse, dbe = packed_to_dev(ce, se, be)
    ids = to_dev(inputs.expert_ids(T, E, topk, seed=91))
    xg = bits_to_dev(inputs.activations(T, K, "f16", seed=91, key=(T,)), "f16")
    yg = torch.empty((T, topk, N), dtype=torch.float16, device=xg.device)
    calls.append(("gather_qmv", yg,
                  lambda: aq.aq_gather_qmv(xg, dce, dse, dbe, ids, G, bits, y=yg)))
    yq = torch.empty((N, K), dtype=torch.bfloat16, device=xg.device)
    calls.append(("dequantize", yq,
                  lambda: aq.aq_dequantize(c, s, b, G, bits, out=yq)))
    fc, fs = oracle.quantize_mxfp4(w)
    fc, fs = torch.from_numpy(fc.view(np.int32)).cuda(), torch.from_numpy(fs).cuda()
    for M in (1, 6):
        x = bits_to_dev(inputs.activations(M, K, "f16", seed=92, key=(M,)), "f16")
        y = torch.empty((M, N), dtype=x.dtype, device=x.device)
        calls.append((f"matmul_fp M{M}", y,
                      lambda x=x, y=y: aq.aq_matmul_fp(x, fc, fs, "mxfp4", 0, y=y)))
    fce = torch.stack([fc] * E)
    fse = torch.stack([fs] * E)
    yf = torch.empty((T, topk, N), dtype=torch.float16, device=xg.device)
    calls.append(("gather_matmul_fp", yf,
                  lambda: aq.aq_gather_matmul_fp(xg, fce, fse, ids, "mxfp4", 0, y=yf)))
    return calls


def test_graph_replays_match_eager(aq):
    import torch
    calls = _calls(aq)
    for _, _, f in calls:
        f()
    torch.cuda.synchronize()
    eager = [y.clone() for _, y, _ in calls]
    stream = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        for _, _, f in calls:  # warm-up on the capture stream
            f()
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=stream):
            for _, _, f in calls:
                f()
    torch.cuda.synchronize()
    junk = torch.empty(1 << 20, dtype=torch.float32, device="cuda")
    for rep in range(4):
        for _, y, _ in calls:  # outputs overwritten between replays
            y.view(torch.int16).fill_(0x7E00 + rep)
        junk.uniform_()  # other work on the default stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (name, y, _), ref in zip(calls, eager):
            assert torch.equal(y.view(torch.int16), ref.view(torch.int16)), \
                f"replay {rep}: {name} differs from the eager call"
