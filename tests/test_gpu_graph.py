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
    """(name, output tensor(s), callable writing them) for one call of each kind."""
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
    # the quantizers, the embedding, the prefill-size gather and the
    # block-scaled quantize / dequantize
    wd = to_dev(w)
    qo = aq.aq_quantize(wd, G, bits)
    calls.append(("quantize", qo, lambda: aq.aq_quantize(wd, G, bits, *qo)))
    mo = aq.aq_quantize_mse(wd, G, bits, 5)
    calls.append(("quantize_mse", mo, lambda: aq.aq_quantize_mse(wd, G, bits, 5, *mo)))
    zo = aq.aq_quantize_zp(wd, G, bits)
    calls.append(("quantize_zp", zo, lambda: aq.aq_quantize_zp(wd, G, bits, *zo)))
    tok = to_dev(inputs.token_ids(33, N, seed=93))
    ye = torch.empty((33, K), dtype=torch.bfloat16, device=xg.device)
    calls.append(("embedding", ye, lambda: aq.aq_embedding(tok, c, s, b, G, bits, out=ye)))
    Tq = 40
    idq = to_dev(inputs.expert_ids(Tq, E, topk, seed=94))
    xq = bits_to_dev(inputs.activations(Tq, K, "bf16", seed=94, key=(Tq,)), "bf16")
    yq2 = torch.empty((Tq, topk, N), dtype=torch.bfloat16, device=xg.device)
    calls.append(("gather_qmm", yq2,
                  lambda: aq.aq_gather_qmm(xq, dce, dse, dbe, idq, G, bits, y=yq2)))
    for mode, t in (("mxfp4", 0), ("nvfp4", -12), ("mxfp8", 0)):
        fo = aq.aq_quantize_fp(wd, mode, t)
        calls.append((f"quantize_fp {mode}", fo,
                      lambda mode=mode, t=t, fo=fo: aq.aq_quantize_fp(wd, mode, t, *fo)))
        yd = torch.empty((N, K), dtype=torch.bfloat16, device=xg.device)
        calls.append((f"dequantize_fp {mode}", yd,
                      lambda mode=mode, t=t, fo=fo, yd=yd:
                      aq.aq_dequantize_fp(*fo, K, mode, t, out=yd)))
    return calls


def _outs(o):
    return list(o) if isinstance(o, (tuple, list)) else [o]


def test_graph_replays_match_eager(aq):
    import torch
    calls = _calls(aq)
    for _, _, f in calls:
        f()
    torch.cuda.synchronize()
    eager = [[t.clone() for t in _outs(o)] for _, o, _ in calls]
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
        for _, o, _ in calls:  # outputs overwritten between replays
            for t in _outs(o):
                t.view(torch.uint8).fill_(0x7E + rep)
        junk.uniform_()  # other work on the default stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for (name, o, _), refs in zip(calls, eager):
            for t, ref in zip(_outs(o), refs):
                assert torch.equal(t.view(torch.uint8), ref.view(torch.uint8)), \
                    f"replay {rep}: {name} differs from the eager call"
