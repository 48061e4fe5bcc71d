"""Seeded synthetic inputs for the quantized-matmul workloads.

This module only draws random numbers and converts between number formats;
it holds none of the quantization arithmetic.  Both the HIP path and the CPU
oracle consume exactly the arrays made here.

Generator: numpy ``PCG64`` seeded through ``SeedSequence(seed, spawn_key=...)``
so that every (workload, tensor role, shape) draws from its own substream.
Values are drawn in float64; weights are cast to float32, activations are
rounded to fp16 (numpy, round-to-nearest-even) or to bf16 (torch CPU cast,
round-to-nearest-even).

Workloads (the shapes discussed on the pages: Llama-3-8B decode matrices,
the 70B MLP up-projection, an MoE expert stack):
  tiny      W fp32 [512, 512] ~ N(0, 0.02), 4-bit G=64; x fp16 [1, 512] ~ N(0, 1)
  decode    W [N, K] in {[4096,4096], [1024,4096], [14336,4096], [4096,14336]},
            N(0, 0.02) with round(0.001*N*K) distinct entries scaled by 20;
            4-bit G=64; x fp16 [1, K] ~ N(0, 1)
  specdec   x bf16 [M, K], M in {2,3,4,6,8}; W [14336,4096] and [4096,14336]
            ~ N(0, 0.02); 4-bit G=64 and 8-bit G=128; also M in {16, 64}
            (a batch of decoding sequences)
  prefill   X bf16 [2048, 8192] ~ N(0, 1); W [28672, 8192] ~ N(0, 0.02) at
            4-bit G=64, 3-bit G=64 and 2-bit G=32
  moe       64 experts W_e [1408, 2048] ~ N(0, 0.02) 4-bit G=64; x fp16
            [32, 2048] ~ N(0, 1); ids [32, 6] = first 6 of a seeded
            permutation of the 64 experts, per token
  embedding table [128256, 4096] ~ N(0, 0.02) (a Llama-3-8B vocabulary) at
            8-bit G=128; token ids uniform over the vocabulary, T = 1
            (decode) and T = 2048 (prefill); bf16 output
"""
from __future__ import annotations

import numpy as np

ROLE_W, ROLE_OUTLIER, ROLE_X, ROLE_IDS = 1, 2, 3, 4

WORKLOADS = {
    "tiny": dict(shapes=[(512, 512)], bits=[4], group_size=[64], M=[1], x_dtype="f16",
                 outliers=False),
    "decode": dict(shapes=[(4096, 4096), (1024, 4096), (14336, 4096), (4096, 14336)], bits=[4],
                   group_size=[64], M=[1], x_dtype="f16", outliers=True),
    "specdec": dict(shapes=[(14336, 4096), (4096, 14336)], bits=[4, 8], group_size=[64, 128],
                    M=[2, 3, 4, 6, 8], M_batch=[16, 64], x_dtype="bf16", outliers=False),
    "prefill": dict(shapes=[(28672, 8192)], bits=[4, 3, 2], group_size=[64, 64, 32], M=[2048],
                    x_dtype="bf16", outliers=False),
    "moe": dict(shapes=[(1408, 2048)], experts=64, tokens=32, topk=6, bits=[4], group_size=[64],
                x_dtype="f16", outliers=False, prefill_tokens=2048),
    "embedding": dict(shapes=[(128256, 4096)], bits=[8], group_size=[128], tokens=[1, 2048],
                      out_dtype="bf16", outliers=False),
}
WORKLOAD_ID = {name: i for i, name in enumerate(WORKLOADS)}


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=key)))


def weights(N: int, K: int, *, seed: int = 0, key=(0,), std: float = 0.02,
            outliers: bool = False) -> np.ndarray:
    """float32 [N, K] ~ N(0, std); with ``outliers`` exactly round(0.001*N*K)
    distinct entries (chosen uniformly without replacement) are multiplied by 20."""
    w = _rng(seed, ROLE_W, N, K, *key).standard_normal((N, K)) * std
    if outliers:
        n_out = int(round(0.001 * N * K))
        pos = _rng(seed, ROLE_OUTLIER, N, K, *key).choice(N * K, size=n_out, replace=False)
        w.reshape(-1)[pos] *= 20.0
    return w.astype(np.float32)


def same_sign_weights(N: int, K: int, G: int, *, seed: int = 0, key=(0,),
                      std: float = 0.02) -> np.ndarray:
    """float32 [N, K] whose groups of G along a row each share one sign:
    |N(0, std)| + std/2, negated in every other group, and in every third
    group one member (at a seeded position) multiplied by 8."""
    r = _rng(seed, ROLE_W, N, K, G, *key)
    w = np.abs(r.standard_normal((N, K))) * std + std / 2
    grp = w.reshape(N, K // G, G)
    grp[:, 1::2, :] *= -1.0
    far = r.integers(0, G, size=(N, K // G))
    rows, gs = np.nonzero(np.broadcast_to(np.arange(K // G) % 3 == 0, (N, K // G)))
    grp[rows, gs, far[rows, gs]] *= 8.0
    return w.astype(np.float32)


def activations(M: int, K: int, dtype: str, *, seed: int = 0, key=(0,)) -> np.ndarray:
    """uint16 bit patterns [M, K] of fp16 or bf16 values ~ N(0, 1)."""
    x = _rng(seed, ROLE_X, M, K, *key).standard_normal((M, K))
    return to_bits(x, dtype)


def expert_ids(T: int, E: int, topk: int, *, seed: int = 0, key=(0,)) -> np.ndarray:
    """int32 [T, topk]: per token, the first ``topk`` entries of a seeded
    permutation of range(E) (distinct, uniformly chosen experts)."""
    r = _rng(seed, ROLE_IDS, T, E, topk, *key)
    return np.stack([r.permutation(E)[:topk] for _ in range(T)]).astype(np.int32)


def token_ids(T: int, V: int, *, seed: int = 0, key=(0,)) -> np.ndarray:
    """int32 [T] token ids, uniform over range(V) (with repeats)."""
    return _rng(seed, ROLE_IDS, T, V, *key).integers(0, V, size=T).astype(np.int32)


# --- number-format plumbing ------------------------------------------------------
def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64/float32 values to fp16 or bf16 (nearest-even); uint16 bits."""
    if dtype == "f16":
        return np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float16)).view(
            np.uint16)
    if dtype == "bf16":
        import torch
        t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    raise ValueError(dtype)


def from_bits(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 fp16/bf16 bit patterns -> exact float64 values."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


# --- device-side generation for benchmark-sized inputs ----------------------------------
def _torch_gen(device, seed: int, *key: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(np.random.SeedSequence(seed, spawn_key=key).generate_state(1)[0]))
    return g


def weights_device(N: int, K: int, *, device="cuda", seed: int = 0, key=(0,), std: float = 0.02,
                   outliers: bool = False):
    """Same distribution as ``weights`` drawn on the device with torch's seeded
    generator (benchmark-sized matrices; the tests use the numpy streams)."""
    import torch
    g = _torch_gen(device, seed, ROLE_W, N, K, *key)
    w = torch.randn((N, K), generator=g, device=device, dtype=torch.float32) * std
    if outliers:
        n_out = int(round(0.001 * N * K))
        go = _torch_gen(device, seed, ROLE_OUTLIER, N, K, *key)
        pos = torch.randperm(N * K, generator=go, device=device)[:n_out]
        w.view(-1)[pos] *= 20.0
    return w


def activations_device(M: int, K: int, dtype: str, *, device="cuda", seed: int = 0, key=(0,)):
    """x ~ N(0, 1) rounded to fp16/bf16 on the device (torch casts round to nearest even)."""
    import torch
    g = _torch_gen(device, seed, ROLE_X, M, K, *key)
    x = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    return x.to(torch.float16 if dtype == "f16" else torch.bfloat16)
