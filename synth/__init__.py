"""Seeded synthetic inputs for the W8A8 FP8 linear path.

This module only draws numbers. It holds none of the method's arithmetic:
no FP8 encoding, no quantisation, no matrix product. Both the CPU oracle
and the GPU path receive the arrays made here, so neither depends on the
other.

Workloads (shapes and value distributions) follow the dense projection and
routed-expert settings that the Metis-1.6 pages describe: activations are
per-token BF16 rows, weights are [out, in] rows with a scale for each
output row (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4"; Lernex/Metis-1.6-
Logos-FP8, "What is in FP8"), the routed experts are stored in global
expert order and each token picks the top-k of them (Lernex/Metis-1.6-
Praxis, "Architecture").

Recipe (all draws from one ``numpy.random.default_rng(seed)``, PCG64, in
this order: activations, outlier channels, weights, routing):

* activations: ``standard_normal(shape, float32)``; ``n_outlier`` channels
  picked by ``rng.choice(K, n_outlier, replace=False)`` are multiplied by
  20 in float32; then one round-to-nearest-even to BF16.
* weights: ``0.02 * standard_normal(shape, float32)``, then BF16.
* routing (per pass): ``rank = rng.permutation(E) + 1``, expert prior
  ``p ~ rank**-1.1`` (Zipf, s = 1.1), logits ``N(0,1)[T,E] + ln p``,
  softmax, top-k by probability (lower expert id first on ties), router
  weights = the top-k probabilities renormalised to sum to one (float32).

The float32 -> BF16 rounding of inputs uses torch's CPU cast, which rounds
to nearest even; BF16 values travel as uint16 bit patterns.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "activations",
    "weights",
    "routing",
    "dense_workload",
    "moe_workload",
    "DENSE_SMALL",
    "DENSE_PREFILL",
    "DENSE_DECODE",
    "MOE_GATE_UP",
    "MOE_TWO_PASS",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 array -> BF16 bit patterns (uint16), round to nearest even."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32, exact widening."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(rng: np.random.Generator, M: int, K: int, n_outlier: int = 0) -> np.ndarray:
    """BF16 bits [M, K]: N(0,1) with ``n_outlier`` channels scaled by 20."""
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_outlier:
        ch = rng.choice(K, n_outlier, replace=False)
        x[:, ch] *= np.float32(20.0)
    return f32_to_bf16_bits(x)


def weights(rng: np.random.Generator, shape, std: float = 0.02) -> np.ndarray:
    """BF16 bits of ``std * N(0,1)`` drawn in float32."""
    w = rng.standard_normal(shape, dtype=np.float32)
    w *= np.float32(std)
    return f32_to_bf16_bits(w)


def routing(rng: np.random.Generator, T: int, E: int, k: int, zipf_s: float = 1.1):
    """Top-k routing with a Zipf prior over experts.

    Returns ``(ids int32 [T,k], w float32 [T,k])``. Within a token the ids
    are distinct and ordered by descending probability (stable, so the
    lower id comes first on a tie).
    """
    rank = rng.permutation(E) + 1
    prior = rank.astype(np.float64) ** (-zipf_s)
    prior /= prior.sum()
    logits = rng.standard_normal((T, E), dtype=np.float32).astype(np.float64) + np.log(prior)[None, :]
    logits -= logits.max(axis=1, keepdims=True)
    probs = np.exp(logits)
    probs /= probs.sum(axis=1, keepdims=True)
    ids = np.argsort(-probs, axis=1, kind="stable")[:, :k]
    top = np.take_along_axis(probs, ids, axis=1)
    w = (top / top.sum(axis=1, keepdims=True)).astype(np.float32)
    return ids.astype(np.int32), w


# Named workloads (sizes as used by the tests and the benchmark).
DENSE_SMALL = dict(name="dense_64x1024x1024", M=64, K=1024, N=1024, n_outlier=8)
DENSE_PREFILL = dict(name="prefill_4096x6144x2048", M=4096, K=2048, N=6144, n_outlier=20)
DENSE_DECODE = dict(name="decode_Mx8192x2048", M=8, K=2048, N=8192, n_outlier=0)
MOE_GATE_UP = dict(name="moe_gate_up_T4096_H2048_I512_E64_k8", T=4096, H=2048, I=512, E=64, k=8,
                   n_outlier=20, passes=1)
MOE_TWO_PASS = dict(name="moe_ffn_2pass_T16384_H2048_I512_E64_k8", T=16384, H=2048, I=512, E=64,
                    k=8, n_outlier=20, passes=2)
# The model pages' own expert shapes: 128 (Praxis) or 192 (Logos) routed experts
# in a 1,024-wide latent space, four per token ("Architecture" sections). The
# expert intermediate width is not on the pages: 512 here, a parameter.
MOE_PRAXIS = dict(name="moe_ffn_2pass_T4096_H1024_I512_E128_k4", T=4096, H=1024, I=512, E=128, k=4,
                  n_outlier=10, passes=2)
MOE_LOGOS = dict(name="moe_ffn_2pass_T4096_H1024_I512_E192_k4", T=4096, H=1024, I=512, E=192, k=4,
                 n_outlier=10, passes=2)


def dense_workload(M: int, K: int, N: int, n_outlier: int = 0, seed: int = 0, **_):
    """Activations then weights: ``{'x': bf16 [M,K], 'w': bf16 [N,K]}``."""
    rng = np.random.default_rng(seed)
    x = activations(rng, M, K, n_outlier)
    w = weights(rng, (N, K))
    return {"x": x, "w": w, "seed": seed, "draw_order": "x, outlier channels, w"}


def moe_workload(T: int, H: int, I: int, E: int, k: int, n_outlier: int = 0, passes: int = 1,
                 seed: int = 0, with_w2: bool = True, **_):
    """Tokens, expert weights and per-pass routing.

    ``w13`` is [E, 2I, H] with rows 0..I-1 the gate and rows I..2I-1 the up
    projection of each expert; ``w2`` is [E, H, I]. Experts are stacked in
    global expert order.
    """
    rng = np.random.default_rng(seed)
    x = activations(rng, T, H, n_outlier)
    w13 = weights(rng, (E, 2 * I, H))
    w2 = weights(rng, (E, H, I)) if with_w2 else None
    routes = [routing(rng, T, E, k) for _ in range(passes)]
    return {
        "x": x, "w13": w13, "w2": w2, "routes": routes, "seed": seed,
        "draw_order": "x, outlier channels, w13, w2, routing per pass",
    }
