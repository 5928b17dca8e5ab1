"""Seeded synthetic inputs for the W4A16 GEMM/GEMV workloads.

This module only draws random numbers and names shapes. It holds none of the method's
arithmetic (no quantisation, packing or products), so both the oracle side and the
HIP side can take their inputs from it without sharing code.

Value distributions: weights W ~ N(0, 0.02) in fp32, laid out [K, N]; activations
x ~ N(0, 1) drawn in fp32 and rounded to fp16. The pages measure on trained models
(decode of current-generation LLMs on an A100, Qwen2.5-1.5B on an RTX 3060); these
seeded draws stand in for those weights with the same projection shapes.
"""
import numpy as np

# Workload ids enter the seeds so that every named workload draws its own numbers.
WORKLOADS = {
    # One decode GEMV: M=1, K=N=4096, group 128.
    "gemv_4096": dict(wid=0, shapes=[(1, 4096, 4096)]),
    # Decode batch sweep on dense-FFN/attention projections.
    "decode_sweep": dict(wid=1, shapes=[(m, k, n) for (k, n) in
                                        [(4096, 14336), (14336, 4096), (4096, 4096)]
                                        for m in (1, 2, 4, 8, 16)]),
    # MoE-expert sized skinny GEMMs.
    "moe_expert": dict(wid=2, shapes=[(m, k, n) for (k, n) in
                                      [(2048, 1408), (1408, 2048), (2048, 768), (768, 2048)]
                                      for m in (1, 4, 16)]),
    # Batch-1 decode of a 32-layer 7B-shaped dense transformer plus its lm_head.
    "decode_chain_7b": dict(wid=3, shapes=None),
    # Prefill-sized GEMMs.
    "prefill": dict(wid=4, shapes=[(m, k, n) for (k, n) in
                                   [(8192, 8192), (8192, 28672), (28672, 8192)]
                                   for m in (32, 128, 512, 2048)]),
}

# Per-layer projections of the 7B-shaped model, as (name, K, N); one token is
# 32 layers of these seven GEMVs followed by lm_head (225 GEMVs).
CHAIN_7B_LAYER = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096),
                  ("o", 4096, 4096), ("gate", 4096, 14336), ("up", 4096, 14336),
                  ("down", 14336, 4096)]
CHAIN_7B_LAYERS = 32
CHAIN_7B_LM_HEAD = ("lm_head", 4096, 128256)

W_STD = np.float32(0.02)


def weight(K, N, wid=0, layer=0):
    """W fp32 [K, N] ~ N(0, 0.02), seeded by (1, wid, K, N, layer)."""
    rng = np.random.default_rng((1, wid, K, N, layer))
    W = rng.standard_normal((K, N), dtype=np.float32)
    W *= W_STD
    return W


def activations(M, K, wid=0):
    """x fp16 [M, K]: N(0, 1) drawn in fp32, rounded to fp16; seeded by (2, wid, M, K)."""
    rng = np.random.default_rng((2, wid, M, K))
    return rng.standard_normal((M, K), dtype=np.float32).astype(np.float16)


def uniform_codes(K, N, seed=0):
    """Random 4-bit codes [K, N] (uint8 0..15) for pack/unpack round trips."""
    rng = np.random.default_rng((3, K, N, seed))
    return rng.integers(0, 16, size=(K, N), dtype=np.uint8)


def weight_custom(K, N, seed, std=0.02, mean=0.0):
    """W fp32 [K, N] ~ N(mean, std) for edge-case tests (one-signed groups, other spreads)."""
    rng = np.random.default_rng((4, K, N, seed))
    W = rng.standard_normal((K, N), dtype=np.float32) * np.float32(std)
    W += np.float32(mean)
    return W


def scales_zeros_custom(G, N, seed, log2_lo=-12.0, log2_hi=-9.0, zero_limit=1024):
    """Hand-built per-(group, column) parameters for packed weights that no quantiser run
    would produce: fp16 scales log-uniform in [2**log2_lo, 2**log2_hi] and integer zero
    points uniform in [-zero_limit, zero_limit], with the first columns of group 0 set to
    the values at and next to the ends of that range (-1024, 1024, -1, 0, 15, 16)."""
    rng = np.random.default_rng((6, G, N, seed))
    s = np.exp2(rng.uniform(log2_lo, log2_hi, size=(G, N))).astype(np.float16)
    z = rng.integers(-zero_limit, zero_limit + 1, size=(G, N)).astype(np.float16)
    edges = np.array([-zero_limit, zero_limit, -1, 0, 15, 16], dtype=np.float16)
    z[0, :min(N, len(edges))] = edges[:min(N, len(edges))]
    return s, z
