"""Seeded synthetic inputs shared by the oracle tests, the GPU tests and the
bench.  This module holds no quantisation or GEMM arithmetic: it draws
random numbers, rounds them to BF16 storage and builds routing/offset
arrays.

Recipe (per workload):
  rng = numpy.random.default_rng(seed); draws in the order routing, A, B,
  bias.  A real sample is float32 standard normal times sigma, rounded to
  BF16 (round-to-nearest-even, done by torch's CPU cast).  Large weight
  tensors are drawn per expert from SeedSequence(seed).spawn(E) child
  streams so that they can be drawn by several threads and still be
  reproducible.

Workloads (sizes from the pages' examples and qualification shapes):
  dense_mxfp8_256   A, B [256, 256] ~ N(0,1), seed 0
  batch_mxfp8       A, W [4, 256, 256] ~ N(0,1), bias [4, 256] ~ N(0, 0.1)
  dense_mxfp4_small A [32, 256], B [512, 256] ~ N(0,1)
  dense_fp4_large   A [M, K] ~ N(0,1), W [N, K] ~ N(0, 0.02),
                    (N, K) in {(17408, 5120), (5120, 17408), (12288, 5120)},
                    M in {1, 16, 512, 4096}
  moe_contiguous    E=32, 16384 tokens x top-4 = 65536 slots; per-expert
                    counts ~ Multinomial(65536, Dirichlet(1)); each group
                    padded to a multiple of 128; K=4096, N=2*1536
  moe_masked        E=64, slot 256 rows, counts ~ U{0..256}; K=7168, N=4096
  moe_dglu_backward the backward of the expert MLP's input at the MoE shape:
                    moe_contiguous's routing, A [R, 4096], B [32, 1536, 4096],
                    C [R, 3072], prob, per-expert alpha / beta
"""

from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch


def to_bf16_bits(x_f32):
    """float32 array -> BF16 bit patterns (uint16), nearest-even rounding."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16(rng, shape, sigma=1.0):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return to_bf16_bits(x)


def normal_bf16_per_expert(seed, E, shape, sigma=1.0, threads=8):
    """[E, *shape] BF16 bits; expert e drawn from child stream e of
    SeedSequence(seed)."""
    children = np.random.SeedSequence(seed).spawn(E)
    out = np.empty((E,) + tuple(shape), dtype=np.uint16)

    def work(e):
        r = np.random.default_rng(children[e])
        out[e] = normal_bf16(r, shape, sigma)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, range(E)))
    return out


# ---------------------------------------------------------------- routing
def moe_contiguous_counts(rng, E=32, slots=65536):
    p = rng.dirichlet(np.ones(E))
    return rng.multinomial(slots, p).astype(np.int64)


def padded_group_ends(counts, align=128):
    padded = ((np.asarray(counts, np.int64) + align - 1) // align) * align
    return np.cumsum(padded).astype(np.int32), padded


def moe_masked_counts(rng, E=64, max_m=256):
    return rng.integers(0, max_m + 1, size=E).astype(np.int32)


# ---------------------------------------------------------------- workloads
def dense_mxfp8_256(seed=0):
    rng = np.random.default_rng(seed)
    a = normal_bf16(rng, (256, 256))
    b = normal_bf16(rng, (256, 256))
    return {"a": a, "b": b}


def batch_mxfp8(seed=1, batch=4, m=256, n=256, k=256):
    rng = np.random.default_rng(seed)
    a = normal_bf16(rng, (batch, m, k))
    b = normal_bf16(rng, (batch, n, k))
    bias = normal_bf16(rng, (batch, n), 0.1)
    return {"a": a, "b": b, "bias": bias}


def dense_mxfp4_small(seed=1, m=32, n=512, k=256):
    rng = np.random.default_rng([seed, 1])
    a = normal_bf16(rng, (m, k))
    b = normal_bf16(rng, (n, k))
    return {"a": a, "b": b}


LARGE_NK = [(17408, 5120), (5120, 17408), (12288, 5120)]
LARGE_M = [1, 16, 512, 4096]


def dense_fp4_large_acts(n, k, m, seed=2):
    """Activations N(0,1) [m, k] from SeedSequence(seed, spawn_key=(n, k, m))."""
    return normal_bf16(np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(n, k, m))), (m, k))


def dense_fp4_large_weights(n, k, seed=2):
    """Weights N(0, 0.02) [n, k] from SeedSequence(seed, spawn_key=(n, k)):
    every M of one (N, K) shares them."""
    return normal_bf16(np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(n, k))), (n, k), 0.02)


def dense_fp4_large(n, k, m, seed=2):
    """Activations [m, k] and weights [n, k] of one qualification shape."""
    return {"a": dense_fp4_large_acts(n, k, m, seed), "b": dense_fp4_large_weights(n, k, seed)}


def moe_contiguous(seed=3, E=32, tokens=16384, topk=4, K=4096, H=1536, align=128,
                   with_weights=True, threads=8):
    rng = np.random.default_rng(seed)
    counts = moe_contiguous_counts(rng, E, tokens * topk)
    ends, padded = padded_group_ends(counts, align)
    R = int(ends[-1])
    a = np.zeros((R, K), np.uint16)
    starts = np.concatenate([[0], ends[:-1]]).astype(np.int64)
    for g in range(E):
        c = int(counts[g])
        if c:
            a[starts[g]:starts[g] + c] = normal_bf16(rng, (c, K))
    out = {"counts": counts, "group_end": ends, "starts": starts, "a": a, "K": K, "N": 2 * H, "H": H}
    if with_weights:
        out["b"] = normal_bf16_per_expert(seed * 1000 + 7, E, (2 * H, K), 0.02, threads)
    return out


def moe_dglu_backward(seed=3, E=32, tokens=16384, topk=4, K=4096, N=1536, align=128, threads=8):
    """Inputs of the backward grouped GEMM with the dSwiGLU epilogue at the
    MoE shape (cuDNN FE "Grouped GEMM + dGLU (SM100)" tensors): the routing
    of moe_contiguous (same seed: same counts and padded ends); A [R, K] the
    upstream gradient N(0, 1) on valid rows, zero on padding rows; B
    [E, N, K] expert weights N(0, 0.02); C [R, 2N] forward activations
    N(0, 1); prob [R] float32 U(0, 1); alpha, beta [E] float32 U(0.5, 2) and
    U(0.5, 1.5)."""
    rng = np.random.default_rng(seed)
    counts = moe_contiguous_counts(rng, E, tokens * topk)
    ends, _ = padded_group_ends(counts, align)
    R = int(ends[-1])
    starts = np.concatenate([[0], ends[:-1]]).astype(np.int64)
    r2 = np.random.default_rng([seed, 21])
    a = np.zeros((R, K), np.uint16)
    for g in range(E):
        c = int(counts[g])
        if c:
            a[starts[g]:starts[g] + c] = normal_bf16(r2, (c, K))
    b = normal_bf16_per_expert(seed * 1000 + 21, E, (N, K), 0.02, threads)
    cact = normal_bf16(r2, (R, 2 * N))
    prob = r2.random(R, dtype=np.float32)
    alpha = r2.uniform(0.5, 2.0, E).astype(np.float32)
    beta = r2.uniform(0.5, 1.5, E).astype(np.float32)
    return {"counts": counts, "group_end": ends, "starts": starts, "a": a, "b": b, "c": cact, "prob": prob,
            "alpha": alpha, "beta": beta, "K": K, "N": N}


def moe_down_weights(E=32, hidden=4096, H=1536, seed=3, threads=8):
    """Down-projection weights of the MoE MLP chain [E, hidden, H] N(0, 0.02)
    (the expert GEMM after the SwiGLU, K = H)."""
    return normal_bf16_per_expert(seed * 1000 + 8, E, (hidden, H), 0.02, threads)


def moe_masked(seed=4, E=64, max_m=256, K=7168, N=4096, with_weights=True, threads=8):
    rng = np.random.default_rng(seed)
    counts = moe_masked_counts(rng, E, max_m)
    a = normal_bf16(rng, (E * max_m, K))
    out = {"counts": counts, "a": a, "max_m": max_m, "K": K, "N": N, "garbage_seed": seed * 1000 + 11}
    if with_weights:
        out["b"] = normal_bf16_per_expert(seed * 1000 + 9, E, (N, K), 0.02, threads)
    return out


def permute_inputs(T, H, topk, E, seed=5):
    """Token-permute inputs shaped like the HALOps "GEMM" page's
    prefill_permute_to_masked_gemm example: BF16 rows N(0,1) [T, H], random
    int32 broadcast scale words [T, H/512] (bytes of UE8M0 values 120..134),
    top-k expert ids uniform in [0, E) [T, topk] int64."""
    rng = np.random.default_rng([seed, T, H, topk, E])
    x = normal_bf16(rng, (T, H))
    sb = rng.integers(120, 135, size=(T, H // 128), dtype=np.uint8)
    scale = np.ascontiguousarray(sb).view(np.int32).reshape(T, H // 512)
    ids = rng.integers(0, E, size=(T, topk)).astype(np.int64)
    return {"x": x, "scale": scale, "topk_ids": ids}


def garbage_bytes(seed, shape):
    """Uniform random bytes (used for padded rows that must be ignored)."""
    return np.random.default_rng(seed).integers(0, 256, size=shape, dtype=np.uint8)
