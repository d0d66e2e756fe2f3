"""Seeded synthetic inputs for the GEMM workloads.

This module holds no GEMM arithmetic.  It only draws numbers, rounds them to
the input element type and lays them out in memory; the HIP path and the
oracle both consume the bit patterns it produces, so they see identical inputs.

Random stream: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014): state advances by 0x9E3779B97F4A7C15 and each
output is the state passed through the 64-bit finaliser.  Draw i of seed s is
mix(s + (i + 1) * 0x9E3779B97F4A7C15).

Distributions:
  uniform : u = (x >> 40) * 2^-24 in [0, 1), value 2u - 1 in [-1, 1)
  normal  : Box-Muller on two consecutive draws, u1 = ((x1 >> 11) + 1) * 2^-53
            in (0, 1], u2 = (x2 >> 11) * 2^-53, value sqrt(-2 ln u1) cos(2 pi u2)
  int     : ((x >> 32) mod 5) - 2, entries in {-2, ..., 2}
Values are rounded to fp32, then to bf16/fp16/fp8 E4M3 (OCP, the encoding
without infinities) with round-to-nearest-even by torch/numpy's own
conversions.  bf16 and fp16 elements are stored as uint16 bit patterns, e4m3
elements as uint8.

The logical matrices are A[m][k] (M x K) and B[k][n] (K x N), drawn in
row-major order, then stored in the requested contiguity:
  A K-contiguous : A[m*lda + k]     A MN-contiguous : A[k*lda + m]
  B MN-contiguous: B[k*ldb + n]     B K-contiguous  : B[n*ldb + k]
Elements between the contiguous extent and the leading dimension are filled
with a NaN pattern, so a kernel that reads padding poisons its result.
"""
from dataclasses import dataclass, field

import numpy as np

GOLDEN = np.uint64(0x9E3779B97F4A7C15)
BF16, F16, E4M3 = "bf16", "f16", "e4m3"
K_CONTIG, MN_CONTIG = "K", "MN"
NAN_BITS = {BF16: 0x7FC0, F16: 0x7E00, E4M3: 0x7F}
STORAGE = {BF16: np.uint16, F16: np.uint16, E4M3: np.uint8}


def splitmix64(seed: int, n: int) -> np.ndarray:
    """n consecutive SplitMix64 outputs for `seed` (uint64 array)."""
    with np.errstate(over="ignore"):
        idx = np.arange(1, n + 1, dtype=np.uint64)
        z = np.uint64(seed) + idx * GOLDEN
        z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
        z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
        z = z ^ (z >> np.uint64(31))
    return z


def draw(seed: int, n: int, dist: str, scale: float = 1.0) -> np.ndarray:
    """n values (float64) of distribution `dist`, times `scale`."""
    if dist == "uniform":
        x = splitmix64(seed, n)
        v = 2.0 * ((x >> np.uint64(40)).astype(np.float64) * 2.0 ** -24) - 1.0
    elif dist == "normal":
        x = splitmix64(seed, 2 * n)
        u1 = ((x[0::2] >> np.uint64(11)).astype(np.float64) + 1.0) * 2.0 ** -53
        u2 = (x[1::2] >> np.uint64(11)).astype(np.float64) * 2.0 ** -53
        v = np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)
    elif dist == "int":
        x = splitmix64(seed, n)
        v = ((x >> np.uint64(32)) % np.uint64(5)).astype(np.float64) - 2.0
    elif dist == "ones":
        v = np.ones(n, dtype=np.float64)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return v * scale


def quantize(values: np.ndarray, dtype: str) -> np.ndarray:
    """float64 -> fp32 -> bf16/fp16 bits (uint16) or e4m3 bits (uint8), round
    to nearest even."""
    f32 = np.ascontiguousarray(np.asarray(values, dtype=np.float32))
    if dtype == F16:
        return f32.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        import torch
        t = torch.from_numpy(f32).to(torch.bfloat16)
        return t.view(torch.int16).numpy().view(np.uint16)
    if dtype == E4M3:
        import torch
        if np.any(np.abs(f32) > 448.0):
            raise ValueError("value beyond the e4m3 range")
        t = torch.from_numpy(f32).to(torch.float8_e4m3fn)
        return t.view(torch.uint8).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def store(logical: np.ndarray, transpose: bool, ld: int, dtype: str) -> np.ndarray:
    """Lay out a logical (R x C) bit matrix row-major with leading dimension
    `ld`, transposed first if `transpose`.  Returns flat uint16 (uint8 for
    e4m3) storage holding rows*ld - (ld - extent) elements, padding filled with
    NaN bits."""
    mat = logical.T if transpose else logical
    rows, extent = mat.shape
    if ld < extent:
        raise ValueError("leading dimension below the contiguous extent")
    if rows == 0:
        return np.zeros(0, dtype=STORAGE[dtype])
    buf = np.full((rows, ld), NAN_BITS[dtype], dtype=STORAGE[dtype])
    buf[:, :extent] = mat
    flat = buf.reshape(-1)
    return np.ascontiguousarray(flat[: (rows - 1) * ld + extent])


@dataclass
class Problem:
    """One GEMM instance: flat operand storage plus its shape and layouts."""
    M: int
    N: int
    K: int
    dtype: str             # input element type
    layoutA: str           # "K" or "MN"
    layoutB: str
    lda: int
    ldb: int
    A: np.ndarray = field(repr=False)   # flat uint16 (uint8 for e4m3) storage
    B: np.ndarray = field(repr=False)
    A_logical: np.ndarray = field(repr=False, default=None)   # M x K bits
    B_logical: np.ndarray = field(repr=False, default=None)   # K x N bits


def make_logical(M, N, K, dtype, dist, seed_a, seed_b, scale=1.0):
    a = quantize(draw(seed_a, M * K, dist, scale), dtype).reshape(M, K)
    b = quantize(draw(seed_b, K * N, dist, scale), dtype).reshape(K, N)
    return a, b


def layout_problem(a, b, dtype, layoutA, layoutB, pad_a=0, pad_b=0):
    """Store logical bit matrices a (M x K) and b (K x N) in the given layouts;
    pad_a / pad_b add that many elements to the minimal leading dimension."""
    M, K = a.shape
    N = b.shape[1]
    if layoutA == K_CONTIG:
        lda = max(K, 1) + pad_a
        A = store(a, False, lda, dtype)
    else:
        lda = max(M, 1) + pad_a
        A = store(a, True, lda, dtype)
    if layoutB == MN_CONTIG:
        ldb = max(N, 1) + pad_b
        B = store(b, False, ldb, dtype)
    else:
        ldb = max(K, 1) + pad_b
        B = store(b, True, ldb, dtype)
    return Problem(M, N, K, dtype, layoutA, layoutB, lda, ldb, A, B, a, b)


def make_problem(M, N, K, dtype, layoutA, layoutB, dist, seed_a, seed_b, scale=1.0,
                 pad_a=0, pad_b=0):
    a, b = make_logical(M, N, K, dtype, dist, seed_a, seed_b, scale)
    return layout_problem(a, b, dtype, layoutA, layoutB, pad_a, pad_b)


# The five workloads: shapes, element types, layouts, distributions and seeds
# (seeds 1000*i + 1 for A and 1000*i + 2 for B).
WORKLOADS = {
    "bf16_256_nn_f32": dict(M=256, N=256, K=256, dtype=BF16, out="f32", layouts=[("K", "MN")],
                            dist="uniform", scale=1.0, seeds=(1001, 1002)),
    "f16_1500x1152x896_nn_f16": dict(M=1500, N=1152, K=896, dtype=F16, out="f16",
                                     layouts=[("K", "MN")], dist="normal", scale=0.1,
                                     seeds=(2001, 2002)),
    "bf16_4096_all_bf16": dict(M=4096, N=4096, K=4096, dtype=BF16, out="bf16",
                               layouts=[("K", "MN"), ("K", "K"), ("MN", "MN"), ("MN", "K")],
                               dist="uniform", scale=1.0, seeds=(3001, 3002)),
    "bf16_8192_nn_f32": dict(M=8192, N=8192, K=8192, dtype=BF16, out="f32", layouts=[("K", "MN")],
                             dist="normal", scale=1.0, seeds=(4001, 4002)),
    "bf16_skinny_32x16384x8192_nn_bf16": dict(M=32, N=16384, K=8192, dtype=BF16, out="bf16",
                                              layouts=[("K", "MN")], dist="uniform", scale=1.0,
                                              seeds=(5001, 5002)),
    # The fp8 variant (the same LDS machinery with 1-byte elements): the
    # headline shape and layout with OCP E4M3 inputs.
    "e4m3_8192_nn_f32": dict(M=8192, N=8192, K=8192, dtype=E4M3, out="f32", layouts=[("K", "MN")],
                             dist="normal", scale=1.0, seeds=(6001, 6002)),
}
