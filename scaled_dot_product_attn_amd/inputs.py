"""Seeded synthetic inputs for the attention forward pass.

This module draws random numbers and rounds them to fp16; it does none of the
attention arithmetic.  Both the HIP path's tests/bench and the float64 oracle
consume its arrays, and it imports neither of them.

Recipe (the workloads are the four SDPA cases of "An Optimal Mapper Meets a
Real GPU", section "Experiment one", case table, plus a head-dim-512 case from
the STAGE_D.md notes):

* generator: SplitMix64 (Steele, Lea and Flood, "Fast splittable pseudorandom
  number generators", OOPSLA 2014), used counter-style: the n-th 64-bit output
  of stream ``seed`` is ``mix(seed + (n + 1) * 0x9E3779B97F4A7C15)``;
* uniforms: the top 53 bits of each output, mapped to (0, 1] as
  ``((z >> 11) + 1) * 2**-53`` so that a logarithm never sees 0;
* normals: the Box-Muller transform in float64, pair k of uniforms (u1, u2)
  giving elements 2k and 2k + 1 as ``r cos(t)`` and ``r sin(t)`` with
  ``r = sqrt(-2 ln u1)``, ``t = 2 pi u2``;
* value: ``sigma * normal`` rounded once to fp16, round-to-nearest-even.

The generator is written out here rather than taken from numpy or torch so that
the bytes do not change with library versions.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass

import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, n: int, start: int = 0) -> np.ndarray:
    """Outputs ``start .. start + n - 1`` of the SplitMix64 stream ``seed``."""
    with np.errstate(over="ignore"):
        ctr = np.arange(start + 1, start + n + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + ctr * _GOLDEN
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        return z ^ (z >> np.uint64(31))


def uniform01(seed: int, n: int) -> np.ndarray:
    """n float64 uniforms in (0, 1], 53 random bits each."""
    z = splitmix64(seed, n)
    return ((z >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def normal_f64(seed: int, n: int) -> np.ndarray:
    """n standard normals from Box-Muller over the seed's uniform stream."""
    pairs = (n + 1) // 2
    u = uniform01(seed, 2 * pairs)
    u1, u2 = u[0::2], u[1::2]
    r = np.sqrt(-2.0 * np.log(u1))
    t = (2.0 * np.pi) * u2
    out = np.empty(2 * pairs, dtype=np.float64)
    out[0::2] = r * np.cos(t)
    out[1::2] = r * np.sin(t)
    return out[:n]


def normal_f16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """sigma * N(0, 1), rounded once to fp16 (numpy's float64 -> float16 cast
    rounds to nearest, ties to even)."""
    n = int(np.prod(shape))
    x = normal_f64(seed, n) * float(sigma)
    return x.astype(np.float16).reshape(shape)


def sha256(a: np.ndarray) -> str:
    return hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()


@dataclass(frozen=True)
class Workload:
    """One SDPA forward problem: contiguous [B, H, S, D] fp16 tensors."""

    name: str
    B: int
    H: int
    S: int
    D: int
    causal: bool
    sigma: float
    seed_base: int

    @property
    def scale(self) -> float:
        """1/sqrt(D) as the float32 value handed to the kernel."""
        return float(np.float32(1.0 / np.sqrt(self.D)))

    @property
    def shape(self):
        return (self.B, self.H, self.S, self.D)

    def flops(self) -> float:
        """Effective FLOPs: 4 B H S^2 D, halved when causal."""
        f = 4.0 * self.B * self.H * self.S * self.S * self.D
        return f / 2 if self.causal else f

    def alg_bytes(self) -> int:
        """Bytes the method must move: read Q, K, V once, write O (fp16) and
        the fp32 log-sum-exp."""
        n = self.B * self.H * self.S
        return 8 * n * self.D + 4 * n

    def qkv(self):
        """(q, k, v) as fp16 numpy arrays; seeds seed_base + 0, 1, 2."""
        return tuple(normal_f16(self.seed_base + t, self.shape, self.sigma)
                     for t in range(3))


# The five workloads.  Cases 1-4 are the case table's A-D (FP16 in, FP32
# accumulate, query length = key length); case 5 is the head-dim-512 problem of
# the sub-tiled kernel notes.  Seeds are 1000*c + {0, 1, 2}.
WORKLOADS = {
    1: Workload("B1_H8_S128_D64_noncausal", 1, 8, 128, 64, False, 1.0, 1000),
    2: Workload("B1_H16_S512_D64_causal", 1, 16, 512, 64, True, 1.0, 2000),
    3: Workload("B1_H32_S1024_D128_causal", 1, 32, 1024, 128, True, 1.0, 3000),
    4: Workload("B8_H32_S512_D128_causal", 8, 32, 512, 128, True, 1.0, 4000),
    5: Workload("B1_H8_S1024_D512_causal", 1, 8, 1024, 512, True, 0.5, 5000),
}


@dataclass(frozen=True)
class DecodeWorkload:
    """Sq query rows against Sk keys: q [B, H, Sq, D], k and v [B, H, Sk, D]."""

    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    causal: bool
    seed_base: int

    @property
    def scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.D)))

    def visible_pairs(self) -> int:
        """(query, key) pairs inside the mask (bottom-right when causal)."""
        if not self.causal:
            return self.Sq * self.Sk
        off = self.Sk - self.Sq
        return sum(min(self.Sk, i + off + 1) for i in range(self.Sq))

    def flops(self) -> float:
        """Effective FLOPs: 4 B H D per visible (query, key) pair."""
        return 4.0 * self.B * self.H * self.D * self.visible_pairs()

    def alg_bytes(self) -> int:
        """Read Q, K, V once, write O (fp16) and the fp32 log-sum-exp."""
        bh = self.B * self.H
        return 2 * bh * self.D * (2 * self.Sq + 2 * self.Sk) + 4 * bh * self.Sq

    def qkv(self):
        """(q, k, v) as fp16 numpy arrays; seeds seed_base + 0, 1, 2."""
        return (normal_f16(self.seed_base, (self.B, self.H, self.Sq, self.D)),
                normal_f16(self.seed_base + 1, (self.B, self.H, self.Sk, self.D)),
                normal_f16(self.seed_base + 2, (self.B, self.H, self.Sk, self.D)))


# Decode shapes (a single or a few new rows against a long key/value cache, the
# O(n) decode kernel whose cost "Validating Memory-Optimal Transformer Kernels
# on Real Hardware" measures against cache length in section 5).  The pages
# give no head or batch counts for it; these reuse the case table's
# H = 32, D = 128.  Seeds are 1000*(10+c) + {0, 1, 2}.
DECODE_WORKLOADS = {
    1: DecodeWorkload("decode_B1_H32_Sq1_Sk4096_D128", 1, 32, 1, 4096, 128, True, 11000),
    2: DecodeWorkload("decode_B1_H32_Sq1_Sk65536_D128", 1, 32, 1, 65536, 128, True, 12000),
    3: DecodeWorkload("decode_B8_H32_Sq4_Sk8192_D128", 8, 32, 4, 8192, 128, True, 13000),
}
