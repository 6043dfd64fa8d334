"""Seeded synthetic inputs for attention forward.

This module only produces data: the workload shapes and bf16 Q/K/V tensors
drawn from a seeded generator. It holds none of the attention arithmetic, so
both the HIP path (through its tests and the benchmark) and the CPU oracle can
consume the same inputs without sharing any of the method's code.

Recipe (the pages give shapes only as "bf16 ~ N(0,1) from seed"):
  * numpy ``default_rng(seed)`` (PCG64); Q, then K, then V are each drawn as
    float32 ``standard_normal((B, H, N, d))`` from that one generator;
  * each float32 is rounded to bf16 with round-to-nearest-even on its bit
    pattern;
  * the "max-tracking stress" variant multiplies every key row whose index is
    a multiple of 7 by 8 after rounding (exact in bf16: an exponent shift);
  * the scale handed to the kernel is the float32 value of 1/sqrt(d).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class AttnConfig:
    """One attention-forward workload: shapes, mask and the input recipe."""

    name: str
    B: int
    H: int
    N: int
    d: int
    causal: bool
    seed: int
    key_stress: bool = False  # every 7th key row multiplied by 8

    @property
    def scale(self) -> np.float32:
        return default_scale(self.d)

    def visible_pairs_per_head(self) -> int:
        """Number of (query, key) pairs that take part in the softmax."""
        n = self.N
        return n * (n + 1) // 2 if self.causal else n * n

    def flops(self) -> int:
        """Algorithmic FLOPs: both contractions over the visible pairs only."""
        return 4 * self.B * self.H * self.d * self.visible_pairs_per_head()


# The five workloads, named by what they are.
SMALL = AttnConfig("b1_h2_n256_d64", 1, 2, 256, 64, False, seed=1)
CAUSAL_2K = AttnConfig("b4_h16_n2048_d128_causal", 4, 16, 2048, 128, True, seed=2)
LONG_16K = AttnConfig("b2_h16_n16384_d128", 2, 16, 16384, 128, False, seed=3)
CAUSAL_8K_STRESS = AttnConfig("b8_h32_n8192_d64_causal_keyx8", 8, 32, 8192, 64, True, seed=4,
                              key_stress=True)
CAUSAL_4K_D256 = AttnConfig("b2_h8_n4096_d256_causal", 2, 8, 4096, 256, True, seed=5)

CONFIGS = [SMALL, CAUSAL_2K, LONG_16K, CAUSAL_8K_STRESS, CAUSAL_4K_D256]
HEADLINE = LONG_16K


@dataclass(frozen=True)
class DecodeConfig:
    """One decoding workload: Nq new query rows per (batch, head) against a
    cache of Nkv keys, every query seeing every key (the split-KV decoding
    microbenchmark of the pages' LLAMA3 configurations, (BS, SEQ) = (1, 1) and
    (32, 1); the cache length, which the pages' table no longer shows, is taken
    as the 4096 of their prefill configuration)."""

    name: str
    B: int
    H: int
    Nq: int
    Nkv: int
    d: int
    seed: int
    Hkv: int = 0  # K/V heads, H / Hkv query heads per K/V head (0: one each)

    @property
    def scale(self) -> np.float32:
        return default_scale(self.d)

    @property
    def kv_heads(self) -> int:
        return self.Hkv or self.H

    def flops(self) -> int:
        """Algorithmic FLOPs: both contractions over all Nq x Nkv pairs."""
        return 4 * self.B * self.H * self.d * self.Nq * self.Nkv

    def kv_bytes(self) -> int:
        """Compulsory HBM bytes: bf16 q, k, v read once (each K/V head once,
        whatever the number of query heads sharing it); fp32 out and lse
        written."""
        return (2 * self.B * (self.H * self.Nq + 2 * self.kv_heads * self.Nkv) * self.d
                + 4 * self.B * self.H * self.Nq * (self.d + 1))


@dataclass(frozen=True)
class ChunkScanConfig:
    """One Mamba2 ChunkScan workload: B sequences of S steps, H heads of P
    channels, chunks of L steps (the pages' linear-attention microbenchmark
    derived from Mamba2-1.3B, measured at BS = 64, SEQ = 8k; 64 heads of 64
    channels and chunks of 256 are that model's published shape)."""

    name: str
    B: int
    S: int
    H: int
    P: int
    L: int
    seed: int

    @property
    def nchunks(self) -> int:
        return (self.S + self.L - 1) // self.L

    def pairs(self) -> int:
        """(step, earlier-or-same step) pairs inside each chunk, per (b, h)."""
        full, tail = divmod(self.S, self.L)
        return full * self.L * (self.L + 1) // 2 + tail * (tail + 1) // 2

    def flops(self) -> int:
        """Algorithmic FLOPs of the contraction over the causal pairs."""
        return 2 * self.B * self.H * self.P * self.pairs()

    def hbm_bytes(self) -> int:
        """Compulsory bytes: bf16 x and cb, fp32 dt and dA_cumsum read once,
        fp32 out written once."""
        return (2 * self.B * self.S * self.H * self.P + 2 * self.B * self.nchunks * self.L * self.L
                + 2 * 4 * self.B * self.H * self.nchunks * self.L + 4 * self.B * self.S * self.H * self.P)


def gen_chunk_scan(B: int, S: int, H: int, P: int, L: int, seed: int):
    """Return (x, cb, dt, dA_cumsum) for ChunkScan, from ``default_rng(seed)``:

      x  [B][S][H][P]          bf16 bits, N(0, 1)
      cb [B][nc][L][L]         bf16 bits, N(0, 1) (one group: shared by all heads)
      dt [B][H][nc][L]         fp32, uniform(0.001, 0.1) (the softplus range of
                               Mamba2's step sizes)
      dA_cumsum [B][H][nc][L]  fp32, the running sum within each chunk of
                               A_h * dt with A_h = -uniform(1, 16) per head
                               (Mamba2's A initialisation), summed in float64
    Steps past S in the last chunk hold dt = 0 and the last running sum.
    """
    rng = np.random.default_rng(seed)
    nc = (S + L - 1) // L
    x = f32_to_bf16_bits(rng.standard_normal((B, S, H, P), dtype=np.float32))
    cb = f32_to_bf16_bits(rng.standard_normal((B, nc, L, L), dtype=np.float32))
    dt = rng.uniform(0.001, 0.1, size=(B, H, nc, L)).astype(np.float32)
    valid = (np.arange(nc * L) < S).reshape(nc, L)
    dt = np.where(valid[None, None], dt, np.float32(0.0)).astype(np.float32)
    a = -rng.uniform(1.0, 16.0, size=(H,))
    dacs = np.cumsum(a[None, :, None, None] * dt.astype(np.float64), axis=3).astype(np.float32)
    return x, cb, dt, dacs


def gen_chunk_scan_config(cfg: ChunkScanConfig):
    return gen_chunk_scan(cfg.B, cfg.S, cfg.H, cfg.P, cfg.L, cfg.seed)


CHUNKSCAN_SMALL = ChunkScanConfig("chunkscan_b1_s1000_h8_p64_l256", 1, 1000, 8, 64, 256, seed=21)
CHUNKSCAN_B64 = ChunkScanConfig("chunkscan_b64_s8192_h64_p64_l256", 64, 8192, 64, 64, 256, seed=22)
CHUNKSCAN_CONFIGS = [CHUNKSCAN_SMALL, CHUNKSCAN_B64]


@dataclass(frozen=True)
class MlaConfig:
    """One MLA decoding workload: per sequence, H query heads of Dk = 576
    (512 latent + 64 rotary) values attend to one shared cache of N latent
    rows whose first Dv = 512 values are the value (the absorbed form of
    DeepSeek-V2/V3 attention: 128 heads, latent 512, rotary 64), decoded at
    the pages' decode batch sizes 1 and 32 against a 4096-row cache."""

    name: str
    B: int
    H: int
    N: int
    seed: int
    Dk: int = 576
    Dv: int = 512

    @property
    def scale(self) -> np.float32:
        # DeepSeek's softmax scale: 1/sqrt(128 + 64) for 128 no-rope and 64 rope channels per head
        return np.float32(1.0 / np.sqrt(192.0))

    def flops(self) -> int:
        return 2 * self.B * self.H * self.N * (self.Dk + self.Dv)

    def hbm_bytes(self) -> int:
        """Compulsory: bf16 q and cache read once, fp32 out and lse written once."""
        return 2 * self.B * (self.H + self.N) * self.Dk + 4 * self.B * self.H * (self.Dv + 1)


def gen_mla(B: int, H: int, N: int, Dk: int, seed: int):
    """(q [B, H, Dk], kv [B, N, Dk]) as bf16 bits, N(0, 1), q then kv from
    ``default_rng(seed)``."""
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, H, Dk), dtype=np.float32))
    kv = f32_to_bf16_bits(rng.standard_normal((B, N, Dk), dtype=np.float32))
    return q, kv


MLA_B1 = MlaConfig("mla_b1_h128_n4096_dk576_dv512", 1, 128, 4096, seed=31)
MLA_B32 = MlaConfig("mla_b32_h128_n4096_dk576_dv512", 32, 128, 4096, seed=32)
MLA_CONFIGS = [MLA_B1, MLA_B32]


DECODE_B1 = DecodeConfig("decode_b1_h32_nq1_nkv4096_d128", 1, 32, 1, 4096, 128, seed=11)
DECODE_B32 = DecodeConfig("decode_b32_h32_nq1_nkv4096_d128", 32, 32, 1, 4096, 128, seed=12)
# LLAMA3-8B's grouping: 32 query heads over 8 K/V heads
DECODE_GQA_B1 = DecodeConfig("decode_b1_h32_kv8_nq1_nkv4096_d128", 1, 32, 1, 4096, 128, seed=13, Hkv=8)
DECODE_GQA_B32 = DecodeConfig("decode_b32_h32_kv8_nq1_nkv4096_d128", 32, 32, 1, 4096, 128, seed=14, Hkv=8)
DECODE_CONFIGS = [DECODE_B1, DECODE_B32, DECODE_GQA_B1, DECODE_GQA_B32]


def default_scale(d: int) -> np.float32:
    """The float32 softmax scale 1/sqrt(d) passed to both sides."""
    return np.float32(1.0 / np.sqrt(d))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even); return uint16 bits.

    Inputs here are finite; NaN handling is not needed for the generator.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to float32 (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def gen_qkv(B: int, H: int, N: int, d: int, seed: int, key_stress: bool = False):
    """Return (q, k, v) as contiguous uint16 bf16 bit arrays of shape [B, H, N, d]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    q = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal(shape, dtype=np.float32))
    if key_stress:
        kf = bf16_bits_to_f32(k)
        kf[:, :, ::7, :] *= np.float32(8.0)
        k = f32_to_bf16_bits(kf)
    return q, k, v


def gen_config(cfg: AttnConfig):
    """Inputs of a named workload."""
    return gen_qkv(cfg.B, cfg.H, cfg.N, cfg.d, cfg.seed, cfg.key_stress)


def gen_decode(B: int, H: int, Nq: int, Nkv: int, d: int, seed: int, Hkv: int = 0):
    """Return (q [B, H, Nq, d], k [B, Hkv, Nkv, d], v [B, Hkv, Nkv, d]) as
    uint16 bf16 bits: Q, then K, then V drawn from one ``default_rng(seed)``
    (Hkv = 0: one K/V head per query head)."""
    hkv = Hkv or H
    rng = np.random.default_rng(seed)
    q = f32_to_bf16_bits(rng.standard_normal((B, H, Nq, d), dtype=np.float32))
    k = f32_to_bf16_bits(rng.standard_normal((B, hkv, Nkv, d), dtype=np.float32))
    v = f32_to_bf16_bits(rng.standard_normal((B, hkv, Nkv, d), dtype=np.float32))
    return q, k, v


def gen_dout(B: int, H: int, N: int, d: int, seed: int):
    """Upstream gradient dO for the backward: bf16 N(0, 1) bits [B, H, N, d],
    drawn from its own stream (entropy (seed, 0xD0)), so that Q, K, V of the
    same seed are exactly the forward workload's."""
    rng = np.random.default_rng((seed, 0xD0))
    return f32_to_bf16_bits(rng.standard_normal((B, H, N, d), dtype=np.float32))


def bwd_flops(cfg: AttnConfig) -> int:
    """Algorithmic FLOPs of the backward: five contractions over the visible
    pairs (S = QK^T recomputed, dP = dO V^T, dV = P^T dO, dQ = dS K,
    dK = dS^T Q), 2.5 times the forward's two."""
    return 10 * cfg.B * cfg.H * cfg.d * cfg.visible_pairs_per_head()


def gen_decode_config(cfg: DecodeConfig):
    return gen_decode(cfg.B, cfg.H, cfg.Nq, cfg.Nkv, cfg.d, cfg.seed, cfg.Hkv)


def sample_rows(B: int, H: int, N: int, per_head: int, seed: int, tile: int = 64) -> np.ndarray:
    """Deterministic stratified sample of flat row ids in [0, B*H*N).

    Every (b, h) gets rows 0 and N-1, rows on both sides of several tile
    boundaries, and random rows; used where the oracle cannot run every row.
    """
    rng = np.random.default_rng(seed + 1000)
    rows = []
    for bh in range(B * H):
        cand = {0, N - 1}
        nt = (N + tile - 1) // tile
        for t in rng.choice(nt, size=min(nt, 3), replace=False):
            for off in (t * tile - 1, t * tile, t * tile + tile - 1):
                if 0 <= off < N:
                    cand.add(int(off))
        rest = np.setdiff1d(np.arange(N), np.fromiter(cand, dtype=np.int64))
        extra = min(rest.size, max(0, per_head - len(cand)))
        cand.update(int(x) for x in rng.choice(rest, size=extra, replace=False))
        rows.extend(bh * N + i for i in sorted(cand))
    return np.asarray(sorted(set(rows)), dtype=np.int64)
