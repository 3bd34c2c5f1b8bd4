"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds no attention arithmetic. It only draws random numbers,
rounds them to the storage format the kernels consume (fp16 / bf16 bit
patterns) and decodes those bit patterns back to float64 for the oracle.

Recipe (workloads of the attention-forward configurations):
  * Q, K, V: numpy ``Generator(PCG64(seed))`` float32 ``standard_normal``,
    drawn in the order Q, K, V, each in C order of its layout
    ((B,S,H,D) padded, (T,H,D) packed), optionally multiplied by a float32
    factor, then rounded to nearest-even to fp16 or bf16.
  * Packed lengths: ``PCG64(seed + 1)`` ``integers(lo, hi, endpoint=True)``
    until the total is reached; the last length is truncated to fit.
  * Sampled query rows: ``PCG64(seed + 2)``, distinct uniform picks plus a
    fixed set of boundary rows.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20261202

DTYPES = ("fp16", "bf16")


def config_seed(k: int) -> int:
    """Seed of configuration ``k`` (1-based)."""
    return SEED_BASE + 10 * k


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def f32_to_fp16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE half (nearest, ties to even); return uint16 bits."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return f32_to_fp16_bits(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def fp8_qkv(shape, seed: int, mult: float = 1.0):
    """Q, K, V as OCP E4M3 codes (uint8) of i.i.d. N(0,1)*mult values, rounded to
    nearest even by torch's float8_e4m3fn conversion."""
    import torch
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out.append(torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy())
    return tuple(out)


def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode fp16/bf16 bit patterns (uint16) exactly to float64."""
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "fp16":
        return bits.view(np.float16).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def sha256_of(*arrays: np.ndarray) -> str:
    h = hashlib.sha256()
    for a in arrays:
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()


def normal_qkv(shape, dtype: str, seed: int, mult: float = 1.0):
    """Q, K, V bit patterns (uint16) of the given shape, i.i.d. N(0,1)*mult."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(3):
        x = rng.standard_normal(size=tuple(shape), dtype=np.float32)
        if mult != 1.0:
            x *= np.float32(mult)
        out.append(to_bits(x, dtype))
        del x
    return tuple(out)


def varlen_lengths(total: int, lo: int, hi: int, seed: int) -> list[int]:
    """Segment lengths drawn uniformly in [lo, hi] until ``total`` is reached."""
    rng = np.random.Generator(np.random.PCG64(seed))
    lens: list[int] = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi, endpoint=True))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def cu_seqlens_of(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64)).astype(np.int32)
    return cu


def sampled_rows(S: int, n: int, seed: int, must=(0, 1, 63, 64, 127, 128)) -> np.ndarray:
    """``n`` distinct query rows in [0, S): the boundary rows plus uniform picks."""
    fixed = sorted({r for r in list(must) + [S - 1] if 0 <= r < S})
    rng = np.random.Generator(np.random.PCG64(seed))
    rest = n - len(fixed)
    chosen = set(fixed)
    picks = []
    while len(picks) < rest and len(chosen) < S:
        r = int(rng.integers(0, S))
        if r not in chosen:
            chosen.add(r)
            picks.append(r)
    return np.array(sorted(fixed + picks), dtype=np.int64)


@dataclass(frozen=True)
class Config:
    """One attention-forward workload."""
    index: int
    name: str
    B: int
    H: int
    S: int
    D: int
    dtype: str
    causal: bool
    mult: float = 1.0
    varlen: bool = False
    seg_lo: int = 0
    seg_hi: int = 0
    sample_rows: int = 0
    extra: dict = field(default_factory=dict)
    window: int = 0             # sliding-window width (0: none)
    n_global: int = 0           # leading query rows that see every key
    alibi: bool = False         # per-head linear distance bias (slopes from alibi_slopes)

    @property
    def seed(self) -> int:
        return config_seed(self.index)

    def describe(self) -> str:
        c = "causal" if self.causal else "non-causal"
        if self.varlen:
            return (f"varlen T={self.S} H={self.H} D={self.D} {self.dtype} {c} "
                    f"segments U[{self.seg_lo},{self.seg_hi}]")
        d = f"B={self.B} H={self.H} S={self.S} D={self.D} {self.dtype} {c}"
        if self.window:
            d += f" window={self.window}"
        if self.n_global:
            d += f" global={self.n_global}"
        if self.alibi:
            d += " alibi"
        return d


CONFIGS = {
    "tiny": Config(1, "tiny", 1, 2, 128, 64, "fp16", False),
    "mha": Config(2, "mha", 4, 12, 2048, 64, "fp16", False),
    "mha_causal": Config(2, "mha_causal", 4, 12, 2048, 64, "fp16", True),
    "llama": Config(3, "llama", 4, 32, 4096, 128, "bf16", True, mult=0.5),
    "long": Config(4, "long", 1, 32, 65536, 64, "fp16", True, sample_rows=256),
    "varlen": Config(5, "varlen", 1, 32, 65536, 128, "bf16", True, varlen=True,
                     seg_lo=128, seg_hi=8192),
    # mask/bias variants: a 128K-token context with a 4096-key causal window
    # and 64 global query rows; the LLaMA-shaped layer with ALiBi slopes
    "window128k": Config(6, "window128k", 1, 32, 131072, 128, "bf16", True, window=4096,
                         n_global=64),
    "llama_alibi": Config(3, "llama_alibi", 4, 32, 4096, 128, "bf16", True, mult=0.5,
                          alibi=True),
}


def alibi_slopes(H: int) -> np.ndarray:
    """Per-head ALiBi slopes, the geometric schedule 2^(-8(h+1)/H), as float32."""
    return np.array([2.0 ** (-8.0 * (h + 1) / H) for h in range(H)], dtype=np.float32)


@dataclass
class Inputs:
    """Bit patterns of one workload plus its packing metadata."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    layout: str                 # "bshd" or "thd"
    cu_seqlens: np.ndarray | None
    sha256: str

    def f64(self):
        return (bits_to_f64(self.q, self.dtype), bits_to_f64(self.k, self.dtype),
                bits_to_f64(self.v, self.dtype))


def make_inputs(cfg: Config, *, S: int | None = None, B: int | None = None,
                H: int | None = None) -> Inputs:
    """Inputs of ``cfg`` (optionally with a reduced B/H/S for fast tests)."""
    B = cfg.B if B is None else B
    H = cfg.H if H is None else H
    S = cfg.S if S is None else S
    if cfg.varlen:
        lens = varlen_lengths(S, cfg.seg_lo, cfg.seg_hi, cfg.seed + 1)
        cu = cu_seqlens_of(lens)
        q, k, v = normal_qkv((S, H, cfg.D), cfg.dtype, cfg.seed, cfg.mult)
        return Inputs(q, k, v, cfg.dtype, "thd", cu, sha256_of(q, k, v, cu))
    q, k, v = normal_qkv((B, S, H, cfg.D), cfg.dtype, cfg.seed, cfg.mult)
    return Inputs(q, k, v, cfg.dtype, "bshd", None, sha256_of(q, k, v))


# ---- KV-cache decode workloads ---------------------------------------------

@dataclass(frozen=True)
class DecodeConfig:
    """One decode step: Sq new rows per sequence against a (B, H, S_max, D) cache."""
    index: int
    name: str
    B: int
    H: int
    Sq: int
    S_max: int
    D: int
    dtype: str
    causal: bool
    len_lo: int = 0          # 0: every cache is full (S_max rows)
    len_hi: int = 0

    @property
    def seed(self) -> int:
        return config_seed(self.index)

    def describe(self) -> str:
        c = " causal" if self.causal else ""
        lens = (f" lengths U[{self.len_lo},{self.len_hi}]" if self.len_lo else " full caches")
        return (f"decode B={self.B} H={self.H} Sq={self.Sq} S_max={self.S_max} D={self.D} "
                f"{self.dtype}{c}{lens}")


DECODE_CONFIGS = {
    # one new token per sequence against a 64K-token cache (LLaMA-shaped heads)
    "decode64k": DecodeConfig(7, "decode64k", 4, 32, 1, 65536, 128, "bf16", False),
    # a serving batch: 32 sequences with cache lengths spread over [1, 8192]
    "decode_batch": DecodeConfig(8, "decode_batch", 32, 32, 1, 8192, 128, "bf16", False,
                                 len_lo=1, len_hi=8192),
}


@dataclass
class DecodeInputs:
    q: np.ndarray                 # (B, Sq, H, D) bits
    k: np.ndarray                 # (B, H, S_max, D) bits
    v: np.ndarray
    seqlens: np.ndarray | None    # int32 (B,) or None
    dtype: str
    sha256: str


def decode_lengths(B: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """Cache lengths drawn uniformly in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.integers(lo, hi, size=B, endpoint=True).astype(np.int32)


def decode_inputs(B: int, Sq: int, H: int, S_max: int, D: int, dtype: str, seed: int,
                  lens=None) -> DecodeInputs:
    """Q then K then V, i.i.d. N(0,1), rounded to the element type."""
    rng = np.random.Generator(np.random.PCG64(seed))
    q = to_bits(rng.standard_normal(size=(B, Sq, H, D), dtype=np.float32), dtype)
    k = to_bits(rng.standard_normal(size=(B, H, S_max, D), dtype=np.float32), dtype)
    v = to_bits(rng.standard_normal(size=(B, H, S_max, D), dtype=np.float32), dtype)
    sl = None if lens is None else np.asarray(lens, dtype=np.int32)
    extra = () if sl is None else (sl,)
    return DecodeInputs(q, k, v, sl, dtype, sha256_of(q, k, v, *extra))


def make_decode_inputs(cfg: DecodeConfig) -> DecodeInputs:
    lens = (decode_lengths(cfg.B, cfg.len_lo, cfg.len_hi, cfg.seed + 1) if cfg.len_lo else None)
    return decode_inputs(cfg.B, cfg.Sq, cfg.H, cfg.S_max, cfg.D, cfg.dtype, cfg.seed, lens)

