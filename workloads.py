"""Seeded synthetic inputs shaped like the Qwen3-8B linear layers the BATQuant pages study.

This module draws inputs and nothing else: bf16 activations with outlier channels, the GPK
factors A (8x8) and B_i (4x4), the clipping logits and fp32 weights.  It holds none of the
method's arithmetic (no transform, clip, scale, encode, sigmoid or inverse), so the oracle
side and the GPU side can both take their inputs from it without sharing any of the
computation under test.

Workloads (the pages evaluate Qwen3-8B / Qwen3-VL-8B and show q_proj and down_proj
activation blocks: thelatestinai listing, Figures 2 and 5; real activations and weights are
not available, so these seeded stand-ins of the same shapes and outlier structure are used):

  tiny        S=16,    N=256,   out=256    N(0,1), 2 outlier channels x50
  q_proj      S=2048,  N=4096,  out=4096   N(0,1), 8 outlier channels x U(20,100)
  gate_up     S=2048,  N=4096,  out=24576  N(0,1), 8 outlier channels x50
  down_proj   S=2048,  N=12288, out=4096   Student-t(3), 4 blocks with one channel x500
  sweep_*     S in {1, 8, 64, 16384} x (N=12288 -> 4096, N=4096 -> 4096), N(0,1) + 8 ch x50

All layers: A = I8 + 0.1 N(0,1), B_i = I4 + 0.1 N(0,1) (fp32), clip logits alpha_min and
alpha_max ~ N(2, 0.5), weights W ~ N(0, 0.02) fp32 [out, N].  Random streams: PCG64 with
one child stream per tensor, SeedSequence(seed).spawn(6) in the order
[X, outliers, A, B, alpha, W].  X is drawn in fp32 and rounded to nearest-even bf16.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np


@dataclass(frozen=True)
class LayerConfig:
    name: str
    S: int
    N: int
    out: int
    seed: tuple
    act: str = "normal"                # "normal" | "student_t3"
    outliers: tuple = ("channels", 8, 50.0)

    @property
    def k(self) -> int:
        return self.N // 32


def _sweep():
    cfgs = {}
    shapes = [(S, N, 4096) for N in (12288, 4096) for S in (1, 8, 64, 16384)]
    for idx, (S, N, out) in enumerate(shapes):
        name = f"sweep_s{S}_n{N}"
        cfgs[name] = LayerConfig(name, S, N, out, seed=(4, idx))
    return cfgs


CONFIGS: dict[str, LayerConfig] = {
    "tiny": LayerConfig("tiny", 16, 256, 256, seed=(0,), outliers=("channels", 2, 50.0)),
    "q_proj": LayerConfig("q_proj", 2048, 4096, 4096, seed=(1,),
                          outliers=("channels_uniform", 8, 20.0, 100.0)),
    "gate_up": LayerConfig("gate_up", 2048, 4096, 24576, seed=(2,)),
    "down_proj": LayerConfig("down_proj", 2048, 12288, 4096, seed=(3,), act="student_t3",
                             outliers=("block_channel", 4, 500.0)),
    **_sweep(),
}


# K/V projection outputs of the evaluated 8B model (8 kv heads x head dim 128: rows of
# N = 1024), as written into the KV cache: a prefill chunk of 2048 tokens and a decode step of
# 64 sequences (one token each).  Keys carry a few strong channels.
KV_CONFIGS: dict[str, LayerConfig] = {
    "kv_prefill": LayerConfig("kv_prefill", 2048, 1024, 0, seed=(7,),
                              outliers=("channels_uniform", 4, 10.0, 50.0)),
    "kv_decode": LayerConfig("kv_decode", 64, 1024, 0, seed=(8,),
                             outliers=("channels_uniform", 4, 10.0, 50.0)),
}


@dataclass
class Layer:
    cfg: LayerConfig
    x_bits: np.ndarray            # uint16 [S, N] bf16 bit patterns
    A: np.ndarray                 # fp32 [8, 8]
    B: np.ndarray                 # fp32 [k, 4, 4]
    alpha_min: np.ndarray         # fp32 [k]
    alpha_max: np.ndarray         # fp32 [k]
    W: np.ndarray | None = field(default=None)   # fp32 [out, N]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest bf16 (ties to even); returns the uint16 bit patterns.
    Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def custom(name: str, S: int, N: int, out: int, seed, act="normal",
           outliers=("channels", 8, 50.0)) -> LayerConfig:
    """A config of any shape (N a multiple of 32), e.g. a scaled-down parity case."""
    seed = tuple(seed) if isinstance(seed, (tuple, list)) else (int(seed),)
    return LayerConfig(name, S, N, out, seed=seed, act=act, outliers=outliers)


def make_layer(cfg: LayerConfig | str, with_weight: bool = True) -> Layer:
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg] if cfg in CONFIGS else KV_CONFIGS[cfg]
    assert cfg.N % 32 == 0 and cfg.N > 0
    S, N, out, k = cfg.S, cfg.N, cfg.out, cfg.k
    ss = np.random.SeedSequence(list(cfg.seed))
    r_x, r_out, r_a, r_b, r_alpha, r_w = (np.random.Generator(np.random.PCG64(c))
                                          for c in ss.spawn(6))

    if cfg.act == "normal":
        x = r_x.standard_normal((S, N), dtype=np.float32)
    elif cfg.act == "student_t3":
        x = r_x.standard_t(3.0, size=(S, N)).astype(np.float32)
    else:
        raise ValueError(cfg.act)

    kind = cfg.outliers[0]
    if kind == "channels":
        n_ch, mult = cfg.outliers[1], cfg.outliers[2]
        ch = r_out.choice(N, size=min(n_ch, N), replace=False)
        x[:, ch] *= np.float32(mult)
    elif kind == "channels_uniform":
        n_ch, lo, hi = cfg.outliers[1], cfg.outliers[2], cfg.outliers[3]
        ch = r_out.choice(N, size=min(n_ch, N), replace=False)
        mult = r_out.uniform(lo, hi, size=ch.size).astype(np.float32)
        x[:, ch] *= mult[None, :]
    elif kind == "block_channel":
        n_blk, mult = cfg.outliers[1], cfg.outliers[2]
        blocks = r_out.choice(k, size=min(n_blk, k), replace=False)
        ch = blocks * 32 + r_out.integers(0, 32, size=blocks.size)
        x[:, ch] *= np.float32(mult)
    elif kind == "none":
        pass
    else:
        raise ValueError(kind)
    x_bits = f32_to_bf16_bits(x)
    del x

    A = (np.eye(8) + 0.1 * r_a.standard_normal((8, 8))).astype(np.float32)
    B = (np.eye(4)[None] + 0.1 * r_b.standard_normal((k, 4, 4))).astype(np.float32)
    alpha = r_alpha.normal(2.0, 0.5, size=(2, k)).astype(np.float32)
    W = None
    if with_weight:
        W = r_w.standard_normal((out, N), dtype=np.float32)
        W *= np.float32(0.02)
    layer = Layer(cfg, x_bits, A, np.ascontiguousarray(B), np.ascontiguousarray(alpha[0]),
                  np.ascontiguousarray(alpha[1]), W)
    # conditioning guard for the generated factors (near-identity draws are far from it)
    assert np.linalg.cond(A.astype(np.float64)) < 1e3
    assert np.max(np.linalg.cond(B.astype(np.float64))) < 1e3
    return layer


def random_mxfp4(rows: int, N: int, seed, scale_lo: int = 110, scale_hi: int = 145):
    """Seeded random MXFP4 operands for the GEMM alone: uniformly random code bytes
    [rows, N/2] and E8M0 scale bytes [rows, N/32] in [scale_lo, scale_hi)."""
    seed = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    q = rng.integers(0, 256, size=(rows, N // 2), dtype=np.uint8)
    e = rng.integers(scale_lo, scale_hi, size=(rows, N // 32), dtype=np.uint8)
    return q, e


def random_mxfp8(rows: int, N: int, seed, scale_lo: int = 110, scale_hi: int = 145):
    """Seeded random MXFP8 (E4M3) operands for the GEMM alone: code bytes [rows, N], uniform
    over the 254 non-NaN E4M3 encodings (the two NaN bytes 0x7F and 0xFF are moved down to
    0x7E and 0xFE), and E8M0 scale bytes [rows, N/32] in [scale_lo, scale_hi)."""
    seed = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    q = rng.integers(0, 256, size=(rows, N), dtype=np.uint8)
    q[(q & 0x7F) == 0x7F] -= 1
    e = rng.integers(scale_lo, scale_hi, size=(rows, N // 32), dtype=np.uint8)
    return q, e


def form_factors(form: int, k: int, seed):
    """Seeded near-identity factors for a transform form (0 GPK, 1 Kronecker with private
    A_i, 2 full 32x32 P_i), drawn like the GPK factors of make_layer: identity plus 0.1 N(0,1)
    (0.05 for the 32x32 P_i).  Returns (F0, F1); F1 is None for the full form."""
    seed = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    if form == 2:
        P = np.eye(32) + 0.05 * rng.standard_normal((k, 32, 32))
        return P.astype(np.float32), None
    B = (np.eye(4) + 0.1 * rng.standard_normal((k, 4, 4))).astype(np.float32)
    if form == 1:
        A = (np.eye(8) + 0.1 * rng.standard_normal((k, 8, 8))).astype(np.float32)
    else:
        A = (np.eye(8) + 0.1 * rng.standard_normal((8, 8))).astype(np.float32)
    return A, B


def kv_slots(T: int, num_slots: int, seed, skip: float = 0.0) -> np.ndarray:
    """Seeded slot map of T tokens into a cache of num_slots rows: distinct rows drawn
    without replacement, then a fraction `skip` of the tokens set to -1 (padding tokens that
    are not cached).  int64 [T]."""
    assert T <= num_slots
    seed = list(seed) if isinstance(seed, (tuple, list)) else [int(seed)]
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed)))
    slots = rng.choice(num_slots, size=T, replace=False).astype(np.int64)
    slots[rng.random(T) < skip] = -1
    return slots
