"""Seeded synthetic inputs and the workload shapes.

This module holds input generation only: it contains none of the method's
arithmetic, so both the HIP path's tests and the CPU oracle may draw from it.

Recipe: numpy PCG64 seeded with crc32 of a tag string
``"cfg{c}/L{layer}/{name}/{W|x}"``.  Latent weights are float32
N(0, 0.02); activations are float32 N(0, 1) rounded to bfloat16 (nearest,
ties to even) and carried as raw uint16 bits.

Shapes come from the pages:
  * "BitNet TinyDialogues 1.58b", "Arquitetura": hidden 256, FFN 512;
  * "halo-sparse-bitnet-3:4-500m", "Recipe": Qwen2.5-0.5B skeleton, d_model
    896, d_ffn 4864, 14 heads / 2 KV heads (head dim 64, so k/v are 128 wide),
    24 layers; batch 16 x seq 2048 = 32768 tokens per micro-batch;
  * "Tritter 500M Hybrid BitNet", "Architecture Specifications": hidden 2048,
    16 layers, 32 heads, intermediate 7168 (no KV-head count is given, so k/v
    are read as full width).
"""
from __future__ import annotations

import zlib

import numpy as np

WEIGHT_STD = 0.02


def rng(tag: str) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(zlib.crc32(tag.encode())))


def latent_weight(tag: str, rows: int, cols: int, std: float = WEIGHT_STD) -> np.ndarray:
    """float32 [rows, cols] ~ N(0, std)."""
    return (rng(tag).standard_normal((rows, cols), dtype=np.float32)
            * np.float32(std)).astype(np.float32)


def float_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even), returning uint16 bits.
    Used for input generation only."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u + bias) >> np.uint64(16)).astype(np.uint16)


def activations_bf16(tag: str, tokens: int, cols: int) -> np.ndarray:
    """uint16 bf16 bits [tokens, cols] of N(0, 1) samples."""
    x = rng(tag).standard_normal((tokens, cols), dtype=np.float32)
    return float_to_bf16_bits(x)


def norm_weight(tag: str, cols: int) -> np.ndarray:
    """float32 [cols] per-channel RMSNorm weight ~ N(1, 0.1) (a trained
    norm's weights sit around 1)."""
    return (np.float32(1) + rng(tag).standard_normal(cols, dtype=np.float32)
            * np.float32(0.1)).astype(np.float32)


def grad_output(tag: str, tokens: int, cols: int) -> np.ndarray:
    """float32 [tokens, cols] ~ N(0, 1e-3): a stand-in for the gradient of
    the loss with respect to a layer's output."""
    return (rng(tag).standard_normal((tokens, cols), dtype=np.float32)
            * np.float32(1e-3)).astype(np.float32)


def mask_flip(tag: str, mask_bits: np.ndarray, fraction: float) -> np.ndarray:
    """A copy of a bit-packed mask with about `fraction` of its bits
    flipped at random (input generation for the mask-monitor tests)."""
    bits = np.unpackbits(np.asarray(mask_bits, dtype=np.uint8), bitorder="little")
    flip = rng(tag).random(bits.size) < fraction
    return np.packbits(bits ^ flip.astype(np.uint8), bitorder="little")


# ---------------------------------------------------------------------------
# Workload shapes: (name, out_features, in_features)
# ---------------------------------------------------------------------------
TINY_LINEAR = ("tiny", 512, 256)
TINY_TOKENS = 128

QWEN05B_D, QWEN05B_FFN, QWEN05B_LAYERS = 896, 4864, 24
QWEN05B_KV = 128  # 2 KV heads x head dim 64
QWEN05B_LINEARS = [
    ("q", QWEN05B_D, QWEN05B_D),
    ("k", QWEN05B_KV, QWEN05B_D),
    ("v", QWEN05B_KV, QWEN05B_D),
    ("o", QWEN05B_D, QWEN05B_D),
    ("gate", QWEN05B_FFN, QWEN05B_D),
    ("up", QWEN05B_FFN, QWEN05B_D),
    ("down", QWEN05B_D, QWEN05B_FFN),
]
QWEN05B_PREFILL_TOKENS = 16 * 2048

WIDE_D, WIDE_FFN, WIDE_LAYERS = 2048, 7168, 16
WIDE_LINEARS = [
    ("q", WIDE_D, WIDE_D),
    ("k", WIDE_D, WIDE_D),
    ("v", WIDE_D, WIDE_D),
    ("o", WIDE_D, WIDE_D),
    ("gate", WIDE_FFN, WIDE_D),
    ("up", WIDE_FFN, WIDE_D),
    ("down", WIDE_D, WIDE_FFN),
]
WIDE_PREFILL_TOKENS = 8192

DECODE_BATCHES = (1, 4, 16)
