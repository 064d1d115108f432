"""Seeded synthetic BF16 weights shaped like Qwen3-14B.

This module only *makes inputs*: it draws random values, rounds them to BF16
bit patterns and lists tensor shapes. It holds none of the codec's arithmetic,
so both the CPU oracle (under ``oracle/``) and the GPU path may use it.

Shapes follow the Qwen3-14B configuration table ("Memory requirements of
language model inference on a consumer GPU", Table 2: V = 151,936, d = 5,120,
L = 40, 40 query heads, 8 KV heads, head_dim 128) and its per-part weight
counts (same page, Table 4: ~330M weights per decoder layer, ~778M for the
embedding and for the output head, 14.8B in total).

Value recipes (the pages print none; these stand in for the released
checkpoint, which is not available):

* ``normal``: N(mu, sigma) drawn in float32, rounded to BF16 with
  round-to-nearest-even. Matrices use N(0, 0.02), RMSNorm vectors N(1, 0.05).
* ``t4``: a heavy-tailed Student-t with 4 degrees of freedom, built as
  Z / sqrt(W / 4) with W = -2 ln(U1 U2) (a chi-square with 4 degrees of
  freedom), scaled by 0.02; then every entry independently, with probability
  0.001, is multiplied by 100 to widen the exponent alphabet.

Streams are drawn block by block: block ``b`` of ``BLOCK`` elements uses its
own PCG64 generator seeded from ``SeedSequence([seed, b])``. The result is
therefore independent of the thread count, and any block can be regenerated
alone (used for sampled checks on multi-GB tensors).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

BLOCK = 1 << 22  # elements per independently seeded generator block

# Qwen3-14B configuration (Table 2 of the first page).
VOCAB = 151_936
HIDDEN = 5_120
N_LAYERS = 40
N_HEADS = 40
N_KV_HEADS = 8
HEAD_DIM = 128
FFN = 17_408  # Qwen3-14B intermediate size; gives the page's ~330M per layer


@dataclass(frozen=True)
class TensorSpec:
    """One synthetic tensor: name, shape, value recipe and seed."""

    name: str
    shape: tuple
    dist: str  # "normal" or "t4"
    seed: int
    mu: float = 0.0
    sigma: float = 0.02

    @property
    def numel(self) -> int:
        n = 1
        for s in self.shape:
            n *= int(s)
        return n


def f32_to_bf16_bits(f: np.ndarray) -> np.ndarray:
    """Round float32 values to BF16 (round to nearest, ties to even).

    Returns the uint16 bit patterns. Inputs here are finite, so the NaN case
    of the rounding rule never arises.
    """
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """Widen BF16 bit patterns to float32 (exact)."""
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _block_rng(seed: int, block: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, block])))


def _draw_block(spec: TensorSpec, block: int, count: int) -> np.ndarray:
    rng = _block_rng(spec.seed, block)
    if spec.dist == "normal":
        z = rng.standard_normal(count, dtype=np.float32)
        v = z * np.float32(spec.sigma) + np.float32(spec.mu)
    elif spec.dist == "t4":
        z = rng.standard_normal(count, dtype=np.float32)
        u1 = np.float32(1.0) - rng.random(count, dtype=np.float32)  # (0, 1]
        u2 = np.float32(1.0) - rng.random(count, dtype=np.float32)
        w = np.float32(-2.0) * np.log(u1 * u2)  # chi-square, 4 dof
        # w == 0 only when u1 == u2 == 1; keep it finite in that event.
        w = np.maximum(w, np.float32(1e-30))
        v = z / np.sqrt(w * np.float32(0.25)) * np.float32(spec.sigma)
        widen = rng.random(count, dtype=np.float32) < np.float32(0.001)
        v[widen] *= np.float32(100.0)
    else:
        raise ValueError(f"unknown distribution {spec.dist!r}")
    return f32_to_bf16_bits(v)


def block_count(n: int) -> int:
    return (n + BLOCK - 1) // BLOCK


def generate_block(spec: TensorSpec, block: int) -> np.ndarray:
    """BF16 bits of elements [block*BLOCK, min(n, (block+1)*BLOCK))."""
    n = spec.numel
    lo = block * BLOCK
    if lo >= n:
        return np.zeros(0, np.uint16)
    return _draw_block(spec, block, min(BLOCK, n - lo))


def generate(spec: TensorSpec, out: np.ndarray | None = None, threads: int | None = None) -> np.ndarray:
    """Flat uint16 BF16 bit patterns of the whole tensor (row-major)."""
    n = spec.numel
    if out is None:
        out = np.empty(n, np.uint16)
    if out.dtype != np.uint16 or out.size != n or not out.flags.c_contiguous:
        raise ValueError(f"out must be a contiguous uint16 array of {n} values")
    nb = block_count(n)
    if threads is None:
        threads = min(16, os.cpu_count() or 1)

    def fill(b: int) -> None:
        lo = b * BLOCK
        out[lo:lo + min(BLOCK, n - lo)] = _draw_block(spec, b, min(BLOCK, n - lo))

    if nb <= 1 or threads <= 1:
        for b in range(nb):
            fill(b)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(fill, range(nb)))
    return out


# --------------------------------------------------------------------------
# Workloads: a single tensor, one decoder layer, the embedding, the model.
# --------------------------------------------------------------------------

LAYER_TENSORS = (
    # name, shape, dist, mu, sigma
    ("q_proj", (N_HEADS * HEAD_DIM, HIDDEN), "normal", 0.0, 0.02),
    ("k_proj", (N_KV_HEADS * HEAD_DIM, HIDDEN), "normal", 0.0, 0.02),
    ("v_proj", (N_KV_HEADS * HEAD_DIM, HIDDEN), "normal", 0.0, 0.02),
    ("o_proj", (HIDDEN, N_HEADS * HEAD_DIM), "normal", 0.0, 0.02),
    ("gate_proj", (FFN, HIDDEN), "normal", 0.0, 0.02),
    ("up_proj", (FFN, HIDDEN), "normal", 0.0, 0.02),
    ("down_proj", (HIDDEN, FFN), "normal", 0.0, 0.02),
    ("input_layernorm", (HIDDEN,), "normal", 1.0, 0.05),
    ("post_attention_layernorm", (HIDDEN,), "normal", 1.0, 0.05),
    ("q_norm", (HEAD_DIM,), "normal", 1.0, 0.05),
    ("k_norm", (HEAD_DIM,), "normal", 1.0, 0.05),
)


def single_tensor(rows: int = 1024, cols: int = 1024, seed: int = 1) -> list[TensorSpec]:
    """A single N(0, 0.02) matrix (1024x1024, or a 5120x5120 q_proj)."""
    return [TensorSpec(f"w{rows}x{cols}", (rows, cols), "normal", seed)]


def decoder_layer(layer: int = 0) -> list[TensorSpec]:
    """The 11 tensors of one Qwen3-14B-shaped decoder layer (~0.66 GB BF16).

    Tensor t of layer l is seeded with 1000 * (l + 1) + t.
    """
    return [TensorSpec(f"layers.{layer}.{name}", shape, dist, 1000 * (layer + 1) + t, mu, sigma)
            for t, (name, shape, dist, mu, sigma) in enumerate(LAYER_TENSORS)]


def embedding(seed: int = 4, name: str = "embed_tokens") -> list[TensorSpec]:
    """Embedding-shaped 151936 x 5120 heavy-tailed tensor (~1.56 GB BF16)."""
    return [TensorSpec(name, (VOCAB, HIDDEN), "t4", seed)]


def model_units(n_layers: int = N_LAYERS) -> list[list[TensorSpec]]:
    """Streaming units of the whole model, in the order a token uses them.

    The embedding, each decoder layer, then the untied output head with the
    final RMSNorm. With 40 layers this totals the page's ~14.8B weights
    (~29.5 GB in BF16).
    """
    units = [embedding(4, "embed_tokens")]
    units += [decoder_layer(l) for l in range(n_layers)]
    units.append(embedding(5, "lm_head") + [TensorSpec("norm", (HIDDEN,), "normal", 6, 1.0, 0.05)])
    return units
