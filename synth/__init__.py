"""Seeded synthetic workloads for sliced r-bit qgemm.

This module produces inputs only: parent codes, bf16 group scales and bf16
activations.  It holds none of the method's arithmetic (no bit-planes, no
slicing, no dequantisation, no products), so the CPU oracle and the GPU library
can both consume its output without sharing any of the computation.

Shapes follow the decoder linears the MatGPTQ pages evaluate (MatGPTQ:
Efficient and Accurate Inference over Nested Quantized Models, Table 3 lists
the Llama-3.1-8B linears as out x in; Tables 2 and 4-7 name Llama3.1-8B-Instruct
and Qwen3-8B).  Trained weights are not available here and are not needed to
measure throughput, so weights are drawn from the recipes below.

Recipes (every draw is seeded; one numpy stream per tensor,
``default_rng([seed, workload_id, shape_id, tensor_id])``):

* ``uniform``: codes i.i.d. uniform on {0..255}; scales U(0.001, 0.01) rounded
  to bf16; activations N(0, 1) rounded to bf16.
* ``gptq_like``: fp32 weights N(0, 0.02); per (row, 128-wide group along k) the
  scale is s = bf16(absmax / 127.5) and the code is the nearest level of the
  8-bit grid s*(c - 127.5), i.e. c = clamp(floor(w/s + 128), 0, 255); an
  all-zero group gets s = 0 and c = 128.  This round-to-nearest pass stands in
  for the calibrated quantiser, which needs data this build does not have.
* activations with outliers: N(0, 1), then round(0.01*k) distinct channels
  (chosen uniformly) multiplied by 10, then rounded to bf16.

bf16 rounding is round-to-nearest-even on the fp32 value.
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# (name, n_out, k_in) per decoder linear; q/k/v and gate/up are fused.
WORKLOADS = {
    "single-1024": [("w", 1024, 1024)],
    "llama3.1-8b": [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 28672, 4096),
                    ("down", 4096, 14336)],
    "qwen3-8b": [("qkv", 6144, 4096), ("o", 4096, 4096), ("gate_up", 24576, 4096),
                 ("down", 4096, 12288)],
    "llama-70b": [("qkv", 10240, 8192), ("o", 8192, 8192), ("gate_up", 57344, 8192),
                  ("down", 8192, 28672)],
}
WORKLOAD_IDS = {name: i for i, name in enumerate(WORKLOADS)}

T_CODES, T_SCALES, T_X, T_OUTLIERS, T_WEIGHTS = range(5)


def rng_for(seed: int, workload_id: int, shape_id: int, tensor_id: int) -> np.random.Generator:
    return np.random.default_rng([seed, workload_id, shape_id, tensor_id])


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if not np.all(np.isfinite(a)):
        raise ValueError("non-finite value in bf16 rounding")
    u = a.view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def uniform_codes(n: int, k: int, rng: np.random.Generator) -> np.ndarray:
    return rng.integers(0, 256, size=(n, k), dtype=np.uint8)


def uniform_scales(n: int, k: int, rng: np.random.Generator, lo: float = 0.001,
                   hi: float = 0.01) -> np.ndarray:
    return f32_to_bf16_bits(rng.uniform(lo, hi, size=(n, k // GROUP)).astype(np.float32))


def gptq_like(n: int, k: int, rng: np.random.Generator, sigma: float = 0.02):
    """Round-to-nearest 8-bit codes and bf16 absmax scales for N(0, sigma) weights."""
    codes = np.empty((n, k), dtype=np.uint8)
    scales = np.empty((n, k // GROUP), dtype=np.uint16)
    step = 4096  # rows per block, to bound temporary memory
    for r0 in range(0, n, step):
        r1 = min(n, r0 + step)
        w = rng.normal(0.0, sigma, size=(r1 - r0, k)).astype(np.float32)
        wg = w.reshape(r1 - r0, k // GROUP, GROUP).astype(np.float64)
        absmax = np.abs(wg).max(axis=2)
        s_bits = f32_to_bf16_bits((absmax / 127.5).astype(np.float32))
        s = bf16_bits_to_f32(s_bits).astype(np.float64)
        safe = np.where(s > 0, s, 1.0)[:, :, None]
        c = np.floor(wg / safe + 128.0)
        c = np.where(s[:, :, None] > 0, c, 128.0)
        codes[r0:r1] = np.clip(c, 0, 255).astype(np.uint8).reshape(r1 - r0, k)
        scales[r0:r1] = s_bits
    return codes, scales


def activations(batch: int, k: int, rng: np.random.Generator, outliers: bool = False,
                outlier_rng: np.random.Generator | None = None) -> np.ndarray:
    x = rng.normal(0.0, 1.0, size=(batch, k)).astype(np.float32)
    if outliers:
        orng = outlier_rng if outlier_rng is not None else rng
        cols = orng.choice(k, size=int(round(0.01 * k)), replace=False)
        x[:, cols] *= np.float32(10.0)
    return f32_to_bf16_bits(x)


def make_linear(workload: str, shape_id: int, batch: int, seed: int = 0, recipe: str | None = None,
                outliers: bool | None = None):
    """Inputs for one linear of a named workload.

    Returns a dict with ``name, n, k, codes [n][k] uint8, scales [n][k/128] uint16 (bf16),
    x [batch][k] uint16 (bf16)``.  Default recipe: ``uniform`` for ``single-1024``, else
    ``gptq_like``; outliers default to batch >= 32.
    """
    wid = WORKLOAD_IDS[workload]
    name, n, k = WORKLOADS[workload][shape_id]
    if recipe is None:
        recipe = "uniform" if workload == "single-1024" else "gptq_like"
    if outliers is None:
        outliers = batch >= 32 and workload != "single-1024"
    if recipe == "uniform":
        codes = uniform_codes(n, k, rng_for(seed, wid, shape_id, T_CODES))
        scales = uniform_scales(n, k, rng_for(seed, wid, shape_id, T_SCALES))
    elif recipe == "gptq_like":
        codes, scales = gptq_like(n, k, rng_for(seed, wid, shape_id, T_WEIGHTS))
    else:
        raise ValueError(f"unknown recipe {recipe!r}")
    x = activations(batch, k, rng_for(seed, wid, shape_id, T_X), outliers=outliers,
                    outlier_rng=rng_for(seed, wid, shape_id, T_OUTLIERS))
    return {"name": name, "n": n, "k": k, "codes": codes, "scales": scales, "x": x,
            "recipe": recipe, "outliers": outliers}


def random_case(n: int, k: int, batch: int, seed: int, recipe: str = "uniform",
                outliers: bool = False):
    """A free-shape case for parity tests (same recipes, shape chosen by the caller)."""
    base = np.random.default_rng([seed, 1000, n, k, batch])
    if recipe == "uniform":
        codes = uniform_codes(n, k, base)
        scales = uniform_scales(n, k, base)
    else:
        codes, scales = gptq_like(n, k, base)
    x = activations(batch, k, base, outliers=outliers)
    return {"n": n, "k": k, "codes": codes, "scales": scales, "x": x}
