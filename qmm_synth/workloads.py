"""The seeded synthetic workloads (shapes, formats, value distributions, seeds).

Weights are drawn N(0, 0.02^2) in fp32 and encoded by ``quantize``; activations
are N(0, 1), cast to fp32 or fp16 (round to nearest even).  RNG: NumPy PCG64
via ``default_rng(seed)`` with the integer-list seeds below.  The workloads
stand in for the pages' models, which are not available: the candle pull
request "Metal: 64-token tile for the quantized matrix-matrix kernel" times the
seven Qwen3-Embedding-4B Q4_K_M projection shapes (section "Numbers", shape
table) with random weights; the tiny-llm pull request "perf: Optimize quantized
matmul for small decode batches" decodes Qwen3-0.6B in MLX 4-bit (section
"Benchmark setup") at batch 1..16; the llama.cpp pull request "metal : fix idle
threads in mul_mv_iq3_xxs for ne00 < 1024" times the expert-indexed
matrix-vector product at ne00 = 512 for n = 2..24 tokens with expert ids
rotated between timed batches (section "Additional information").
"""

import numpy as np

from .quantize import quantize

# Decoder projections of a Qwen3-Embedding-4B layer: (name, M rows, K, format).
DECODE_SHAPES = [
    ("attn_q", 4096, 2560, "q4_k"),
    ("attn_k", 1024, 2560, "q4_k"),
    ("attn_v", 1024, 2560, "q6_k"),
    ("attn_output", 2560, 4096, "q4_k"),
    ("ffn_gate", 9728, 2560, "q4_k"),
    ("ffn_up", 9728, 2560, "q4_k"),
    ("ffn_down", 2560, 9728, "q6_k"),
]

# One Qwen3-0.6B decoder layer, all in 4-bit affine groups of 64.
SMALL_DECODE_SHAPES = [
    ("q", 2048, 1024),
    ("k", 1024, 1024),
    ("v", 1024, 1024),
    ("o", 1024, 2048),
    ("gate", 3072, 1024),
    ("up", 3072, 1024),
    ("down", 1024, 3072),
]
SMALL_DECODE_TOKENS = [1, 2, 4, 8, 16]

PREFILL_TOKENS = [7, 33, 64, 96, 130, 512, 2048]
FORMAT_ORDER = ["q4_0", "q8_0", "q4_k", "q6_k", "a4g64"]
# every block format, for the per-format sweep (one 4096 x 4096 matrix each)
ALL_FORMATS = FORMAT_ORDER + ["q4_1", "q5_0", "q5_1", "q2_k", "q3_k", "q5_k"]
SWEEP_M = SWEEP_K = 4096
SWEEP_TOKENS = [1, 512]

# Expert-indexed narrow-K matvec: E experts of M x K in Q4_0, S ids per token.
MOE_EXPERTS, MOE_M, MOE_K, MOE_SLOTS = 128, 4096, 512, 8
MOE_TOKENS = [2, 4, 8, 12, 16, 24]


def rng(seed):
    return np.random.default_rng(seed)


def draw_weights(g, M, K):
    return g.normal(0.0, 0.02, size=(M, K)).astype(np.float32)


def draw_x(g, shape, dtype):
    return g.standard_normal(size=shape).astype(np.float32).astype(dtype)


# --- the single small matvec: Q4_0 256 x 512, one fp32 token, seed 0 ---------------------
def single_matvec():
    g = rng(0)
    w = draw_weights(g, 256, 512)
    blob = quantize("q4_0", w)
    x = draw_x(g, (1, 512), np.float32)
    return {"fmt": "q4_0", "M": 256, "K": 512, "blob": blob, "x": x}


# --- decode layer (Q4_K / Q6_K), and the prefill that reuses its weights ------------------
def decode_weights(i):
    name, M, K, fmt = DECODE_SHAPES[i]
    w = draw_weights(rng([1, i]), M, K)
    return {"name": name, "fmt": fmt, "M": M, "K": K, "blob": quantize(fmt, w)}


def decode_weights_fp32(i):
    """The fp32 weights decode_weights(i) encodes (same seed)."""
    _, M, K, _ = DECODE_SHAPES[i]
    return draw_weights(rng([1, i]), M, K)


def decode_x(i, n=1):
    _, _, K, _ = DECODE_SHAPES[i]
    return draw_x(rng([1, i, n]), (n, K), np.float32)


def prefill_x(i, n):
    _, _, K, _ = DECODE_SHAPES[i]
    return draw_x(rng([3, i, n]), (n, K), np.float16)


def prefill_batch(fmt_index):
    """A batch of 2 sequences of 65 tokens (flattened to 130) on a 128 x 768 matrix."""
    fmt = FORMAT_ORDER[fmt_index]
    g = rng([3, 99, fmt_index])
    w = draw_weights(g, 128, 768)
    blob = quantize(fmt, w)
    x = draw_x(g, (2 * 65, 768), np.float16)
    return {"fmt": fmt, "M": 128, "K": 768, "blob": blob, "x": x}


# --- small-batch decode in 4-bit affine groups -----------------------------------------------
def small_decode_weights(i):
    name, M, K = SMALL_DECODE_SHAPES[i]
    w = draw_weights(rng([2, i]), M, K)
    return {"name": name, "fmt": "a4g64", "M": M, "K": K, "blob": quantize("a4g64", w)}


def small_decode_x(i, n):
    _, _, K = SMALL_DECODE_SHAPES[i]
    return draw_x(rng([2, i, n]), (n, K), np.float16)


# --- expert-indexed matvec ------------------------------------------------------------------------
def moe_expert(e):
    """Expert e's blocks (Q4_0, MOE_M x MOE_K), seed [4, e]."""
    w = draw_weights(rng([4, e]), MOE_M, MOE_K)
    return quantize("q4_0", w)


def moe_stack(n_experts=MOE_EXPERTS):
    return np.concatenate([moe_expert(e) for e in range(n_experts)])


def moe_x(n):
    return draw_x(rng([4, n]), (n, MOE_SLOTS, MOE_K), np.float32)


MOE_PREFILL_TOKENS = [64, 256, 1024]


def moe_prefill_x(n):
    """[n, slots, K] fp16 activations of a prefill-sized expert-indexed call."""
    return draw_x(rng([4, n, 7]), (n, MOE_SLOTS, MOE_K), np.float16)


def moe_ids(n, call, n_experts=MOE_EXPERTS, slots=MOE_SLOTS):
    """[n, slots] int32: per token, ``slots`` distinct experts drawn uniformly."""
    g = rng([4, n, call])
    return np.stack([g.choice(n_experts, slots, replace=False) for _ in range(n)]).astype(np.int32)


def generic(fmt, M, K, n, seed, xdtype=np.float32):
    """Any shape: weights then activations from one seed."""
    g = rng(seed)
    w = draw_weights(g, M, K)
    return {"fmt": fmt, "M": M, "K": K, "blob": quantize(fmt, w), "x": draw_x(g, (n, K), xdtype)}


# --- per-format sweep: one 4096 x 4096 matrix per block format ------------------------------
def format_sweep_weights(fmt):
    """Weights N(0, 0.02^2) of a 4096 x 4096 matrix encoded as `fmt`, seed [5, format index]."""
    w = draw_weights(rng([5, ALL_FORMATS.index(fmt)]), SWEEP_M, SWEEP_K)
    return {"fmt": fmt, "M": SWEEP_M, "K": SWEEP_K, "blob": quantize(fmt, w)}


def format_sweep_x(n):
    """n tokens of activations for the sweep: fp32 for the matrix-vector call, fp16 otherwise."""
    return draw_x(rng([5, 99, n]), (n, SWEEP_K), np.float32 if n == 1 else np.float16)
