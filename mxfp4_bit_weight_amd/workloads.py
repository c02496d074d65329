"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module draws random numbers and builds input structure only; it holds none
of the 4-bit format's arithmetic.  Every tensor comes from its own stream,
``numpy.random.Generator(PCG64(SeedSequence([seed, tensor_id])))``, drawn in
binary32 and rounded to nearest even to bf16 (by PyTorch's CPU cast).  bf16
tensors are returned as ``uint16`` bit patterns.

Shapes and distributions follow the workloads the pages discuss: Qwen-2.5-7B
decode projections (Telegram post tggo.me/sberlogasci/42740, section
"Eksperimenty": the method is validated on the Qwen-2.5 family), a batch of
8 x 2k tokens for the training-shaped GEMM (same section), and a 30B-A3B-class
mixture of experts (Nemotron 3.5 Lightning page, section 02: the 30B-A3B base
model; QATFactory page: dense and MoE models are supported).
"""
import numpy as np
import torch

# Named weight shapes (N, K) of a Qwen-2.5-7B decoder layer's projections.
QWEN7B_SHAPES = {
    "gate_up": (18944, 3584),
    "down": (3584, 18944),
    "qkv_o": (3584, 3584),
}
# One decoder layer's worth of tensors for the 7B-shaped quantize set
# (gate and up, down, and four 3584x3584 attention-sized projections).
QWEN7B_LAYER = [(18944, 3584)] * 2 + [(3584, 18944)] + [(3584, 3584)] * 4
QWEN7B_LAYERS = 28
LORA_RANK = 16
PREFILL_M = 8 * 2048                   # batch 8 x sequence 2048
MOE = dict(experts=128, topk=8, tokens=64, d_model=2048, d_ff=768)

# tensor ids inside one workload (draw order W, x, A, B)
TID_W, TID_X, TID_A, TID_B, TID_DELTA, TID_LOGITS, TID_DOWN_IN = 0, 1, 2, 3, 4, 5, 6


def rng(seed: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), int(tensor_id)])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """(binary64 ->) binary32 -> bf16 (round to nearest even), as uint16 bits."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _normal32(g: np.random.Generator, shape, std: float) -> np.ndarray:
    a = g.standard_normal(shape, dtype=np.float32)
    a *= np.float32(std)
    return a


def bernoulli_positions(g: np.random.Generator, count: int, p: float) -> np.ndarray:
    """Flat indices of a Bernoulli(p) mask over `count` entries, drawn as the
    geometric gaps between successes (the same process, far fewer draws)."""
    out = []
    pos = -1
    while True:
        gaps = g.geometric(p, size=int(count * p * 1.2) + 64)
        idx = pos + np.cumsum(gaps)
        out.append(idx[idx < count])
        if idx[-1] >= count:
            break
        pos = int(idx[-1])
    return np.concatenate(out)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to binary32 values."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(seed: int, tid: int, shape, std: float) -> np.ndarray:
    return to_bf16_bits(_normal32(rng(seed, tid), shape, std))


def outlier_weights(seed: int, tid: int, shape, std=0.02, p=0.001, mult=20.0) -> np.ndarray:
    """N(0, std) with a Bernoulli(p) mask of entries multiplied by ``mult`` (sign kept)."""
    g = rng(seed, tid)
    w = _normal32(g, shape, std)
    flat = w.reshape(-1)
    flat[bernoulli_positions(g, flat.size, p)] *= np.float32(mult)
    return to_bf16_bits(w)


def student_t_weights(seed: int, tid: int, shape, std=0.02, nu=4.0) -> np.ndarray:
    """Student-t(nu) scaled to standard deviation ``std`` (t_nu has std sqrt(nu/(nu-2))),
    drawn as Z * sqrt(nu / (2 G)) with Z ~ N(0, 1) and G ~ Gamma(nu/2, 1); for an
    even nu, G is the sum of nu/2 standard exponentials."""
    g = rng(seed, tid)
    z = g.standard_normal(shape, dtype=np.float32)
    if float(nu).is_integer() and int(nu) % 2 == 0:
        gam = g.standard_exponential(shape, dtype=np.float32)
        for _ in range(int(nu) // 2 - 1):
            gam += g.standard_exponential(shape, dtype=np.float32)
    else:
        gam = g.standard_gamma(nu / 2.0, size=shape, dtype=np.float32)
    z *= np.sqrt(np.float32(nu) / (np.float32(2.0) * gam))
    z *= np.float32(std / np.sqrt(nu / (nu - 2.0)))
    return to_bf16_bits(z)


def weights(kind: str, seed: int, tid: int, shape) -> np.ndarray:
    if kind == "normal":
        return normal_bf16(seed, tid, shape, 0.02)
    if kind == "outlier":
        return outlier_weights(seed, tid, shape)
    if kind == "student_t":
        return student_t_weights(seed, tid, shape)
    raise ValueError(kind)


def linear_inputs(seed: int, n: int, k: int, m: int, rank: int = LORA_RANK, wkind: str = "normal"):
    """W (n, k), x (m, k) ~ N(0, 1), LoRA A (rank, k) and B (n, rank) ~ N(0, 0.01)."""
    w = weights(wkind, seed, TID_W, (n, k))
    x = normal_bf16(seed, TID_X, (m, k), 1.0)
    a = normal_bf16(seed, TID_A, (rank, k), 0.01) if rank else None
    b = normal_bf16(seed, TID_B, (n, rank), 0.01) if rank else None
    return w, x, a, b


def merge_noise(seed: int, count: int) -> np.ndarray:
    """Standard normal draws, one per block; a scale-delta is 0.05 * s * z for the
    block's decoded scale s (the caller multiplies)."""
    return rng(seed, TID_DELTA).standard_normal(count, dtype=np.float32)


def moe_routing(seed: int, tokens=MOE["tokens"], experts=MOE["experts"], topk=MOE["topk"]):
    """Top-k routing from N(0, 1) logits (softmax is monotone, so top-k of the
    logits).  Returns (row_index (tokens*topk,) int32, offsets (experts+1,) int32):
    rows are sorted stably by (expert, token) and row_index holds the token."""
    logits = rng(seed, TID_LOGITS).standard_normal((tokens, experts))
    top = np.argsort(-logits, axis=1, kind="stable")[:, :topk]            # (tokens, topk)
    tok = np.repeat(np.arange(tokens), topk)
    exp = top.reshape(-1)
    order = np.lexsort((tok, exp))                                          # by expert, then token
    row_index = tok[order].astype(np.int32)
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_index, offsets


def moe_expert_weights(seed: int, experts: int, n: int, k: int, tid_base: int = 100):
    """(experts, n, k) bf16 expert weights ~ N(0, 0.02), one stream per expert."""
    out = np.empty((experts, n, k), np.uint16)
    for e in range(experts):
        out[e] = normal_bf16(seed, tid_base + e, (n, k), 0.02)
    return out
