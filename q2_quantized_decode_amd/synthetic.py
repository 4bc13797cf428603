"""Seeded synthetic inputs for the Q2_K decode path.

This module only draws random bytes and numbers. It holds none of the
method's arithmetic: no Q2_K decoding, no q8_1 quantisation, no dot
products. Both the HIP path (through the tests and the bench) and the CPU
oracle are fed from here, so it is the one module they share.

Distributions follow the workloads the pages describe:

* Q2_K weight blocks: scale/min bytes and 2-bit quant bytes uniform in
  0..255 (both nibbles and all four bit-pairs uniform), super-block scales
  ``d`` and ``dmin`` drawn as fp16 of ``|N(0, 0.02)|``. The block is the
  84-byte, 256-weight record the metrale ``engram_v41.rs`` page names
  (``ENGRAM_ROW_BYTES``; ``EngramLayerWeights::wkv_q2k``, "as the GGUF ships
  it"), in the GGUF Q2_K byte order: 16 scale bytes, 64 quant bytes, fp16 d,
  fp16 dmin.
* Activations: bf16 values of ``N(0, 1)``, optionally with a Bernoulli
  fraction replaced by ``+-magnitude`` outliers.

bf16 and fp16 values are returned as their raw ``uint16`` bit patterns, so
no consumer has to agree on a rounding helper from here.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np
import torch

Q2K_BLOCK_BYTES = 84
Q2K_BLOCK_WEIGHTS = 256


def rng_for(*key: int) -> np.random.Generator:
    """A PCG64 generator seeded from an integer tuple (SeedSequence entropy)."""
    return np.random.default_rng(list(key))


def q2k_blocks(rng: np.random.Generator, n_rows: int, n_blocks: int,
               d_sigma: float = 0.02) -> np.ndarray:
    """Random Q2_K blocks as ``uint8 [n_rows, n_blocks, 84]``."""
    raw = rng.integers(0, 256, size=(n_rows, n_blocks, Q2K_BLOCK_BYTES), dtype=np.uint8)
    dd = np.abs(rng.normal(0.0, d_sigma, size=(n_rows, n_blocks, 2))).astype(np.float16)
    raw[:, :, 80:84] = dd.view(np.uint8).reshape(n_rows, n_blocks, 4)
    return raw


def f32_to_bf16_bits_torch(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 with torch's own conversion; return bits."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_normal(rng: np.random.Generator, shape, outlier_frac: float = 0.0,
                outlier_mag: float = 20.0) -> np.ndarray:
    """bf16 bits of N(0,1) samples; a Bernoulli(outlier_frac) subset is +-outlier_mag."""
    x = rng.standard_normal(size=shape).astype(np.float32)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape) < outlier_frac
        sign = np.where(rng.random(size=shape) < 0.5, -1.0, 1.0).astype(np.float32)
        x = np.where(mask, sign * np.float32(outlier_mag), x).astype(np.float32)
    return f32_to_bf16_bits_torch(x)


def bf16_bits_to_tensor(bits: np.ndarray) -> torch.Tensor:
    """Reinterpret uint16 bit patterns as a CPU bf16 tensor (no rounding)."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)


# --------------------------------------------------------------------------
# Workloads. Each is named for what it is; sizes are the pages' shapes.
# --------------------------------------------------------------------------

@dataclass
class SingleGemvCase:
    """One Q2_K matrix against one bf16 token: W [n, k/256 blocks], x [m, k]."""
    w: np.ndarray          # uint8 [n, k/256, 84]
    x_bits: np.ndarray     # uint16 [m, k] bf16 bits
    n: int
    k: int
    m: int


def single_gemv_case(n: int = 256, k: int = 1024, m: int = 1, seed: int = 1000,
                     outlier_frac: float = 0.0) -> SingleGemvCase:
    """Single Q2_K GEMV. Default: 256 rows x 1024 (4 super-blocks), one token."""
    rng = rng_for(seed)
    w = q2k_blocks(rng, n, k // Q2K_BLOCK_WEIGHTS)
    x = bf16_normal(rng, (m, k), outlier_frac=outlier_frac)
    return SingleGemvCase(w=w, x_bits=x, n=n, k=k, m=m)


def large_verify_case(m: int = 8, seed: int = 1004, n: int = 32768,
                      k: int = 7168) -> SingleGemvCase:
    """Large batched verify: one Q2_K matrix [32768, 7168] (28 super-blocks per
    row), bf16 activations [8, 7168] ~ N(0,1) with 5% outliers at +-20."""
    rng = rng_for(seed)
    w = q2k_blocks(rng, n, k // Q2K_BLOCK_WEIGHTS)
    x = bf16_normal(rng, (8, k), outlier_frac=0.05, outlier_mag=20.0)
    return SingleGemvCase(w=w, x_bits=x[:m].copy(), n=n, k=k, m=m)


@dataclass
class PairCase:
    """Two Q2_K matrices that read one shared input (attention wq_a / wkv)."""
    wa: np.ndarray
    wb: np.ndarray
    x_bits: np.ndarray
    na: int
    nb: int
    k: int
    m: int


def attention_pair_case(m: int, seed: int = 1002, na: int = 1024, nb: int = 512,
                        k: int = 4096) -> PairCase:
    """Attention input pair: x [m, 4096], wq_a [1024, 4096], wkv [512, 4096]."""
    rng = rng_for(seed, m)
    wa = q2k_blocks(rng, na, k // Q2K_BLOCK_WEIGHTS)
    wb = q2k_blocks(rng, nb, k // Q2K_BLOCK_WEIGHTS)
    x = bf16_normal(rng, (m, k))
    return PairCase(wa=wa, wb=wb, x_bits=x, na=na, nb=nb, k=k, m=m)


@dataclass
class GroupedCase:
    """Grouped-input product: x [m, groups*k] (the attention output), w
    [groups*rows, k] (wo_a), output [m, groups*rows]."""
    w: np.ndarray          # uint8 [groups*rows, k/256, 84]
    x_bits: np.ndarray     # uint16 [m, groups*k]
    groups: int
    rows: int
    k: int
    m: int


def grouped_case(m: int, seed: int = 1005, groups: int = 8, rows: int = 1024,
                 k: int = 2048) -> GroupedCase:
    """wo_a-shaped grouped product (the pages give no group sizes): 8 groups
    of 1024 rows over 2048-wide slices of a [m, 16384] input ~ N(0,1)."""
    rng = rng_for(seed, m)
    w = q2k_blocks(rng, groups * rows, k // Q2K_BLOCK_WEIGHTS)
    x = bf16_normal(rng, (m, groups * k))
    return GroupedCase(w=w, x_bits=x, groups=groups, rows=rows, k=k, m=m)


@dataclass
class EngramHashCase:
    """Hash tables of the engram n-gram hash and a token sequence."""
    token_map: np.ndarray      # int64 [vocab]; -1 = unmapped
    multipliers: np.ndarray    # int64 [n_layers, max_ngram]
    primes: np.ndarray         # int64 [n_layers, max_ngram - 1, n_heads]
    offsets: np.ndarray        # int64 [n_layers, (max_ngram - 1) * n_heads]
    pad_id: int
    n_heads: int
    tokens: np.ndarray         # int32 [seqlen]


def _primes_from(start: int, count: int) -> list:
    out, v = [], start
    while len(out) < count:
        v += 1
        if v > 1 and all(v % d for d in range(2, int(v ** 0.5) + 1)):
            out.append(v)
    return out


def engram_hash_case(seed: int = 1006, vocab: int = 4096, n_layers: int = 2, max_ngram: int = 3,
                     n_heads: int = 4, seqlen: int = 64, table_rows: int = 500000,
                     unmapped: float = 0.05) -> EngramHashCase:
    """Synthetic tables (the real ones ship in the GGUF metadata): compressed
    ids are a random map of the vocabulary with a share of unmapped (-1)
    entries; multipliers random non-negative 63-bit values; one distinct
    prime per (layer, column) near table_rows / (layers * columns); offsets
    lay the columns' ranges end to end, so every row id falls in
    [0, table_rows)."""
    rng = rng_for(seed)
    cols = (max_ngram - 1) * n_heads
    compressed = max(2, vocab * 3 // 4)
    token_map = rng.integers(0, compressed, size=vocab, dtype=np.int64)
    token_map[rng.random(vocab) < unmapped] = -1
    pad_token = int(rng.integers(0, vocab))
    token_map[pad_token] = int(rng.integers(0, compressed))
    multipliers = rng.integers(1, 1 << 63, size=(n_layers, max_ngram), dtype=np.int64)
    per = table_rows // (n_layers * cols)
    plist = _primes_from(per - 2000, n_layers * cols)
    primes = np.array(plist, dtype=np.int64).reshape(n_layers, max_ngram - 1, n_heads)
    flat = primes.reshape(n_layers, cols)
    offsets = np.zeros((n_layers, cols), dtype=np.int64)
    acc = 0
    for l in range(n_layers):
        for c in range(cols):
            offsets[l, c] = acc
            acc += int(flat[l, c])
    tokens = rng.integers(0, vocab, size=seqlen, dtype=np.int64).astype(np.int32)
    return EngramHashCase(token_map=token_map, multipliers=multipliers, primes=primes,
                          offsets=offsets, pad_id=int(token_map[pad_token]), n_heads=n_heads,
                          tokens=tokens)


@dataclass
class ExpertCase:
    """Routed-expert decode batch over a resident expert set."""
    n_experts: int
    dim: int
    inter: int
    ids: np.ndarray        # int32 [n_ids], drawn without replacement
    x_bits: np.ndarray     # uint16 [1, dim]
    seed: int

    # Matrix kinds: gate and up are [inter, dim]; down is [dim, inter].
    def expert_matrix(self, expert: int, kind: str) -> np.ndarray:
        kind_id = {"gate": 0, "up": 1, "down": 2}[kind]
        rng = rng_for(self.seed, expert, kind_id)
        if kind == "down":
            return q2k_blocks(rng, self.dim, self.inter // Q2K_BLOCK_WEIGHTS)
        return q2k_blocks(rng, self.inter, self.dim // Q2K_BLOCK_WEIGHTS)


def expert_batch_case(seed: int = 1003, n_experts: int = 256, dim: int = 4096,
                      inter: int = 2048, n_ids: int = 8) -> ExpertCase:
    """256 experts of Q2_K gate/up [2048, 4096] and down [4096, 2048]; 8 ids
    drawn without replacement; one bf16 token [1, 4096] ~ N(0,1)."""
    rng = rng_for(seed)
    ids = rng.choice(n_experts, size=n_ids, replace=False).astype(np.int32)
    x = bf16_normal(rng, (1, dim))
    return ExpertCase(n_experts=n_experts, dim=dim, inter=inter, ids=ids, x_bits=x, seed=seed)


@dataclass
class EngramCase:
    """Engram single-token step: row gather, wkv projection, gate."""
    table: np.ndarray      # uint8 [n_table_rows, 1, 84] (one block per row)
    ids: np.ndarray        # int64 [cols]
    wkv: np.ndarray        # uint8 [dim*(hc+1), cols*256/256, 84]
    h: np.ndarray          # float32 [1, hc, dim]
    qk: np.ndarray         # float32 [hc, dim]
    dim: int
    hc: int
    cols: int
    eps: float
    extra: dict = field(default_factory=dict)


def engram_step_case(seed: int = 1001, n_table_rows: int = 500_000, cols: int = 8,
                     dim: int = 4096, hc: int = 4, eps: float = 1e-6,
                     tokens: int = 1) -> EngramCase:
    """Engram-shaped step: 8 gathered Q2_K table rows (ids uniform in
    [0, 500000)), wkv [4096*(hc+1), 2048] with hc = 4, stream h [1, 4, 4096]
    ~ N(0,1), qk = f32 product of two bf16 weight vectors ~ 1 + 0.1 N(0,1)."""
    rng = rng_for(seed)
    table = q2k_blocks(rng, n_table_rows, 1)
    ids = rng.integers(0, n_table_rows, size=tokens * cols, dtype=np.int64)
    in_features = cols * Q2K_BLOCK_WEIGHTS
    wkv = q2k_blocks(rng, dim * (hc + 1), in_features // Q2K_BLOCK_WEIGHTS)
    h = rng.standard_normal(size=(tokens, hc, dim)).astype(np.float32)
    qw = f32_to_bf16_bits_torch((1.0 + 0.1 * rng.standard_normal(size=(hc, dim))).astype(np.float32))
    kw = f32_to_bf16_bits_torch((1.0 + 0.1 * rng.standard_normal(size=(hc, dim))).astype(np.float32))
    # The caller-side upload of the gate weights: the f32 product of the two
    # bf16-valued weight vectors (metrale engram_v41.rs, EngramV41::upload_qk).
    qf = (qw.astype(np.uint32) << 16).view(np.float32)
    kf = (kw.astype(np.uint32) << 16).view(np.float32)
    qk = (qf * kf).astype(np.float32)
    return EngramCase(table=table, ids=ids, wkv=wkv, h=h, qk=qk, dim=dim, hc=hc,
                      cols=cols, eps=eps)


def gate_case(seed: int, tokens: int, hc: int, dim: int, eps: float = 1e-6):
    """Stand-alone gate inputs: h [T, hc, dim], kv [T, (hc+1)*dim], qk [hc, dim]."""
    rng = rng_for(seed, tokens, hc, dim)
    h = rng.standard_normal(size=(tokens, hc, dim)).astype(np.float32)
    kv = rng.standard_normal(size=(tokens, (hc + 1) * dim)).astype(np.float32)
    qk = (1.0 + 0.1 * rng.standard_normal(size=(hc, dim))).astype(np.float32)
    return h, kv, qk, eps


def summation_order_case(n_rows: int, n_blocks: int, m: int):
    """Hand-built input whose f32 product depends on the order of the fp64
    sums (no randomness). Every row: scale nibble 1 and min nibble 0 in each
    sub-block, d = 1.0, dmin = 0, and quant 1 only at elements 0 and 128 of
    each super-block (qs[0] and qs[32] = 0x01), 0 elsewhere. Every token:
    x = 127 * v at element 256b + 128h for the (b, h, v) below, 0 elsewhere,
    so q8 block 8b + 4h holds one value +-127 with scale |v| and the half
    block (b, h) of the product is exactly 127 * v:
        (0, 0): 2^60   (1, 0): 1   (2, 0): -2^60   (3, 0): 2   (0, 1): 1.
    Returns (w uint8 [n_rows, n_blocks, 84], x bf16 bits [m, 256 * n_blocks]);
    n_blocks >= 4."""
    assert n_blocks >= 4
    w = np.zeros((n_rows, n_blocks, Q2K_BLOCK_BYTES), dtype=np.uint8)
    w[..., 0:16] = 0x01
    w[..., 16] = 0x01
    w[..., 48] = 0x01
    w[..., 80:82] = np.frombuffer(np.float16(1.0).tobytes(), np.uint8)
    x = np.zeros((m, Q2K_BLOCK_WEIGHTS * n_blocks), dtype=np.float32)
    for b, h, v in ((0, 0, 2.0 ** 60), (1, 0, 1.0), (2, 0, -2.0 ** 60), (3, 0, 2.0), (0, 1, 1.0)):
        x[:, 256 * b + 128 * h] = 127.0 * v
    return w, f32_to_bf16_bits_torch(x)
