"""CPU oracle for the Q2_K quantised decode path.

TEST INFRASTRUCTURE ONLY. Only the tests, the smoke check and the bench's CPU
baseline may import this module. The product path (the HIP library and its
Python binding) never calls it, and this module imports nothing from the
product package. It is plain, slow and written to be checked by eye against
the definitions below.

What it computes, and where each definition comes from (the pages are the
rustdoc source views of the metrale engine: ``engram_v41/apply.rs``,
``engram_v41.rs``, ``attn_v41/decode.rs`` and ``moe_v41/init.rs``):

* Q2_K super-block, 84 bytes per 256 weights: ``engram_v41.rs``,
  ``const ENGRAM_ROW_BYTES`` and the ``EngramLayerWeights::wkv_q2k`` doc ("as
  the GGUF ships it", 84 bytes against 512 in bf16). The pages give only the
  size; the byte layout is GGUF's Q2_K record (16 scale bytes whose low
  nibble is the sub-block scale and high nibble the sub-block min, 64 bytes
  of 2-bit quants, fp16 ``d``, fp16 ``dmin``). Element ``128h + 32j + l``
  takes bits ``2j..2j+1`` of ``qs[32h + l]`` and sub-block ``8h + 2j + (l>=16)``;
  its value is ``d*sc*q - dmin*m``.
* q8_1 activation rows: ``moe_v41/init.rs`` (``kquant_q8_1_rows_bytes``,
  the ``kquant_q8_1_rows_bf16`` kernel) and ``attn_v41/decode.rs``
  (``q_kv_projections``: one q8_1 quantisation shared by two Q2_K matrices).
  32-wide blocks, scale ``amax/127``, round to nearest.
* The Q2_K x q8_1 product (``kquant_mmvq_q2_k_w``, ``mmvq_q2k_pair_w``,
  ``kquant_mmvq_q2_k_experts_w*``, and the grouped ``wo_a`` step of
  ``attn_v41/decode.rs``): ``y[t, n] = sum_e W[n, e] * a[t, e]`` with
  ``W`` the dequantised weights and ``a = d8 * xq`` the dequantised
  activations, accumulated here in fp64.
* Row dequantisation to bf16 (``dequant_q2_k_to_bf16``,
  ``EngramV41::rows_from_q2k``), and the product of that bf16 expansion with
  bf16 activations (``engram_v41_wkv_q2k_gemv``).
* SwiGLU then q8_1 re-quantisation (``kquant_swiglu_q8_1_rows_bf16``).
* The engram n-gram hash (``EngramHasher::hash``): window of compressed
  token ids, rolling xor of wrapping products, Euclidean remainder by a
  prime per head, plus an offset per column.
* The engram gate (``engram_v41_gate``; module doc step 4 "normalised dot of
  stream against key, signed-sqrt sigmoid, h += gate * value"; ``qk`` is
  ``q_weight * k_weight``).

Readings taken where the pages are silent (each is listed in the design
notes): q8_1 rounds half away from zero after a correctly rounded f32
division and keeps an f32 scale plus per-16 integer sums; the dequantised
value is formed in f32 and rounded to bf16 to nearest-even; the gate
RMS-normalises both vectors with ``eps`` inside each root, divides the
weighted dot by ``sqrt(dim)``, and takes the keys of streams ``0..hc-1``
before the one shared value in each ``kv`` row. The gate formula is that
reading: parity unpinned by the pages' own numbers (they print none); it is
pinned by the closed forms in the oracle tests.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK_BYTES = 84          # engram_v41.rs: const ENGRAM_ROW_BYTES
BLOCK_WEIGHTS = 256
Q8_BLOCK = 32


# ----------------------------------------------------------------------------
# Scalar formats
# ----------------------------------------------------------------------------

def fp16_bits_to_f64(bits) -> np.ndarray:
    """IEEE binary16 decode from the bit fields (sign, 5-bit exponent with bias
    15, 10-bit fraction; exponent 0 is subnormal, 31 is inf/NaN)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = sign * (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = sign * (f / 1024.0) * 2.0 ** -14
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == 0, sub, np.where(e == 31, special, normal))


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bf16 is the top half of an f32: shift the 16 bits into place."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32)


def f32_to_bf16_bits_rne(x) -> np.ndarray:
    """Round f32 to bf16, to nearest with ties to even, returning bits.

    Keep the top 16 bits; round up when the dropped 16 bits exceed half, or
    equal half with an odd kept part. NaN keeps a quiet NaN pattern.
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    kept = u >> 16
    dropped = u & 0xFFFF
    up = (dropped > 0x8000) | ((dropped == 0x8000) & ((kept & 1) == 1))
    out = (kept + up.astype(np.uint64)) & 0xFFFF
    isnan = np.isnan(np.asarray(x, dtype=np.float32))
    out = np.where(isnan, (kept | 0x40), out)
    return out.astype(np.uint16)


def round_half_away(v32) -> np.ndarray:
    """Round an f32 value to the nearest integer, halves away from zero.

    |v| + 0.5 is exact in fp64 for any f32 v of magnitude below 2**52, so the
    floor sees the true value.
    """
    v = np.asarray(v32, dtype=np.float32).astype(np.float64)
    return np.sign(v) * np.floor(np.abs(v) + 0.5)


# ----------------------------------------------------------------------------
# Q2_K blocks (GGUF layout; size from engram_v41.rs ENGRAM_ROW_BYTES)
# ----------------------------------------------------------------------------

def q2k_fields(blocks: np.ndarray):
    """Split ``uint8 [..., 84]`` blocks into (sc, m, q, d, dmin).

    sc, m: int64 [..., 16] sub-block scale and min nibbles.
    q:     int64 [..., 256] the 2-bit quant of each element, element order.
    d, dmin: fp64 [...] super-block scales (fp16 bit patterns decoded).
    """
    blocks = np.asarray(blocks, dtype=np.uint8)
    assert blocks.shape[-1] == BLOCK_BYTES
    scales = blocks[..., 0:16].astype(np.int64)
    qs = blocks[..., 16:80].astype(np.int64)
    sc = scales & 0xF
    m = scales >> 4
    lead = blocks.shape[:-1]
    q = np.zeros(lead + (BLOCK_WEIGHTS,), dtype=np.int64)
    # element 128h + 32j + l takes bits 2j..2j+1 of qs[32h + l]
    for h in range(2):
        for j in range(4):
            for_l = qs[..., 32 * h: 32 * h + 32]
            q[..., 128 * h + 32 * j: 128 * h + 32 * j + 32] = (for_l >> (2 * j)) & 3
    d_bits = blocks[..., 80].astype(np.uint16) | (blocks[..., 81].astype(np.uint16) << 8)
    dmin_bits = blocks[..., 82].astype(np.uint16) | (blocks[..., 83].astype(np.uint16) << 8)
    return sc, m, q, fp16_bits_to_f64(d_bits), fp16_bits_to_f64(dmin_bits)


def subblock_of_element() -> np.ndarray:
    """Sub-block index of each element 128h + 32j + l: 8h + 2j + (l >= 16)."""
    e = np.arange(BLOCK_WEIGHTS)
    h, j, l = e // 128, (e % 128) // 32, e % 32
    return 8 * h + 2 * j + (l >= 16).astype(np.int64)


def q2k_dequant_f64(blocks: np.ndarray) -> np.ndarray:
    """Exact weight values d*sc*q - dmin*m in fp64, shape [..., 256].

    Each product has at most 17 significant bits, so both products and (for
    fp16 scales of ordinary range) their difference are exact in fp64.
    """
    sc, m, q, d, dmin = q2k_fields(blocks)
    sb = subblock_of_element()
    return (d[..., None] * sc[..., sb] * q) - (dmin[..., None] * m[..., sb])


def q2k_matrix_f64(w: np.ndarray) -> np.ndarray:
    """Dequantise a Q2_K matrix ``[n, k/256, 84]`` to fp64 ``[n, k]``."""
    n, nb = w.shape[0], w.shape[1]
    return q2k_dequant_f64(w).reshape(n, nb * BLOCK_WEIGHTS)


def q2k_dequant_bf16_bits(blocks: np.ndarray) -> np.ndarray:
    """``dequant_q2_k_to_bf16`` (engram_v41.rs, EngramV41::rows_from_q2k):
    the value formed in f32 (d*sc*q and dmin*m are exact in f32, the
    subtraction rounds once), then rounded to bf16 to nearest-even."""
    sc, m, q, d, dmin = q2k_fields(blocks)
    sb = subblock_of_element()
    d32 = d.astype(np.float32)[..., None]
    dmin32 = dmin.astype(np.float32)[..., None]
    a = d32 * (sc[..., sb] * q).astype(np.float32)
    b = dmin32 * m[..., sb].astype(np.float32)
    v = (a - b).astype(np.float32)
    return f32_to_bf16_bits_rne(v)


def dequant_rows_bf16_bits(table: np.ndarray, ids) -> np.ndarray:
    """Gather table rows by id, then dequantise each (one block per row).

    ``table``: uint8 [n_table_rows, 84] (or [n_table_rows, 1, 84]).
    ``ids``: int sequence, or None for rows 0..n-1 in order.
    Returns uint16 bf16 bits [n_rows, 256].
    """
    t = np.asarray(table, dtype=np.uint8).reshape(-1, BLOCK_BYTES)
    rows = t if ids is None else t[np.asarray(ids, dtype=np.int64)]
    return q2k_dequant_bf16_bits(rows)


# ----------------------------------------------------------------------------
# q8_1 activation rows
# ----------------------------------------------------------------------------

def q8_1_quantize(x_f32: np.ndarray):
    """q8_1 of rows ``[m, k]`` (exact f32 values, e.g. from bf16).

    Per 32-wide block: amax = max |x|, d = amax / 127 (f32, correctly rounded),
    xq = round(x / d) with the f32 quotient rounded half away from zero, and
    xq = 0 when amax = 0. Also returns the integer sum of each 16-wide half.

    Returns (xq int64 [m, k], d f32 [m, k/32], s int64 [m, k/16]).
    """
    x = np.asarray(x_f32, dtype=np.float32)
    m, k = x.shape
    assert k % Q8_BLOCK == 0
    xb = x.reshape(m, k // Q8_BLOCK, Q8_BLOCK)
    amax = np.max(np.abs(xb), axis=-1).astype(np.float32)
    d = (amax / np.float32(127.0)).astype(np.float32)
    safe = np.where(d > 0, d, np.float32(1.0)).astype(np.float32)
    quot = (xb / safe[..., None]).astype(np.float32)
    xq = np.clip(round_half_away(quot), -127, 127).astype(np.int64)
    xq = np.where((d > 0)[..., None], xq, 0)
    xq = xq.reshape(m, k)
    s = xq.reshape(m, k // 16, 16).sum(axis=-1)
    return xq, d, s


def q8_1_from_bf16_bits(x_bits: np.ndarray):
    """q8_1 of bf16 rows given as bit patterns."""
    return q8_1_quantize(bf16_bits_to_f32(x_bits))


def q8_1_dequant_f64(xq: np.ndarray, d: np.ndarray) -> np.ndarray:
    """a[t, e] = d[t, e // 32] * xq[t, e], exact in fp64."""
    m, k = xq.shape
    return d.astype(np.float64).repeat(Q8_BLOCK, axis=1) * xq.astype(np.float64)


# ----------------------------------------------------------------------------
# Q2_K x q8_1 products
# ----------------------------------------------------------------------------

def mmvq(w: np.ndarray, xq: np.ndarray, d8: np.ndarray) -> np.ndarray:
    """y[t, n] = sum_e W[n, e] * d8[t, e//32] * xq[t, e] in fp64 (dense route).

    ``w``: uint8 [n, k/256, 84]; ``xq``: int [m, k]; ``d8``: f32 [m, k/32].
    Returns fp64 [m, n].
    """
    wf = q2k_matrix_f64(w)
    a = q8_1_dequant_f64(xq, d8)
    return a @ wf.T


def block_dots(w: np.ndarray, xq: np.ndarray):
    """Integer sums per (token t, row n, q8 block c of the row):

    I = sum over the 32 elements e of block c of sc(e) * q(e) * xq(e)
    M = sum over the same elements of m(e) * xq(e)

    where sc(e), m(e) are the scale and min nibbles of e's 16-wide sub-block.
    Returns (I, M) int64 [m, n, k/32].
    """
    sc, mn, q, _, _ = q2k_fields(w)          # [n, nb, 16], [n, nb, 256]
    sb = subblock_of_element()
    n, nb = w.shape[0], w.shape[1]
    wsq = (sc[..., sb] * q).reshape(n, nb * BLOCK_WEIGHTS)     # [n, k]
    wm = mn[..., sb].reshape(n, nb * BLOCK_WEIGHTS)
    mt, k = xq.shape
    nq8 = k // Q8_BLOCK
    I = np.einsum("nce,tce->tnc", wsq.reshape(n, nq8, Q8_BLOCK),
                  xq.reshape(mt, nq8, Q8_BLOCK).astype(np.int64))
    M = np.einsum("nce,tce->tnc", wm.reshape(n, nq8, Q8_BLOCK),
                  xq.reshape(mt, nq8, Q8_BLOCK).astype(np.int64))
    return I, M


def mmvq_from_block_dots(w: np.ndarray, I: np.ndarray, M: np.ndarray, d8: np.ndarray):
    """The integer route: y[t, n] = sum_b sum_c d8[t, 8b+c] * (d_b * I - dmin_b * M),
    in fp64. Equal to ``mmvq`` up to fp64 rounding."""
    _, _, _, d, dmin = q2k_fields(w)         # [n, nb]
    n, nb = d.shape
    d_e = np.repeat(d, 8, axis=1)            # per q8 block of the row
    dmin_e = np.repeat(dmin, 8, axis=1)
    inner = d_e[None] * I.astype(np.float64) - dmin_e[None] * M.astype(np.float64)
    return np.einsum("tnc,tc->tn", inner, d8.astype(np.float64))


def mmvq_f32(w: np.ndarray, xq: np.ndarray, d8: np.ndarray) -> np.ndarray:
    """The f32 product in the library's fixed summation order, bit for bit.

    The pages fix no order for the fp64 sums of the product. The library fixes
    one, so that every kernel returns the same bits for the same inputs, and
    this is that order written out from the integer block sums of
    ``block_dots`` (the plain definition is ``mmvq``; the two agree to fp64
    rounding):

    * leaf (token t, row n, super-block b, half h; q8 blocks c = 8b+4h+j):
      fI = ((0 + d8_0*I_0) + d8_1*I_1) + d8_2*I_2) + d8_3*I_3, each product
      exact in fp64 (24 + 18 bits), fM likewise with M, and
      v = RN(d_b * fI) - RN(dmin_b * fM);
    * for each half h, the pairwise tree over b = 0 .. NBP-1 (NBP the row's
      block count rounded up to a power of two, leaves past the row +0):
      (b, b+1) first, then pairs of pairs, and so on;
    * y = f32(T_0 + T_1), the two halves added and rounded once to f32.

    numpy's fp64 operations are IEEE round-to-nearest and are not fused, so
    each step above is one rounding. Returns f32 [m, n].
    """
    I, M = block_dots(w, xq)
    return mmvq_f32_from_block_dots(w, I, M, d8)


def fixed_order_leaves(w: np.ndarray, I: np.ndarray, M: np.ndarray, d8: np.ndarray):
    """The leaf values of the fixed summation orders, fp64 [m, n, nb, 2]
    (token, row, super-block b, half h): fI and fM chained over the four q8
    blocks 8b+4h+j from +0, then RN(d_b * fI) - RN(dmin_b * fM)."""
    _, _, _, d, dmin = q2k_fields(w)                    # fp64 [n, nb]
    mt, n, nq = I.shape
    nb = nq // 8
    If = I.reshape(mt, n, nb, 2, 4).astype(np.float64)
    Mf = M.reshape(mt, n, nb, 2, 4).astype(np.float64)
    d8r = np.asarray(d8, dtype=np.float32).astype(np.float64).reshape(mt, 1, nb, 2, 4)
    fI = np.zeros((mt, n, nb, 2))
    fM = np.zeros((mt, n, nb, 2))
    for j in range(4):
        fI = fI + d8r[..., j] * If[..., j]
        fM = fM + d8r[..., j] * Mf[..., j]
    return d[None, :, :, None] * fI - dmin[None, :, :, None] * fM


def mmvq_f32_from_block_dots(w: np.ndarray, I: np.ndarray, M: np.ndarray, d8: np.ndarray):
    """``mmvq_f32`` from integer block sums already formed by ``block_dots``
    (int [m, n, k/32] each)."""
    v = fixed_order_leaves(w, I, M, d8)
    mt, n, nb, _ = v.shape
    nbp = 1
    while nbp < nb:
        nbp *= 2
    leaves = np.zeros((mt, n, nbp, 2))
    leaves[:, :, :nb, :] = v
    while leaves.shape[2] > 1:
        leaves = leaves[:, :, 0::2, :] + leaves[:, :, 1::2, :]
    return (leaves[:, :, 0, 0] + leaves[:, :, 0, 1]).astype(np.float32)


def mmq_f32(w: np.ndarray, xq: np.ndarray, d8: np.ndarray) -> np.ndarray:
    """The f32 product past 8 tokens (``q2k_mmq``) in its fixed order, bit for
    bit: the leaves of ``mmvq_f32`` added to one running fp64 sum from +0 in
    row order, (b, h) = (0, 0), (0, 1), (1, 0), ..., (nb-1, 1) (no padding),
    then y = f32(T). The order differs from ``mmvq_f32`` only in how the
    leaves are added (a running sum instead of the pairwise tree per half),
    which a kernel that walks the row block by block for many tokens at once
    can keep in one register pair per output. Returns f32 [m, n]."""
    I, M = block_dots(w, xq)
    return mmq_f32_from_block_dots(w, I, M, d8)


def mmq_f32_from_block_dots(w: np.ndarray, I: np.ndarray, M: np.ndarray, d8: np.ndarray):
    """``mmq_f32`` from integer block sums already formed by ``block_dots``."""
    v = fixed_order_leaves(w, I, M, d8)
    mt, n, nb, _ = v.shape
    t = np.zeros((mt, n))
    for b in range(nb):
        for h in range(2):
            t = t + v[:, :, b, h]
    return t.astype(np.float32)


def mmvq_pair(wa, wb, xq, d8):
    """``mmvq_q2k_pair_w`` (attn_v41/decode.rs, q_kv_projections): two
    matrices against the same q8_1 rows."""
    return mmvq(wa, xq, d8), mmvq(wb, xq, d8)


def mmvq_experts(matrices_by_id, xq, d8, x_per_id: bool):
    """Expert-batch product (``kquant_mmvq_q2_k_experts_w*``, moe_v41/init.rs):
    ``matrices_by_id[i]`` is the Q2_K matrix of the i-th selected id; the input
    is shared (``x_per_id`` False) or the i-th group of ``m`` rows.
    Returns fp64 [n_ids, m, n] in id-list order."""
    outs = []
    m_per = xq.shape[0] if not x_per_id else xq.shape[0] // len(matrices_by_id)
    for i, w in enumerate(matrices_by_id):
        if x_per_id:
            sl = slice(i * m_per, (i + 1) * m_per)
            outs.append(mmvq(w, xq[sl], d8[sl]))
        else:
            outs.append(mmvq(w, xq, d8))
    return np.stack(outs)


def mmvq_grouped(w: np.ndarray, xq: np.ndarray, d8: np.ndarray, groups: int) -> np.ndarray:
    """Grouped-input product, the Q2_K route of the attention output
    projection ``wo_a`` (attn_v41/decode.rs, decode body: output column
    ``g*o_rank + r`` is the dot of row ``g*o_rank + r`` of ``wo_a`` with the
    g-th column slice ``o_g`` of the attention output).

    ``w``: uint8 [groups*R, k/256, 84]; ``xq``: int [m, groups*k] and ``d8``:
    f32 [m, groups*k/32] (the q8_1 rows of the whole attention output).
    Returns fp64 [m, groups*R]: y[t, g*R + r] = sum_e W[g*R + r, e] *
    a[t, g*k + e], ``a = d8 * xq``."""
    n_total, nb = w.shape[0], w.shape[1]
    if n_total % groups:
        raise ValueError("rows must split evenly into groups")
    rows, k = n_total // groups, 256 * nb
    if xq.shape[1] != groups * k:
        raise ValueError("activation width must be groups * k")
    wf = q2k_matrix_f64(w)
    a = q8_1_dequant_f64(xq, d8)
    y = np.empty((a.shape[0], n_total), dtype=np.float64)
    for g in range(groups):
        y[:, g * rows:(g + 1) * rows] = a[:, g * k:(g + 1) * k] @ wf[g * rows:(g + 1) * rows].T
    return y


def gemv_bf16(w: np.ndarray, x_bits: np.ndarray) -> np.ndarray:
    """Q2_K weights times bf16 activations (``engram_v41_wkv_q2k_gemv``,
    engram_v41/apply.rs; engram_v41.rs ``EngramLayerWeights::wkv_q2k``: the
    bf16 GEMV over the bf16 expansion of the blocks).

    ``w``: uint8 [n, k/256, 84]; ``x_bits``: uint16 bf16 [m, k]. Each weight
    is expanded to bf16 exactly as the row dequantisation does; the dot
    product of the expansion with x is formed in fp64 (every bf16 x bf16
    product is exact) and rounded to f32. Returns f32 [m, n]."""
    n, nb = w.shape[0], w.shape[1]
    wf = bf16_bits_to_f32(q2k_dequant_bf16_bits(w).reshape(n, nb * 256)).astype(np.float64)
    xf = bf16_bits_to_f32(x_bits).astype(np.float64)
    return (xf @ wf.T).astype(np.float32)


# ----------------------------------------------------------------------------
# Engram n-gram hash (integers only)
# ----------------------------------------------------------------------------

_U64 = (1 << 64) - 1


def _as_i64(v: int) -> int:
    """Two's-complement reading of the low 64 bits of a Python int."""
    v &= _U64
    return v - (1 << 64) if v >> 63 else v


def engram_hash(token_map, multipliers, primes, offsets, pad_id: int, n_heads: int,
                cache, input_ids, start_pos: int):
    """The engram n-gram hash of one sequence (engram_v41.rs,
    ``EngramHasher::hash``), in plain Python integers with explicit 64-bit
    wrap-around.

    ``token_map``: compressed id per vocabulary id (-1 = unmapped);
    ``multipliers[l][i]`` (i < max_ngram); ``primes[l][i-1][h]``;
    ``offsets[l][(i-1)*n_heads + h]``; ``cache``: compressed ids of the
    positions already seen (at least ``start_pos + len(input_ids)`` long; its
    entries from ``start_pos`` on are overwritten here).

    Steps, for each new token s at position pos = start_pos + s:
      1. cache[pos] = token_map[id] (an id outside the map is an error);
      2. window tokens tok[i] = cache[pos - i] for i < max_ngram, except that
         from the first i with pos < i or cache[pos - i] == -1 on, every
         tok[i] is pad_id;
      3. per hashed layer l: rolling = tok[0]*mult[l][0], then for i >= 1
         rolling ^= tok[i]*mult[l][i] (64-bit wrapping products) and, for each
         head h, row id = (rolling mod primes[l][i-1][h], in [0, prime)) +
         offsets[l][(i-1)*n_heads + h].
    Returns (ids [seqlen][n_layers][(max_ngram-1)*n_heads] as Python ints,
    the updated cache)."""
    cache = list(cache)
    n_layers = len(multipliers)
    ng = len(multipliers[0])
    cols = (ng - 1) * n_heads
    for s, tid in enumerate(input_ids):
        if not 0 <= tid < len(token_map):
            raise ValueError(f"token {tid} outside token_map")
        cache[start_pos + s] = token_map[tid]
    out = []
    for s in range(len(input_ids)):
        pos = start_pos + s
        tok = []
        blocked = False
        for i in range(ng):
            src = cache[max(pos - i, 0)]
            blocked = blocked or pos < i or src == -1
            tok.append(pad_id if blocked else src)
        per_layer = []
        for l in range(n_layers):
            row = [0] * cols
            rolling = _as_i64(tok[0] * multipliers[l][0])
            for i in range(1, ng):
                rolling = _as_i64(rolling ^ _as_i64(tok[i] * multipliers[l][i]))
                for h in range(n_heads):
                    p = primes[l][i - 1][h]
                    row[(i - 1) * n_heads + h] = _as_i64(rolling % p + offsets[l][(i - 1) * n_heads + h])
            per_layer.append(row)
        out.append(per_layer)
    return out, cache


# ----------------------------------------------------------------------------
# SwiGLU and the engram gate
# ----------------------------------------------------------------------------

def swiglu_bf16_bits(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """bf16 SwiGLU of the gate/up outputs (``kquant_swiglu_q8_1_rows_bf16``):
    silu(g) * u = g / (1 + exp(-g)) * u in fp64, rounded to f32 and then to
    bf16, nearest-even both times."""
    g64 = np.asarray(g, dtype=np.float64)
    u64 = np.asarray(u, dtype=np.float64)
    h = g64 / (1.0 + np.exp(-g64)) * u64
    return f32_to_bf16_bits_rne(h.astype(np.float32))


def engram_gate(h: np.ndarray, kv: np.ndarray, qk: np.ndarray, eps: float) -> np.ndarray:
    """Engram gate (engram_v41.rs module doc, step 4; ``engram_v41_gate`` in
    engram_v41/apply.rs with arguments streams, kv, qk, dim, hc, eps).

    For token t and stream j, with key k_j = kv[t, j*dim:(j+1)*dim] and value
    v = kv[t, hc*dim:(hc+1)*dim]:
        rms(x) = sqrt(mean(x^2) + eps)
        s = sum_i qk[j, i] * h[t, j, i] * k_j[i] / (rms(h[t, j]) * rms(k_j) * sqrt(dim))
        g = 1 / (1 + exp(-sign(s) * sqrt(|s|)))
        h[t, j, :] += g * v
    Returns the updated stream in fp64; the input is not modified.
    """
    h = np.asarray(h, dtype=np.float64)
    kv = np.asarray(kv, dtype=np.float64)
    qk = np.asarray(qk, dtype=np.float64)
    T, hc, dim = h.shape
    out = h.copy()
    for t in range(T):
        v = kv[t, hc * dim:(hc + 1) * dim]
        for j in range(hc):
            x = h[t, j]
            k = kv[t, j * dim:(j + 1) * dim]
            rx = math.sqrt(float(np.mean(x * x)) + eps)
            rk = math.sqrt(float(np.mean(k * k)) + eps)
            s = float(np.sum(qk[j] * x * k)) / (rx * rk * math.sqrt(dim))
            sg = math.copysign(math.sqrt(abs(s)), s) if s != 0.0 else 0.0
            g = 1.0 / (1.0 + math.exp(-sg))
            out[t, j] = x + g * v
    return out
