"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars: q8_1 bytes, integer block sums and dequantised bf16 rows bit-exact;
f32 products bit for bit the oracle's evaluation of the library's fixed
summation order (orc.mmvq_f32) and within |gpu - ref| <= 1e-4 + 2e-3 |ref| of
the fp64 definition (orc.mmvq, the integer route on every row, the dense
route on all rows of small matrices and sampled rows of large ones); the
gated stream within the same tolerance; the bf16 SwiGLU value within one
bf16 ulp (the GPU forms it in f32, the oracle in fp64), with its q8_1 bytes
bit-exact from the GPU's own h.
"""

import dataclasses

import numpy as np
import pytest
import torch

import q2_quantized_decode_amd as q2
from oracle import q2k_oracle as orc
from q2_quantized_decode_amd import synthetic as syn

pytestmark = pytest.mark.gpu

ATOL, RTOL = 1e-4, 2e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    assert torch.cuda.is_available(), "GPU tests need a HIP device"
    q2.lib()
    torch.cuda.set_device(0)
    yield
    torch.cuda.synchronize()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    return syn.bf16_bits_to_tensor(bits).cuda()


def split_q8(buf: np.ndarray, m: int, k: int):
    """Unpack the library's q8_1 rows (layout stated in the header)."""
    rb = k * 5 // 4
    rows = buf[: m * rb].reshape(m, rb)
    xq = rows[:, :k].view(np.int8).astype(np.int64)
    d = rows[:, k:k + k // 8].copy().view(np.float32)
    s = rows[:, k + k // 8:k + k // 4].copy().view(np.int16).astype(np.int64)
    return xq, d, s


def assert_q8_equal(buf_dev: torch.Tensor, x_bits: np.ndarray):
    m, k = x_bits.shape
    xq, d, s = split_q8(buf_dev.cpu().numpy(), m, k)
    oq, od, os_ = orc.q8_1_from_bf16_bits(x_bits)
    assert np.array_equal(d.view(np.uint32), od.view(np.uint32)), "q8_1 scales differ"
    assert np.array_equal(xq, oq), "q8_1 quants differ"
    assert np.array_equal(s, os_), "q8_1 half sums differ"
    return oq, od


def bf16_ulp_distance(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Distance in bf16 steps (+0 and -0 are the same point)."""
    def key(bits):
        v = bits.astype(np.int64)
        return np.where(v & 0x8000, -(v & 0x7FFF), v)
    return np.abs(key(a) - key(b))


def assert_close(got, ref, what=""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    excess = np.abs(got - ref) - (ATOL + RTOL * np.abs(ref))
    i = int(np.argmax(excess))
    assert excess.flat[i] <= 0, (f"{what}: element {np.unravel_index(i, got.shape)} "
                                 f"gpu {got.flat[i]!r} ref {ref.flat[i]!r}")


# Rows per oracle chunk of a product check, and the largest n * k checked
# through the dense fp64 route on every row (larger ones: sampled rows there,
# every row through the integer route and the fixed order).
CHUNK_ROWS = 4096
DENSE_ALL_MAX = 1 << 24


def assert_bits(got, ref32, what=""):
    """f32 arrays equal bit for bit."""
    g = np.ascontiguousarray(np.asarray(got, dtype=np.float32))
    r = np.ascontiguousarray(np.asarray(ref32, dtype=np.float32))
    assert g.shape == r.shape, (g.shape, r.shape)
    bad = np.flatnonzero(g.view(np.uint32) != r.view(np.uint32))
    assert bad.size == 0, (f"{what}: {bad.size} of {g.size} outputs differ from the fixed-order "
                           f"oracle; first {np.unravel_index(bad[0], g.shape)}: gpu {g.flat[bad[0]]!r} "
                           f"oracle {r.flat[bad[0]]!r}")


def assert_product(got, w, oq, od, what="", dense_rows=None, order="tree"):
    """One matrix's product y [m, n] against the oracle: bit for bit the fixed
    summation order (``order``: "tree", the one-to-eight-token products'
    pairwise tree, or "running", q2k_mmq's running sum past 8 tokens) and
    within tolerance of the integer route on every row (both from one
    block_dots per CHUNK_ROWS rows), and within tolerance of the dense fp64
    definition on every row (small matrices) or on ``dense_rows``."""
    got = np.asarray(got)
    n = w.shape[0]
    bits = {"tree": orc.mmvq_f32_from_block_dots, "running": orc.mmq_f32_from_block_dots}[order]
    for r0 in range(0, n, CHUNK_ROWS):
        wc = w[r0:r0 + CHUNK_ROWS]
        I, M = orc.block_dots(wc, oq)
        gc = got[:, r0:r0 + CHUNK_ROWS]
        assert_bits(gc, bits(wc, I, M, od), f"{what} rows {r0}..")
        assert_close(gc, orc.mmvq_from_block_dots(wc, I, M, od), f"{what} rows {r0}.. (integer route)")
    if dense_rows is None and n * w.shape[1] * 256 > DENSE_ALL_MAX:
        dense_rows = _sample_rows(n, n + w.shape[1])
    if dense_rows is None:
        assert_close(got, orc.mmvq(w, oq, od), what)
    else:
        assert_close(got[:, dense_rows], orc.mmvq(w[dense_rows], oq, od), f"{what} (dense, sampled)")


def assert_pair(ya, yb, wa, wb, oq, od, what=""):
    assert_product(ya, wa, oq, od, what + " a")
    assert_product(yb, wb, oq, od, what + " b")


def assert_experts(got, mats, oq, od, x_per_id, what=""):
    """got [n_ids, m, n]: id i against mats[i], shared input or its own rows."""
    m_per = oq.shape[0] // len(mats) if x_per_id else oq.shape[0]
    for i, w in enumerate(mats):
        sl = slice(i * m_per, (i + 1) * m_per) if x_per_id else slice(0, m_per)
        assert_product(got[i], w, oq[sl], od[sl], f"{what} id #{i}")


def assert_grouped(got, w, oq, od, groups, what=""):
    """got [m, groups * R]: group g's rows against the g-th input slice."""
    rows = w.shape[0] // groups
    k = w.shape[1] * 256
    for g in range(groups):
        assert_product(got[:, g * rows:(g + 1) * rows], w[g * rows:(g + 1) * rows],
                       oq[:, g * k:(g + 1) * k], od[:, g * k // 32:(g + 1) * k // 32], f"{what} group {g}")


# ----------------------------------------------------------------- q8_1 -----

@pytest.mark.parametrize("m,k,seed,outliers", [
    (1, 1024, 1000, 0.0), (8, 7168, 1004, 0.05), (3, 256, 5, 0.0), (5, 4096, 6, 0.2),
    (64, 2048, 7, 0.05)])
def test_q8_1_rows_bit_exact(m, k, seed, outliers):
    x = syn.bf16_normal(syn.rng_for(seed, m, k), (m, k), outlier_frac=outliers)
    assert_q8_equal(q2.q8_1_rows(bf16_dev(x)), x)


def test_q8_1_rows_strided_and_special_blocks():
    k = 512
    rng = syn.rng_for(77)
    x = syn.bf16_normal(rng, (4, k)).astype(np.uint16)
    f = orc.bf16_bits_to_f32(x).copy()
    f[0, 0:32] = 0.0                                 # all-zero block
    f[1, 32:64] = 0.0
    f[1, 40] = -3.0                                  # single nonzero
    f[2, 64:96] = np.float32(1.0)                    # ties: elements at amax / 2
    f[2, 65] = 0.5
    f[2, 66] = -0.5
    f[3, 96:128] = np.arange(-16, 16, dtype=np.float32) * 4
    f[3, 127] = 127.0                                # d = 1
    x = syn.f32_to_bf16_bits_torch(f)
    big = np.zeros((4, k + 64), dtype=np.uint16)     # rows 576 apart (stride % 8 == 0)
    big[:, :k] = x
    xt = bf16_dev(big)[:, :k]
    assert xt.stride(0) == k + 64
    assert_q8_equal(q2.q8_1_rows(xt), x)


def test_q8_1_rows_tiny_blocks_keep_subnormal_scales():
    # amax at the bottom of the bf16 normal range: d = amax / 127 is subnormal in f32
    k = 256
    f = np.zeros((1, k), dtype=np.float32)
    f[0, :32] = np.float32(2.0 ** -126) * np.arange(1, 33, dtype=np.float32) / 32
    f[0, 32:64] = np.float32(2.0 ** -120)
    x = syn.f32_to_bf16_bits_torch(f)
    assert_q8_equal(q2.q8_1_rows(bf16_dev(x)), x)


def _near_half_blocks():
    """Blocks [A, x_1..x_31] with every bf16 x in [A/2^20, A] (random signs),
    for all 128 bf16 mantissas of A at exponents 0, -60, -120 and -125 (the
    last gives a subnormal d = A/127): every quotient x/d that bf16 inputs can
    produce near a block maximum, exact ties (x = A/2) included."""
    rng = syn.rng_for(7777)
    blocks = []
    for ea in (0, -60, -120, -125):
        for ma in range(128):
            a_bits = ((ea + 127) << 7) | ma
            xs = []
            for e in range(ea - 20, ea + 1):
                if e + 127 <= 0:
                    continue
                xs.append(((e + 127) << 7) | np.arange(128))
            xs = np.concatenate(xs)
            xs = xs[xs <= a_bits]
            xs = xs | (rng.integers(0, 2, size=xs.size) << 15)
            n_blk = -(-xs.size // 31)
            blk = np.zeros((n_blk, 32), dtype=np.int64)
            blk[:, 0] = a_bits
            flat = np.zeros(n_blk * 31, dtype=np.int64)
            flat[:xs.size] = xs
            blk[:, 1:] = flat.reshape(n_blk, 31)
            blocks.append(blk)
    allb = np.concatenate(blocks)
    rows = -(-allb.shape[0] // 64)
    out = np.zeros((rows * 64, 32), dtype=np.int64)
    out[:allb.shape[0]] = allb
    return out.reshape(rows, 64 * 32).astype(np.uint16)


def test_q8_1_rows_near_half_quotients():
    """The quantisers divide once per block and take a product per value
    where that provably rounds alike: bit-exact against the oracle's
    per-value division on every quotient bf16 inputs give near a block's
    maximum, and the fused product's q8_1 row equals q8_1_rows on them."""
    x = _near_half_blocks()
    xq = q2.q8_1_rows(bf16_dev(x))
    assert_q8_equal(xq, x)
    # the fused product (one launch: [8192, 2048] has enough row steps)
    n, k = 8192, x.shape[1]
    w = dev(syn.q2k_blocks(syn.rng_for(7778), n, k // 256).reshape(-1))
    rb = q2.q8_1_rows_bytes(1, k)
    xd = bf16_dev(x)
    for r in range(x.shape[0]):
        _, xq_f = q2.q8_1_q2k_mmvq(w, xd[r:r + 1], n, k)
        assert torch.equal(xq_f[:rb], xq[r * rb:(r + 1) * rb]), f"row {r}"


# ---------------------------------------------------------------- mmvq ------

SHAPES = [
    (256, 1024, 1), (1, 256, 1), (3, 256, 8), (37, 512, 2), (1000, 2048, 1), (333, 4096, 3),
    (130, 7168, 1), (130, 7168, 8), (77, 1792, 5), (10, 8448, 1), (9, 9216, 4), (257, 1024, 7),
    (64, 2560, 6),
]


@pytest.mark.parametrize("n,k,m", SHAPES)
def test_mmvq_and_block_dots(n, k, m):
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=n * 31 + k + m)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    y = q2.q2k_mmvq(w, xq, n, k, m)
    dots = q2.q2k_block_dots(w, xq, n, k, m)
    torch.cuda.synchronize()
    I, M = orc.block_dots(case.w, oq)
    got = dots.cpu().numpy().astype(np.int64)
    assert np.array_equal(got[..., 0], I), "I sums differ"
    assert np.array_equal(got[..., 1], M), "M sums differ"
    assert_product(y.cpu().numpy(), case.w, oq, od, f"mmvq n={n} k={k} m={m}")


def test_mmvq_single_gemv_workload():
    """256 x 1024 (4 super-blocks) Q2_K against one bf16 token."""
    case = syn.single_gemv_case()
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    y = q2.q2k_mmvq(dev(case.w.reshape(-1)), xq, 256, 1024, 1)
    assert_product(y.cpu().numpy(), case.w, oq, od, "single gemv")


def test_mmvq_exact_closed_form():
    # W = 3 (q = 3, sc = 1, m = 0, d = 1); x = 127 everywhere: d8 = 1, y = 3*127*k exactly
    n, k = 96, 2048
    w = np.zeros((n, k // 256, 84), dtype=np.uint8)
    w[..., 0:16] = 0x01
    w[..., 16:80] = 0xFF
    w[..., 81] = 0x3C
    x = syn.f32_to_bf16_bits_torch(np.full((2, k), 127.0, np.float32))
    y = q2.q2k_mmvq(dev(w.reshape(-1)), q2.q8_1_rows(bf16_dev(x)), n, k, 2)
    assert np.all(y.cpu().numpy() == 3 * 127 * k)


def test_mmvq_deterministic_and_stride_independent():
    case = syn.single_gemv_case(n=2048, k=4096, m=4, seed=42)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    a = q2.q2k_mmvq(w, xq, 2048, 4096, 4).cpu().numpy()
    b = q2.q2k_mmvq(w, xq, 2048, 4096, 4).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
    # the first 1000 rows alone give the same bytes as inside the bigger launch
    c = q2.q2k_mmvq(w[: 1000 * 16 * 84], xq, 1000, 4096, 4).cpu().numpy()
    assert np.array_equal(c.view(np.uint32), a[:, :1000].view(np.uint32))


# ------------------------------------------------- fixed summation order ---

MC, PD, AUTO = q2.KERNEL_MATRIX_CORES, q2.KERNEL_PACKED_DOTS, q2.KERNEL_AUTO


class kernel_choice:
    """with kernel_choice(c): products run with q2k_set_product_kernel(c)."""

    def __init__(self, choice):
        self.choice = choice

    def __enter__(self):
        self.prev = q2.q2k_set_product_kernel(self.choice)

    def __exit__(self, *exc):
        q2.q2k_set_product_kernel(self.prev)


# (rows, blocks per row, tokens, choice, kernel the product takes)
HAND_CASES = [
    (16384, 4, 1, AUTO, PD),      # run kernel, 8 rows per row step
    (4096, 28, 1, AUTO, PD),      # run kernel, one row per step, idle lanes
    (37, 4, 1, AUTO, PD),         # one-step kernel
    (37, 5, 2, AUTO, PD),         # one-step kernel, tokens split, padded tree
    (8197, 4, 2, MC, MC), (8197, 4, 2, PD, PD),
    (8197, 8, 5, MC, MC), (4099, 16, 3, MC, MC), (4099, 16, 3, PD, PD),
    (8197, 28, 8, MC, MC), (8197, 28, 8, PD, PD),
    (64, 36, 1, AUTO, PD), (64, 36, 3, AUTO, PD),   # wide kernel (k > 8192)
]


@pytest.mark.parametrize("n,nb,m,choice,kernel", HAND_CASES)
def test_fixed_order_hand_case_every_kernel(n, nb, m, choice, kernel):
    """The hand-built input of synthetic.summation_order_case, whose f32
    result depends on the order of the fp64 sums (the oracle's derivation:
    127 where the exact sum is 508), gives exactly 127 on every kernel:
    every row and token, through q2k_mmvq, the pair form and, for one token,
    the fused quantisation."""
    k = 256 * nb
    w_np, x = syn.summation_order_case(n, nb, m)
    w = dev(w_np.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(x))
    assert_q8_equal(xq, x)
    with kernel_choice(choice):
        assert q2.q2k_product_kernel(n, k, m) == kernel
        y = q2.q2k_mmvq(w, xq, n, k, m).cpu().numpy()
        ya, yb = q2.q2k_mmvq_pair(w, n, w[: 5 * nb * 84], 5, xq, k, m)
        outs = [y, ya.cpu().numpy(), yb.cpu().numpy()]
        if m == 1:
            outs.append(q2.q8_1_q2k_mmvq(w, bf16_dev(x), n, k)[0].cpu().numpy())
    for o in outs:
        assert np.all(o == 127.0), np.unique(o)


def test_fixed_order_hand_case_mmq_grouped_experts():
    """The same input through q2k_mmq (20 tokens: the tile kernel's running
    sum gives 254, the oracle's derivation, whatever the kernel choice; 16
    and 8 tokens: groups of 8 on the q2k_mmvq kernels, the tree's 127), the
    grouped form and the expert batch."""
    nb, k = 4, 1024
    w_np, x = syn.summation_order_case(300, nb, 20)
    w = dev(w_np.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(x))
    for choice in (MC, PD):
        with kernel_choice(choice):
            assert np.all(q2.q2k_mmq(w, xq, 300, k, 20).cpu().numpy() == 254.0)
            assert np.all(q2.q2k_mmq(w, xq, 300, k, 16).cpu().numpy() == 127.0)
            assert np.all(q2.q2k_mmq(w, xq, 300, k, 8).cpu().numpy() == 127.0)
    _, x2 = syn.summation_order_case(1, nb, 3)
    xg = np.concatenate([x2, x2], axis=1)                     # two groups of 1024
    yg = q2.q2k_mmvq_grouped(w[: 2 * 150 * nb * 84], q2.q8_1_rows(bf16_dev(xg)), 2, 150, k, 3)
    assert np.all(yg.cpu().numpy() == 127.0)
    ids = dev(np.array([1, 0, 1], dtype=np.int32))
    ye = q2.q2k_mmvq_experts([w], 150 * nb * 84, 2, ids, q2.q8_1_rows(bf16_dev(x2)), False, 150, k, 3)
    assert np.all(ye.cpu().numpy() == 127.0)


@pytest.mark.parametrize("choice", [MC, PD])
def test_block_dots_of_the_kernel_taken(choice):
    """q2k_block_dots returns the integer sums of the kernel the product
    takes: on the matrix cores the v_mfma_i32_16x16x64_i8 outputs (I and M),
    else the packed-dot sums; all rows of [8197, 1024] at m = 5, bit-exact."""
    n, k, m = 8197, 1024, 5
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=7300)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, _ = assert_q8_equal(xq, case.x_bits)
    with kernel_choice(choice):
        assert q2.q2k_product_kernel(n, k, m) == choice
        dots = q2.q2k_block_dots(w, xq, n, k, m).cpu().numpy().astype(np.int64)
    I, M = orc.block_dots(case.w, oq)
    assert np.array_equal(dots[..., 0], I), "I sums differ"
    assert np.array_equal(dots[..., 1], M), "M sums differ"


def test_block_dots_large_verify_matrix_cores(large):
    """The [32768, 7168] matrix at m = 8 (the product's automatic choice is
    the matrix cores): their integer sums on sampled rows, bit-exact."""
    case, w = large
    m = 8
    assert q2.q2k_product_kernel(case.n, case.k, m) == MC
    xq = q2.q8_1_rows(bf16_dev(case.x_bits[:m]))
    oq, _ = assert_q8_equal(xq, case.x_bits[:m])
    dots = q2.q2k_block_dots(w, xq, case.n, case.k, m)
    rows = _sample_rows(case.n, 91, extra=256)
    got = dots[:, torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.int64)
    del dots
    I, M = orc.block_dots(case.w[rows], oq)
    assert np.array_equal(got[..., 0], I), "I sums differ"
    assert np.array_equal(got[..., 1], M), "M sums differ"


@pytest.mark.parametrize("m", [1, 4, 8])
def test_every_kernel_choice_same_bits_attention_pair(m):
    """The attention pair (wq_a [1024, 4096], wkv [512, 4096]) under every
    product kernel choice: identical bits."""
    pc = syn.attention_pair_case(m)
    wa, wb = dev(pc.wa.reshape(-1)), dev(pc.wb.reshape(-1))
    x = bf16_dev(pc.x_bits)
    outs = []
    for choice in (AUTO, MC, PD):
        with kernel_choice(choice):
            ya, yb, _ = q2.q8_1_q2k_mmvq_pair(wa, pc.na, wb, pc.nb, x, pc.k)
            outs.append(torch.cat([ya.reshape(-1), yb.reshape(-1)]).cpu().numpy())
    for o in outs[1:]:
        assert_bits(o, outs[0], f"attention pair m={m}")


def test_every_kernel_choice_same_bits_large_verify(large):
    """[32768, 7168] at m = 8: the matrix cores (automatic) and the packed
    dots (tokens split over waves) return identical bits."""
    case, w = large
    xq = q2.q8_1_rows(bf16_dev(case.x_bits[:8]))
    outs = []
    for choice in (AUTO, PD):
        with kernel_choice(choice):
            outs.append(q2.q2k_mmvq(w, xq, case.n, case.k, 8).cpu().numpy())
    assert_bits(outs[1], outs[0], "large verify m=8: packed dots vs matrix cores")


# ------------------------------------------------- matrix-core path ---------

@pytest.fixture
def matrix_cores():
    """Runs the test with the matrix-core kernel wherever it applies (the
    automatic choice takes it only where its cost model says it is faster)."""
    prev = q2.q2k_set_product_kernel(q2.KERNEL_MATRIX_CORES)
    yield
    q2.q2k_set_product_kernel(prev)


@pytest.fixture
def packed_dots():
    prev = q2.q2k_set_product_kernel(q2.KERNEL_PACKED_DOTS)
    yield
    q2.q2k_set_product_kernel(prev)

# 2..8 tokens against matrices of at least 64 workgroups of 128 rows (8192
# rows) with 4, 8, 16 or 28 super-blocks per row run on the matrix cores.

MFMA_ROWS = 8192 + 5     # 65 workgroups, the last tile ragged


def _sample_rows(n, seed, extra=256):
    """Both ends, every tile boundary of one workgroup, and random rows."""
    rows = [np.arange(0, 160), np.arange(n - 160, n), syn.rng_for(seed).choice(n, extra, replace=False)]
    return np.unique(np.concatenate(rows))


@pytest.mark.parametrize("k,m", [(1024, 2), (1024, 8), (2048, 3), (4096, 5), (4096, 8), (7168, 4)])
def test_mfma_mmvq(k, m, matrix_cores):
    n = MFMA_ROWS
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=7000 + k + m)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    y = q2.q2k_mmvq(w, xq, n, k, m).cpu().numpy()
    assert_product(y, case.w, oq, od, f"mfma n={n} k={k} m={m}")
    again = q2.q2k_mmvq(w, xq, n, k, m).cpu().numpy()
    assert np.array_equal(again.view(np.uint32), y.view(np.uint32)), "not deterministic"


def _constant_blocks(n, k, scale_byte, qs_byte, d_bits, dmin_bits):
    w = np.zeros((n, k // 256, 84), dtype=np.uint8)
    w[..., 0:16] = scale_byte
    w[..., 16:80] = qs_byte
    w[..., 80:82] = np.frombuffer(np.uint16(d_bits).tobytes(), np.uint8)
    w[..., 82:84] = np.frombuffer(np.uint16(dmin_bits).tobytes(), np.uint8)
    return w


@pytest.mark.parametrize("k", [1024, 7168])
def test_mfma_closed_forms(k, matrix_cores):
    """x = 127 everywhere (d8 = 1, every half sum 16*127). I term: q = 3,
    sc = 1, d = 1, m = 0 gives 3*127*k. M term: sc = 0, m = 5, dmin = 1
    gives -5*127*k."""
    n, m = MFMA_ROWS, 6
    x = syn.f32_to_bf16_bits_torch(np.full((m, k), 127.0, np.float32))
    xq = q2.q8_1_rows(bf16_dev(x))
    w_i = _constant_blocks(n, k, 0x01, 0xFF, 0x3C00, 0x0000)
    y = q2.q2k_mmvq(dev(w_i.reshape(-1)), xq, n, k, m).cpu().numpy()
    assert np.all(y == 3 * 127 * k)
    w_m = _constant_blocks(n, k, 0x50, 0xFF, 0x0000, 0x3C00)
    y = q2.q2k_mmvq(dev(w_m.reshape(-1)), xq, n, k, m).cpu().numpy()
    assert np.all(y == -5 * 127 * k)


def test_mfma_pair(matrix_cores):
    pc = syn.attention_pair_case(4, seed=77, na=4096 + 7, nb=4096 + 100, k=2048)
    xq = q2.q8_1_rows(bf16_dev(pc.x_bits))
    oq, od = assert_q8_equal(xq, pc.x_bits)
    ya, yb = q2.q2k_mmvq_pair(dev(pc.wa.reshape(-1)), pc.na, dev(pc.wb.reshape(-1)), pc.nb, xq, pc.k, 4)
    assert_pair(ya.cpu().numpy(), yb.cpu().numpy(), pc.wa, pc.wb, oq, od, "mfma pair")


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_fused_q8_1_pair_equals_two_calls(m):
    """q8_1_q2k_mmvq_pair on the attention pair shapes gives the xq bytes and
    output bits of q8_1_rows + q2k_mmvq_pair."""
    pc = syn.attention_pair_case(m)
    wa, wb = dev(pc.wa.reshape(-1)), dev(pc.wb.reshape(-1))
    x = bf16_dev(pc.x_bits)
    ya, yb, xq = q2.q8_1_q2k_mmvq_pair(wa, pc.na, wb, pc.nb, x, pc.k)
    xq2 = q2.q8_1_rows(x)
    ya2, yb2 = q2.q2k_mmvq_pair(wa, pc.na, wb, pc.nb, xq2, pc.k, m)
    need = q2.q8_1_rows_bytes(m, pc.k)
    assert torch.equal(xq[:need], xq2[:need])
    assert torch.equal(ya.view(torch.int32), ya2.view(torch.int32))
    assert torch.equal(yb.view(torch.int32), yb2.view(torch.int32))
    oq, od = assert_q8_equal(xq, pc.x_bits)
    assert_pair(ya.cpu().numpy(), yb.cpu().numpy(), pc.wa, pc.wb, oq, od, f"fused pair m={m}")


def test_pair_token_split_and_matrix_cores_agree():
    """The pair at m = 8 through the packed-dot kernel (tokens split over
    waves) and through the matrix cores: the same bits, the oracle's."""
    pc = syn.attention_pair_case(8, seed=78, na=2048 + 3, nb=1024 + 9, k=4096)
    xq = q2.q8_1_rows(bf16_dev(pc.x_bits))
    oq, od = assert_q8_equal(xq, pc.x_bits)
    wa, wb = dev(pc.wa.reshape(-1)), dev(pc.wb.reshape(-1))
    outs = []
    for choice in (q2.KERNEL_PACKED_DOTS, q2.KERNEL_MATRIX_CORES):
        prev = q2.q2k_set_product_kernel(choice)
        try:
            ya, yb = q2.q2k_mmvq_pair(wa, pc.na, wb, pc.nb, xq, pc.k, 8)
        finally:
            q2.q2k_set_product_kernel(prev)
        outs.append((ya.cpu().numpy(), yb.cpu().numpy()))
        assert_pair(outs[-1][0], outs[-1][1], pc.wa, pc.wb, oq, od, f"pair, kernel {choice}")
    assert_bits(outs[0][0], outs[1][0], "pair a: packed dots vs matrix cores")
    assert_bits(outs[0][1], outs[1][1], "pair b: packed dots vs matrix cores")


@pytest.mark.parametrize("n,k,m", [(1536, 4096, 8), (4103, 2048, 4), (300, 1024, 5),
                                   (1000, 2048, 2), (77, 512, 3), (64, 7168, 7)])
def test_token_split(n, k, m, packed_dots):
    """m > 1 on the packed-dot kernels: each wave takes one token. The first
    two shapes have enough (row step, token) pairs for the run kernel, the
    others take one step per wave; k = 512 has fewer than 8 lanes per row."""
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=7400 + n + m)
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    y = q2.q2k_mmvq(dev(case.w.reshape(-1)), xq, n, k, m).cpu().numpy()
    assert_product(y, case.w, oq, od, f"token split n={n} k={k} m={m}")


@pytest.mark.parametrize("n,k,m", [(20480, 2048, 1), (16384, 1024, 1), (8192, 4096, 1),
                                   (4099, 8192, 1), (4103, 2048, 4), (2050, 4096, 5),
                                   (4099, 7168, 3), (513, 8192, 8),
                                   (4096, 1024, 1), (300, 4096, 1), (1, 1280, 1), (3, 256, 1),
                                   (37, 2560, 1), (1, 8192, 1), (1000, 2048, 3), (8197, 7168, 8)])
def test_fused_q8_1_equals_two_calls(n, k, m):
    """q8_1_q2k_mmvq gives the bytes of q8_1_rows and the bits of q2k_mmvq on
    them. One token runs as one launch: the first four shapes on the run
    kernel (k = 8192 has 256 blocks, one per thread), the next six on the
    one-step kernel (one row, idle lanes past 2*k/256 half blocks, a single
    block per row); the last two take a q8_1 launch ahead of the product
    (tokens split over waves, the matrix cores). Rows are strided on the
    input for m > 1."""
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=7600 + n + k + m)
    w = dev(case.w.reshape(-1))
    if m == 1:
        x = bf16_dev(case.x_bits)
    else:
        wide = torch.zeros((m, k + 64), dtype=torch.bfloat16, device="cuda")
        wide[:, :k] = bf16_dev(case.x_bits)
        x = wide[:, :k]
    y, xq = q2.q8_1_q2k_mmvq(w, x, n, k)
    xq2 = q2.q8_1_rows(x)
    y2 = q2.q2k_mmvq(w, xq2, n, k, m)
    need = q2.q8_1_rows_bytes(m, k)
    assert torch.equal(xq[:need], xq2[:need])
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    oq, od = assert_q8_equal(xq, case.x_bits)
    assert_product(y.cpu().numpy(), case.w, oq, od, f"fused n={n} k={k} m={m}")


def _experts_check(x_per_id):
    rng = syn.rng_for(56, int(x_per_id))
    n, k, m, n_exp = 2048, 1024, 3, 10
    mats = [[syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)] for _ in range(2)]
    stride = n * (k // 256) * 84
    bases = [dev(np.concatenate([mt.reshape(-1) for mt in mats[b]])) for b in range(2)]
    ids_np = np.array([3, 9, 0, 12, 5, 1, 7, 2], dtype=np.int32)   # 12 is out of range
    x = syn.bf16_normal(rng, ((len(ids_np) if x_per_id else 1) * m, k))
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    y = q2.q2k_mmvq_experts(bases, stride, n_exp, dev(ids_np), xq, x_per_id, n, k, m,
                            err_flag=flag).cpu().numpy()
    assert int(flag.item()) == 1
    for b in range(2):
        for i, e in enumerate(ids_np.tolist()):
            if e >= n_exp:
                assert np.all(np.isnan(y[b, i]))
                continue
            xs = slice(i * m, (i + 1) * m) if x_per_id else slice(0, m)
            assert_product(y[b, i], mats[b][e], oq[xs], od[xs], f"expert base={b} id={e}")


@pytest.mark.parametrize("x_per_id", [False, True])
def test_mfma_experts(x_per_id, matrix_cores):
    """Gate/up-shaped experts (2048 rows) over 8 ids and two bases: 256
    workgroups; one id out of range gives NaN rows and the flag."""
    _experts_check(x_per_id)


@pytest.mark.parametrize("x_per_id", [False, True])
def test_experts_token_split(x_per_id, packed_dots):
    """The same batch (m = 3) on the packed-dot kernels, tokens split over
    waves."""
    _experts_check(x_per_id)


# ---------------------------------------------------------------- pair ------

@pytest.mark.parametrize("m", [1, 4, 8])
def test_pair_attention_inputs(m):
    """x [m, 4096] quantised once, wq_a [1024, 4096] and wkv [512, 4096]."""
    pc = syn.attention_pair_case(m)
    xq = q2.q8_1_rows(bf16_dev(pc.x_bits))
    oq, od = assert_q8_equal(xq, pc.x_bits)
    wa, wb = dev(pc.wa.reshape(-1)), dev(pc.wb.reshape(-1))
    ya, yb = q2.q2k_mmvq_pair(wa, pc.na, wb, pc.nb, xq, pc.k, m)
    assert_pair(ya.cpu().numpy(), yb.cpu().numpy(), pc.wa, pc.wb, oq, od, "pair")
    sa = q2.q2k_mmvq(wa, xq, pc.na, pc.k, m).cpu().numpy()
    sb = q2.q2k_mmvq(wb, xq, pc.nb, pc.k, m).cpu().numpy()
    assert np.array_equal(sa.view(np.uint32), ya.cpu().numpy().view(np.uint32))
    assert np.array_equal(sb.view(np.uint32), yb.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("n,k", [(1000, 2048), (130, 7168), (4099, 1024)])
def test_single_token_launch_forms_agree(n, k):
    """One token: a single-matrix launch (arguments in the leading scalars)
    and the same matrix as half of a pair (arguments in the block) give the
    same bits, including waves whose runs end early."""
    case = syn.single_gemv_case(n=n, k=k, m=1, seed=n + k)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    single = q2.q2k_mmvq(w, xq, n, k, 1).cpu().numpy()
    ya, yb = q2.q2k_mmvq_pair(w, n, w, n, xq, k, 1)
    assert np.array_equal(single.view(np.uint32), ya.cpu().numpy().view(np.uint32))
    assert np.array_equal(single.view(np.uint32), yb.cpu().numpy().view(np.uint32))
    assert_product(single, case.w, oq, od, f"single token n={n} k={k}")


def test_pair_ragged():
    pc = syn.attention_pair_case(3, seed=9, na=37, nb=5, k=1280)
    xq = q2.q8_1_rows(bf16_dev(pc.x_bits))
    oq, od = assert_q8_equal(xq, pc.x_bits)
    ya, yb = q2.q2k_mmvq_pair(dev(pc.wa.reshape(-1)), 37, dev(pc.wb.reshape(-1)), 5, xq, 1280, 3)
    assert_pair(ya.cpu().numpy(), yb.cpu().numpy(), pc.wa, pc.wb, oq, od, "ragged pair")


# -------------------------------------------------------------- grouped -----

@pytest.mark.parametrize("m", [1, 4, 8])
def test_grouped_wo_a(m):
    """8 groups of 1024 rows over 2048-wide slices of x [m, 16384]: the m = 1
    kernel at m = 1, the matrix cores above (64 workgroups)."""
    gc = syn.grouped_case(m)
    xq = q2.q8_1_rows(bf16_dev(gc.x_bits))
    oq, od = assert_q8_equal(xq, gc.x_bits)
    y = q2.q2k_mmvq_grouped(dev(gc.w.reshape(-1)), xq, gc.groups, gc.rows, gc.k, m).cpu().numpy()
    assert_close(y, orc.mmvq_grouped(gc.w, oq, od, gc.groups), f"grouped m={m}")
    assert_grouped(y, gc.w, oq, od, gc.groups, f"grouped m={m}")


@pytest.mark.parametrize("groups,rows,k,m", [(3, 37, 1280, 3), (5, 16, 256, 1), (2, 130, 9216, 2)])
def test_grouped_ragged_equals_slices(groups, rows, k, m):
    """Small and ragged groups (packed-dot kernels, k > 8192 on the wide one):
    the oracle, and bit-for-bit the plain product of each group's rows with
    the q8_1 rows of its slice (the kernels' sums do not depend on the grid)."""
    gc = syn.grouped_case(m, seed=60 + groups, groups=groups, rows=rows, k=k)
    w = dev(gc.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(gc.x_bits))
    oq, od = assert_q8_equal(xq, gc.x_bits)
    y = q2.q2k_mmvq_grouped(w, xq, groups, rows, k, m).cpu().numpy()
    assert_close(y, orc.mmvq_grouped(gc.w, oq, od, groups), "grouped ragged")
    assert_grouped(y, gc.w, oq, od, groups, "grouped ragged")
    per = rows * (k // 256) * 84
    for g in range(groups):
        xs = q2.q8_1_rows(bf16_dev(np.ascontiguousarray(gc.x_bits[:, g * k:(g + 1) * k])))
        ys = q2.q2k_mmvq(w[g * per:(g + 1) * per], xs, rows, k, m).cpu().numpy()
        assert np.array_equal(ys.view(np.uint32), y[:, g * rows:(g + 1) * rows].view(np.uint32))


# -------------------------------------------------------------- experts -----

POISON = 0x7E   # every byte 0x7E: d = dmin = fp16 0x7E7E, a NaN


def _expert_set(case, kind, n_rows, n_blocks):
    """Resident set of all experts of one kind: unselected experts are
    poisoned (NaN scales), the selected ones hold their seeded matrices."""
    per = n_rows * n_blocks * 84
    buf = torch.full((case.n_experts * per,), POISON, dtype=torch.uint8, device="cuda")
    for e in case.ids.tolist():
        buf[e * per:(e + 1) * per] = dev(case.expert_matrix(e, kind).reshape(-1))
    return buf, per


@pytest.fixture(scope="module")
def expert_batch():
    case = syn.expert_batch_case()
    gate, per_gu = _expert_set(case, "gate", case.inter, case.dim // 256)
    up, _ = _expert_set(case, "up", case.inter, case.dim // 256)
    down, per_d = _expert_set(case, "down", case.dim, case.inter // 256)
    return case, gate, up, down, per_gu, per_d


def test_expert_batch_stagewise(expert_batch):
    """Gate/up over 8 of 256 experts, bf16 SwiGLU + q8_1, down: [8, 4096]."""
    case, gate, up, down, per_gu, per_d = expert_batch
    ids = dev(case.ids)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    oq, od = assert_q8_equal(xq, case.x_bits)
    gu = q2.q2k_mmvq_experts([gate, up], per_gu, case.n_experts, ids, xq, False,
                             case.inter, case.dim, 1, err_flag=flag)
    gu_h = gu.cpu().numpy()
    for bi, kind in enumerate(("gate", "up")):
        mats = [case.expert_matrix(e, kind) for e in case.ids.tolist()]
        assert_experts(gu_h[bi], mats, oq, od, False, kind)
    g = gu[0].reshape(len(case.ids), case.inter).contiguous()
    u = gu[1].reshape(len(case.ids), case.inter).contiguous()
    h, hq = q2.swiglu_q8_1_rows(g, u)
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_h = orc.swiglu_bf16_bits(g.cpu().numpy(), u.cpu().numpy())
    assert bf16_ulp_distance(h_bits, ref_h).max() <= 1, "SwiGLU more than one bf16 ulp off"
    hq_o, hd_o = assert_q8_equal(hq, h_bits)
    yd = q2.q2k_mmvq_experts([down], per_d, case.n_experts, ids, hq, True, case.dim,
                             case.inter, 1, err_flag=flag)
    mats = [case.expert_matrix(e, "down") for e in case.ids.tolist()]
    assert_experts(yd.cpu().numpy()[0], mats, hq_o, hd_o, True, "down")
    assert int(flag.item()) == 0
    # experts == per-expert singles, bit for bit
    for i, e in enumerate(case.ids.tolist()):
        s = q2.q2k_mmvq(down[e * per_d:(e + 1) * per_d], hq[i * q2.q8_1_rows_bytes(1, 2048):],
                        case.dim, case.inter, 1).cpu().numpy()
        assert np.array_equal(s.view(np.uint32), yd.cpu().numpy()[0, i].view(np.uint32))


def test_fused_q8_1_experts_equals_two_calls(expert_batch):
    """q8_1_q2k_mmvq_experts (gate/up form, one launch for one token) gives
    the bytes of q8_1_rows and the bits of q2k_mmvq_experts on them; an id
    out of range still NaN-fills its rows and sets the flag."""
    case, gate, up, down, per_gu, per_d = expert_batch
    x = bf16_dev(case.x_bits)
    for ids_np in (case.ids, np.array([case.ids[0], 300, case.ids[2], -4], dtype=np.int32)):
        ids = dev(ids_np.astype(np.int32))
        f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        f2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        y, xq = q2.q8_1_q2k_mmvq_experts([gate, up], per_gu, case.n_experts, ids, x, case.inter,
                                         case.dim, err_flag=f1)
        xq2 = q2.q8_1_rows(x)
        y2 = q2.q2k_mmvq_experts([gate, up], per_gu, case.n_experts, ids, xq2, False, case.inter,
                                 case.dim, 1, err_flag=f2)
        need = q2.q8_1_rows_bytes(1, case.dim)
        assert torch.equal(xq[:need], xq2[:need])
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
        assert int(f1.item()) == int(f2.item()) == int(np.any((ids_np < 0) | (ids_np >= case.n_experts)))


def test_fused_swiglu_down_equals_two_calls(expert_batch):
    """swiglu_q2k_mmvq_experts on the gate/up outputs of the expert batch
    (one launch: SwiGLU and q8_1 of each id's row inside the down product)
    gives the hq bytes of swiglu_q8_1_rows and the y bits of the down
    product on them; the down output is within tolerance of the oracle on
    the oracle's q8_1 of that h, and a bad id still NaN-fills and flags."""
    case, gate, up, down, per_gu, per_d = expert_batch
    x = bf16_dev(case.x_bits)
    for ids_np in (case.ids, np.array(list(case.ids[:5]) + [999, case.ids[6], case.ids[7]], dtype=np.int32)):
        ids = dev(ids_np.astype(np.int32))
        gu, _ = q2.q8_1_q2k_mmvq_experts([gate, up], per_gu, case.n_experts, ids, x, case.inter, case.dim)
        g = gu[0].reshape(len(ids_np), case.inter).contiguous()
        u = gu[1].reshape(len(ids_np), case.inter).contiguous()
        f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        f2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        y, hq = q2.swiglu_q2k_mmvq_experts([down], per_d, case.n_experts, ids, g, u, case.dim, err_flag=f1)
        h2, hq2 = q2.swiglu_q8_1_rows(g, u)
        y2 = q2.q2k_mmvq_experts([down], per_d, case.n_experts, ids, hq2, True, case.dim, case.inter, 1,
                                 err_flag=f2)
        need = q2.q8_1_rows_bytes(len(ids_np), case.inter)
        assert torch.equal(hq[:need], hq2[:need])
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
        bad = (ids_np < 0) | (ids_np >= case.n_experts)
        assert int(f1.item()) == int(f2.item()) == int(np.any(bad))
        if not np.any(bad):
            h_bits = h2.view(torch.int16).cpu().numpy().view(np.uint16)
            hq_o, hd_o = assert_q8_equal(hq, h_bits)
            mats = [case.expert_matrix(e, "down") for e in ids_np.tolist()]
            assert_experts(y.cpu().numpy()[0], mats, hq_o, hd_o, True, "fused SwiGLU down")


def _gate_up_swiglu_two_calls(gate, up, stride, n_experts, ids, x, n, k, n_ids):
    """The calls q8_1_q2k_mmvq_experts_swiglu stands for: gate/up with x's
    q8_1 in the product, then swiglu_q8_1_rows of the two result sets."""
    f = torch.zeros(1, dtype=torch.int32, device="cuda")
    y, xq = q2.q8_1_q2k_mmvq_experts([gate, up], stride, n_experts, ids, x, n, k, err_flag=f)
    g = y[0].reshape(n_ids, n).contiguous()
    u = y[1].reshape(n_ids, n).contiguous()
    h, hq = q2.swiglu_q8_1_rows(g, u)
    return y, xq, h, hq, f


def test_fused_gate_up_swiglu_equals_calls(expert_batch):
    """q8_1_q2k_mmvq_experts_swiglu (one launch: gate and up rows of one id
    per workgroup, SwiGLU and q8_1 in its epilogue) gives the bits of y and
    the bytes of xq, h and hq of the separate calls; a bad id NaN-fills its
    rows and sets the flag as there; the whole chain through the down
    product matches the oracle."""
    case, gate, up, down, per_gu, per_d = expert_batch
    x = bf16_dev(case.x_bits)
    n, k = case.inter, case.dim
    for ids_np in (case.ids, np.array([case.ids[0], 300, case.ids[2], -4], dtype=np.int32)):
        ids = dev(ids_np.astype(np.int32))
        n_ids = len(ids_np)
        for want_h in (True, False):
            f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
            y, xq, h, hq = q2.q8_1_q2k_mmvq_experts_swiglu([gate, up], per_gu, case.n_experts, ids, x,
                                                           n, k, want_h=want_h, err_flag=f1)
            y2, xq2, h2, hq2, f2 = _gate_up_swiglu_two_calls(gate, up, per_gu, case.n_experts, ids, x,
                                                             n, k, n_ids)
            need = q2.q8_1_rows_bytes(1, k)
            assert torch.equal(xq[:need], xq2[:need])
            assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
            hneed = q2.q8_1_rows_bytes(n_ids, n)
            assert torch.equal(hq[:hneed], hq2[:hneed])
            if want_h:
                assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
            else:
                assert h is None
            bad = (ids_np < 0) | (ids_np >= case.n_experts)
            assert int(f1.item()) == int(f2.item()) == int(np.any(bad))
    # the chain against the oracle: gate/up, the SwiGLU within one bf16 step,
    # q8_1 of the GPU's h exact, then the down product
    ids = dev(case.ids)
    y, xq, h, hq = q2.q8_1_q2k_mmvq_experts_swiglu([gate, up], per_gu, case.n_experts, ids, x, n, k,
                                                   want_h=True)
    oq, od = assert_q8_equal(xq, case.x_bits)
    gu_h = y.cpu().numpy()
    for bi, kind in enumerate(("gate", "up")):
        mats = [case.expert_matrix(e, kind) for e in case.ids.tolist()]
        assert_experts(gu_h[bi], mats, oq, od, False, f"fused {kind}")
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_h = orc.swiglu_bf16_bits(gu_h[0].reshape(-1, n), gu_h[1].reshape(-1, n))
    assert bf16_ulp_distance(h_bits, ref_h).max() <= 1, "SwiGLU more than one bf16 ulp off"
    hq_o, hd_o = assert_q8_equal(hq, h_bits)
    yd = q2.q2k_mmvq_experts([down], per_d, case.n_experts, ids, hq, True, case.dim, n, 1)
    mats = [case.expert_matrix(e, "down") for e in case.ids.tolist()]
    assert_experts(yd.cpu().numpy()[0], mats, hq_o, hd_o, True, "down after the fused SwiGLU")


@pytest.mark.parametrize("n,k,n_ids", [(256, 2048, 1), (512, 8192, 3), (1280, 2304, 2),
                                       (512, 1024, 3), (256, 12288, 2), (320 * 8, 4096, 5)])
def test_fused_gate_up_swiglu_shapes(n, k, n_ids):
    """Row lengths of 2048 to 8192 values (16, 32 or 64 lanes per row, so
    8, 16 or 32 row steps per wave) in one launch; k = 1024 and the wide
    rows past 8192 values take the SwiGLU launch after the product; the
    same bits as the separate calls either way."""
    rng = syn.rng_for(59, n, k)
    n_exp = 6
    gm = [syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)]
    um = [syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)]
    stride = n * (k // 256) * 84
    gate = dev(np.concatenate([mt.reshape(-1) for mt in gm]))
    up = dev(np.concatenate([mt.reshape(-1) for mt in um]))
    ids = dev(rng.choice(n_exp, n_ids, replace=False).astype(np.int32))
    xb = syn.bf16_normal(rng, (1, k))
    x = bf16_dev(xb)
    y, xq, h, hq = q2.q8_1_q2k_mmvq_experts_swiglu([gate, up], stride, n_exp, ids, x, n, k, want_h=True)
    y2, xq2, h2, hq2, _ = _gate_up_swiglu_two_calls(gate, up, stride, n_exp, ids, x, n, k, n_ids)
    assert torch.equal(xq[:q2.q8_1_rows_bytes(1, k)], xq2[:q2.q8_1_rows_bytes(1, k)])
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    assert torch.equal(h.view(torch.int16), h2.view(torch.int16))
    hneed = q2.q8_1_rows_bytes(n_ids, n)
    assert torch.equal(hq[:hneed], hq2[:hneed])
    oq, od = assert_q8_equal(xq, xb)
    sel = ids.cpu().numpy().tolist()
    assert_experts(y.cpu().numpy()[0], [gm[i] for i in sel], oq, od, False, "fused gate")
    assert_experts(y.cpu().numpy()[1], [um[i] for i in sel], oq, od, False, "fused up")


@pytest.mark.parametrize("n,k,n_ids", [(4096, 4096, 3), (200, 1024, 5), (1000, 2048, 3)])
def test_fused_swiglu_down_fallback_shapes(n, k, n_ids):
    """Rows over 2048 values, too few row steps, or ids whose waves do not
    fill whole workgroups: a SwiGLU launch ahead of the product, same bits."""
    rng = syn.rng_for(58, n, k)
    n_exp = 6
    mats = [syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)]
    stride = n * (k // 256) * 84
    base = dev(np.concatenate([mt.reshape(-1) for mt in mats]))
    ids = dev(rng.choice(n_exp, n_ids, replace=False).astype(np.int32))
    g = torch.from_numpy(rng.standard_normal((n_ids, k)).astype(np.float32) * 3).cuda()
    u = torch.from_numpy(rng.standard_normal((n_ids, k)).astype(np.float32) * 3).cuda()
    y, hq = q2.swiglu_q2k_mmvq_experts([base], stride, n_exp, ids, g, u, n)
    _, hq2 = q2.swiglu_q8_1_rows(g, u, want_h=False)
    y2 = q2.q2k_mmvq_experts([base], stride, n_exp, ids, hq2, True, n, k, 1)
    need = q2.q8_1_rows_bytes(n_ids, k)
    assert torch.equal(hq[:need], hq2[:need])
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))


def test_fused_q8_1_experts_small_and_multi_token():
    """Shapes that take a q8_1 launch ahead of the product (few row steps;
    m = 3): still the bits of the two calls."""
    rng = syn.rng_for(57)
    n, k, n_exp = 200, 1024, 6
    mats = [syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)]
    stride = n * (k // 256) * 84
    base = dev(np.concatenate([mt.reshape(-1) for mt in mats]))
    ids = dev(np.array([5, 0, 3], dtype=np.int32))
    for m in (1, 3):
        xb = syn.bf16_normal(rng, (m, k))
        x = bf16_dev(xb)
        y, xq = q2.q8_1_q2k_mmvq_experts([base], stride, n_exp, ids, x, n, k)
        xq2 = q2.q8_1_rows(x)
        y2 = q2.q2k_mmvq_experts([base], stride, n_exp, ids, xq2, False, n, k, m)
        assert torch.equal(xq[:q2.q8_1_rows_bytes(m, k)], xq2[:q2.q8_1_rows_bytes(m, k)])
        assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
        oq, od = assert_q8_equal(xq, xb)
        assert_experts(y.cpu().numpy()[0], [mats[i] for i in (5, 0, 3)], oq, od, False,
                       f"fused experts m={m}")


def test_expert_bad_id_flags_and_nans(expert_batch):
    case, gate, up, down, per_gu, per_d = expert_batch
    ids = dev(np.array([case.ids[0], 300, -1, case.ids[1]], dtype=np.int32))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    y = q2.q2k_mmvq_experts([gate], per_gu, case.n_experts, ids, xq, False, case.inter,
                            case.dim, 1, err_flag=flag).cpu().numpy()
    assert int(flag.item()) == 1
    assert np.all(np.isnan(y[0, 1])) and np.all(np.isnan(y[0, 2]))
    assert np.all(np.isfinite(y[0, 0])) and np.all(np.isfinite(y[0, 3]))


def test_experts_multi_token_shared_and_per_id():
    rng = syn.rng_for(55)
    n, k, m, n_exp = 200, 1024, 3, 6
    mats = [syn.q2k_blocks(rng, n, k // 256) for _ in range(n_exp)]
    stride = n * (k // 256) * 84 + 4            # padded stride
    buf = np.zeros(n_exp * stride, dtype=np.uint8)
    for e in range(n_exp):
        buf[e * stride:e * stride + mats[e].size] = mats[e].reshape(-1)
    ids_np = np.array([5, 0, 3], dtype=np.int32)
    x = syn.bf16_normal(rng, (len(ids_np) * m, k))
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    y = q2.q2k_mmvq_experts([dev(buf)], stride, n_exp, dev(ids_np), xq, True, n, k, m).cpu().numpy()
    assert_experts(y[0], [mats[i] for i in ids_np], oq, od, True, "per-id experts")
    ys = q2.q2k_mmvq_experts([dev(buf)], stride, n_exp, dev(ids_np), xq, False, n, k, m).cpu().numpy()
    assert_experts(ys[0], [mats[i] for i in ids_np], oq[:m], od[:m], False, "shared-input experts")


# --------------------------------------------------------------- engram -----

@pytest.fixture(scope="module")
def engram():
    return syn.engram_step_case()


def test_dequant_rows_bit_exact(engram):
    table = dev(engram.table.reshape(-1))
    ids = dev(engram.ids)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    out = q2.q2k_dequant_rows(table, engram.table.shape[0], ids, len(engram.ids), err_flag=flag)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc.dequant_rows_bf16_bits(engram.table, engram.ids))
    assert int(flag.item()) == 0
    many = dev(syn.rng_for(3).integers(0, engram.table.shape[0], size=4099, dtype=np.int64))
    out = q2.q2k_dequant_rows(table, engram.table.shape[0], many, 4099)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc.dequant_rows_bf16_bits(engram.table, many.cpu().numpy()))
    out = q2.q2k_dequant_rows(table, engram.table.shape[0], None, 13)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got, orc.dequant_rows_bf16_bits(engram.table[:13], None))


@pytest.mark.parametrize("n_rows", [1, 8, 37])
def test_dequant_rows_q8_1_is_the_composition(engram, n_rows):
    """One launch gives the bits of q2k_dequant_rows then q8_1_rows on the
    rows viewed as one [1, 256 n_rows] row, and matches the oracle."""
    table = dev(engram.table.reshape(-1))
    nt = engram.table.shape[0]
    ids_np = syn.rng_for(7300, n_rows).integers(0, nt, size=n_rows, dtype=np.int64)
    ids = dev(ids_np)
    rows = q2.q2k_dequant_rows(table, nt, ids, n_rows)
    xq_ref = q2.q8_1_rows(rows.view(1, n_rows * 256))
    xq, out = q2.q2k_dequant_rows_q8_1(table, nt, ids, n_rows, want_rows=True)
    need = q2.q8_1_rows_bytes(1, n_rows * 256)
    assert torch.equal(xq[:need], xq_ref[:need])
    assert torch.equal(out.view(torch.int16), rows.view(torch.int16))
    bits = orc.dequant_rows_bf16_bits(engram.table, ids_np).reshape(1, -1)
    assert_q8_equal(xq, bits)
    xq2, none = q2.q2k_dequant_rows_q8_1(table, nt, ids, n_rows)    # no bf16 copy
    assert none is None and torch.equal(xq2[:need], xq_ref[:need])


def test_dequant_rows_q8_1_bad_ids_match_the_composition():
    table = np.zeros((3, 84), dtype=np.uint8)
    table[:, 0:16] = 0x25
    table[:, 16:80] = 0x9C
    table[:, 80:84] = [0x00, 0x3C, 0x00, 0x38]
    ids = dev(np.array([0, 5, 2, -1], dtype=np.int64))
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = q2.q2k_dequant_rows(dev(table.reshape(-1)), 3, ids, 4)
    xq_ref = q2.q8_1_rows(rows.view(1, 1024))
    xq, out = q2.q2k_dequant_rows_q8_1(dev(table.reshape(-1)), 3, ids, 4, want_rows=True, err_flag=flag)
    need = q2.q8_1_rows_bytes(1, 1024)
    assert torch.equal(xq[:need], xq_ref[:need])
    assert torch.equal(out.view(torch.int16), rows.view(torch.int16))
    assert int(flag.item()) == 1


def test_dequant_rows_hand_blocks_and_bad_ids():
    table = np.zeros((3, 84), dtype=np.uint8)
    table[0, 0:16] = [((15 - s) << 4) | s for s in range(16)]
    table[0, 16:80] = 0xE4
    table[0, 80:84] = [0x00, 0x3C, 0x00, 0x38]
    table[1, 0:16] = 0x1F                           # sc = 15, m = 1
    table[1, 16:80] = 0xFF
    table[1, 80:84] = [0x00, 0x3C, 0x00, 0xB0]     # 45 - (-0.125) = 45.125: a tie
    table[2, 80:84] = [0x00, 0x00, 0x00, 0x00]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    ids = dev(np.array([0, 1, 2, 3, -7], dtype=np.int64))
    out = q2.q2k_dequant_rows(dev(table.reshape(-1)), 3, ids, 5, err_flag=flag)
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    assert np.array_equal(got[:3], orc.dequant_rows_bf16_bits(table, [0, 1, 2]))
    assert got[1, 0] == 0x4234 and np.all(got[2] == 0)
    assert np.all(got[3:] == 0x7FC0) and int(flag.item()) == 1


@pytest.mark.parametrize("t,hc,dim", [(1, 4, 4096), (2, 1, 4096), (3, 3, 1000), (1, 2, 7), (4, 4, 256),
                                      (1, 4, 16384), (2, 2, 6000), (1, 3, 4100)])
def test_engram_gate(t, hc, dim):
    h, kv, qk, eps = syn.gate_case(11, t, hc, dim)
    hd = dev(h)
    q2.engram_gate(hd, dev(kv), dev(qk), eps)
    assert_close(hd.cpu().numpy(), orc.engram_gate(h, kv, qk, eps), f"gate {t},{hc},{dim}")


def test_engram_gate_unaligned_takes_scalar_path():
    """h, kv and qk 4 bytes past a 16-byte boundary: the strided scalar
    kernel runs (the 16-byte one needs aligned rows); same tolerance."""
    t, hc, dim = 1, 4, 4096
    h, kv, qk, eps = syn.gate_case(12, t, hc, dim)
    hb = torch.zeros(h.size + 1, dtype=torch.float32, device="cuda")
    kb = torch.zeros(kv.size + 1, dtype=torch.float32, device="cuda")
    qb = torch.zeros(qk.size + 1, dtype=torch.float32, device="cuda")
    hb[1:] = dev(h.reshape(-1))
    kb[1:] = dev(kv.reshape(-1))
    qb[1:] = dev(qk.reshape(-1))
    hv = hb[1:].view(t, hc, dim)
    q2.engram_gate(hv, kb[1:].view(t, (hc + 1) * dim), qb[1:].view(hc, dim), eps)
    ref = orc.engram_gate(h, kv, qk, eps)
    assert_close(hv.cpu().numpy(), ref, "gate, scalar path")
    ha = dev(h)
    q2.engram_gate(ha, dev(kv), dev(qk), eps)
    assert_close(ha.cpu().numpy(), ref, "gate, 16-byte path")


def test_engram_gate_closed_forms():
    dim = 64
    h = np.zeros((1, 2, dim), np.float32)
    h[0, :, :32] = 1.0
    kv = np.zeros((1, 3 * dim), np.float32)
    kv[0, 32:64] = 2.0
    kv[0, 96:128] = -3.0
    kv[0, 128:] = np.arange(dim, dtype=np.float32)
    qk = np.ones((2, dim), np.float32)
    hd = dev(h)
    q2.engram_gate(hd, dev(kv), dev(qk), 1e-6)
    expect = h + 0.5 * np.arange(dim, dtype=np.float32)      # s = 0 -> g = 1/2
    assert np.array_equal(hd.cpu().numpy(), expect)
    kv[0, 128:] = 0.0
    hd = dev(h)
    q2.engram_gate(hd, dev(kv), dev(qk), 1e-6)
    assert np.array_equal(hd.cpu().numpy(), h)                # v = 0: unchanged


@pytest.mark.parametrize("dim", [4, 4096])
def test_engram_gate_small_vectors_eps(dim):
    """Constant vectors small enough that eps = 1e-6 matters (h = 1e-3,
    keys 2e-3, value 1): the oracle's eps-inside-each-rms reading, and for
    dim = 4 its closed form s = 4/sqrt(10)."""
    a, b, eps, hc = 1e-3, 2e-3, 1e-6, 2
    h = np.full((1, hc, dim), a, np.float32)
    kv = np.concatenate([np.full(hc * dim, b, np.float32), np.ones(dim, np.float32)])[None]
    qk = np.ones((hc, dim), np.float32)
    hd = dev(h)
    q2.engram_gate(hd, dev(kv), dev(qk), eps)
    got = hd.cpu().numpy()
    ref = orc.engram_gate(h, kv, qk, eps)
    assert_close(got, ref, f"gate small vectors dim={dim}")
    if dim == 4:
        g = 1.0 / (1.0 + np.exp(-np.sqrt(4.0 / np.sqrt(10.0))))
        assert_close(got, np.full_like(ref, a + g), "closed form")


def test_engram_step(engram):
    """Row gather [8 x 256] -> [1, 2048] -> q8_1 -> wkv [20480, 2048] -> gate on [1, 4, 4096]."""
    e = engram
    table = dev(e.table.reshape(-1))
    rows = q2.q2k_dequant_rows(table, e.table.shape[0], dev(e.ids), e.cols)
    rows_bits = rows.view(torch.int16).cpu().numpy().view(np.uint16)
    ref_rows = orc.dequant_rows_bf16_bits(e.table, e.ids)
    assert np.array_equal(rows_bits, ref_rows)
    x = rows.view(1, e.cols * 256)
    xq = q2.q8_1_rows(x)
    oq, od = assert_q8_equal(xq, ref_rows.reshape(1, -1))
    n_out = e.dim * (e.hc + 1)
    kv = q2.q2k_mmvq(dev(e.wkv.reshape(-1)), xq, n_out, e.cols * 256, 1)
    assert_product(kv.cpu().numpy(), e.wkv, oq, od, "wkv")
    I, M = orc.block_dots(e.wkv, oq)
    ref_kv = orc.mmvq_from_block_dots(e.wkv, I, M, od)[0][None]
    hd = dev(e.h)
    q2.engram_gate(hd, kv, dev(e.qk), e.eps)
    kv_h = kv.cpu().numpy()
    assert_close(hd.cpu().numpy(), orc.engram_gate(e.h, kv_h, e.qk, e.eps), "gate (stage)")
    assert_close(hd.cpu().numpy(), orc.engram_gate(e.h, ref_kv, e.qk, e.eps), "gate (end to end)")


# ------------------------------------------------- bf16-activation GEMV -----

@pytest.mark.parametrize("n,k,m", [(257, 1024, 1), (100, 2048, 3), (33, 7168, 8), (10, 9216, 2),
                                   (5, 256, 1), (64, 4096, 5), (300, 768, 1), (70, 4096, 1),
                                   (70001, 256, 1), (901, 6144, 1), (333, 512, 1), (40, 256, 2),
                                   (40, 512, 3), (40, 1024, 4), (65832, 512, 1)])
def test_gemv_bf16_bit_exact(n, k, m):
    """Exact expansion, exact products, fp64 sums: the f32 bits of the oracle.
    One-token shapes with k <= 4096 run the quarter kernel, whose waves keep
    a ring of three row steps: [70001, 256] gives its 2048 waves two or three
    steps, [65832, 512] four or five (a second pass through the ring that
    stops after one or two slots), the engram projection five."""
    case = syn.single_gemv_case(n=n, k=k, m=m, seed=900 + n + k + m)
    y = q2.q2k_gemv_bf16(dev(case.w.reshape(-1)), bf16_dev(case.x_bits), n, k).cpu().numpy()
    ref = orc.gemv_bf16(case.w, case.x_bits)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), f"n={n} k={k} m={m}"


def test_gemv_bf16_strided_input():
    case = syn.single_gemv_case(n=70, k=1024, m=3, seed=905)
    xb = torch.zeros((3, 1024 + 64), dtype=torch.bfloat16, device="cuda")
    xb[:, :1024] = bf16_dev(case.x_bits)
    y = q2.q2k_gemv_bf16(dev(case.w.reshape(-1)), xb[:, :1024], 70, 1024).cpu().numpy()
    assert np.array_equal(y.view(np.uint32), orc.gemv_bf16(case.w, case.x_bits).view(np.uint32))


def test_engram_step_bf16_projection(engram):
    """The pages' single-token route: gathered bf16 rows [1, 2048] straight
    into the Q2_K wkv [20480, 2048] (no q8_1; every row bit for bit against
    the oracle, in chunks), then the gate."""
    e = engram
    rows = q2.q2k_dequant_rows(dev(e.table.reshape(-1)), e.table.shape[0], dev(e.ids), e.cols)
    x = rows.view(1, e.cols * 256)
    n_out = e.dim * (e.hc + 1)
    kv = q2.q2k_gemv_bf16(dev(e.wkv.reshape(-1)), x, n_out, e.cols * 256)
    kv_h = kv.cpu().numpy()
    x_bits = rows.view(torch.int16).cpu().numpy().view(np.uint16).reshape(1, -1)
    for r0 in range(0, n_out, CHUNK_ROWS):
        r1 = min(n_out, r0 + CHUNK_ROWS)
        ref = orc.gemv_bf16(e.wkv[r0:r1], x_bits)
        assert np.array_equal(kv_h[:, r0:r1].view(np.uint32), ref.view(np.uint32)), f"rows {r0}..{r1}"
    hd = dev(e.h)
    q2.engram_gate(hd, kv, dev(e.qk), e.eps)
    assert_close(hd.cpu().numpy(), orc.engram_gate(e.h, kv_h, e.qk, e.eps), "gate after bf16 wkv")


# ---------------------------------------------------- engram n-gram hash ---

def _hash_tables_dev(hc):
    return (dev(hc.token_map), dev(hc.multipliers), dev(hc.primes), dev(hc.offsets))


def _oracle_hash_layer_major(hc, cache, tokens, start):
    ids, cache = orc.engram_hash(hc.token_map.tolist(), hc.multipliers.tolist(), hc.primes.tolist(),
                                 hc.offsets.tolist(), hc.pad_id, hc.n_heads, cache, tokens, start)
    return np.array(ids, dtype=np.int64).transpose(1, 0, 2), cache


def test_engram_hash_prefill_then_decode():
    """Prefill of 64 positions, then single-token decode steps carrying the
    device cache: every row id and the cache bit-exact against the oracle."""
    hc = syn.engram_hash_case(seqlen=80)
    tm, mu, pr, of = _hash_tables_dev(hc)
    cache = torch.zeros(128, dtype=torch.int64, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(hc.tokens[:64]), 0, err_flag=flag)
    want, ocache = _oracle_hash_layer_major(hc, [0] * 128, hc.tokens[:64].tolist(), 0)
    assert np.array_equal(got.cpu().numpy(), want)
    for s in range(64, 80):
        got = q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(hc.tokens[s:s + 1]), s, err_flag=flag)
        want, ocache = _oracle_hash_layer_major(hc, ocache, [int(hc.tokens[s])], s)
        assert np.array_equal(got.cpu().numpy(), want), f"decode step {s}"
    assert np.array_equal(cache.cpu().numpy(), np.array(ocache, dtype=np.int64))
    assert int(flag.item()) == 0


def test_engram_hash_moduli_across_the_range():
    """Row ids for moduli from 1 to 2^62, both sides of 2^32 (the kernels take
    the remainder 16 bits at a time in fp64 below 2^32, by integer division
    above): every id bit for bit against the oracle's Python remainder, over
    rolling hashes of both signs."""
    hc = syn.engram_hash_case(seed=14, seqlen=48)
    mods = [(1 << 32) - 5, (1 << 32) - 1, (1 << 31) + 11, 1, 2, 65537, 1 << 32, (1 << 32) + 15,
            (1 << 40) + 7, (1 << 62) + 3, 3, 1234567891, 999999937, (1 << 33) - 9, 7, 65521]
    primes = np.array(mods, dtype=np.int64).reshape(hc.primes.shape)
    offsets = np.zeros_like(hc.offsets)
    big = dataclasses.replace(hc, primes=primes, offsets=offsets)
    tm, mu, pr, of = _hash_tables_dev(big)
    cache = torch.zeros(64, dtype=torch.int64, device="cuda")
    got = q2.engram_hash(tm, mu, pr, of, big.pad_id, cache, dev(big.tokens[:48]), 0)
    want, _ = _oracle_hash_layer_major(big, [0] * 64, big.tokens[:48].tolist(), 0)
    assert np.array_equal(got.cpu().numpy(), want)
    assert (want < 0).sum() < want.size // 4        # mostly real ids, not blocked columns


def test_engram_hash_wide_ngram_and_large_ids():
    """max_ngram 6, 16 heads, compressed ids near 2^62 (products wrap)."""
    hc = syn.engram_hash_case(seed=8, vocab=512, n_layers=3, max_ngram=6, n_heads=16, seqlen=40)
    hc.token_map[hc.token_map >= 0] += 1 << 62
    tm, mu, pr, of = _hash_tables_dev(hc)
    cache = torch.zeros(40, dtype=torch.int64, device="cuda")
    got = q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(hc.tokens), 0)
    want, _ = _oracle_hash_layer_major(hc, [0] * 40, hc.tokens.tolist(), 0)
    assert np.array_equal(got.cpu().numpy(), want)


def test_engram_hash_bad_token_flags_its_windows():
    hc = syn.engram_hash_case(seed=9, seqlen=12)
    toks = hc.tokens.copy()
    toks[5] = len(hc.token_map) + 3                        # outside the map
    tm, mu, pr, of = _hash_tables_dev(hc)
    cache = torch.zeros(12, dtype=torch.int64, device="cuda")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    got = q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(toks), 0, err_flag=flag).cpu().numpy()
    assert int(flag.item()) == 1
    assert np.all(got[:, 5:8] == -1)                       # windows of 3 reading position 5
    want, _ = _oracle_hash_layer_major(hc, [0] * 12, toks[:5].tolist(), 0)
    assert np.array_equal(got[:, :5], want)
    assert int(cache[5].item()) == -1


def test_engram_hashed_rows_gather():
    """Hashed ids of one layer feed the row gather directly (bit-exact)."""
    hc = syn.engram_hash_case(seqlen=16)
    table = syn.q2k_blocks(syn.rng_for(1001, 7), 500000, 1)
    tm, mu, pr, of = _hash_tables_dev(hc)
    cache = torch.zeros(16, dtype=torch.int64, device="cuda")
    ids = q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(hc.tokens), 0)
    layer1 = ids[1].reshape(-1)                           # [tokens * cols]
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    rows = q2.q2k_dequant_rows(dev(table.reshape(-1)), 500000, layer1, layer1.numel(), err_flag=flag)
    want_ids = _oracle_hash_layer_major(hc, [0] * 16, hc.tokens.tolist(), 0)[0][1].reshape(-1)
    assert np.array_equal(layer1.cpu().numpy(), want_ids)
    ref = orc.dequant_rows_bf16_bits(table[:, 0], want_ids)
    assert np.array_equal(rows.view(torch.int16).cpu().numpy().view(np.uint16), ref)
    assert int(flag.item()) == 0


def _engram_rows_both_ways(hc, table_np, tokens, start, layer, n_table_rows, bad_prime=False):
    """Decode tokens one at a time through engram_rows_q8_1 and through
    engram_hash + q2k_dequant_rows_q8_1 with separate caches; every id, row,
    q8_1 byte, cache entry and flag must agree."""
    tm, mu, pr, of = _hash_tables_dev(hc)
    if bad_prime:
        pr.view(-1)[3] = 0
    table = dev(table_np.reshape(-1))
    cols = (mu.shape[1] - 1) * pr.shape[-1]
    c1 = torch.zeros(len(tokens) + start + 8, dtype=torch.int64, device="cuda")
    c2 = c1.clone()
    # a prefill through the plain hash gives both caches the same history
    if start > 0:
        pre = dev(hc.tokens[:start].astype(np.int32))
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, c1, pre, 0)
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, c2, pre, 0)
    need = q2.q8_1_rows_bytes(1, cols * 256)
    for s, t in enumerate(tokens):
        pos = start + s
        tok = dev(np.array([t], dtype=np.int32))
        f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        f2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        ids1 = torch.empty(cols, dtype=torch.int64, device="cuda")
        rows1 = torch.empty((cols, 256), dtype=torch.bfloat16, device="cuda")
        xq1 = q2.engram_rows_q8_1(tm, mu, pr, of, hc.pad_id, c1, tok, pos, layer, table, n_table_rows,
                                  ids_out=ids1, rows_out=rows1, err_flag=f1)
        ids2 = q2.engram_hash(tm, mu, pr, of, hc.pad_id, c2, tok, pos, err_flag=f2)[layer].reshape(-1)
        xq2, rows2 = q2.q2k_dequant_rows_q8_1(table, n_table_rows, ids2, cols, want_rows=True, err_flag=f2)
        assert torch.equal(ids1, ids2), f"ids, position {pos}"
        assert torch.equal(rows1.view(torch.int16), rows2.view(torch.int16)), f"rows, position {pos}"
        assert torch.equal(xq1[:need], xq2[:need]), f"q8_1, position {pos}"
        assert int(f1.item()) == int(f2.item()), f"flag, position {pos}"
    assert torch.equal(c1, c2)


def test_engram_rows_q8_1_is_the_composition():
    """One launch for hash (one layer) + gather + dequant + q8_1 of a decode
    token: the bits of engram_hash then q2k_dequant_rows_q8_1, after a
    prefill, for both hashed layers."""
    hc = syn.engram_hash_case(seqlen=48)
    table = syn.q2k_blocks(syn.rng_for(1001, 8), 500000, 1)
    for layer in (0, 1):
        _engram_rows_both_ways(hc, table, hc.tokens[32:48].tolist(), 32, layer, 500000)


def test_engram_rows_q8_1_bad_token_prime_and_wide():
    """A token outside the map (every id -1: NaN rows, flag), a zero prime
    (ids -1 from its column on), and 16 heads x 2 (32 rows, 8192 values)."""
    hc = syn.engram_hash_case(seed=9, seqlen=20)
    table = syn.q2k_blocks(syn.rng_for(1001, 9), 500000, 1)
    toks = hc.tokens[10:14].tolist()
    toks[1] = len(hc.token_map) + 5
    _engram_rows_both_ways(hc, table, toks, 10, 1, 500000)
    _engram_rows_both_ways(hc, table, hc.tokens[10:13].tolist(), 10, 0, 500000, bad_prime=True)
    wide = syn.engram_hash_case(seed=10, vocab=512, n_layers=2, max_ngram=3, n_heads=16, seqlen=12)
    _engram_rows_both_ways(wide, table, wide.tokens[4:12].tolist(), 4, 1, 500000)


def _engram_step_both_ways(hc, table_np, wkv_np, h_np, qk_np, eps, tokens, start, layer,
                           n_table_rows, hcs, dim):
    """Decode tokens through engram_step and through engram_rows_q8_1 +
    q2k_mmvq + engram_gate with separate caches and streams h: the h bits,
    cache, kv, q8_1 row and flag must agree at every position; returns the
    last q8_1 row (oracle side) and the last h."""
    tm, mu, pr, of = _hash_tables_dev(hc)
    table = dev(table_np.reshape(-1))
    wkv = dev(wkv_np.reshape(-1))
    qk = dev(qk_np)
    cols = (mu.shape[1] - 1) * pr.shape[-1]
    n_out = (hcs + 1) * dim
    c1 = torch.zeros(len(tokens) + start + 8, dtype=torch.int64, device="cuda")
    c2 = c1.clone()
    if start > 0:
        pre = dev(hc.tokens[:start].astype(np.int32))
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, c1, pre, 0)
        q2.engram_hash(tm, mu, pr, of, hc.pad_id, c2, pre, 0)
    h1, h2 = dev(h_np), dev(h_np)
    need_ws = q2.engram_step_workspace_bytes(mu.shape[1], pr.shape[-1], hcs, dim)
    kv_bytes = (n_out * 4 + 255) // 256 * 256
    need_q8 = q2.q8_1_rows_bytes(1, cols * 256)
    assert need_ws == kv_bytes + need_q8
    ws = torch.full((need_ws + 512,), 0x55, dtype=torch.uint8, device="cuda")
    kv2 = torch.empty((1, n_out), dtype=torch.float32, device="cuda")
    for s_, t in enumerate(tokens):
        pos = start + s_
        tok = dev(np.array([t], dtype=np.int32))
        f1 = torch.zeros(1, dtype=torch.int32, device="cuda")
        f2 = torch.zeros(1, dtype=torch.int32, device="cuda")
        q2.engram_step(tm, mu, pr, of, hc.pad_id, c1, tok, pos, layer, table, n_table_rows, wkv, qk, h1,
                       eps, workspace=ws, err_flag=f1)
        xq2 = q2.engram_rows_q8_1(tm, mu, pr, of, hc.pad_id, c2, tok, pos, layer, table, n_table_rows,
                                  err_flag=f2)
        q2.q2k_mmvq(wkv, xq2, n_out, cols * 256, 1, out=kv2)
        q2.engram_gate(h2, kv2, qk, eps)
        assert torch.equal(h1.view(torch.int32), h2.view(torch.int32)), f"h, position {pos}"
        assert torch.equal(ws[:n_out * 4].view(torch.int32), kv2.view(-1).view(torch.int32)), f"kv, position {pos}"
        assert torch.equal(ws[kv_bytes:kv_bytes + need_q8], xq2[:need_q8]), f"q8_1, position {pos}"
        assert int(f1.item()) == int(f2.item()), f"flag, position {pos}"
    assert torch.equal(c1, c2)
    assert torch.all(ws[need_ws:] == 0x55), "wrote past its workspace"
    return xq2, h1


def test_engram_step_is_the_composition():
    """engram_step on the engram workload (wkv [20480, 2048], hc = 4, dim =
    4096: the rows formed in the run kernel's prologue) after a prefill, both
    hashed layers: every bit of the three calls it replaces; the last token
    also against the oracle end to end (hash, rows, q8_1, the fixed-order
    projection, the gate)."""
    e = syn.engram_step_case()
    hc = syn.engram_hash_case(seqlen=40)
    assert q2.q2k_product_kernel(20480, 2048, 1) == PD
    for layer in (0, 1):
        xq2, h1 = _engram_step_both_ways(hc, e.table, e.wkv, e.h, e.qk, e.eps, hc.tokens[32:40].tolist(), 32,
                                         layer, e.table.shape[0], e.hc, e.dim)
    # the oracle: the hash of the last position, its rows and q8_1, kv, the
    # gate applied once per decoded token to the stream (layer 1 run)
    ids, _ = orc.engram_hash(hc.token_map.tolist(), hc.multipliers.tolist(), hc.primes.tolist(),
                             hc.offsets.tolist(), hc.pad_id, hc.n_heads, [0] * 48, hc.tokens[:40].tolist(), 0)
    h_ref = e.h.astype(np.float64)
    for pos in range(32, 40):
        rows = orc.dequant_rows_bf16_bits(e.table, ids[pos][1])
        oq, od, _ = orc.q8_1_from_bf16_bits(rows.reshape(1, -1))
        kv = orc.mmvq_f32(e.wkv, oq, od).astype(np.float64)
        h_ref = orc.engram_gate(h_ref.astype(np.float32), kv, e.qk, e.eps)
    assert_q8_equal(xq2, rows.reshape(1, -1))
    assert_close(h1.cpu().numpy(), h_ref, "engram step, 8 tokens end to end")


@pytest.mark.parametrize("start", [0, 32])
def test_engram_step_longest_window(start):
    """The longest n-gram window (8 tokens: 7 cached ids per column), two
    heads (14 row ids, k = 3584) and a projection large enough for the rows
    to be formed in the product's prologue ([4096, 3584]: 2048 row steps):
    every bit of the separate calls, from the first positions (windows that
    reach before the sequence) and after a prefill."""
    hc = syn.engram_hash_case(seqlen=48, max_ngram=8, n_heads=2)
    rng = syn.rng_for(1012)
    table = syn.q2k_blocks(rng, 500000, 1)
    dim, hcs = 1024, 3
    wkv = syn.q2k_blocks(rng, (hcs + 1) * dim, 14)
    h, _, qk, eps = syn.gate_case(1012, 1, hcs, dim)
    assert q2.q2k_product_kernel((hcs + 1) * dim, 14 * 256, 1) == PD
    for layer in (0, 1):
        _engram_step_both_ways(hc, table, wkv, h, qk, eps, hc.tokens[start:start + 8].tolist(), start,
                               layer, 500000, hcs, dim)


def test_engram_step_small_and_bad_token():
    """A projection too small for the run kernel (dim 256: the rows launch
    ahead of the product) and a token outside the vocabulary (NaN rows, the
    flag): still the bits of the composition."""
    hc = syn.engram_hash_case(seqlen=24, vocab=512, n_heads=2)
    rng = syn.rng_for(1011)
    table = syn.q2k_blocks(rng, 500000, 1)
    dim, hcs = 256, 2
    wkv = syn.q2k_blocks(rng, (hcs + 1) * dim, 4)
    h, _, qk, eps = syn.gate_case(1011, 1, hcs, dim)
    assert q2.q2k_product_kernel((hcs + 1) * dim, 1024, 1) == PD
    toks = hc.tokens[16:24].tolist()
    toks[3] = 100000                                    # outside the vocabulary
    _engram_step_both_ways(hc, table, wkv, h, qk, eps, toks, 16, 1, 500000, hcs, dim)


# ------------------------------------------------------- m > 8 (MMQ) ------

MMQ_SHAPES = [(300, 1024, 9), (1000, 2048, 16), (130, 7168, 33), (257, 4096, 64), (100, 1280, 20),
              (64, 9216, 12), (40, 2048, 200), (65, 256, 17), (129, 2304, 31), (191, 512, 65),
              (70, 7168, 130), (1, 256, 17), (63, 8192, 47), (64, 10240, 32)]


def mmq_order(m):
    return "running" if m >= 17 else "tree"


@pytest.mark.parametrize("n,k,m", MMQ_SHAPES)
def test_mmq(n, k, m):
    """Past 8 tokens: up to 16 tokens the q2k_mmvq kernels on groups of 8
    (matrix cores for k/256 in {4, 8, 16, 28}, else the packed dots; the
    tree order), from 17 the tile kernel (32 tokens and 64 rows per
    workgroup, any row length; the running-sum order), ragged in rows and
    tokens; bit for bit."""
    rng = syn.rng_for(7100, n, k, m)
    w = syn.q2k_blocks(rng, n, k // 256)
    x = syn.bf16_normal(rng, (m, k), outlier_frac=0.05)
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    y = q2.q2k_mmq(dev(w.reshape(-1)), xq, n, k, m).cpu().numpy()
    assert_product(y, w, oq, od, f"mmq n={n} k={k} m={m}", order=mmq_order(m))


@pytest.mark.parametrize("n,k,m", [(300, 1024, 9), (300, 1024, 16), (100, 1280, 12), (129, 2304, 31),
                                   (191, 512, 65), (70, 7168, 40)])
def test_mmq_block_dots(n, k, m):
    """q2k_block_dots past 8 tokens, the integer sums of the kernel
    q2k_mmq takes, every (token, row, block) bit-exact: groups of 8 on the
    matrix-core kernel (k = 1024) or the packed dots (k = 1280) up to 16
    tokens, the tile kernel's own v_mfma_i32_16x16x32_i8 outputs from 17."""
    rng = syn.rng_for(7110, n, k, m)
    w = syn.q2k_blocks(rng, n, k // 256)
    x = syn.bf16_normal(rng, (m, k), outlier_frac=0.05)
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, _ = assert_q8_equal(xq, x)
    assert q2.q2k_product_kernel(n, k, m) == (PD if k == 1280 else MC)
    dots = q2.q2k_block_dots(dev(w.reshape(-1)), xq, n, k, m).cpu().numpy().astype(np.int64)
    I, M = orc.block_dots(w, oq)
    assert np.array_equal(dots[..., 0], I), "I sums differ"
    assert np.array_equal(dots[..., 1], M), "M sums differ"


@pytest.mark.parametrize("m", [12, 24])
def test_mmq_same_bits_for_every_kernel_choice(m):
    """Every kernel choice gives the same bits past 8 tokens: up to 16 the
    choice picks the kernel and all kernels keep the tree order; from 17 it
    does not apply (the query names the matrix cores whatever the choice)."""
    n, k = 200, 2048
    rng = syn.rng_for(7120, m)
    w = dev(syn.q2k_blocks(rng, n, k // 256).reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(syn.bf16_normal(rng, (m, k), outlier_frac=0.05)))
    outs = []
    for choice in (AUTO, MC, PD):
        with kernel_choice(choice):
            if m >= 17:
                assert q2.q2k_product_kernel(n, k, m) == MC
            outs.append(q2.q2k_mmq(w, xq, n, k, m).cpu().numpy().view(np.uint32))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_mmq_max_tokens():
    """The largest token count q2k_mmq takes (Q2K_MMQ_MAX_M = 4096), ragged rows."""
    n, k, m = 37, 1024, 4096
    rng = syn.rng_for(7150)
    w = syn.q2k_blocks(rng, n, k // 256)
    x = syn.bf16_normal(rng, (m, k), outlier_frac=0.05)
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    y = q2.q2k_mmq(dev(w.reshape(-1)), xq, n, k, m).cpu().numpy()
    assert_product(y, w, oq, od, "mmq m=4096", order="running")


def test_mmq_small_m_is_mmvq():
    case = syn.single_gemv_case(n=8197, k=2048, m=5, seed=7200)
    w = dev(case.w.reshape(-1))
    xq = q2.q8_1_rows(bf16_dev(case.x_bits))
    a = q2.q2k_mmq(w, xq, 8197, 2048, 5).cpu().numpy()
    b = q2.q2k_mmvq(w, xq, 8197, 2048, 5).cpu().numpy()
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


# ------------------------------------------------------- full-size verify ---

@pytest.fixture(scope="module")
def large():
    case = syn.large_verify_case(m=8)
    return case, dev(case.w.reshape(-1))


def test_fused_q8_1_large_verify(large):
    """q8_1_q2k_mmvq on the [32768, 7168] matrix, one token (one launch, the
    quantisation inside the product): the same q8_1 bytes and output bits as
    q8_1_rows + q2k_mmvq, and within tolerance of the oracle on sampled rows."""
    case, w = large
    x = bf16_dev(case.x_bits[:1])
    y, xq = q2.q8_1_q2k_mmvq(w, x, case.n, case.k)
    xq2 = q2.q8_1_rows(x)
    y2 = q2.q2k_mmvq(w, xq2, case.n, case.k, 1)
    need = q2.q8_1_rows_bytes(1, case.k)
    assert torch.equal(xq[:need], xq2[:need])
    assert torch.equal(y.view(torch.int32), y2.view(torch.int32))
    oq, od = assert_q8_equal(xq, case.x_bits[:1])
    assert_product(y.cpu().numpy(), case.w, oq, od, "fused large verify",
                   dense_rows=_sample_rows(case.n, 77, extra=128))


def test_large_mmq_sampled(large):
    """[32768, 7168] against 64 tokens (one 64-token tile per 64 rows):
    sampled rows (every token) bit for bit the running-sum order."""
    case, w = large
    x = syn.bf16_normal(syn.rng_for(1004, 64), (64, case.k), outlier_frac=0.05)
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    y = q2.q2k_mmq(w, xq, case.n, case.k, 64).cpu().numpy()
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(case.n - 64, case.n),
                                     syn.rng_for(5).choice(case.n, 128, replace=False)]))
    assert_product(y[:, rows], case.w[rows], oq, od, "large mmq m=64", order="running")


@pytest.mark.parametrize("m", [1, 3, 8])
def test_large_verify_all_rows(large, m):
    """[32768, 7168] Q2_K against m bf16 tokens with 5% +-20 outliers, in the
    launch configuration the benchmark times: all 32768 rows bit for bit the
    fixed order and within tolerance of the integer route (in 4096-row
    chunks), sampled rows of the dense fp64 definition."""
    case, w = large
    x = case.x_bits[:m]
    xq = q2.q8_1_rows(bf16_dev(x))
    oq, od = assert_q8_equal(xq, x)
    y = q2.q2k_mmvq(w, xq, case.n, case.k, m).cpu().numpy()
    rows = np.unique(np.concatenate([
        np.arange(0, 64), np.arange(case.n - 64, case.n),
        syn.rng_for(4, m).choice(case.n, 384, replace=False)]))
    assert_product(y, case.w, oq, od, f"large m={m}", dense_rows=rows)


def test_swiglu_extreme_gates():
    """Gate values where exp(-g) overflows f32 (g < -88.7) and the far tails."""
    k = 256
    g = np.linspace(-120.0, 120.0, 2 * k, dtype=np.float32).reshape(2, k)
    g[0, :8] = [-1e30, -200.0, -103.9, -88.8, -88.7, -87.0, 0.0, -0.0]
    u = np.full((2, k), 1.5, np.float32)
    u[1] = -3.25
    h, hq = q2.swiglu_q8_1_rows(dev(g), dev(u))
    h_bits = h.view(torch.int16).cpu().numpy().view(np.uint16)
    assert bf16_ulp_distance(h_bits, orc.swiglu_bf16_bits(g, u)).max() <= 1
    assert_q8_equal(hq, h_bits)


# ------------------------------------------------------------ graphs ------

def test_graph_replays_match_eager():
    """Every call is enqueue-only, so a decode sequence captured in a HIP
    graph must give, on each replay, the bits of the same calls run eagerly:
    the fused single and expert products (quantisation and SwiGLU in their
    prologues, the SwiGLU in the gate/up epilogue, 4 tokens quantised one
    per workgroup), the pair, and an engram step (hash + gather + q8_1, wkv
    product, gate on a stream restored inside the graph). Replays alternate
    with eager work and synchronisations."""
    rng = syn.rng_for(4242)
    n, k = 8192, 2048
    w = dev(syn.q2k_blocks(rng, n, k // 256).reshape(-1))
    xb = syn.bf16_normal(rng, (1, k))
    x = bf16_dev(xb)
    x4 = bf16_dev(np.concatenate([xb, syn.bf16_normal(rng, (3, k))]))   # token 0 is x
    n_exp, inter, dim = 6, 2048, 2048
    per_gu = inter * (dim // 256) * 84
    per_d = dim * (inter // 256) * 84
    gate = dev(np.concatenate([syn.q2k_blocks(rng, inter, dim // 256).reshape(-1) for _ in range(n_exp)]))
    up = dev(np.concatenate([syn.q2k_blocks(rng, inter, dim // 256).reshape(-1) for _ in range(n_exp)]))
    down = dev(np.concatenate([syn.q2k_blocks(rng, dim, inter // 256).reshape(-1) for _ in range(n_exp)]))
    ids = dev(np.array([4, 1, 5, 2], dtype=np.int32))
    pc = syn.attention_pair_case(1, seed=4243)
    wa, wb = dev(pc.wa.reshape(-1)), dev(pc.wb.reshape(-1))
    xp = bf16_dev(pc.x_bits)
    e = syn.engram_step_case()
    hc = syn.engram_hash_case(seqlen=40)
    tm, mu, pr, of = _hash_tables_dev(hc)
    cache = torch.zeros(64, dtype=torch.int64, device="cuda")
    q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, dev(hc.tokens[:32]), 0)
    table = dev(e.table.reshape(-1))
    wkv = dev(e.wkv.reshape(-1))
    h0 = dev(e.h)
    qk = dev(e.qk)
    tok = dev(hc.tokens[32:33].astype(np.int32))
    n_out = e.dim * (e.hc + 1)

    outs = {name: None for name in ("y", "xq", "gu", "xq_gu", "yd", "hq", "ya", "yb", "xq_p",
                                    "xq_e", "kv", "h", "y4", "xq4", "gu2", "xq_gu2", "h2", "hq2",
                                    "yd2")}
    outs["y"] = torch.empty((1, n), dtype=torch.float32, device="cuda")
    outs["xq"] = torch.empty(q2.q8_1_rows_bytes(1, k), dtype=torch.uint8, device="cuda")
    outs["gu"] = torch.empty((2, 4, 1, inter), dtype=torch.float32, device="cuda")
    outs["xq_gu"] = torch.empty(q2.q8_1_rows_bytes(1, dim), dtype=torch.uint8, device="cuda")
    outs["yd"] = torch.empty((1, 4, 1, dim), dtype=torch.float32, device="cuda")
    outs["hq"] = torch.empty(q2.q8_1_rows_bytes(4, inter), dtype=torch.uint8, device="cuda")
    outs["ya"] = torch.empty((1, pc.na), dtype=torch.float32, device="cuda")
    outs["yb"] = torch.empty((1, pc.nb), dtype=torch.float32, device="cuda")
    outs["xq_p"] = torch.empty(q2.q8_1_rows_bytes(1, pc.k), dtype=torch.uint8, device="cuda")
    outs["xq_e"] = torch.empty(q2.q8_1_rows_bytes(1, 8 * 256), dtype=torch.uint8, device="cuda")
    outs["kv"] = torch.empty((1, n_out), dtype=torch.float32, device="cuda")
    outs["h"] = torch.empty_like(h0)
    outs["y4"] = torch.empty((4, n), dtype=torch.float32, device="cuda")
    outs["xq4"] = torch.empty(q2.q8_1_rows_bytes(4, k), dtype=torch.uint8, device="cuda")
    outs["gu2"] = torch.empty((2, 4, 1, inter), dtype=torch.float32, device="cuda")
    outs["xq_gu2"] = torch.empty(q2.q8_1_rows_bytes(1, dim), dtype=torch.uint8, device="cuda")
    outs["h2"] = torch.empty((4, inter), dtype=torch.bfloat16, device="cuda")
    outs["hq2"] = torch.empty(q2.q8_1_rows_bytes(4, inter), dtype=torch.uint8, device="cuda")
    outs["yd2"] = torch.empty((1, 4, 1, dim), dtype=torch.float32, device="cuda")

    def seq():
        q2.q8_1_q2k_mmvq(w, x, n, k, xq=outs["xq"], out=outs["y"])
        q2.q8_1_q2k_mmvq_experts([gate, up], per_gu, n_exp, ids, x, inter, dim, xq=outs["xq_gu"],
                                 out=outs["gu"])
        g = outs["gu"][0].view(4, inter)
        u = outs["gu"][1].view(4, inter)
        q2.swiglu_q2k_mmvq_experts([down], per_d, n_exp, ids, g, u, dim, hq=outs["hq"], out=outs["yd"])
        q2.q8_1_q2k_mmvq_pair(wa, pc.na, wb, pc.nb, xp, pc.k, xq=outs["xq_p"], ya=outs["ya"], yb=outs["yb"])
        q2.engram_rows_q8_1(tm, mu, pr, of, hc.pad_id, cache, tok, 32, 1, table, 500000, xq=outs["xq_e"])
        q2.q2k_mmvq(wkv, outs["xq_e"], n_out, 2048, 1, out=outs["kv"])
        outs["h"].copy_(h0)
        q2.engram_gate(outs["h"], outs["kv"], qk, e.eps)
        q2.q8_1_q2k_mmvq(w, x4, n, k, xq=outs["xq4"], out=outs["y4"])
        q2.q8_1_q2k_mmvq_experts_swiglu([gate, up], per_gu, n_exp, ids, x, inter, dim, xq=outs["xq_gu2"],
                                        out=outs["gu2"], h=outs["h2"], hq=outs["hq2"])
        q2.q2k_mmvq_experts([down], per_d, n_exp, ids, outs["hq2"], True, dim, inter, 1, out=outs["yd2"])

    seq()
    torch.cuda.synchronize()
    eager = {name: t.clone() for name, t in outs.items()}
    stream = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        seq()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        seq()
    for rep in range(3):
        for t in outs.values():
            t.zero_()
        q2.q2k_mmvq(w, eager["xq"], n, k, 1)          # unrelated eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for name, t in outs.items():
            assert torch.equal(t.view(torch.uint8), eager[name].view(torch.uint8)), f"{name}, replay {rep}"
    # the two expert routes and the token-per-workgroup quantisation agree
    assert torch.equal(eager["gu2"], eager["gu"]) and torch.equal(eager["yd2"], eager["yd"])
    assert torch.equal(eager["hq2"], eager["hq"])
    assert torch.equal(eager["y4"][:1], eager["y"])
    assert torch.equal(eager["xq4"][:q2.q8_1_rows_bytes(1, k)], eager["xq"])
