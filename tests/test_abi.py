"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch.

The pointers passed here are never dereferenced: every call below fails
validation, which runs before any HIP call."""

import ctypes
import os
import re

import pytest

import q2_quantized_decode_amd as q2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "q2k_decode.h")

EINVAL, ESHAPE, ESPACE, EALIGN = -1, -2, -3, -4
P = 0x7f0000000000          # a 256-byte aligned fake device address
Q = 0x7f0001000000


def _declared():
    text = open(HEADER).read()
    return re.findall(r"Q2K_API\s+[\w\s\*]+?\b(\w+)\s*\(", text)


@pytest.fixture(scope="module")
def L():
    return q2.lib()


def test_header_symbols_exported(L):
    names = _declared()
    assert set(names) == set(q2.SIGNATURES), names
    for n in names:
        assert hasattr(L, n)


def test_version_and_sizes(L):
    assert L.q2k_abi_version() == 5
    assert L.q8_1_rows_bytes(1, 1024) == 1280
    assert L.q8_1_rows_bytes(8, 7168) == 8 * 8960
    assert L.q8_1_rows_bytes(0, 1024) == 0
    assert L.q8_1_rows_bytes(1, 100) == 0
    assert L.q8_1_rows_bytes(1, -256) == 0


def test_product_kernel_choice(L):
    """The kernel choice is host state only (no launch): unknown values are
    refused, valid ones return the previous choice."""
    prev = L.q2k_set_product_kernel(q2.KERNEL_AUTO)
    assert prev in (q2.KERNEL_AUTO, q2.KERNEL_PACKED_DOTS)
    assert L.q2k_set_product_kernel(3) == EINVAL
    assert "unknown choice" in _err(L)
    assert L.q2k_set_product_kernel(-1) == EINVAL
    assert L.q2k_set_product_kernel(q2.KERNEL_MATRIX_CORES) == q2.KERNEL_AUTO
    assert L.q2k_set_product_kernel(q2.KERNEL_PACKED_DOTS) == q2.KERNEL_MATRIX_CORES
    assert L.q2k_set_product_kernel(prev) == q2.KERNEL_PACKED_DOTS


def test_product_kernel_query(L):
    """q2k_product_kernel reports, on the host, which kernel a single-matrix
    product of a shape runs: the measured cost model under the automatic
    choice (the large verify matrix: packed dots at one token, the matrix
    cores at eight; rows of 5 blocks have no matrix-core tile), or the forced
    choice."""
    MC, PD = q2.KERNEL_MATRIX_CORES, q2.KERNEL_PACKED_DOTS
    assert L.q2k_product_kernel(0, 1024, 1) == ESHAPE
    assert L.q2k_product_kernel(10, 1000, 1) == ESHAPE
    assert L.q2k_product_kernel(10, 1024, 0) == ESHAPE
    assert L.q2k_product_kernel(10, 1024, 4097) == ESHAPE
    prev = L.q2k_set_product_kernel(q2.KERNEL_AUTO)
    try:
        assert L.q2k_product_kernel(32768, 7168, 1) == PD
        assert L.q2k_product_kernel(32768, 7168, 8) == MC
        assert L.q2k_product_kernel(100, 1280, 8) == PD
        assert L.q2k_product_kernel(300, 1024, 20) == MC
        L.q2k_set_product_kernel(PD)
        assert L.q2k_product_kernel(32768, 7168, 8) == PD
        L.q2k_set_product_kernel(MC)
        assert L.q2k_product_kernel(10, 1024, 2) == MC
        assert L.q2k_product_kernel(10, 1024, 1) == PD
        assert L.q2k_product_kernel(10, 1280, 3) == PD
    finally:
        L.q2k_set_product_kernel(prev)


def _err(L):
    return L.q2k_last_error().decode()


def test_q8_1_rows_validation(L):
    assert L.q8_1_rows(None, 1024, P, 1280, 1, 1024, None) == EINVAL
    assert L.q8_1_rows(P, 1024, Q, 1280, 1, 1000, None) == ESHAPE
    assert "multiple of 256" in _err(L)
    assert L.q8_1_rows(P, 1024, Q, 1280, 0, 1024, None) == ESHAPE
    assert L.q8_1_rows(P, 512, Q, 1280, 1, 1024, None) == ESHAPE       # stride < k
    assert L.q8_1_rows(P + 2, 1024, Q, 1280, 1, 1024, None) == EALIGN
    assert L.q8_1_rows(P, 1028, Q, 2560, 2, 1024, None) == EALIGN     # stride % 8
    assert L.q8_1_rows(P, 1024, Q, 1279, 1, 1024, None) == ESPACE
    assert L.q8_1_rows(P, 1024, P + 16, 1280, 1, 1024, None) == EINVAL  # overlap


def test_fused_q8_1_mmvq_validation(L):
    """q8_1_q2k_mmvq takes both calls' checks, before any launch."""
    X, XQ, Y = 0x10000000, 0x20000000, 0x30000000
    f = L.q8_1_q2k_mmvq
    assert f(None, X, 1024, XQ, 1280, Y, 256, 1024, 1, None) == EINVAL
    assert f(P, None, 1024, XQ, 1280, Y, 256, 1024, 1, None) == EINVAL
    assert f(P, X, 1024, None, 1280, Y, 256, 1024, 1, None) == EINVAL
    assert f(P, X, 1024, XQ, 1280, None, 256, 1024, 1, None) == EINVAL
    assert f(P, X, 1000, XQ, 1250, Y, 256, 1000, 1, None) == ESHAPE
    assert f(P, X, 1024, XQ, 1280 * 9, Y, 256, 1024, 9, None) == ESHAPE
    assert f(P, X, 1024, XQ, 1280, Y, 0, 1024, 1, None) == ESHAPE
    assert f(P, X, 512, XQ, 1280, Y, 256, 1024, 1, None) == ESHAPE          # stride < k
    assert f(P, X + 2, 1024, XQ, 1280, Y, 256, 1024, 1, None) == EALIGN
    assert f(P, X, 1028, XQ, 2560, Y, 256, 1024, 2, None) == EALIGN         # stride % 8
    assert f(P, X, 1024, XQ + 4, 1280, Y, 256, 1024, 1, None) == EALIGN
    assert f(P, X, 1024, XQ, 1279, Y, 256, 1024, 1, None) == ESPACE
    assert "1280 needed" in _err(L)
    assert f(P, X, 1024, X + 1024, 1280, Y, 256, 1024, 1, None) == EINVAL  # xq inside x
    assert f(P, X, 1024, XQ, 1280, XQ + 64, 256, 1024, 1, None) == EINVAL  # y inside xq
    assert f(P, X, 1024, XQ, 1280, X + 16, 256, 1024, 1, None) == EINVAL   # y inside x


def test_fused_q8_1_experts_validation(L):
    import ctypes
    X, XQ, Y, IDS = 0x10000000, 0x20000000, 0x30000000, 0x40000000
    arr = (ctypes.c_void_p * 2)(P, Q)
    f = L.q8_1_q2k_mmvq_experts
    stride = 256 * 4 * 84
    args = lambda **kw: [kw.get("bases", arr), kw.get("nb", 2), kw.get("stride", stride), 4,
                         kw.get("ids", IDS), 8, kw.get("x", X), kw.get("xs", 1024), kw.get("xq", XQ),
                         kw.get("xqb", 1280), kw.get("y", Y), 256, kw.get("k", 1024), kw.get("m", 1),
                         None, None]
    assert f(*args(x=None)) == EINVAL
    assert f(*args(xq=None)) == EINVAL
    assert f(*args(ids=None)) == EINVAL
    assert f(*args(nb=5)) == ESHAPE
    assert f(*args(k=1000, xs=1000)) == ESHAPE
    assert f(*args(m=9, xqb=1280 * 9)) == ESHAPE
    assert f(*args(stride=100)) == ESHAPE
    assert f(*args(xs=512)) == ESHAPE
    assert f(*args(x=X + 2)) == EALIGN
    assert f(*args(xq=XQ + 4)) == EALIGN
    assert f(*args(xqb=1279)) == ESPACE
    assert f(*args(xq=X + 512)) == EINVAL            # xq inside x
    assert f(*args(y=X + 16)) == EINVAL             # y inside x
    assert f(*args(xq=IDS)) == EINVAL               # xq over the ids


def test_fused_gate_up_swiglu_validation(L):
    import ctypes
    X, XQ, Y, IDS, H, HQ = 0x10000000, 0x20000000, 0x30000000, 0x40000000, 0x50000000, 0x60000000
    arr = (ctypes.c_void_p * 2)(P, Q)
    f = L.q8_1_q2k_mmvq_experts_swiglu
    stride = 256 * 4 * 84
    args = lambda **kw: [kw.get("bases", arr), kw.get("stride", stride), 4, kw.get("ids", IDS), 8,
                         kw.get("x", X), kw.get("xq", XQ), kw.get("xqb", 1280), kw.get("y", Y),
                         kw.get("h", H), kw.get("hq", HQ), kw.get("hqb", 8 * 320), kw.get("n", 256),
                         kw.get("k", 1024), None, None]
    assert f(*args(x=None)) == EINVAL
    assert f(*args(xq=None)) == EINVAL
    assert f(*args(hq=None)) == EINVAL
    assert f(*args(ids=None)) == EINVAL
    assert f(*args(k=1000)) == ESHAPE
    assert f(*args(n=320)) == ESHAPE                # h is a Q2_K product's input
    assert f(*args(stride=100)) == ESHAPE
    assert f(*args(x=X + 2)) == EALIGN
    assert f(*args(hq=HQ + 8)) == EALIGN
    assert f(*args(h=H + 2)) == EALIGN
    assert f(*args(xqb=1279)) == ESPACE
    assert f(*args(hqb=8 * 320 - 1)) == ESPACE
    assert f(*args(hq=X + 64)) == EINVAL             # hq inside x
    assert f(*args(h=Y + 64)) == EINVAL              # h inside y
    assert f(*args(hq=IDS)) == EINVAL                # hq over the ids
    assert f(*args(xq=HQ + 256)) == EINVAL           # xq inside hq
    assert f(*args(h=P + 64)) == EINVAL              # h inside the gate set
    assert f(*args(y=X + 16)) == EINVAL              # y inside x


def test_fused_swiglu_experts_validation(L):
    import ctypes
    G, U, HQ, Y, IDS = 0x10000000, 0x11000000, 0x20000000, 0x30000000, 0x40000000
    arr = (ctypes.c_void_p * 1)(P,)
    f = L.swiglu_q2k_mmvq_experts
    stride = 4096 * 8 * 84
    args = lambda **kw: [arr, 1, stride, 16, kw.get("ids", IDS), 8, kw.get("g", G), kw.get("u", U),
                         kw.get("hq", HQ), kw.get("hqb", 8 * 2560), kw.get("y", Y), 4096,
                         kw.get("k", 2048), None, None]
    assert f(*args(g=None)) == EINVAL
    assert f(*args(u=None)) == EINVAL
    assert f(*args(hq=None)) == EINVAL
    assert f(*args(k=2000)) == ESHAPE
    assert f(*args(g=G + 4)) == EALIGN
    assert f(*args(hq=HQ + 8)) == EALIGN
    assert f(*args(hqb=8 * 2560 - 1)) == ESPACE
    assert f(*args(hq=G + 64)) == EINVAL             # hq inside g
    assert f(*args(y=U + 64)) == EINVAL              # y inside u
    assert f(*args(hq=IDS)) == EINVAL


def test_fused_q8_1_pair_validation(L):
    X, XQ, YA, YB = 0x10000000, 0x20000000, 0x30000000, 0x31000000
    f = L.q8_1_q2k_mmvq_pair
    args = lambda **kw: [P, kw.get("ya", YA), 1024, Q, kw.get("yb", YB), 512, kw.get("x", X),
                         kw.get("xs", 4096), kw.get("xq", XQ), kw.get("xqb", 5120), kw.get("k", 4096),
                         kw.get("m", 1), None]
    assert f(*args(x=None)) == EINVAL
    assert f(*args(xq=None)) == EINVAL
    assert f(*args(k=4000, xs=4000)) == ESHAPE
    assert f(*args(m=9)) == ESHAPE
    assert f(*args(xs=2048)) == ESHAPE
    assert f(*args(x=X + 8)) == EALIGN
    assert f(*args(xqb=5119)) == ESPACE
    assert f(*args(xq=X + 16)) == EINVAL      # xq inside x
    assert f(*args(ya=X)) == EINVAL           # an output over x
    assert f(*args(yb=YA + 4)) == EINVAL      # ya and yb overlap


def test_engram_rows_q8_1_validation(L):
    TM, MU, PR, OF, C, T, TB, XQ = (0x10000000 + 0x1000000 * i for i in range(8))
    f = L.engram_rows_q8_1
    args = lambda **kw: [kw.get("tm", TM), 4096, MU, PR, OF, kw.get("nl", 2), kw.get("ng", 3),
                         kw.get("nh", 4), 0, kw.get("c", C), kw.get("cl", 64), kw.get("t", T),
                         kw.get("pos", 10), kw.get("layer", 1), kw.get("tb", TB), 500000,
                         kw.get("ids", None), kw.get("rows", None), kw.get("xq", XQ),
                         kw.get("xqb", 2560), None, None]
    assert f(*args(tm=None)) == EINVAL
    assert f(*args(t=None)) == EINVAL
    assert f(*args(xq=None)) == EINVAL
    assert f(*args(layer=2)) == ESHAPE
    assert f(*args(nh=17)) == ESHAPE                 # 2 * 17 = 34 row ids > 32
    assert f(*args(pos=64)) == ESHAPE
    assert f(*args(ng=9)) == ESHAPE
    assert f(*args(c=C + 4)) == EALIGN
    assert f(*args(xq=XQ + 8)) == EALIGN
    assert f(*args(xqb=2559)) == ESPACE
    assert f(*args(xq=C + 64)) == EINVAL             # xq inside the cache
    assert f(*args(rows=XQ + 16)) == EINVAL          # rows over xq
    assert f(*args(ids=TB)) == EINVAL                # ids over the table


def test_engram_step_validation(L):
    """engram_step refuses bad arguments on the host before any launch; the
    workspace is sized by engram_step_workspace_bytes (kv rounded to 256
    bytes, then the q8_1 row of 256 * cols values)."""
    TM, MU, PR, OF, C, T, TB, W, QK, H, WS = (0x10000000 + 0x1000000 * i for i in range(11))
    need = L.engram_step_workspace_bytes(3, 4, 4, 4096)
    assert need == (5 * 4096 * 4 + 255) // 256 * 256 + 2048 * 5 // 4
    assert L.engram_step_workspace_bytes(3, 17, 4, 4096) == 0        # 34 row ids
    assert L.engram_step_workspace_bytes(3, 4, 5, 4096) == 0
    f = L.engram_step
    args = lambda **kw: [kw.get("tm", TM), 4096, MU, PR, OF, kw.get("nl", 2), kw.get("ng", 3),
                         kw.get("nh", 4), 0, kw.get("c", C), kw.get("cl", 64), kw.get("t", T),
                         kw.get("pos", 10), kw.get("layer", 1), kw.get("tb", TB), 500000,
                         kw.get("w", W), kw.get("qk", QK), kw.get("h", H), kw.get("hc", 4),
                         kw.get("dim", 4096), kw.get("eps", 1e-6), kw.get("ws", WS),
                         kw.get("wsb", need), None, None]
    assert f(*args(tm=None)) == EINVAL
    assert f(*args(w=None)) == EINVAL
    assert f(*args(ws=None)) == EINVAL
    assert f(*args(layer=2)) == ESHAPE
    assert f(*args(nh=17)) == ESHAPE
    assert f(*args(pos=64)) == ESHAPE
    assert f(*args(hc=5)) == ESHAPE
    assert f(*args(dim=0)) == ESHAPE
    assert f(*args(eps=-1.0)) == ESHAPE
    assert f(*args(ws=WS + 16)) == EALIGN
    assert f(*args(w=W + 2)) == EALIGN
    assert f(*args(wsb=need - 1)) == ESPACE
    assert f(*args(ws=C + 256)) == EINVAL              # workspace inside the cache
    assert f(*args(h=W + 64)) == EINVAL                # h inside wkv
    assert f(*args(ws=H + 256)) == EINVAL              # workspace over h


def test_engram_step_noalloc_checks_before_any_hip_call(L):
    """engram_step_noalloc runs every argument check before it looks up its
    array's device address (a HIP call; none here, there is no GPU), and
    refuses steps whose workspace would pass Q2K_ENGRAM_SCRATCH_BYTES."""
    TM, MU, PR, OF, C, T, TB, W, QK, H = (0x10000000 + 0x1000000 * i for i in range(10))
    f = L.engram_step_noalloc
    args = lambda **kw: [kw.get("tm", TM), 4096, MU, PR, OF, 2, 3, 4, 0, C, 64, T, 10, 1, TB, 500000,
                         W, QK, kw.get("h", H), kw.get("hc", 4), kw.get("dim", 4096), 1e-6, None, None]
    assert f(*args(tm=None)) == EINVAL
    assert f(*args(hc=5)) == ESHAPE
    assert f(*args(dim=16384)) == ESPACE
    assert "scratch array" in _err(L)
    assert f(*args(h=W + 64)) == EINVAL
    assert L.engram_step_workspace_bytes(3, 16, 4, 8192) <= 176 * 1024   # the stated limit fits


def test_mmvq_validation(L):
    assert L.q2k_mmvq(None, Q, P, 256, 1024, 1, None) == EINVAL
    assert L.q2k_mmvq(P, Q, 0x100, 256, 1000, 1, None) == ESHAPE
    assert L.q2k_mmvq(P, Q, 0x100, 256, 1024, 9, None) == ESHAPE
    assert "1..8" in _err(L)
    assert L.q2k_mmvq(P, Q, 0x100, 256, 1024, 0, None) == ESHAPE
    assert L.q2k_mmvq(P, Q, 0x100, 0, 1024, 1, None) == ESHAPE
    assert L.q2k_mmvq(P + 2, Q, 0x100, 256, 1024, 1, None) == EALIGN
    assert L.q2k_mmvq(P, Q + 4, 0x100, 256, 1024, 1, None) == EALIGN
    assert L.q2k_mmvq(P, Q, P + 100, 256, 1024, 1, None) == EINVAL    # y inside w


def test_pair_validation(L):
    assert L.q2k_mmvq_pair(P, 0x100, 1024, None, 0x10000, 512, Q, 4096, 1, None) == EINVAL
    assert L.q2k_mmvq_pair(P, 0x100, 1024, P, 0x200, 512, Q, 4096, 1, None) == EINVAL  # ya/yb overlap
    assert L.q2k_mmvq_pair(P, 0x100, 1024, P, 0x100000, 512, Q, 4096, 9, None) == ESHAPE


def test_grouped_validation(L):
    # w at P: 8 x 1024 rows of 2048 (5.5 MB); xq at Q; y far above both
    y = 0x40000000
    assert L.q2k_mmvq_grouped(P, Q, y, 0, 1024, 2048, 4, None) == ESHAPE
    assert L.q2k_mmvq_grouped(P, Q, y, 8, 0, 2048, 4, None) == ESHAPE
    assert L.q2k_mmvq_grouped(P, Q, y, 8, 1024, 2000, 4, None) == ESHAPE
    assert L.q2k_mmvq_grouped(P, Q, y, 8, 1024, 2048, 9, None) == ESHAPE
    assert L.q2k_mmvq_grouped(P, Q, y, 1 << 16, 1 << 16, 2048, 1, None) == ESHAPE   # rows >= 2^31
    assert L.q2k_mmvq_grouped(None, Q, y, 8, 1024, 2048, 4, None) == EINVAL
    assert L.q2k_mmvq_grouped(P, None, y, 8, 1024, 2048, 4, None) == EINVAL
    assert L.q2k_mmvq_grouped(P + 2, Q, y, 8, 1024, 2048, 4, None) == EALIGN
    assert L.q2k_mmvq_grouped(P, Q + 4, y, 8, 1024, 2048, 4, None) == EALIGN
    assert L.q2k_mmvq_grouped(P, Q, P + 64, 8, 1024, 2048, 4, None) == EINVAL    # y inside w


def test_engram_hash_validation(L):
    T = 0x7f0002000000

    def call(**kw):
        a = dict(tm=T, vocab=4096, mult=T + 0x100000, primes=T + 0x200000, offs=T + 0x300000,
                 nl=2, ng=3, nh=4, pad=0, cache=T + 0x400000, cache_len=128, ids=T + 0x500000,
                 seqlen=64, start=0, out=T + 0x600000)
        a.update(kw)
        return L.engram_hash(a["tm"], a["vocab"], a["mult"], a["primes"], a["offs"], a["nl"],
                             a["ng"], a["nh"], a["pad"], a["cache"], a["cache_len"], a["ids"],
                             a["seqlen"], a["start"], a["out"], None, None)
    assert call(tm=None) == EINVAL
    assert call(vocab=0) == ESHAPE
    assert call(nl=0) == ESHAPE
    assert call(ng=1) == ESHAPE
    assert call(ng=9) == ESHAPE
    assert call(nh=0) == ESHAPE
    assert call(seqlen=0) == ESHAPE
    assert call(start=100) == ESHAPE                  # 100 + 64 > 128
    assert call(start=-1) == ESHAPE
    assert call(cache=T + 0x400004) == EALIGN
    assert call(ids=T + 0x500002) == EALIGN
    assert call(out=T + 0x400000) == EINVAL           # out on the cache


def test_dequant_rows_q8_1_validation(L):
    T, X, O, I = 0x7f0002000000, 0x7f0003000000, 0x7f0004000000, 0x7f0005000000
    need = L.q8_1_rows_bytes(1, 8 * 256)
    assert L.q2k_dequant_rows_q8_1(None, 10, I, 8, O, X, need, None, None) == EINVAL
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 8, O, None, need, None, None) == EINVAL
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 0, O, X, need, None, None) == ESHAPE
    assert L.q2k_dequant_rows_q8_1(T, 0, I, 8, O, X, need, None, None) == ESHAPE
    assert L.q2k_dequant_rows_q8_1(T, 4, None, 8, O, X, need, None, None) == ESPACE   # rows past the table
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 8, O, X, need - 1, None, None) == ESPACE
    assert "needed" in _err(L)
    assert L.q2k_dequant_rows_q8_1(T + 2, 10, I, 8, O, X, need, None, None) == EALIGN
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 8, O + 8, X, need, None, None) == EALIGN
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 8, O, X + 8, need, None, None) == EALIGN
    assert L.q2k_dequant_rows_q8_1(T, 10, I + 4, 8, O, X, need, None, None) == EALIGN
    assert L.q2k_dequant_rows_q8_1(T, 1000, I, 8, O, T + 256, need, None, None) == EINVAL   # xq in the table
    assert L.q2k_dequant_rows_q8_1(T, 10, I, 8, X + 1024, X, need, None, None) == EINVAL    # out on xq


def test_gemv_bf16_validation(L):
    assert L.q2k_gemv_bf16(None, Q, 1024, 0x100, 256, 1024, 1, None) == EINVAL
    assert L.q2k_gemv_bf16(P, Q, 1024, 0x100, 256, 1000, 1, None) == ESHAPE
    assert L.q2k_gemv_bf16(P, Q, 1024, 0x100, 256, 1024, 9, None) == ESHAPE
    assert L.q2k_gemv_bf16(P, Q, 512, 0x100, 256, 1024, 1, None) == ESHAPE      # stride < k
    assert L.q2k_gemv_bf16(P, Q + 8, 1024, 0x100, 256, 1024, 1, None) == EALIGN
    assert L.q2k_gemv_bf16(P, Q, 1028, 0x100, 256, 1024, 2, None) == EALIGN     # stride % 8
    assert L.q2k_gemv_bf16(P, Q, 1024, P + 64, 256, 1024, 1, None) == EINVAL    # y inside w


def test_mmq_validation(L):
    assert L.q2k_mmq(None, Q, 0x100, 256, 1024, 16, None) == EINVAL
    assert L.q2k_mmq(P, Q, 0x100, 256, 1000, 16, None) == ESHAPE
    assert L.q2k_mmq(P, Q, 0x100, 256, 1024, 0, None) == ESHAPE
    assert L.q2k_mmq(P, Q, 0x100, 256, 1024, 4097, None) == ESHAPE
    assert "4096" in _err(L)
    assert L.q2k_mmq(P, Q + 4, 0x100, 256, 1024, 16, None) == EALIGN
    assert L.q2k_mmq(P, Q, P + 64, 256, 1024, 16, None) == EINVAL    # y inside w


def test_experts_validation(L):
    arr = (ctypes.c_void_p * 2)(P, Q)
    ok = dict(stride=1024 * 16 * 84, n_experts=4, ids=0x200000, n_ids=8, xq=0x300000,
              y=0x400000, n=1024, k=4096, m=1)

    def call(**kw):
        a = dict(ok, **kw)
        return L.q2k_mmvq_experts(arr, kw.get("n_bases", 2), a["stride"], a["n_experts"],
                                  a["ids"], a["n_ids"], a["xq"], kw.get("x_per_id", 0), a["y"],
                                  a["n"], a["k"], a["m"], None, None)
    assert call(n_bases=0) == ESHAPE
    assert call(n_bases=5) == ESHAPE
    assert call(stride=100) == ESHAPE
    assert call(stride=1024 * 16 * 84 + 2) == EALIGN
    assert call(n_ids=0) == ESHAPE
    assert call(n_ids=65) == ESHAPE
    assert call(x_per_id=2) == ESHAPE
    assert call(ids=0) == EINVAL
    assert call(k=4000) == ESHAPE
    assert call(n_experts=0) == ESHAPE
    assert L.q2k_mmvq_experts(None, 1, ok["stride"], 4, 0x200000, 8, 0x300000, 0, 0x400000,
                              1024, 4096, 1, None, None) == EINVAL


def test_swiglu_dequant_gate_dots_validation(L):
    assert L.swiglu_q8_1_rows(P, Q, None, 0x10000000, 100, 8, 2048, None) == ESPACE
    assert L.swiglu_q8_1_rows(P, Q, None, 0x10000000, 8 * 2560, 8, 2000, None) == ESHAPE
    assert L.swiglu_q8_1_rows(P + 4, Q, None, 0x10000000, 8 * 2560, 8, 2048, None) == EALIGN
    assert L.swiglu_q8_1_rows(None, Q, None, 0x10000000, 8 * 2560, 8, 2048, None) == EINVAL
    assert L.q2k_dequant_rows(None, 10, None, 8, Q, None, None) == EINVAL
    assert L.q2k_dequant_rows(P, 4, None, 8, Q, None, None) == ESPACE
    assert L.q2k_dequant_rows(P, 10, None, 0, Q, None, None) == ESHAPE
    assert L.q2k_dequant_rows(P + 2, 10, None, 8, Q, None, None) == EALIGN
    assert L.engram_gate(P, Q, 0x10000000, 1, 5, 4096, 1e-6, None) == ESHAPE
    assert L.engram_gate(P, Q, 0x10000000, 1, 0, 4096, 1e-6, None) == ESHAPE
    assert "1..4" in _err(L)
    assert L.engram_gate(P, Q, 0x10000000, 0, 4, 4096, 1e-6, None) == ESHAPE
    assert L.engram_gate(P, P + 64, 0x10000000, 1, 4, 4096, 1e-6, None) == EINVAL
    assert L.engram_gate(P, Q, 0x10000000, 1, 4, 4096, -1.0, None) == ESHAPE
    assert L.q2k_block_dots(P, Q, 0x10000000, 256, 1024, 4097, None) == ESHAPE
    assert L.q2k_block_dots(P, Q, 0x10000000, 256, 1024, 0, None) == ESHAPE
    assert L.q2k_block_dots(P, Q, 0x10000004, 256, 1024, 1, None) == EALIGN


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros((1, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        q2.q8_1_rows(x)


def test_engram_bindings_refuse_mis_shaped_tables():
    """The kernels index the hash tables and the wkv matrix from the shapes
    the binding derives (n_layers, max_ngram, n_heads, hc, dim): tables of
    another shape, or a wkv of another size, are refused before any call."""
    import numpy as np
    import torch

    from q2_quantized_decode_amd import synthetic as syn
    hc = syn.engram_hash_case(seqlen=8)
    e = syn.engram_step_case()
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    cache = torch.zeros(16, dtype=torch.int64)
    tok = torch.zeros(1, dtype=torch.int32)
    good = (t(hc.token_map), t(hc.multipliers), t(hc.primes), t(hc.offsets))
    flat = (good[0], good[1], t(hc.primes.reshape(hc.primes.shape[0], -1)), good[3])
    for fn in (q2.engram_step, q2.engram_step_noalloc):
        with pytest.raises(ValueError, match="primes"):
            fn(*flat, hc.pad_id, cache, tok, 3, 0, t(e.table.reshape(-1)), e.table.shape[0],
               t(e.wkv.reshape(-1)), t(e.qk), t(e.h), 1e-6)
        with pytest.raises(ValueError, match="wkv"):
            fn(*good, hc.pad_id, cache, tok, 3, 0, t(e.table.reshape(-1)), e.table.shape[0],
               t(e.wkv.reshape(-1)[: 84 * 1000]), t(e.qk), t(e.h), 1e-6)
        with pytest.raises(ValueError, match="table"):
            fn(*good, hc.pad_id, cache, tok, 3, 0, t(e.table.reshape(-1)[:84]), e.table.shape[0],
               t(e.wkv.reshape(-1)), t(e.qk), t(e.h), 1e-6)
    with pytest.raises(ValueError, match="primes"):
        q2.engram_hash(*flat, hc.pad_id, cache, t(hc.tokens[:4].astype(np.int32)), 0)
    with pytest.raises(ValueError, match="primes"):
        q2.engram_rows_q8_1(*flat, hc.pad_id, cache, tok, 3, 0, t(e.table.reshape(-1)), e.table.shape[0])
