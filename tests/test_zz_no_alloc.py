"""engram_step_noalloc (no allocation: kv and the q8_1 row live in the
library's own device array) against engram_step with a caller workspace:
the same h bits, cache and error flag, on two calls in a row, the second on
a smaller step (the array keeps the first call's contents)."""

import numpy as np
import pytest
import torch

import q2_quantized_decode_amd as q2
from q2_quantized_decode_amd import synthetic as syn

pytestmark = pytest.mark.gpu


def _case(dim, hcs, n_heads, seed):
    hc = syn.engram_hash_case(seed=seed, seqlen=24, n_heads=n_heads)
    rng = syn.rng_for(seed, 7)
    cols = 2 * n_heads
    table = syn.q2k_blocks(rng, 500000, 1)
    wkv = syn.q2k_blocks(rng, (hcs + 1) * dim, cols)
    h, _, qk, eps = syn.gate_case(seed, 1, hcs, dim)
    return hc, table, wkv, h, qk, eps


def _run(step, case, pos, layer, noalloc):
    hc, table, wkv, h, qk, eps = case
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    tm, mu, pr, of = d(hc.token_map), d(hc.multipliers), d(hc.primes), d(hc.offsets)
    cache = torch.zeros(64, dtype=torch.int64, device="cuda")
    q2.engram_hash(tm, mu, pr, of, hc.pad_id, cache, d(hc.tokens[:pos].astype(np.int32)), 0)
    tok = d(np.array([hc.tokens[pos]], dtype=np.int32))
    hd = d(h)
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    args = (tm, mu, pr, of, hc.pad_id, cache, tok, pos, layer, d(table), 500000, d(wkv), d(qk), hd, eps)
    if noalloc:
        q2.engram_step_noalloc(*args, err_flag=flag)
    else:
        q2.engram_step(*args, err_flag=flag)
    torch.cuda.synchronize()
    return hd.cpu().numpy(), cache.cpu().numpy(), int(flag.item())


def test_engram_step_noalloc_matches_engram_step_twice():
    assert torch.cuda.is_available()
    big = _case(4096, 4, 4, 1001)        # the engram workload: wkv [20480, 2048], run kernel
    small = _case(512, 2, 2, 1012)       # wkv [1536, 1024], rows launch ahead of the product
    for case, pos, layer in ((big, 20, 1), (small, 17, 0)):
        got = _run(None, case, pos, layer, noalloc=True)
        ref = _run(None, case, pos, layer, noalloc=False)
        assert np.array_equal(got[0].view(np.uint32), ref[0].view(np.uint32)), "h differs"
        assert np.array_equal(got[1], ref[1]), "cache differs"
        assert got[2] == ref[2]
        assert np.all(np.isfinite(got[0]))


def test_engram_step_noalloc_refuses_steps_past_its_array():
    hc = syn.engram_hash_case(seqlen=8)
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    dim = 16384                          # kv of 5 * 16384 values: past the 176 KiB array
    h = torch.zeros((1, 4, dim), dtype=torch.float32, device="cuda")
    with pytest.raises(q2.Q2KError) as e:
        q2.engram_step_noalloc(d(hc.token_map), d(hc.multipliers), d(hc.primes), d(hc.offsets), hc.pad_id,
                               torch.zeros(16, dtype=torch.int64, device="cuda"),
                               d(np.array([1], dtype=np.int32)), 3, 0,
                               torch.zeros(84 * 16, dtype=torch.uint8, device="cuda"), 16,
                               torch.zeros(5 * dim * 8 * 84, dtype=torch.uint8, device="cuda"),
                               torch.zeros((4, dim), dtype=torch.float32, device="cuda"), h, 1e-6)
    assert e.value.code == -3 and "scratch array" in str(e.value)
