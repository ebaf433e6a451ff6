"""GPU parity of the token permute into the masked-GEMM layout (HALOps "GEMM"
page, prefill_permute_to_masked_gemm section) against the oracle.

The order of rows inside an expert is free (the device's follows atomic
arrival), so the tests compare what is unique -- counts, which pairs were
placed (all of them unless an expert overflows; then how many), the bytes of
every placed row and of its scale row -- and check that the map is valid:
each expert's rows are exactly 0 .. count-1, and rows past the count keep
their sentinel."""
import numpy as np
import pytest
import torch

import fp4_gemm_moe_amd as hq
from oracle import permute as P
from tests import _gpu as U

pytestmark = pytest.mark.gpu

SENT = 0xA5


def _run(x_rows, scale, ids, E, M, hidden, mode, dev):
    T, RB = x_rows.shape
    x = U.dev_u8(x_rows, dev)
    sc = torch.from_numpy(np.ascontiguousarray(scale)).to(dev)
    tid = torch.from_numpy(np.ascontiguousarray(ids, dtype=np.int64)).to(dev)
    px = torch.full((E * M, RB), SENT, dtype=torch.uint8, device=dev)
    osf = torch.full((E, M, hidden // 32), SENT, dtype=torch.uint8, device=dev)
    imap = torch.full((T, ids.shape[1]), -7, dtype=torch.int32, device=dev)
    nums = torch.full((E,), 12345, dtype=torch.int32, device=dev)
    hq.hq_prefill_permute_to_masked_gemm(x, sc, tid, E, M, px, osf, imap, nums, hidden)
    torch.cuda.synchronize()
    return U.host_u8(px), U.host_u8(osf), imap.cpu().numpy(), nums.cpu().numpy()


def _check(x_rows, scale, ids, E, M, hidden, mode, got, what):
    px, osf, imap, nums = got
    want = P.permute_to_masked(x_rows, scale, ids, E, M, hidden, mode)
    sf = P.expand_scales(scale, hidden, mode)
    assert np.array_equal(nums, want["counts"]), f"{what}: counts"
    valid = (ids >= 0) & (ids < E)
    assert np.all(imap[~valid] == -1), f"{what}: unassigned pairs must map to -1"
    for e in range(E):
        sel = ids == e
        rows = imap[sel]
        placed = rows[rows >= 0]
        # every pair placed unless the expert overflows, then exactly M of them
        assert placed.size == min(int(sel.sum()), M), f"{what}: expert {e} placed {placed.size}"
        assert np.array_equal(np.sort(placed), np.arange(nums[e])), f"{what}: expert {e} rows not 0..count-1"
        assert np.all(rows >= -1), f"{what}: expert {e} map values"
        for t, j in zip(*np.nonzero(sel & (imap >= 0))):
            r = e * M + imap[t, j]
            assert np.array_equal(px[r], x_rows[t]), f"{what}: row of ({t},{j})"
            assert np.array_equal(osf[e, imap[t, j]], sf[t]), f"{what}: scales of ({t},{j})"
        assert np.all(px[e * M + nums[e]:(e + 1) * M] == SENT), f"{what}: expert {e} rows past the count written"
        assert np.all(osf[e, nums[e]:] == SENT), f"{what}: expert {e} scale rows past the count written"


def test_page_example_bf16_broadcast():
    """The section's example: 1024 tokens of hidden 2048 (BF16 rows), top-8
    of 16 experts, max_token_num 1024, int32 broadcast scales."""
    dev = U.require_gpu()
    rng = np.random.default_rng(11)
    T, H, topk, E, M = 1024, 2048, 8, 16, 1024
    U.banner(f"permute bf16 broadcast T={T} H={H} topk={topk} E={E} M={M}")
    x = rng.integers(0, 256, (T, 2 * H), dtype=np.uint8)
    ids = rng.integers(0, E, (T, topk)).astype(np.int64)
    scale = rng.integers(0, 2 ** 32, (T, H // 512), dtype=np.uint64).astype(np.uint32).view(np.int32)
    got = _run(x, scale, ids, E, M, H, P.BROADCAST, dev)
    _check(x, scale, ids, E, M, H, P.BROADCAST, got, "page example")


def test_fp8_direct_with_unassigned_ids():
    dev = U.require_gpu()
    rng = np.random.default_rng(12)
    T, H, topk, E, M = 300, 1152, 3, 5, 256
    U.banner(f"permute fp8 direct T={T} H={H} ids incl. -1 and >= E")
    x = rng.integers(0, 256, (T, H), dtype=np.uint8)
    ids = rng.integers(-1, E + 2, (T, topk)).astype(np.int64)
    scale = rng.integers(0, 256, (T, H // 32), dtype=np.uint8)
    got = _run(x, scale, ids, E, M, H, P.DIRECT, dev)
    _check(x, scale, ids, E, M, H, P.DIRECT, got, "fp8 direct")


def test_overflowing_expert_and_fp4_rows():
    """Packed FP4 rows (hidden / 2 bytes); expert 0 receives more pairs than
    max_token_num: exactly max_token_num of them are placed."""
    dev = U.require_gpu()
    rng = np.random.default_rng(13)
    T, H, topk, E, M = 400, 1024, 2, 3, 128
    U.banner(f"permute fp4 overflow T={T} M={M}")
    x = rng.integers(0, 256, (T, H // 2), dtype=np.uint8)
    ids = np.stack([np.zeros(T, np.int64), rng.integers(1, E, T)], axis=1)
    scale = rng.integers(0, 2 ** 32, (T, H // 512), dtype=np.uint64).astype(np.uint32).view(np.int32)
    got = _run(x, scale, ids, E, M, H, P.BROADCAST, dev)
    assert got[3][0] == M
    _check(x, scale, ids, E, M, H, P.BROADCAST, got, "overflow")


def test_no_tokens_clears_counts():
    dev = U.require_gpu()
    U.banner("permute T=0")
    x = np.zeros((0, 64), np.uint8)
    got = _run(x, np.zeros((0, 1), np.int32), np.zeros((0, 4), np.int64), 7, 128, 512, P.BROADCAST, dev)
    assert got[3].tolist() == [0] * 7
    assert np.all(got[0] == SENT)


def test_page_call_feeds_the_masked_gemm():
    """The page's call end to end: MXFP8 codes permuted by routing, then the
    masked GEMM on the permuted rows equals the oracle's GEMM of each
    expert's tokens (in the device's row order)."""
    dev = U.require_gpu()
    from oracle import gemm as G
    from oracle import quant as Q
    import synth
    rng = np.random.default_rng(14)
    T, H, topk, E, M, N = 256, 512, 2, 4, 256, 128
    U.banner("permute -> masked GEMM")
    xb = synth.normal_bf16(rng, (T, H))
    codes, sf32 = Q.mx_quant_bf16(xb, "mxfp8")
    ids = np.stack([rng.integers(0, E, T), rng.integers(0, E, T)], axis=1).astype(np.int64)
    w = synth.normal_bf16(rng, (E * N, H), 0.05)
    wc, ws = Q.mx_quant_bf16(w, "mxfp8")
    px, osf, imap, nums = hq.prefill_permute_to_masked_gemm(
        U.dev_u8(codes, dev), U.dev_u8(sf32, dev), torch.from_numpy(ids).to(dev), E, M)
    out = torch.zeros(E * M, N, dtype=torch.bfloat16, device=dev)
    hq.hq_group_masked_gemm("mxfp8", px, osf.view(E * M, H // 32), U.dev_u8(wc, dev).view(E, N, H),
                            U.dev_u8(ws, dev).view(E, N, H // 32), nums.view(E), out, M)
    torch.cuda.synchronize()
    imap, nums, got = imap.cpu().numpy(), nums.view(E).cpu().numpy(), U.host_bits(out)
    for e in range(E):
        tok = np.full(nums[e], -1)
        for t, j in zip(*np.nonzero(ids == e)):
            tok[imap[t, j]] = t
        assert np.all(tok >= 0)
        want = G.dense_gemm("mxfp8", codes[tok], sf32[tok], wc[e * N:(e + 1) * N], ws[e * N:(e + 1) * N])
        U.assert_gemm_close(got[e * M:e * M + nums[e]], want, U.deq("mxfp8", codes[tok], sf32[tok]),
                            U.deq("mxfp8", wc[e * N:(e + 1) * N], ws[e * N:(e + 1) * N]), what=f"expert {e}")
