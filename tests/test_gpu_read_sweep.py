"""GPU test of isd_kv_read_sweep: the tiles it reads are exactly the cached tiles an
attention step reads (pages 0 .. ceil(L_b/16) - 1 of every request and KV head, K and V),
each once.  Every page of the cache -- the block's pages and pages no request uses
included -- holds random bits, so the XOR checksum changes if any tile is missed, read
twice or read in excess; the expected value is the XOR of exactly those tiles, computed
on the host."""
import numpy as np
import pytest
import torch

from strided_verify_propose_amd import isd
from tests.helpers import DEV

pytestmark = pytest.mark.gpu

PAGE = 16


def make_case(seed, B, Hkv, D, ctx, spare_pages=7, bad_ids=False):
    """Random-bit caches [P, Hkv, 16*D] (bf16 words), a permuted page table with room for
    the 2N-1 = 7 block rows, and the expected XOR of the tiles an attention step reads."""
    rng = np.random.default_rng(seed)
    L = np.asarray(ctx, np.int64)
    n_pages = (L + 7 + PAGE - 1) // PAGE
    used = int(n_pages.sum())
    P = used + spare_pages
    perm = rng.permutation(P).astype(np.int32)
    maxp = int(n_pages.max())
    pt = np.zeros((B, maxp), np.int32)
    off = 0
    for b in range(B):
        pt[b, :n_pages[b]] = perm[off:off + n_pages[b]]
        off += n_pages[b]
    if bad_ids:  # ids past either end are clamped into [0, P), as the attention step does
        pt[0, 0] = -5
        pt[-1, 0] = P + 100
    words = PAGE * D // 2  # 32-bit words per (page, head) tile
    k = rng.integers(0, 1 << 32, size=(P, Hkv, words), dtype=np.uint64).astype(np.uint32)
    v = rng.integers(0, 1 << 32, size=(P, Hkv, words), dtype=np.uint64).astype(np.uint32)
    return L, pt, k, v


def expected_xor(L, pt, k, v, max_ctx_len):
    P = k.shape[0]
    x = np.uint32(0)
    for b in range(len(L)):
        Lb = min(max(int(L[b]), 0), max_ctx_len)
        for j in range((Lb + PAGE - 1) // PAGE):
            p = min(max(int(pt[b, j]), 0), P - 1)
            x ^= np.bitwise_xor.reduce(k[p], axis=None) ^ np.bitwise_xor.reduce(v[p], axis=None)
    return int(x)


def run(seed, B, Hkv, D, ctx, max_ctx_len=None, **kw):
    L, pt, k, v = make_case(seed, B, Hkv, D, ctx, **kw)
    mcl = int(L.max()) if max_ctx_len is None else max_ctx_len
    print(f"read sweep case seed={seed} B={B} Hkv={Hkv} D={D} ctx={L.tolist()[:8]} max_ctx_len={mcl}", flush=True)
    P = k.shape[0]
    kd = torch.from_numpy(k.view(np.int16).reshape(P, Hkv, D // 8, PAGE, 8)).view(torch.bfloat16).to(DEV)
    vd = torch.from_numpy(v.view(np.int16).reshape(P, Hkv, D // 16, 4, PAGE, 4)).view(torch.bfloat16).to(DEV)
    ptd = torch.from_numpy(pt).to(DEV)
    cld = torch.from_numpy(L.astype(np.int32)).to(DEV)
    cs = isd.kv_read_sweep(kd, vd, ptd, cld, mcl)
    got = int(cs.cpu().numpy().view(np.uint32)[0])
    want = expected_xor(L, pt, k, v, mcl)
    assert got == want, f"checksum {got:#010x}, expected {want:#010x}"
    # a second sweep into the same word cancels the first: the reads are the same each call
    isd.kv_read_sweep(kd, vd, ptd, cld, mcl, checksum=cs)
    assert int(cs.cpu().numpy().view(np.uint32)[0]) == 0


def test_ragged_contexts_d64():
    run(11, 4, 2, 64, [0, 1, 17, 300])


def test_ragged_contexts_d128():
    run(12, 11, 8, 128, [0, 1, 15, 16, 17, 31, 511, 512, 513, 1100, 2047])


def test_clamped_page_ids_and_lengths():
    """Negative and too-large page ids are clamped; lengths past max_ctx_len count as it."""
    run(13, 5, 4, 128, [40, 100, 900, 33, 260], max_ctx_len=600, bad_ids=True)


def test_all_contexts_empty():
    run(14, 3, 8, 128, [0, 0, 0])


def test_one_long_request():
    run(15, 1, 8, 128, [32000])


def test_benchmark_shape():
    """64 requests with contexts from U[512, 4096], 8 KV heads, D = 128."""
    rng = np.random.default_rng(16)
    run(16, 64, 8, 128, rng.integers(512, 4097, size=64).tolist())
