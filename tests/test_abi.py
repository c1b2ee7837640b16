"""The C ABI on the CPU: the library loads, exports what include/isd.h declares, and host
validation rejects bad arguments with the documented status before anything is launched.
(No call here reaches a kernel: every one fails validation first.)"""
import ctypes
import os
import re

import pytest

from strided_verify_propose_amd import isd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "isd.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
FAKE = ctypes.c_void_p(0x1000)     # never dereferenced: validation fails before any launch


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(isd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    return isd.lib()


def test_exports_every_declared_symbol(L):
    names = declared_functions()
    assert len(names) == 23
    assert sorted(isd.EXPORTS) == names
    for n in names:
        assert hasattr(L, n), n


def test_version_and_status_strings(L):
    assert L.isd_abi_version() == 1
    assert L.isd_status_string(0) == b"ok"
    assert L.isd_status_string(3) == b"workspace too small"


def att(L, **kw):
    a = dict(dt=1, B=2, N=4, Hq=32, Hkv=8, D=128, page=16, maxp=10, P=20, maxctx=100,
             scale=0.088, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    ptrs = [None if kw.get("null_at") == i else FAKE for i in range(8)]
    return L.isd_attention_step(a["dt"], *ptrs, a["B"], a["N"], a["Hq"], a["Hkv"], a["D"],
                                a["page"], a["maxp"], a["P"], a["maxctx"], a["scale"],
                                a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=7), INVALID),
    (dict(null_at=0), INVALID),
    (dict(null_at=6), INVALID),
    (dict(B=0), INVALID),
    (dict(Hq=30), INVALID),
    (dict(D=96), UNSUPPORTED),
    (dict(page=32), UNSUPPORTED),
    (dict(maxctx=160), INVALID),           # 160 + 7 > 10 pages * 16
    (dict(maxctx=-1), INVALID),
    (dict(N=10, Hq=32, Hkv=4, maxp=100), UNSUPPORTED),   # 19 rows * 8 heads > 64
    (dict(scale=float("inf")), INVALID),
    (dict(wsb=100, maxctx=3000, maxp=200), WORKSPACE),   # long enough to need splits
    (dict(ws=None, maxctx=3000, maxp=200), WORKSPACE),
    (dict(dt=0, maxctx=20000, maxp=2000), UNSUPPORTED),  # f32 path token limit
    # 2048 requests x 8 KV heads at 2.2M tokens: the work list's 32-bit cost sum would overflow
    (dict(B=2048, maxctx=2200000, maxp=137502), UNSUPPORTED),
    (dict(Hq=65536 * 8), INVALID),
])
def test_attention_validation(L, kw, status):
    assert att(L, **kw) == status
    assert L.isd_last_error() != b""


def ver(L, **kw):
    a = dict(dt=1, B=4, N=4, V=151936, T=1.0, ws=FAKE, wsb=1 << 30, draft=FAKE, ids=FAKE, acc=FAKE)
    a.update(kw)
    return L.isd_verify(a["dt"], FAKE, a["draft"], a["ids"], FAKE, a["B"], a["N"], a["V"],
                        ctypes.c_float(a["T"]), FAKE, a["acc"], FAKE, FAKE, FAKE, None, None,
                        None, a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dt=3), INVALID),
    (dict(B=0), INVALID),
    (dict(N=9), UNSUPPORTED),
    (dict(N=0), UNSUPPORTED),
    (dict(V=1), UNSUPPORTED),
    (dict(V=(1 << 20) + 1), UNSUPPORTED),
    (dict(T=0.0), INVALID),
    (dict(T=float("nan")), INVALID),
    (dict(ids=None), INVALID),
    (dict(acc=None), INVALID),
    (dict(wsb=16), WORKSPACE),
])
def test_verify_validation(L, kw, status):
    assert ver(L, **kw) == status


def test_verify_workspace_query(L):
    assert L.isd_verify_workspace_bytes(64, 4, 151936) > 0
    assert L.isd_verify_workspace_bytes(0, 4, 151936) == 0


def ver_carry(L, prev, nxt, **kw):
    a = dict(dt=1, B=4, N=4, V=151936, T=1.0, ws=FAKE, wsb=1 << 30, draft=FAKE, ids=FAKE, acc=FAKE)
    a.update(kw)
    return L.isd_verify_carry(a["dt"], FAKE, a["draft"], a["ids"], FAKE, a["B"], a["N"], a["V"],
                              ctypes.c_float(a["T"]), FAKE, a["acc"], FAKE, FAKE, FAKE, None, None,
                              None, prev, nxt, a["ws"], a["wsb"], None)


OTHER = ctypes.c_void_p(0x2000)


@pytest.mark.parametrize("prev,nxt,kw,status", [
    (FAKE, FAKE, {}, INVALID),                      # one buffer for both
    (FAKE, None, dict(draft=None), INVALID),        # carried draft statistics with argmax drafts
    (None, FAKE, dict(N=1, ids=None, acc=None), INVALID),  # N = 1 has nothing to carry
    (FAKE, OTHER, dict(wsb=16), WORKSPACE),         # isd_verify's own checks still apply
    (FAKE, OTHER, dict(T=0.0), INVALID),
])
def test_verify_carry_validation(L, prev, nxt, kw, status):
    assert ver_carry(L, prev, nxt, **kw) == status


def test_verify_carry_bytes(L):
    # per request and carried row: SV chunk maxima and references, NSUB sub-chunk sums
    SV, NSUB = (151936 + 16383) // 16384, (151936 + 1023) // 1024
    assert L.isd_verify_carry_bytes(64, 4, 151936) == 64 * 3 * (2 * SV + NSUB) * 4
    assert L.isd_verify_carry_bytes(64, 1, 151936) == 0
    assert L.isd_verify_carry_bytes(0, 4, 151936) == 0


def proj(L, **kw):
    a = dict(M=448, K=4096, Nout=4096, r=128, gate=FAKE, a=FAKE, b=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.isd_gated_lora_proj(FAKE, FAKE, a["a"], a["b"], a["gate"], FAKE, a["M"], a["K"],
                                 a["Nout"], a["r"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), INVALID),
    (dict(K=100), UNSUPPORTED),
    (dict(Nout=200), UNSUPPORTED),
    (dict(r=64), UNSUPPORTED),
    (dict(a=None), INVALID),
    (dict(wsb=1000), WORKSPACE),
])
def test_proj_validation(L, kw, status):
    assert proj(L, **kw) == status


def proj_packed(L, **kw):
    a = dict(M=448, K=4096, Nout=4096, r=128, gate=FAKE, packed=FAKE, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return L.isd_gated_lora_proj_packed(FAKE, a["packed"], a["gate"], FAKE, a["M"], a["K"], a["Nout"],
                                        a["r"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(M=0), INVALID),
    (dict(packed=None), INVALID),
    (dict(K=100), UNSUPPORTED),
    (dict(Nout=200), UNSUPPORTED),
    (dict(r=64), UNSUPPORTED),
    (dict(r=0), INVALID),          # gated call on weights packed without a rank
    (dict(wsb=1000), WORKSPACE),
])
def test_proj_packed_validation(L, kw, status):
    assert proj_packed(L, **kw) == status


@pytest.mark.parametrize("K,Nout,r,ok", [(4096, 4096, 128, True), (64, 128, 0, True), (64, 128, 256, True),
                                        (100, 128, 0, False), (64, 100, 0, False), (64, 128, 64, False)])
def test_proj_packed_bytes(L, K, Nout, r, ok):
    n = L.isd_proj_packed_bytes(K, Nout, r)
    assert n == (((Nout + r) * K + Nout * r) * 2 if ok else 0)


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE, FAKE, 64, 128, 128), INVALID),
    ((FAKE, FAKE, FAKE, None, 64, 128, 128), INVALID),
    ((FAKE, None, FAKE, FAKE, 64, 128, 128), INVALID),   # rank without a
    ((FAKE, FAKE, FAKE, FAKE, 96, 128, 128), UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 64, 192, 128), UNSUPPORTED),
    ((FAKE, FAKE, FAKE, FAKE, 64, 128, 96), UNSUPPORTED),
])
def test_pack_validation(L, args, status):
    assert L.isd_pack_proj_weights(*args, None) == status
    assert L.isd_pack_proj_weights_kn(*args, None) == status


def test_workspace_queries_grow_with_shape(L):
    small = L.isd_attention_workspace_bytes(2, 2, 8, 8, 128, 512)      # 3 query rows per KV head
    big = L.isd_attention_workspace_bytes(64, 4, 32, 8, 128, 4096)    # 28 query rows per KV head
    assert 0 < small < big
    assert L.isd_gated_lora_workspace_bytes(448, 4096, 4096, 128) > \
        L.isd_gated_lora_workspace_bytes(448, 4096, 4096, 0) > 0


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 0, 4), INVALID),        # B < 1
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 4, 9), UNSUPPORTED),        # N > 8
    ((FAKE, FAKE, FAKE, FAKE, FAKE, None, None, 4, 0), UNSUPPORTED),        # N < 1
    ((None, FAKE, FAKE, FAKE, FAKE, None, None, 4, 4), INVALID),      # null n_accept
    ((FAKE, FAKE, FAKE, None, FAKE, None, None, 4, 4), INVALID),      # null draft ids, N > 1
    ((FAKE, FAKE, FAKE, FAKE, None, None, None, 4, 4), INVALID),      # null ctx_lens
])
def test_commit_validation(L, args, status):
    """Checked on the host before any launch (no GPU needed)."""
    assert L.isd_commit(*args, None) == status


@pytest.mark.parametrize("args,status", [
    ((None, FAKE, FAKE, 448, 4096, 151936), INVALID),            # null hidden
    ((FAKE, FAKE, None, 448, 4096, 151936), INVALID),            # null logits
    ((FAKE, FAKE, FAKE, 0, 4096, 151936), INVALID),              # no rows
    ((FAKE, FAKE, FAKE, 65537, 4096, 151936), INVALID),          # too many rows
    ((FAKE, FAKE, FAKE, 448, 4080, 151936), UNSUPPORTED),        # Dm % 32
    ((FAKE, FAKE, FAKE, 448, 4096, 151937), UNSUPPORTED),        # V % 8
    ((FAKE, FAKE, FAKE, 448, 4096, (1 << 20) + 8), UNSUPPORTED), # V too large
])
def test_lm_head_validation(L, args, status):
    assert L.isd_lm_head(*args, None) == status


def lmv(L, **kw):
    a = dict(B=64, N=4, Dm=4096, V=151936, T=1.0, h=FAKE, ids=FAKE, acc=FAKE, ws=FAKE, wsb=1 << 40)
    a.update(kw)
    return L.isd_lm_head_verify(a["h"], FAKE, FAKE, FAKE, a["ids"], FAKE, a["B"], a["N"], a["Dm"],
                                a["V"], ctypes.c_float(a["T"]), FAKE, a["acc"], FAKE, FAKE, FAKE,
                                None, None, None, a["ws"], ctypes.c_size_t(a["wsb"]), None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID),
    (dict(N=9), UNSUPPORTED),
    (dict(B=10000, N=4), INVALID),       # 70000 rows > 65536
    (dict(h=None), INVALID),
    (dict(Dm=100), UNSUPPORTED),
    (dict(V=1001), UNSUPPORTED),
    (dict(T=-1.0), INVALID),
    (dict(ids=None), INVALID),
    (dict(acc=None), INVALID),
    (dict(wsb=4096), WORKSPACE),
    (dict(ws=None), WORKSPACE),
])
def test_lm_head_verify_validation(L, kw, status):
    assert lmv(L, **kw) == status


def test_lm_head_verify_workspace_holds_the_verification_records(L):
    need = L.isd_lm_head_verify_workspace_bytes(64, 4, 151936)
    assert need > L.isd_verify_workspace_bytes(64, 4, 151936) > 0
    assert L.isd_lm_head_verify_workspace_bytes(0, 4, 151936) == 0


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback of any kind: without the built library every call raises."""
    monkeypatch.setattr(isd, "_lib", None)
    monkeypatch.setattr(isd, "_LIB_PATH", str(tmp_path / "libisd.so"))
    with pytest.raises(RuntimeError, match="is not built"):
        isd.lib()


@pytest.mark.parametrize("args,status", [
    ((7, FAKE, FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 10, 8, 128), INVALID),
    ((1, None, FAKE, ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 10, 8, 128), INVALID),
    ((1, FAKE, ctypes.c_void_p(0x1800), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 0, 8, 128), INVALID),
    ((1, FAKE, ctypes.c_void_p(0x1800), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 10, 8, 96), UNSUPPORTED),
    ((1, FAKE, ctypes.c_void_p(0x1800), FAKE, ctypes.c_void_p(0x3000), 10, 8, 128), INVALID),   # overlap
    ((1, FAKE, ctypes.c_void_p(0x1800), ctypes.c_void_p(0x2000), ctypes.c_void_p(0x3000), 1 << 30, 65535, 128),
     UNSUPPORTED),
])
def test_kv_pages_validation(L, args, status):
    assert L.isd_pack_kv_pages(*args, None) == status
    assert L.isd_unpack_kv_pages(*args, None) == status
    assert L.isd_last_error() != b""


_K, _V, _PT, _CL, _CS = (ctypes.c_void_p(a) for a in (0x1000, 0x2000, 0x3000, 0x4000, 0x5000))


@pytest.mark.parametrize("args,status", [
    ((None, _V, _PT, _CL, 64, 8, 128, 257, 20000, 4096, _CS), INVALID),       # null k_cache
    ((_K, _V, _PT, _CL, 64, 8, 128, 257, 20000, 4096, None), INVALID),        # null checksum
    ((_K, _V, _PT, _CL, 0, 8, 128, 257, 20000, 4096, _CS), INVALID),          # B = 0
    ((_K, _V, _PT, _CL, 2049, 8, 128, 257, 20000, 4096, _CS), INVALID),       # B past the bf16 limit
    ((_K, _V, _PT, _CL, 64, 0, 128, 257, 20000, 4096, _CS), INVALID),         # Hkv = 0
    ((_K, _V, _PT, _CL, 64, 8, 96, 257, 20000, 4096, _CS), UNSUPPORTED),      # D
    ((_K, _V, _PT, _CL, 64, 8, 128, 0, 20000, 4096, _CS), INVALID),           # no pages per request
    ((_K, _V, _PT, _CL, 64, 8, 128, 256, 20000, 4097, _CS), INVALID),         # max_ctx_len past the table
    ((_K, _V, _PT, _CL, 2048, 65535, 128, 1 << 20, 1 << 30, 1 << 24, _CS), UNSUPPORTED),  # tiles past 2^31 - 1
])
def test_kv_read_sweep_validation(L, args, status):
    """Argument errors of the read sweep come back before anything is launched."""
    assert L.isd_kv_read_sweep(*args, None) == status
    assert L.isd_last_error() != b""
