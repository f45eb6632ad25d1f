"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/ddtree.h, and rejects bad arguments on the host before
anything would be enqueued (no compute call is made here)."""
import ctypes
import os
import re

import pytest

import draft_tree_build_amd as dtb
from draft_tree_build_amd import api

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ddtree.h")

OK, ERR_ARG, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_SCRATCH = 0, -1, -2, -3, -4, -5


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ddtree_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert len(names) == 14, names
    L = ctypes.CDLL(api.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_strerror_and_sizes():
    assert dtb.version() == 10100
    for code in (OK, ERR_ARG, ERR_UNSUP, ERR_WS, ERR_HIP, ERR_SCRATCH):
        assert dtb.strerror(code) and dtb.strerror(code) != "unknown status"
    assert dtb.strerror(-99) == "unknown status"
    assert dtb.ddtree_build_workspace_size(32, 16, 151936, 8, 128) >= 32 * 16 * 8 * 8
    assert dtb.ddtree_build_workspace_size(0, 16, 100, 8, 8) == 0
    assert dtb.ddtree_accept_workspace_size(4, 513) >= 2 * 4 * 513 * 4
    # split-KV partials only when a small batch meets a long prefix
    small = dtb.ddtree_verify_workspace_size(0, 1, 65, 32, 8, 128, 2048)
    big = dtb.ddtree_verify_workspace_size(0, 4, 513, 64, 8, 128, 65536)
    assert small > 1 << 20 and big > 0 and big % 256 == 0
    assert dtb.ddtree_verify_workspace_size(0, 1, 65, 30, 8, 128, 2048) == 0  # Hq % Hkv


def test_verify_workspace_v_copy_threshold():
    """The bf16 verify plans its fp16 V copy from 16 row tiles of 128 query
    rows per (request, kv-head): one request, one kv-head, 8 query heads and
    a 100-key prefix (6 key tiles, too few to split) give 15 row tiles at
    T = 240 (no copy: the minimum workspace) and 16 at T = 241, where the
    copy holds ceil(100/64) + ceil(241/64) = 6 tiles of 64 x 128 fp16 values.
    Two requests and two kv-heads hold four times as many."""
    assert dtb.ddtree_verify_workspace_size(0, 1, 240, 8, 1, 128, 100) == 256
    assert dtb.ddtree_verify_workspace_size(0, 1, 241, 8, 1, 128, 100) == 6 * 64 * 128 * 2
    assert dtb.ddtree_verify_workspace_size(0, 2, 241, 16, 2, 128, 100) == 4 * 6 * 64 * 128 * 2
    assert dtb.ddtree_verify_workspace_size(1, 1, 241, 8, 1, 128, 100) == 256   # f32: no copy


@pytest.mark.parametrize("batch,T,Hq,max_prefix,nsplit,row_tiles,v_copy", [
    (4, 513, 64, 65536, 5, 33, True),       # B4_L32_V151936_K16_N512_P65536
    (32, 129, 32, 16384, 2, 5, False),      # B32_L16_V151936_K8_N128_P512-16384
    (1, 257, 32, 8192, 7, 9, False),        # L16_V151936_K16_N256_P8192
    (1, 65, 32, 2048, 7, 3, False),         # L16_V32000_K8_N64_P2048
])
def test_verify_split_plan_at_benchmark_shapes(batch, T, Hq, max_prefix, nsplit, row_tiles, v_copy):
    """The key splits the planner picks at the benchmark shapes (8 kv-heads)
    -- the counts a sweep of 1 to 12 splits measured best or within 1% of
    it -- read back from the workspace size: fp32 partial O and (m, l) per
    split, row and kv-head, plus the fp16 V copy where it is planned."""
    Hkv = 8
    rows = nsplit * batch * Hkv * row_tiles * 128
    align = lambda x: (x + 255) // 256 * 256
    want = align(rows * 128 * 4) + align(rows * 2 * 4)
    if v_copy:
        want += batch * Hkv * (-(-max_prefix // 64) + -(-T // 64)) * 64 * 128 * 2
    assert dtb.ddtree_verify_workspace_size(0, batch, T, Hq, Hkv, 128, max_prefix) == want


# Host validation. Pointers are fake non-null addresses: every case below has
# exactly one invalid field and must be rejected before any HIP call.
P = ctypes.c_void_p(0x1000)
N0 = None


def _no_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host-validation cases use fake pointers; run them where no GPU is visible")


def _build(**kw):
    a = dict(logits=P, dt=0, root=P, batch=2, L=4, V=64, K=4, N=8, temp=1.0, tokens=P, parents=P,
             depths=P, scores=P, nn=P, mask=N0, tk=N0, tl=N0, st=N0, ws=P, wsb=1 << 20)
    a.update(kw)
    return api.lib().ddtree_build(a["logits"], a["dt"], a["root"], a["batch"], a["L"], a["V"],
                                  a["K"], a["N"], a["temp"], a["tokens"], a["parents"], a["depths"],
                                  a["scores"], a["nn"], a["mask"], a["tk"], a["tl"], a["st"],
                                  a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=N0), ERR_ARG), (dict(tokens=N0), ERR_ARG), (dict(nn=N0), ERR_ARG),
    (dict(batch=0), ERR_ARG), (dict(L=0), ERR_ARG), (dict(K=0), ERR_ARG), (dict(N=0), ERR_ARG),
    (dict(K=65, V=64), ERR_ARG), (dict(temp=-1.0), ERR_ARG), (dict(temp=float("inf")), ERR_ARG),
    (dict(temp=float("nan")), ERR_ARG), (dict(dt=7), ERR_UNSUP), (dict(K=33, V=100), ERR_UNSUP),
    (dict(N=1025), ERR_UNSUP), (dict(L=65), ERR_UNSUP), (dict(V=(1 << 19) + 1), ERR_UNSUP),
    (dict(ws=N0), ERR_WS), (dict(wsb=16), ERR_WS),
])
def test_build_rejects(kw, code):
    _no_gpu()
    assert _build(**kw) == code


def _build_noalloc(**kw):
    a = dict(logits=P, dt=0, root=P, batch=2, L=4, V=64, K=4, N=8, temp=1.0, tokens=P, parents=P,
             depths=P, scores=P, nn=P, mask=N0, tk=N0, tl=N0, st=N0)
    a.update(kw)
    return api.lib().ddtree_build_noalloc(a["logits"], a["dt"], a["root"], a["batch"], a["L"],
                                          a["V"], a["K"], a["N"], a["temp"], a["tokens"],
                                          a["parents"], a["depths"], a["scores"], a["nn"],
                                          a["mask"], a["tk"], a["tl"], a["st"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(logits=N0), ERR_ARG), (dict(nn=N0), ERR_ARG), (dict(N=0), ERR_ARG),
    (dict(temp=float("nan")), ERR_ARG), (dict(dt=7), ERR_UNSUP), (dict(K=33, V=100), ERR_UNSUP),
    (dict(V=(1 << 19) + 1), ERR_UNSUP),
    # scratch beyond the static buffer (6.5 MB for 256 x 16 rows of 151936): rejected
    (dict(batch=256, L=16, V=151936, K=8, N=128), ERR_SCRATCH),
])
def test_build_noalloc_rejects(kw, code):
    """Same argument checks as ddtree_build, then the scratch limit; all on
    the host before any HIP call."""
    _no_gpu()
    assert _build_noalloc(**kw) == code
    need = dtb.ddtree_build_workspace_size(256, 16, 151936, 8, 128)
    assert need > 4 << 20 >= dtb.ddtree_build_workspace_size(32, 16, 151936, 8, 128)


def _verify(**kw):
    a = dict(q=P, k=P, v=P, dt=0, offs=P, pl=P, nn=P, mask=P, batch=1, T=9, Hq=4, Hkv=2, D=128,
             maxp=16, rows=100, scale=0.0, out=P, st=N0, ws=P, wsb=1 << 24)
    a.update(kw)
    return api.lib().ddtree_verify_attn(a["q"], a["k"], a["v"], a["dt"], a["offs"], a["pl"],
                                        a["nn"], a["mask"], a["batch"], a["T"], a["Hq"], a["Hkv"],
                                        a["D"], a["maxp"], a["rows"], a["scale"], a["out"],
                                        a["st"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=N0), ERR_ARG), (dict(mask=N0), ERR_ARG), (dict(out=N0), ERR_ARG),
    (dict(Hq=5), ERR_ARG), (dict(T=0), ERR_ARG), (dict(maxp=-1), ERR_ARG), (dict(rows=0), ERR_ARG),
    (dict(scale=float("nan")), ERR_ARG), (dict(dt=3), ERR_UNSUP), (dict(D=96), ERR_UNSUP),
    (dict(D=64), ERR_UNSUP), (dict(T=1026), ERR_UNSUP), (dict(ws=N0), ERR_WS),
    (dict(wsb=0), ERR_WS),
])
def test_verify_rejects(kw, code):
    _no_gpu()
    assert _verify(**kw) == code


def _accept(**kw):
    a = dict(tl=P, dt=0, ids=N0, tok=P, par=P, nn=P, batch=1, T=9, V=64, L=4, acc=P, accn=N0,
             alen=P, bonus=P, targ=N0, ws=P, wsb=1 << 16)
    a.update(kw)
    return api.lib().ddtree_accept(a["tl"], a["dt"], a["ids"], a["tok"], a["par"], a["nn"],
                                   a["batch"], a["T"], a["V"], a["L"], a["acc"], a["accn"],
                                   a["alen"], a["bonus"], a["targ"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(tl=N0), ERR_ARG), (dict(tok=N0), ERR_ARG), (dict(bonus=N0), ERR_ARG),
    (dict(L=0), ERR_ARG), (dict(V=0), ERR_ARG), (dict(batch=0), ERR_ARG), (dict(dt=9), ERR_UNSUP),
    (dict(L=65), ERR_UNSUP), (dict(T=2000), ERR_UNSUP), (dict(wsb=4), ERR_WS),
])
def test_accept_rejects(kw, code):
    _no_gpu()
    assert _accept(**kw) == code


def _sample(**kw):
    a = dict(tl=P, dt=0, tok=P, par=P, nn=P, batch=1, T=9, V=64, L=4, temp=1.0, seed=1, off=0,
             acc=P, accn=N0, alen=P, bonus=P, targ=N0, ws=P, wsb=1 << 16)
    a.update(kw)
    return api.lib().ddtree_accept_sample(a["tl"], a["dt"], a["tok"], a["par"], a["nn"],
                                          a["batch"], a["T"], a["V"], a["L"], a["temp"],
                                          a["seed"], a["off"], a["acc"], a["accn"], a["alen"],
                                          a["bonus"], a["targ"], a["ws"], a["wsb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(tl=N0), ERR_ARG), (dict(par=N0), ERR_ARG), (dict(acc=N0), ERR_ARG), (dict(V=0), ERR_ARG),
    (dict(T=0), ERR_ARG), (dict(L=0), ERR_ARG), (dict(temp=0.0), ERR_ARG),
    (dict(temp=-0.5), ERR_ARG), (dict(temp=float("inf")), ERR_ARG),
    (dict(temp=float("nan")), ERR_ARG), (dict(dt=5), ERR_UNSUP), (dict(L=65), ERR_UNSUP),
    (dict(T=1026), ERR_UNSUP), (dict(V=(1 << 19) + 1), ERR_UNSUP), (dict(V=(1 << 31) - 1), ERR_UNSUP),
    (dict(ws=N0), ERR_WS), (dict(wsb=8), ERR_WS),
])
def test_accept_sample_rejects(kw, code):
    _no_gpu()
    assert _sample(**kw) == code


def _commit(**kw):
    a = dict(k=P, v=P, dt=0, offs=P, pl=P, alen=P, accn=P, bonus=P, batch=2, Hkv=8, D=128, L=16,
             T=65, rows=10000, newp=ctypes.c_void_p(0x2000), roots=N0)
    a.update(kw)
    return api.lib().ddtree_commit_kv(a["k"], a["v"], a["dt"], a["offs"], a["pl"], a["alen"],
                                      a["accn"], a["bonus"], a["batch"], a["Hkv"], a["D"], a["L"],
                                      a["T"], a["rows"], a["newp"], a["roots"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(k=N0), ERR_ARG), (dict(accn=N0), ERR_ARG), (dict(newp=N0), ERR_ARG),
    (dict(newp=P), ERR_ARG),                      # new prefix lengths over the old ones
    (dict(batch=0), ERR_ARG), (dict(L=0), ERR_ARG), (dict(T=0), ERR_ARG), (dict(rows=0), ERR_ARG),
    (dict(dt=4), ERR_UNSUP), (dict(L=65), ERR_UNSUP), (dict(T=1026), ERR_UNSUP),
    (dict(D=100), ERR_UNSUP), (dict(D=1024), ERR_UNSUP), (dict(dt=1, D=257), ERR_UNSUP),
    (dict(k=ctypes.c_void_p(0x1008)), ERR_UNSUP), (dict(Hkv=70000), ERR_UNSUP),
])
def test_commit_rejects(kw, code):
    _no_gpu()
    assert _commit(**kw) == code


def test_mask_rejects():
    _no_gpu()
    L = api.lib()
    assert L.ddtree_mask(None, P, 1, 9, P, None) == ERR_ARG
    assert L.ddtree_mask(P, P, 0, 9, P, None) == ERR_ARG
    assert L.ddtree_mask(P, P, 1, 2000, P, None) == ERR_UNSUP


@pytest.mark.parametrize("call,code", [
    (lambda L: L.ddtree_probe_mfma_bf16(None, 1, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_mfma_bf16(P, 0, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_mfma_bf16(P, 1, 0, None), ERR_ARG),
    (lambda L: L.ddtree_probe_mfma_bf16(P, (1 << 20) + 1, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(None, 16, P, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(P, 16, None, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(P, 24, P, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(P, 0, P, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(ctypes.c_void_p(0x1008), 16, P, 1, None), ERR_ARG),
    (lambda L: L.ddtree_probe_hbm_read(P, 16, P, 0, None), ERR_ARG),
])
def test_probes_reject(call, code):
    """The calibration kernels' host checks (measurement only)."""
    _no_gpu()
    assert call(api.lib()) == code
