"""C ABI checks that need no GPU: the library loads, exports every function
declared in include/*.h, and rejects bad arguments on the host with the
documented status before any HIP call (so nothing here touches a device)."""

import ctypes
import glob
import os
import re

import pytest

import invariant_token_log_amd as itl
from invariant_token_log_amd import _lib
from invariant_token_log_amd.build import LIB_PATH, build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB_PATH):
        build()
    return _lib.lib()


def _declared_functions():
    names = []
    for hdr in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(hdr).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        names += re.findall(r"^[A-Za-z_][\w \t\*]*?\b([a-z_][a-z0-9_]*)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_every_declared_symbol_is_exported(L):
    names = _declared_functions()
    assert {"logp_fwd", "logp_bwd", "linear_logp_fwd"} <= set(names)
    raw = ctypes.CDLL(LIB_PATH)
    for name in names:
        assert hasattr(raw, name), name
    assert set(names) == set(_lib._SIGNATURES)


def test_strings(L):
    assert itl.status_str(0) == "ok"
    assert "tile" in itl.status_str(_lib.LOGP_ERR_TILE)
    assert itl.status_str(99) == "unknown status"
    cid = itl.contract_id()
    assert cid.startswith("itl.logp.v1[") and "gfx950" in cid


FAKE = 0x10000  # a non-NULL address that the checks never dereference


def _fwd(L, logits=FAKE, dtype=1, n=4, v=151936, ld=None, targets=FAKE, tdt=0, w=4096,
         shards=1, validate=0, logp=FAKE, lse=FAKE, ent=None, ws=None, ws_bytes=0):
    return L.logp_fwd(logits, dtype, n, v, v if ld is None else ld, targets, tdt, -100, w,
                      shards, validate, logp, lse, ent, ws, ws_bytes, None)


def test_fwd_argument_errors(L):
    assert _fwd(L, dtype=3) == _lib.LOGP_ERR_DTYPE
    assert _fwd(L, tdt=2) == _lib.LOGP_ERR_DTYPE
    assert _fwd(L, dtype=2, w=256, v=4096) == _lib.LOGP_ERR_TILE  # fp16 tiles start at 512
    assert _fwd(L, n=-1) == _lib.LOGP_ERR_SHAPE
    assert _fwd(L, v=0) == _lib.LOGP_ERR_SHAPE
    assert _fwd(L, ld=100) == _lib.LOGP_ERR_SHAPE
    for w in (0, 256, 1000, 1536, 3072, 16384):
        assert _fwd(L, w=w) == _lib.LOGP_ERR_TILE, w
    assert _fwd(L, dtype=0, w=128, v=4096) == _lib.LOGP_ERR_TILE
    assert _fwd(L, v=512 * 4097, w=512) == _lib.LOGP_ERR_SHAPE  # T > 4096
    assert _fwd(L, shards=0) == _lib.LOGP_ERR_SHARDS
    assert _fwd(L, shards=3) == _lib.LOGP_ERR_SHARDS  # 151936 % 3 != 0
    assert _fwd(L, logits=None) == _lib.LOGP_ERR_NULL
    assert _fwd(L, targets=None) == _lib.LOGP_ERR_NULL
    assert _fwd(L, logp=None) == _lib.LOGP_ERR_NULL
    assert _fwd(L, shards=2) == _lib.LOGP_ERR_WORKSPACE
    need = L.logp_fwd_workspace_bytes(4, 151936, 4096, 2, 0)
    assert _fwd(L, shards=2, ws=FAKE, ws_bytes=need - 1) == _lib.LOGP_ERR_WORKSPACE
    assert _fwd(L, shards=2, ws=FAKE + 16, ws_bytes=need) == _lib.LOGP_ERR_WORKSPACE
    assert _fwd(L, validate=1) == _lib.LOGP_ERR_WORKSPACE
    # n = 0 is a no-op that succeeds without touching any pointer
    assert _fwd(L, n=0, logits=None, targets=None, logp=None) == _lib.LOGP_OK


def test_fwd_workspace_sizes(L):
    n, v = 8192, 151936
    assert L.logp_fwd_workspace_bytes(n, v, 4096, 1, 0) == 0
    assert L.logp_fwd_workspace_bytes(n, v, 4096, 1, 1) == 256
    table = -(-(38 * n * 4) // 256) * 256
    rows = -(-(n * 4) // 256) * 256
    for s in (2, 4):  # m, s and the entropy moment w, then the target logits
        assert L.logp_fwd_workspace_bytes(n, v, 4096, s, 0) == 256 + 3 * table + rows
    assert L.logp_fwd_workspace_bytes(n, v, 1000, 1, 0) == 0  # rejected tile
    assert L.logp_fwd_workspace_bytes(n, v, 4096, 3, 0) == 0  # rejected shards


def test_bwd_argument_errors(L):
    def bwd(**kw):
        a = dict(logits=FAKE, dtype=1, n=4, v=151936, ld=151936, targets=FAKE, tdt=0, w=4096,
                 lse=FAKE, g=FAKE, ent=None, gent=None, d=FAKE, ld_out=151936)
        a.update(kw)
        return L.logp_bwd(a["logits"], a["dtype"], a["n"], a["v"], a["ld"], a["targets"],
                          a["tdt"], -100, a["w"], a["lse"], a["g"], a["ent"], a["gent"],
                          a["d"], a["ld_out"], None)
    assert bwd(ent=FAKE) == _lib.LOGP_ERR_NULL  # entropy without its gradient
    assert bwd(gent=FAKE) == _lib.LOGP_ERR_NULL
    assert bwd(dtype=5) == _lib.LOGP_ERR_DTYPE
    assert bwd(tdt=-1) == _lib.LOGP_ERR_DTYPE
    assert bwd(ld_out=10) == _lib.LOGP_ERR_SHAPE
    assert bwd(w=100) == _lib.LOGP_ERR_TILE
    for k in ("logits", "targets", "lse", "g", "d"):
        assert bwd(**{k: None}) == _lib.LOGP_ERR_NULL, k
    assert bwd(n=0, logits=None, d=None) == _lib.LOGP_OK


def test_linear_argument_errors(L):
    def lin(**kw):
        a = dict(h_ptr=FAKE, ld_h=4096, w_ptr=FAKE, ld_w=4096, n=8, h=4096, v=151936,
                 targets=FAKE, tdt=0, tile=256, temp=1.0, rnd=0, logp=FAKE, lse=FAKE,
                 ent=None, z=None, zdt=1, ldz=0, pw=None, pwb=0, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return L.linear_logp_fwd(a["h_ptr"], a["ld_h"], a["w_ptr"], a["ld_w"], a["n"], a["h"],
                                 a["v"], a["targets"], a["tdt"], -100, a["tile"], a["temp"],
                                 a["rnd"], a["logp"], a["lse"], a["ent"], a["z"], a["zdt"],
                                 a["ldz"], a["pw"], a["pwb"], a["ws"], a["ws_bytes"], None)
    for bad in (0.0, -1.0, float("inf"), float("nan")):
        assert lin(temp=bad) == _lib.LOGP_ERR_VALUE, bad
    for bad in (-1, 2, 7):
        assert lin(rnd=bad) == _lib.LOGP_ERR_VALUE, bad
    assert lin(z=FAKE, zdt=2, ldz=151936) == _lib.LOGP_ERR_DTYPE
    assert lin(z=FAKE, zdt=0, ldz=100) == _lib.LOGP_ERR_SHAPE
    assert lin(tdt=9) == _lib.LOGP_ERR_DTYPE
    assert lin(tile=4096) == _lib.LOGP_ERR_TILE
    # prepared weight: at least linear_logp_prepared_bytes, 16-byte aligned
    assert lin(pw=FAKE, pwb=2491416576 - 1) == _lib.LOGP_ERR_SHAPE
    assert lin(pw=FAKE + 8, pwb=2491416576) == _lib.LOGP_ERR_ALIGN
    assert lin(h=100, ld_h=100, ld_w=100) == _lib.LOGP_ERR_SHAPE
    assert lin(ld_h=10) == _lib.LOGP_ERR_SHAPE
    assert lin(h_ptr=None) == _lib.LOGP_ERR_NULL
    assert lin(h_ptr=FAKE + 2) == _lib.LOGP_ERR_ALIGN
    assert lin(ld_w=4100) == _lib.LOGP_ERR_ALIGN
    assert lin(ws_bytes=16) == _lib.LOGP_ERR_WORKSPACE
    assert lin(n=0, h_ptr=None, w_ptr=None) == _lib.LOGP_OK
    need = L.linear_logp_fwd_workspace_bytes(8, 4096, 151936, 256)
    assert need == 256 + 3 * 256 * (-(-(594 * 8 * 4) // 256)) + 256
    assert L.linear_logp_fwd_workspace_bytes(8, 4096, 151936, 512) == 0
    assert L.linear_logp_fwd_workspace_bytes(8, 100, 151936, 256) == 0
    # n > 128: plus the re-laid hidden copy, 256-row padded, and the 8
    # tile-queue counters (64 bytes apart)
    tables = 256 + 3 * 256 * (-(-(594 * 200 * 4) // 256)) + 256 * (-(-(200 * 4) // 256))
    assert L.linear_logp_fwd_workspace_bytes(200, 4096, 151936, 256) == (
        tables + 256 * 4096 * 2 + 512)


def test_linear_bwd_argument_errors(L):
    def lb(**kw):
        a = dict(h_ptr=FAKE, ld_h=4096, w_ptr=FAKE, ld_w=4096, n=8, h=4096, v=151936,
                 targets=FAKE, tdt=0, tile=256, temp=1.0, rnd=0, z=None, zdt=0, ldz=0,
                 wt=None, ldwt=0, lse=FAKE, g=FAKE, ent=None, gent=None, out=0, dh=FAKE,
                 ld_dh=4096, dw=FAKE, ld_dw=4096, vc=0, ws=FAKE, ws_bytes=1 << 40)
        a.update(kw)
        return L.linear_logp_bwd(a["h_ptr"], a["ld_h"], a["w_ptr"], a["ld_w"], a["n"], a["h"],
                                 a["v"], a["targets"], a["tdt"], -100, a["tile"], a["temp"],
                                 a["rnd"], a["z"], a["zdt"], a["ldz"], a["wt"], a["ldwt"],
                                 a["lse"], a["g"], a["ent"], a["gent"], a["out"], a["dh"],
                                 a["ld_dh"], a["dw"], a["ld_dw"], a["vc"], a["ws"],
                                 a["ws_bytes"], None)
    assert lb(temp=0.0) == _lib.LOGP_ERR_VALUE
    assert lb(rnd=3) == _lib.LOGP_ERR_VALUE
    # saved logits: fp32, or bf16 only in the bf16-rounded contract
    assert lb(z=FAKE, zdt=_lib.LOGP_BF16, ldz=151936) == _lib.LOGP_ERR_DTYPE
    assert lb(z=FAKE, zdt=_lib.LOGP_F16, ldz=151936, rnd=1) == _lib.LOGP_ERR_DTYPE
    assert lb(z=FAKE, zdt=_lib.LOGP_F32, ldz=100) == _lib.LOGP_ERR_SHAPE
    assert lb(z=FAKE + 4, zdt=_lib.LOGP_F32, ldz=151936) == _lib.LOGP_ERR_ALIGN
    assert lb(z=FAKE, zdt=_lib.LOGP_F32, ldz=151937) == _lib.LOGP_ERR_ALIGN
    # prepared weight: at least linear_logp_prepared_bytes, 16-byte aligned
    assert lb(wt=FAKE, ldwt=2491416576 - 1) == _lib.LOGP_ERR_SHAPE
    assert lb(wt=FAKE + 8, ldwt=2491416576) == _lib.LOGP_ERR_ALIGN
    assert lb(ent=FAKE) == _lib.LOGP_ERR_NULL
    assert lb(tdt=5) == _lib.LOGP_ERR_DTYPE
    assert lb(out=2) == _lib.LOGP_ERR_DTYPE
    assert lb(tile=512) == _lib.LOGP_ERR_TILE
    assert lb(h=100, ld_h=100, ld_w=100) == _lib.LOGP_ERR_SHAPE
    assert lb(h=0, ld_h=0, ld_w=0) == _lib.LOGP_ERR_SHAPE
    assert lb(ld_dh=100) == _lib.LOGP_ERR_SHAPE
    assert lb(ld_dw=100) == _lib.LOGP_ERR_SHAPE
    assert lb(out=7) == _lib.LOGP_ERR_DTYPE
    assert lb(dh=None, dw=None) == _lib.LOGP_ERR_NULL
    for k in ("h_ptr", "w_ptr", "targets", "lse", "g"):
        assert lb(**{k: None}) == _lib.LOGP_ERR_NULL, k
    assert lb(h_ptr=FAKE + 2) == _lib.LOGP_ERR_ALIGN
    assert lb(ld_w=4100) == _lib.LOGP_ERR_ALIGN
    assert lb(ws_bytes=16) == _lib.LOGP_ERR_WORKSPACE
    assert lb(ws=FAKE + 16) == _lib.LOGP_ERR_WORKSPACE
    assert lb(n=0, h_ptr=None, targets=None, lse=None, g=None, dw=None) == _lib.LOGP_OK
    assert lb(vc=-1) == _lib.LOGP_ERR_SHAPE
    # the workspace is checked against this call's own options: dh only,
    # fp32 out, no prepared weight needs blocked h + dz_c + W^T_c
    only_dh = L.linear_logp_bwd_workspace_bytes(8, 4096, 151936, 256, _lib.LOGP_BWD_DHIDDEN, 0)
    both = L.linear_logp_bwd_workspace_bytes(8, 4096, 151936, 256,
                                             _lib.LOGP_BWD_DHIDDEN | _lib.LOGP_BWD_DWEIGHT, 0)
    assert only_dh < both
    assert lb(dw=None, ws_bytes=only_dh - 1) == _lib.LOGP_ERR_WORKSPACE
    assert lb(ws_bytes=both - 1) == _lib.LOGP_ERR_WORKSPACE


def test_linear_bwd_workspace_sizes(L):
    """Regions in use only: blocked h (recompute), h^T (dW), dz_c (dh and dW),
    fp32 dh between chunks (bf16 dh over several chunks); bf16 unless noted,
    Np = round_up(n, 256), chunk C = min(round_up(vocab_chunk or 32768, 256),
    Vp).  The weight is read as it is (no per-chunk copy), prepared or not."""
    B = _lib
    n, h, v = 8, 4096, 151936
    np_, vp, c = 256, 152064, 32768

    def ws(flags, vc=0, nn=n):
        return L.linear_logp_bwd_workspace_bytes(nn, h, v, 256, flags, vc)

    both = B.LOGP_BWD_DHIDDEN | B.LOGP_BWD_DWEIGHT
    assert ws(both) == 2 * (np_ * h + h * np_ + np_ * c)
    assert ws(both | B.LOGP_BWD_PREPARED) == ws(both)
    assert ws(both | B.LOGP_BWD_SAVED_LOGITS) == 2 * (h * np_ + np_ * c)
    assert ws(B.LOGP_BWD_DHIDDEN) == 2 * (np_ * h + np_ * c)
    assert ws(B.LOGP_BWD_DWEIGHT) == 2 * (np_ * h + h * np_ + np_ * c)
    assert ws(both | B.LOGP_BWD_BF16_OUT) == ws(both) + n * h * 4  # fp32 dh between chunks
    assert ws(both, vc=1000) == 2 * (np_ * h + h * np_ + np_ * 1024)
    # one chunk over the whole vocabulary: no fp32 dh staging for bf16 output
    one = ws(both, vc=v)
    assert one == 2 * (np_ * h + h * np_ + np_ * vp)
    assert ws(both | B.LOGP_BWD_BF16_OUT, vc=v) == one
    # the benchmarked head: N = H = 4096 with both outputs stays under 1 GB
    assert L.linear_logp_bwd_workspace_bytes(4096, 4096, v, 256, both, 0) < 1 << 30
    assert ws(both, nn=0) == 0
    assert L.linear_logp_bwd_workspace_bytes(8, 4096, v, 4096, both, 0) == 0
    assert L.linear_logp_bwd_workspace_bytes(8, 100, v, 256, both, 0) == 0
    assert ws(both, vc=-5) == 0


def test_prepare_weight_argument_errors(L):
    def pw(**kw):
        a = dict(w=FAKE, ld_w=4096, v=151936, h=4096, wt=FAKE, ldwt=2491416576)
        a.update(kw)
        return L.linear_logp_prepare_weight(a["w"], a["ld_w"], a["v"], a["h"], a["wt"],
                                            a["ldwt"], None)
    assert pw(ldwt=2491416576 - 2) == _lib.LOGP_ERR_SHAPE
    assert pw(v=0) == _lib.LOGP_ERR_SHAPE
    assert pw(h=100, ld_w=100) == _lib.LOGP_ERR_SHAPE
    assert pw(ld_w=4000) == _lib.LOGP_ERR_SHAPE
    assert pw(w=None) == _lib.LOGP_ERR_NULL
    assert pw(wt=None) == _lib.LOGP_ERR_NULL
    assert pw(wt=FAKE + 8) == _lib.LOGP_ERR_ALIGN
    assert pw(ld_w=4100) == _lib.LOGP_ERR_ALIGN
    assert pw(w=FAKE + 2) == _lib.LOGP_ERR_ALIGN
    # the weight and its transpose, vocabulary padded to 256
    assert L.linear_logp_prepared_bytes(151936, 4096) == 2 * 4096 * 152064 * 2
    assert L.linear_logp_prepared_bytes(1, 64) == 2 * 64 * 256 * 2
    assert L.linear_logp_prepared_bytes(0, 4096) == 0
    assert L.linear_logp_prepared_bytes(151936, 100) == 0


def test_temperature_bounds(L):
    """A temperature is usable when it is finite, > 0 and its fp32 reciprocal
    is finite: below about 2.9e-39 the reciprocal overflows and is refused;
    FLT_MAX passes the check (the call then stops at a NULL pointer)."""
    def lin(temp, h_ptr=FAKE):
        return L.linear_logp_fwd(h_ptr, 4096, FAKE, 4096, 8, 4096, 151936, FAKE, 0, -100, 256,
                                 temp, 0, FAKE, FAKE, None, None, 1, 0, None, 0, FAKE, 1 << 40,
                                 None)
    flt_max = 3.4028234663852886e38
    for bad in (1e-39, 1.0e-45, 2.0e-39):
        assert lin(bad) == _lib.LOGP_ERR_VALUE, bad
    for ok in (3.0e-38, 1.0, flt_max):
        assert lin(ok, h_ptr=None) == _lib.LOGP_ERR_NULL, ok
    lb = L.linear_logp_bwd(FAKE, 4096, FAKE, 4096, 8, 4096, 151936, FAKE, 0, -100, 256, 1e-39,
                           0, None, 0, 0, None, 0, FAKE, FAKE, None, None, 0, FAKE, 4096, FAKE,
                           4096, 0, FAKE, 1 << 40, None)
    assert lb == _lib.LOGP_ERR_VALUE


def test_noalloc_argument_errors(L):
    """linear_logp_fwd_noalloc runs linear_logp_fwd's checks, then refuses a
    problem whose workspace exceeds the static scratch array, all before any
    HIP call."""
    def na(**kw):
        a = dict(h_ptr=FAKE, ld_h=4096, w_ptr=FAKE, n=8, h=4096, v=151936, temp=1.0, logp=FAKE)
        a.update(kw)
        return L.linear_logp_fwd_noalloc(a["h_ptr"], a["ld_h"], a["w_ptr"], 4096, a["n"],
                                         a["h"], a["v"], FAKE, 0, -100, 256, a["temp"], 0,
                                         a["logp"], FAKE, None, None, 1, 0, None, 0, None)
    assert na(temp=0.0) == _lib.LOGP_ERR_VALUE
    assert na(h_ptr=None) == _lib.LOGP_ERR_NULL
    assert na(h_ptr=FAKE + 2) == _lib.LOGP_ERR_ALIGN
    assert na(ld_h=10) == _lib.LOGP_ERR_SHAPE
    assert na(n=0, h_ptr=None, w_ptr=None, logp=None) == _lib.LOGP_OK
    # N = 8192 at the Qwen3-8B head needs ~125 MB > 64 MiB of scratch
    assert L.linear_logp_fwd_workspace_bytes(8192, 4096, 151936, 256) > _lib.NOALLOC_SCRATCH_BYTES
    assert na(n=8192) == _lib.LOGP_ERR_SCRATCH
    # the largest N that fits at that head: 4352 (17 blocks of 256 rows)
    assert L.linear_logp_fwd_workspace_bytes(4352, 4096, 151936, 256) <= _lib.NOALLOC_SCRATCH_BYTES
    assert L.linear_logp_fwd_workspace_bytes(4353, 4096, 151936, 256) > _lib.NOALLOC_SCRATCH_BYTES
    assert "scratch" in itl.status_str(_lib.LOGP_ERR_SCRATCH)
