"""The C ABI on the CPU: the library loads, exports every entry point the header
declares, and rejects bad arguments with the documented status before any device
work.  Pointers here are fake addresses: every call below must fail a host-side
check, so none of them is ever dereferenced or reaches a kernel."""
import ctypes
import math
import os
import re

import pytest

import block_sparse_flash_mask_amd as bs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsattn.h")

OK, NULL, SHAPE, UNSUP, ALIGN, WS, SCALE, ALIAS, HIP, IO = range(10)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(bs.LIB_PATH):
        from block_sparse_flash_mask_amd import build
        build.build()
    return bs.library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bsattn_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings(lib):
    for code, name in bs.STATUS.items():
        s = lib.bsattn_status_string(code).decode()
        assert s.startswith(name), (code, s)
    assert lib.bsattn_status_string(99).decode().startswith("BSATTN")


def test_version(lib):
    assert bs.version() >= (0, 1, 0)


def test_workspace_sizes(lib):
    # counts (R int32) + lists (R*n_k int32) + dispatch order of the rows (8 chunks
    # of ceil(R/8), int32) + that of the row pairs (8 chunks of ceil(P/8)), each
    # rounded up to 256 bytes
    rnd = lambda x: (x + 255) // 256 * 256
    for B, H, S, bq, bk in ((4, 16, 2048, 128, 128), (1, 3, 640, 64, 128), (1, 1, 64, 64, 64)):
        R, nk = B * H * (S // bq), S // bk
        P = B * H * ((S // bq + 1) // 2)
        order = 8 * ((R + 7) // 8) * 4
        porder = 8 * ((P + 7) // 8) * 4
        assert bs.workspace_size(B, H, S, bq, bk) == (rnd(R * 4) + rnd(R * nk * 4) + rnd(order)
                                                      + rnd(porder))
    assert bs.compact_workspace_size(1, 2, 3, 5) == rnd(6 * 4) + rnd(30 * 4)
    n = ctypes.c_size_t()
    assert lib.bsattn_workspace_size(1, 1, 100, 64, 64, ctypes.byref(n)) == SHAPE
    assert lib.bsattn_workspace_size(0, 1, 128, 64, 64, ctypes.byref(n)) == SHAPE
    assert lib.bsattn_workspace_size(1, 1, 128, 64, 64, None) == NULL
    assert lib.bsattn_compact_workspace_size(1, 1, 1 << 16, 1 << 16, ctypes.byref(n)) == SHAPE


def test_list_configs(lib):
    import torch
    c = bs.list_configs(torch.bfloat16, 128, 128, 128)
    assert c and all(t.tile_q in (64, 128, 256) and t.tile_k in (32, 64, 128) for t in c)
    # a wave owns 32 or 64 query rows; the 8-wave two-group kernel has two waves per 32 rows
    assert all(t.tile_q in (16 * t.waves, 32 * t.waves, 64 * t.waves) and t.stages in (1, 2, 3) for t in c)
    assert any(t.tile_q == 256 for t in c)  # row pairs, block_q 128 only
    assert not any(t.tile_q == 256 for t in bs.list_configs(torch.bfloat16, 128, 64, 128))
    assert all(t.tile_q <= 64 for t in bs.list_configs(torch.bfloat16, 64, 64, 128))
    assert all(t.tile_k <= 64 for t in bs.list_configs(torch.float32, 64, 64, 64))
    n = ctypes.c_int()
    assert lib.bsattn_list_configs(7, 64, 64, 64, None, 0, ctypes.byref(n)) == UNSUP


A = 1 << 20  # fake, 16-byte-aligned, far-apart device addresses


def _fwd(lib, q=1 * A, k=3 * A, v=5 * A, mask=7 * A, out=9 * A, lse=11 * A, B=1, H=1, S=256,
         D=64, bq=64, bk=64, scale=0.125, dtype=1, ws=13 * A, wsb=1 << 20, cfg=None):
    p = lambda x: ctypes.c_void_p(x) if x else None
    c = ctypes.byref(bs.TileConfig(*cfg)) if cfg else None
    return lib.bsattn_fwd_config(p(q), p(k), p(v), p(mask), p(out), p(lse), B, H, S, D, bq, bk,
                                 scale, dtype, p(ws), wsb, c, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), NULL), (dict(k=0), NULL), (dict(v=0), NULL), (dict(mask=0), NULL),
    (dict(out=0), NULL), (dict(lse=0), NULL),
    (dict(B=0), SHAPE), (dict(H=-1), SHAPE), (dict(S=250), SHAPE), (dict(S=0), SHAPE),
    (dict(D=96), UNSUP), (dict(D=256), UNSUP), (dict(dtype=5), UNSUP), (dict(bq=32, S=256), UNSUP),
    (dict(bk=256), UNSUP),
    (dict(q=A + 8), ALIGN), (dict(out=9 * A + 4), ALIGN), (dict(lse=11 * A + 2), ALIGN),
    (dict(scale=math.nan), SCALE), (dict(scale=math.inf), SCALE), (dict(scale=-math.inf), SCALE),
    (dict(out=1 * A + 1024), ALIAS), (dict(lse=5 * A + 64), ALIAS), (dict(lse=9 * A), ALIAS),
    (dict(ws=0), WS), (dict(wsb=16), WS), (dict(ws=9 * A + 256), ALIAS), (dict(ws=3 * A), ALIAS),
    (dict(cfg=(256, 64, 8, 2)), UNSUP), (dict(cfg=(128, 64, 4, 2), bq=64), UNSUP),
    (dict(cfg=(64, 48, 2, 1)), UNSUP),
])
def test_fwd_argument_checks(lib, kw, code):
    assert _fwd(lib, **kw) == code


def test_fwd_head_size_limit(lib):
    """One head of K/V is read through a buffer with a 32-bit byte range, so S*D*4
    must stay below 2^31 (the sizes just under pass the shape checks and then fail
    on the fake, overlapping pointers)."""
    kw = dict(D=128, bq=128, bk=128)
    assert _fwd(lib, S=(1 << 22) - 128, **kw) not in (OK, SHAPE)
    assert _fwd(lib, S=1 << 22, **kw) == SHAPE


def test_env_config_parse_error(lib, monkeypatch):
    monkeypatch.setenv("BSATTN_CONFIG", "not-a-config")
    assert _fwd(lib) == UNSUP
    monkeypatch.setenv("BSATTN_CONFIG", "256,64,8,2")
    assert _fwd(lib) == UNSUP


def test_compact_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.bsattn_compact_mask
    assert f(None, 1, 1, 4, 4, p(A), p(2 * A), p(3 * A), 1 << 20, None) == NULL
    assert f(p(A), 0, 1, 4, 4, p(2 * A), p(3 * A), p(4 * A), 1 << 20, None) == SHAPE
    assert f(p(A), 1, 1, 4, 4, p(2 * A), p(3 * A), p(4 * A), 8, None) == WS
    assert f(p(A), 1, 1, 4, 4, p(2 * A + 2), p(3 * A), p(4 * A), 1 << 20, None) == ALIGN


def test_plan_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.bsattn_plan
    ok = [p(A), 1, 2, 512, 128, 64, p(3 * A), 1 << 20, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    assert call(0, None) == NULL and call(6, None) == NULL
    assert call(1, 0) == SHAPE and call(3, 500) == SHAPE and call(3, -512) == SHAPE
    assert call(4, 32) == UNSUP and call(5, 256) == UNSUP
    assert call(7, 64) == WS
    assert call(6, p(3 * A + 2)) == ALIGN
    # the workspace the plan writes overlapping the mask it reads (8 mask bytes at A)
    assert call(6, p(A - 256)) == ALIAS and call(6, p(A + 4)) == ALIAS


def test_planned_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.bsattn_fwd_planned
    ok = [p(A), p(3 * A), p(5 * A), p(9 * A), p(11 * A), 1, 1, 256, 64, 64, 64, 0.1, 1,
          p(13 * A), 1 << 20, None, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    assert call(13, None) == NULL and call(0, None) == NULL and call(3, None) == NULL
    assert call(7, 100) == SHAPE and call(8, 96) == UNSUP
    assert call(14, 16) == WS
    assert call(13, p(13 * A + 2)) == ALIGN
    assert call(13, p(9 * A + 512)) == ALIAS and call(13, p(11 * A)) == ALIAS
    assert call(3, p(1 * A)) == ALIAS
    assert call(11, math.nan) == SCALE
    assert call(15, ctypes.byref(bs.TileConfig(256, 64, 8, 2))) == UNSUP


def test_compacted_argument_checks(lib):
    p = ctypes.c_void_p
    f = lib.bsattn_fwd_compacted
    args = [p(A), p(3 * A), p(5 * A), p(7 * A), p(8 * A), 1024, p(9 * A), p(11 * A), 1, 1, 256, 64,
            64, 64, 0.1, 1, None, None]
    bad = list(args)
    bad[3] = None
    assert f(*bad) == NULL
    bad = list(args)
    bad[10] = 100
    assert f(*bad) == SHAPE
    bad = list(args)
    bad[14] = math.inf
    assert f(*bad) == SCALE


def test_autotune_argument_checks(lib):
    p = ctypes.c_void_p
    best = bs.TileConfig()
    n = ctypes.c_int()
    f = lib.bsattn_autotune
    base = [p(A), p(3 * A), p(5 * A), p(7 * A), p(9 * A), p(11 * A), 1, 1, 256, 64, 64, 64, 0.1,
            1, p(13 * A), 1 << 20, 1, 1, ctypes.byref(best), None, 0, ctypes.byref(n), None, None]
    bad = list(base)
    bad[18] = None
    assert f(*bad) == NULL
    bad = list(base)
    bad[17] = 0  # iters
    assert f(*bad) == SHAPE
    bad = list(base)
    bad[15] = 4
    assert f(*bad) == WS


def _cache_entry(S, BH, bucket, cfg, t=1.0e-4):
    return ('  {"dtype": 1, "D": 128, "block_q": 128, "block_k": 128, "S": %d, "BH": %d, '
            '"mask_bucket": %d, "tile_q": %d, "tile_k": %d, "waves": %d, "stages": %d, '
            '"t_mean_s": %.6e}' % ((S, BH, bucket) + tuple(cfg) + (t,)))


def test_tune_cache_roundtrip(lib, tmp_path):
    path = tmp_path / "tune.json"
    path.write_text('{"bsattn_tune_cache": 1, "entries": [\n' + _cache_entry(2048, 64, 8, (128, 32, 4, 3))
                    + '\n]}\n')
    lib.bsattn_clear_tune_cache()
    assert lib.bsattn_load_tune_cache(str(path).encode()) == OK
    assert lib.bsattn_load_tune_cache(str(tmp_path / "missing.json").encode()) == IO
    assert lib.bsattn_load_tune_cache(None) == NULL
    lib.bsattn_clear_tune_cache()


def test_tune_cache_keys_on_mask_statistic(lib, tmp_path):
    """Two masks of one shape (B*H = 64 heads of S = 2048, 1024 mask rows) with
    mean row lengths 16 (bucket 8) and 4 (bucket 4) keep separate entries;
    bsattn_tune_lookup picks by the caller's active-block count, and a call that
    does not know it (nnz < 0, like bsattn_fwd) gets the densest bucket."""
    path = tmp_path / "tune.json"
    path.write_text('{"bsattn_tune_cache": 1, "entries": [\n'
                    + _cache_entry(2048, 64, 4, (128, 64, 4, 2)) + ',\n'
                    + _cache_entry(2048, 64, 8, (256, 128, 8, 2)) + '\n]}\n')
    lib.bsattn_clear_tune_cache()
    assert lib.bsattn_load_tune_cache(str(path).encode()) == OK
    look = lambda nnz: bs.tune_lookup(__import__("torch").bfloat16, 128, 4, 16, 2048, 128, 128, nnz)
    assert look(16384).as_tuple() == (256, 128, 8, 2)      # 16 blocks per row
    assert look(4096).as_tuple() == (128, 64, 4, 2)        # 4 blocks per row
    assert look(4 * 1024 + 300).as_tuple() == (128, 64, 4, 2)  # same half-octave
    assert look(-1).as_tuple() == (256, 128, 8, 2)         # mask statistic unknown
    assert look(1024) is None                               # 1 block per row: not tuned
    assert bs.tune_lookup(__import__("torch").bfloat16, 128, 4, 16, 4096, 128, 128, -1) is None
    cfg = bs.TileConfig()
    f = lib.bsattn_tune_lookup
    assert f(1, 128, 4, 16, 2048, 128, 128, 16384, None) == NULL
    assert f(1, 128, 4, 16, 2000, 128, 128, 16384, ctypes.byref(cfg)) == SHAPE
    assert f(1, 128, 0, 16, 2048, 128, 128, 16384, ctypes.byref(cfg)) == SHAPE
    lib.bsattn_clear_tune_cache()
    assert look(16384) is None


def test_elem_argument_checks(lib):
    """Element-level masks: every call below fails a host check (fake pointers)."""
    p = ctypes.c_void_p
    f = lib.bsattn_fwd_elem
    # q k v states pidx bits n_tiles out lse B H S D bq bk scale dtype ws wsb cfg stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), p(8 * A), p(15 * A), 2, p(9 * A), p(11 * A),
          1, 1, 256, 64, 64, 64, 0.1, 1, p(13 * A), 16, None, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    assert call(3, None) == NULL and call(4, None) == NULL and call(5, None) == NULL
    assert call(0, None) == NULL
    assert call(6, 0) == SHAPE and call(6, 40000) == SHAPE and call(11, 100) == SHAPE
    assert call(13, 32) == UNSUP and call(12, 96) == UNSUP
    assert call(18, 16) == WS and call(17, None) == WS
    ok[18] = 4096  # enough workspace: alignment, aliasing and the config decide
    assert call(5, p(15 * A + 2)) == ALIGN and call(4, p(8 * A + 1)) == ALIGN
    assert call(17, p(3 * A + 128)) == ALIAS and call(16, 2) == UNSUP

    g = lib.bsattn_fwd_planned_elem
    # q k v out lse B H S D bq bk scale dtype bits n_tiles ws wsb cfg stream
    okp = [p(A), p(3 * A), p(5 * A), p(9 * A), p(11 * A), 1, 1, 256, 64, 64, 64, 0.1, 1,
           p(15 * A), 2, p(13 * A), 16, None, None]

    def callp(i, x):
        a = list(okp)
        a[i] = x
        return g(*a)
    assert callp(13, None) == NULL and callp(15, None) == NULL
    assert callp(14, 0) == SHAPE
    assert callp(16, 16) == WS
    # with a large enough workspace (1 KiB here) the alignment and alias checks decide
    okp[16] = 4096
    assert callp(13, p(15 * A + 1)) == ALIGN
    assert callp(13, p(9 * A + 64)) == ALIAS      # bit tiles overlap out
    assert callp(13, p(11 * A + 8)) == ALIAS      # ... lse
    assert callp(13, p(13 * A + 128)) == ALIAS    # ... the plan
    assert callp(15, p(5 * A + 64)) == ALIAS      # the plan overlaps v
    assert callp(12, 2) == UNSUP                  # no such dtype
    assert callp(8, 96) == UNSUP                  # no such head dimension

    h = lib.bsattn_plan_elem
    # states pidx n_tiles B H S bq bk ws wsb stream
    okh = [p(7 * A), p(8 * A), 2, 1, 1, 256, 64, 64, p(13 * A), 16, None]

    def callh(i, x):
        a = list(okh)
        a[i] = x
        return h(*a)
    assert callh(0, None) == NULL and callh(1, None) == NULL and callh(8, None) == NULL
    assert callh(2, 0) == SHAPE and callh(5, 250) == SHAPE
    assert callh(6, 32) == UNSUP
    assert callh(9, 16) == WS
    okh[9] = 4096
    assert callh(1, p(8 * A + 2)) == ALIGN and callh(8, p(13 * A + 2)) == ALIGN
    # the plan's workspace over the states or the tile index it reads
    assert callh(8, p(7 * A + 4)) == ALIAS and callh(8, p(8 * A - 64)) == ALIAS
    # one-shot forward: bit tiles over the workspace are refused before the plan runs
    ok[18] = 4096
    assert call(5, p(13 * A + 256)) == ALIAS


def test_elem_configs(lib):
    n = ctypes.c_int(-1)
    assert lib.bsattn_list_configs_elem(0, 64, 64, 64, None, 0, ctypes.byref(n)) == OK
    assert n.value == 2  # fp32: the two-wave kernel at 32- and 64-key steps (tile_q 64)
    for D in (64, 128):
        cfgs = bs.list_configs_elem(__import__("torch").bfloat16, D, 128, 128)
        assert len(cfgs) >= 3
        assert bs.list_configs_elem(__import__("torch").bfloat16, D, 64, 64)  # tile_q 64 too
        for c in cfgs:
            assert (c.tile_q, c.waves) in ((64, 2), (128, 4), (256, 8)) and c.stages in (2, 3)
        assert any(c.tile_q == 256 for c in cfgs)  # row pairs
        assert not any(c.tile_q == 256 for c in bs.list_configs_elem(__import__("torch").bfloat16, D, 64, 64))


def test_ragged_argument_checks(lib):
    """Ragged dot: every call below fails a host check (fake pointers)."""
    p = ctypes.c_void_p
    f = lib.bsattn_ragged_dot
    # lhs rhs sizes out M K N G dtype out_dtype ws wsb stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), 256, 128, 256, 4, 1, 0, p(9 * A), 16, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    for i in (0, 1, 2, 3, 10):
        assert call(i, None) == NULL
    assert call(4, 0) == SHAPE and call(7, 0) == SHAPE
    assert call(5, 96) == SHAPE and call(6, 200) == SHAPE          # K % 64, N % 128
    big = list(ok)
    big[5], big[6] = 1 << 20, 1024
    assert f(*big) == SHAPE                                         # one expert of 2 GiB
    assert call(8, 0) == UNSUP and call(9, 5) == UNSUP
    assert call(11, 16) == WS
    ok[11] = 1 << 16
    assert call(0, p(A + 8)) == ALIGN and call(2, p(5 * A + 2)) == ALIGN and call(10, p(9 * A + 4)) == ALIGN
    assert call(3, p(A + 64)) == ALIAS and call(10, p(7 * A + 256)) == ALIAS
    n = ctypes.c_size_t(0)
    assert lib.bsattn_ragged_dot_workspace_size(256, 4, ctypes.byref(n)) == OK
    assert n.value == (1 + 4 + 1) * 16 + 16
    g = lib.bsattn_ragged_plan
    assert g(None, 256, 4, p(9 * A), 4096, None) == NULL and g(p(5 * A), 0, 4, p(9 * A), 4096, None) == SHAPE
    assert g(p(5 * A), 256, 4, p(9 * A), 16, None) == WS and g(p(5 * A + 2), 256, 4, p(9 * A), 4096, None) == ALIGN
    assert g(p(5 * A), 256, 4, p(5 * A - 64), 4096, None) == ALIAS
    h = lib.bsattn_ragged_dot_planned
    okp = [p(A), p(3 * A), p(7 * A), 256, 128, 256, 4, 1, 0, p(9 * A), 16, None]

    def callp(i, x):
        a = list(okp)
        a[i] = x
        return h(*a)
    assert callp(0, None) == NULL and callp(9, None) == NULL and callp(5, 100) == SHAPE
    assert callp(10, 16) == WS and callp(7, 0) == UNSUP
    okp[10] = 4096
    assert callp(2, p(A + 64)) == ALIAS and callp(9, p(9 * A + 8)) == ALIGN
    assert lib.bsattn_ragged_dot_workspace_size(0, 4, ctypes.byref(n)) == SHAPE


def test_bwd_argument_checks(lib):
    """Backward: every call below fails a host check (fake pointers)."""
    p = ctypes.c_void_p
    B, H, S, D, bq, bk = 1, 2, 256, 128, 128, 64
    n = ctypes.c_size_t(0)
    assert lib.bsattn_bwd_workspace_size(B, H, S, bq, bk, ctypes.byref(n)) == OK
    rnd = lambda x: (x + 255) // 256 * 256
    R, nk, nq = B * H * (S // bq), S // bk, S // bq
    fwd = ctypes.c_size_t(0)
    assert lib.bsattn_workspace_size(B, H, S, bq, bk, ctypes.byref(fwd)) == OK
    C = B * H * nk
    slots = max(16, (C // 4 + 1) & ~1)
    assert n.value == (fwd.value + rnd(C * 4) + rnd(C * nq * 4) + rnd((C + slots) * 16) + rnd(slots // 2 * 16)
                       + rnd(8) + rnd(B * H * S * 8) + rnd(slots * 2 * bk * 128 * 4))
    wsn = n.value
    assert lib.bsattn_bwd_workspace_size(B, H, 250, bq, bk, ctypes.byref(n)) == SHAPE
    assert lib.bsattn_bwd_workspace_size(B, H, S, bq, bk, None) == NULL

    f = lib.bsattn_bwd
    # q k v out lse dout mask B H S D bq bk scale dtype dq dk dv gdtype ws wsb stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), p(9 * A), p(11 * A), p(13 * A), B, H, S, D, bq, bk, 0.1, 1,
          p(15 * A), p(17 * A), p(19 * A), 1, p(21 * A), wsn, None]

    def call(i, x, base=ok):
        a = list(base)
        a[i] = x
        return f(*a)
    for i in (0, 1, 2, 3, 4, 5, 6, 15, 16, 17, 19):
        assert call(i, None) == NULL, i
    assert call(9, 250) == SHAPE and call(7, 0) == SHAPE
    assert call(10, 96) == UNSUP and call(11, 32) == UNSUP and call(14, 0) == UNSUP  # D, block, fp32 inputs
    assert call(18, 7) == UNSUP
    assert call(20, wsn - 1) == WS
    for i in (0, 3, 5, 15, 19):
        assert call(i, p(ok[i].value + 8)) == ALIGN, i
    assert call(4, p(9 * A + 2)) == ALIGN
    assert call(13, float("nan")) == SCALE and call(13, math.inf) == SCALE
    assert call(19, p(3 * A + 64)) == ALIAS                 # workspace over k
    assert call(15, p(A + 128)) == ALIAS                    # dq over q
    assert call(16, p(15 * A + 64)) == ALIAS                # dk over dq
    assert call(17, p(9 * A)) == ALIAS                      # dv over lse
    g = lib.bsattn_bwd_plan
    assert g(None, B, H, S, bq, bk, p(21 * A), wsn, None) == NULL
    assert g(p(13 * A), B, H, S, 32, bk, p(21 * A), wsn, None) == UNSUP
    assert g(p(13 * A), B, H, S, bq, bk, p(21 * A), 64, None) == WS
    assert g(p(13 * A), B, H, S, bq, bk, p(21 * A + 4), wsn, None) == ALIGN
    assert g(p(13 * A), B, H, S, bq, bk, p(13 * A - 64), wsn, None) == ALIAS
    h = lib.bsattn_bwd_planned
    okp = ok[:6] + ok[7:19] + [7] + ok[19:]

    def callp(i, x):
        a = list(okp)
        a[i] = x
        return h(*a)
    for i in (0, 5, 14, 19):
        assert callp(i, None) == NULL, i
    assert callp(20, 64) == WS and callp(13, 0) == UNSUP and callp(9, 96) == UNSUP
    assert callp(18, 0) == UNSUP and callp(18, 8) == UNSUP   # parts
    assert callp(14, p(11 * A + 32)) == ALIAS               # dq over dout
    assert callp(19, p(15 * A + 64)) == ALIAS               # workspace over dq


def test_fp8_argument_checks(lib):
    """fp8 forward: every call below fails a host check (fake pointers)."""
    p = ctypes.c_void_p
    B, H, S, D, bq, bk = 1, 2, 256, 128, 128, 64
    n = ctypes.c_size_t(0)
    assert lib.bsattn_fp8_workspace_size(B, H, S, D, bq, bk, ctypes.byref(n)) == OK
    fwd = ctypes.c_size_t(0)
    assert lib.bsattn_workspace_size(B, H, S, bq, bk, ctypes.byref(fwd)) == OK
    rnd = lambda x: (x + 255) // 256 * 256
    assert n.value == fwd.value + rnd(B * H * S * D)
    wsn = n.value
    f = lib.bsattn_fwd_fp8
    # q k v mask out lse B H S D bq bk scale ws wsb stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), p(9 * A), p(11 * A), B, H, S, D, bq, bk, 0.1, p(13 * A), wsn, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    for i in (0, 1, 2, 3, 4, 5, 13):
        assert call(i, None) == NULL, i
    assert call(8, 250) == SHAPE and call(9, 96) == UNSUP and call(10, 32) == UNSUP
    assert call(14, wsn - 1) == WS
    assert call(0, p(A + 8)) == ALIGN and call(4, p(9 * A + 8)) == ALIGN and call(13, p(13 * A + 8)) == ALIGN
    assert call(12, float("nan")) == SCALE
    assert call(4, p(A + 64)) == ALIAS                  # out over q
    assert call(13, p(5 * A + 64)) == ALIAS             # workspace over v
    g = lib.bsattn_fwd_fp8_planned
    okp = ok[:3] + ok[4:]
    assert g(*(okp[:12] + [p(13 * A), 64, None])) == WS
    assert g(*(okp[:12] + [None, wsn, None])) == NULL

    # element masks: q k v states pidx bits n_tiles out lse B H S D bq bk scale ws wsb stream
    fe = lib.bsattn_fwd_fp8_elem
    oke = [p(A), p(3 * A), p(5 * A), p(7 * A), p(8 * A), p(15 * A), 2, p(9 * A), p(11 * A),
           B, H, S, D, bq, bk, 0.1, p(13 * A), wsn, None]

    def calle(i, x):
        a = list(oke)
        a[i] = x
        return fe(*a)
    for i in (0, 3, 4, 5, 7, 16):
        assert calle(i, None) == NULL, i
    assert calle(6, 0) == SHAPE and calle(6, 40000) == SHAPE and calle(11, 250) == SHAPE
    assert calle(12, 96) == UNSUP and calle(14, 32) == UNSUP
    assert calle(17, wsn - 1) == WS
    assert calle(5, p(15 * A + 2)) == ALIGN and calle(4, p(8 * A + 1)) == ALIGN
    assert calle(15, float("inf")) == SCALE
    assert calle(5, p(9 * A + 64)) == ALIAS              # bit tiles over out
    assert calle(5, p(13 * A + 512)) == ALIAS            # ... over the workspace
    assert calle(16, p(5 * A + 64)) == ALIAS             # workspace over v
    ge = lib.bsattn_fwd_fp8_planned_elem
    # q k v out lse B H S D bq bk scale bits n_tiles ws wsb stream
    okq = [p(A), p(3 * A), p(5 * A), p(9 * A), p(11 * A), B, H, S, D, bq, bk, 0.1, p(15 * A), 2,
           p(13 * A), wsn, None]

    def callq(i, x):
        a = list(okq)
        a[i] = x
        return ge(*a)
    assert callq(12, None) == NULL and callq(14, None) == NULL
    assert callq(13, 0) == SHAPE and callq(15, 64) == WS
    assert callq(12, p(15 * A + 1)) == ALIGN
    assert callq(12, p(11 * A + 8)) == ALIAS and callq(12, p(13 * A + 128)) == ALIAS


def test_c_program_builds(lib):
    """The plain-C user of the ABI (tests/c_abi_fwd.c, run by the GPU tests) compiles
    and links against libbsattn.so, liboracle.so and the HIP runtime."""
    import c_abi_build
    import oracle
    oracle.build(force=False)
    exe = c_abi_build.build(force=True)
    assert os.access(exe, os.X_OK)


def test_bwd_elem_argument_checks(lib):
    """Backward with element-level masks: the element arguments' host checks, and
    the backward's own checks still reached through this entry point."""
    p = ctypes.c_void_p
    B, H, S, D, bq, bk = 1, 2, 256, 128, 128, 64
    n = ctypes.c_size_t(0)
    assert lib.bsattn_bwd_workspace_size(B, H, S, bq, bk, ctypes.byref(n)) == OK
    f = lib.bsattn_bwd_elem
    # q k v out lse dout states pidx pbits n_tiles B H S D bq bk scale dtype dq dk dv gdtype ws wsb stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), p(9 * A), p(11 * A), p(13 * A), p(14 * A), p(15 * A), 2,
          B, H, S, D, bq, bk, 0.1, 1, p(17 * A), p(19 * A), p(21 * A), 1, p(23 * A), n.value, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)
    for i in (0, 6, 7, 8, 18, 22):
        assert call(i, None) == NULL, i
    assert call(9, 0) == SHAPE and call(9, 40000) == SHAPE       # n_tiles
    assert call(12, 250) == SHAPE                                  # S
    assert call(7, p(14 * A + 2)) == ALIGN and call(8, p(15 * A + 1)) == ALIGN
    assert call(13, 96) == UNSUP                                   # D
    assert call(22, p(15 * A)) == ALIAS                            # workspace over the bit tiles
    assert call(23, n.value - 1) == WS


# ---- the Python binding refuses bad tensor arguments before any library call ----

def test_binding_refuses_host_tensors():
    import torch
    q = torch.zeros(1, 1, 128, 64, dtype=torch.bfloat16)
    m = torch.ones(1, 1, 1, 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="GPU"):
        bs.fwd(q, q, q, m, 128, 128)
    with pytest.raises(ValueError, match="GPU"):
        bs.plan(m, 128, 128, 128)
    with pytest.raises(ValueError, match="GPU"):
        bs.ragged_dot(torch.zeros(4, 8, dtype=torch.bfloat16), torch.zeros(1, 8, 8, dtype=torch.bfloat16),
                      torch.zeros(1, dtype=torch.int32))
    with pytest.raises(TypeError):
        bs.fwd(None, q, q, m, 128, 128)


def test_binding_tensor_checks():
    """_check_tensor, the check every mask, index, bit-tile, output, gradient and
    workspace tensor goes through (here with host tensors standing in for the
    device one): device, contiguity, dtype, shape and size."""
    import torch
    cpu = torch.device("cpu")
    t = torch.zeros(2, 3, dtype=torch.int32)
    assert bs._check_tensor(t, "t", cpu, (torch.int32,), (2, 3), 24) is t
    with pytest.raises(ValueError, match="must be on"):
        bs._check_tensor(t, "t", torch.device("meta"))
    with pytest.raises(ValueError, match="contiguous"):
        bs._check_tensor(t.t(), "t", cpu)
    with pytest.raises(TypeError, match="dtype"):
        bs._check_tensor(t, "t", cpu, (torch.float32,))
    with pytest.raises(ValueError, match="shape"):
        bs._check_tensor(t, "t", cpu, shape=(3, 2))
    with pytest.raises(ValueError, match="too small"):
        bs._check_tensor(t, "t", cpu, min_bytes=25)
    with pytest.raises(TypeError):
        bs._check_tensor([1, 2], "t", cpu)
    # masks: bool is viewed as uint8, other dtypes refused; device and shape checked
    m = torch.ones(1, 2, 3, 3, dtype=torch.bool)
    assert bs._mask_u8(m, cpu, (1, 2, 3, 3)).dtype == torch.uint8
    with pytest.raises(TypeError):
        bs._mask_u8(m.to(torch.int32), cpu)
    with pytest.raises(ValueError, match="shape"):
        bs._mask_u8(m, cpu, (1, 2, 3, 4))
    with pytest.raises(ValueError, match="must be on"):
        bs._mask_u8(m, torch.device("meta"), (1, 2, 3, 3))
    # element-mask tensors
    st = torch.zeros(1, 2, 3, 3, dtype=torch.uint8)
    pidx = torch.zeros(1, 2, 3, 3, dtype=torch.int32)
    bits = torch.zeros(2, 128, 4, dtype=torch.int32)
    assert bs._elem_tensors(st, pidx, bits, cpu, (1, 2, 3, 3)) == 2
    with pytest.raises(ValueError):
        bs._elem_tensors(st, pidx[:, :, :2].contiguous(), bits, cpu)
    with pytest.raises(TypeError):
        bs._elem_tensors(st, pidx.to(torch.int64), bits, cpu)
    with pytest.raises(ValueError):
        bs._check_bits(bits, 128, 64)
    # outputs: given out / lse must match q's shape and dtype
    q = torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16)
    o, l = bs._outputs(q, None, None)
    assert o.shape == q.shape and o.dtype == q.dtype and l.shape == (1, 2, 256) and l.dtype == torch.float32
    with pytest.raises(TypeError):
        bs._outputs(q, torch.zeros(1, 2, 256, 64), None)
    with pytest.raises(ValueError):
        bs._outputs(q, None, torch.zeros(1, 2, 255))
    with pytest.raises(ValueError):
        bs._outputs(q, torch.zeros(1, 2, 256, 63, dtype=torch.bfloat16), None)
    # gradients
    with pytest.raises(ValueError):
        bs._grads(q, None, torch.zeros(1, 2, 256, 64, dtype=torch.bfloat16), None,
                  torch.zeros(1, 2, 256, 64, dtype=torch.float32))
    with pytest.raises(TypeError):
        bs._grads(q, torch.float16, None, None, None)
    with pytest.raises(ValueError, match="multiple"):
        bs._mask_shape(q.shape, 128, 96)
    # workspaces
    with pytest.raises(ValueError, match="too small"):
        bs._workspace(1000, cpu, torch.zeros(999, dtype=torch.uint8))


def test_noalloc_argument_checks(lib):
    """bsattn_fwd_noalloc: host checks as bsattn_fwd_config, and a plan larger
    than the fixed array (bsattn_noalloc_max_bytes) is refused before any HIP call."""
    p = ctypes.c_void_p
    f = lib.bsattn_fwd_noalloc
    assert lib.bsattn_noalloc_max_bytes() == 16 << 20
    # q k v mask out lse B H S D bq bk scale dtype cfg stream
    ok = [p(A), p(3 * A), p(5 * A), p(7 * A), p(9 * A), p(11 * A), 1, 1, 256, 64, 64, 64, 0.1, 1, None, None]

    def call(i, x):
        a = list(ok)
        a[i] = x
        return f(*a)

    assert call(3, None) == NULL and call(0, None) == NULL and call(5, None) == NULL
    assert call(8, 100) == SHAPE and call(9, 96) == UNSUP
    assert call(12, math.nan) == SCALE
    assert call(4, p(1 * A)) == ALIAS
    assert call(14, ctypes.byref(bs.TileConfig(256, 64, 8, 2))) == UNSUP  # no pairs for block_q 64
    # 64 heads of 512 x 512 blocks: the plan needs more than 16 MiB
    big = list(ok)
    big[7], big[8], big[10], big[11] = 64, 65536, 128, 128
    big[0], big[1], big[2], big[4], big[5] = p(1 << 40), p(2 << 40), p(3 << 40), p(4 << 40), p(5 << 40)
    assert f(*big) == WS
