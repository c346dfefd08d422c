"""The C ABI library: loads, exports every declared symbol, validates
arguments before any HIP call (these calls return early; nothing runs)."""

import ctypes
import math
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "ssa.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(ssa_[a-z_0-9]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def lib():
    import sparse_attention_long_skip_amd as ssa
    if not os.path.exists(ssa.LIB_PATH):
        pytest.fail("libssa.so is not built (run __graft_entry__.build())")
    return ssa.lib()


def test_every_declared_symbol_is_exported(lib):
    names = _declared()
    assert {"ssa_prefill", "ssa_decode", "ssa_block_mask"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_helpers(lib):
    import sparse_attention_long_skip_amd as ssa
    for st in (0, -1, -2, -3, -4, -5):
        assert ssa.status_string(st).startswith("SSA")
    assert ssa.abi_version() == 101
    lam = ssa.lambda_from_scale_factor(1000.0, 131072)
    assert abs(lam - math.log(1000.0 / 131072)) < 1e-5
    assert ssa.lambda_from_scale_factor(1e9, 10) == 0.0
    assert math.isnan(ssa.lambda_from_scale_factor(-1.0, 10))
    assert ssa.block_mask_max_blocks(32768, 64, 64, 1, 1024) == 81
    assert ssa.block_mask_max_blocks(1000, 64, 64, 1, 1024) == 16
    # partials, then the 256-byte block of the work counter
    assert ssa.decode_workspace_size(32, 32, 32768, 128, 64, 32) == 32 * 32 * 16 * 130 * 4 + 256
    assert ssa.decode_workspace_size(0, 32, 32768, 128, 64, 32) == 0


FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced


def _prefill(lib, **kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, out=FAKE, B=1, Hq=4, Hkv=2, L=128, d=128, Br=128, Bc=64,
             lam=-1.0, causal=1, bi=None, bc=None, mb=0)
    a.update(kw)
    return lib.ssa_prefill(a["q"], a["k"], a["v"], a["out"], None, None, None, None, a["B"], a["Hq"],
                           a["Hkv"], a["L"], a["d"], a["Br"], a["Bc"], ctypes.c_float(a["lam"]),
                           a["causal"], a["bi"], a["bc"], a["mb"], None)


def test_prefill_validation(lib):
    assert _prefill(lib, q=None) == -1
    assert _prefill(lib, Hq=3) == -1            # Hq % Hkv != 0
    assert _prefill(lib, L=0) == -1
    assert _prefill(lib, lam=0.5) == -1          # lambda > 0
    assert _prefill(lib, lam=float("nan")) == -1
    assert _prefill(lib, causal=2) == -1
    assert _prefill(lib, q=FAKE + 2) == -1       # misaligned
    assert _prefill(lib, bi=FAKE) == -1          # block_idx without block_cnt
    assert _prefill(lib, bi=FAKE, bc=FAKE, mb=0) == -1
    assert _prefill(lib, d=96) == -2
    assert _prefill(lib, Br=16) == -2
    assert _prefill(lib, Br=32, bi=FAKE, bc=FAKE, mb=4) == -2
    assert _prefill(lib, Bc=128) == -2


def _decode(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, S=1024, d=128, Bc=64,
             T=4, lam=-1.0, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.ssa_decode(a["q"], a["kc"], a["vc"], a["sl"], a["out"], None, None, None, None, a["B"],
                          a["Hq"], a["Hkv"], a["S"], a["d"], a["Bc"], a["T"], ctypes.c_float(a["lam"]),
                          a["ws"], a["wsb"], None)


def test_decode_validation(lib):
    assert _decode(lib, sl=None) == -1
    assert _decode(lib, T=0) == -1
    assert _decode(lib, lam=1.0) == -1
    assert _decode(lib, Hq=7) == -1             # 7 % 2 != 0
    assert _decode(lib, Hq=12, Hkv=4) == -2     # G = 3 not built
    assert _decode(lib, d=80) == -2
    assert _decode(lib, ws=None) == -3
    assert _decode(lib, wsb=16) == -3
    # splits are numbered by a 32-bit work counter: B * Hkv * nS < 2^31
    # (4096 * 512 * 1024 = 2^31 splits with S_max = 65536, one-tile splits)
    assert _decode(lib, B=4096, Hq=512, Hkv=512, S=65536, T=1) == -2
    assert _decode(lib, B=4095, Hq=512, Hkv=512, S=65536, T=1) == -3   # fits; workspace too small


def _decode_noalloc(lib, **kw):
    a = dict(q=FAKE, kc=FAKE, vc=FAKE, sl=FAKE, out=FAKE, B=2, Hq=8, Hkv=2, S=1024, d=128, Bc=64,
             T=4, lam=-1.0)
    a.update(kw)
    return lib.ssa_decode_noalloc(a["q"], a["kc"], a["vc"], a["sl"], a["out"], None, None, None, None,
                                  a["B"], a["Hq"], a["Hkv"], a["S"], a["d"], a["Bc"], a["T"],
                                  ctypes.c_float(a["lam"]), None)


def test_decode_noalloc_validation(lib):
    import sparse_attention_long_skip_amd as ssa
    # the decode checks apply unchanged
    assert _decode_noalloc(lib, sl=None) == -1
    assert _decode_noalloc(lib, T=0) == -1
    assert _decode_noalloc(lib, lam=1.0) == -1
    assert _decode_noalloc(lib, Hq=12, Hkv=4) == -2
    # partials beyond the static scratch are refused before any HIP call:
    # B=32, Hq=32, S_max=8192, split 2 tiles -> 64 splits of 130 floats = 34.1 MB
    need = ssa.decode_workspace_size(32, 32, 8192, 128, 64, 2)
    assert need > ssa.DECODE_SCRATCH_BYTES
    assert _decode_noalloc(lib, B=32, Hq=32, Hkv=8, S=8192, T=2) == ssa.SSA_ERR_SCRATCH
    assert ssa.status_string(ssa.SSA_ERR_SCRATCH).startswith("SSA_ERR_SCRATCH")
    # the 32-sequence decode workload (16-tile splits: 17.0 MB) fits
    assert ssa.decode_workspace_size(32, 32, 32768, 128, 64, 16) <= ssa.DECODE_SCRATCH_BYTES


def _mask(lib, **kw):
    a = dict(q=FAKE, k=FAKE, B=1, H=2, L=32768, d=64, pool=64, topk=64, sink=1, win=1024, causal=1,
             bi=FAKE, bc=FAKE, mb=81, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.ssa_block_mask(a["q"], a["k"], a["B"], a["H"], a["L"], a["d"], a["pool"], a["topk"],
                              a["sink"], a["win"], a["causal"], a["bi"], a["bc"], a["mb"], None,
                              a["ws"], a["wsb"], None)


def test_mask_validation(lib):
    assert _mask(lib, bi=None) == -1
    assert _mask(lib, topk=-1) == -1
    assert _mask(lib, mb=80) == -1
    assert _mask(lib, causal=0) == -2
    assert _mask(lib, pool=32, mb=200) == -2
    assert _mask(lib, d=32) == -2
    assert _mask(lib, L=64 * 5000, mb=81) == -2
    assert _mask(lib, ws=None) == -3
    assert _mask(lib, wsb=100) == -3


def test_prefill_nm_validation(lib):
    def call(n, m, sink=0, recent=0, d=128):
        return lib.ssa_prefill_nm(FAKE, FAKE, FAKE, FAKE, None, None, None, None, 1, 2, 1, 128, d, 128, 64,
                                  ctypes.c_float(-1.0), 1, n, m, sink, recent, None)
    assert call(0, 4) == -1
    assert call(5, 4) == -1
    assert call(2, 4, sink=-1) == -1
    assert call(2, 4, recent=-3) == -1
    assert call(2, 8) == -2
    assert call(1, 3) == -2
    assert call(2, 4, d=96) == -2


def _sparge(lib, **kw):
    a = dict(q=FAKE, k=FAKE, B=1, H=2, L=32768, d=64, pool=64, theta=0.3, tau=0.9, mode=0, causal=1,
             bi=FAKE, bc=FAKE, mb=512, ws=FAKE, wsb=1 << 30)
    a.update(kw)
    return lib.ssa_sparge_mask(a["q"], a["k"], a["B"], a["H"], a["L"], a["d"], a["pool"],
                               ctypes.c_float(a["theta"]), ctypes.c_double(a["tau"]), a["mode"],
                               a["causal"], a["bi"], a["bc"], a["mb"], None, None, a["ws"], a["wsb"],
                               None)


def test_sparge_validation(lib):
    assert _sparge(lib, bc=None) == -1
    assert _sparge(lib, theta=float("nan")) == -1
    assert _sparge(lib, tau=0.0) == -1
    assert _sparge(lib, tau=1.5) == -1
    assert _sparge(lib, tau=float("nan")) == -1
    assert _sparge(lib, mode=2) == -1
    assert _sparge(lib, mb=511) == -1
    assert _sparge(lib, causal=0) == -2
    assert _sparge(lib, pool=32, mb=1024) == -2
    assert _sparge(lib, d=32) == -2
    assert _sparge(lib, L=64 * 5000, mb=5000) == -2
    assert _sparge(lib, ws=None) == -3
    need = lib.ssa_sparge_mask_workspace_size(1, 2, 32768, 64, 64)
    assert need == 2 * 2 * 512 * 64 * 4 + 2 * 2 * 512 * 4
    assert _sparge(lib, wsb=need - 1) == -3


def test_compressed_mask_validation(lib):
    def call(kernel=32, stride=16, **kw):
        a = dict(q=FAKE, k=FAKE, B=1, H=2, L=32768, d=64, pool=64, topk=64, sink=1, win=1024,
                 causal=1, bi=FAKE, bc=FAKE, mb=81, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.ssa_block_mask_compressed(a["q"], a["k"], a["B"], a["H"], a["L"], a["d"], a["pool"],
                                             kernel, stride, a["topk"], a["sink"], a["win"], a["causal"],
                                             a["bi"], a["bc"], a["mb"], None, a["ws"], a["wsb"], None)
    assert call(kernel=0) == -1
    assert call(stride=-1) == -1
    assert call(bi=None) == -1
    assert call(mb=80) == -1
    assert call(kernel=64, stride=32) == -2
    assert call(causal=0) == -2
    need = lib.ssa_block_mask_compressed_workspace_size(1, 2, 32768, 64, 64)
    assert need == 2 * (512 + 2048) * 64 * 4
    assert call(wsb=need - 1) == -3


def test_vertical_slash_validation(lib):
    def call(**kw):
        a = dict(q=FAKE, k=FAKE, B=1, H=2, L=32768, d=64, R=64, nv=1000, ns=64, pool=64, causal=1,
                 bi=FAKE, bc=FAKE, mb=512, ws=FAKE, wsb=1 << 30)
        a.update(kw)
        return lib.ssa_vertical_slash_mask(a["q"], a["k"], a["B"], a["H"], a["L"], a["d"], a["R"],
                                           a["nv"], a["ns"], a["pool"], a["causal"], a["bi"], a["bc"],
                                           a["mb"], None, None, None, None, a["ws"], a["wsb"], None)
    assert call(q=None) == -1
    assert call(R=0) == -1
    assert call(R=40000) == -1
    assert call(nv=-1) == -1
    assert call(ns=-2) == -1
    assert call(mb=511) == -1
    assert call(R=65) == -2
    assert call(pool=32, mb=1024) == -2
    assert call(d=96) == -2
    assert call(causal=0) == -2
    assert call(ws=None) == -3
    need = lib.ssa_vertical_slash_workspace_size(1, 2, 32768)
    assert need > 2 * 2 * 32768 * 4
    assert call(wsb=need - 1) == -3
