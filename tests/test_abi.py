"""The C-ABI library on the host: it loads, exports every entry point the header declares, sizes
workspaces, and rejects bad arguments with the documented status before launching anything.

No call here reaches a kernel launch, so these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import lm_head_log_lmhead_amd as lmh

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lmhead_logprob.h")


def _declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"LMH_API\s+[\w\s\*]+?\b(lmhead_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(lmh.LIB_PATH):
        pytest.fail("HIP library not built; run __graft_entry__.build() first")
    return lmh.lib()


def test_header_declares_the_entry_points():
    syms = _declared_symbols()
    for name in ("lmhead_logprob_fwd", "lmhead_logprob_bwd", "lmhead_logprob_fwd_workspace_size",
                 "lmhead_logprob_bwd_workspace_size", "lmhead_status_string",
                 "lmhead_logprob_fwd_partials", "lmhead_logprob_fwd_finalize"):
        assert name in syms
    assert set(syms) == set(lmh._SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol(lib):
    raw = ctypes.CDLL(lmh.LIB_PATH)
    for name in _declared_symbols():
        assert hasattr(raw, name), f"missing export {name}"


def test_status_strings(lib):
    for code in range(5):
        assert len(lmh.lmhead_status_string(code)) > 0
    assert lmh.lmhead_status_string(0) == "ok"
    assert "unknown" in lmh.lmhead_status_string(99)


def test_workspace_sizes(lib):
    T, H, V = 8192, 4096, 152064
    n_c = (V + 127) // 128
    fwd = lmh.lmhead_logprob_fwd_workspace_size(T, H, V)
    assert fwd >= n_c * T * 20 + T * 4 and fwd % 256 == 0
    assert lmh.lmhead_logprob_fwd_workspace_size(0, H, V) > 0       # the scheduler counters
    assert lmh.lmhead_logprob_fwd_workspace_size(4, 12, 10) == 0     # H % 8 != 0
    assert lmh.lmhead_logprob_fwd_workspace_size(-1, 8, 10) == 0
    assert lmh.lmhead_logprob_fwd_workspace_size(4, 8, 0) == 0
    # at most 2^36 (row, 128-column chunk) records: 1188 chunks x 2^26 rows is past it
    assert lmh.lmhead_logprob_fwd_workspace_size(1 << 26, 8, V) == 0
    assert lmh.lmhead_logprob_fwd_workspace_size(1 << 25, 8, V) > 0
    bwd = lmh.lmhead_logprob_bwd_workspace_size(4096, 5120, V)
    assert bwd >= 4096 * 16384 * 2 * 2 + 5120 * 16384 * 2 + 5120 * 4096 * 2
    # the workspace grows linearly in T for the forward
    assert lmh.lmhead_logprob_fwd_workspace_size(2 * T, H, V) > fwd
    # few tiles per compute unit: the fast size adds the K-split schedule's accumulator slots (256 of
    # 256 x 256 fp32) and its counter, flags and ranges; the smallest accepted size leaves them out
    assert lmh.lmhead_logprob_fwd_workspace_size_min(T, H, V) == fwd        # 594 x 32 tiles: no split
    for t in (192, 200, 256):                                               # 594 tiles
        lo, hi = lmh.lmhead_logprob_fwd_workspace_size_min(t, H, V), lmh.lmhead_logprob_fwd_workspace_size(t, H, V)
        assert hi - lo == 256 * 256 * 256 * 4 + 5376 and lo >= n_c * t * 20 + t * 4  # slots + counter, flags, ranges
    for t in (1, 64, 128, 129, 191, 257, 2048):                             # below 192, or two token tiles
        assert lmh.lmhead_logprob_fwd_workspace_size(t, H, V) == lmh.lmhead_logprob_fwd_workspace_size_min(t, H, V)
    assert lmh.lmhead_logprob_fwd_workspace_size_min(4, 12, 10) == 0


def _fwd(lib, hidden=16, weight=16, labels=16, T=4, H=8, V=10, logprob=16, entropy=None, lse=None,
         ws=256, ws_bytes=1 << 20):
    return lib.lmhead_logprob_fwd(hidden, weight, labels, T, H, V, logprob, entropy, lse, ws, ws_bytes, None)


def test_fwd_validation_codes(lib):
    # Fake, never-dereferenced addresses: validation fails before anything is launched.
    assert _fwd(lib, hidden=None) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, logprob=None) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, T=-1) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, V=0) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, H=12) == lmh.LMH_ERR_UNSUPPORTED
    assert _fwd(lib, H=0) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, V=2**31 - 1) == lmh.LMH_ERR_UNSUPPORTED
    # the header's bounds: V < 2^31 - 2^16 and T < 2^31 - 2^16 (tile-rounded indices stay in int32)
    assert lmh.lmhead_logprob_fwd_workspace_size(1, 8, 2**31 - 2**16) == 0
    assert lmh.lmhead_logprob_fwd_workspace_size(1, 8, 2**31 - 2**16 - 1) > 0
    assert lmh.lmhead_logprob_fwd_workspace_size(2**31 - 2**16, 8, 128) == 0
    assert lmh.lmhead_logprob_fwd_workspace_size(2**31 - 2**16 - 1, 8, 128) > 0
    assert _fwd(lib, H=8 * (1 << 20)) == lmh.LMH_ERR_UNSUPPORTED
    assert _fwd(lib, T=1 << 26, V=152064) == lmh.LMH_ERR_UNSUPPORTED  # more than 2^36 records
    assert _fwd(lib, hidden=24) == lmh.LMH_ERR_UNSUPPORTED          # not 16-byte aligned
    assert _fwd(lib, labels=18) == lmh.LMH_ERR_UNSUPPORTED
    assert _fwd(lib, entropy=2) == lmh.LMH_ERR_UNSUPPORTED
    assert _fwd(lib, ws_bytes=16) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert _fwd(lib, ws=None) == lmh.LMH_ERR_INVALID_ARG
    assert _fwd(lib, ws=128) == lmh.LMH_ERR_UNSUPPORTED             # workspace not 256-aligned
    # T == 0: OK, nothing launched, even with null pointers
    assert _fwd(lib, T=0, hidden=None, weight=None, labels=None, logprob=None, ws=None, ws_bytes=0) == lmh.LMH_OK


def test_stage_validation_codes(lib):
    assert lib.lmhead_logprob_fwd_partials(None, 16, 16, 4, 8, 10, 256, 1 << 20, None) == lmh.LMH_ERR_INVALID_ARG
    assert lib.lmhead_logprob_fwd_partials(16, 16, 16, 4, 8, 10, 256, 8, None) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert lib.lmhead_logprob_fwd_finalize(16, 4, 8, 10, None, None, None, 256, 1 << 20, None) == lmh.LMH_ERR_INVALID_ARG
    assert lib.lmhead_logprob_fwd_finalize(None, 4, 8, 10, 16, None, None, 256, 1 << 20, None) == lmh.LMH_ERR_INVALID_ARG
    assert lib.lmhead_logprob_fwd_finalize(16, 0, 8, 10, None, None, None, None, 0, None) == lmh.LMH_OK


def test_bwd_validation_codes(lib):
    ok = dict(h=16, w=16, y=16, T=4, H=8, V=10, g=16, lse=16, gh=16, gw=16, acc=0, ws=256, wsb=1 << 30)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return lib.lmhead_logprob_bwd(a["h"], a["w"], a["y"], a["T"], a["H"], a["V"], a["g"], a["lse"], a["gh"],
                                      a["gw"], a["acc"], a["ws"], a["wsb"], None)

    assert call(g=None) == lmh.LMH_ERR_INVALID_ARG
    assert call(lse=None) == lmh.LMH_ERR_INVALID_ARG
    assert call(acc=2) == lmh.LMH_ERR_INVALID_ARG
    assert call(H=10) == lmh.LMH_ERR_UNSUPPORTED
    assert call(gh=6) == lmh.LMH_ERR_UNSUPPORTED
    assert call(wsb=64) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert call(T=0, h=None, w=None, y=None, g=None, lse=None) == lmh.LMH_OK
    # no gradient requested: validated, nothing to do
    assert call(gh=None, gw=None) == lmh.LMH_OK


def test_extended_entry_validation_codes(lib):
    nan = float("nan")

    def fwd_ex(temp=1.0, **kw):
        a = dict(h=16, w=16, y=16, T=4, H=8, V=10, lp=16, ent=None, lse=None, p2=None, ws=256, wsb=1 << 20)
        a.update(kw)
        return lib.lmhead_logprob_fwd_ex(a["h"], a["w"], a["y"], a["T"], a["H"], a["V"], temp, a["lp"], a["ent"],
                                         a["lse"], a["p2"], a["ws"], a["wsb"], None)

    for bad in (0.0, -0.7, nan, float("inf")):
        assert fwd_ex(bad) == lmh.LMH_ERR_INVALID_ARG
    assert fwd_ex(0.7, p2=6) == lmh.LMH_ERR_UNSUPPORTED
    assert fwd_ex(0.7, wsb=64) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    # the forward workspace also holds the squared-sum records: strictly larger than the records
    assert lmh.lmhead_logprob_fwd_workspace_size(64, 8, 1000) >= 64 * 8 * 20

    def part(vs, vt, V=256, temp=1.0, p2=0, wsb=1 << 22):
        return lib.lmhead_logprob_fwd_partials_ex(16, 16, 16, 4, 8, V, temp, vs, vt, p2, 256, wsb, None)

    assert part(0, 128, V=256) == lmh.LMH_ERR_INVALID_ARG          # shard past the vocabulary
    assert part(-128, 1024) == lmh.LMH_ERR_INVALID_ARG
    assert part(64, 1024) == lmh.LMH_ERR_UNSUPPORTED               # not on a 128-row chunk
    assert part(0, 1024, V=200) == lmh.LMH_ERR_UNSUPPORTED         # partial chunk in a middle shard
    assert part(0, 1024, p2=2) == lmh.LMH_ERR_INVALID_ARG
    assert part(0, 1024, temp=nan) == lmh.LMH_ERR_INVALID_ARG
    assert part(0, 1024, wsb=64) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert lib.lmhead_logprob_fwd_finalize_ex(16, 4, 8, 10, 16, None, None, 6, 256, 1 << 20, None) == \
        lmh.LMH_ERR_UNSUPPORTED

    def bwd_ex(temp=1.0, **kw):
        a = dict(h=16, w=16, y=16, T=4, H=8, V=10, vs=0, g=16, lse=16, ge=None, ent=None, gh=16, gw=16, acc=0,
                 ws=256, wsb=1 << 30)
        a.update(kw)
        return lib.lmhead_logprob_bwd_ex(a["h"], a["w"], a["y"], a["T"], a["H"], a["V"], temp, a["vs"], a["g"],
                                         a["lse"], a["ge"], a["ent"], a["gh"], a["gw"], a["acc"], a["ws"], a["wsb"],
                                         None)

    assert bwd_ex(0.0) == lmh.LMH_ERR_INVALID_ARG
    assert bwd_ex(1.0, ge=16) == lmh.LMH_ERR_INVALID_ARG            # entropy gradient without the entropy
    assert bwd_ex(1.0, ge=16, ent=6) == lmh.LMH_ERR_UNSUPPORTED
    assert bwd_ex(1.3, wsb=64) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert bwd_ex(1.3, gh=None, gw=None, ge=16, ent=16) == lmh.LMH_OK
    assert bwd_ex(1.0, vs=-128) == lmh.LMH_ERR_INVALID_ARG           # vocabulary shard before id 0
    max_v = 2**31 - 2**16                                            # vocabulary ids stay below this
    assert bwd_ex(1.0, vs=max_v - 10) == lmh.LMH_ERR_INVALID_ARG     # shard past the id range
    assert bwd_ex(1.0, vs=max_v - 11, gh=None, gw=None) == lmh.LMH_OK
    assert bwd_ex(1.0, vs=77, gh=None, gw=None) == lmh.LMH_OK        # any start: no records are written


def test_noalloc_validation_codes(lib):
    # refused on the host before the device is touched: sizes past the built-in scratch, bad sizes,
    # null or misaligned pointers (fake, never-dereferenced addresses)
    def call(hidden=16, weight=16, labels=16, T=4, H=8, V=10, logprob=16):
        return lib.lmhead_logprob_fwd_noalloc(hidden, weight, labels, T, H, V, logprob, None, None, None)
    V = 152064
    T = 1
    while lmh.lmhead_logprob_fwd_workspace_size_min(T + 1, 8, V) <= lmh.NOALLOC_SCRATCH_BYTES:
        T += 1
    assert call(T=T + 1, V=V) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert call(T=1 << 30, V=V) == lmh.LMH_ERR_UNSUPPORTED             # past 2^36 record slots
    assert call(T=0) == lmh.LMH_OK
    assert call(hidden=None) == lmh.LMH_ERR_INVALID_ARG
    assert call(logprob=None) == lmh.LMH_ERR_INVALID_ARG
    assert call(weight=8) == lmh.LMH_ERR_UNSUPPORTED
    assert call(H=12) == lmh.LMH_ERR_UNSUPPORTED
    assert call(V=0) == lmh.LMH_ERR_INVALID_ARG


def test_bwd_workspace_step_sizes(lib):
    T, H, V = 4096, 5120, 152064
    fast = lmh.lmhead_logprob_bwd_workspace_size(T, H, V)
    assert lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, 65536) == fast
    assert lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, 10**9) == fast      # clamped to 65536
    sizes = [lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, s) for s in range(256, 65537, 256)]
    assert all(a < b for a, b in zip(sizes, sizes[1:])), "workspace must grow with the step"
    assert lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, 1) == sizes[0]       # rounded up to 256
    assert sizes[0] < 256 << 20 < fast
    assert lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, 0) == 0
    assert lmh.lmhead_logprob_bwd_workspace_size_step(T, 12, V, 256) == 0
    # a small V needs no more than V rounded up to 256 rows per step
    assert lmh.lmhead_logprob_bwd_workspace_size_step(64, 64, 300, 65536) == \
        lmh.lmhead_logprob_bwd_workspace_size_step(64, 64, 300, 512)


def test_bwd_accepts_any_workspace_down_to_the_narrowest_step(lib):
    T, H, V = 300, 64, 5000
    least = lmh.lmhead_logprob_bwd_workspace_size_step(T, H, V, 256)

    def call(wsb, gh=16, gw=16):
        return lib.lmhead_logprob_bwd(16, 16, 16, T, H, V, 16, 16, gh, gw, 0, 256, wsb, None)

    assert call(least - 1) == lmh.LMH_ERR_WORKSPACE_TOO_SMALL
    assert call(least, gh=None, gw=None) == lmh.LMH_OK          # validated; nothing to compute
    assert call((least + lmh.lmhead_logprob_bwd_workspace_size(T, H, V)) // 2, gh=None, gw=None) == lmh.LMH_OK
