"""The C ABI library loads, exports every declared entry point, and refuses bad
arguments on the host with the documented status codes (no GPU needed: every
case here is rejected before any HIP call)."""
import ctypes
import os
import re

import pytest

from long_context_prefill_attn_amd import _lib

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "prefill_attn.h")
FAKE = 0x100000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(?:int|size_t|const char\*)\s+(\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib.lib()
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS), names
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = _lib.lib()
    for code in (0, -1, -2, -3, -4, -5, 7):
        assert lib.pa_status_string(code)


def dense(**kw):
    a = dict(Q=FAKE, C=64, n_q=4, K=FAKE, V=FAKE, T=256, n_kv=2, d=128, mask=FAKE, ld=256,
             scale=0.125, O=FAKE, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    return _lib.lib().prefill_attn_dense(a["Q"], a["C"], a["n_q"], a["K"], a["V"], a["T"], a["n_kv"],
                                         a["d"], a["mask"], a["ld"], a["scale"], a["O"], a["ws"],
                                         a["ws_bytes"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.PA_EINVAL),
    (dict(K=FAKE + 2), _lib.PA_EINVAL),           # misaligned
    (dict(C=0), _lib.PA_EINVAL),
    (dict(T=0), _lib.PA_EINVAL),
    (dict(n_q=3), _lib.PA_EINVAL),                # not a multiple of n_kv
    (dict(ld=255), _lib.PA_EINVAL),               # mask_ld < T
    (dict(scale=float("nan")), _lib.PA_EINVAL),
    (dict(scale=-1.0), _lib.PA_EINVAL),
    (dict(scale=float("inf")), _lib.PA_EINVAL),
    (dict(d=96), _lib.PA_EUNSUPPORTED),
    (dict(T=(1 << 22) - 4095, ld=1 << 22), _lib.PA_EUNSUPPORTED),   # flag row would not fit in LDS
    (dict(), _lib.PA_EWORKSPACE),                 # no workspace
    (dict(ws=FAKE + 16, ws_bytes=1 << 30), _lib.PA_EWORKSPACE),  # workspace not 256-aligned
    (dict(ws=FAKE, ws_bytes=1), _lib.PA_EWORKSPACE),
])
def test_dense_rejects(kw, code):
    assert dense(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(mask=FAKE + 4), _lib.PA_EINVAL),        # misaligned bits
    (dict(ld=7), _lib.PA_EINVAL),                 # 7 words < ceil(256 / 32)
    (dict(ld=8, d=96), _lib.PA_EUNSUPPORTED),
    (dict(ld=8, T=(1 << 22) + 1), _lib.PA_EINVAL),   # ld too small for that T
    (dict(ld=1 << 17, T=(1 << 22) - 4095), _lib.PA_EUNSUPPORTED),  # longest key range exceeded
    (dict(ld=8), _lib.PA_EWORKSPACE),             # no workspace
])
def test_dense_bits_rejects(kw, code):
    a = dict(Q=FAKE, C=64, n_q=4, K=FAKE, V=FAKE, T=256, n_kv=2, d=128, mask=FAKE, ld=8, scale=0.125,
             O=FAKE, ws=None, ws_bytes=0, stream=None)
    a.update(kw)
    assert _lib.lib().prefill_attn_dense_bits(a["Q"], a["C"], a["n_q"], a["K"], a["V"], a["T"], a["n_kv"],
                                              a["d"], a["mask"], a["ld"], a["scale"], a["O"], a["ws"],
                                              a["ws_bytes"], a["stream"]) == code


def test_dense_noalloc_rejects():
    """The allocation-free entry: bad arguments as prefill_attn_dense, and sizes whose
    workspace exceeds its static scratch refused with PA_ESCRATCH (before any launch)."""
    lib = _lib.lib()
    f = lambda **kw: lib.prefill_attn_dense_noalloc(
        kw.get("Q", FAKE), kw.get("C", 64), 4, FAKE, FAKE, kw.get("T", 256), kw.get("n_kv", 2), kw.get("d", 128),
        FAKE, kw.get("ld", kw.get("T", 256)), kw.get("scale", 0.125), FAKE, None)
    limit = lib.prefill_attn_dense_noalloc_limit()
    assert limit == 80 << 20
    assert f(Q=None) == _lib.PA_EINVAL
    assert f(ld=100) == _lib.PA_EINVAL
    assert f(scale=0.0) == _lib.PA_EINVAL
    assert f(d=96) == _lib.PA_EUNSUPPORTED
    T = 200_000                                    # staged values alone: 200,000 x 4 x 128 x 2 bytes > 80 MiB
    assert lib.prefill_attn_dense_workspace(64, T, 4, 4, 128) > limit
    assert f(T=T, n_kv=4) == _lib.PA_ESCRATCH
    assert lib.prefill_attn_dense_workspace(64, 32768, 4, 2, 128) <= limit
    assert b"static" in lib.pa_status_string(_lib.PA_ESCRATCH)


def test_dense_workspace_size():
    lib = _lib.lib()
    assert lib.prefill_attn_dense_workspace(64, 256, 4, 2, 128) >= 256 * 2 * 128 * 2   # staged fp16 values
    assert lib.prefill_attn_dense_workspace(0, 256, 4, 2, 128) == 0
    assert lib.prefill_attn_dense_workspace(64, 256, 4, 2, 96) == 0


def sel(**kw):
    a = dict(Q=FAKE, C=256, q_start=0, n_q=4, n_kv=2, d=128, Kp=FAKE, T=256, block=128, alpha=0.1,
             scale=0.125, idx=FAKE, cnt=FAKE, stream=None)
    a.update(kw)
    return _lib.lib().select_blocks(a["Q"], a["C"], a["q_start"], a["n_q"], a["n_kv"], a["d"], a["Kp"],
                                    a["T"], a["block"], a["alpha"], a["scale"], a["idx"], a["cnt"],
                                    a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Q=None), _lib.PA_EINVAL),
    (dict(T=300), _lib.PA_EINVAL),                # T != q_start + C
    (dict(alpha=float("nan")), _lib.PA_EINVAL),
    (dict(alpha=-0.1), _lib.PA_EINVAL),
    (dict(alpha=float("inf")), _lib.PA_EINVAL),
    (dict(scale=0.0), _lib.PA_EINVAL),
    (dict(block=100), _lib.PA_EUNSUPPORTED),
    (dict(block=512), _lib.PA_EUNSUPPORTED),
    (dict(d=80), _lib.PA_EUNSUPPORTED),
    (dict(C=16 * 8192 + 16, T=16 * 8192 + 16, block=16), _lib.PA_EUNSUPPORTED),  # > 8192 blocks
])
def test_select_rejects(kw, code):
    assert sel(**kw) == code


def test_pool_and_blocksparse_reject():
    lib = _lib.lib()
    assert lib.build_pooled_index(None, FAKE, 10, 1, 128, 128, FAKE, FAKE, None) == _lib.PA_EINVAL
    assert lib.build_pooled_index(FAKE, FAKE, 0, 1, 128, 128, FAKE, FAKE, None) == _lib.PA_EINVAL
    assert lib.build_pooled_index(FAKE, FAKE, 10, 1, 128, 48, FAKE, FAKE, None) == _lib.PA_EUNSUPPORTED
    bs = lambda **kw: lib.prefill_attn_blocksparse(
        kw.get("Q", FAKE), 256, 0, 4, FAKE, FAKE, kw.get("T", 256), 2, kw.get("d", 128), FAKE, FAKE,
        kw.get("block", 128), FAKE, FAKE, kw.get("scale", 0.1), FAKE, kw.get("ws", FAKE),
        kw.get("ws_bytes", 0), None)
    assert bs(Q=None) == _lib.PA_EINVAL
    assert bs(T=255) == _lib.PA_EINVAL
    assert bs(scale=float("nan")) == _lib.PA_EINVAL
    assert bs(block=48) == _lib.PA_EUNSUPPORTED
    assert bs(block=512) == _lib.PA_EUNSUPPORTED
    assert bs(d=256) == _lib.PA_EUNSUPPORTED
    for block in (16, 32, 64, 128, 256):                  # every block size is taken: the workspace is next
        assert bs(block=block) == _lib.PA_EWORKSPACE
    assert bs(ws=None, ws_bytes=1 << 30) == _lib.PA_EWORKSPACE
    assert bs(ws=FAKE + 16, ws_bytes=1 << 30) == _lib.PA_EWORKSPACE   # not 256-aligned
    need = lib.prefill_attn_blocksparse_workspace(256, 2, 128)
    assert need >= 256 * 2 * 128 * 2                     # holds the staged fp16 values
    assert bs(ws_bytes=need - 1) == _lib.PA_EWORKSPACE
    assert lib.prefill_attn_blocksparse_workspace(0, 2, 128) == 0
    assert lib.prefill_attn_blocksparse_workspace(256, 2, 96) == 0


def test_ld_forms_reject():
    """Pooled-index capacity and incremental range checks of the *_ld entry points."""
    lib = _lib.lib()
    # T = 1000, block 128 -> 8 blocks: capacity 7 is too small, b_first 9 is past the end
    assert lib.build_pooled_index_ld(FAKE, FAKE, 1000, 2, 128, 128, 0, FAKE, FAKE, 7, None) == _lib.PA_EINVAL
    assert lib.build_pooled_index_ld(FAKE, FAKE, 1000, 2, 128, 128, 9, FAKE, FAKE, 8, None) == _lib.PA_EINVAL
    assert lib.build_pooled_index_ld(FAKE, FAKE, 1000, 2, 128, 128, -1, FAKE, FAKE, 8, None) == _lib.PA_EINVAL
    assert lib.build_pooled_index_ld(FAKE, FAKE, 1000, 2, 128, 96, 0, FAKE, FAKE, 8, None) == _lib.PA_EUNSUPPORTED
    assert lib.select_blocks_ld(FAKE, 256, 744, 4, 2, 128, FAKE, 7, 1000, 128, 0.1, 0.125, 0, 0, 0,
                                FAKE, FAKE, None) == _lib.PA_EINVAL
    for rules in ((-1, 0, 0), (0, -1, 0), (0, 0, -1)):
        assert lib.select_blocks_ld(FAKE, 256, 744, 4, 2, 128, FAKE, 8, 1000, 128, 0.1, 0.125, *rules,
                                    FAKE, FAKE, None) == _lib.PA_EINVAL
    assert lib.prefill_attn_blocksparse_ld(FAKE, 256, 744, 4, FAKE, FAKE, 1000, 2, 128, FAKE, FAKE, 7,
                                           128, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, None) == _lib.PA_EINVAL
    assert lib.prefill_attn_blocksparse_ld(FAKE, 256, 744, 4, FAKE, FAKE, 1000, 2, 128, FAKE, FAKE, 8,
                                           96, FAKE, FAKE, 0.1, FAKE, FAKE, 1 << 30, None) == _lib.PA_EUNSUPPORTED
    assert lib.prefill_attn_blocksparse_ld(FAKE, 256, 744, 4, FAKE, FAKE, 1000, 2, 128, FAKE, FAKE, 16,
                                           64, FAKE, FAKE, 0.1, FAKE, FAKE, 0, None) == _lib.PA_EWORKSPACE


def test_fold_rejects():
    lib = _lib.lib()
    f = lambda **kw: lib.fold_keep_mask(kw.get("idx", FAKE), kw.get("K", 8), kw.get("cnt", FAKE),
                                        kw.get("C", 16), kw.get("q0", 100), kw.get("T", 116),
                                        kw.get("width", 4), kw.get("recent", 3), kw.get("mask", FAKE),
                                        kw.get("ld", 116), None)
    assert f(T=115) == _lib.PA_EINVAL          # rows past the mask's columns
    assert f(width=0) == _lib.PA_EINVAL
    assert f(recent=-1) == _lib.PA_EINVAL
    assert f(ld=100) == _lib.PA_EINVAL
    assert f(K=-1) == _lib.PA_EINVAL
    assert f(cnt=None) == _lib.PA_EINVAL
    assert f(mask=FAKE + 4) == _lib.PA_EINVAL   # misaligned


def test_fold_bits_rejects():
    lib = _lib.lib()
    f = lambda **kw: lib.fold_keep_bits(kw.get("idx", FAKE), kw.get("K", 8), kw.get("cnt", FAKE),
                                        kw.get("C", 16), kw.get("q0", 100), kw.get("T", 116),
                                        kw.get("width", 4), kw.get("recent", 3), kw.get("bits", FAKE),
                                        kw.get("ld", 4), None)
    assert f(T=115) == _lib.PA_EINVAL          # rows past the last key
    assert f(width=0) == _lib.PA_EINVAL
    assert f(recent=-1) == _lib.PA_EINVAL
    assert f(ld=3) == _lib.PA_EINVAL           # fewer words than ceil(T / 32)
    assert f(K=-1) == _lib.PA_EINVAL
    assert f(cnt=None) == _lib.PA_EINVAL
    assert f(bits=FAKE + 4) == _lib.PA_EINVAL   # misaligned


def test_gather_rejects():
    """The gather entry's host-side checks (no kernel is launched on any of these)."""
    lib = _lib.lib()
    f = lambda **kw: lib.prefill_attn_gather(kw.get("Q", FAKE), kw.get("C", 16), kw.get("q0", 100),
                                             kw.get("nq", 4), kw.get("K", FAKE), kw.get("V", FAKE),
                                             kw.get("T", 116), kw.get("nkv", 2), kw.get("d", 128),
                                             kw.get("idx", FAKE), kw.get("kl", 8), kw.get("cnt", FAKE),
                                             kw.get("width", 4), kw.get("recent", 3), kw.get("scale", 0.1),
                                             kw.get("O", FAKE), None)
    assert f(T=115) == _lib.PA_EINVAL                   # rows past the history
    assert f(q0=-1) == _lib.PA_EINVAL
    assert f(C=0) == _lib.PA_EINVAL
    assert f(nq=3) == _lib.PA_EINVAL                    # heads not a multiple of the KV heads
    assert f(width=0) == _lib.PA_EINVAL
    assert f(recent=-1) == _lib.PA_EINVAL
    assert f(kl=-1) == _lib.PA_EINVAL
    assert f(cnt=None) == _lib.PA_EINVAL
    assert f(idx=None) == _lib.PA_EINVAL                # lists declared but missing
    assert f(scale=0.0) == _lib.PA_EINVAL
    assert f(scale=float("nan")) == _lib.PA_EINVAL
    assert f(O=FAKE + 4) == _lib.PA_EINVAL              # misaligned
    assert f(d=96) == _lib.PA_EUNSUPPORTED
    assert f(width=65) == _lib.PA_EUNSUPPORTED
    # one row's block bitmap and list beyond the LDS of a CU
    assert f(T=1 << 24, width=1, kl=1 << 20) == _lib.PA_EUNSUPPORTED


def test_timing_api_host_side():
    lib = _lib.lib()
    ms, n = ctypes.c_double(), ctypes.c_int64()
    assert lib.pa_timing_read(b"nope", ctypes.byref(ms), ctypes.byref(n)) == _lib.PA_EINVAL
    assert lib.pa_timing_reset() == 0
    assert lib.pa_timing_read(b"attn_dense", ctypes.byref(ms), ctypes.byref(n)) == 0
    assert n.value == 0


def test_bisect_alpha_host_logic():
    # a monotone step function with known jumps: the smallest alpha reaching each
    # target is found to the bisection's resolution
    import long_context_prefill_attn_amd as lp
    steps = [(0.0, 0.0), (0.05, 0.30), (0.2, 0.62), (0.5, 0.85), (0.9, 0.97)]

    def skip_of(a):
        return max(s for x, s in steps if x <= a)
    for target, want in [(0.3, 0.05), (0.6, 0.2), (0.85, 0.5), (0.9, 0.9)]:
        a, s = lp.bisect_alpha(skip_of, target, iters=40)
        assert abs(a - want) < 1e-9 and s >= target, (target, a, s)
    assert lp.bisect_alpha(skip_of, 0.99) == (1.0, 0.97)    # unreachable: hi and its share
    assert lp.bisect_alpha(skip_of, 0.0) == (0.0, 0.0)      # reached at lo


def test_select_path_counts_rejects_null():
    assert _lib.lib().pa_select_path_counts(None, 0) == _lib.PA_EINVAL
