"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/wushkv.h declares, and rejects bad arguments on the host before any
HIP call."""
import ctypes
import os
import re
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    import bit_kv_cache_rope_amd as bk
    if not os.path.exists(bk._lib.LIB_PATH):
        from bit_kv_cache_rope_amd import build
        build.build()
    return bk._lib.load()


def declared_functions():
    src = open(os.path.join(ROOT, "include", "wushkv.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wushkv_[a-z_0-9]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
    from bit_kv_cache_rope_amd import _lib
    assert sorted(_lib.EXPORTED) == names
    out = subprocess.run(["nm", "-D", "--defined-only", os.path.join(ROOT, "bit_kv_cache_rope_amd", "libwushkv.so")],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r" T (wushkv_\w+)", out))
    assert set(names) <= exported


def test_version_and_status_strings(lib):
    assert lib.wushkv_version() == 1
    for s in range(7):
        assert lib.wushkv_status_string(s)
    assert lib.wushkv_status_string(99) == b"unknown status"


@pytest.mark.parametrize("theta", [1e6, 1e4, 5e5, 10000.0])
def test_frequencies_match_oracle(lib, oracle_mod, theta):
    import bit_kv_cache_rope_amd as bk
    om = np.array(bk.wushkv_rope_frequencies(theta), np.float32)
    ref = np.array([oracle_mod.omega(theta, i) for i in range(64)], np.float32)
    assert np.array_equal(om.view(np.uint32), ref.view(np.uint32))


def _q(kind=0, alpha=2.0, group=128, plo=1.0, phi=99.0):
    from bit_kv_cache_rope_amd import _lib
    return _lib.Quantizer(kind, alpha, group, plo, phi)


def _packed(codes=16, scales=16, zeros=None, slots=None, rows=10):
    from bit_kv_cache_rope_amd import _lib
    return _lib.Packed(codes, scales, zeros, slots, rows)


def test_validation_without_device(lib):
    from bit_kv_cache_rope_amd import _lib
    L = lib
    vp = ctypes.c_void_p
    q, p = _q(), _packed()
    call = lambda *a: L.wushkv_quantize_values(*a)
    # bad dtype, heads, stride, bits, quantizer, NULLs and alignment -- all before any HIP call
    assert call(vp(16), 7, 4, 2, 256, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 0, 256, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 2, 200, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 2, 260, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_ALIGNMENT
    assert call(vp(16), 1, 4, 2, 256, 5, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 2, 256, 1, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(8), 1, 4, 2, 256, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_ALIGNMENT
    assert call(None, 1, 4, 2, 256, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, -1, 2, 256, 2, ctypes.byref(q), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 2, 256, 2, None, ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    assert call(vp(16), 1, 4, 2, 256, 2, ctypes.byref(q), None, None) == _lib.ERR_INVALID_ARG
    bad = _packed(codes=8)
    assert call(vp(16), 1, 4, 2, 256, 2, ctypes.byref(q), ctypes.byref(bad), None) == _lib.ERR_ALIGNMENT
    small = _packed(rows=3)
    assert call(vp(16), 1, 4, 2, 256, 2, ctypes.byref(q), ctypes.byref(small), None) == _lib.ERR_INVALID_ARG
    assert L.wushkv_last_error()
    # quantizer descriptions
    for qq, want in ((_q(group=32), _lib.ERR_UNSUPPORTED), (_q(alpha=0.0), _lib.ERR_INVALID_ARG),
                     # general percentiles are accepted: these stop at the missing zeros
                     (_q(kind=1, group=32, plo=5.0), _lib.ERR_INVALID_ARG),
                     (_q(kind=1, group=32, phi=90.0), _lib.ERR_INVALID_ARG),
                     (_q(kind=1, group=32, plo=50.0, phi=10.0), _lib.ERR_INVALID_ARG),
                     (_q(kind=1, group=128), _lib.ERR_UNSUPPORTED), (_q(kind=7), _lib.ERR_INVALID_ARG)):
        assert call(vp(16), 1, 4, 2, 256, 2, ctypes.byref(qq), ctypes.byref(p), None) == want
    # affine needs zeros
    qa = _q(kind=1, group=32)
    assert call(vp(16), 1, 4, 2, 256, 2, ctypes.byref(qa), ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    pz = _packed(zeros=16)
    # n_tokens == 0 is a no-op once the arguments are well formed
    assert call(None, 1, 0, 2, 256, 2, ctypes.byref(qa), ctypes.byref(pz), None) == _lib.OK
    # keys: NULL handles
    assert L.wushkv_quantize_keys(vp(16), 1, 4, 2, 256, vp(16), None, None, 2, ctypes.byref(q),
                                  ctypes.byref(p), None) == _lib.ERR_INVALID_ARG
    # fused keys + values: both tensors are checked, then the handles
    kv = lambda K=vp(16), V=vp(16), dt=1, ks=256, vs=256, rope=None, T=None: L.wushkv_quantize_kv(
        K, V, dt, 4, 2, ks, vs, vp(16), rope, T, 2, ctypes.byref(q), ctypes.byref(p), ctypes.byref(p), None)
    assert kv(dt=7) == _lib.ERR_INVALID_ARG
    assert kv(V=vp(8)) == _lib.ERR_ALIGNMENT
    assert kv(vs=260) == _lib.ERR_ALIGNMENT
    assert kv(ks=200) == _lib.ERR_INVALID_ARG
    assert kv(V=None) == _lib.ERR_INVALID_ARG
    assert kv() == _lib.ERR_INVALID_ARG  # NULL rope and transform handles
    assert L.wushkv_debug_check_arith(None, None) == _lib.ERR_INVALID_ARG
    assert L.wushkv_debug_check_arith(vp(2), None) == _lib.ERR_ALIGNMENT
    # read path
    assert L.wushkv_dequantize(ctypes.byref(p), 4, 2, 9, ctypes.byref(q), None, vp(16), 1, None) == _lib.ERR_INVALID_ARG
    assert L.wushkv_dequantize(ctypes.byref(p), 4, 2, 2, ctypes.byref(q), None, vp(16), 3, None) == _lib.ERR_INVALID_ARG
    assert L.wushkv_dequantize(ctypes.byref(p), 0, 2, 2, ctypes.byref(q), None, None, 1, None) == _lib.OK
    # query pairing and decode attention
    assert L.wushkv_pair_queries(vp(16), 1, 4, 8, 1024, None, vp(16), None) == _lib.ERR_INVALID_ARG
    assert L.wushkv_pair_queries(vp(16), 1, 4, 8, 1000, None, vp(16), None) == _lib.ERR_INVALID_ARG
    nb = ctypes.c_size_t()
    assert L.wushkv_decode_attention_workspace(64, 32, 8, 32768, ctypes.byref(nb)) == _lib.OK
    assert nb.value == 64 * 32 * 16 * 132 * 4
    assert L.wushkv_decode_attention_workspace(2, 12, 8, 100, ctypes.byref(nb)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_decode_attention_workspace(2, 72, 8, 100, ctypes.byref(nb)) == _lib.ERR_UNSUPPORTED
    att = lambda n, bits=2, qq=q, kc=p, ws=1 << 20, sc=0.1: L.wushkv_decode_attention(
        vp(16), n, 32, ctypes.byref(kc), ctypes.byref(p), 8, bits, ctypes.byref(qq), vp(16), vp(16), 4096,
        ctypes.c_float(sc), vp(16), ws, vp(16), None)
    assert att(2, bits=5) == _lib.ERR_INVALID_ARG
    assert att(2, qq=_q(kind=1, group=32)) == _lib.ERR_INVALID_ARG  # affine caches need zeros
    assert att(2, kc=_packed(rows=3)) == _lib.ERR_INVALID_ARG
    assert att(2, ws=100) == _lib.ERR_INVALID_ARG
    assert att(2, sc=float("inf")) == _lib.ERR_INVALID_ARG
    assert att(0) == _lib.OK
    # dispatch sizes: every grid stays below 2^32 work-items (256-thread blocks)
    assert L.wushkv_decode_attention_workspace(65535, 64, 8, 131072, ctypes.byref(nb)) == _lib.ERR_UNSUPPORTED
    assert L.wushkv_decode_attention_workspace(32767, 64, 8, 131072, ctypes.byref(nb)) == _lib.OK  # 2^24 - 512 blocks
    big = lambda n, H, heads, dl: L.wushkv_decode_attention(
        vp(16), n, H, ctypes.byref(p), ctypes.byref(p), heads, 2, ctypes.byref(q), vp(16), vp(16), dl,
        ctypes.c_float(0.1), vp(16), 1 << 20, vp(16), None)
    assert big(65535, 64, 8, 131072) == _lib.ERR_UNSUPPORTED
    assert L.wushkv_pair_queries(vp(16), 1, (1 << 26) - 3, 8, 1024, None, vp(16), None) == _lib.ERR_UNSUPPORTED
    assert L.wushkv_pair_queries(vp(16), 1, (1 << 26) - 4, 8, 1024, None, vp(16), None) == _lib.ERR_INVALID_ARG
    huge = _packed(rows=(1 << 31) - 1)
    assert L.wushkv_dequantize(ctypes.byref(huge), 1 << 24, 512, 2, ctypes.byref(q), None, vp(16), 1,
                               None) == _lib.ERR_UNSUPPORTED
    assert L.wushkv_debug_rope_cos_sin(None, vp(16), (1 << 26) + 1, vp(16), None) == _lib.ERR_UNSUPPORTED
    assert L.wushkv_debug_rope_cos_sin(None, vp(16), 1 << 26, vp(16), None) == _lib.ERR_INVALID_ARG
    # handles
    h = vp()
    assert L.wushkv_rope_create(ctypes.c_float(1e6), 0, ctypes.byref(h)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_rope_create(ctypes.c_float(1e6), (1 << 24) + 1, ctypes.byref(h)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_rope_create(ctypes.c_float(0.5), 10, ctypes.byref(h)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_transform_create(None, 2, ctypes.byref(h)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_transform_create(vp(16), 0, ctypes.byref(h)) == _lib.ERR_INVALID_ARG
    assert L.wushkv_transform_destroy(None) == _lib.OK and L.wushkv_rope_destroy(None) == _lib.OK


def test_missing_library_fails_loudly(tmp_path):
    code = ("import bit_kv_cache_rope_amd as bk\n"
            "try:\n    bk.library()\nexcept ImportError as e:\n    print('IMPORTERROR', e)\n")
    env = dict(os.environ, WUSHKV_LIB=str(tmp_path / "nope.so"), PYTHONPATH=ROOT)
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, env=env, timeout=300)
    assert "IMPORTERROR" in out.stdout, out.stderr
