"""The allocation-free decode attention entry point (the library's own scratch
buffer instead of a caller workspace) against the workspace entry point it
shares its kernels with: bit-identical outputs on two calls in a row, the
second smaller than the first, and a clear error for a call whose split
partials exceed the buffer (rejected on the host, nothing launched)."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

D = 128


def say(msg):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def env():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import bit_kv_cache_rope_amd as bk
    bk.library()
    return dict(torch=torch, bk=bk)


def _batch(env, B, Hq, Hkv, bits, max_len, seed):
    """Random packed caches of B sequences (lengths up to max_len, one run of
    rows each) with random codes and fp16 steps, and random paired queries."""
    torch, bk = env["torch"], env["bk"]
    rng = np.random.default_rng(seed)
    lens = rng.integers(1, max_len + 1, B).astype(np.int32)
    lens[0] = max_len
    row0 = (np.arange(B, dtype=np.int64) * max_len)
    rows = B * max_len
    q = bk.sym(2.0)
    kc, vc = bk.alloc_packed(rows, Hkv, bits, q), bk.alloc_packed(rows, Hkv, bits, q)
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    for c in (kc, vc):
        c.codes.copy_(torch.randint(0, 256, c.codes.shape, dtype=torch.uint8, device="cuda", generator=g))
        c.scales.copy_((torch.rand(c.scales.shape, device="cuda", generator=g) * 0.05 + 0.02).to(torch.float16))
    qp = (torch.randn((B, Hq, D), device="cuda", generator=g) * 3.0).to(torch.bfloat16)
    return dict(q=q, kc=kc, vc=vc, qp=qp, row0=torch.from_numpy(row0).cuda(), lens=torch.from_numpy(lens).cuda(),
                max_len=max_len, Hkv=Hkv, bits=bits)


def _both(env, b):
    torch, bk = env["torch"], env["bk"]
    scale = 1.0 / np.sqrt(D)
    ref = bk.wushkv_decode_attention(b["qp"], b["kc"], b["vc"], b["Hkv"], b["bits"], b["q"], b["row0"], b["lens"],
                                     b["max_len"], scale)
    out = torch.full_like(ref, float("nan"))
    bk.wushkv_decode_attention_noalloc(b["qp"], b["kc"], b["vc"], b["Hkv"], b["bits"], b["q"], b["row0"], b["lens"],
                                       b["max_len"], scale, out)
    torch.cuda.synchronize()
    return ref, out


def test_noalloc_attention_equals_workspace_call_twice(env):
    """A large batch (split partials of 4.3 MB), then a smaller one on the
    same GPU: each output is bit-identical to the workspace call's."""
    torch = env["torch"]
    for B, Hq, Hkv, bits, max_len, seed in ((32, 32, 8, 2, 16384, 5), (5, 16, 4, 4, 3000, 6)):
        say(f"noalloc attention B={B} Hq={Hq} Hkv={Hkv} bits={bits} max_len={max_len}")
        ref, out = _both(env, _batch(env, B, Hq, Hkv, bits, max_len, seed))
        assert torch.isfinite(ref).all()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32))


def test_noalloc_attention_rejects_partials_beyond_its_buffer(env):
    """128 sequences x 64 query heads x 32 splits of 132 floats need 138 MB of
    partials: rejected with WUSHKV_ERR_UNSUPPORTED before anything runs."""
    torch, bk = env["torch"], env["bk"]
    need = bk.wushkv_decode_attention_workspace(128, 64, 8, 65536)
    assert need > bk._lib.NOALLOC_SCRATCH_BYTES
    q = bk.sym(2.0)
    kc, vc = bk.alloc_packed(0, 8, 2, q), bk.alloc_packed(0, 8, 2, q)
    qp = torch.zeros((128, 64, D), dtype=torch.bfloat16, device="cuda")
    out = torch.zeros((128, 64, D), dtype=torch.float32, device="cuda")
    row0 = torch.zeros(128, dtype=torch.int64, device="cuda")
    lens = torch.zeros(128, dtype=torch.int32, device="cuda")
    with pytest.raises(bk.WushKVError) as e:
        bk.wushkv_decode_attention_noalloc(qp, kc, vc, 8, 2, q, row0, lens, 65536, 0.1, out)
    assert e.value.status == bk._lib.ERR_UNSUPPORTED and "scratch" in str(e.value)
