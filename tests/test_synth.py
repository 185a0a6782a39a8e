"""The seeded input generator: determinism, slice consistency, shapes and the
distributions the workloads name."""
import numpy as np


def test_slices_regenerate_identically(synth_mod):
    w = synth_mod.WORKLOADS["qwen3_8b_prefill"]
    full = synth_mod.kv(w, 0, "K", 0, 512, threads=3)
    part = synth_mod.kv(w, 0, "K", 200, 100, threads=1)
    assert np.array_equal(full[200:300], part)
    assert np.array_equal(full, synth_mod.kv(w, 0, "K", 0, 512, threads=5))
    assert not np.array_equal(full, synth_mod.kv(w, 0, "V", 0, 512))
    assert not np.array_equal(full, synth_mod.kv(w, 1, "K", 0, 512))


def test_shapes_and_dtypes(synth_mod):
    for name in synth_mod.WORKLOAD_ORDER:
        w = synth_mod.WORKLOADS[name]
        a = synth_mod.kv(w, 0, "V", 0, 8)
        assert a.shape == (8, w.heads, 128)
        assert a.dtype == (np.uint16 if w.dtype == "bf16" else np.float32)
        T, Ti = synth_mod.transform(w, 0)
        assert T.shape == (w.heads, 128, 128)
        for h in range(w.heads):
            assert np.abs(T[h].astype(np.float64) @ Ti[h] - np.eye(128)).max() < 1e-5
            # general invertible, not orthogonal
            assert np.abs(T[h].astype(np.float64) @ T[h].T - np.eye(128)).max() > 0.1


def test_distributions(synth_mod):
    w = synth_mod.WORKLOADS["tiny"]
    k = synth_mod.kv(w, 0, "K")
    for h in range(w.heads):
        out = synth_mod.outliers(w, 0, "K", h)
        assert len(set(out)) == 4
        normal = np.delete(k[:, h, :], out, axis=1)
        assert abs(normal.mean()) < 0.05 and abs(normal.std() - 1) < 0.05
        assert abs(k[:, h, out].std() / 20 - 1) < 0.15
    w = synth_mod.WORKLOADS["qwen3_8b_prefill"]
    v = synth_mod.bf16_bits_to_f32(synth_mod.kv(w, 0, "V", 0, 8192)).astype(np.float64)
    sig = synth_mod.channel_sigma(w, 0, "V")
    t = v / sig[None]
    # Student-t(3): median |t| = 0.765, heavy tails
    assert abs(np.median(np.abs(t)) - 0.765) < 0.02
    assert np.mean(np.abs(t) > 5) > 0.005


def test_positions_and_slots(synth_mod):
    w = synth_mod.WORKLOADS["decode_append"]
    p = synth_mod.positions(w)
    assert p.shape == (64,) and p.min() >= 0 and p.max() < 32768
    s = synth_mod.slots(w)
    assert np.array_equal(s, np.arange(64) * 32768 + p)
    w4 = synth_mod.WORKLOADS["affine_pct"]
    p4 = synth_mod.positions(w4, 16380, 8)
    assert p4.tolist() == [16380, 16381, 16382, 16383, 0, 1, 2, 3]
