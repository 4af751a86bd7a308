"""The seeded generators are deterministic and have the configured shapes."""
import numpy as np

from workloads import synth


def test_deterministic_and_shaped():
    a = synth.config0(BS=2, V=1000)
    b = synth.config0(BS=2, V=1000)
    for k in ("target", "draft", "tokens", "u_acc", "u_smp", "ctx"):
        assert np.array_equal(a[k], b[k])
    assert a["target"].shape == (2, 8, 1000) and a["draft"].shape == (2, 7, 1000)
    assert a["ctx"].shape == (2, 512) and a["ctx"].dtype == np.int32
    assert np.all((a["tokens"] >= 0) & (a["tokens"] < 1000))
    assert np.all((a["u_acc"] >= 0) & (a["u_acc"] < 1))


def test_planted_spans_and_copy_heavy():
    rng = np.random.Generator(np.random.Philox(1))
    x = synth.uniform_tokens(rng, 512, 32000)
    pairs = synth.plant_spans(rng, x, 3, 40, live_end=True)
    starts = sorted([s for s, _ in pairs] + [d for _, d in pairs])
    assert all(b - a >= 40 for a, b in zip(starts, starts[1:]))
    assert pairs[-1][1] + 40 == 512
    for s, d in pairs:
        assert np.array_equal(x[s:s + 40], x[d:d + 40])
    ctx, tr = synth.copy_heavy(rng, 4096, 1000, 3000, 16)
    assert len(ctx) == 4096 and len(tr) == 16
    same = np.mean(ctx[3000:] == ctx[:1096])
    assert 0.85 < same < 0.95          # 10% of the copy replaced


def test_bf16_round_trip():
    x = np.array([1.0, -2.5, 3.14159, 1e-3, 65504.0], np.float32)
    y = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(x))
    assert np.allclose(x, y, rtol=2 ** -8)
    assert y[0] == 1.0 and y[1] == -2.5
