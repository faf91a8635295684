"""The seeded generator: determinism, chunk independence and the pages' KV statistics."""
import numpy as np

from video_model_kv_amd import synth


def test_deterministic_and_chunk_local():
    wl = synth.workload(2, n_heads=2)
    a = synth.kv_chunk(wl, "K", 1)
    b = synth.kv_chunk(wl, "K", 1)
    assert a.tobytes() == b.tobytes()
    part = synth.kv_tokens(wl, "K", 6000, 6500)
    whole = np.concatenate([synth.kv_chunk(wl, "K", 0), synth.kv_chunk(wl, "K", 1)])[6000:6500]
    assert part.tobytes() == whole.tobytes()
    # a head generated alone equals the same head generated with others
    solo = synth.kv_chunk(wl, "K", 1, heads=[1])
    assert solo[:, 0].tobytes() == a[:, 1].tobytes()


def test_magnitudes_match_the_pages():
    wl = synth.workload(2, n_heads=2)
    k = synth.kv_chunk(wl, "K", 0)
    v = synth.kv_chunk(wl, "V", 0)
    assert 50 <= np.abs(k).max() <= 110        # max|K| ~ 1e2
    assert 500 <= np.abs(v).max() <= 1100      # max|V| ~ 1e3
    # bf16 values
    u = k.view(np.uint32)
    assert not np.any(u & 0xFFFF)
    # outlier channels vary with the token
    big = np.abs(k[:, 0]) > 20
    assert len({tuple(np.nonzero(r)[0]) for r in big}) > 4


def test_tiny_is_fp32_and_sized():
    wl = synth.workload(1)
    k = synth.kv_chunk(wl, "K", 0)
    assert k.shape == (1560, 1, 128)
    assert np.any(k.view(np.uint32) & 0xFFFF)   # genuinely float32 values
    q = synth.queries(wl)
    assert q.shape == (1560, 1, 128)
