"""Pins of the oracle's rotary temporal band and streaming sink.

Page: model card "GTA world model: weights and inference code", sections "Running
for a long time: the start image follows the window" ([sink]), "Telling a summary
from a pixel: level planes" ([level]) and the "Positions" item of "The rest of the
model" ([positions]).  Each test names the fact it checks.  Planted mistakes at the
end must each be caught by one of these pins.
"""
import numpy as np
import pytest

from oracle import sf_oracle as so

RNG = np.random.default_rng(11)


def test_level_twelve_temporal_planes_at_head_dim_64():
    # [level]: each attention head (head_dim 64) has 12 temporal planes
    assert so.temporal_planes(64) == 12
    assert len(so.temporal_frequencies(64)) == 12


def test_level_exactly_two_slow_planes():
    # [level]: the two slowest temporal planes turn by less than half a radian over
    # 1024 frames; the band's other planes turn by more
    turn = so.temporal_frequencies(64, 10000.0) * 1024
    slow = np.nonzero(turn < 0.5)[0]
    assert list(slow) == [10, 11]
    assert np.all(np.diff(turn) < 0)          # plane i+1 is slower than plane i
    assert turn[9] > 0.5


def test_rotation_is_the_complex_product():
    # [sink], [positions]: a rotary key is the complex product (x + iy) * exp(i * id * w)
    k = RNG.standard_normal((5, 3, 64))
    T = 7.0
    got = so.rotate_temporal(k, 64, T)
    n = so.temporal_planes(64)
    z = k[..., 0:2 * n:2] + 1j * k[..., 1:2 * n:2]
    want = z * np.exp(1j * so.temporal_frequencies(64) * T)
    np.testing.assert_allclose(got[..., 0:2 * n:2], want.real, rtol=0, atol=1e-12)
    np.testing.assert_allclose(got[..., 1:2 * n:2], want.imag, rtol=0, atol=1e-12)
    np.testing.assert_array_equal(got[..., 2 * n:], k[..., 2 * n:])   # height / width bands untouched


def test_rotation_composes():
    # [sink]: rotation(id + T) = rotation(id) * rotation(T)
    k = RNG.standard_normal((4, 2, 128))
    for a, b in ((3.0, 4.0), (0.5, 1024.0), (17.0, -5.0)):
        twice = so.rotate_temporal(so.rotate_temporal(k, 128, a), 128, b)
        once = so.rotate_temporal(k, 128, a + b)
        np.testing.assert_allclose(twice, once, rtol=0, atol=1e-12)


def test_moved_key_scores_as_if_written_later():
    # [sink]: a start-image key moved forward by T scores against any query exactly as a
    # key written T frames later (RoPE scores depend only on the difference of ids)
    q = RNG.standard_normal((6, 64))
    k = RNG.standard_normal((6, 64))
    tq, T = 40.0, 4.0
    qr = so.rotate_temporal(q, 64, tq)
    moved = so.rotate_temporal(so.rotate_temporal(k, 64, 0.0), 64, T)
    fresh = so.rotate_temporal(k, 64, T)
    np.testing.assert_allclose((qr * moved).sum(-1), (qr * fresh).sum(-1), rtol=1e-12)
    # and the score depends on the id difference only
    np.testing.assert_allclose((so.rotate_temporal(q, 64, tq + 9) * so.rotate_temporal(k, 64, T + 9)).sum(-1),
                               (qr * fresh).sum(-1), rtol=1e-10)


def test_bf16_rounding_is_nearest_even():
    # bfloat16 rounding against brute force: the pattern chosen is the nearest of its
    # neighbours, and on a tie the even one; exact values and float32 agree with numpy
    x = np.concatenate([RNG.standard_normal(4000) * 3, RNG.standard_normal(1000) * 1e-3])
    b = so.f64_to_bf16_bits(x).astype(np.int64)
    for d in (-1, 1):
        nb = np.clip(b + d, 0, 0xffff).astype(np.uint16)
        closer = np.abs(so.bf16_bits_to_f64(b.astype(np.uint16)) - x) <= np.abs(so.bf16_bits_to_f64(nb) - x)
        assert closer.all()
    lo = so.bf16_bits_to_f64(np.array([0x3f80], dtype=np.uint16))[0]      # 1.0
    step = 2.0 ** -7
    ties = np.array([lo + step / 2, lo + 3 * step / 2])                      # halfway cases
    assert list(so.f64_to_bf16_bits(ties)) == [0x3f80, 0x3f82]              # to even
    exact = so.bf16_bits_to_f64(np.arange(0x3000, 0x5000, 7, dtype=np.uint16))
    np.testing.assert_array_equal(so.f64_to_bf16_bits(exact), np.arange(0x3000, 0x5000, 7, dtype=np.uint16))


def _sink_replay(g, frames, gap=5, cls=so.MemoryReplay, seed=3):
    m = cls(g, sink_gap=gap)
    rng = np.random.default_rng(seed)
    hist = []
    for t in range(frames):
        m.evict(t) if t >= 1 else None
        k = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
        v = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
        for b in range(g.n_blocks):
            m.write(b, t, k, v)
        hist.append((t, m.oldest_frame(), m.z0_frame, m.k.copy(), m.v.copy()))
    return m, hist


G_SMALL = so.Geometry(hw=4, x=2, y=2, w=6, n_heads=2, head_dim=64, n_blocks=2, dtype="f32")


def test_sink_schedule():
    # [sink]: the gap between the start image and the oldest frame in memory reaches 5,
    # then the start image is moved so the gap is 1 again; it is never 5 when a frame reads
    m, hist = _sink_replay(G_SMALL, 60)
    moves = [(t, z) for (t, old, z, _, _) in hist if z > 0]
    gaps = [old - z for (t, old, z, _, _) in hist if old >= 1]
    assert min(gaps) >= 1 and max(gaps) <= 4
    firsts = [t for (t, old, z, _, _), prev in zip(hist[1:], hist[:-1]) if z != prev[2]]
    assert firsts[0] == G_SMALL.w + 5                 # oldest = t - w reaches 5 at t = w + 5
    assert np.all(np.diff(firsts) == 4)               # then every 4 frames, by 4
    for (t, old, z, _, _) in hist:
        if t in firsts:
            assert old - z == 1
        assert z == max(0, (old - 1) // 4 * 4) if old >= 1 else z == 0


def test_sink_moves_z0_keys_only():
    # [sink]: only the start image's keys move; values and every other row are untouched
    m, hist = _sink_replay(G_SMALL, 40)
    t0 = [i for i in range(1, len(hist)) if hist[i][2] != hist[i - 1][2]][0]
    _, _, z_before, k_before, v_before = hist[t0 - 1]
    _, _, z_after, k_after, v_after = hist[t0]
    r = G_SMALL.r
    np.testing.assert_array_equal(v_after[:, :r], v_before[:, :r])
    want = so.rotate_temporal(k_before[:, :r].astype(np.float64), 64, z_after - z_before).astype(np.float32)
    np.testing.assert_array_equal(k_after[:, :r], want)


class _SinkWrongGap(so.MemoryReplay):
    """Mistake: the start image moves when the gap reaches 4."""

    def sink_step(self):
        T = so.sink_shift(self.oldest_frame(), self.z0_frame, 4)
        if T > 0:
            self.z0_frame += T
        return T


class _SinkShiftByGap(so.MemoryReplay):
    """Mistake: the start image moves by the whole gap (gap 0 afterwards)."""

    def sink_step(self):
        T = so.sink_shift(self.oldest_frame(), self.z0_frame, self.sink_gap)
        if T > 0:
            self.z0_frame += T + 1
        return T


class _SinkMovesValues(so.MemoryReplay):
    """Mistake: the values of the start image are rotated too."""

    def sink_step(self):
        T = super().sink_step()
        if T > 0:
            r = self.g.r
            self.v[:, :r] = so.rotate_temporal(self.v[:, :r].astype(np.float64), self.g.head_dim, T).astype(np.float32)
        return T


_ROTATE = so.rotate_temporal


def _rotate_conjugate(k, head_dim, frames, theta=10000.0):
    """Mistake: turns the wrong way (the sine's sign flipped)."""
    return _ROTATE(k, head_dim, -frames, theta)


def _rotate_split_halves(k, head_dim, frames, theta=10000.0):
    """Mistake: pairs dim i with dim i + n (the rotate-half layout) instead of (2i, 2i+1)."""
    n = so.temporal_planes(head_dim)
    perm = np.concatenate([np.ravel(np.column_stack([np.arange(n), np.arange(n) + n])), np.arange(2 * n, head_dim)])
    inv = np.argsort(perm)
    return _ROTATE(np.asarray(k)[..., perm], head_dim, frames, theta)[..., inv]


@pytest.mark.parametrize("cls", [_SinkWrongGap, _SinkShiftByGap, _SinkMovesValues])
def test_planted_sink_mistakes_are_caught(cls):
    caught = False
    for check in (test_sink_schedule, test_sink_moves_z0_keys_only):
        orig = _sink_replay.__defaults__
        try:
            _sink_replay.__defaults__ = (5, cls, 3)
            check()
        except AssertionError:
            caught = True
        finally:
            _sink_replay.__defaults__ = orig
    assert caught, cls.__doc__


@pytest.mark.parametrize("bad", [_rotate_conjugate, _rotate_split_halves])
def test_planted_rotation_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(so, "rotate_temporal", bad)
    with pytest.raises(AssertionError):
        test_rotation_is_the_complex_product()
