"""Pins of the oracle's temporal band applied at the write, with level planes.

Page: model card "GTA world model: weights and inference code", sections "Telling a
summary from a pixel: level planes" ([level]), "Running for a long time: the start
image follows the window" ([sink]) and the "Positions" item of "The rest of the model"
([positions]).  The facts checked: a record is rotated by its frame id on the temporal
planes (the complex product); summary rows carry an exact quarter turn on the two
slowest planes; those planes turn by under half a radian over 1024 frames, which the
construction check enforces; RoPE scores depend only on the difference of frame ids;
the sink's multiply moves a rotated start image to where a later write would put it.
Each planted mistake at the end must be caught by one of these pins.
"""
import numpy as np
import pytest

from oracle import sf_oracle as so

RNG = np.random.default_rng(23)
MODES = (so.ROPE_LEVEL_REPLACE, so.ROPE_LEVEL_ADD)


def planes(a: np.ndarray, head_dim: int) -> np.ndarray:
    """Temporal planes of a [..., head_dim] array as complex numbers x + iy."""
    n = so.temporal_planes(head_dim)
    return a[..., 0:2 * n:2] + 1j * a[..., 1:2 * n:2]


def test_idle_check_follows_the_page_bound():
    # [level]: the two slowest of the 12 planes (head_dim 64) turn by under half a radian
    # over 1024 frames at the table's base 10000: the check passes.  Plane 10's turn is
    # 1024 * 10000^(-20/24) = 1024 * 10^(-10/3) = 0.4753 rad.
    assert so.level_planes_idle(64, 10000.0)
    assert abs(so.temporal_frequencies(64)[10] * 1024 - 1024 * 10.0 ** (-10.0 / 3.0)) < 1e-12
    assert so.level_planes_idle(128, 10000.0)
    # a base of 1000 makes plane 10 turn by 1024 * 10^(-2.5) = 3.2 rad: the model refuses to build
    assert not so.level_planes_idle(64, 1000.0)
    # the bound sits where the page puts it: plane 10 turns exactly 0.5 rad over 1024 frames
    # at base 2048^(6/5); a base a little above passes, a little below fails
    theta_edge = (1024 / 0.5) ** (24 / 20)
    assert so.level_planes_idle(64, theta_edge * 1.001)
    assert not so.level_planes_idle(64, theta_edge * 0.999)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("head_dim", (64, 128))
def test_raw_rows_are_the_complex_product(mode, head_dim):
    # [positions]: a raw token at frame t is (x + iy) * exp(i w t) on every temporal plane;
    # the height and width bands are not touched
    hw, x, t = 5, 3, 37
    a = RNG.standard_normal((hw + x, 2, head_dim))
    got = so.rope_record_f64(a, hw, t, head_dim, mode=mode)
    w = so.temporal_frequencies(head_dim)
    n = len(w)
    np.testing.assert_allclose(planes(got[:hw], head_dim), planes(a[:hw], head_dim) * np.exp(1j * w * t),
                               rtol=0, atol=1e-12)
    np.testing.assert_array_equal(got[..., 2 * n:], a[..., 2 * n:])
    # summary rows: the same on every plane but the two slowest
    np.testing.assert_allclose(planes(got[hw:], head_dim)[..., :n - 2],
                               (planes(a[hw:], head_dim) * np.exp(1j * w * t))[..., :n - 2], rtol=0, atol=1e-12)


@pytest.mark.parametrize("t", (0, 1, 29, 1000))
def test_summary_rows_carry_an_exact_quarter_turn(t):
    # [level]: summary tokens get an exact quarter turn on the two slowest planes.
    # REPLACE: the quarter turn of the input, whatever the frame; ADD: the quarter turn of
    # what a raw token with the same content gets at the same frame.
    hw, x, hd = 4, 3, 64
    a = RNG.standard_normal((hw + x, 3, hd))
    same = np.concatenate([a[hw:], a[hw:]])       # rows 0..2 raw, rows 3..5 summary, same content
    n = so.temporal_planes(hd)
    rep = planes(so.rope_record_f64(a, hw, t, hd, mode=so.ROPE_LEVEL_REPLACE), hd)
    np.testing.assert_array_equal(rep[hw:, :, n - 2:], 1j * planes(a[hw:], hd)[..., n - 2:])
    add = planes(so.rope_record_f64(same, x, t, hd, mode=so.ROPE_LEVEL_ADD), hd)
    np.testing.assert_array_equal(add[x:, :, n - 2:], 1j * add[:x, :, n - 2:])
    # at frame 0 the time angle is zero and the two readings agree
    if t == 0:
        np.testing.assert_array_equal(rep, planes(so.rope_record_f64(a, hw, 0, hd, mode=so.ROPE_LEVEL_ADD), hd))


def test_quarter_turn_is_exact_in_storage():
    # [level] "exact": in bf16 and fp32 storage the REPLACE quarter turn is a swap of the
    # two values with the new first one negated, bit for bit (one rounding of an exact result)
    hw, x, hd = 2, 5, 64
    n = so.temporal_planes(hd)
    for dtype, sign in (("bf16", np.uint16(0x8000)), ("f32", None)):
        a = RNG.standard_normal((hw + x, 2, hd))
        stored = so.f64_to_storage(a, dtype)
        got = so.rope_record(stored, hw, 777, hd, dtype, mode=so.ROPE_LEVEL_REPLACE)
        xs, ys = stored[hw:, :, 2 * n - 4:2 * n:2], stored[hw:, :, 2 * n - 3:2 * n:2]
        if dtype == "bf16":
            np.testing.assert_array_equal(got[hw:, :, 2 * n - 4:2 * n:2], ys ^ sign)
        else:
            np.testing.assert_array_equal(got[hw:, :, 2 * n - 4:2 * n:2], -ys)
        np.testing.assert_array_equal(got[hw:, :, 2 * n - 3:2 * n:2], xs)


def test_level_axis_is_independent_of_time_match():
    # [level]: a query can weight "summary of frame t" and "pixel of frame t" independently:
    # against a raw and a summary key of the same content and frame, the level planes give
    # the real and the imaginary part of one complex product (ADD), so the two weights are
    # separate projections
    hd, t = 64, 12
    n = so.temporal_planes(hd)
    q = RNG.standard_normal((1, 1, hd))
    k = RNG.standard_normal((1, 1, hd))
    rq = so.rope_record_f64(q, 1, t, hd, mode=so.ROPE_LEVEL_ADD)[0, 0]           # a raw query row
    kk = so.rope_record_f64(np.concatenate([k, k]), 1, t, hd, mode=so.ROPE_LEVEL_ADD)
    lv = slice(2 * n - 4, 2 * n)
    s_raw = float(rq[lv] @ kk[0, 0, lv])
    s_sum = float(rq[lv] @ kk[1, 0, lv])
    zq, zk = planes(q[0, 0], hd)[n - 2:], planes(k[0, 0], hd)[n - 2:]
    prod = zq * np.conj(zk)                   # the time angles cancel at equal frames
    assert abs(s_raw - prod.real.sum()) < 1e-12
    assert abs(s_sum - prod.imag.sum()) < 1e-12


@pytest.mark.parametrize("mode", MODES)
def test_scores_depend_on_frame_difference_only(mode):
    # [positions]: RoPE scores depend only on the difference of frame ids.  Raw rows in both
    # readings, summary rows too under ADD; under REPLACE a summary row's level planes hold
    # no time, so only its other planes follow the rule.
    hw, x, hd = 3, 2, 64
    n = so.temporal_planes(hd)
    q = RNG.standard_normal((hw + x, 2, hd))
    k = RNG.standard_normal((hw + x, 2, hd))

    def scores(tq, tk, cut):
        a = so.rope_record_f64(q, hw, tq, hd, mode=mode)[..., :cut]
        b = so.rope_record_f64(k, hw, tk, hd, mode=mode)[..., :cut]
        return np.einsum("rhd,shd->hrs", a, b)

    cut = hd if mode == so.ROPE_LEVEL_ADD else 2 * n - 4
    for tq, tk, s in ((30, 26, 100), (5, 0, 900)):
        np.testing.assert_allclose(scores(tq, tk, cut), scores(tq + s, tk + s, cut), rtol=0, atol=1e-10)
    raw = scores(30, 26, hd)[:, :hw, :hw]
    np.testing.assert_allclose(raw, scores(130, 126, hd)[:, :hw, :hw], rtol=0, atol=1e-10)


G_SINK = so.Geometry(hw=4, x=2, y=2, w=6, n_heads=2, head_dim=64, n_blocks=1, dtype="f32")


@pytest.mark.parametrize("mode", MODES)
def test_sink_moves_a_rotated_start_image_to_a_later_write(mode):
    # [sink] with [level]: after the start image has been moved forward to frame z, its keys
    # are (to one rounding per move) the keys a write of the same record at frame z would
    # store, summary rows' level planes included; values and the other rows never change
    g = G_SINK
    m = so.MemoryReplay(g, sink_gap=5, rope_mode=mode)
    recs = {}
    moves = 0
    for t in range(40):
        k = so.f64_to_storage(RNG.standard_normal((g.r, g.n_heads, g.head_dim)), "f32")
        v = so.f64_to_storage(RNG.standard_normal((g.r, g.n_heads, g.head_dim)), "f32")
        z = m.z0_frame
        m.step(t, {0: (k, v)})
        recs[t] = (k, v)
        if m.z0_frame != z:
            moves += 1
            want = so.rope_record(recs[0][0], g.hw, m.z0_frame, g.head_dim, "f32", mode=mode)
            got = m.k[0, :g.r]
            assert np.abs(got.astype(np.float64) - want).max() <= moves * 4 * 2.0 ** -23 * np.abs(want).max()
            if mode == so.ROPE_LEVEL_REPLACE:
                n = so.temporal_planes(g.head_dim)
                np.testing.assert_array_equal(got[g.hw:, :, 2 * n - 4:2 * n], want[g.hw:, :, 2 * n - 4:2 * n])
        np.testing.assert_array_equal(m.v[0, :g.r], recs[0][1])
    assert moves >= 3


def _twin_rotate(a, hw, f, hd, mode):
    """Rotation of a record at frame f, stated on complex planes (for the brute-force twin)."""
    w = so.temporal_frequencies(hd)
    n = len(w)
    z = planes(a, hd) * np.exp(1j * w * f)
    zs = z[hw:].copy()
    base = planes(a[hw:], hd) if mode == so.ROPE_LEVEL_REPLACE else zs
    zs[..., n - 2:] = 1j * base[..., n - 2:]
    z[hw:] = zs
    out = a.astype(np.float64).copy()
    out[..., 0:2 * n:2] = z.real
    out[..., 1:2 * n:2] = z.imag
    return out


@pytest.mark.parametrize("mode", MODES)
def test_rotated_read_equals_the_history_twin(mode):
    # [attends] with [positions]: reading the buffer of rotated records with the query
    # rotated by the current frame is masked attention over the history in which every
    # record carries its own frame id (not its slot) and the query the current one
    g = so.Geometry(hw=6, x=2, y=2, w=5, n_heads=2, head_dim=64, n_blocks=1, dtype="f32")
    m = so.MemoryReplay(g, rope_mode=mode)
    hk, hv = [], []
    for t in range(14):
        k = so.f64_to_storage(RNG.standard_normal((g.r, g.n_heads, g.head_dim)), "f32")
        v = so.f64_to_storage(RNG.standard_normal((g.r, g.n_heads, g.head_dim)), "f32")
        q = so.f64_to_storage(RNG.standard_normal((g.r, g.n_heads, g.head_dim)), "f32")
        m.step(t, {0: (k, v)})
        hk.append(_twin_rotate(k.astype(np.float64), g.hw, t, g.head_dim, mode))
        hv.append(v.astype(np.float64))
        qt = _twin_rotate(q.astype(np.float64), g.hw, t, g.head_dim, mode)
        want = so.history_attention(g, t, qt, hk, hv, so.default_scale(g.head_dim))
        # the replay rounds rotated keys and queries to fp32 storage; the twin does not
        np.testing.assert_allclose(m.attend(0, q), want, rtol=0, atol=1e-5)


# ---------------------------------------------------------------------------
# Planted mistakes
# ---------------------------------------------------------------------------
_ROPE = so.rope_record_f64


def _quarter_turn_backwards(a, hw, t, hd, theta=10000.0, mode=so.ROPE_LEVEL_REPLACE):
    """Mistake: the quarter turn goes the other way, (x, y) -> (y, -x)."""
    out = _ROPE(a, hw, t, hd, theta, mode)
    n = so.temporal_planes(hd)
    out[hw:, ..., 2 * n - 4:2 * n] *= -1
    return out


def _level_from_row_before(a, hw, t, hd, theta=10000.0, mode=so.ROPE_LEVEL_REPLACE):
    """Mistake: the last raw row is treated as a summary row."""
    return _ROPE(a, hw - 1, t, hd, theta, mode)


def _level_on_three_planes(a, hw, t, hd, theta=10000.0, mode=so.ROPE_LEVEL_REPLACE):
    """Mistake: the third-slowest plane is also taken as a level plane."""
    out = _ROPE(a, hw, t, hd, theta, mode)
    n = so.temporal_planes(hd)
    src = np.asarray(a, dtype=np.float64)[hw:, ..., 2 * n - 6:2 * n - 4]
    out[hw:, ..., 2 * n - 6] = -src[..., 1]
    out[hw:, ..., 2 * n - 5] = src[..., 0]
    return out


@pytest.mark.parametrize("bad", [_quarter_turn_backwards, _level_from_row_before, _level_on_three_planes])
def test_planted_rope_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(so, "rope_record_f64", bad)
    caught = 0
    for check in (lambda: test_raw_rows_are_the_complex_product(so.ROPE_LEVEL_REPLACE, 64),
                  lambda: test_summary_rows_carry_an_exact_quarter_turn(29),
                  lambda: test_rotated_read_equals_the_history_twin(so.ROPE_LEVEL_REPLACE)):
        try:
            check()
        except AssertionError:
            caught += 1
    assert caught >= 1, bad.__doc__


class _SinkTurnsLevelPlanes(so.MemoryReplay):
    """Mistake: under REPLACE the sink also turns the summary rows' level planes."""

    def sink_step(self):
        mode = self.rope_mode
        self.rope_mode = so.ROPE_CALLER
        try:
            return super().sink_step()
        finally:
            self.rope_mode = mode


class _QueryNotRotated(so.MemoryReplay):
    """Mistake: the query is read as it came in."""

    def attend(self, block, q, scale=None, rows=None):
        mode = self.rope_mode
        self.rope_mode = so.ROPE_CALLER
        try:
            return super().attend(block, q, scale, rows)
        finally:
            self.rope_mode = mode


class _KeysBySlot(so.MemoryReplay):
    """Mistake: a record is rotated by its RAW slot instead of its frame id."""

    def write(self, block, t, k, v):
        g = self.g
        slot_t = 0 if t == 0 else self.raw_slot(t) + 1
        mode = self.rope_mode
        self.rope_mode = so.ROPE_CALLER
        try:
            k = so.rope_record(np.asarray(k).reshape(g.r, g.n_heads, g.head_dim), g.hw, slot_t, g.head_dim,
                               g.dtype, self.rope_theta, mode)
            super().write(block, t, k, v)
        finally:
            self.rope_mode = mode


@pytest.mark.parametrize("cls,check", [
    (_SinkTurnsLevelPlanes, lambda: test_sink_moves_a_rotated_start_image_to_a_later_write(so.ROPE_LEVEL_REPLACE)),
    (_QueryNotRotated, lambda: test_rotated_read_equals_the_history_twin(so.ROPE_LEVEL_ADD)),
    (_KeysBySlot, lambda: test_rotated_read_equals_the_history_twin(so.ROPE_LEVEL_ADD)),
])
def test_planted_replay_mistakes_are_caught(monkeypatch, cls, check):
    monkeypatch.setattr(so, "MemoryReplay", cls)
    with pytest.raises(AssertionError):
        check()
