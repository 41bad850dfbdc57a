"""Pins of the oracle's recency bias on summary keys.

Page: model card "GTA world model: weights and inference code", sections "Files" (an
optional recency bias on summary keys) and "Credits" (it follows a paper the page does not
reproduce).  The reading: a term added to the scaled scores of summary keys, in natural-log
units, that depends on the head and on the age t - f of the key's frame; the caller gives
its values as a table over ages 0 .. W.

What fixes the oracle here is not the oracle: exp(s + ln n) = n exp(s), so a bias of ln n
on some keys equals n copies of those keys in a plain softmax, and a bias of -inf equals
leaving them out.  The reference side of every check is built from the frame-level
attention rule of section "What a frame attends to" (``frame_visibility``) over the full
history of records, with keys repeated or dropped; it never looks at the buffer's slot
tables.  The figure "The buffer one frame apart" fixes which frame has which age at t = 31.
Planted mistakes at the end must each fail one of these pins.
"""
import math

import numpy as np
import pytest

from oracle import sf_oracle as so

G = so.Geometry(hw=6, x=3, y=2, w=6, n_heads=2, head_dim=8, n_blocks=1, dtype="f32")
FIG = so.Geometry(hw=4, x=3, y=2, w=24, n_heads=1, head_dim=8, n_blocks=1, dtype="f32")


def rollout(g, t_last, seed, cls=so.MemoryReplay, rewrites=()):
    """Random f32 records through frames 0..t_last; yields (t, replay, history K, history V, rng)."""
    rng = np.random.default_rng(seed)
    m = cls(g, recency_bias=np.zeros((g.n_heads, g.w + 1)))
    hk, hv = {}, {}
    for t in range(t_last + 1):
        if t >= 1:
            m.evict(t)
        for _ in range(1 + (t in rewrites)):
            k = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
            v = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
            m.write(0, t, k, v)
        hk[t], hv[t] = k.astype(np.float64), v.astype(np.float64)
        yield t, m, hk, hv, rng


def history_read(g, t, q, hk, hv, scale, copies):
    """Attention of frame t over the rows [attends] lets it see, each row taken
    copies(h, f, row) times (0: left out), per head, with no bias."""
    out = np.empty(q.shape, dtype=np.float64)
    for h in range(g.n_heads):
        ks, vs = [], []
        for f in range(t + 1):
            vis = so.frame_visibility(g, t, f)
            for row in range(g.r):
                if vis == "whole" or (vis == "summary" and row >= g.hw):
                    n = copies(h, f, row)
                    ks += [hk[f][row, h]] * n
                    vs += [hv[f][row, h]] * n
        kk = np.array(ks)[:, None, :]
        vv = np.array(vs)[:, None, :]
        out[:, h:h + 1] = so.attention_f64(q[:, h:h + 1], kk, vv, scale)
    return out


# ---------------------------------------------------------------- the pins
def check_log_n_is_n_copies(cls=so.MemoryReplay):
    """A bias of ln 3 at age a on head h equals three copies of frame t-a's summary rows
    in head h, for ages in the record (0), in RAW (1..Y) and in SUM (Y+1..W)."""
    g = G
    scale = so.default_scale(g.head_dim)
    for t, m, hk, hv, rng in rollout(g, 16, seed=3, cls=cls, rewrites={5}):
        for a in sorted({0, 1, g.y, g.y + 1, g.w - 1, g.w}):
            if t - a < 1:
                continue
            h = (t + a) % g.n_heads
            tab = np.zeros((g.n_heads, g.w + 1))
            tab[h, a] = math.log(3.0)
            m.set_recency_bias(tab)
            q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
            got = m.attend(0, q, scale)
            want = history_read(g, t, q, hk, hv, scale,
                                lambda hh, f, row: 3 if (hh == h and f == t - a and row >= g.hw) else 1)
            np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13, err_msg=f"t={t} age={a}")


def check_minus_inf_leaves_summaries_out(cls=so.MemoryReplay):
    """-inf at every age: the read sees the start image whole and only the raw rows of the
    frames kept whole, as if no summary row of a generated frame were there."""
    g = G
    scale = so.default_scale(g.head_dim)
    for t, m, hk, hv, rng in rollout(g, 14, seed=4, cls=cls):
        m.set_recency_bias(np.full((g.n_heads, g.w + 1), -np.inf))
        q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
        got = m.attend(0, q, scale)
        want = history_read(g, t, q, hk, hv, scale, lambda h, f, row: 1 if (f == 0 or row < g.hw) else 0)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13, err_msg=f"t={t}")


def check_figure_ages(cls=so.MemoryReplay):
    """At t = 31 with Y = 2, W = 24 (the figure "The buffer one frame apart"): frame 28's
    summary has just taken frame 6's SUM slot and has age 3 = Y+1; the oldest summary
    kept is frame 7's, age 24 = W.  -inf at exactly those ages drops exactly those rows."""
    g = FIG
    scale = so.default_scale(g.head_dim)
    for t, m, hk, hv, rng in rollout(g, 31, seed=5, cls=cls):
        pass
    assert m.sum_frame[6] == 28                      # the figure's move
    for a, f_gone in ((3, 28), (24, 7)):
        tab = np.zeros((1, g.w + 1))
        tab[0, a] = -np.inf
        m.set_recency_bias(tab)
        q = rng.standard_normal((g.r, 1, g.head_dim))
        got = m.attend(0, q, scale)
        want = history_read(g, t, q, hk, hv, scale, lambda h, f, row: 0 if (f == f_gone and row >= g.hw) else 1)
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-13, err_msg=f"age {a}")


def test_log_n_bias_equals_n_copies():
    check_log_n_is_n_copies()


def test_minus_inf_bias_leaves_summaries_out():
    check_minus_inf_leaves_summaries_out()


def test_figure_frame31_ages():
    check_figure_ages()


def test_zero_table_and_no_table_agree():
    """A zero table is no bias; the table is per head."""
    g = G
    plain = so.MemoryReplay(g)
    for t, m, hk, hv, rng in rollout(g, 12, seed=6):
        plain.evict(t) if t >= 1 else None
        plain.write(0, t, hk[t].astype(np.float32), hv[t].astype(np.float32))
        q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
        np.testing.assert_array_equal(m.attend(0, q), plain.attend(0, q))
        tab = np.zeros((g.n_heads, g.w + 1))
        tab[0] = rng.standard_normal(g.w + 1)
        m.set_recency_bias(tab)
        np.testing.assert_array_equal(m.attend(0, q)[:, 1], plain.attend(0, q)[:, 1])
        m.set_recency_bias(np.zeros((g.n_heads, g.w + 1)))


def test_table_shape_is_checked():
    with pytest.raises(ValueError):
        so.MemoryReplay(G, recency_bias=np.zeros((G.n_heads, G.w)))


# ---------------------------------------------------------------- planted mistakes
class _BiasBySlot(so.MemoryReplay):
    """Bias looked up by the SUM slot index instead of the frame's age."""

    def key_bias(self, rows):
        if self.recency_bias is None:
            return None
        g = self.g
        bias = np.zeros((len(rows), g.n_heads))
        sum0 = g.r * (g.y + 2)
        for j, row in enumerate(rows):
            if row >= sum0:
                bias[j] = self.recency_bias[:, (row - sum0) // g.x]
        return bias


class _BiasOnRawRows(so.MemoryReplay):
    """Every row of a generated frame biased, raw rows included."""

    def row_frames(self, rows):
        frame, summary = super().row_frames(rows)
        return frame, np.ones_like(summary)


class _BiasOnStartImage(so.MemoryReplay):
    """The start image's summary rows biased as a frame of age t."""

    def row_frames(self, rows):
        frame, summary = super().row_frames(rows)
        z0 = np.asarray(rows) < self.g.r
        frame = np.where(z0, 0, frame)
        summary = summary | (z0 & (np.asarray(rows) % self.g.r >= self.g.hw))
        return frame, summary

    def key_bias(self, rows):
        frame, summary = self.row_frames(rows)
        bias = np.zeros((len(rows), self.g.n_heads))
        for j in np.nonzero(summary & (frame >= 0))[0]:
            bias[j] = self.recency_bias[:, min(self.t - frame[j], self.g.w)]
        return bias


class _AgeOffByOne(so.MemoryReplay):
    """Age counted as t - f - 1 (the newest summary taken as age 0 ... )."""

    def key_bias(self, rows):
        frame, summary = self.row_frames(rows)
        bias = np.zeros((len(rows), self.g.n_heads))
        for j in np.nonzero(summary & (frame >= 1))[0]:
            bias[j] = self.recency_bias[:, max(self.t - frame[j] - 1, 0)]
        return bias


class _BiasInLog2Units(so.MemoryReplay):
    """The table read as log2 units (multiplied by log2 e before the natural exp)."""

    def key_bias(self, rows):
        b = super().key_bias(rows)
        return None if b is None else b * math.log2(math.e)


class _BiasSubtracted(so.MemoryReplay):
    """The bias subtracted from the scores."""

    def key_bias(self, rows):
        b = super().key_bias(rows)
        return None if b is None else -b


@pytest.mark.parametrize("cls", [_BiasBySlot, _BiasOnRawRows, _BiasOnStartImage, _AgeOffByOne,
                                 _BiasInLog2Units, _BiasSubtracted])
def test_planted_bias_mistakes_are_caught(cls):
    caught = []
    for check in (check_log_n_is_n_copies, check_minus_inf_leaves_summaries_out, check_figure_ages):
        try:
            check(cls)
        except (AssertionError, IndexError, FloatingPointError):
            caught.append(check.__name__)
    assert caught, f"{cls.__doc__} was not caught"
