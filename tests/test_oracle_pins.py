"""Pins of the oracle against facts fixed by the page, not by the oracle itself.

Page: model card "GTA world model: weights and inference code".  Each test
names the part of the page (or the piece of mathematics) that fixes it.  The
mutation tests at the end plant plausible mistakes in copies of the oracle and
check that some pin here catches each one.
"""
import math
import os

import numpy as np
import pytest
import torch

import sf_inputs
from oracle import sf_oracle as so

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

SERVED = so.Geometry(hw=1008, x=96, y=2, w=24, n_heads=1, head_dim=1, n_blocks=1, dtype="f32")
TINY = so.Geometry(**{k: sf_inputs.WORKLOADS["tiny"][k] for k in
                      ("hw", "x", "y", "w", "n_heads", "head_dim", "n_blocks", "dtype")})
LONG = so.Geometry(hw=3600, x=256, y=4, w=96, n_heads=1, head_dim=1, n_blocks=1, dtype="f32")


def read_golden(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, val = line.split()
            out[key] = int(val)
    return out


def identity_record(g, f):
    """A record whose every value names (frame, row): f * 10000 + row."""
    vals = (f * 10000 + np.arange(g.r)).astype(np.float32)
    return np.broadcast_to(vals[:, None, None], (g.r, g.n_heads, g.head_dim)).copy()


def replay_identity(g, t_last, replay_cls=so.MemoryReplay):
    """Replay frames 0..t_last with identity records; yield (t, replay) after each step."""
    m = replay_cls(g)
    for t in range(t_last + 1):
        rec = identity_record(g, t)
        m.step(t, {0: (rec, rec)})
        yield t, m


def seen_pairs_buffer(g, m):
    """Set of (frame, row) whose keys the buffer read sees."""
    vals = m.k[0, m.readable_rows(), 0, 0].astype(np.int64)
    return set(zip((vals // 10000).tolist(), (vals % 10000).tolist()))


def seen_pairs_rule(g, t):
    out = set()
    for f in range(t + 1):
        vis = so.frame_visibility(g, t, f)
        lo = 0 if vis == "whole" else (g.hw if vis == "summary" else g.r)
        out.update((f, r) for r in range(lo, g.r))
    return out


# --------------------------------------------------------------------------
# The figure "The buffer one frame apart" (section "One buffer, no mask")
# --------------------------------------------------------------------------
def _figure_check(replay_cls=so.MemoryReplay):
    fx = read_golden("buffer_figure_frame31.txt")
    g = so.Geometry(fx["hw"], fx["x"], fx["y"], fx["w"], 1, 1, 1, "f32")
    before = after = None
    for t, m in replay_identity(g, fx["step_to"], replay_cls):
        if t == fx["step_from"]:
            before = (list(m.raw_frame), list(m.sum_frame))
        if t == fx["step_to"]:
            after = (list(m.raw_frame), list(m.sum_frame))
    raw_b, sum_b = before
    raw_a, sum_a = after
    assert raw_a[raw_b.index(fx["raw_old"])] == fx["raw_new"]
    assert sum_a[sum_b.index(fx["sum_old"])] == fx["sum_new"]
    # the summary now in that SUM slot really is frame 28's summary rows
    u = sum_b.index(fx["sum_old"])
    lo, hi = g.sum_rows(u)
    vals = m.k[0, lo:hi, 0, 0].astype(np.int64)
    assert (vals // 10000 == fx["sum_new"]).all()
    assert ((vals % 10000) == np.arange(g.hw, g.r)).all()


def test_figure_frame31_slots():
    _figure_check()


def _full_tables_check(replay_cls=so.MemoryReplay):
    """The whole slot tables around the figure's step, from the slot formulas
    (RAW slot t mod (Y+1), SUM slot f mod (W-Y) for the summarised frame f)."""
    tables = {}
    for t, m in replay_identity(SERVED, 31, replay_cls):
        if t in (30, 31):
            tables[t] = (list(m.raw_frame), list(m.sum_frame))
    assert tables[30][0] == [30, 28, 29]
    assert tables[31][0] == [30, 31, 29]
    assert tables[30][1] == [22, 23, 24, 25, 26, 27, 6] + list(range(7, 22))
    assert tables[31][1] == [22, 23, 24, 25, 26, 27, 28] + list(range(7, 22))


def test_figure_frame31_full_tables():
    _full_tables_check()


# --------------------------------------------------------------------------
# The caption at the top of the page: 6,528 keys instead of 26,208
# --------------------------------------------------------------------------
def test_caption_key_counts():
    fx = read_golden("caption_key_counts.txt")
    g = so.Geometry(fx["hw"], fx["x"], fx["y"], fx["w"], 1, 1, 1, "f32")
    for t, m in replay_identity(g, 60):
        if t < g.w + 1:
            continue
        assert m.n_keys() == fx["keys"]
        pairs = seen_pairs_buffer(g, m)
        frames = sorted({f for f, _ in pairs})
        whole = [f for f in frames if f != 0 and sum(1 for ff, _ in pairs if ff == f) == g.r]
        summ = [f for f in frames if sum(1 for ff, _ in pairs if ff == f) == g.x]
        assert 0 in frames
        assert len(whole) == fx["whole_frames_besides_start"]
        assert len(summ) == fx["summary_frames"]
        # the same frames, each kept at full resolution (raw rows only)
        assert len(frames) * g.hw == fx["keys_full_resolution"]
    assert so.key_count(g, 31) == fx["keys"]


def test_key_counts_across_fill_levels():
    """Batched workload's fill levels: K(t) from the rule, the replay agrees."""
    want = {0: 1104, 1: 2208, 2: 3312, 3: 4416, 4: 4512, 10: 5088, 23: 6336, 24: 6432, 25: 6528, 31: 6528}
    got = {}
    for t, m in replay_identity(SERVED, 31):
        got[t] = m.n_keys()
        assert got[t] == so.key_count(SERVED, t)
    for t, k in want.items():
        assert got[t] == k
    assert so.key_count(TINY, 11) == 128 and TINY.capacity == 128
    assert [so.key_count(TINY, t) for t in range(8)] == [28, 56, 84, 112, 116, 120, 124, 128]
    assert so.key_count(LONG, 127) == 46688 == LONG.capacity


# --------------------------------------------------------------------------
# Section "What a frame attends to" against section "One buffer, no mask"
# --------------------------------------------------------------------------
@pytest.mark.parametrize("g", [TINY, SERVED, LONG,
                               so.Geometry(5, 3, 1, 4, 1, 1, 1, "f32"),
                               so.Geometry(7, 2, 3, 5, 1, 1, 1, "f32"),
                               so.Geometry(4, 1, 0, 3, 1, 1, 1, "f32")],
                         ids=["tiny", "served", "long", "g5x3y1w4", "g7x2y3w5", "g4x1y0w3"])
def test_window_membership_exhaustive(g):
    """The buffer sees exactly the (frame, row) pairs the attention-set rule lists, t <= 200."""
    t_last = 200 if g.r < 2000 else 120
    for t, m in replay_identity(g, t_last):
        assert seen_pairs_buffer(g, m) == seen_pairs_rule(g, t), f"t={t}"
        assert len(m.readable_segments()) <= 2
        assert m.n_keys() == so.key_count(g, t)


def _random_rollout(g, frames, seed, rewrites=()):
    """Replay with random f32 records; returns (replay snapshots, history)."""
    rng = np.random.default_rng(seed)
    m = so.MemoryReplay(g)
    hist_k, hist_v = {}, {}
    for t in frames:
        ev = m.evict(t) if t >= 1 else None
        for _ in range(1 + (t in rewrites)):
            k = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
            v = rng.standard_normal((g.r, g.n_heads, g.head_dim)).astype(np.float32)
            m.write(0, t, k, v)
        hist_k[t], hist_v[t] = k.astype(np.float64), v.astype(np.float64)
        yield t, m, hist_k, hist_v, rng


def test_bruteforce_tiny_buffer_equals_masked_history():
    """Buffer read == masked attention over all records, every t of the tiny rollout and past it."""
    g = TINY
    scale = so.default_scale(g.head_dim)
    for t, m, hk, hv, rng in _random_rollout(g, range(24), seed=11, rewrites={3, 9}):
        q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
        a = m.attend(0, q, scale)
        b = so.history_attention(g, t, q, hk, hv, scale)
        np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-14)


def test_bruteforce_multihead_geometry():
    g = so.Geometry(10, 3, 1, 5, 3, 8, 1, "f32")
    for t, m, hk, hv, rng in _random_rollout(g, range(14), seed=5):
        q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
        np.testing.assert_allclose(m.attend(0, q), so.history_attention(g, t, q, hk, hv, so.default_scale(8)),
                                   rtol=1e-12, atol=1e-14)


def test_eviction_and_write_invariants():
    """Z0 = record 0; RAW slot = its frame's last write; SUM slot = rows [HW, R) of its frame; empty = 0."""
    g = so.Geometry(6, 2, 2, 6, 2, 4, 1, "f32")
    for t, m, hk, hv, _ in _random_rollout(g, range(20), seed=3, rewrites={2, 5, 6, 13}):
        lo, hi = g.z0_rows()
        np.testing.assert_array_equal(m.k[0, lo:hi], hk[0].astype(np.float32))
        for s, f in enumerate(m.raw_frame):
            lo, hi = g.raw_rows(s)
            if f >= 1:
                np.testing.assert_array_equal(m.v[0, lo:hi], hv[f].astype(np.float32))
            elif t >= 0 and f < 0:
                assert not m.k[0, lo:hi].any()
        for u, f in enumerate(m.sum_frame):
            lo, hi = g.sum_rows(u)
            if f >= 1:
                np.testing.assert_array_equal(m.k[0, lo:hi], hk[f][g.hw:].astype(np.float32))
                np.testing.assert_array_equal(m.v[0, lo:hi], hv[f][g.hw:].astype(np.float32))
            else:
                assert not m.k[0, lo:hi].any() and not m.v[0, lo:hi].any()


# --------------------------------------------------------------------------
# Closed forms of softmax attention
# --------------------------------------------------------------------------
def test_two_key_closed_form():
    """q=(1,0), k1=(2,0), k2=(0,0), scale 1: weights e^2/(e^2+1) and 1/(e^2+1)."""
    q = np.array([[[1.0, 0.0]]])
    k = np.array([[[2.0, 0.0]], [[0.0, 0.0]]])
    v = np.array([[[3.0, -1.0]], [[1.0, 5.0]]])
    e2 = math.exp(2.0)
    want = (e2 * v[0, 0] + v[1, 0]) / (e2 + 1.0)
    np.testing.assert_allclose(so.attention_f64(q, k, v, 1.0)[0, 0], want, rtol=1e-15)
    # the same with scale 0.5 halves the score: weights e/(e+1), 1/(e+1)
    e1 = math.exp(1.0)
    np.testing.assert_allclose(so.attention_f64(q, k, v, 0.5)[0, 0], (e1 * v[0, 0] + v[1, 0]) / (e1 + 1.0),
                               rtol=1e-15)


def test_closed_forms_random():
    rng = np.random.default_rng(0)
    n, m, h, d = 7, 33, 3, 16
    q = rng.standard_normal((n, h, d))
    k = rng.standard_normal((m, h, d))
    v = rng.standard_normal((m, h, d))
    s = 0.25
    # Q = 0: uniform weights, O = mean of V
    np.testing.assert_allclose(so.attention_f64(np.zeros_like(q), k, v, s),
                               np.broadcast_to(v.mean(0), (n, h, d)), rtol=1e-13, atol=1e-15)
    # all keys equal: uniform weights again
    kk = np.broadcast_to(k[:1], k.shape).copy()
    np.testing.assert_allclose(so.attention_f64(q, kk, v, s),
                               np.broadcast_to(v.mean(0), (n, h, d)), rtol=1e-12, atol=1e-14)
    # one key: O = that V row
    np.testing.assert_allclose(so.attention_f64(q, k[:1], v[:1], s), np.broadcast_to(v[0], (n, h, d)), rtol=1e-15)
    # permuting keys (with their values) changes nothing
    p = rng.permutation(m)
    np.testing.assert_allclose(so.attention_f64(q, k[p], v[p], s), so.attention_f64(q, k, v, s), rtol=1e-12)
    # a dominant key (50 x q for query 0) selects its value row
    k2 = k.copy()
    k2[5] = 50.0 * q[0]
    o = so.attention_f64(q[:1], k2, v, 1.0)
    np.testing.assert_allclose(o[0], v[5], rtol=0, atol=1e-12)


def test_matches_torch_sdpa_float64():
    """The exact attention is textbook SDPA: torch float64 on gathered buffer rows agrees."""
    g = so.Geometry(12, 4, 2, 7, 4, 16, 1, "f32")
    for t, m, hk, hv, rng in _random_rollout(g, range(12), seed=9):
        q = rng.standard_normal((g.r, g.n_heads, g.head_dim))
        kf, vf = m.gathered(0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(kf).permute(1, 0, 2),
            torch.from_numpy(vf).permute(1, 0, 2)).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(m.attend(0, q), ref, rtol=1e-11, atol=1e-13)


def test_default_scale():
    assert so.default_scale(64) == 0.125
    assert so.default_scale(128) == 1.0 / math.sqrt(128.0)


def test_bf16_decode():
    bits = np.array([0x3F80, 0xC000, 0x3F81, 0x0000, 0x8000, 0x7F7F, 0x0001], dtype=np.uint16)
    want = np.array([1.0, -2.0, 1.0078125, 0.0, -0.0, 3.3895313892515355e38, 9.183549615799121e-41])
    np.testing.assert_array_equal(so.bf16_bits_to_f64(bits), want)
    # agrees with torch's own bfloat16 -> float64 conversion
    x = sf_inputs.draw((1000,), 1234, "bf16")
    np.testing.assert_array_equal(so.bf16_bits_to_f64(sf_inputs.to_host_bytes(x)), x.double().numpy())


def test_served_bf16_step_matches_sdpa():
    """One served-shape block at frame 3 in bf16 storage: replay + attention against torch SDPA."""
    wl = dict(sf_inputs.WORKLOADS["served1"])
    g = so.Geometry.from_workload(wl)
    m = so.MemoryReplay(g)
    for t in range(4):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t)
        m.step(t, {0: (sf_inputs.to_host_bytes(k), sf_inputs.to_host_bytes(v))})
    rows = np.arange(0, g.r, 37)
    o = m.attend(0, sf_inputs.to_host_bytes(q), rows=rows)
    kf, vf = m.gathered(0)
    qd = q.double()[torch.from_numpy(rows)]
    ref = torch.nn.functional.scaled_dot_product_attention(
        qd.permute(1, 0, 2), torch.from_numpy(kf).permute(1, 0, 2), torch.from_numpy(vf).permute(1, 0, 2)
    ).permute(1, 0, 2).numpy()
    np.testing.assert_allclose(o, ref, rtol=1e-10, atol=1e-13)
    assert m.n_keys() == 4416


# --------------------------------------------------------------------------
# Planted mistakes: each must be caught by some pin above
# --------------------------------------------------------------------------
class _EvictRawRows(so.MemoryReplay):
    """Mistake: copies the first X rows of the leaving record (raw rows) instead of the summary rows."""

    def evict(self, t):
        g = self.g
        s = self.raw_slot(t)
        f = self.raw_frame[s]
        if t <= g.y or f < 1:
            return None
        u = self.sum_slot(f)
        src0 = g.raw_rows(s)[0]
        d0, d1 = g.sum_rows(u)
        self.k[:, d0:d1] = self.k[:, src0:src0 + g.x]
        self.v[:, d0:d1] = self.v[:, src0:src0 + g.x]
        self.sum_frame[u] = f
        return s, u, f


class _SumSlotByCurrentFrame(so.MemoryReplay):
    """Mistake: SUM slot chosen by the frame being written, not the frame being summarised."""

    def evict(self, t):
        g = self.g
        s = self.raw_slot(t)
        f = self.raw_frame[s]
        if t <= g.y or f < 1:
            return None
        u = t % g.n_sum
        d0, d1 = g.sum_rows(u)
        self.k[:, d0:d1] = self.k[:, g.raw_rows(s)[0] + g.hw:g.raw_rows(s)[1]]
        self.v[:, d0:d1] = self.v[:, g.raw_rows(s)[0] + g.hw:g.raw_rows(s)[1]]
        self.sum_frame[u] = f
        return s, u, f


class _NoZ0(so.MemoryReplay):
    """Mistake: the start image is left out of the read."""

    def readable_segments(self):
        segs = super().readable_segments()
        b, n = segs[0]
        return ([(b + self.g.r, n - self.g.r)] if n > self.g.r else []) + segs[1:]


class _WriteBeforeEvict(so.MemoryReplay):
    """Mistake: the new record is written before the leaving frame's summary is copied."""

    def step(self, t, records):
        for b, (k, v) in records.items():
            self.write(b, t, k, v)
        s = self.raw_slot(t)
        g = self.g
        if t > g.y:
            f = t - g.y - 1
            if f >= 1:
                u = self.sum_slot(f)
                d0, d1 = g.sum_rows(u)
                self.k[:, d0:d1] = self.k[:, g.raw_rows(s)[0] + g.hw:g.raw_rows(s)[1]]
                self.v[:, d0:d1] = self.v[:, g.raw_rows(s)[0] + g.hw:g.raw_rows(s)[1]]
                self.sum_frame[u] = f


def _membership_check(cls, g=TINY, t_last=30):
    for t, m in replay_identity(g, t_last, cls):
        if seen_pairs_buffer(g, m) != seen_pairs_rule(g, t):
            raise AssertionError(f"membership differs at t={t}")


@pytest.mark.parametrize("cls", [_EvictRawRows, _SumSlotByCurrentFrame, _NoZ0, _WriteBeforeEvict])
def test_planted_mistakes_are_caught(cls):
    caught = []
    for check in (_membership_check, _figure_check, _full_tables_check):
        try:
            check(cls)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"{cls.__doc__} was not caught"


def test_planted_attention_mistakes_are_caught():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((5, 2, 8))
    k = rng.standard_normal((9, 2, 8))
    v = rng.standard_normal((9, 2, 8))
    sd = lambda: torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q).permute(1, 0, 2), torch.from_numpy(k).permute(1, 0, 2),
        torch.from_numpy(v).permute(1, 0, 2)).permute(1, 0, 2).numpy()
    ref = sd()
    good = so.attention_f64(q, k, v, so.default_scale(8))
    np.testing.assert_allclose(good, ref, rtol=1e-12)
    bad_scale = so.attention_f64(q, k, v, 1.0)
    assert not np.allclose(bad_scale, ref, rtol=1e-6)
    # keys of the wrong head
    bad_head = so.attention_f64(q, k[:, ::-1], v, so.default_scale(8))
    assert not np.allclose(bad_head, ref, rtol=1e-6)
