"""Host logic of libsf on the CPU: exports, slot map against the oracle, ordering and error rules.

No device work: dry-run handles (dev_mem NULL) validate and advance state like
real ones without touching a GPU.  Page: model card "GTA world model: weights
and inference code", section "One buffer, no mask".
"""
import os
import re

import ctypes

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import compressed_memory_kv_amd as sf
import sf_inputs
from oracle import sf_oracle as so

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    with open(os.path.join(ROOT, "include", "sf.h")) as fh:
        text = fh.read()
    return sorted(set(re.findall(r"\b(sf_[a-z_0-9]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    names = header_functions()
    assert len(names) >= 14
    lib = sf._lib
    for n in names:
        assert hasattr(lib, n), f"{n} declared in include/sf.h but not exported by libsf.so"
    assert set(names) == set(sf.EXPORTED)


def test_exports_via_nm():
    import subprocess
    out = subprocess.run(["nm", "-D", "--defined-only", sf.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (sf_[a-z_0-9]+)$", out, re.M))
    assert set(header_functions()) <= exported


GEOMS = {
    "tiny": sf_inputs.WORKLOADS["tiny"],
    "served": sf_inputs.WORKLOADS["rollout"],
    "long": sf_inputs.WORKLOADS["long"],
    "odd": dict(hw=5, x=3, y=1, w=4, n_heads=2, head_dim=64, n_blocks=3, dtype="bf16"),
    "y0": dict(hw=7, x=2, y=0, w=3, n_heads=1, head_dim=128, n_blocks=2, dtype="f32"),
    "served16": sf_inputs.WORKLOADS["served16"],
}


def oracle_tables(wl, t_last):
    g = so.Geometry(wl["hw"], wl["x"], wl["y"], wl["w"], 1, 1, 1, "f32")
    m = so.MemoryReplay(g)
    one = np.zeros((g.r, 1, 1), np.float32)
    for t in range(t_last + 1):
        m.step(t, {0: (one, one)})
        yield t, m


@pytest.mark.parametrize("name", list(GEOMS))
def test_plan_matches_oracle(name):
    wl = GEOMS[name]
    cfg = sf.make_config(**wl)
    empty = sf.sf_plan(cfg, -1)
    assert empty["t_cur"] == -1 and empty["n_keys"] == 0 and empty["segments"] == []
    t_last = 140 if name != "long" else 110
    for t, m in oracle_tables(wl, t_last):
        p = sf.sf_plan(cfg, t)
        assert p["raw_frame"] == m.raw_frame, t
        assert p["sum_frame"] == m.sum_frame, t
        assert p["segments"] == m.readable_segments(), t
        assert p["n_keys"] == m.n_keys() == so.key_count(so.Geometry.from_workload(dict(wl)), t)
        assert p["t_cur"] == t
        assert p["raw_slot"] == (t % (wl["y"] + 1) if t >= 1 else -1)


def test_buffer_sizes_and_offsets():
    wl = sf_inputs.WORKLOADS["rollout"]
    cfg = sf.make_config(**wl)
    C = 1104 * 4 + 22 * 96
    assert C == 6528
    per_tensor = C * 16 * 64 * 2
    assert sf.sf_kv_bytes(cfg) == 28 * 2 * per_tensor
    assert sf.sf_kv_offset(cfg, 0, 0) == 0
    assert sf.sf_kv_offset(cfg, 0, 1) == per_tensor
    assert sf.sf_kv_offset(cfg, 5, 1) == 5 * 2 * per_tensor + per_tensor
    assert sf.sf_kv_offset(cfg, 28, 0) == -1 and sf.sf_kv_offset(cfg, 0, 2) == -1
    assert sf.sf_buffer_bytes(cfg) >= sf.sf_kv_bytes(cfg)
    lwl = sf_inputs.WORKLOADS["long"]
    lcfg = sf.make_config(**lwl)
    assert sf.sf_kv_bytes(lcfg) == 28 * 2 * 46688 * 24 * 128 * 2


@pytest.mark.parametrize("bad,code", [
    (dict(hw=0), sf.SF_E_ARG), (dict(x=0), sf.SF_E_ARG), (dict(y=-1), sf.SF_E_ARG), (dict(w=2), sf.SF_E_ARG),
    (dict(n_heads=0), sf.SF_E_ARG), (dict(n_blocks=0), sf.SF_E_ARG), (dict(dtype=7), sf.SF_E_ARG),
    (dict(head_dim=96), sf.SF_E_UNSUPPORTED), (dict(max_frames=-1), sf.SF_E_ARG),
    (dict(sink_gap=1), sf.SF_E_ARG), (dict(sink_gap=-2), sf.SF_E_ARG), (dict(sink_gap=5, rope_theta=1.0), sf.SF_E_ARG),
    (dict(rope_mode=3), sf.SF_E_ARG), (dict(rope_mode="replace", rope_theta=0.5), sf.SF_E_ARG),
    # [level]: at base 1000 the two slowest planes turn 3.2 rad over 1024 frames: not idle
    (dict(rope_mode="replace", rope_theta=1000.0), sf.SF_E_UNSUPPORTED),
    (dict(rope_mode="add", rope_theta=2048.0 ** 1.2 * 0.999), sf.SF_E_UNSUPPORTED),
])
def test_config_errors(bad, code):
    wl = dict(GEOMS["tiny"])
    wl.update(bad)
    cfg = sf.make_config(**wl)
    with pytest.raises(sf.SfError) as ei:
        sf.sf_config_check(cfg)
    assert ei.value.status == code
    assert sf.sf_buffer_bytes(cfg) == 0


def dry_session(name="tiny", **over):
    wl = dict(GEOMS[name])
    wl.update(over)
    return sf.Session(sf.make_config(**wl), dry=True), wl


def advance(s, wl, t):
    for b in range(wl["n_blocks"]):
        sf.sf_step(s.handle, b, t, None, None, None, None)


def test_dry_session_follows_plan():
    for name in ("tiny", "odd", "y0"):
        s, wl = dry_session(name)
        for t in range(40):
            advance(s, wl, t)
            v = s.view()
            p = sf.sf_plan(s.cfg, t)
            for key in ("t_cur", "n_keys", "segments", "raw_frame", "sum_frame", "evicted_for", "raw_slot"):
                assert v[key] == p[key], (name, t, key)
            assert v["blocks_written"] == wl["n_blocks"]


def test_explicit_evict_write_attend_sequence():
    s, wl = dry_session("odd")
    h = s.handle
    for t in range(12):
        if t >= 1:
            sf.sf_evict(h, t)
            sf.sf_evict(h, t)  # repeating the eviction for the same frame is a no-op
        for b in range(wl["n_blocks"]):
            sf.sf_write_record(h, b, t, None, None)
            sf.sf_write_record(h, b, t, None, None)  # the clean pass rewrites the entry
            sf.sf_attend([h], b, None, None)
        assert s.view() == {**sf.sf_plan(s.cfg, t), "blocks_written": wl["n_blocks"]}


def expect(code, fn, *args):
    with pytest.raises(sf.SfError) as ei:
        fn(*args)
    assert ei.value.status == code, (ei.value, code)


def test_ordering_errors_leave_state_unchanged():
    s, wl = dry_session("tiny", max_frames=20)
    h = s.handle
    expect(sf.SF_E_STATE, sf.sf_attend, [h], 0, None, None)       # nothing written yet
    expect(sf.SF_E_ORDER, sf.sf_write_record, h, 0, 1, None, None)  # skipping frame 0
    for t in range(5):
        advance(s, wl, t)
    before = s.view()
    expect(sf.SF_E_ORDER, sf.sf_write_record, h, 0, 6, None, None)  # skipping a frame
    expect(sf.SF_E_ORDER, sf.sf_write_record, h, 0, 3, None, None)  # going back
    expect(sf.SF_E_ORDER, sf.sf_write_record, h, 0, 5, None, None)  # frame 4 leaves RAW unevicted
    expect(sf.SF_E_ORDER, sf.sf_evict, h, 4)                          # eviction is for t_cur + 1
    expect(sf.SF_E_ORDER, sf.sf_evict, h, 7)
    expect(sf.SF_E_ARG, sf.sf_write_record, h, 1, 4, None, None)     # block out of range
    expect(sf.SF_E_ARG, sf.sf_write_record, h, -1, 4, None, None)
    expect(sf.SF_E_ARG, sf.sf_attend, [h], 3, None, None)
    assert s.view() == before
    for t in range(5, 20):
        advance(s, wl, t)
    expect(sf.SF_E_RANGE, sf.sf_evict, h, 20)
    expect(sf.SF_E_RANGE, sf.sf_write_record, h, 0, 20, None, None)
    expect(sf.SF_E_RANGE, sf.sf_step, h, 0, 20, None, None, None, None)


def test_advance_needs_every_block():
    s, wl = dry_session("odd")
    h = s.handle
    advance(s, wl, 0)
    sf.sf_write_record(h, 0, 1, None, None)
    expect(sf.SF_E_ORDER, sf.sf_evict, h, 2)                         # blocks 1, 2 still hold frame 0
    expect(sf.SF_E_ORDER, sf.sf_write_record, h, 0, 2, None, None)
    expect(sf.SF_E_STATE, sf.sf_attend, [h], 1, None, None)           # block 1 does not hold frame 1
    sf.sf_attend([h], 0, None, None)


def test_attend_refused_after_next_eviction():
    """[attends]: once sf_evict(t_cur + 1) has run, SUM no longer holds what frame t_cur sees
    (the leaving frame's summary replaced an older one), so a read of t_cur is SF_E_STATE, and
    so is an sf_step rewrite of t_cur; the write of t_cur + 1 then reopens reads."""
    s, wl = dry_session("tiny", hw=4, x=2, y=2, w=6, n_blocks=1)
    h = s.handle
    for t in range(10):
        advance(s, wl, t)
    sf.sf_attend([h], 0, None, None)
    sf.sf_evict(h, 10)
    v = s.view()
    assert v["t_cur"] == 9 and v["evicted_for"] == 10
    # frame 7's summary now sits in SUM beside its raw rows: frame 9 would count it twice
    assert 7 in v["raw_frame"] and 7 in v["sum_frame"] and 3 not in v["sum_frame"]
    expect(sf.SF_E_STATE, sf.sf_attend, [h], 0, None, None)
    expect(sf.SF_E_STATE, sf.sf_step, h, 0, 9, None, None, None, None)
    sf.sf_write_record(h, 0, 9, None, None)          # a rewrite of frame 9's rows is harmless
    assert s.view() == v
    sf.sf_write_record(h, 0, 10, None, None)
    sf.sf_attend([h], 0, None, None)


def test_batched_attend_checks():
    a, wl = dry_session("odd")
    b, _ = dry_session("odd")
    c, _ = dry_session("odd", n_heads=4)
    for s in (a, b, c):
        advance(s, wl, 0)
    sf.sf_attend([a.handle, b.handle], 1, None, None)
    expect(sf.SF_E_ARG, sf.sf_attend, [a.handle, c.handle], 1, None, None)  # heads differ
    expect(sf.SF_E_ARG, sf.sf_attend, [a.handle, a.handle], 1, None, None)  # listed twice
    expect(sf.SF_E_ARG, sf.sf_attend, [], 0, None, None)
    expect(sf.SF_E_ARG, sf.sf_attend, [a.handle] * 65, 0, None, None)


def test_injected_launch_failure_keeps_state():
    s, wl = dry_session("tiny")
    h = s.handle
    for t in range(6):
        advance(s, wl, t)
    before = s.view()
    sf.sf_debug_fail_next_launch(h)
    expect(sf.SF_E_HIP, sf.sf_step, h, 0, 6, None, None, None, None)
    assert s.view() == before
    assert "injected" in sf.sf_last_error(h)
    sf.sf_step(h, 0, 6, None, None, None, None)                      # the next call goes through
    assert s.view()["t_cur"] == 6
    sf.sf_debug_fail_next_launch(h)
    expect(sf.SF_E_HIP, sf.sf_attend, [h], 0, None, None)
    sf.sf_attend([h], 0, None, None)


def test_status_strings():
    assert sf.sf_status_str(sf.SF_E_ORDER) == "SF_E_ORDER"
    assert sf.sf_status_str(0) == "SF_OK"
    assert sf.sf_status_str(-99) == "SF_E_UNKNOWN"


@settings(max_examples=150, deadline=None)
@given(hw=st.integers(1, 40), x=st.integers(1, 12), y=st.integers(0, 5), extra=st.integers(1, 12),
       t=st.integers(-1, 90))
def test_plan_properties(hw, x, y, extra, t):
    w = y + extra
    cfg = sf.make_config(hw, x, y, w, 1, 64, 1, "f32")
    p = sf.sf_plan(cfg, t)
    g = so.Geometry(hw, x, y, w, 1, 1, 1, "f32")
    if t < 0:
        assert p["n_keys"] == 0
        return
    assert p["n_keys"] == so.key_count(g, t)
    assert 1 <= len(p["segments"]) <= 2
    assert sum(n for _, n in p["segments"]) == p["n_keys"]
    C = g.capacity
    ends = [b + n for b, n in p["segments"]]
    assert all(0 <= b < e <= C for (b, _), e in zip(p["segments"], ends))
    frames = [f for f in p["raw_frame"] if f >= 0] + [f for f in p["sum_frame"] if f >= 0]
    assert len(frames) == len(set(frames))                         # slots disjoint
    assert set(f for f in p["raw_frame"] if f >= 1) == set(range(max(1, t - y), t + 1))
    assert set(f for f in p["sum_frame"] if f >= 1) == set(range(max(1, t - w), t - y))
    if t >= w + 1:
        assert p["segments"] == [(0, C)]                           # steady state: one dense prefix


def test_tracing_on_dry_handles():
    s, wl = dry_session("tiny")
    expect(sf.SF_E_STATE, sf.sf_profile_enable, s.handle, True)
    times = sf.sf_kernel_times_read(s.handle)
    assert all(ms == 0.0 and n == 0 for ms, n in times.values())
    assert set(times) == set(sf.KERNEL_KINDS)


@pytest.mark.parametrize("name,gap", [("tiny", 5), ("odd", 3), ("y0", 5), ("tiny", 0)])
def test_sink_schedule_matches_oracle(name, gap):
    """[sink]: the frame Z0's keys are rotated to, in the plan and in a dry session
    stepped frame by frame, follows the oracle's replay (no device work)."""
    wl = dict(GEOMS[name], sink_gap=gap)
    cfg = sf.make_config(**wl)
    g = so.Geometry.from_workload(wl)
    m = so.MemoryReplay(g, blocks=[0], sink_gap=gap)
    one = np.zeros((g.r, g.n_heads, g.head_dim), np.float32)
    s = sf.Session(cfg, dry=True)
    moved = 0
    for t in range(90):
        m.step(t, {0: (one, one)})
        advance(s, wl, t)
        p = sf.sf_plan(cfg, t)
        assert p["z0_frame"] == m.z0_frame == s.view()["z0_frame"], (name, t)
        moved += m.z0_frame > 0
    assert (moved > 0) == (gap > 0)


def test_served16_key_count():
    """The server's default window W = 16 ([buffer] parameter table): R(Y+2) + (W-Y)X keys."""
    cfg = sf.make_config(**GEOMS["served16"])
    assert sf.sf_plan(cfg, 40)["n_keys"] == 1104 * 4 + 14 * 96 == 5760


def test_zero_copy_slot_rules():
    """sf_record_slot / sf_commit_record follow the write rules and move the state like a write."""
    s, wl = dry_session("tiny")
    for t in range(12):
        if t >= 1:
            if t > wl["y"] + 1:
                with pytest.raises(sf.SfError) as ei:   # a frame must leave RAW first
                    sf.sf_record_slot(s.handle, 0, t)
                assert ei.value.status == sf.SF_E_ORDER
                with pytest.raises(sf.SfError):
                    sf.sf_commit_record(s.handle, 0, t)
            s.evict(t)
        before = s.view()
        assert sf.sf_record_slot(s.handle, 0, t) == (0, 0)   # dry handle: no device rows
        assert s.view() == before                            # asking changes nothing
        s.commit_record(0, t)
        p = sf.sf_plan(s.cfg, t)
        for key in ("t_cur", "n_keys", "segments", "raw_frame", "sum_frame"):
            assert s.view()[key] == p[key], (t, key)
        s.commit_record(0, t)                                # a rewrite commit
    with pytest.raises(sf.SfError) as ei:
        sf.sf_commit_record(s.handle, 0, 14)
    assert ei.value.status == sf.SF_E_ORDER


def test_four_pass_frames_evict_once():
    """[sampling]: three denoising passes and a clean pass rewrite the same frame; the state
    after each frame equals one write per frame."""
    s, wl = dry_session("odd")
    for t in range(30):
        for _ in range(4):
            advance(s, wl, t)
        p = sf.sf_plan(s.cfg, t)
        v = s.view()
        for key in ("t_cur", "n_keys", "segments", "raw_frame", "sum_frame", "evicted_for"):
            assert v[key] == p[key], (t, key)


def test_state_export_import():
    """A session's host state moves to a new handle and both continue alike; bad records fail."""
    a, wl = dry_session("tiny", sink_gap=5)
    for t in range(25):
        advance(a, wl, t)
    data = a.export_state()
    assert len(data) == sf.sf_state_bytes(a.cfg) > 0
    b = sf.Session(a.cfg, dry=True)
    b.import_state(data)
    assert b.view() == a.view()
    for t in range(25, 40):
        advance(a, wl, t)
        advance(b, wl, t)
        assert b.view() == a.view(), t
    fresh = sf.Session(a.cfg, dry=True)
    empty = fresh.view()
    bad = bytearray(data)
    bad[0] ^= 1                                              # not a state record
    with pytest.raises(sf.SfError):
        fresh.import_state(bytes(bad))
    other = sf.Session(sf.make_config(**dict(wl, sink_gap=0)), dry=True)
    with pytest.raises(sf.SfError):                          # another config
        other.import_state(data)
    off = 8 + ctypes.sizeof(sf.sf_config) + 3 * 8           # raw_frame[0]
    bad = bytearray(data)
    bad[off:off + 8] = (7).to_bytes(8, "little", signed=True)   # frame 7 cannot sit in RAW slot 0
    with pytest.raises(sf.SfError):
        fresh.import_state(bytes(bad))
    assert fresh.view() == empty


@pytest.mark.parametrize("head_dim,theta", [(64, 10000.0), (128, 10000.0), (64, 2048.0 ** 1.2 * 1.001),
                                            (64, 1000.0), (128, 500.0)])
def test_level_idle_check_matches_oracle(head_dim, theta):
    """[level]: the library builds a rope-mode session exactly when the oracle's idle check passes."""
    cfg = sf.make_config(**dict(GEOMS["tiny"], head_dim=head_dim, rope_mode="add", rope_theta=theta))
    ok = sf.sf_buffer_bytes(cfg) > 0
    assert ok == so.level_planes_idle(head_dim, theta)


def test_rope_mode_sizes_and_rules():
    """Rope modes keep the K/V layout, add room for one rotated query, refuse zero-copy writes
    and otherwise follow the same plan as the caller mode."""
    wl = GEOMS["served"]
    base = sf.make_config(**wl)
    for mode in ("replace", "add"):
        cfg = sf.make_config(**dict(wl, rope_mode=mode))
        assert sf.sf_kv_bytes(cfg) == sf.sf_kv_bytes(base)
        assert sf.sf_kv_offset(cfg, 3, 1) == sf.sf_kv_offset(base, 3, 1)
        assert sf.sf_buffer_bytes(cfg) >= sf.sf_buffer_bytes(base) + 1104 * 16 * 64 * 2
    s, wl2 = dry_session("odd", rope_mode="replace", sink_gap=3)
    with pytest.raises(sf.SfError) as ei:
        sf.sf_record_slot(s.handle, 0, 0)
    assert ei.value.status == sf.SF_E_UNSUPPORTED
    with pytest.raises(sf.SfError) as ei:
        sf.sf_commit_record(s.handle, 0, 0)
    assert ei.value.status == sf.SF_E_UNSUPPORTED
    for t in range(30):
        advance(s, wl2, t)
        p = sf.sf_plan(s.cfg, t)
        v = s.view()
        for key in ("t_cur", "n_keys", "segments", "raw_frame", "sum_frame", "z0_frame"):
            assert v[key] == p[key], (t, key)
    with pytest.raises(sf.SfError) as ei:           # the caller mode has nothing to turn
        sf.sf_rope_rows(sf.make_config(**GEOMS["tiny"]), 0, 16, 16)
    assert ei.value.status == sf.SF_E_ARG
    cfg = sf.make_config(**dict(GEOMS["tiny"], rope_mode="add"))
    for t, src, code in ((0, 8, sf.SF_E_ARG), (-1, 16, sf.SF_E_RANGE), (0, None, sf.SF_E_ARG)):
        with pytest.raises(sf.SfError) as ei:       # misaligned, bad frame id, NULL: refused before any launch
            sf.sf_rope_rows(cfg, t, src, 16)
        assert ei.value.status == code
    bad = sf.make_config(**GEOMS["tiny"])
    bad.recency_bias = 2
    with pytest.raises(sf.SfError):
        sf.sf_config_check(bad)


def test_recency_bias_sizes_and_rules():
    """[files], [credits] The recency bias: room for its table [H][W+1] and the per-row
    biases [H][C] (fp32), the split-key scratch at bf16 head_dim 64, and its call rules."""
    for name in ("tiny", "served"):
        wl = GEOMS[name]
        plain = sf.make_config(**wl)
        cfg = sf.make_config(**dict(wl, recency_bias=True))
        sf.sf_config_check(cfg)
        h, w = wl["n_heads"], wl["w"]
        r = wl["hw"] + wl["x"]
        c = r * (wl["y"] + 2) + (w - wl["y"]) * wl["x"]
        assert sf.sf_buffer_bytes(cfg) >= sf.sf_kv_bytes(cfg) + h * (w + 1) * 4 + h * c * 4
        assert sf.sf_kv_bytes(cfg) == sf.sf_kv_bytes(plain)
        if wl["dtype"] == "f32":                     # no scratch: exactly the bias regions more
            assert sf.sf_buffer_bytes(cfg) - sf.sf_buffer_bytes(plain) >= h * (w + 1) * 4 + h * c * 4
        s = sf.Session(cfg, dry=True)
        s.set_recency_bias(None)                     # a dry handle takes no table
        for t in range(12):                          # the bias changes no slot rule
            advance(s, wl, t)
            s.set_recency_bias(None)
            p = sf.sf_plan(cfg, t)
            assert all(s.view()[k] == p[k] for k in ("t_cur", "n_keys", "segments", "raw_frame", "sum_frame"))
        with pytest.raises(sf.SfError) as ei:       # no bias in this config
            sf.Session(plain, dry=True).set_recency_bias(None)
        assert ei.value.status == sf.SF_E_UNSUPPORTED
    with pytest.raises(sf.SfError) as ei:
        sf.sf_set_recency_bias(0, None)
    assert ei.value.status == sf.SF_E_ARG


def test_lds_copy_argument_checks():
    """The calibration copy checks its arguments before any launch (no GPU needed)."""
    sf.sf_debug_lds_copy(0x100000, 0x200000, 0)  # nothing to copy: no launch
    for dst, src, n in ((0, 0x200000, 16384), (0x100008, 0x200000, 16384), (0x100000, 0x200000, 16000),
                        (0x100000, 0x102000, 16384)):
        with pytest.raises(sf.SfError) as ei:
            sf.sf_debug_lds_copy(dst, src, n)
        assert ei.value.status == sf.SF_E_ARG
