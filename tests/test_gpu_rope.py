"""GPU parity of the temporal band applied by the memory, with level planes.

Page: model card "GTA world model: weights and inference code", sections "Telling a
summary from a pixel: level planes" and "Running for a long time: the start image
follows the window", and the "Positions" item.  The library turns in fp32 and rounds
to the storage type; the oracle turns in fp64 and rounds once.  So a turned value may
differ by one unit in the last place of the storage type, at rounding ties only; the
quarter turn of the replace reading, the bands past the temporal one, values and slot
tables must match exactly, and attention outputs within the usual tolerance.
"""
import sys

import numpy as np
import pytest
import torch

import sf_inputs
from oracle import sf_oracle as so
from test_gpu_sink import TOL, plane_norm, ulp

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")
MODES = {"replace": so.ROPE_LEVEL_REPLACE, "add": so.ROPE_LEVEL_ADD}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host_bits(t: torch.Tensor) -> np.ndarray:
    return sf_inputs.to_host_bytes(t)


def check_turned(got: np.ndarray, want: np.ndarray, head_dim: int, dtype: str, hw: int, mode: int, what: str,
                 moves: int = 1):
    """got against the oracle's bytes: equal outside the temporal band and on the replace
    reading's quarter turn; elsewhere within `moves` units in the last place plus fp32 error."""
    n = so.temporal_planes(head_dim)
    np.testing.assert_array_equal(got[..., 2 * n:], want[..., 2 * n:], err_msg=f"{what}: past the temporal band")
    if mode == so.ROPE_LEVEL_REPLACE:
        np.testing.assert_array_equal(got[hw:, ..., 2 * n - 4:2 * n], want[hw:, ..., 2 * n - 4:2 * n],
                                      err_msg=f"{what}: quarter turn")
    a, o = so.stored_to_f64(got), so.stored_to_f64(want)
    bound = moves * (ulp(o, dtype) + 16 * 2.0 ** -24 * plane_norm(o, head_dim)) + 1e-30
    ratio = float((np.abs(a - o) / bound).max())
    say(f"   {what}: {int((got != want).sum())} of {got.size} differ from the oracle's rounding; "
        f"worst {ratio:.2f} of the bound")
    assert ratio <= 1.0, what


CASES = {
    "served_bf16": dict(hw=1008, x=96, y=2, w=24, n_heads=16, head_dim=64, n_blocks=1, dtype="bf16", seed=1,
                        v_scale=1.0),
    "tiny_f32": dict(sf_inputs.WORKLOADS["tiny"]),
    "hd128_bf16": dict(hw=40, x=8, y=0, w=3, n_heads=3, head_dim=128, n_blocks=2, dtype="bf16", seed=9,
                       v_scale=1.0),
    "hd128_f32": dict(hw=33, x=5, y=1, w=4, n_heads=2, head_dim=128, n_blocks=1, dtype="f32", seed=12,
                      v_scale=1.0),
}


@needs_gpu
@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("case", list(CASES))
def test_rope_rows_matches_oracle(case, mode):
    """sf_rope_rows on a record's rows at several frame ids, out of place and in place."""
    wl = dict(CASES[case], rope_mode=mode)
    cfg = sf.make_config(**wl)
    g = so.Geometry.from_workload(wl)
    for t in (0, 1, 37, 1023, 4095):
        say(f"[rope_rows] {case} {mode} t={t}")
        q = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")[0]
        dst = torch.empty_like(q)
        sf.sf_rope_rows(cfg, t, q, dst)
        inplace = q.clone()
        sf.sf_rope_rows(cfg, t, inplace, inplace)
        torch.cuda.synchronize()
        want = so.rope_record(host_bits(q), g.hw, t, g.head_dim, g.dtype, mode=MODES[mode])
        got = host_bits(dst)
        check_turned(got, want, g.head_dim, g.dtype, g.hw, MODES[mode], f"t={t}")
        np.testing.assert_array_equal(host_bits(inplace), got)


def run_rollout(wl, frames, attend_at, use_step):
    g = so.Geometry.from_workload(wl)
    mode = so.ROPE_LEVEL_REPLACE if wl["rope_mode"] == "replace" else so.ROPE_LEVEL_ADD
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g, sink_gap=wl.get("sink_gap", 0), rope_mode=mode)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    nb, r = wl["n_blocks"], g.r
    moves = 0
    for t in frames:
        z = sess.view()["z0_frame"]
        recs, qs = {}, {}
        if not use_step and t >= 1:
            sess.evict(t)
        for b in range(nb):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            if use_step:
                sess.step(b, t, q, k, v, out)
            else:
                sess.write_record(b, t, k, v)
            recs[b] = (host_bits(k), host_bits(v))
            qs[b] = q
        torch.cuda.synchronize()
        orc.step(t, recs)
        view = sess.view()
        assert view["z0_frame"] == orc.z0_frame and view["raw_frame"] == orc.raw_frame, t
        assert view["sum_frame"] == orc.sum_frame, t
        if view["z0_frame"] != z:
            moves += 1
            say(f"[rope] t={t}: Z0 moved to frame {view['z0_frame']}")
        # every frame: Z0 and the record just written; at the read checks: the whole buffer
        lo = 0 if t == 0 else r * (1 + t % (g.y + 1))
        for b in range(nb):
            kg, vg = sess.kv(b)
            i = orc.index[b]
            if t in attend_at:
                kh, vh = host_bits(kg), host_bits(vg)
                np.testing.assert_array_equal(vh, orc.v[i], err_msg=f"V, t={t}")
                # record rows are turned once by the kernel; Z0 once more per move
                check_turned(kh[r:], orc.k[i][r:], g.head_dim, g.dtype, 0, so.ROPE_CALLER, f"t={t} b={b} all")
            elif lo:
                np.testing.assert_array_equal(host_bits(vg[lo:lo + r]), orc.v[i][lo:lo + r], err_msg=f"V, t={t}")
                check_turned(host_bits(kg[lo:lo + r]), orc.k[i][lo:lo + r], g.head_dim, g.dtype, g.hw, mode,
                             f"t={t} b={b} record")
            check_turned(host_bits(kg[:r]), orc.k[i][:r], g.head_dim, g.dtype, g.hw, mode, f"t={t} b={b} Z0",
                         moves + 1)
        if t in attend_at:
            for b in range(nb):
                sess.attend(b, qs[b], out)
                torch.cuda.synchronize()
                ref = orc.attend(b, host_bits(qs[b]))
                got = out.double().cpu().numpy()
                err = np.abs(got - ref)
                rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
                say(f"   attention t={t} b={b}: max-abs {err.max():.2e} rel-L2 {rel:.2e}")
                assert err.max() <= TOL[g.dtype]["max_abs"] and rel <= TOL[g.dtype]["rel_l2"]
    return moves


@needs_gpu
@pytest.mark.parametrize("mode", list(MODES))
def test_rope_served_rollout_bf16(mode):
    """Served grid, one block, bf16, sink gap 5, frames 0..33 through sf_step."""
    wl = dict(CASES["served_bf16"], rope_mode=mode, sink_gap=5)
    assert run_rollout(wl, range(34), attend_at=(0, 3, 29, 33), use_step=True) == 2


@needs_gpu
@pytest.mark.parametrize("mode", list(MODES))
def test_rope_tiny_f32_separate_calls(mode):
    """fp32 storage, W = 6, gap 5, through sf_evict / sf_write_record / sf_attend."""
    wl = dict(CASES["tiny_f32"], rope_mode=mode, sink_gap=5)
    assert run_rollout(wl, range(21), attend_at=(0, 5, 11, 20), use_step=False) == 3


@needs_gpu
@pytest.mark.parametrize("mode", list(MODES))
def test_rope_head_dim_128_two_blocks(mode):
    """bf16, head_dim 128 (22 temporal planes, level planes 20 and 21), two blocks, gap 3."""
    wl = dict(CASES["hd128_bf16"], rope_mode=mode, sink_gap=3)
    assert run_rollout(wl, range(14), attend_at=(1, 8, 13), use_step=True) >= 3


@needs_gpu
def test_rope_step_equals_separate_calls():
    """sf_step under a rope mode is the write, the query turn and the read, bit for bit."""
    wl = dict(CASES["served_bf16"], rope_mode="add", sink_gap=5)
    a = sf.Session(sf.make_config(**wl))
    b = sf.Session(sf.make_config(**wl))
    oa = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    ob = torch.empty_like(oa)
    for t in range(31):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        a.step(0, t, q, k, v, oa)
        if t >= 1:
            b.evict(t)
        b.write_record(0, t, k, v)
        b.attend(0, q, ob)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), t
    assert torch.equal(a.kv_bytes_view(), b.kv_bytes_view())


@needs_gpu
def test_rope_batched_attend_mixed_modes():
    """One batched sf_attend over sessions with different rope modes and fill levels: each
    session's query is turned by its own current frame."""
    base = dict(CASES["served_bf16"], n_blocks=1)
    plan = [("replace", 2, 11), ("add", 5, 12), ("caller", 3, 13), ("add", 9, 14)]
    sessions, oracles, qs = [], [], []
    for mode, t_last, seed in plan:
        wl = dict(base, rope_mode=mode, seed=seed, sink_gap=0)
        sess = sf.Session(sf.make_config(**wl))
        m = {"replace": so.ROPE_LEVEL_REPLACE, "add": so.ROPE_LEVEL_ADD, "caller": so.ROPE_CALLER}[mode]
        orc = so.MemoryReplay(so.Geometry.from_workload(wl), rope_mode=m)
        out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
        for t in range(t_last + 1):
            q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
            sess.step(0, t, q, k, v, out)
            orc.step(t, {0: (host_bits(k), host_bits(v))})
        sessions.append(sess)
        oracles.append(orc)
        qs.append(q)
        say(f"[rope batched] {mode} at t={t_last}: {orc.n_keys()} keys")
    outs = [torch.empty(sf_inputs.record_shape(base), dtype=torch.float32, device="cuda") for _ in plan]
    sf.sf_attend([s.handle for s in sessions], 0, qs, outs)
    torch.cuda.synchronize()
    for (mode, t_last, _), orc, q, out in zip(plan, oracles, qs, outs):
        ref = orc.attend(0, host_bits(q))
        got = out.double().cpu().numpy()
        err = np.abs(got - ref)
        rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
        say(f"   {mode} t={t_last}: max-abs {err.max():.2e} rel-L2 {rel:.2e}")
        assert err.max() <= TOL["bf16"]["max_abs"] and rel <= TOL["bf16"]["rel_l2"]


@needs_gpu
@pytest.mark.parametrize("mode", list(MODES))
def test_rope_four_pass_rewrites(mode):
    """Three denoising passes and a clean pass per frame, each a write of the same frame id
    (turned by it) and a read, with the sink on; buffers and reads against the oracle."""
    wl = dict(CASES["tiny_f32"], rope_mode=mode, sink_gap=3, w=4)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g, sink_gap=3, rope_mode=MODES[mode])
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    for t in range(14):
        for p in range(4):
            q, k, v = sf_inputs.frame_tensors(wl, p, 0, t, device="cuda")
            sess.step(0, t, q, k, v, out)
            torch.cuda.synchronize()
            if p == 0:
                orc.step(t, {0: (host_bits(k), host_bits(v))})
            else:
                orc.write(0, t, host_bits(k), host_bits(v))
            ref = orc.attend(0, host_bits(q))
            err = float(np.abs(out.double().cpu().numpy() - ref).max())
            assert err <= TOL["f32"]["max_abs"], (t, p, err)
        kg, vg = sess.kv(0)
        np.testing.assert_array_equal(host_bits(vg), orc.v[0], err_msg=f"V t={t}")
        check_turned(host_bits(kg)[g.r:], orc.k[0][g.r:], g.head_dim, g.dtype, 0, so.ROPE_CALLER, f"t={t} records")
    assert sess.view()["z0_frame"] == orc.z0_frame > 0
