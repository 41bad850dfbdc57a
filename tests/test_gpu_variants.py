"""GPU parity of the served variants: the server's default window (W = 16), the four-pass
frame loop, the zero-copy record write and a session moved between handles.

Page: model card "GTA world model: weights and inference code": the [buffer] parameter
table (W = 24 trained, 16 served by default) and the "Sampling" item of "The rest of
the model" (three denoising passes and a clean pass that rewrites the frame's entry).
Buffers must match the oracle bit for bit; attention within max-abs 2e-2 and relative
L2 1e-2 (bf16) or 1e-5 (fp32).
"""
import sys

import numpy as np
import pytest
import torch

import sf_inputs
from oracle import sf_oracle as so

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")
TOL = {"f32": dict(max_abs=1e-5, rel_l2=1e-5), "bf16": dict(max_abs=2e-2, rel_l2=1e-2)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(x):
    return sf_inputs.to_host_bytes(x)


def check_attention(got, ref, dtype, what):
    g = got.double().cpu().numpy()
    err = np.abs(g - ref)
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    assert np.isfinite(g).all(), what
    assert err.max() <= TOL[dtype]["max_abs"] and rel <= TOL[dtype]["rel_l2"], (what, float(err.max()), rel)
    return float(err.max()), rel


def check_buffer(sess, orc, block, what):
    k, v = sess.kv(block)
    i = orc.index[block]
    np.testing.assert_array_equal(host(k), orc.k[i], err_msg=f"K {what}")
    np.testing.assert_array_equal(host(v), orc.v[i], err_msg=f"V {what}")


@needs_gpu
def test_served16_rollout():
    """W = 16 on the served grid, two blocks, frames 0..39 (5760 keys once full)."""
    wl = sf_inputs.WORKLOADS["served16"]
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    for t in wl["frames"]:
        recs = {}
        for b in range(wl["n_blocks"]):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
            recs[b] = (host(k), host(v))
            if t in (0, 17, 18, 39) and b == 1:
                torch.cuda.synchronize()
                orc_b = so.MemoryReplay(g)  # the attention sees block 1 after its write
                orc_b.k, orc_b.v = orc.k.copy(), orc.v.copy()
                orc_b.raw_frame, orc_b.sum_frame, orc_b.t = list(orc.raw_frame), list(orc.sum_frame), orc.t
                orc_b.step(t, {1: recs[1]})
                ma, rel = check_attention(out, orc_b.attend(1, host(q)), "bf16", f"W=16 t={t}")
                say(f"[served16] t={t} keys={orc_b.n_keys()} max-abs {ma:.2e} rel-L2 {rel:.2e}")
        orc.step(t, recs)
        torch.cuda.synchronize()
        for b in range(wl["n_blocks"]):
            check_buffer(sess, orc, b, f"W=16 t={t} b{b}")
    assert orc.n_keys() == 5760


@needs_gpu
def test_four_pass_frames():
    """Each frame: three denoising passes and a clean pass through sf_step (the first
    advances and evicts, the others rewrite); one eviction per frame; every pass's read
    is checked."""
    wl = dict(sf_inputs.WORKLOADS["served1"])
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    sf.sf_profile_enable(sess.handle, True)
    frames = range(0, 31)
    for t in frames:
        for p in range(4):                      # session id = pass: a different draw per pass
            q, k, v = sf_inputs.frame_tensors(wl, p, 0, t, device="cuda")
            sess.step(0, t, q, k, v, out)
            orc.step(t, {0: (host(k), host(v))}) if p == 0 else orc.write(0, t, host(k), host(v))
            if t in (0, 3, 30):
                torch.cuda.synchronize()
                ma, rel = check_attention(out, orc.attend(0, host(q)), "bf16", f"t={t} pass {p}")
                say(f"[4-pass] t={t} pass {p} max-abs {ma:.2e} rel-L2 {rel:.2e}")
        torch.cuda.synchronize()
        check_buffer(sess, orc, 0, f"t={t}")
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["evict"][1] == sum(1 for t in frames if t >= g.y + 2)   # one per frame that moves one
    assert times["attend"][1] == 4 * len(frames)


@needs_gpu
@pytest.mark.parametrize("name", ["tiny", "served1"])
def test_zero_copy_write(name):
    """Records written straight into the rows sf_record_slot gives, then committed."""
    wl = sf_inputs.WORKLOADS[name]
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    for t in range(min(len(wl["frames"]), 30)):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        if t >= 1:
            sess.evict(t)
        kd, vd = sess.record_slot(0, t)
        kd.copy_(k)                              # stands for a projection writing in place
        vd.copy_(v)
        sess.commit_record(0, t)
        sess.attend(0, q, out)
        orc.step(t, {0: (host(k), host(v))})
        torch.cuda.synchronize()
        check_buffer(sess, orc, 0, f"{name} t={t}")
        if t % 7 == 0:
            check_attention(out, orc.attend(0, host(q)), g.dtype, f"{name} t={t}")


@needs_gpu
def test_session_moves_between_handles():
    """Export the host state, copy the device bytes, import into a new handle: both sessions
    then produce identical reads and buffers (and match the oracle)."""
    wl = dict(sf_inputs.WORKLOADS["served1"], n_blocks=2, sink_gap=5)
    g = so.Geometry.from_workload(wl)
    cfg = sf.make_config(**wl)
    a = sf.Session(cfg)
    orc = so.MemoryReplay(g, sink_gap=5)
    out_a = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    out_b = torch.empty_like(out_a)
    for t in range(27):
        recs = {}
        for blk in range(2):
            q, k, v = sf_inputs.frame_tensors(wl, 0, blk, t, device="cuda")
            a.step(blk, t, q, k, v, out_a)
            recs[blk] = (host(k), host(v))
        orc.step(t, recs)
    torch.cuda.synchronize()
    b = sf.Session(cfg)
    b.mem.copy_(a.mem)                           # the device bytes are the caller's to move
    b.import_state(a.export_state())
    assert b.view() == a.view()
    for t in range(27, 36):
        recs = {}
        for blk in range(2):
            q, k, v = sf_inputs.frame_tensors(wl, 0, blk, t, device="cuda")
            a.step(blk, t, q, k, v, out_a)
            b.step(blk, t, q, k, v, out_b)
            recs[blk] = (host(k), host(v))
            torch.cuda.synchronize()
            assert torch.equal(out_a, out_b), (t, blk)
        orc.step(t, recs)
        assert b.view() == a.view() and b.view()["z0_frame"] == orc.z0_frame
    torch.cuda.synchronize()
    for blk in range(2):
        ka, va = a.kv(blk)
        kb, vb = b.kv(blk)
        assert torch.equal(ka, kb) and torch.equal(va, vb)
    q_last = sf_inputs.frame_tensors(wl, 0, 1, 35, device="cuda")[0]
    check_attention(out_b, orc.attend(1, host(q_last)), "bf16", "moved session, last read")
