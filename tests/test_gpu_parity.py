"""GPU parity: the HIP path through the C-ABI against the CPU oracle, on the same input bytes.

Buffers and slot tables must match bit for bit; attention outputs within
max-abs 1e-5 (fp32) or 2e-2 (bf16), and for bf16 also a relative L2 error
below 1e-2 (the output's RMS is near sqrt(e/K), so max-abs alone is weak).
Inputs come from sf_inputs (seeded torch.randn on the GPU); the oracle gets
host copies of those bytes.  Page: model card "GTA world model: weights and
inference code", sections "What a frame attends to" and "One buffer, no mask".
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
else:  # collected on a CPU-only machine: every test here is skipped
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

TOL = {"f32": dict(max_abs=1e-5, rel_l2=1e-5), "bf16": dict(max_abs=2e-2, rel_l2=1e-2)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def host(x):
    return sf_inputs.to_host_bytes(x)


def check_attention(got: torch.Tensor, ref: np.ndarray, dtype: str, what: str):
    g = got.detach().double().cpu().numpy()
    err = np.abs(g - ref)
    max_abs = float(err.max()) if err.size else 0.0
    rel = float(np.linalg.norm(g - ref) / max(np.linalg.norm(ref), 1e-300))
    tol = TOL[dtype]
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    assert max_abs <= tol["max_abs"], f"{what}: max-abs {max_abs:.3e} > {tol['max_abs']}"
    assert rel <= tol["rel_l2"], f"{what}: rel-L2 {rel:.3e} > {tol['rel_l2']}"
    return max_abs, rel


def check_buffer(sess, orc: so.MemoryReplay, block: int, what: str):
    k, v = sess.kv(block)
    i = orc.index[block]
    if k.dtype == torch.bfloat16:
        ok = torch.equal(k.view(torch.int16), torch.from_numpy(orc.k[i].view(np.int16)).to(k.device))
        ov = torch.equal(v.view(torch.int16), torch.from_numpy(orc.v[i].view(np.int16)).to(v.device))
    else:
        ok = torch.equal(k.view(torch.int32), torch.from_numpy(orc.k[i].view(np.int32)).to(k.device))
        ov = torch.equal(v.view(torch.int32), torch.from_numpy(orc.v[i].view(np.int32)).to(v.device))
    assert ok and ov, f"{what}: buffer bytes differ from the oracle (K ok={ok}, V ok={ov})"


def check_tables(sess, orc: so.MemoryReplay, what: str):
    v = sess.view()
    assert v["raw_frame"] == orc.raw_frame, what
    assert v["sum_frame"] == orc.sum_frame, what
    assert v["segments"] == orc.readable_segments(), what
    assert v["n_keys"] == orc.n_keys(), what


def new_session(wl):
    return sf.Session(sf.make_config(**wl))


def out_like(wl):
    return torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")


@needs_gpu
def test_tiny_f32_rollout_with_rewrites():
    """Tiny fp32 workload, t = 0..11 plus a rewrite at t = 4 and t = 9: every step checked in full."""
    wl = sf_inputs.WORKLOADS["tiny"]
    g = so.Geometry.from_workload(wl)
    sess = new_session(wl)
    orc = so.MemoryReplay(g)
    out = out_like(wl)
    for t in wl["frames"]:
        say(f"[tiny] t={t}")
        if t in (4, 9):  # a first write that the clean pass overwrites
            q0, k0, v0 = sf_inputs.frame_tensors(wl, 1, 0, t, device="cuda")
            sess.step(0, t, q0, k0, v0, out)
            orc.step(t, {0: (host(k0), host(v0))})
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        if t in (4, 9):
            orc.write(0, t, host(k), host(v))  # the rewrite: no second eviction
        else:
            orc.step(t, {0: (host(k), host(v))})
        torch.cuda.synchronize()
        check_tables(sess, orc, f"tiny t={t}")
        check_buffer(sess, orc, 0, f"tiny t={t}")
        check_attention(out, orc.attend(0, host(q)), "f32", f"tiny t={t}")


@needs_gpu
def test_served_single_block_fill_levels():
    """Served shape, one block, frames 0..31: buffer every frame, attention at each fill level."""
    wl = sf_inputs.WORKLOADS["served1"]
    g = so.Geometry.from_workload(wl)
    sess = new_session(wl)
    orc = so.MemoryReplay(g)
    out = out_like(wl)
    check_at = {0, 1, 2, 3, 4, 10, 23, 24, 25, 31}
    for t in wl["frames"]:
        say(f"[served1] t={t}")
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        orc.step(t, {0: (host(k), host(v))})
        torch.cuda.synchronize()
        check_tables(sess, orc, f"served1 t={t}")
        check_buffer(sess, orc, 0, f"served1 t={t}")
        if t in check_at:
            ma, rel = check_attention(out, orc.attend(0, host(q)), "bf16", f"served1 t={t}")
            say(f"   attention keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert orc.n_keys() == 6528


@needs_gpu
def test_served_repeat_attend_is_deterministic():
    """Two attends of the same state give identical bits (no atomics in the reduction);
    the step that wrote the last record gives the same attention within tolerance."""
    wl = sf_inputs.WORKLOADS["served1"]
    sess = new_session(wl)
    out = out_like(wl)
    for t in range(27):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
    out2 = out_like(wl)
    out3 = out_like(wl)
    sess.attend(0, q, out2)
    sess.attend(0, q, out3)
    torch.cuda.synchronize()
    assert torch.equal(out2, out3)
    # sf_step reads the new record's keys last (from its source), sf_attend in buffer
    # order: the same softmax over the same keys, summed in another order.
    check_attention(out, out2.double().cpu().numpy(), "bf16", "step vs attend")


@needs_gpu
def test_batched_sessions_ragged():
    """Eight sessions at fill levels 0,1,2,3,10,23,24,31; one batched attend per block, 28 blocks."""
    wl = sf_inputs.WORKLOADS["batched"]
    g = so.Geometry.from_workload(wl)
    levels = wl["frames"]
    nb = wl["n_blocks"]
    check_blocks = (0, 13, 27)
    sessions, oracles = [], []
    for si, t_end in enumerate(levels):
        say(f"[batched] replay session {si} to t={t_end}")
        sess = new_session(wl)
        orc = so.MemoryReplay(g, blocks=check_blocks)
        for t in range(t_end + 1):
            recs = {}
            if t >= 1:
                sess.evict(t)  # explicit eviction, then the writes (sf_step is used elsewhere)
            for b in range(nb):
                _, k, v = sf_inputs.frame_tensors(wl, si, b, t, device="cuda")
                sess.write_record(b, t, k, v)
                if b in check_blocks:
                    recs[b] = (host(k), host(v))
            orc.step(t, recs)
        torch.cuda.synchronize()
        check_tables(sess, orc, f"batched session {si}")
        sessions.append(sess)
        oracles.append(orc)
    outs = [out_like(wl) for _ in levels]
    for b in range(nb):
        qs = [sf_inputs.frame_tensors(wl, si, b, levels[si], device="cuda")[0] for si in range(len(levels))]
        say(f"[batched] attend block {b}")
        sf.attend_batch(sessions, b, qs, outs)
        if b not in check_blocks:
            continue
        torch.cuda.synchronize()
        for si, (sess, orc) in enumerate(zip(sessions, oracles)):
            check_buffer(sess, orc, b, f"batched s{si} b{b}")
            rows = None if b != 13 else np.arange(0, g.r, 16)
            ref = orc.attend(b, host(qs[si]), rows=rows)
            got = outs[si] if rows is None else outs[si][torch.from_numpy(rows).cuda()]
            ma, rel = check_attention(got, ref, "bf16", f"batched s{si} t={levels[si]} b{b}")
            say(f"   s{si} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")


def _replay(wl, si, t_end, rows_for_oracle=True):
    """A one-block session replayed to frame t_end (explicit eviction, then the write), with
    its oracle."""
    g = so.Geometry.from_workload(wl)
    sess = new_session(wl)
    orc = so.MemoryReplay(g)
    for t in range(t_end + 1):
        if t >= 1:
            sess.evict(t)
        _, k, v = sf_inputs.frame_tensors(wl, si, 0, t, device="cuda")
        sess.write_record(0, t, k, v)
        orc.step(t, {0: (host(k), host(v))})
    torch.cuda.synchronize()
    check_tables(sess, orc, f"mixed session {si}")
    return g, sess, orc


@needs_gpu
@pytest.mark.timeout(600)
def test_batched_mixed_geometries():
    """One batched read over sessions whose records differ in size: 1, 3, 9 and 13 query tiles
    (workgroup groups of 13 members, most idle for the smaller sessions), key counts with and
    without a tail; then one session of 65 query tiles, more than one XCD's workgroups, so a
    group member takes two query tiles of a column.  Every session against the oracle."""
    base = dict(y=2, w=6, n_heads=16, head_dim=64, n_blocks=1, dtype="bf16", v_scale=1.0)
    shapes = [(100, 28, 3), (280, 20, 5), (1008, 96, 8), (1500, 100, 6)]  # (hw, x, frame)
    wls, sessions, oracles, geos = [], [], [], []
    for si, (hw, x, t_end) in enumerate(shapes):
        wl = dict(base, hw=hw, x=x, frames=list(range(t_end + 1)), seed=40 + si)
        say(f"[mixed] replay session {si}: R={hw + x}, to t={t_end}")
        g, sess, orc = _replay(wl, si, t_end)
        wls.append(wl)
        sessions.append(sess)
        oracles.append(orc)
        geos.append(g)
    qs = [sf_inputs.frame_tensors(wl, si, 0, wl["frames"][-1], device="cuda")[0] for si, wl in enumerate(wls)]
    outs = [out_like(wl) for wl in wls]
    say("[mixed] batched attend")
    sf.attend_batch(sessions, 0, qs, outs)
    torch.cuda.synchronize()
    for si, (orc, g) in enumerate(zip(oracles, geos)):
        rows = None if g.r <= 1104 else np.unique(np.concatenate([np.arange(0, g.r, 7), np.arange(g.r - 70, g.r)]))
        ref = orc.attend(0, host(qs[si]), rows=rows)
        got = outs[si] if rows is None else outs[si][torch.from_numpy(rows).cuda()]
        ma, rel = check_attention(got, ref, "bf16", f"mixed s{si} R={g.r} keys={orc.n_keys()}")
        say(f"   s{si} R={g.r} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")

    # 8320 rows = 65 query tiles; Y = 1, W = 2: frame 1 reads 16,640 keys
    wl = dict(base, hw=8192, x=128, y=1, w=2, frames=[0, 1], seed=47)
    say("[mixed] replay the 65-tile session")
    g, sess, orc = _replay(wl, 0, 1)
    q = sf_inputs.frame_tensors(wl, 0, 0, 1, device="cuda")[0]
    out = out_like(wl)
    sess.attend(0, q, out)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.arange(0, g.r, 61), np.arange(8192 - 8, g.r, 3)]))
    ref = orc.attend(0, host(q), rows=rows)
    ma, rel = check_attention(out[torch.from_numpy(rows).cuda()], ref, "bf16", "65-tile session")
    say(f"   R={g.r} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")


@needs_gpu
@pytest.mark.timeout(900)
def test_rollout_28_blocks_64_frames():
    """Served rollout through 28 blocks, frames 0..63: every block's buffer and the slot tables
    every frame; attention in full at blocks 0 and 27 on fill-level frames, sampled elsewhere."""
    wl = sf_inputs.WORKLOADS["rollout"]
    g = so.Geometry.from_workload(wl)
    nb = wl["n_blocks"]
    sess = new_session(wl)
    orc = so.MemoryReplay(g)
    out = out_like(wl)
    full_at = {0, 1, 2, 3, 4, 24, 25, 31, 63}
    sample_rows = np.unique(np.concatenate([np.arange(0, g.r, 16), np.arange(g.hw, g.r, 4)]))
    for t in wl["frames"]:
        say(f"[rollout] t={t}")
        recs = {}
        for b in range(nb):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
            recs[b] = (host(k), host(v))
            if (b in (0, 27) and t in full_at) or b == t % nb:
                torch.cuda.synchronize()
                rows = None if (b in (0, 27) and t in full_at) else sample_rows
                tmp = _oracle_after(orc, t, b, *recs[b])
                ref = tmp.attend(b, host(q), rows=rows)
                got = out if rows is None else out[torch.from_numpy(rows).cuda()]
                ma, rel = check_attention(got, ref, "bf16", f"rollout t={t} b{b}")
                if rows is None:
                    say(f"   b{b} keys={tmp.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
        orc.step(t, recs)
        torch.cuda.synchronize()
        check_tables(sess, orc, f"rollout t={t}")
        for b in range(nb):
            check_buffer(sess, orc, b, f"rollout t={t} b{b}")


def _oracle_after(orc: so.MemoryReplay, t: int, block: int, k, v) -> so.MemoryReplay:
    """The oracle's state of one block once frame t's record (k, v) is written to it.

    `orc` holds every checked block at frame t-1; this copies only `block`."""
    tmp = so.MemoryReplay.__new__(so.MemoryReplay)
    tmp.__dict__.update(orc.__dict__)     # settings and scalar state; the tables and rows are copied below
    tmp.blocks = [block]
    tmp.index = {block: 0}
    i = orc.index[block]
    tmp.k = orc.k[i:i + 1].copy()
    tmp.v = orc.v[i:i + 1].copy()
    tmp.raw_frame = list(orc.raw_frame)
    tmp.sum_frame = list(orc.sum_frame)
    tmp.step(t, {block: (k, v)})
    return tmp


@needs_gpu
@pytest.mark.timeout(1200)
def test_long_horizon_sampled():
    """Long-horizon workload (24 heads of 128, 46,688 keys): 28 blocks, 128 frames.

    Blocks 0, 9, 18 and 27 get their own seeded inputs and are checked against the
    oracle: every frame, the rows the frame changed (the record's rows and, from the
    first eviction on, the SUM slot it filled); the whole buffers at three frames;
    attention on sampled rows at seven frames.  The other blocks reuse block 0's inputs,
    so their buffers must equal block 0's bit for bit every frame."""
    wl = sf_inputs.WORKLOADS["long"]
    g = so.Geometry.from_workload(wl)
    nb = wl["n_blocks"]
    own = (0, 9, 18, 27)
    sess = new_session(wl)
    orc = so.MemoryReplay(g, blocks=own)
    out = out_like(wl)
    att_at = {0, 1, 5, 6, 96, 97, 127}
    att_blocks = {0, 27}
    full_buf_at = {6, 97, 127}
    rows = np.unique(np.concatenate([np.arange(0, g.r, 128), np.arange(g.hw, g.r, 8), [g.r - 1]]))
    evictions = 0
    for t in wl["frames"]:
        say(f"[long] t={t}")
        inputs = {b: sf_inputs.frame_tensors(wl, 0, b, t, device="cuda") for b in own}
        for b in range(nb):
            q, k, v = inputs[b if b in own else 0]
            sess.step(b, t, q, k, v, out)
            if b in att_blocks and t in att_at:
                torch.cuda.synchronize()
                tmp = _oracle_after(orc, t, b, host(k), host(v))
                ref = tmp.attend(b, host(q), rows=rows)
                ma, rel = check_attention(out[torch.from_numpy(rows).cuda()], ref, "bf16", f"long t={t} b{b}")
                say(f"   b{b} keys={tmp.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
        moved = orc.step(t, {b: (host(inputs[b][1]), host(inputs[b][2])) for b in own})
        torch.cuda.synchronize()
        check_tables(sess, orc, f"long t={t}")
        k0, v0 = sess.kv(0)
        for b in range(1, nb):
            if b in own:
                continue
            kb, vb = sess.kv(b)
            assert torch.equal(kb.view(torch.int16), k0.view(torch.int16)) and \
                torch.equal(vb.view(torch.int16), v0.view(torch.int16)), f"long t={t}: block {b} != block 0"
        evictions += moved is not None
        if t in full_buf_at:
            for b in own:
                check_buffer(sess, orc, b, f"long t={t} b{b}")
            continue
        # rows this frame changed: the record's rows and the SUM slot its eviction filled
        changed = [(0, g.r) if t == 0 else g.raw_rows(t % g.n_raw)]
        if moved is not None:
            changed.append(g.sum_rows(moved[1]))
        for b in own:
            kk, vv = sess.kv(b)
            i = orc.index[b]
            for lo, hi in changed:
                for name, gpu_t, ora in (("K", kk, orc.k), ("V", vv, orc.v)):
                    assert torch.equal(gpu_t[lo:hi].view(torch.int16),
                                       torch.from_numpy(ora[i, lo:hi].view(np.int16)).cuda()), \
                        f"long t={t} b{b} {name} rows [{lo}, {hi})"
    assert orc.n_keys() == 46688
    assert evictions == 122  # frames Y+2 = 6 .. 127 move a summary
