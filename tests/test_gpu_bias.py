"""GPU parity of the recency bias on summary keys.

Page: model card "GTA world model: weights and inference code", sections "Files" (an
optional recency bias on summary keys) and "Credits".  A session configured with a bias
adds its table's entry for a summary row's age to that key's scaled score, per head.  The
library reads such sessions through the split-key kernel (bf16) or the fp32 kernel, with
the per-row biases rebuilt once per frame; the oracle adds the same table in fp64 after
finding each row's frame in its slot tables.  Same bar as the other parity tests: buffers
and slot tables bit for bit, attention within max-abs 1e-5 (fp32) or 2e-2 and relative L2
1e-2 (bf16).
"""
import numpy as np
import pytest
import torch

import sf_inputs
from oracle import sf_oracle as so
from test_gpu_parity import check_attention, check_buffer, check_tables, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")

CASES = {
    # fp32 kernel, every frame checked in full, rewrites at t = 4 and 9
    "tiny_f32": dict(sf_inputs.WORKLOADS["tiny"], frames=list(range(14)), check=set(range(14))),
    # split-key kernel at head_dim 64, the served shape (6,528 keys once full)
    "served_bf16": dict(sf_inputs.WORKLOADS["served1"], frames=list(range(32)),
                        check={0, 1, 2, 3, 4, 10, 24, 25, 31}),
    # split-key kernel at head_dim 128, two blocks
    "hd128_bf16": dict(hw=40, x=8, y=1, w=5, n_heads=3, head_dim=128, n_blocks=2, dtype="bf16", seed=9,
                       v_scale=1.0, frames=list(range(12)), check=set(range(12))),
    # fp32 kernel at head_dim 128
    "hd128_f32": dict(hw=33, x=5, y=2, w=6, n_heads=2, head_dim=128, n_blocks=1, dtype="f32", seed=12,
                      v_scale=1.0, frames=list(range(12)), check=set(range(12))),
}


def out_like(wl):
    return torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")


def table(wl, session, version, scale=2.0):
    return sf_inputs.bias_table(wl, session, version, scale, device="cuda").contiguous()


@needs_gpu
@pytest.mark.parametrize("case", list(CASES))
def test_bias_rollout_matches_oracle(case):
    """Frames 0..n with the table set at t = 0 and replaced at t = 6 (a new frame) and at a
    rewrite; the step path writes first and reads through the bias kernel."""
    wl = dict(CASES[case], recency_bias=True)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g, blocks=sorted({0, wl["n_blocks"] - 1}))
    out = out_like(wl)
    tab = table(wl, 0, 0)
    sess.set_recency_bias(tab)
    orc.set_recency_bias(tab.cpu().numpy())
    for t in wl["frames"]:
        if t == 6:
            tab = table(wl, 0, 1)
            sess.set_recency_bias(tab)
            orc.set_recency_bias(tab.cpu().numpy())
        recs = {}
        for b in range(wl["n_blocks"]):
            if t in (4, 9) and b == 0:      # a first pass that the clean pass rewrites
                q0, k0, v0 = sf_inputs.frame_tensors(wl, 1, b, t, device="cuda")
                sess.step(b, t, q0, k0, v0, out)
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            if t == 9 and b == 0:           # the table changes between the passes of a frame
                tab = table(wl, 0, 2)
                sess.set_recency_bias(tab)
            sess.step(b, t, q, k, v, out)
            if b in orc.index:
                recs[b] = (host(k), host(v))
            if b == 0:
                q_first, out_first = q, out.clone()
        orc.step(t, recs)
        if t == 9:
            orc.set_recency_bias(tab.cpu().numpy())
        torch.cuda.synchronize()
        check_tables(sess, orc, f"{case} t={t}")
        for b in orc.blocks:
            check_buffer(sess, orc, b, f"{case} t={t} b{b}")
        if t in wl["check"]:
            b = wl["n_blocks"] - 1
            ma, rel = check_attention(out, orc.attend(b, host(q)), wl["dtype"], f"{case} t={t} b{b}")
            say(f"[bias {case}] t={t} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
            if wl["n_blocks"] > 1:
                check_attention(out_first, orc.attend(0, host(q_first)), wl["dtype"], f"{case} t={t} b0")


@needs_gpu
@pytest.mark.parametrize("fill", [-1e4, float("-inf")])
def test_bias_that_drops_every_summary(fill):
    """A table of -1e4 (or -inf, which the library raises to -1e30) at every age: the read
    sees the start image and the raw rows only.  Exercises the split-key kernel's reference
    moving past tiles whose every key carries the floor."""
    wl = dict(CASES["served_bf16"], recency_bias=True)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    tab = torch.full((wl["n_heads"], wl["w"] + 1), fill, dtype=torch.float32, device="cuda")
    sess.set_recency_bias(tab)
    orc.set_recency_bias(tab.cpu().numpy().astype(np.float64))
    out = out_like(wl)
    for t in range(27):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        orc.step(t, {0: (host(k), host(v))})
        if t in (0, 3, 26):
            torch.cuda.synchronize()
            ma, rel = check_attention(out, orc.attend(0, host(q)), "bf16", f"fill={fill} t={t}")
            say(f"[bias drop {fill}] t={t} max_abs={ma:.2e} rel_l2={rel:.2e}")


@needs_gpu
def test_batch_mixes_sessions_with_and_without_bias():
    """One sf_attend over six sessions at different fill levels, half of them with a bias: the
    batch splits by read path (stream-K for the others) and each result matches its oracle."""
    base = dict(hw=100, x=12, y=2, w=8, n_heads=4, head_dim=64, n_blocks=1, dtype="bf16", seed=31, v_scale=1.0)
    g = so.Geometry.from_workload(base)
    levels = [0, 3, 5, 9, 12, 14]
    sessions, oracles, qs = [], [], []
    for si, t_end in enumerate(levels):
        wl = dict(base, recency_bias=(si % 2 == 0))
        sess = sf.Session(sf.make_config(**wl))
        orc = so.MemoryReplay(g)
        if wl["recency_bias"]:
            tab = table(base, si, 0)
            sess.set_recency_bias(tab)
            orc.set_recency_bias(tab.cpu().numpy())
        for t in range(t_end + 1):
            q, k, v = sf_inputs.frame_tensors(base, si, 0, t, device="cuda")
            if t >= 1:
                sess.evict(t)
            sess.write_record(0, t, k, v)
            orc.step(t, {0: (host(k), host(v))})
        sessions.append(sess)
        oracles.append(orc)
        qs.append(q)
    outs = [out_like(base) for _ in levels]
    say(f"[bias batch] {len(levels)} sessions")
    sf.attend_batch(sessions, 0, qs, outs)
    torch.cuda.synchronize()
    for si, (orc, q, out) in enumerate(zip(oracles, qs, outs)):
        check_buffer(sessions[si], orc, 0, f"s{si}")
        check_attention(out, orc.attend(0, host(q)), "bf16", f"s{si} bias={si % 2 == 0} keys={orc.n_keys()}")


@needs_gpu
@pytest.mark.parametrize("mode", ["replace", "add"])
def test_bias_with_rope_mode_and_sink(mode):
    """The bias together with the library's temporal band and the streaming sink."""
    wl = dict(hw=64, x=16, y=2, w=10, n_heads=2, head_dim=64, n_blocks=2, dtype="bf16", seed=41, v_scale=1.0,
              recency_bias=True, rope_mode=mode, sink_gap=5)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g, sink_gap=5, rope_mode=so.ROPE_LEVEL_REPLACE if mode == "replace" else so.ROPE_LEVEL_ADD)
    tab = table(wl, 0, 0)
    sess.set_recency_bias(tab)
    orc.set_recency_bias(tab.cpu().numpy())
    out = out_like(wl)
    for t in range(24):
        recs = {}
        for b in range(wl["n_blocks"]):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
            recs[b] = (host(k), host(v))
        orc.step(t, recs)
        torch.cuda.synchronize()
        check_tables(sess, orc, f"{mode} t={t}")
        check_attention(out, orc.attend(wl["n_blocks"] - 1, host(q)), "bf16", f"{mode} t={t}")


@needs_gpu
def test_step_equals_write_then_attend_and_repeats_exactly():
    """sf_step and sf_write_record + sf_attend give the same bytes; a repeated read too."""
    wl = dict(CASES["hd128_bf16"], recency_bias=True, n_blocks=1)
    a = sf.Session(sf.make_config(**wl))
    b = sf.Session(sf.make_config(**wl))
    tab = table(wl, 0, 0)
    a.set_recency_bias(tab)
    b.set_recency_bias(tab)
    oa, ob, oc = out_like(wl), out_like(wl), out_like(wl)
    for t in range(10):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        a.step(0, t, q, k, v, oa)
        if t >= 1:
            b.evict(t)
        b.write_record(0, t, k, v)
        b.attend(0, q, ob)
        b.attend(0, q, oc)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob) and torch.equal(ob, oc), f"t={t}"


@needs_gpu
def test_bias_calls_and_launch_counts():
    """Error rules on a real handle, and one table copy per set plus one row rebuild per frame."""
    wl = dict(CASES["tiny_f32"], recency_bias=True)
    plain = sf.Session(sf.make_config(**CASES["tiny_f32"]))
    with pytest.raises(sf.SfError) as ei:
        plain.set_recency_bias(table(wl, 0, 0))
    assert ei.value.status == sf.SF_E_UNSUPPORTED
    sess = sf.Session(sf.make_config(**wl))
    tab = table(wl, 0, 0)
    for bad in (0, tab.data_ptr() + 2):
        with pytest.raises(sf.SfError) as ei:
            sf.sf_set_recency_bias(sess.handle, bad)
        assert ei.value.status == sf.SF_E_ARG
    with pytest.raises(sf.SfError):
        sess.set_recency_bias(tab[:, :-1].contiguous())
    sf.sf_profile_enable(sess.handle, True)
    sess.set_recency_bias(tab)
    out = out_like(wl)
    for t in range(5):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        sess.attend(0, q, out)              # same frame: no rebuild
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["bias"][1] == 1 + 5, times["bias"]
    assert times["attend"][1] == 10
    sf.sf_profile_enable(sess.handle, False)


@needs_gpu
@pytest.mark.timeout(900)
def test_bias_long_horizon_sampled():
    """The long-horizon shape (24 heads of 128, 46,688 keys, SUM ages up to W = 96), one
    block, with a bias: slot tables every frame, the whole buffer at three frames, attention
    on sampled query rows as the window fills and once it is full."""
    wl = dict(sf_inputs.WORKLOADS["long"], n_blocks=1, recency_bias=True)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    tab = table(wl, 0, 0)
    sess.set_recency_bias(tab)
    orc.set_recency_bias(tab.cpu().numpy())
    out = out_like(wl)
    rows = np.unique(np.concatenate([np.arange(0, g.r, 256), np.arange(g.hw, g.r, 16), [g.r - 1]]))
    for t in range(101):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        orc.step(t, {0: (host(k), host(v))})
        torch.cuda.synchronize()
        check_tables(sess, orc, f"long t={t}")
        if t in (6, 97, 100):
            check_buffer(sess, orc, 0, f"long t={t}")
        if t in (0, 5, 96, 97, 100):
            ref = orc.attend(0, host(q), rows=rows)
            ma, rel = check_attention(out[torch.from_numpy(rows).cuda()], ref, "bf16", f"long t={t}")
            say(f"[bias long] t={t} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert orc.n_keys() == 46688


@needs_gpu
def test_bias_batch_beyond_one_launch():
    """20 sessions in one sf_attend: 18 with a bias (two split-key launches of at most 16)
    and 2 without (the stream-K read), at fill levels 0 .. 11."""
    base = dict(hw=40, x=8, y=2, w=6, n_heads=2, head_dim=64, n_blocks=1, dtype="bf16", seed=51, v_scale=1.0)
    g = so.Geometry.from_workload(base)
    sessions, oracles, qs = [], [], []
    for si in range(20):
        biased = si not in (7, 13)
        sess = sf.Session(sf.make_config(**dict(base, recency_bias=biased)))
        orc = so.MemoryReplay(g)
        if biased:
            tab = table(base, si, 0)
            sess.set_recency_bias(tab)
            orc.set_recency_bias(tab.cpu().numpy())
        for t in range(si % 12 + 1):
            q, k, v = sf_inputs.frame_tensors(base, si, 0, t, device="cuda")
            sess.step(0, t, q, k, v, out_like(base))
            orc.step(t, {0: (host(k), host(v))})
        sessions.append(sess)
        oracles.append(orc)
        qs.append(q)
    outs = [out_like(base) for _ in sessions]
    say("[bias batch 20]")
    sf.attend_batch(sessions, 0, qs, outs)
    torch.cuda.synchronize()
    for si, (orc, q, out) in enumerate(zip(oracles, qs, outs)):
        check_attention(out, orc.attend(0, host(q)), "bf16", f"s{si} keys={orc.n_keys()}")
