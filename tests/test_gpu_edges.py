"""GPU parity at the edges: the largest batch one call takes, batches that need several
launches, and the smallest geometries (one raw token, one summary token, no raw history,
a one-slot window) where reads are shorter than one 64-key tile.

Page: model card "GTA world model: weights and inference code", sections "What a frame
attends to" and "One buffer, no mask".  Same bar as the other parity tests: buffers bit
for bit, attention within max-abs 1e-5 (fp32) or 2e-2 and relative L2 1e-2 (bf16).
"""
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


def replay(wl, session, t_end, use_step=True):
    """A session and its oracle stepped through frames 0..t_end (one block)."""
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    q = None
    for t in range(t_end + 1):
        q, k, v = sf_inputs.frame_tensors(wl, session, 0, t, device="cuda")
        if use_step:
            sess.step(0, t, q, k, v, out)
        else:
            if t >= 1:
                sess.evict(t)
            sess.write_record(0, t, k, v)
        orc.step(t, {0: (host(k), host(v))})
    torch.cuda.synchronize()
    return sess, orc, q


@needs_gpu
@pytest.mark.parametrize("name,wl,n", [
    # bf16 head_dim 64 (stream-K read): the largest batch, four launches of 16 sessions
    ("bf16-64", dict(hw=40, x=8, y=2, w=6, n_heads=2, head_dim=64, n_blocks=1, dtype="bf16", seed=21,
                     v_scale=1.0), 64),
    # bf16 head_dim 128 (split-key read): two launches
    ("bf16-128", dict(hw=33, x=5, y=1, w=4, n_heads=3, head_dim=128, n_blocks=1, dtype="bf16", seed=22,
                      v_scale=1.0), 20),
    # fp32: two launches
    ("f32-64", dict(hw=24, x=4, y=2, w=6, n_heads=1, head_dim=64, n_blocks=1, dtype="f32", seed=23,
                    v_scale=1.0), 18),
])
def test_batches_beyond_one_launch(name, wl, n):
    """n sessions at fill levels 0 .. 11 (cycling) in one sf_attend call."""
    sessions, oracles, qs = [], [], []
    for si in range(n):
        sess, orc, q = replay(wl, si, si % 12, use_step=(si % 2 == 0))
        sessions.append(sess)
        oracles.append(orc)
        qs.append(q)
    outs = [torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda") for _ in range(n)]
    say(f"[batch {name}] {n} sessions")
    sf.attend_batch(sessions, 0, qs, outs)
    torch.cuda.synchronize()
    for si, (sess, orc, q, out) in enumerate(zip(sessions, oracles, qs, outs)):
        check_buffer(sess, orc, 0, f"{name} s{si}")
        ref = orc.attend(0, host(q))
        check_attention(out, ref, wl["dtype"], f"{name} s{si} keys={orc.n_keys()}")
    with pytest.raises(sf.SfError):                       # one more than a call takes
        sf.attend_batch(sessions + sessions[:1], 0, qs + qs[:1], outs + outs[:1])


@needs_gpu
@pytest.mark.parametrize("wl", [
    dict(hw=1, x=1, y=0, w=1, n_heads=1, head_dim=64, n_blocks=2, dtype="bf16", seed=31, v_scale=1.0),
    dict(hw=1, x=1, y=0, w=1, n_heads=3, head_dim=128, n_blocks=1, dtype="bf16", seed=32, v_scale=1.0),
    dict(hw=1, x=1, y=0, w=1, n_heads=2, head_dim=64, n_blocks=1, dtype="f32", seed=33, v_scale=1.0),
    dict(hw=3, x=2, y=3, w=4, n_heads=2, head_dim=64, n_blocks=1, dtype="bf16", seed=34, v_scale=1.0),
], ids=["min-bf16-64", "min-bf16-128", "min-f32", "one-sum-slot"])
def test_smallest_geometries(wl):
    """Records of 2 or 5 rows, windows of one SUM slot: every read is shorter than a tile."""
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    for t in range(12):
        recs = {}
        for b in range(wl["n_blocks"]):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
            recs[b] = (host(k), host(v))
        orc.step(t, recs)
        torch.cuda.synchronize()
        check_tables(sess, orc, f"t={t}")
        b = wl["n_blocks"] - 1
        ref = orc.attend(b, host(q))
        check_attention(out, ref, wl["dtype"], f"t={t} keys={orc.n_keys()}")
        for bb in range(wl["n_blocks"]):
            check_buffer(sess, orc, bb, f"t={t} b{bb}")


@needs_gpu
def test_whole_units_over_stale_scratch():
    """Units one workgroup reads whole, over scratch that holds finite stale partials.

    Record of 128 rows (one query tile), 4 heads of 64: at t = 0 each of the 4 columns is
    two full tiles and one group range, so the stream-K read writes every unit's output
    itself and marks it; the combine must leave those units alone.  From t = 1 on the
    columns are cut into several pieces.  The scratch is filled with 1.0f before the first
    read, so a combine that merged unmarked slots would fold in finite wrong partials."""
    wl = dict(hw=120, x=8, y=2, w=24, n_heads=4, head_dim=64, n_blocks=1, dtype="bf16", seed=35, v_scale=1.0)
    g = so.Geometry.from_workload(wl)
    cfg = sf.make_config(**wl)
    sess = sf.Session(cfg)
    torch.cuda.synchronize()
    kv = sf.sf_kv_bytes(cfg)
    rest = (sess.mem.numel() - kv) // 4 * 4
    assert rest > 0
    sess.mem[kv:kv + rest].view(torch.int32).fill_(0x3F800000)  # 1.0f everywhere in the scratch
    torch.cuda.synchronize()
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    for t in range(6):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        out.fill_(float("nan"))
        sess.step(0, t, q, k, v, out)
        orc.step(t, {0: (host(k), host(v))})
        torch.cuda.synchronize()
        check_tables(sess, orc, f"t={t}")
        ma, rel = check_attention(out, orc.attend(0, host(q)), "bf16", f"t={t} keys={orc.n_keys()}")
        say(f"[whole] t={t} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
