"""The allocation-free read, sf_attend_static_scratch, against sf_attend through the C-ABI.

Both entry points run the same kernels on the same inputs; the static one takes its
scratch (the split reads' partial results, a rope-mode session's turned query) from the
library's static device array instead of the sessions' memory, so the outputs must be
identical bit for bit.  Two calls in a row, the second with a smaller input (the array
then holds the first call's larger layout), on each read path that uses scratch: the
head_dim-64 stream-K read, the split-key read (a session with a recency bias, under a rope
mode, and head_dim 128), plus a batch whose scratch does not fit, which is refused before
anything is enqueued.
"""
import sys

import numpy as np
import pytest
import torch

import sf_inputs

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:  # collected on a CPU-only machine: every test here is skipped
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def replayed(wl, t_end, session=0, **cfg):
    """A session stepped through frames 0..t_end with writes and evictions only, and the
    query of frame t_end for block 0."""
    sess = sf.Session(sf.make_config(**dict(wl, **cfg)))
    for t in range(t_end + 1):
        if t >= 1:
            sess.evict(t)
        for b in range(wl["n_blocks"]):
            _, k, v = sf_inputs.frame_tensors(wl, session, b, t, device="cuda")
            sess.write_record(b, t, k, v)
    q = sf_inputs.frame_tensors(wl, session, 0, t_end, device="cuda")[0]
    return sess, q


def both_reads(sessions, qs, what, scale=0.0):
    """sf_attend, then sf_attend_static_scratch on the same inputs; outputs compared."""
    shape = sf_inputs.record_shape({"hw": sessions[0].cfg.hw, "x": sessions[0].cfg.x,
                                    "n_heads": sessions[0].cfg.n_heads, "head_dim": sessions[0].cfg.head_dim})
    ref = [torch.full(shape, float("nan"), dtype=torch.float32, device="cuda") for _ in sessions]
    got = [torch.full(shape, float("nan"), dtype=torch.float32, device="cuda") for _ in sessions]
    handles = [s.handle for s in sessions]
    say(f"[static scratch] {what}: sf_attend")
    sf.sf_attend(handles, 0, qs, ref, scale)
    torch.cuda.synchronize()
    say(f"[static scratch] {what}: sf_attend_static_scratch")
    sf.sf_attend_static_scratch(handles, 0, qs, got, scale)
    torch.cuda.synchronize()
    for i, (r, g) in enumerate(zip(ref, got)):
        assert torch.isfinite(r).all(), f"{what} s{i}: sf_attend output not finite"
        assert torch.equal(r, g), f"{what} s{i}: outputs differ, max {float((r - g).abs().max()):.3e}"


SERVED = sf_inputs.WORKLOADS["served1"]
SMALL = dict(hw=500, x=60, y=2, w=8, n_heads=4, head_dim=64, n_blocks=1, dtype="bf16", seed=21, v_scale=1.0)
SMALL128 = dict(SMALL, head_dim=128, seed=22)


@needs_gpu
def test_static_scratch_stream_k_two_calls():
    """Served shape at frame 31 (6,528 keys, ~29.2 MB of partials), then a smaller session
    (2,600 keys, a 40-key tail) at a caller scale."""
    big, qb = replayed(SERVED, 31)
    both_reads([big], [qb], "served t=31")
    small, qs = replayed(SMALL, 12)
    both_reads([small], [qs], "smaller t=12 scale=0.3", scale=0.3)


@needs_gpu
def test_static_scratch_split_key_paths():
    """The split-key read: a served-shape session with a recency bias under the replace rope
    mode (its turned query and its partials both in the static array), then a smaller
    head_dim-128 session."""
    sess, q = replayed(SERVED, 30, recency_bias=True, rope_mode="replace")
    tab = sf_inputs.bias_table(SERVED, 0, 0, 2.0, device="cuda").contiguous()
    sess.set_recency_bias(tab)
    both_reads([sess], [q], "served bias+rope t=30")
    small, qs = replayed(SMALL128, 12)
    both_reads([small], [qs], "smaller head_dim 128 t=12")


@needs_gpu
def test_static_scratch_refuses_what_does_not_fit():
    """Three served sessions in one read need about 44 MB of partials, more than the 32 MiB
    array: the call returns SF_E_UNSUPPORTED and leaves the outputs untouched; sf_attend
    reads them."""
    sess = [replayed(SERVED, 31, session=i) for i in range(3)]
    handles = [s.handle for s, _ in sess]
    qs = [q for _, q in sess]
    outs = [torch.full(sf_inputs.record_shape(SERVED), 7.0, dtype=torch.float32, device="cuda") for _ in sess]
    with pytest.raises(sf.SfError) as ei:
        sf.sf_attend_static_scratch(handles, 0, qs, outs)
    assert ei.value.status == sf.SF_E_UNSUPPORTED
    assert "scratch" in str(ei.value)
    torch.cuda.synchronize()
    assert all(bool((o == 7.0).all()) for o in outs)
    sf.sf_attend(handles, 0, qs, outs)
    torch.cuda.synchronize()
    assert all(bool(torch.isfinite(o).all()) for o in outs)
