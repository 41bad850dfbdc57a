"""The library's kernel tracing: one event pair per launch, per kernel kind, on the caller's stream."""
import pytest
import torch

import sf_inputs

pytestmark = pytest.mark.gpu
needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


@needs_gpu
def test_kernel_times_count_every_launch():
    import compressed_memory_kv_amd as sf
    wl = dict(sf_inputs.WORKLOADS["served1"], n_blocks=2)
    sess = sf.Session(sf.make_config(**wl))
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    sf.sf_profile_enable(sess.handle, True)
    frames = 6
    for t in range(frames):   # the separate calls: evict, then per block write and attend
        if t >= 1:
            sess.evict(t)
        for b in range(2):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.write_record(b, t, k, v)
            sess.attend(b, q, out)
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["write"][1] == 2 * frames
    assert times["attend"][1] == 2 * frames
    assert times["combine"][1] == 2 * frames
    # keys past the last full 64-key tile are read by workgroups of the attention launch
    # itself when the read has full tiles (every read here), so no tail launch is made
    tails = sum(1 for t in range(frames) if sf.sf_plan(sess.cfg, t)["n_keys"] % 64)
    assert tails > 0 and times["tail"][1] == 0
    assert times["evict"][1] == frames - 4          # at t = 4, 5 frames 1, 2 leave RAW (Y = 2)
    assert all(times[k][0] > 0.0 for k in ("write", "attend", "combine", "evict"))
    again = sf.sf_kernel_times_read(sess.handle)   # a read starts a new period
    assert all(n == 0 for _, n in again.values())

    # sf_step, bf16 head_dim 64: the attention launch writes the record itself
    for t in range(frames, frames + 2):
        for b in range(2):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["write"][1] == 0
    assert times["attend"][1] == 4 and times["evict"][1] == 2
    sf.sf_profile_enable(sess.handle, False)


@needs_gpu
def test_rope_mode_launches():
    """Under a rope mode sf_step turns the query in its write launch; sf_attend turns it in a
    launch of its own."""
    import compressed_memory_kv_amd as sf
    wl = dict(sf_inputs.WORKLOADS["served1"], rope_mode="replace")
    sess = sf.Session(sf.make_config(**wl))
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    sf.sf_profile_enable(sess.handle, True)
    for t in range(4):
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["write"][1] == 4 and times["rope"][1] == 0 and times["attend"][1] == 4
    sess.attend(0, q, out)
    times = sf.sf_kernel_times_read(sess.handle)
    assert times["rope"][1] == 1 and times["attend"][1] == 1 and times["write"][1] == 0
    sf.sf_profile_enable(sess.handle, False)
