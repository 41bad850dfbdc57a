"""The head_dim-64 read with its workgroup ranges computed in the kernel in 64-bit arithmetic
against the same read in its usual form and against the oracle.

Model card "GTA world model: weights and inference code", section "One buffer, no mask": the
read is one dense softmax over every filled row.  How the bf16 head_dim-64 read splits that
work over workgroups is the kernel's own affair: the host tabulates each group's first
iteration when the launch has at most 384 groups, and the kernel otherwise computes them, in
32-bit integers when cost units times groups stay below 2^31 and in 64-bit integers beyond.
Test launches mostly stay in the table, so `sf_debug_wide_ranges` forces the computed
64-bit form: all forms give the same ranges, so outputs must match bit for bit, and they are
checked against the oracle as well.
"""
import numpy as np
import pytest
import torch

import sf_inputs
from test_gpu_parity import _replay, check_attention, host, say

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:  # collected on a CPU-only machine: every test here is skipped
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


@needs_gpu
def test_wide_ranges_bit_identical():
    """A single read and a batch of three record sizes (9, 3 and 13 query tiles, two with key
    tails), each in both range forms."""
    base = dict(y=2, w=6, n_heads=16, head_dim=64, n_blocks=1, dtype="bf16", v_scale=1.0)
    shapes = [(1008, 96, 8), (280, 20, 5), (1500, 100, 6)]  # (hw, x, frame)
    wls, sessions, oracles = [], [], []
    for si, (hw, x, t_end) in enumerate(shapes):
        wl = dict(base, hw=hw, x=x, frames=list(range(t_end + 1)), seed=60 + si)
        say(f"[wide] replay session {si}: R={hw + x}, to t={t_end}")
        _, sess, orc = _replay(wl, si, t_end)
        wls.append(wl)
        sessions.append(sess)
        oracles.append(orc)
    qs = [sf_inputs.frame_tensors(wl, si, 0, wl["frames"][-1], device="cuda")[0] for si, wl in enumerate(wls)]

    def read_all():
        single = torch.empty(sf_inputs.record_shape(wls[0]), dtype=torch.float32, device="cuda")
        sessions[0].attend(0, qs[0], single)
        outs = [torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda") for wl in wls]
        sf.attend_batch(sessions, 0, qs, outs)
        torch.cuda.synchronize()
        return [single] + outs

    say("[wide] 32-bit ranges")
    narrow = read_all()
    say("[wide] 64-bit ranges")
    sf.sf_debug_wide_ranges(True)
    try:
        wide = read_all()
    finally:
        sf.sf_debug_wide_ranges(False)
    for i, (a, b) in enumerate(zip(narrow, wide)):
        assert torch.equal(a, b), f"read {i}: 64-bit and 32-bit ranges differ"
    for si, orc in enumerate(oracles):
        ref = orc.attend(0, host(qs[si]))
        ma, rel = check_attention(wide[1 + si], ref, "bf16", f"wide s{si} keys={orc.n_keys()}")
        say(f"   s{si} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
