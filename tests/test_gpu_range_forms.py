"""The head_dim-64 read under each way of cutting its work into workgroup ranges, against
the oracle and (where the ranges are the same) against each other.

Model card "GTA world model: weights and inference code", section "One buffer, no mask": the
read is one dense softmax over every filled row.  How the bf16 head_dim-64 read splits that
work over workgroups is the kernel's own affair, with three forms (`sf_debug_range_form`):
0, the library's choice, a range table the host makes, weighted by how fast each group of
workgroups runs; 1, the kernel's own unweighted formula in 32-bit arithmetic; 2, the same
formula in 64-bit arithmetic, the form of launches too large for the other two.  Forms 1 and 2
give the same ranges, so their outputs must match bit for bit; every form is checked against
the oracle at the bf16 bar.
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
def test_range_forms():
    """A single read and a batch of three record sizes (9, 3 and 13 query tiles, two with key
    tails), in each range form."""
    base = dict(y=2, w=6, n_heads=16, head_dim=64, n_blocks=1, dtype="bf16", v_scale=1.0)
    shapes = [(1008, 96, 8), (280, 20, 5), (1500, 100, 6)]  # (hw, x, frame)
    wls, sessions, oracles = [], [], []
    for si, (hw, x, t_end) in enumerate(shapes):
        wl = dict(base, hw=hw, x=x, frames=list(range(t_end + 1)), seed=60 + si)
        say(f"[forms] replay session {si}: R={hw + x}, to t={t_end}")
        _, sess, orc = _replay(wl, si, t_end)
        wls.append(wl)
        sessions.append(sess)
        oracles.append(orc)
    qs = [sf_inputs.frame_tensors(wl, si, 0, wl["frames"][-1], device="cuda")[0] for si, wl in enumerate(wls)]
    refs = [orc.attend(0, host(qs[si])) for si, orc in enumerate(oracles)]

    def read_all(form):
        sf.sf_debug_range_form(form)
        try:
            single = torch.empty(sf_inputs.record_shape(wls[0]), dtype=torch.float32, device="cuda")
            sessions[0].attend(0, qs[0], single)
            outs = [torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda") for wl in wls]
            sf.attend_batch(sessions, 0, qs, outs)
            torch.cuda.synchronize()
        finally:
            sf.sf_debug_range_form(0)
        return [single] + outs

    got = {}
    for form in (0, 1, 2):
        say(f"[forms] form {form}")
        got[form] = read_all(form)
        for i, out in enumerate(got[form]):
            si = 0 if i == 0 else i - 1
            ma, rel = check_attention(out, refs[si], "bf16", f"form {form} read {i} keys={oracles[si].n_keys()}")
            say(f"   read {i} (session {si}) max_abs={ma:.2e} rel_l2={rel:.2e}")
    for i, (a, b) in enumerate(zip(got[1], got[2])):
        assert torch.equal(a, b), f"read {i}: the formula's 32-bit and 64-bit forms differ"
    with pytest.raises(sf.SfError):
        sf.sf_debug_range_form(3)
