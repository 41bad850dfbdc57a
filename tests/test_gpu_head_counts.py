"""GPU parity at other head counts of the served geometry.

2 and 4 heads are one GPU's share of the served 16 heads under 8- and 4-way head
sharding (the memory of a head never leaves its GPU), the case where the
stream-K read has the fewest units (2 x 9 and 4 x 9 query tiles) and splits every
column's keys most; 20 heads of 64 is the width the model card gives its model
(1280).  One block, frames 0..31 through sf_step (evictions, writes, rotations of
the slot map), buffers and slot tables bit for bit every frame, attention against
the oracle at fill levels with two segments, the first full window and frame 31.
Page: model card "GTA world model: weights and inference code", sections "What a
frame attends to" and "One buffer, no mask".
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


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def check(got: torch.Tensor, ref: np.ndarray, what: str):
    g = got.detach().double().cpu().numpy()
    err = np.abs(g - ref)
    max_abs = float(err.max())
    rel = float(np.linalg.norm(g - ref) / np.linalg.norm(ref))
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    assert max_abs <= 2e-2, f"{what}: max-abs {max_abs:.3e} > 2e-2"
    assert rel <= 1e-2, f"{what}: rel-L2 {rel:.3e} > 1e-2"
    return max_abs, rel


@needs_gpu
@pytest.mark.parametrize("heads", [2, 4, 20])
def test_served_geometry_head_counts(heads):
    wl = dict(sf_inputs.WORKLOADS["served1"], n_heads=heads, seed=6)
    g = so.Geometry.from_workload(wl)
    sess = sf.Session(sf.make_config(**wl))
    orc = so.MemoryReplay(g)
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    # at 20 heads every 3rd query row (plus the last) keeps the oracle's time in seconds
    rows = None if heads <= 4 else np.unique(np.concatenate([np.arange(0, g.r, 3), [g.r - 1]]))
    for t in wl["frames"]:
        q, k, v = sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")
        sess.step(0, t, q, k, v, out)
        orc.step(t, {0: (sf_inputs.to_host_bytes(k), sf_inputs.to_host_bytes(v))})
        torch.cuda.synchronize()
        view = sess.view()
        assert view["raw_frame"] == orc.raw_frame and view["sum_frame"] == orc.sum_frame, f"H={heads} t={t}"
        assert view["segments"] == orc.readable_segments() and view["n_keys"] == orc.n_keys(), f"H={heads} t={t}"
        kb, vb = sess.kv(0)
        assert torch.equal(kb.view(torch.int16), torch.from_numpy(orc.k[orc.index[0]].view(np.int16)).cuda()) and \
            torch.equal(vb.view(torch.int16), torch.from_numpy(orc.v[orc.index[0]].view(np.int16)).cuda()), \
            f"H={heads} t={t}: buffer bytes differ"
        if t in (3, 25, 31):
            ref = orc.attend(0, sf_inputs.to_host_bytes(q), rows=rows)
            got = out if rows is None else out[torch.from_numpy(rows).cuda()]
            ma, rel = check(got, ref, f"H={heads} t={t}")
            say(f"[heads {heads}] t={t} keys={orc.n_keys()} max_abs={ma:.2e} rel_l2={rel:.2e}")
    assert orc.n_keys() == 6528
