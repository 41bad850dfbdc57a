"""GPU parity of the streaming sink: Z0's keys rotated forward in place.

Page: model card "GTA world model: weights and inference code", section "Running
for a long time: the start image follows the window".  The library rotates in
fp32 and rounds to the storage type; the oracle rotates in fp64 and rounds once.
So a rotation of the same stored keys may differ by one unit in the last place of
the storage type, at rounding ties only; every other byte (V, all rows past Z0, the
slot tables) must match exactly, and attention outputs within the usual tolerance.
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


def ulp(v: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type at fp64 values v (bf16: 8 significant bits, f32: 24)."""
    bits = 8 if dtype == "bf16" else 24
    e = np.frexp(np.abs(v))[1]
    return np.ldexp(1.0, np.maximum(e, -125) - bits)


def plane_norm(k: np.ndarray, head_dim: int) -> np.ndarray:
    """|x| + |y| of each value's temporal plane (0 outside the band), same shape as k."""
    n = so.temporal_planes(head_dim)
    out = np.zeros_like(k)
    s = np.abs(k[..., 0:2 * n:2]) + np.abs(k[..., 1:2 * n:2])
    out[..., 0:2 * n:2] = s
    out[..., 1:2 * n:2] = s
    return out


def host_bits(t: torch.Tensor) -> np.ndarray:
    return sf_inputs.to_host_bytes(t)


def check_rotation(before: np.ndarray, after: np.ndarray, T: int, head_dim: int, dtype: str, what: str):
    """One rotation step of the library against the exact rotation of the same stored keys:
    within half a unit of the storage type's last place of the exact value, plus the
    error of fp32 products and sums (a few 2**-24 of the plane's |x| + |y|)."""
    x = so.stored_to_f64(before)
    exact = so.rotate_temporal(x, head_dim, T)
    got = so.stored_to_f64(after)
    bound = 0.505 * ulp(exact, dtype) + 8 * 2.0 ** -24 * plane_norm(x, head_dim) + 1e-30
    ratio = np.abs(got - exact) / bound
    say(f"   {what}: worst error {ratio.max():.2f} of the bound; "
        f"{int((so.f64_to_storage(exact, dtype) != after).sum())} of {after.size} differ from the oracle's rounding")
    assert ratio.max() <= 1.0, what


def run_case(wl, frames, check_attention_at=()):
    g = so.Geometry.from_workload(wl)
    cfg = sf.make_config(**wl)
    sess = sf.Session(cfg)
    orc = so.MemoryReplay(g, sink_gap=wl["sink_gap"])
    out = torch.empty(sf_inputs.record_shape(wl), dtype=torch.float32, device="cuda")
    nb = wl["n_blocks"]
    r = g.r
    rotations = 0
    for t in frames:
        z_before = sess.view()["z0_frame"]
        k0_before = [host_bits(sess.kv(b)[0][:r]) for b in range(nb)]
        recs = {}
        for b in range(nb):
            q, k, v = sf_inputs.frame_tensors(wl, 0, b, t, device="cuda")
            sess.step(b, t, q, k, v, out)
            recs[b] = (host_bits(k), host_bits(v))
            if t in check_attention_at and b == 0:
                torch.cuda.synchronize()
                qh = host_bits(q)
        torch.cuda.synchronize()
        orc.step(t, recs)
        view = sess.view()
        assert view["z0_frame"] == orc.z0_frame, t
        assert view["raw_frame"] == orc.raw_frame and view["sum_frame"] == orc.sum_frame, t
        if view["z0_frame"] != z_before:
            rotations += 1
            T = view["z0_frame"] - z_before
            say(f"[sink] t={t}: Z0 moved by {T} to frame {view['z0_frame']}")
            for b in range(nb):
                check_rotation(k0_before[b], host_bits(sess.kv(b)[0][:r]), T, g.head_dim, g.dtype, f"block {b}")
        for b in range(nb):
            kg, vg = sess.kv(b)
            kh, vh = host_bits(kg), host_bits(vg)
            i = orc.index[b]
            np.testing.assert_array_equal(vh, orc.v[i], err_msg=f"V, t={t}")
            np.testing.assert_array_equal(kh[r:], orc.k[i][r:], err_msg=f"K past Z0, t={t}")
            if rotations == 0:
                np.testing.assert_array_equal(kh[:r], orc.k[i][:r], err_msg=f"Z0 K, t={t}")
            else:  # each rotation may round a tie the other way; differences stay that small
                a, o = so.stored_to_f64(kh[:r]), so.stored_to_f64(orc.k[i][:r])
                bound = rotations * (ulp(o, g.dtype) + 16 * 2.0 ** -24 * plane_norm(o, g.head_dim)) + 1e-30
                assert (np.abs(a - o) <= bound).all(), (t, float((np.abs(a - o) / bound).max()))
        if t in check_attention_at:
            # sf_step attended from the buffer as it stood after this frame's writes (block nb-1's
            # output is in `out`); compare block 0 instead: attend again and check
            sess.attend(0, sf_inputs.frame_tensors(wl, 0, 0, t, device="cuda")[0], out)
            torch.cuda.synchronize()
            ref = orc.attend(0, qh)
            got = out.double().cpu().numpy()
            err = np.abs(got - ref)
            rel = float(np.linalg.norm(got - ref) / np.linalg.norm(ref))
            say(f"   attention t={t}: max-abs {err.max():.2e} rel-L2 {rel:.2e}")
            assert err.max() <= TOL[g.dtype]["max_abs"] and rel <= TOL[g.dtype]["rel_l2"]
    return rotations


@needs_gpu
def test_sink_served_bf16():
    """Served grid (16 heads x 64, bf16), 1 block, sink gap 5: Z0 moves at t = 29, 33, 37."""
    wl = dict(sf_inputs.WORKLOADS["served1"], sink_gap=5)
    n = run_case(wl, range(38), check_attention_at=(29, 37))
    assert n == 3


@needs_gpu
def test_sink_tiny_f32():
    """fp32 storage, head_dim 64, W = 6, gap 5: Z0 moves at t = 11, 15, 19."""
    wl = dict(sf_inputs.WORKLOADS["tiny"], sink_gap=5)
    n = run_case(wl, range(21), check_attention_at=(11, 20))
    assert n == 3


@needs_gpu
def test_sink_head_dim_128_two_blocks():
    """bf16, head_dim 128 (22 temporal planes), two blocks, W = 3, gap 3."""
    wl = dict(hw=40, x=8, y=0, w=3, n_heads=3, head_dim=128, n_blocks=2, dtype="bf16", seed=9, v_scale=1.0,
              sink_gap=3)
    n = run_case(wl, range(16), check_attention_at=(8, 15))
    assert n >= 4
