"""The counter-calibration copy (sf_debug_lds_copy) moves its bytes exactly.

It is a measurement aid, not part of the method: a copy of known size through LDS with
the head_dim-64 attention's buffer-to-LDS transfer, which the counter runs use to scale
FETCH_SIZE on that path.  Its figure is only worth something if the copy is exact.
"""
import sys

import pytest
import torch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import compressed_memory_kv_amd as sf
else:  # collected on a CPU-only machine: every test here is skipped
    sf = None

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs an MI355X GPU")


@needs_gpu
@pytest.mark.parametrize("nbytes", [16384, 3 * 16384, 1 << 20])
def test_lds_copy_is_exact(nbytes):
    print(f"[lds copy] {nbytes} bytes", flush=True)
    sys.stdout.flush()
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes + 16384,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros(nbytes + 16384, dtype=torch.uint8, device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        sf.sf_debug_lds_copy(dst, src, nbytes, s)
    s.synchronize()
    assert torch.equal(dst[:nbytes], src[:nbytes])
    assert not dst[nbytes:].any(), "bytes past the copy were written"
