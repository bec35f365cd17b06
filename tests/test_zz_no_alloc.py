"""The allocation-free PhaseQuant (fairy_phasequant_noalloc, buckets in a
static device array) against fairy_phasequant with a caller workspace: codes,
scales and residuals bit for bit, on two calls in a row, the second with a
smaller input (fewer elements and fewer stages), so the second call runs on
the array the first one left behind.  The first case is also held to the
oracle."""
import numpy as np
import pytest

import oracle
from bit_complex_weight_amd import fairy as F
from bit_complex_weight_amd import synth
from tests._gpu import dev, host, log, phasequant_on_gpu, torch

pytestmark = pytest.mark.gpu


def noalloc(w_re, w_im, count, stages):
    t = torch()
    codes = t.full((stages * count,), 255, dtype=t.uint8, device="cuda")
    scales = t.full((stages * 2,), float("nan"), dtype=t.float32, device="cuda")
    rr = t.empty(count, dtype=t.float32, device="cuda")
    ri = t.empty(count, dtype=t.float32, device="cuda")
    F.fairy_phasequant_noalloc(w_re, w_im, count, stages, codes, scales, rr, ri)
    t.cuda.synchronize()
    return host(codes), host(scales), host(rr), host(ri)


@pytest.mark.parametrize("shapes", [((2048 * 2048, 3), (4099, 2)), ((256 * 256, 8), (5, 1))])
def test_phasequant_noalloc_matches_workspace_call(shapes):
    t = torch()
    for i, (count, stages) in enumerate(shapes):
        log(f"noalloc phasequant call {i}: count={count} stages={stages}")
        re, im = synth.complex_gaussian((count,), 0.02, 730 + i + count)
        wr, wi = dev(re), dev(im)
        got = noalloc(wr, wi, count, stages)
        c, s, rr, ri = phasequant_on_gpu(wr, wi, count, stages, want_resid=True)
        t.cuda.synchronize()
        want = (host(c), host(s), host(rr), host(ri))
        assert np.array_equal(got[0], want[0])
        assert np.array_equal(got[1].view(np.uint32), want[1].view(np.uint32))
        assert np.array_equal(got[2].view(np.uint32), want[2].view(np.uint32))
        assert np.array_equal(got[3].view(np.uint32), want[3].view(np.uint32))
        if i == 0 and count <= 256 * 256:
            oc, osc, orr, ori = oracle.phasequant(re, im, stages, want_resid=True)
            assert np.array_equal(got[0].reshape(stages, count), oc)
            assert np.array_equal(got[1].reshape(stages, 2).view(np.uint32), osc.view(np.uint32))
