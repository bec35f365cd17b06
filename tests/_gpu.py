"""GPU-side helpers for the parity tests: upload seeded inputs, run the
library through its C ABI, bring results back as NumPy arrays."""
import sys

import numpy as np

from bit_complex_weight_amd import fairy as F


def torch():
    import torch as _t
    return _t


def dev(a):
    t = torch()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    if a.dtype == np.uint32:
        a = a.view(np.int32)
    return t.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


class GpuLayer:
    """Device buffers of a quantised layer plus its C descriptor."""

    def __init__(self, n, m, stages, has_conj, packed, scales):
        self.n, self.m, self.stages, self.has_conj = n, m, stages, has_conj
        self.packed, self.scales = packed, scales
        self.desc = F.make_clinear(n, m, stages, has_conj, packed, scales)

    @property
    def planes(self):
        return self.stages * (2 if self.has_conj else 1)


def pack_on_gpu(codes_dev, planes, rows, m, layout=F.FAIRY_LAYOUT_TILED64):
    t = torch()
    nw = F.fairy_packed_words(rows, m, planes, layout)
    packed = t.empty(nw, dtype=t.int32, device="cuda")
    F.fairy_pack(codes_dev, planes, rows, m, layout, packed)
    return packed


def layer_from_codes(codes, scales, stages, has_conj):
    """Upload host codes [P][n][m] and scales [P][2]; pack on the GPU."""
    P, n, m = codes.shape
    packed = pack_on_gpu(dev(codes), P, n, m)
    return GpuLayer(n, m, stages, has_conj, packed, dev(np.ascontiguousarray(scales, np.float32)))


def phasequant_on_gpu(w_re_dev, w_im_dev, count, stages, want_resid=True):
    t = torch()
    codes = t.empty(stages * count, dtype=t.uint8, device="cuda")
    scales = t.empty(stages * 2, dtype=t.float32, device="cuda")
    rr = t.empty(count, dtype=t.float32, device="cuda") if want_resid else None
    ri = t.empty(count, dtype=t.float32, device="cuda") if want_resid else None
    wsb = F.fairy_phasequant_workspace_bytes(count, stages)
    ws = t.empty(wsb, dtype=t.uint8, device="cuda")
    F.fairy_phasequant(w_re_dev, w_im_dev, count, stages, codes, scales, rr, ri, ws, wsb)
    return codes, scales, rr, ri


def quantize_widely_linear_on_gpu(u_re, u_im, w_re, w_im, n, m, stages):
    """U, W device planes [n][m] -> GpuLayer with planes U_1..U_S, W_1..W_S."""
    t = torch()
    count = n * m
    cu, su, _, _ = phasequant_on_gpu(u_re, u_im, count, stages, want_resid=False)
    cw, sw, _, _ = phasequant_on_gpu(w_re, w_im, count, stages, want_resid=False)
    codes = t.cat([cu, cw])
    scales = t.cat([su, sw])
    packed = pack_on_gpu(codes, 2 * stages, n, m)
    return GpuLayer(n, m, stages, 1, packed, scales), codes, scales


def run_gemv(layer, x_re, x_im, xdtype, B, want_acc=False, gemm=False, algo=F.FAIRY_ALGO_AUTO, workspace=False):
    """workspace (GEMM only): pass the optional K-split workspace, filled with
    0xFF bytes (NaNs if read before written)."""
    t = torch()
    n, m = layer.n, layer.m
    y_re = t.empty((B, n), dtype=t.float32, device="cuda")
    y_im = t.empty((B, n), dtype=t.float32, device="cuda")
    acc = t.empty((layer.planes, 4, B, n), dtype=t.int32, device="cuda") if want_acc else None
    ldx = x_re.shape[-1]
    if gemm:
        ws, wsb = None, 0
        if workspace:
            wsb = F.fairy_cgemm_workspace_bytes(layer.desc, B, xdtype, algo)
            ws = t.full((max(wsb, 16),), 255, dtype=t.uint8, device="cuda")
        F.fairy_cgemm(layer.desc, x_re, x_im, xdtype, B, ldx, y_re, y_im, n, acc, algo, ws, wsb)
    else:
        F.fairy_cgemv(layer.desc, x_re, x_im, xdtype, B, ldx, y_re, y_im, n, acc)
    t.cuda.synchronize()
    return host(y_re), host(y_im), (host(acc) if want_acc else None)


def rel_l2(got, want):
    """Relative L2 error of complex (or real) arrays, in float64."""
    got = np.asarray(got).astype(np.complex128)
    want = np.asarray(want).astype(np.complex128)
    assert got.shape == want.shape, (got.shape, want.shape)
    return float(np.linalg.norm((got - want).ravel()) / max(np.linalg.norm(want.ravel()), 1e-300))
