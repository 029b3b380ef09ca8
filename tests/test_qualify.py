"""Vendor-BLAS qualification probe (diagnostic): rocBLAS strided-batched SGEMM and torch.baddbmm against the fixed
chain, per pattern and alignment class. The chain side is pinned to the oracle here; the vendor side is checked to
compute the same update (within the forward error bound of the exact result on finite inputs) and reported as
equal / differ bit for bit."""

import numpy as np
import pytest

from deterministic_fp32_gemm_amd import inputs, qualify
from tests.gpu_util import expected, say

pytestmark = pytest.mark.gpu

CASES = ((64, 64, 64, 0), (128, 128, 128, 0), (64, 256, 260, 4), (37, 150, 157, 12))


def test_vendor_blas_qualification_report():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible")
    say(f"rocBLAS {qualify.rocblas_version()}")
    patterns = ("normal", "zeros", "large", "hazard_cancel", "hazard_subnormal", "nan")
    rows = qualify.qualify(cases=CASES, patterns=patterns)
    assert len(rows) == len(CASES) * len(patterns) * 2
    for r in rows:
        say(f"{r['backend']:8s} C={r['C']:3d} hd={r['hd']:3d} ld={r['ld']:3d} res={r['residue']:2d} "
            f"{r['pattern']:15s} {r['verdict']:6s} differ {r['differ']:6d}/{r['outputs']} max_ulp {r['max_ulp']}")
        assert r["verdict"] in ("equal", "differ")
        if r["pattern"] == "zeros":                 # x = d_dv = d_u = +0: every path gives +0
            assert r["verdict"] == "equal"


@pytest.mark.parametrize("C,hd,ld,res", CASES)
def test_qualification_reference_is_the_chain(C, hd, ld, res):
    """The probe's reference (this library's update) equals the oracle, and the vendor paths compute the same
    update: within the forward error bound of the exact sum on normal inputs (a wrong transpose or stride would
    fail by orders of magnitude)."""
    import torch
    from deterministic_fp32_gemm_amd.step import aligned_empty

    N, P = 8, 8
    x_h, dv_h, du_h = inputs.shape_inputs(N, C, hd, ld, "normal", seed=7 + C + hd + res)
    want = expected(x_h, dv_h, du_h, hd, 0, N)
    exact = du_h[:, :, :hd].astype(np.float64) + np.einsum("nji,njc->nic", x_h.astype(np.float64),
                                                            dv_h[:, :, :hd].astype(np.float64))
    mag = np.abs(du_h[:, :, :hd]).astype(np.float64) + np.einsum("nji,njc->nic", np.abs(x_h).astype(np.float64),
                                                                  np.abs(dv_h[:, :, :hd]).astype(np.float64))
    bound = (C + 1) * np.finfo(np.float32).eps * mag * 1.01 + 1e-30
    for who in ("chain", "rocblas", "torch"):
        x = aligned_empty(x_h.size, 0)
        dv = aligned_empty(dv_h.size, res)
        du = aligned_empty(du_h.size, res)
        x.copy_(torch.from_numpy(x_h.reshape(-1)))
        dv.copy_(torch.from_numpy(dv_h.reshape(-1)))
        du.copy_(torch.from_numpy(du_h.reshape(-1)))
        if who == "chain":
            import deterministic_fp32_gemm_amd as g
            g.sdm_gx_gemm_steps(du, ld, x, dv, ld, N, P, C, hd, 0, 1, g.SDM_GX_STEPS_FUSED)
        elif who == "rocblas":
            qualify.rocblas_update(du, ld, x, dv, ld, 0, N, C, hd)
        else:
            x3 = x.view(N, C, C).transpose(1, 2).contiguous()
            du3 = du.view(N, C, ld)[:, :, :hd]
            du3.copy_(torch.baddbmm(du3, x3, dv.view(N, C, ld)[:, :, :hd]))
        torch.cuda.synchronize()
        got = du.cpu().numpy().reshape(N, C, ld)
        assert (got[:, :, hd:].view(np.uint32) == du_h[:, :, hd:].view(np.uint32)).all(), f"{who}: padding touched"
        err = np.abs(got[:, :, :hd].astype(np.float64) - exact)
        assert (err <= bound).all(), f"{who}: outside the error bound (max ratio {(err / bound).max():.3g})"
        if who == "chain":
            assert (got.view(np.uint32) == want.view(np.uint32)).all(), "chain differs from the oracle"
