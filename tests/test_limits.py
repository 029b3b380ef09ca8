"""GPU parity at the far end of the 32-bit offsets: chunks of d_u and d_dv whose byte extent comes within a few KiB of
2^31, the largest the matrix-core kernels address with 32-bit offsets (C * ld_u * 4 < 2^31 for d_u; (C + 32) * ld_dv
* 4 < 2^31 for slabs moved straight to LDS). Two chunks, so the second chunk starts about 2 GiB past the first.

Only the hd data columns are generated on the host; the padded device buffers (about 4 GiB each) are filled with a
sentinel on the device, the data columns copied in, and after the run every padding word is checked on the device.
The oracle runs on the compact (N, C, hd) arrays: each output reads only its own column of d_dv.
"""

import numpy as np
import pytest

import deterministic_fp32_gemm_amd as g
from deterministic_fp32_gemm_amd import inputs
from tests.gpu_util import expected, say
from tests.compare import mismatch_report, same_bits

pytestmark = pytest.mark.gpu

SENTINEL = 0x7FC5A5A5                 # a NaN pattern no output can take by arithmetic on these inputs
C, HD, N, P = 256, 64, 2, 1
LD_U = (1 << 21) - 4                  # C * LD_U * 4 = 2^31 - 4096
LD_DV_DMA = 1864132                   # (C + 32) * LD_DV * 4 = 2^31 - 3584
assert C * LD_U * 4 < 1 << 31 and (C + 32) * LD_DV_DMA * 4 < 1 << 31
assert (C + 32) * LD_U * 4 >= 1 << 31                 # with ld_dv = LD_U, slabs cannot go straight to LDS


@pytest.fixture(scope="module")
def host_inputs():
    x, dv, du = inputs.shape_inputs(N, C, HD, HD, "hazard_cancel", seed=2031)
    return x, dv, du, expected(x, dv, du, HD, 0, N)


def padded(compact: np.ndarray, ld: int, residue_bytes: int):
    """A device float32 buffer [N, C, ld] at residue_bytes past a 256-byte boundary: sentinel everywhere, then the
    compact columns copied into columns 0..hd-1. Returns (flat view, [N, C, ld] view)."""
    import torch
    n = N * C * ld
    raw = torch.empty(n + 64, dtype=torch.float32, device="cuda")
    off = ((residue_bytes - raw.data_ptr()) % 256) // 4
    buf = raw[off:off + n]
    buf.view(torch.int32).fill_(SENTINEL)
    v = buf.view(N, C, ld)
    v[:, :, :HD].copy_(torch.from_numpy(compact))
    return buf, v


def padding_untouched(v) -> bool:
    import torch
    for n in range(N):
        pad = v[n, :, HD:].view(torch.int32)
        if not bool((pad == SENTINEL).all()):
            return False
    return True


@pytest.mark.parametrize("name,ld_dv,residue,plan", [
    ("planner, direct-to-LDS slabs", LD_DV_DMA, 0, None),
    ("direct-to-LDS, d_u and d_dv rows at +4 B", LD_DV_DMA, 4, ("mfma", 2, 2, 3, 0, 1, 0, 0, 16, 16)),
    ("direct-to-LDS plan, ld_dv too wide: register ring", LD_U, 0, ("mfma", 2, 2, 3, 0, 1, 0, 0, 16, 32)),
    ("register ring", LD_U, 0, ("mfma", 2, 2, 4, 2, 4, 0, 0, 32, 16)),
    ("vector ALU", LD_U, 0, ("valu", 8, 1, 4, 1, 1)),
])
def test_chunk_offsets_near_2_31(host_inputs, name, ld_dv, residue, plan):
    import torch
    x_h, dv_h, du_h, want = host_inputs
    say(f"offsets near 2^31: {name}: N={N} C={C} hd={HD} ld_u={LD_U} ld_dv={ld_dv} residue {residue} plan {plan}")
    x = torch.from_numpy(x_h).cuda()
    dv, _ = padded(dv_h, ld_dv, residue)
    du, du_v = padded(du_h, LD_U, residue)
    if plan is not None:
        plan = g.make_mfma_plan(*plan[1:]) if plan[0] == "mfma" else g.make_plan(*plan[1:])
    g.sdm_gx_gemm_steps(du, LD_U, x, dv, ld_dv, N, P, C, HD, 0, N // P, g.SDM_GX_STEPS_FUSED, plan)
    torch.cuda.synchronize()
    got = du_v[:, :, :HD].cpu().numpy()
    ok = same_bits(got, want)
    assert ok.all(), f"{name}: " + mismatch_report(got, want, ok)
    assert padding_untouched(du_v), f"{name}: a padding word of d_u was written"
    del dv, du, du_v
    torch.cuda.empty_cache()
