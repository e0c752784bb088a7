"""Parity of the layer steps (short convolution, gated RMSNorm) with the CPU
oracle (GPU tests, through the C ABI).  Same bar as the forward: max|err| /
rms(ref) <= 1e-4 for fp32 and <= 2e-2 for bf16 data; a bf16 result adds its
own final rounding (at most 2^-8 |ref|) to the allowance."""
import sys

import numpy as np
import pytest

from gated_delta_rule_33_amd.inputs import bf16_bits_to_f32, f32_to_bf16_bits, segment_ids_from_lengths
from oracle import layer_ops as lo
from tests.gpu_helpers import TOL_BF16, TOL_F32, check

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _data(shape, seed, dtype, scale=1.0):
    """Seeded N(0, scale^2) values, rounded to bf16 for bf16 data; returns the
    exact values (fp32 numpy) and the device tensor."""
    import torch
    x = (scale * np.random.default_rng(seed).standard_normal(shape)).astype(np.float32)
    if dtype == "bf16":
        bits = f32_to_bf16_bits(x)
        return bf16_bits_to_f32(bits), torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    return x, torch.from_numpy(x).cuda()


CONV = {
    "bf16_w4": dict(dtype="bf16", B=2, T=150, D=64, W=4, seg=None),
    "f32_w4": dict(dtype="f32", B=2, T=150, D=64, W=4, seg=None),
    "bf16_w1": dict(dtype="bf16", B=1, T=70, D=128, W=1, seg=None),
    "f32_w8_tail": dict(dtype="f32", B=1, T=200, D=1032, W=8, seg=None),
    "bf16_w3_packed": dict(dtype="bf16", B=2, T=160, D=96, W=3, seg=[[5, 60, 1, 2, 0], [100, 30]]),
    "f32_w4_packed": dict(dtype="f32", B=1, T=140, D=64, W=4, seg=[[1, 1, 1, 64, 70]]),
}


@pytest.mark.parametrize("case", list(CONV))
def test_short_conv(case):
    import torch
    from gated_delta_rule_33_amd import kda
    c = CONV[case]
    x, xd = _data((c["B"], c["T"], c["D"]), 41, c["dtype"])
    w = (0.5 * np.random.default_rng(42).standard_normal((c["D"], c["W"]))).astype(np.float32)
    seg = None
    if c["seg"] is not None:
        seg = segment_ids_from_lengths([[n for n in r if n > 0] for r in c["seg"]], c["T"])
        if case == "bf16_w3_packed":
            seg[0, 20:23] = 0          # padding inside a segment splits it
    _say(f"[parity] short conv {case}")
    y = kda.short_convolution(xd, torch.from_numpy(w).cuda(),
                              segment_ids=None if seg is None else torch.from_numpy(seg).cuda())
    torch.cuda.synchronize()
    ref = lo.short_conv(x, w, segment_ids=seg)
    got = y.float().cpu().numpy()
    tol = TOL_F32 if c["dtype"] == "f32" else TOL_BF16
    e = check(f"{case}", got, ref, tol, bf16_out=c["dtype"] == "bf16")
    _say(f"[parity] short conv {case} rel err {e:.3e}")
    if seg is not None:
        assert np.all(got[seg == 0] == 0.0)


def test_short_conv_full_size():
    """The q projection's shape at the benchmark workload: [1, 8192, 32*128] bf16."""
    import torch
    from gated_delta_rule_33_amd import kda
    x, xd = _data((1, 8192, 4096), 43, "bf16")
    w = (0.5 * np.random.default_rng(44).standard_normal((4096, 4))).astype(np.float32)
    _say("[parity] short conv full size")
    y = kda.short_convolution(xd, torch.from_numpy(w).cuda())
    torch.cuda.synchronize()
    ref = lo.short_conv(x[:, :, :512], w[:512])     # channels are independent
    check("full", y[:, :, :512].float().cpu().numpy(), ref, TOL_BF16, bf16_out=True)


NORM = {
    "f32_v128": dict(o="f32", g="f32", y="f32", shape=(2, 100, 3, 128)),
    "f32o_bf16g_bf16y": dict(o="f32", g="bf16", y="bf16", shape=(1, 77, 4, 128)),
    "bf16_v64": dict(o="bf16", g="bf16", y="bf16", shape=(3, 50, 2, 64)),
    "f32_v256_eps": dict(o="f32", g="f32", y="f32", shape=(2, 33, 256), eps=1e-2),
}


@pytest.mark.parametrize("case", list(NORM))
def test_gated_rmsnorm(case):
    import torch
    from gated_delta_rule_33_amd import kda
    c = NORM[case]
    V = c["shape"][-1]
    o, od = _data(c["shape"], 51, c["o"], scale=3.0)
    z, zd = _data(c["shape"], 52, c["g"], scale=2.0)
    w = (1.0 + 0.3 * np.random.default_rng(53).standard_normal(V)).astype(np.float32)
    eps = c.get("eps", 1e-6)
    _say(f"[parity] gated rmsnorm {case}")
    y = kda.gated_rmsnorm(od, zd, torch.from_numpy(w).cuda(), eps=eps,
                          out_dtype=torch.bfloat16 if c["y"] == "bf16" else torch.float32)
    torch.cuda.synchronize()
    ref = lo.gated_rmsnorm(o, z, w, eps=eps)
    tol = TOL_F32 if (c["o"], c["g"]) == ("f32", "f32") else TOL_BF16
    e = check(case, y.float().cpu().numpy(), ref, tol, bf16_out=c["y"] == "bf16")
    _say(f"[parity] gated rmsnorm {case} rel err {e:.3e}")
