"""GPU parity of kda_gated_rmsnorm against the oracle.

Every element against the fp64 oracle on the same seeded inputs: fp32 out
within max |gpu - oracle| / rms(oracle) <= 1e-4; bf16 out within one bf16
rounding of the exact value plus the fp32 error, |gpu - oracle| <= 2^-8
|oracle| + 1e-5 rms(oracle).  Every head dim, fp32 and bf16 gates and outputs,
in place over o, and the full output of the 4 x 4096-token, 16-head workload.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, err
from kda_inputs import to_f64

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # collected on CPU, skipped there
    pytest.skip("needs a GPU", allow_module_level=True)

import gated_delta_rule_67_amd as kda  # noqa: E402


def inputs(B, T, H, D, gate_dtype, seed):
    rng = np.random.default_rng(seed)
    o = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32) * np.float32(0.3))
    g = torch.from_numpy(rng.standard_normal((B, T, H, D), dtype=np.float32) * np.float32(2.0))
    g = g.to(torch.bfloat16) if gate_dtype == "bf16" else g
    w = torch.from_numpy(rng.standard_normal(D).astype(np.float32))
    return o, g, w


def check(tag, y, ref, out_dtype):
    y = y.float().cpu().numpy().astype(np.float64)
    if out_dtype == torch.bfloat16:
        bound = 2.0 ** -8 * np.abs(ref) + 1e-5 * np.sqrt(np.mean(ref ** 2))
        worst = float(np.max(np.abs(y - ref) / bound))
        print(f"[norm {tag}] within {worst:.2f} of the bf16 bound", flush=True)
        assert np.all(np.isfinite(y)) and worst <= 1.0
    else:
        e = err(y, ref)
        print(f"[norm {tag}] {e:.2e}", flush=True)
        assert e <= TOL["f32"]


@pytest.mark.parametrize("D,gate_dtype,out_dtype", [(128, "bf16", torch.bfloat16), (128, "f32", torch.float32),
                                                    (64, "bf16", torch.float32), (32, "f32", torch.bfloat16),
                                                    (16, "bf16", torch.bfloat16)])
def test_shapes_and_dtypes(D, gate_dtype, out_dtype):
    o, g, w = inputs(2, 37, 3, D, gate_dtype, seed=400 + D)
    eps = 1e-6
    y = kda.gated_rmsnorm(o.cuda(), g.cuda(), w.cuda(), eps, out_dtype=out_dtype)
    torch.cuda.synchronize()
    check(f"D={D} gate={gate_dtype} out={out_dtype}", y, oracle.gated_rmsnorm(to_f64(o), to_f64(g), to_f64(w), eps),
          out_dtype)


def test_in_place_over_o():
    o, g, w = inputs(1, 50, 4, 128, "bf16", seed=410)
    od = o.cuda()
    y = kda.gated_rmsnorm(od, g.cuda(), w.cuda(), 1e-5, out=od)
    torch.cuda.synchronize()
    assert y.data_ptr() == od.data_ptr()
    check("in place", y, oracle.gated_rmsnorm(to_f64(o), to_f64(g), to_f64(w), 1e-5), torch.float32)


def test_full_size_workload():
    o, g, w = inputs(4, 4096, 16, 128, "bf16", seed=420)
    y = kda.gated_rmsnorm(o.cuda(), g.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    check("full size", y, oracle.gated_rmsnorm(to_f64(o), to_f64(g), to_f64(w), 1e-6), torch.bfloat16)
