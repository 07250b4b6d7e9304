"""Helpers for GPU tests: move exact-valued float64 arrays to the device in the
kernel's dtype, call the HIP library through its binding, bring results back."""
from __future__ import annotations

import numpy as np

TOL = {"bf16": 2e-2, "f32": 1e-4}


def torch_dtype(dtype):
    import torch

    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def to_device(x, dtype):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch_dtype(dtype))
    # inputs already hold dtype values: the conversion must be exact
    assert np.array_equal(t.double().numpy(), x), "input not exactly representable"
    return t.to("cuda")


def run_hip(q, k, v, cu, mask, scale, dtype, out=None):
    import torch

    import long_context_attention_prefill_amd as lcap

    tq, tk, tv = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    res = lcap.attn_prefill(tq, tk, tv, [int(x) for x in cu], mask=mask, scale=scale, out=out)
    torch.cuda.synchronize()
    return res.double().cpu().numpy()


def max_err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.size == 0:
        return 0.0
    assert np.all(np.isfinite(a)), "non-finite GPU output"
    return float(np.max(np.abs(a - b)))


# log-sum-exp tolerance: the bf16 path sums bf16-rounded probabilities (each
# within 2^-8 relative: round to nearest keeps 8 significant bits), so
# ln(sum) is within about 2^-8 of exact; 2^-7 leaves a factor 2 for the fp32
# score and exp2 rounding.  The fp32 path sums fp32
# probabilities: within n * 2^-24 relative, < 1e-4 for the sizes tested.
LSE_TOL = {"bf16": 2.0 ** -7, "f32": 1e-4}


def run_hip_kv(q, k, v, cu_q, cu_k, mask, scale, dtype, lse=True):
    import torch

    import long_context_attention_prefill_amd as lcap

    tq, tk, tv = to_device(q, dtype), to_device(k, dtype), to_device(v, dtype)
    res = lcap.attn_prefill_kv(tq, tk, tv, [int(x) for x in cu_q], [int(x) for x in cu_k],
                               mask=mask, scale=scale, lse=lse)
    torch.cuda.synchronize()
    if lse:
        out, l = res
        return out.double().cpu().numpy(), l.double().cpu().numpy()
    return res.double().cpu().numpy()
