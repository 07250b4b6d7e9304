"""attn_decode_noalloc (the library's static device workspace) against
attn_decode with a caller workspace, through the C ABI, on two calls in a row
(the second smaller), each also checked against the fp64 oracle."""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(lens, hq, hkv, d, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = W.round_to(rng.standard_normal((len(lens), hq, d)), W.BF16)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    return q, k, v, cu_k


# a batch that splits its caches (workspace needed), then a smaller one
CASES = [([3000, 7000, 1, 4096, 250], 16, 2, 128, "causal", 41),
         ([1500, 70, 800], 8, 8, 64, ("window", 512), 42)]


def test_noalloc_matches_caller_workspace_twice(orc):
    import torch

    import long_context_attention_prefill_amd as lcap

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    needs = []
    for lens, hq, hkv, d, mask, seed in CASES:
        q, k, v, cu_k = _case(lens, hq, hkv, d, seed)
        cu = [int(x) for x in cu_k]
        scale = 1.0 / math.sqrt(d)
        need = lcap.attn_decode_workspace_size(cu, hq, hkv, d, lcap.ATTN_BF16, mask)
        needs.append(need)
        assert need <= lcap.ATTN_DECODE_SCRATCH_BYTES
        tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        ref_out, ref_lse = lcap.attn_decode(tq, tk, tv, cu, mask=mask, scale=scale, lse=True,
                                            workspace=ws)
        out = torch.full_like(tq, float("nan"))
        lse = torch.full((len(lens), hq), float("nan"), dtype=torch.float32, device="cuda")
        lcap.attn_decode_noalloc(tq, tk, tv, cu, mask=mask, scale=scale, out=out, lse=lse)
        torch.cuda.synchronize()
        # the same kernels on the same inputs: identical results
        assert torch.equal(out, ref_out), "output differs from attn_decode"
        assert torch.equal(lse, ref_lse), "lse differs from attn_decode"
        want, want_lse = orc.attention(q, k, v, np.arange(len(lens) + 1), mask, scale,
                                       return_lse=True, cu_seqlens_k=cu_k)
        assert G.max_err(out.double().cpu().numpy(), want) <= G.TOL["bf16"]
        assert G.max_err(lse.double().cpu().numpy(), want_lse) <= G.LSE_TOL["bf16"]
    assert needs[0] > needs[1] > 0, needs
