"""The binding on a stream other than torch's current one: tensors a call
allocates (outputs, workspaces) belong to the stream its kernels run on, so
the caching allocator cannot hand their memory to work on the current stream
while those kernels may still use it.  Each case passes ``stream=s`` (s kept
busy first, so its kernels run late), then allocates and overwrites
same-size tensors on the current stream before synchronising, and checks
that none of them reuses a block the call allocated and that the results
still match the fp64 oracle."""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


@pytest.fixture
def record_allocs(monkeypatch):
    """Data pointers of every tensor torch.empty / empty_like return during the
    call (the binding allocates through these two)."""
    import torch

    seen = []
    empty, empty_like = torch.empty, torch.empty_like

    def rec_empty(*a, **kw):
        t = empty(*a, **kw)
        seen.append((t.data_ptr(), t.numel() * t.element_size()))
        return t

    def rec_empty_like(*a, **kw):
        t = empty_like(*a, **kw)
        seen.append((t.data_ptr(), t.numel() * t.element_size()))
        return t

    monkeypatch.setattr(torch, "empty", rec_empty)
    monkeypatch.setattr(torch, "empty_like", rec_empty_like)
    yield seen
    monkeypatch.setattr(torch, "empty", empty)
    monkeypatch.setattr(torch, "empty_like", empty_like)


def _busy(s):
    """Queue a few milliseconds of unrelated work on s."""
    import torch

    with torch.cuda.stream(s):
        a = torch.ones(4096, 4096, device="cuda")
        for _ in range(8):
            a = a @ a * 1e-4
    return a


def _clobber(allocs):
    """On the current stream: same-size tensors, filled with NaN; none may sit
    in a block the call allocated (those stay with the call's stream)."""
    import torch

    junk = []
    for ptr, nbytes in allocs:
        t = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
        t.fill_(0xFF)
        junk.append(t)
        assert t.data_ptr() not in {p for p, _ in allocs}, "a block of the call was reused"
    return junk


def test_decode_side_stream(orc, record_allocs):
    import torch

    import long_context_attention_prefill_amd as lcap

    lens, hq, hkv, d = [3000, 7000, 1, 4096], 16, 2, 128
    rng = np.random.Generator(np.random.PCG64(71))
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = W.round_to(rng.standard_normal((len(lens), hq, d)), W.BF16)
    k = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    v = W.round_to(rng.standard_normal((int(cu_k[-1]), hkv, d)), W.BF16)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    assert lcap.attn_decode_workspace_size([int(x) for x in cu_k], hq, hkv, d) > 0
    s = torch.cuda.Stream()
    keep = _busy(s)
    record_allocs.clear()
    out, lse = lcap.attn_decode(tq, tk, tv, [int(x) for x in cu_k], lse=True, stream=s)
    allocs = list(record_allocs)
    assert len(allocs) == 3  # out, lse, workspace
    junk = _clobber(allocs)
    s.synchronize()
    torch.cuda.synchronize()
    del keep, junk
    want, want_lse = orc.attention(q, k, v, np.arange(len(lens) + 1), "causal", 1 / math.sqrt(d),
                                   return_lse=True, cu_seqlens_k=cu_k)
    assert G.max_err(out.double().cpu().numpy(), want) <= G.TOL["bf16"]
    assert G.max_err(lse.double().cpu().numpy(), want_lse) <= G.LSE_TOL["bf16"]


def test_gdn_side_stream(record_allocs):
    import torch

    import long_context_attention_prefill_amd as lcap
    from oracle import gdn

    lens, H = [300, 65], 2
    cu = [0, 300, 365]
    q, k, v, g, beta = W.make_gdn_inputs(lens, H, 128, 128, 72)
    dev = [G.to_device(x, "bf16") for x in (q, k, v)]
    gd, bd = (torch.from_numpy(x).to(torch.float32).cuda() for x in (g, beta))
    s = torch.cuda.Stream()
    keep = _busy(s)
    record_allocs.clear()
    out, fin = lcap.gdn_prefill(*dev, gd, bd, cu, final_state=True, stream=s)
    allocs = list(record_allocs)
    assert len(allocs) == 3  # out, final state, workspace
    junk = _clobber(allocs)
    s.synchronize()
    torch.cuda.synchronize()
    del keep, junk
    want, want_fin = gdn.load().gated_delta_rule(q, k, v, g, beta, cu, 1 / math.sqrt(128))
    got = out.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    assert float(np.max(np.abs(got - want))) <= 2.0 ** -5 * float(np.max(np.abs(want)))
    gf = fin.double().cpu().numpy()
    assert float(np.max(np.abs(gf - want_fin))) <= 2.0 ** -5 * float(np.max(np.abs(want_fin)))


def test_vision_side_stream(orc, record_allocs):
    import torch

    import long_context_attention_prefill_amd as lcap
    from oracle import vision

    lens, hidden, H, d = [130, 77], 256, 2, 72
    inputs = W.make_vision_inputs(lens, hidden, H, d, W.BF16, 73)
    dev = [G.to_device(x, "bf16") for x in inputs]
    cu = [0, 130, 207]
    s = torch.cuda.Stream()
    keep = _busy(s)
    record_allocs.clear()
    out = lcap.vision_attention_block(*dev, cu, H, mask="full", stream=s)
    allocs = list(record_allocs)
    assert len(allocs) == 2  # out, workspace
    junk = _clobber(allocs)
    s.synchronize()
    torch.cuda.synchronize()
    del keep, junk
    want = vision.attention_block(orc, *inputs, cu, H, "full", None)
    got = out.double().cpu().numpy()
    err = np.abs(got - want)
    assert float(err.max()) <= 2.0 ** -5 * float(np.max(np.abs(want)))
