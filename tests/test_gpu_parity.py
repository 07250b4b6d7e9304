"""HIP path vs the fp64 oracle, element by element, through the C ABI.

Tolerances: max abs error 2e-2 for bf16 inputs, 1e-4 for fp32 inputs, over
every compared element.  Mask and index handling is checked bit-exactly by
the probes (expected integers from the mask definitions, at full size).
"""
import math
import zlib

import numpy as np
import pytest

import gpu_util as G
import probes
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()
    print(f"\n[gpu] {torch.cuda.get_device_name(0)}", flush=True)


LAYOUTS = {
    "one-short": [0, 5],
    "one-tile": [0, 128],
    "ragged": [0, 129],
    "multi": [0, 300, 300, 301, 777],
    "empties": [0, 0, 64, 64, 200, 200],
}
MASKS = ["causal", "full", ("window", 1), ("window", 7), ("window", 64), ("window", 100),
         ("window", 256)]


def _case(cu, hq, hkv, d, dtype, seed):
    q, k, v = W.draw_qkv(np.array(cu), hq, hkv, d, dtype, 1.0, seed)
    return q, k, v


@pytest.mark.parametrize("layout", sorted(LAYOUTS))
@pytest.mark.parametrize("mask", MASKS, ids=str)
@pytest.mark.parametrize("d", [64, 72, 128])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_parity(orc, dtype, d, mask, layout):
    cu = LAYOUTS[layout]
    hq, hkv = (4, 2) if d != 72 else (3, 1)
    q, k, v = _case(cu, hq, hkv, d, dtype, seed=zlib.crc32(f"{dtype}{d}{mask}{layout}".encode()) % 10000)
    scale = 1.0 / math.sqrt(d)
    want = orc.attention(q, k, v, cu, mask, scale)
    got = G.run_hip(q, k, v, cu, mask, scale, dtype)
    err = G.max_err(got, want)
    assert err <= G.TOL[dtype], f"max abs err {err:.3e}"


@pytest.mark.parametrize("seed", range(40))
def test_fuzz_bf16(orc, seed):
    c = W.random_case(seed, dtype="bf16")
    want = orc.attention(c["q"], c["k"], c["v"], c["cu"], c["mask"], c["scale"])
    got = G.run_hip(c["q"], c["k"], c["v"], c["cu"], c["mask"], c["scale"], "bf16")
    assert G.max_err(got, want) <= G.TOL["bf16"], (c["cu"].tolist(), c["mask"], c["d"])


@pytest.mark.parametrize("seed", range(16))
def test_fuzz_f32(orc, seed):
    c = W.random_case(1000 + seed, dtype="f32")
    want = orc.attention(c["q"], c["k"], c["v"], c["cu"], c["mask"], c["scale"])
    got = G.run_hip(c["q"], c["k"], c["v"], c["cu"], c["mask"], c["scale"], "f32")
    assert G.max_err(got, want) <= G.TOL["f32"], (c["cu"].tolist(), c["mask"], c["d"])


# bf16: 0, -0.1 and 0.15 run the prescaled-query kernels (|scale log2 e| <=
# 0.25), -0.3 and 2.5 the exact-query ones
@pytest.mark.parametrize("scale", [0.0, -0.1, 0.15, -0.3, 2.5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_unusual_scales(orc, dtype, scale):
    cu = [0, 200, 450]
    q, k, v = _case(cu, 2, 1, 64, dtype, seed=77)
    for mask in ("causal", ("window", 33)):
        want = orc.attention(q, k, v, cu, mask, scale)
        got = G.run_hip(q, k, v, cu, mask, scale, dtype)
        assert G.max_err(got, want) <= G.TOL[dtype], mask


# ---------------------------------------------------------------- workloads

def _sample_rows(cu, hq, rng, per_seq=12):
    rows = []
    for b in range(len(cu) - 1):
        s, n = int(cu[b]), int(cu[b + 1] - cu[b])
        pick = {0, 1, n // 2, n - 2, n - 1} | set(rng.integers(0, n, per_seq).tolist())
        rows += [s + i for i in sorted(pick) if 0 <= i < n]
    rows = np.array(rows)
    return np.repeat(rows, hq), np.tile(np.arange(hq), rows.size)


@pytest.mark.parametrize("name", ["1", "2", "3", "4", "5a", "5b"])
def test_workload_parity(orc, name):
    """Element by element against the oracle: every element up to 2048 tokens;
    beyond, every row of one query head per key/value head (heads 0 and 8 at
    16/2 heads) and sampled rows (first, last, middle, random) of every head."""
    w = W.WORKLOADS[name]
    q, k, v, cu = W.make_inputs(w)
    print(f"[workload {name}] {w.name}", flush=True)
    got = G.run_hip(q, k, v, cu, w.mask, w.scale, w.dtype)
    if w.total_tokens <= 2048:
        want = orc.attention(q, k, v, cu, w.mask, w.scale)
        err = G.max_err(got, want)
    else:
        group = w.n_q_heads // w.n_kv_heads
        full_heads = np.arange(w.n_kv_heads) * group
        T = w.total_tokens
        rows = np.repeat(np.arange(T), full_heads.size)
        heads = np.tile(full_heads, T)
        want = orc.attention_rows(q, k, v, cu, w.mask, w.scale, rows, heads)
        err = G.max_err(got[rows, heads], want)
        assert err <= G.TOL[w.dtype], f"{name}: heads {full_heads.tolist()}, every row: {err:.3e}"
        rows, heads = _sample_rows(cu, w.n_q_heads, np.random.Generator(np.random.PCG64(5)))
        want = orc.attention_rows(q, k, v, cu, w.mask, w.scale, rows, heads)
        err = G.max_err(got[rows, heads], want)
    assert err <= G.TOL[w.dtype], f"{name}: max abs err {err:.3e}"
    if w.needle_pos is not None:
        import pins

        pins.check_needle(got[w.total_tokens - 1], w)


@pytest.mark.parametrize("name", ["1", "2", "3", "4", "5a", "5b"])
def test_workload_probe_count(name):
    """Every row of the full-size shape: exact count of visible keys per class."""
    w = W.WORKLOADS[name]
    cu = np.array(w.cu_seqlens)
    q, k, v = W.probe_count_inputs(cu, w.n_q_heads, w.n_kv_heads, w.head_dim)
    got = G.run_hip(q, k, v, cu, w.mask, w.scale, w.dtype)
    probes.check_count_output(got, cu, w.mask, w.head_dim)


@pytest.mark.parametrize("sign", [1, -1])
@pytest.mark.parametrize("name", ["1", "3", "4", "5a", "5b"])
def test_workload_probe_index(name, sign):
    """Every row: exact first (sign -1) or last (sign +1) visible key and KV head."""
    w = W.WORKLOADS[name]
    cu = np.array(w.cu_seqlens)
    hq, hkv = w.n_q_heads, w.n_kv_heads
    q, k, v = W.probe_index_inputs(cu, hq, hkv, w.head_dim, sign)
    got = G.run_hip(q, k, v, cu, w.mask, w.scale, w.dtype)
    probes.check_index_output(got, cu, w.mask, hq, hkv, sign)


def test_determinism():
    w = W.WORKLOADS["5a"]
    q, k, v, cu = W.make_inputs(w)
    a = G.run_hip(q, k, v, cu, w.mask, w.scale, w.dtype)
    b = G.run_hip(q, k, v, cu, w.mask, w.scale, w.dtype)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------- boundary

def test_empty_batches():
    import torch

    import long_context_attention_prefill_amd as lcap

    for dt in (torch.bfloat16, torch.float32):
        z = torch.empty((0, 4, 64), dtype=dt, device="cuda")
        zk = torch.empty((0, 2, 64), dtype=dt, device="cuda")
        assert lcap.attn_prefill(z, zk, zk, [0]).shape == (0, 4, 64)
        assert lcap.attn_prefill(z, zk, zk, [0, 0, 0], mask="full").shape == (0, 4, 64)


def test_errors_leave_output_untouched():
    import torch

    import long_context_attention_prefill_amd as lcap

    q = torch.randn(64, 2, 64, device="cuda").to(torch.bfloat16)
    k = torch.randn(64, 1, 64, device="cuda").to(torch.bfloat16)
    out = torch.full_like(q, 7.0)
    with pytest.raises(lcap.AttnError) as e:
        lcap.attn_prefill(q, k, k, [0, 64], mask=("window", 0), out=out)
    assert e.value.status == lcap.ATTN_EINVAL
    with pytest.raises(lcap.AttnError) as e:
        lcap.attn_prefill(q, k, k, [0, 64], scale=float("nan"), out=out)
    assert e.value.status == lcap.ATTN_EINVAL
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
    # out aliasing an input
    with pytest.raises(lcap.AttnError) as e:
        lcap.attn_prefill(q, k, k, [0, 64], out=q)
    assert e.value.status == lcap.ATTN_EINVAL


def test_misaligned_pointer_rejected():
    import ctypes

    import torch

    import long_context_attention_prefill_amd as lcap

    lib = lcap.load_library()
    buf = torch.zeros(4 * 64 * 2 + 8, dtype=torch.bfloat16, device="cuda")
    cu = (ctypes.c_int32 * 2)(0, 4)
    p = buf.data_ptr()
    st = lib.attn_prefill(p + 2, p, p, p + 4 * 64 * 4, cu, 1, 1, 1, 64, lcap.ATTN_BF16,
                          lcap.ATTN_CAUSAL, 0, 0.125, None)
    assert st == lcap.ATTN_EINVAL


def test_side_stream(orc):
    import torch

    import long_context_attention_prefill_amd as lcap

    cu = [0, 333]
    q, k, v = _case(cu, 2, 2, 128, "bf16", seed=5)
    tq, tk, tv = (G.to_device(x, "bf16") for x in (q, k, v))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        out = lcap.attn_prefill(tq, tk, tv, cu)
    s.synchronize()
    want = orc.attention(q, k, v, cu, "causal", 1 / math.sqrt(128))
    assert G.max_err(out.double().cpu().numpy(), want) <= G.TOL["bf16"]
