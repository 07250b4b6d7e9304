"""gdn_prefill (chunked gated delta rule, HIP) against the fp64 scan oracle,
through the C ABI, on the same seeded inputs.

Tolerance.  The kernels round six operand kinds to bf16 before MFMA products
(within 2^-8 relative each: round to nearest keeps 8 significant bits): the
chunk's inverse system T, the WY combinations W and U, the gated scores P,
the decayed keys, the state S entering each chunk and the corrected values
U'; sums are fp32.  A numpy replay of exactly those
roundings on these input distributions (unit-norm q and k, v ~ N(0, 1),
alpha ~ U(0.85, 1), beta ~ U(0, 1), up to 10240 tokens) stays within 0.8 % of
max |o| (max abs error) and 0.4 % of rms(o) (rms error).  The bars below are
2^-5 of max |o_ref| and 2^-6 of rms(o_ref), a factor 4 over that; a dropped
chunk, a wrong gate or a sign slip moves outputs by tens of percent.  Final
states are held to the same relative bars against their own magnitude.
"""
import math

import numpy as np
import pytest

import gpu_util as G
from long_context_attention_prefill_amd import workloads as W

pytestmark = pytest.mark.gpu

MAX_REL = 2.0 ** -5
RMS_REL = 2.0 ** -6


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch

    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import long_context_attention_prefill_amd as lcap

    lcap.load_library()


@pytest.fixture(scope="module")
def gdn_orc():
    from oracle import gdn

    return gdn.load()


def _dev(x, dtype):
    return G.to_device(x, dtype)


def _run(q, k, v, g, beta, cu, scale, s0=None, want_state=True, workspace=None):
    import torch

    import long_context_attention_prefill_amd as lcap

    tq, tk, tv = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    tg, tb = _dev(g, "f32"), _dev(beta, "f32")
    ts0 = None if s0 is None else _dev(s0.astype(np.float32).astype(np.float64), "f32")
    res = lcap.gdn_prefill(tq, tk, tv, tg, tb, [int(x) for x in cu], scale=scale,
                           initial_state=ts0, final_state=want_state, workspace=workspace)
    torch.cuda.synchronize()
    if want_state:
        out, fin = res
        return out.double().cpu().numpy(), fin.double().cpu().numpy()
    return res.double().cpu().numpy(), None


def _assert_close(got, want, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    if want.size == 0:
        return
    err = np.abs(got - want)
    mx = float(np.max(np.abs(want)))
    rms = float(np.sqrt(np.mean(want ** 2)))
    assert float(err.max()) <= MAX_REL * mx + 1e-30, f"{what}: max err {err.max():.3e} vs max|ref| {mx:.3e}"
    assert float(np.sqrt(np.mean(err ** 2))) <= RMS_REL * rms + 1e-30, \
        f"{what}: rms err {np.sqrt(np.mean(err ** 2)):.3e} vs rms(ref) {rms:.3e}"


def _state0(n, H, seed, scale=0.3):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (scale * rng.standard_normal((n, H, 128, 128))).astype(np.float32).astype(np.float64)


def _check(gdn_orc, lens, H, seed, with_s0, scale=None):
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, v, g, beta = W.make_gdn_inputs(lens, H, 128, 128, seed)
    scale = 1 / math.sqrt(128) if scale is None else scale
    s0 = _state0(len(lens), H, seed + 100) if with_s0 else None
    got, fin = _run(q, k, v, g, beta, cu, scale, s0=s0)
    want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale, initial_state=s0)
    _assert_close(got, want, "outputs")
    _assert_close(fin, want_fin, "final state")


@pytest.mark.parametrize("lens", [[1], [63], [64], [65], [200], [37, 64, 200, 1, 130]], ids=str)
@pytest.mark.parametrize("with_s0", [False, True], ids=["zero_state", "initial_state"])
def test_gdn_small(gdn_orc, lens, with_s0):
    _check(gdn_orc, lens, 3, seed=len(lens) * 7 + sum(lens), with_s0=with_s0)


@pytest.mark.parametrize("H", [1, 2, 16])
def test_gdn_heads(gdn_orc, H):
    _check(gdn_orc, [300, 129], H, seed=40 + H, with_s0=True)


@pytest.mark.parametrize("scale", [1.0, 0.05])
def test_gdn_scales(gdn_orc, scale):
    _check(gdn_orc, [190], 2, seed=50, with_s0=True, scale=scale)


def test_gdn_empty_sequences_pass_state_through(gdn_orc):
    """Sequences without tokens hand their initial state over unchanged."""
    _check(gdn_orc, [0, 70, 0, 0, 5], 2, seed=60, with_s0=True)
    lens = [0, 0]
    s0 = _state0(2, 2, 61)
    z = np.zeros((0, 2, 128))
    got, fin = _run(z, z, z, np.zeros((0, 2)), np.zeros((0, 2)), [0, 0, 0], 0.1, s0=s0)
    assert got.shape == (0, 2, 128)
    assert np.array_equal(fin, s0)


def test_gdn_many_sequences(gdn_orc):
    """More than 64 sequences: several launches share the workspace in order."""
    rng = np.random.Generator(np.random.PCG64(70))
    lens = rng.integers(0, 150, 90).tolist()
    _check(gdn_orc, lens, 2, seed=71, with_s0=True)


def test_gdn_state_in_place_and_split_sequence(gdn_orc):
    """final_state may be initial_state itself; a sequence run as two calls
    with the state handed over equals one call (and the oracle)."""
    import torch

    import long_context_attention_prefill_amd as lcap

    lens = [500]
    cu = [0, 500]
    q, k, v, g, beta = W.make_gdn_inputs(lens, 2, 128, 128, 80)
    s0 = _state0(1, 2, 81)
    scale = 1 / math.sqrt(128)
    want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale, initial_state=s0)
    tq, tk, tv = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    tg, tb = _dev(g, "f32"), _dev(beta, "f32")
    state = _dev(s0, "f32")
    outs = []
    for a, b in ((0, 200), (200, 500)):  # the cut is not a multiple of 64
        o = lcap.gdn_prefill(tq[a:b], tk[a:b], tv[a:b], tg[a:b], tb[a:b], [0, b - a],
                             scale=scale, initial_state=state, final_state=state)[0]
        outs.append(o)
    torch.cuda.synchronize()
    got = torch.cat(outs).double().cpu().numpy()
    _assert_close(got, want, "outputs over two calls")
    _assert_close(state.double().cpu().numpy(), want_fin, "state over two calls")


def test_gdn_without_states_and_determinism(gdn_orc):
    import torch

    import long_context_attention_prefill_amd as lcap

    lens = [333, 64]
    cu = [0, 333, 397]
    q, k, v, g, beta = W.make_gdn_inputs(lens, 4, 128, 128, 90)
    scale = 1 / math.sqrt(128)
    want, _ = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale)
    a, _ = _run(q, k, v, g, beta, cu, scale, want_state=False)
    b, _ = _run(q, k, v, g, beta, cu, scale, want_state=False)
    _assert_close(a, want, "outputs")
    assert np.array_equal(a, b), "two runs differ"


def test_gdn_workspace_reuse(gdn_orc):
    """One workspace for a large call and then a smaller one."""
    import torch

    import long_context_attention_prefill_amd as lcap

    need = lcap.gdn_prefill_workspace_size([0, 1000], 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    for lens, seed in (([1000], 91), ([70, 20], 92)):
        cu = np.concatenate([[0], np.cumsum(lens)])
        q, k, v, g, beta = W.make_gdn_inputs(lens, 4, 128, 128, seed)
        got, fin = _run(q, k, v, g, beta, cu, 0.1, workspace=ws)
        want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, 0.1)
        _assert_close(got, want, f"outputs {lens}")
        _assert_close(fin, want_fin, f"final state {lens}")


@pytest.mark.parametrize("name", sorted(W.GDN_WORKLOADS))
def test_gdn_workloads_full_size(gdn_orc, name):
    """The bench workloads at full size, every output and final state."""
    spec = W.GDN_WORKLOADS[name]
    lens = spec["lens"]
    cu = np.concatenate([[0], np.cumsum(lens)])
    q, k, v, g, beta = W.make_gdn_inputs(lens, spec["n_heads"], spec["dk"], spec["dv"], spec["seed"])
    scale = 1 / math.sqrt(spec["dk"])
    got, fin = _run(q, k, v, g, beta, cu, scale)
    want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale)
    _assert_close(got, want, "outputs")
    _assert_close(fin, want_fin, "final state")


@pytest.mark.parametrize("lens", [[4096], [4100, 0, 70], [9000, 130]], ids=str)
@pytest.mark.parametrize("with_s0", [False, True], ids=["zero_state", "initial_state"])
def test_gdn_long_and_ragged(gdn_orc, lens, with_s0):
    """Sequences of 64 to 141 chunks (one ending one token into a chunk),
    packed with short and empty ones."""
    _check(gdn_orc, lens, 2, seed=sum(lens) % 1000, with_s0=with_s0)


def test_gdn_long_state_in_place(gdn_orc):
    """A long sequence updating the state in place, then run without any state."""
    import torch

    import long_context_attention_prefill_amd as lcap

    lens = [4200, 300]
    cu = [0, 4200, 4500]
    q, k, v, g, beta = W.make_gdn_inputs(lens, 2, 128, 128, 95)
    s0 = _state0(2, 2, 96)
    scale = 1 / math.sqrt(128)
    want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale, initial_state=s0)
    tq, tk, tv = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    tg, tb = _dev(g, "f32"), _dev(beta, "f32")
    state = _dev(s0, "f32")
    out = lcap.gdn_prefill(tq, tk, tv, tg, tb, cu, scale=scale, initial_state=state, final_state=state)[0]
    torch.cuda.synchronize()
    _assert_close(out.double().cpu().numpy(), want, "outputs")
    _assert_close(state.double().cpu().numpy(), want_fin, "state in place")
    want0, _ = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale)
    got0, _ = _run(q, k, v, g, beta, cu, scale, want_state=False)
    _assert_close(got0, want0, "outputs without states")


def _check_gates(gdn_orc, lens, H, seed, decays, with_s0=True):
    """Like _check, with the decay of sequence b drawn from decays[b]: strong
    gates (alpha down to 0.001) drive the cumulative log-gate of a 64-token
    chunk far below fp32's exponent range, where only ratios of gates
    (differences of log-gates) stay finite."""
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q, k, v, g, beta = W.make_gdn_inputs(lens, H, 128, 128, seed)
    rng = np.random.Generator(np.random.PCG64(seed + 1))
    for b, (lo, hi) in enumerate(decays):
        s, e = int(cu[b]), int(cu[b + 1])
        alpha = rng.uniform(lo, hi, (e - s, H))
        g[s:e] = W.round_to(np.log(alpha), W.F32)
    scale = 1 / math.sqrt(128)
    s0 = _state0(len(lens), H, seed + 100) if with_s0 else None
    got, fin = _run(q, k, v, g, beta, cu, scale, s0=s0)
    want, want_fin = gdn_orc.gated_delta_rule(q, k, v, g, beta, cu, scale, initial_state=s0)
    _assert_close(got, want, f"outputs, decays {decays}")
    _assert_close(fin, want_fin, f"final state, decays {decays}")


@pytest.mark.parametrize("decay", [(0.01, 1.0), (0.001, 0.05)], ids=str)
@pytest.mark.parametrize("lens", [[200], [37, 64, 130], [1000]], ids=str)
def test_gdn_strong_decay(gdn_orc, lens, decay):
    _check_gates(gdn_orc, lens, 2, seed=300 + sum(lens), decays=[decay] * len(lens))


def test_gdn_mixed_strong_and_weak_gates(gdn_orc):
    """One batch whose sequences alternate strong and weak gates."""
    lens = [130, 200, 64, 300, 1]
    decays = [(0.001, 0.05), (0.85, 1.0), (0.01, 1.0), (0.95, 1.0), (0.001, 0.01)]
    _check_gates(gdn_orc, lens, 3, seed=400, decays=decays)
