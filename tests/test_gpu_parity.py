"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Exact-sum inputs (every FP32 partial sum exact) and closed forms must match
bit for bit whatever the kernel's summation order; random seeded inputs of
the configurations' shapes and distributions must pass the G1/G2/D1 gates.
Every output of every full-shape case is compared: the oracle computes all
B x N elements, no column sample.
"""
import numpy as np
import pytest
import torch

import oracle
import tp1_skinny_bf16_amd as tp
import workloads as wl
from gpu_util import (DEV, candidate_tactics, check_exact, check_random, gpu_run, say,
                      tactic_label)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    torch.cuda.set_device(DEV)


# ---------------------------------------------------------------- small shapes
SMALL = [(1000, 1032), (77, 520), (33, 8)]      # ragged N, K not a multiple of 512
BINS = [1, 2, 4, 8, 16, 32, 64, 128, 256]


@pytest.mark.parametrize("N,K", SMALL)
def test_every_tactic_exact_on_small_shapes(N, K):
    x, W = wl.exact_sum_case(256, N, K, seed=N + K)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    tried = 0
    for bin_ in BINS:
        for t in candidate_tactics(N, K, bin_):
            try:
                plan.set_tactic(bin_, t)
            except tp.ProjError:
                continue                      # e.g. the x slice exceeds the LDS
            for B in sorted({bin_, max(1, bin_ // 2 + 1)}):
                y = gpu_run(plan, x[:B], Wd)
                check_exact(f"N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)
                tried += 1
    say(f"{tried} tactic/batch combinations exact")


@pytest.mark.parametrize("N,K", SMALL)
def test_default_tactics_random_small(N, K):
    x, W = wl.random_case(256, N, K, seed=7)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    for B in [1, 2, 3, 5, 8, 13, 16, 17, 31, 64, 100, 256]:
        y = gpu_run(plan, x[:B], Wd)
        check_random(f"N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)


# ------------------------------------------------------------ full-size configs
_CACHE = {}


def _config(name):
    if name not in _CACHE:
        _CACHE.clear()
        cfg = wl.BY_NAME[name]
        t = wl.config_tensors(cfg)
        _CACHE[name] = (cfg, t, t["W"].to(DEV))
    return _CACHE[name]


FULL_POINTS = [(c.name, B) for c in wl.CONFIGS if c.layers == 1 for B in c.batches]


@pytest.mark.parametrize("name,B", FULL_POINTS)
def test_full_config_random(name, B):
    cfg, t, Wd = _config(name)
    plan = tp.Plan(cfg.N, cfg.K, cfg.batches)
    say(f"{name} B={B}: {tactic_label(plan, B)}")
    y = gpu_run(plan, t["x"][:B], Wd)
    check_random(f"{name} B={B}", y, t["x"][:B], t["W"])        # every output


def _structured_inputs(N, K, B, seed):
    """Inputs unlike the configurations' (every output still gated):
    x scaled by 1e3 and W by 1e-3 of the usual spread, so products keep their
    size but every operand sits ~10 binades away; half of x's entries exact
    zeros; row 0 all +0, row 1 all -0, and row 5 a copy of row 2."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    W = wl.normal_bf16((N, K), wl.W_STD * 1e-3, g)
    x = wl.normal_bf16((B, K), 1e3, g)
    keep = torch.rand((B, K), generator=g) < 0.5
    x = torch.where(keep, x, torch.zeros_like(x))
    x[0] = 0.0
    x[1] = -0.0
    x[5] = x[2]
    return x, W


@pytest.mark.parametrize("N,K", [(wl.DSA_N, wl.DSA_K), (wl.OPROJ_N, wl.OPROJ_K),
                                 (wl.KDA_N, wl.KDA_K)])
def test_structured_inputs_full_shape(N, K):
    """Scaled, sparse and degenerate rows at full shape through the planned
    tactics of B = 8, 16, 64 and 256: every output against the oracle's gates,
    the zero rows +0 bit for bit (both sides start their sums from +0), and a
    repeated row repeated bit for bit."""
    x, W = _structured_inputs(N, K, 256, seed=N + K + 101)
    assert x[1].view(torch.int16).eq(-32768).all()          # really -0
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    for B in (8, 16, 64, 256):
        y = gpu_run(plan, x[:B], Wd)
        check_random(f"structured N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)
        assert (y[0] == 0).all() and (y[1] == 0).all(), "zero rows must give +0"
        assert np.array_equal(y[2], y[5]), "a repeated row must repeat its outputs"


VERIFY_BINS = [3, 6, 12, 24, 48, 96, 192]   # requests x (1 + speculative tokens)


@pytest.mark.parametrize("N,K", [(wl.DSA_N, wl.DSA_K), (wl.OPROJ_N, wl.OPROJ_K)])
def test_verify_step_batches_full_shape(N, K):
    """Plans listing verify-step batches (not powers of two) borrow the next
    measured bin's tactic; every bin, and a batch below its bin, is exact on
    exact-sum inputs."""
    x, W = wl.exact_sum_case(192, N, K, seed=13)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, VERIFY_BINS)
    for b in VERIFY_BINS:
        for B in sorted({b, b - 1}):
            y = gpu_run(plan, x[:B], Wd)
            check_exact(f"verify N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)


@pytest.mark.parametrize("N,K", [(wl.DSA_N, wl.DSA_K), (wl.OPROJ_N, wl.OPROJ_K),
                                 (wl.KDA_N, wl.KDA_K)])
def test_full_shape_exact_sum_every_planned_tactic(N, K):
    x, W = wl.exact_sum_case(256, N, K, seed=11)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    for B in BINS:
        y = gpu_run(plan, x[:B], Wd)
        check_exact(f"N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)


@pytest.mark.parametrize("N,K", [(wl.DSA_N, wl.DSA_K), (wl.OPROJ_N, wl.OPROJ_K),
                                 (wl.KDA_N, wl.KDA_K)])
def test_one_hot_weight_full_shape(N, K):
    # W[n, k] = 2^-3 [k == n mod K]: y[b, n] = x[b, n mod K] / 8 exactly.
    W = wl.one_hot_weight(N, K, 0.125)
    Wd = W.to(DEV)
    x, _ = wl.random_case(256, 8, K, seed=3)
    plan = tp.Plan(N, K, BINS)
    n = np.arange(N)
    for B in (1, 5, 16, 64, 256):
        y = gpu_run(plan, x[:B], Wd)
        want = wl.bits((x[:B, torch.as_tensor(n % K)].float() * 0.125).to(torch.bfloat16))
        bad = np.argwhere(y != want)
        say(f"one-hot N={N} K={K} B={B} {tactic_label(plan, B)}: {len(bad)} mismatches")
        assert bad.size == 0


def test_closed_forms_on_gpu():
    for K, wval, want in [(7168, 2.0 ** -10, 7.0), (12288, 2.0 ** -12, 3.0)]:
        W = torch.full((300, K), wval, dtype=torch.bfloat16)
        x = torch.ones((16, K), dtype=torch.bfloat16)
        x[1::2] = -1
        plan = tp.Plan(300, K, [1, 4, 16])
        for B in (1, 4, 16):
            y = gpu_run(plan, x[:B], W.to(DEV))
            exp = np.where(np.arange(B)[:, None] % 2 == 1, -want, want)
            got = wl.from_bits(y).float().numpy()
            assert np.array_equal(got, np.broadcast_to(exp, got.shape)), (K, B)


def test_golden_ties_on_gpu():
    import pins
    for xs, ws, want in pins.load_golden_ties():
        K = 8                                  # pad the K < 8 cases with zeros
        xb = np.zeros((1, K), dtype=np.uint16)
        wb = np.zeros((3, K), dtype=np.uint16)
        xb[0, :len(xs)] = xs
        wb[:, :len(ws)] = ws
        for bin_ in (1, 16):
            plan = tp.Plan(3, K, [bin_])
            y = gpu_run(plan, wl.from_bits(xb), wl.from_bits(wb).to(DEV))
            assert all(int(v) == want for v in y[0]), (xs, ws, [hex(v) for v in y[0]], hex(want))


def test_determinism_and_invariants():
    """Bitwise reproducibility and power-of-two scaling on every path; exact
    negation where the sums are IEEE FP32 (the stream kernel's FMAs).  The
    MFMA units add their products with a rounding that is not symmetric in
    sign (measured), so on MFMA tactics y(-x) is held to the parity gates."""
    N, K = wl.DSA_N, wl.DSA_K
    x, W = wl.random_case(64, N, K, seed=5)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    for B in (1, 4, 8, 16, 64):
        y1 = gpu_run(plan, x[:B], Wd)
        y2 = gpu_run(plan, x[:B], Wd)
        assert np.array_equal(y1, y2), f"B={B} not deterministic"
        y4 = gpu_run(plan, (x[:B].float() * 4).to(torch.bfloat16), Wd)
        assert np.array_equal(wl.from_bits(y4).float().numpy(),
                              wl.from_bits(y1).float().numpy() * 4), f"B={B} scaling"
        yn = gpu_run(plan, -x[:B], Wd)
        t, _ = plan.tactic(B)
        if t.kernel == tp.KERNEL_STREAM:
            assert np.array_equal(wl.from_bits(yn).float().numpy(),
                                  -wl.from_bits(y1).float().numpy()), f"B={B} negation"
        else:
            check_random(f"B={B} negated x", yn, -x[:B], W)
        say(f"B={B} deterministic, scaling exact, negation ok ({tactic_label(plan, B)})")


def test_edge_cases():
    N, K = 515, 264
    x, W = wl.random_case(40, N, K, seed=9)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, [4, 32])
    # B == 0: a no-op that leaves the output untouched
    y = torch.full((1, N), 7.0, dtype=torch.bfloat16, device=DEV)
    assert plan.run_ptr(0, Wd.data_ptr(), K, Wd.data_ptr(), y.data_ptr()) == tp.PROJ_OK
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    # batches below their bin, and x read through a row stride (a gather)
    for B in (1, 3, 4, 5, 31, 32):
        for pad in (0, 24):
            yb = gpu_run(plan, x[:B], Wd, ldx_pad=pad)
            check_random(f"edge B={B} pad={pad} {tactic_label(plan, B)}", yb, x[:B], W)
    # batch above the largest bin is refused
    with pytest.raises(tp.ProjError):
        gpu_run(plan, x[:33], Wd)
    # minimal shapes
    for (n, k) in ((1, 8), (1, 4096), (16, 8), (17, 40)):
        xs, Ws = wl.random_case(20, n, k, seed=n * k)
        p = tp.Plan(n, k, [1, 2, 16, 20])
        for B in (1, 2, 16, 20):
            check_random(f"tiny n={n} k={k} B={B}", gpu_run(p, xs[:B], Ws.to(DEV)), xs[:B], Ws)


def test_side_stream_and_returned_tensor():
    N, K = 2048, 1024
    x, W = wl.random_case(8, N, K, seed=2)
    plan = tp.Plan(N, K, [8])
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        xd, Wd = x.to(DEV), W.to(DEV)
        out = plan.run(xd, Wd)                 # uses the current (side) stream
    s.synchronize()
    check_random("side stream", wl.bits(out.cpu()), x, W)


def test_multilayer_stream_per_layer_parity():
    cfg = wl.BY_NAME["multilayer"]
    t = wl.config_tensors(cfg)
    B = cfg.bmax
    pin = tp.Plan(wl.DSA_N, wl.DSA_K, [B])
    po = tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [B])
    w_in = [w.to(DEV) for w in t["W_in"]]
    w_o = [w.to(DEV) for w in t["W_o"]]
    stack = tp.LayerStack(pin, po, w_in, w_o)
    y_in, y_o = stack.run(t["x"].to(DEV))
    torch.cuda.synchronize()
    y_in, y_o = y_in.cpu(), y_o.cpu()
    x_l = t["x"]
    for l in range(cfg.layers):
        # each layer is checked on its own GPU input (tolerances scale)
        yi = wl.bits(y_in[l])
        check_random(f"layer {l} in-proj", yi, x_l, t["W_in"][l])
        xo = y_in[l][:, :wl.OPROJ_K]
        check_random(f"layer {l} o_proj", wl.bits(y_o[l]), xo, t["W_o"][l])
        x_l = y_o[l]
    say(f"final |y| rms = {float(y_o[-1].float().pow(2).mean().sqrt()):.4g}")


@pytest.mark.parametrize("B", [37, 5])
def test_layer_chain_ragged_batch(B):
    """The chain at a batch inside a bin (B rows of a 16- or 64-row tile): the
    padded rows of every tile, the gather through the in-projection's row
    stride and the split-K passes at B < bin, per layer on the GPU's own
    layer input."""
    L = 2
    g = torch.Generator().manual_seed(90 + B)
    w_in = [wl.normal_bf16((wl.DSA_N, wl.DSA_K), wl.W_STD, g) for _ in range(L)]
    w_o = [wl.normal_bf16((wl.OPROJ_N, wl.OPROJ_K), wl.W_STD, g) for _ in range(L)]
    x0 = wl.normal_bf16((B, wl.DSA_K), wl.X_STD, g)
    pin = tp.Plan(wl.DSA_N, wl.DSA_K, [16, 64])
    po = tp.Plan(wl.OPROJ_N, wl.OPROJ_K, [16, 64])
    say(f"chain B={B}: {pin.kernel_name(B)} / {po.kernel_name(B)}")
    stack = tp.LayerStack(pin, po, [w.to(DEV) for w in w_in], [w.to(DEV) for w in w_o])
    y_in, y_o = stack.run(x0.to(DEV))
    torch.cuda.synchronize()
    y_in, y_o = y_in.cpu(), y_o.cpu()
    x_l = x0
    for l in range(L):
        check_random(f"chain B={B} layer {l} in-proj", wl.bits(y_in[l]), x_l, w_in[l])
        check_random(f"chain B={B} layer {l} o_proj", wl.bits(y_o[l]),
                     y_in[l][:, :wl.OPROJ_K], w_o[l])
        x_l = y_o[l]


def test_fused_split_matches_two_pass_bitwise():
    """The in-kernel split-K reduction (last workgroup to arrive sums the
    slices) and the two-pass reduction add the slices in the same order, so
    they agree bit for bit; repeated calls also check that the arrival
    counters are left at zero."""
    N, K = 2000, 3072
    x, W = wl.random_case(64, N, K, seed=21)
    Wd = W.to(DEV)
    fused = tp.Plan(N, K, [4, 16, 64], fused_split=True)
    twop = tp.Plan(N, K, [4, 16, 64])
    tactics = [(4, tp.Tactic(tp.KERNEL_STREAM, 4, 3, 2, 4, 8)),
               (4, tp.Tactic(tp.KERNEL_STREAM_DOT2, 4, 2, 4, 2, 4)),
               (16, tp.Tactic(tp.KERNEL_MFMA_XS, 16, 4, 8, 1, 2, 128, 1)),
               (64, tp.Tactic(tp.KERNEL_MFMA_XS, 64, 3, 4, 4, 2, 128, 1)),
               (16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 4, 4, 1, 2, 128, 4, 1, 4)),
               (16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 2, 2, 1, 1, 256, 4, 2, 4)),
               (64, tp.Tactic(tp.KERNEL_MFMA_PIPE, 64, 3, 8, 2, 2, 64, 4, 1, 4)),
               (64, tp.Tactic(tp.KERNEL_MFMA_PIPE, 64, 4, 16, 2, 1, 64, 3, 1, 8)),
               (16, tp.Tactic(tp.KERNEL_MFMA_PIPE, 16, 3, 2, 1, 1, 256, 4, 4, 8, stagger=1)),
               (64, tp.Tactic(tp.KERNEL_MFMA_XS, 64, 2, 4, 2, 1, 128, 2, stagger=1))]
    for bin_, t in tactics:
        fused.set_tactic(bin_, t)
        twop.set_tactic(bin_, t)
        assert "+splitk_reduce" not in fused.kernel_name(bin_)
        assert "+splitk_reduce" in twop.kernel_name(bin_)
        for B in (bin_, max(1, bin_ - 3)):
            a1 = gpu_run(fused, x[:B], Wd)
            a2 = gpu_run(fused, x[:B], Wd)
            b1 = gpu_run(twop, x[:B], Wd)
            assert np.array_equal(a1, a2), f"{t} B={B}: fused not reproducible"
            assert np.array_equal(a1, b1), f"{t} B={B}: fused != two-pass"
            check_random(f"fused split {tactic_label(fused, B)} B={B}", a1, x[:B], W)


@pytest.mark.parametrize("N,K", [(wl.DSA_N, wl.DSA_K), (wl.OPROJ_N, wl.OPROJ_K)])
def test_fused_split_bitwise_at_full_shapes(N, K):
    """The planned split tactics of B = 64, 128 and 256 at full shape (the
    8-layer stream uses those of B = 64) under the in-kernel reduction: bit
    for bit the two-pass result.  Two inputs in turn: a counter left non-zero
    by one call would send the next call's sum to the wrong workgroup."""
    bins = [64, 128, 256]
    x1, W = wl.random_case(256, N, K, seed=31)
    x2 = wl.random_case(256, N, K, seed=32)[0]
    Wd = W.to(DEV)
    fused = tp.Plan(N, K, bins, fused_split=True)
    twop = tp.Plan(N, K, bins)
    for B in (64, 128, 256, 61):
        assert "+splitk_reduce" not in fused.kernel_name(B)
        for xx in (x1, x2, x1):
            a = gpu_run(fused, xx[:B], Wd)
            b = gpu_run(twop, xx[:B], Wd)
            assert np.array_equal(a, b), f"N={N} B={B}: fused != two-pass"
        check_random(f"fused split N={N} K={K} B={B} {tactic_label(fused, B)}", a, x1[:B], W)


# Per-GPU shards of a G-way tensor-parallel step (the vLLM API page
# "vllm.models.kimi_k3.nvidia.specialized_decode.runtime.hybrid", section
# "HybridAttention"): the input projections column-sharded (N/G x K), o_proj
# row-sharded (N x K/G), G = 2, 4, 8.  Each shape has its own measured table.
TP_SHARDS = [(wl.DSA_N // g, wl.DSA_K) for g in (2, 4, 8)] + \
            [(wl.OPROJ_N, wl.OPROJ_K // g) for g in (2, 4, 8)] + \
            [(wl.KDA_N // g, wl.KDA_K) for g in (2, 4, 8)]


@pytest.mark.parametrize("N,K", TP_SHARDS, ids=lambda v: str(v))
def test_tp_shard_shapes_exact_and_random(N, K):
    x, W = wl.exact_sum_case(256, N, K, seed=17)
    Wd = W.to(DEV)
    plan = tp.Plan(N, K, BINS)
    for B in BINS:
        y = gpu_run(plan, x[:B], Wd)
        check_exact(f"shard N={N} K={K} B={B} {tactic_label(plan, B)}", y, x[:B], W)
    x, W = wl.random_case(64, N, K, seed=18)
    Wd = W.to(DEV)
    for B in (1, 16, 64):
        y = gpu_run(plan, x[:B], Wd)
        check_random(f"shard N={N} K={K} B={B} random", y, x[:B], W)
