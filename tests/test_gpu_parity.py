"""GPU parity: the HIP library (through its C-ABI) against the CPU oracle.

Element-by-element on shapes that span several tiles and ragged tails, the
edge cases of the method, and the five workload configurations (in full for
the three smaller ones, on seeded row samples at full size for the two
largest).  Tolerances: loss/lse absolute 2e-3 (bf16) / 1e-5 (fp32); dH, dW
relative Frobenius 1e-2 (bf16) / 1e-5 (fp32).
"""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import TOL, compare, device_inputs, log, logit_tol, max_abs, rel_fro, run_gpu

pytestmark = pytest.mark.gpu

IGN = wl.IGNORE_INDEX


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_flce_amd as flce
    flce.load()
    yield
    torch.cuda.empty_cache()


def _ref(inp, g):
    loss, lse, dH, dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y, IGN, g)
    return dict(loss=loss, lse=lse, dH=dH, dW=dW)


UNIT = [
    # T, d, V, ignore fraction
    (1, 8, 1, 0.0),
    (1, 8, 2, 0.0),
    (5, 16, 7, 0.0),
    (63, 72, 1000, 0.2),
    (257, 128, 1000, 0.0),
    (300, 136, 515, 0.3),
    (257, 72, 32007, 0.1),
    (520, 64, 2049, 0.0),
]


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("T,d,V,ign", UNIT, ids=lambda v: str(v))
def test_unit_shapes(T, d, V, ign, dtype):
    log(f"unit T={T} d={d} V={V} ign={ign} {dtype}")
    inp = wl.make_inputs(T, d, V, dtype, seed=100 + T + d + V, sigma_w=0.5, ignore_frac=ign)
    g = 1.0 / max(1, T)
    got = run_gpu(inp, loss_scale=g, grad_scale=g)
    ref = _ref(inp, g)
    errs = compare(got, ref, dtype)
    red = oracle.reduced_loss(ref["loss"], g)
    assert abs(got["red"][0] - red) <= TOL[dtype]["loss"] * max(1.0, abs(red))
    log("  errors", errs)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_empty_batch(dtype):
    """T = 0: the reduced loss is 0, dW is zeroed (or left as it was when
    accumulating), and the fused call does the same, for every dtype."""
    import linear_cross_entropy_flce_amd as flce
    d, V = 64, 1000
    et = torch.float32 if dtype == wl.DTYPE_F32 else torch.bfloat16
    dev = torch.device("cuda:0")
    H = torch.empty((0, d), dtype=et, device=dev)
    W = torch.randn((V, d), device=dev).to(et)
    y = torch.empty(0, dtype=torch.int64, device=dev)
    plan = flce.flce_plan(0, d, V, dtype)
    ws = flce.workspace(plan, dev)
    red = torch.full((1,), float("nan"), device=dev)
    loss, lse, _ = flce.flce_forward(plan, H, W, y, IGN, 0.5, loss_reduced=red, ws=ws)
    dW = torch.full((V, d), 7.0, device=dev)
    dH, _ = flce.flce_backward(plan, H, W, y, lse, IGN, 1.0, dW=dW, ws=ws)
    torch.cuda.synchronize()
    assert loss.numel() == 0 and lse.numel() == 0 and dH.numel() == 0
    assert red.item() == 0.0 and torch.count_nonzero(dW).item() == 0
    dW.fill_(7.0)
    flce.flce_backward(plan, H, W, y, lse, IGN, 1.0, dW=dW, accumulate_dW=True, ws=ws)
    torch.cuda.synchronize()
    assert torch.all(dW == 7.0).item()
    dW.fill_(7.0)
    dWb = torch.full((V, d), 7.0, device=dev).to(torch.bfloat16)
    out = flce.flce_forward_backward(plan, H, W, y, IGN, "mean_valid", 1.0, dW=dW, dW_bf16=dWb,
                                     ws=ws)
    torch.cuda.synchronize()
    assert out["loss_reduced"].item() == 0.0
    assert torch.count_nonzero(dW).item() == 0 and torch.count_nonzero(dWb).item() == 0


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_targets_at_tile_edges(dtype):
    T, d, V = 64, 32, 1030
    inp = wl.make_inputs(T, d, V, dtype, seed=7, sigma_w=0.5)
    edges = [0, 1, 31, 32, 63, 64, 127, 128, 255, 256, 257, 511, 512, 767, 768, 1023, 1024, V - 1]
    inp.y[:] = np.array([edges[i % len(edges)] for i in range(T)])
    got = run_gpu(inp, grad_scale=0.5)
    compare(got, _ref(inp, 0.5), dtype)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_all_ignored_and_none_ignored(dtype):
    inp = wl.make_inputs(130, 40, 600, dtype, seed=11, sigma_w=0.3)
    inp.y[:] = IGN
    got = run_gpu(inp)
    assert np.all(got["loss"] == 0.0)
    assert np.all(got["dH"] == 0.0) and np.all(got["dW"] == 0.0)
    ref = _ref(inp, 1.0)
    assert max_abs(got["lse"], ref["lse"]) <= TOL[dtype]["loss"]
    inp2 = wl.make_inputs(130, 40, 600, dtype, seed=12, sigma_w=0.3)
    compare(run_gpu(inp2), _ref(inp2, 1.0), dtype)


def test_large_logits_running_max():
    """Shift every row of W by c with h . c near 100 (fp32) or 400 (bf16):
    logits far beyond exp()'s float range; lse shifts by h . c, loss and
    gradients do not change.  A kernel without the running max overflows."""
    for dtype, target in ((wl.DTYPE_F32, 100.0), (wl.DTYPE_BF16, 400.0)):
        inp = wl.make_inputs(200, 64, 900, dtype, seed=13, sigma_w=0.2)
        H = inp.H_f32().astype(np.float64)
        c = np.zeros(64)
        c[0] = target / np.abs(H[:, 0]).max()
        W = inp.W_f32().astype(np.float64) + c
        if dtype == wl.DTYPE_F32:
            inp.W = W.astype(np.float32)
        else:
            inp.W = wl.f32_to_bf16_bits(W.astype(np.float32))
        got = run_gpu(inp)
        ref = _ref(inp, 1.0)
        assert np.all(np.isfinite(got["loss"])) and np.all(np.isfinite(got["lse"]))
        # float32 logits near |lse| carry an absolute error of a few ulp(|lse|):
        # the loss tolerance grows by that much
        ulp = np.abs(ref["lse"]).max() * 2.0 ** -23
        tl = TOL[dtype]["loss"] + 4 * ulp
        assert max_abs(got["loss"], ref["loss"]) <= tl
        assert max_abs(got["lse"], ref["lse"]) <= tl
        # the gathered target logit (pure log-sum-exp sweep) sums its 64
        # products in another order: sqrt(d) more ulps of |z| in fp32
        assert np.array_equal(got["lse_gather"], got["lse"])
        assert max_abs(got["loss_gather"], ref["loss"]) <= tl + np.sqrt(64) * ulp
        # the same absolute error in z - lse is a relative error of every
        # softmax entry, hence of dZ
        tg = TOL[dtype]["grad"] + 8 * ulp
        assert rel_fro(got["dW"], ref["dW"]) <= tg
        assert rel_fro(got["dH"][:, 1:], ref["dH"][:, 1:]) <= tg
        # column 0 of dH is sum_j dZ_ij (w_j0 + c0): the c0 part is zero in exact
        # arithmetic (dZ rows sum to 0) but carries c0 times the rounding of dZ,
        # whose row sums of magnitudes are at most 2 (grad scale 1); bf16 dZ
        # storage rounds to 2^-9 relative
        u = (2.0 ** -8 if dtype == wl.DTYPE_BF16 else 0.0) + 8 * ulp
        bound = 2 * c[0] * u + tg * np.abs(ref["dH"][:, 0]).max()
        assert max_abs(got["dH"][:, 0], ref["dH"][:, 0]) <= bound


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("d", [16384, 65536])
def test_long_hidden(d, dtype):
    """d = 16,384 and the largest supported d = 65,536 (long K loops for the
    logit tiles, long rows for every operand offset, 256 hidden tiles in dH
    and dW) with a ragged token count and vocabulary."""
    T, V = 300, 700
    inp = wl.make_inputs(T, d, V, dtype, seed=37, sigma_w=0.02, ignore_frac=0.1)
    got = run_gpu(inp, grad_scale=0.5)
    # fp32: sums of 16,384 terms round by ~sqrt(d) ulps of |z|; the same
    # absolute error in z - lse is the relative error of each dZ entry
    zmax = float(np.abs(oracle.logits(inp.H_f32(), inp.W_f32())).max())
    extra = logit_tol(dtype, d, zmax) - TOL[dtype]["loss"]
    errs = compare(got, _ref(inp, 0.5), dtype, loss_tol=TOL[dtype]["loss"] + extra,
                   grad_tol=TOL[dtype]["grad"] + extra)
    log("  errors", errs)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_several_blocks_and_slabs(dtype):
    """A small workspace cap forces several token blocks and vocab slabs: the
    fp32 dH accumulator and the block-ordered dW accumulation are exercised."""
    T, d, V = 1100, 96, 3000
    inp = wl.make_inputs(T, d, V, dtype, seed=17, sigma_w=0.4, ignore_frac=0.1)
    esz = 4 if dtype == wl.DTYPE_F32 else 2
    tile_v = 128 if dtype == wl.DTYPE_F32 else 256
    # room for a 512-token block, its fp32 dH accumulator and one vocab tile
    cap = 512 * (d * 4 + tile_v * esz)
    got = run_gpu(inp, grad_scale=0.25, cap=cap)
    plan = got["plan"]
    log("plan", plan.n_blocks, plan.n_slabs, plan.bwd_block, plan.bwd_slab)
    assert plan.n_blocks >= 2 and plan.n_slabs >= 2
    compare(got, _ref(inp, 0.25), dtype)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("pattern", ["suffix", "prefix", "alternate"])
def test_ignored_tokens_across_blocks(pattern, dtype):
    """The backward runs over the non-ignored tokens only, compacted into
    token blocks; with small blocks, whole blocks fall empty (suffix), the
    compacted order starts late in the batch (prefix) or interleaves
    (alternate), and accumulate_dW must still see every block's part."""
    T, d, V = 1500, 64, 900
    inp = wl.make_inputs(T, d, V, dtype, seed=41, sigma_w=0.4)
    if pattern == "suffix":
        inp.y[300:] = IGN
    elif pattern == "prefix":
        inp.y[:1200] = IGN
    else:
        inp.y[::2] = IGN
    esz = 4 if dtype == wl.DTYPE_F32 else 2
    tile_v = 128 if dtype == wl.DTYPE_F32 else 256
    cap = 512 * (d * 4 + tile_v * esz)
    base = np.random.default_rng(3).standard_normal((V, d)).astype(np.float32)
    got = run_gpu(inp, grad_scale=0.5, cap=cap, accumulate_dW=True, dW_init=base)
    plan = got["plan"]
    assert plan.n_blocks >= 4
    ref = _ref(inp, 0.5)
    ref["dW"] = ref["dW"] + base
    compare(got, ref, dtype)
    assert np.all(got["dH"][inp.y == IGN] == 0.0)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_split_dH_over_slabs(dtype):
    """dH of a 600-token block has 3 (bf16) or 5 (fp32) tiles at d = 64, so
    the planner reserves partial tiles and the device cuts each slab's K loop
    into many parts; the cap forces several vocab slabs, so the parts' sum
    passes through the first / middle / last accumulator modes."""
    T, d, V = 600, 64, 150000
    inp = wl.make_inputs(T, d, V, dtype, seed=29, sigma_w=0.4, ignore_frac=0.1)
    cap = 124_000_000 if dtype == wl.DTYPE_BF16 else 116_000_000
    got = run_gpu(inp, grad_scale=0.5, cap=cap)
    plan = got["plan"]
    log("plan", plan.n_blocks, plan.n_slabs, plan.bwd_block, plan.bwd_slab, plan.dh_split_bytes)
    assert plan.n_slabs >= 3 and plan.dh_split_bytes > 0
    compare(got, _ref(inp, 0.5), dtype)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("pattern", ["suffix", "prefix", "alternate"])
def test_split_dH_thinned_blocks(pattern, dtype):
    """Token blocks of 8,192 with split dH, thinned by ignored tokens: the
    device picks each block's split from its token count (full blocks, a
    half-full one, an empty one), and dH rows land at the tokens' own rows."""
    T, d, V = 20000, 64, 900
    inp = wl.make_inputs(T, d, V, dtype, seed=43, sigma_w=0.4)
    if pattern == "suffix":
        inp.y[12000:] = IGN
    elif pattern == "prefix":
        inp.y[:15000] = IGN
    else:
        inp.y[::2] = IGN
    base = np.random.default_rng(5).standard_normal((V, d)).astype(np.float32)
    got = run_gpu(inp, grad_scale=0.5, accumulate_dW=True, dW_init=base)
    plan = got["plan"]
    assert plan.n_blocks >= 3 and plan.dh_split_bytes > 0
    ref = _ref(inp, 0.5)
    ref["dW"] = ref["dW"] + base
    compare(got, ref, dtype)
    assert np.all(got["dH"][inp.y == IGN] == 0.0)


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("fused", [False, True], ids=["separate", "fused"])
def test_invalid_targets_poison(dtype, fused):
    """The header's contract for a target outside [0, V) that is not
    ignore_index: that token's loss and dH row are NaN and every element of
    dW is NaN; its lse and every other token's loss, lse and dH row are those
    of the same batch with the bad targets ignored; ignored tokens get loss 0
    and a zero dH row.  Unsharded flce_forward + flce_backward, and the fused
    call (sum reduction, whose reduced loss is then NaN)."""
    import linear_cross_entropy_flce_amd as flce
    T, d, V, g = 300, 64, 1100, 0.25
    inp = wl.make_inputs(T, d, V, dtype, seed=31, sigma_w=0.4, ignore_frac=0.15)
    bad = np.array([5, 6, 257])
    inp.y[bad] = [V + 3, -7, V]
    H, W, y = device_inputs(inp)
    plan = flce.flce_plan(T, d, V, dtype)
    ws = flce.workspace(plan, W.device)
    if fused:
        out = flce.flce_forward_backward(plan, H, W, y, IGN, "sum", g, ws=ws)
        loss, lse, dH, dW, red = (out[k] for k in ("loss", "lse", "dH", "dW", "loss_reduced"))
    else:
        red = torch.empty(1, dtype=torch.float32, device=W.device)
        loss, lse, _ = flce.flce_forward(plan, H, W, y, IGN, g, loss_reduced=red, ws=ws)
        dH, dW = flce.flce_backward(plan, H, W, y, lse, IGN, g, ws=ws)
    torch.cuda.synchronize()
    loss, lse = loss.cpu().numpy(), lse.cpu().numpy()
    dH, dW = dH.float().cpu().numpy(), dW.cpu().numpy()
    assert np.all(np.isnan(loss[bad])) and np.all(np.isnan(dH[bad]))
    assert np.all(np.isnan(dW)) and np.isnan(red.item())
    ok = np.ones(T, bool)
    ok[bad] = False
    ign = inp.y == IGN
    assert np.all(loss[ign] == 0.0) and np.all(dH[ign] == 0.0)
    clean = wl.Inputs(inp.H, inp.W, inp.y.copy(), dtype)
    clean.y[bad] = IGN
    rl, rs, rdH, _ = oracle.forward_backward(clean.H_f32(), clean.W_f32(), clean.y, IGN, g)
    assert np.all(np.isfinite(lse)) and max_abs(lse, rs) <= TOL[dtype]["loss"]
    assert max_abs(loss, rl, ok) <= TOL[dtype]["loss"]
    assert rel_fro(dH[ok], rdH[ok]) <= TOL[dtype]["grad"]


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
def test_accumulate_dW(dtype):
    inp = wl.make_inputs(300, 48, 700, dtype, seed=19, sigma_w=0.4)
    base = np.random.default_rng(0).standard_normal((700, 48)).astype(np.float32)
    got = run_gpu(inp, accumulate_dW=True, dW_init=base)
    ref = _ref(inp, 1.0)
    ref["dW"] = ref["dW"] + base
    compare(got, ref, dtype)


def test_deterministic():
    inp = wl.make_inputs(700, 256, 5000, wl.DTYPE_BF16, seed=23, ignore_frac=0.1)
    dev = device_inputs(inp)
    a = run_gpu(inp, grad_scale=0.01, dev=dev)
    b = run_gpu(inp, grad_scale=0.01, dev=dev)
    for k in ("loss", "lse", "dH", "dW"):
        assert np.array_equal(a[k], b[k]), k


def test_zero_weights_closed_form():
    """W = 0 on the GPU: lse = loss = ln V exactly (up to float rounding)."""
    inp = wl.make_inputs(256, 64, 3000, wl.DTYPE_BF16, seed=29)
    inp.W[:] = 0
    got = run_gpu(inp)
    assert max_abs(got["lse"], math.log(3000)) <= 1e-5
    assert max_abs(got["loss"], math.log(3000)) <= 1e-5
    assert np.all(got["dH"] == 0.0)


# ------------------------------------------------------------------ configs

@pytest.mark.parametrize("ci", [0, 1])
def test_config_full(ci):
    cfg = wl.CONFIGS[ci]
    log(f"config {ci} {cfg.name}: inputs")
    inp = wl.config_inputs(cfg)
    ls, gs = cfg.scales()
    got = run_gpu(inp, loss_scale=ls, grad_scale=gs)
    log("  oracle")
    ref = _ref(inp, gs)
    errs = compare(got, ref, cfg.dtype)
    red = oracle.reduced_loss(ref["loss"], ls)
    assert abs(got["red"][0] - red) <= TOL[cfg.dtype]["loss"] * max(1.0, abs(red))
    log("  errors", errs)


@pytest.mark.timeout(900)
def test_config2_full():
    cfg = wl.CONFIGS[2]
    log(f"{cfg.name}: inputs")
    inp = wl.config_inputs(cfg)
    ls, gs = cfg.scales()
    got = run_gpu(inp, loss_scale=ls, grad_scale=gs)
    log("  oracle (full, row chunks)")
    last = [0]

    def progress(r, T):
        if r - last[0] >= 2048 or r == T:
            last[0] = r
            log(f"  oracle rows {r}/{T}")

    loss, lse, dH, dW = oracle.forward_backward(inp.H_f32(), inp.W_f32(), inp.y, IGN, gs,
                                                progress=progress)
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH, dW=dW), cfg.dtype)
    log("  errors", errs)


@pytest.mark.timeout(600)
def test_dW_beyond_2GiB():
    """A large-vocabulary shape whose fp32 dW (152,064 x 3,584 x 4 bytes =
    2.03 GiB) reaches past 2^31 bytes while W and H stay below it: every
    output against the oracle, and the dW rows that start past the 2 GiB
    byte offset on their own."""
    T, d, V = 320, 3584, 152064
    log(f"dW beyond 2 GiB: T={T} d={d} V={V} bf16")
    inp = wl.make_inputs(T, d, V, wl.DTYPE_BF16, seed=4242, sigma_w=0.02, ignore_frac=0.1)
    g = 1.0 / T
    got = run_gpu(inp, loss_scale=g, grad_scale=g)
    log("  oracle")
    ref = _ref(inp, g)
    errs = compare(got, ref, wl.DTYPE_BF16)
    first = -(-(1 << 31) // (d * 4))  # first dW row whose bytes start at or past 2^31
    assert first < V
    tail = rel_fro(got["dW"][first:], ref["dW"][first:])
    log("  errors", errs, f"dW rows {first}..{V - 1}: {tail:.3e}")
    assert tail <= TOL[wl.DTYPE_BF16]["grad"]


@pytest.mark.timeout(900)
def test_W_beyond_2GiB():
    """An LM head whose bf16 W (131,200 x 8,192 x 2 bytes = 2.15 GB) is
    larger than the 2^31 bytes a 32-bit buffer offset reaches: the kernels
    address each W tile (and dH each vocab slab) from its own first row.
    Every output against the oracle, and the rows of W that lie past 2^31
    bytes on their own (their loss gradient dW rows)."""
    T, d, V = 384, 8192, 131200
    log(f"W beyond 2 GiB: T={T} d={d} V={V} bf16")
    inp = wl.make_inputs(T, d, V, wl.DTYPE_BF16, seed=4343, sigma_w=0.02, ignore_frac=0.1)
    assert V * d * 2 > 2 ** 31
    # targets in the rows past 2^31 bytes for a third of the tokens
    first = (1 << 31) // (d * 2)
    inp.y[::3] = np.where(inp.y[::3] == IGN, IGN, first + np.arange(len(inp.y[::3])) % (V - first))
    g = 1.0 / T
    got = run_gpu(inp, loss_scale=g, grad_scale=g)
    assert got["plan"].n_slabs >= 2 and got["plan"].bwd_slab * d * 2 < 2 ** 31
    log("  oracle")
    ref = _ref(inp, g)
    errs = compare(got, ref, wl.DTYPE_BF16)
    tail = rel_fro(got["dW"][first:], ref["dW"][first:])
    log("  errors", errs, f"dW rows {first}..{V - 1}: {tail:.3e}")
    assert tail <= TOL[wl.DTYPE_BF16]["grad"]


@pytest.mark.timeout(900)
def test_H_beyond_2GiB():
    """131,100 tokens of d = 8,192 in bf16: H is 2.15 GB, past 2^31 bytes;
    each forward token tile is addressed from its own first row (the
    backward gathers its token blocks with 64-bit addresses).  Every output
    against the oracle, and the token rows past 2^31 bytes on their own."""
    T, d, V = 131100, 8192, 1000
    log(f"H beyond 2 GiB: T={T} d={d} V={V} bf16")
    inp = wl.make_inputs(T, d, V, wl.DTYPE_BF16, seed=4444, sigma_w=0.02, ignore_frac=0.1)
    assert T * d * 2 > 2 ** 31
    got = run_gpu(inp, grad_scale=1.0 / T)
    log("  oracle")
    ref = _ref(inp, 1.0 / T)
    errs = compare(got, ref, wl.DTYPE_BF16)
    first = (1 << 31) // (d * 2)
    tail = dict(loss=max_abs(got["loss"][first:], ref["loss"][first:]),
                loss_gather=max_abs(got["loss_gather"][first:], ref["loss"][first:]),
                dH=rel_fro(got["dH"][first:], ref["dH"][first:]))
    log("  errors", errs, f"rows {first}..{T - 1}:", tail)
    assert tail["loss"] <= TOL[wl.DTYPE_BF16]["loss"]
    assert tail["loss_gather"] <= TOL[wl.DTYPE_BF16]["loss"]
    assert tail["dH"] <= TOL[wl.DTYPE_BF16]["grad"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("ci", [3, 4])
def test_config_sampled(ci):
    """Full-size run; the oracle checks 256 seeded rows (loss, lse, dH) and a
    seeded 2,048-token sub-batch run through both paths (dW).  At full size
    the dW rows must sum to zero (each dZ row sums to zero)."""
    cfg = wl.CONFIGS[ci]
    log(f"config {ci} {cfg.name}: inputs")
    inp = wl.config_inputs(cfg)
    ls, gs = cfg.scales()
    log("  gpu full size")
    got = run_gpu(inp, loss_scale=ls, grad_scale=gs)
    assert np.all(np.isfinite(got["loss"])) and np.all(np.isfinite(got["dW"]))
    rows = wl.sample_rows(cfg, 256)
    log("  oracle rows")
    Hf = inp.H_f32()
    Wf = inp.W_f32()
    loss, lse, dH = oracle.rows_forward_dH(Hf, Wf, inp.y, rows, IGN, gs)
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH), cfg.dtype, what=("loss", "lse", "dH"),
                   rows=rows)
    log("  row errors", errs)
    # sum over the vocab of dW is zero up to fp32/bf16 rounding
    colsum = got["dW"].astype(np.float64).sum(axis=0)
    scale = np.abs(got["dW"]).astype(np.float64).sum(axis=0).max()
    assert np.abs(colsum).max() <= 1e-3 * scale
    del got
    torch.cuda.empty_cache()
    # dW on a 2,048-token sub-batch through both paths
    sub = np.sort(wl.streams(cfg.seed_base + cfg.index)[4].choice(cfg.T, 2048, replace=False))
    sinp = inp.rows(sub)
    log("  gpu sub-batch")
    sg = run_gpu(sinp, loss_scale=ls, grad_scale=gs)
    log("  oracle sub-batch")
    sref = _ref(sinp, gs)
    errs = compare(sg, sref, cfg.dtype)
    log("  sub-batch errors", errs)
