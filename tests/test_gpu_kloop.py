"""GPU parity at the K-loop's stage-count boundaries.

The tile engine's K loop runs pairs of branch-free steady stages while the
stages they load are whole, then at most three stages of the general body
(partial last stage, no loads past K).  The contraction lengths here, d for the
logit recompute and the forward, the vocabulary for dH and the token count for
dW, run through 1 to 8 whole stages (64 bf16 or 32 fp32 elements of k each),
with and without a partial last stage of 8 elements, so that every split
between the two bodies is met by each kernel.
"""
import pytest
import torch

import oracle
import workloads as wl
from gpu_helpers import TOL, compare, log, logit_tol, run_gpu

pytestmark = pytest.mark.gpu

IGN = wl.IGNORE_INDEX

# (stages of T, of d, of V) and the partial extra elements of each
CASES = [
    ((1, 0), (1, 0), (1, 0)),
    ((2, 0), (2, 0), (2, 8)),
    ((3, 8), (3, 0), (4, 0)),
    ((4, 0), (4, 8), (5, 0)),
    ((5, 8), (5, 0), (6, 8)),
    ((6, 0), (6, 8), (7, 0)),
    ((7, 8), (7, 0), (8, 8)),
    ((8, 0), (8, 0), (8, 0)),
]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_cross_entropy_flce_amd as flce
    flce.load()
    yield
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", [wl.DTYPE_F32, wl.DTYPE_BF16])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "T%d+%d_d%d+%d_V%d+%d" % (*c[0], *c[1], *c[2]))
def test_stage_counts(case, dtype):
    bk = 64 if dtype == wl.DTYPE_BF16 else 32
    (nt, pt), (nd, pd), (nv, pv) = case
    T, d, V = nt * bk + pt, nd * bk + pd, nv * bk + pv
    log(f"k-loop T={T} d={d} V={V} {dtype}")
    inp = wl.make_inputs(T, d, V, dtype, seed=4000 + T + d + V, sigma_w=0.5, ignore_frac=0.0)
    g = 1.0 / T
    got = run_gpu(inp, loss_scale=g, grad_scale=g)
    Hf, Wf = inp.H_f32(), inp.W_f32()
    loss, lse, dH, dW = oracle.forward_backward(Hf, Wf, inp.y, IGN, g)
    # fp32: the kernels sum the d products in another order than the oracle
    ltol = logit_tol(dtype, d, float(abs(oracle.logits(Hf, Wf)).max()))
    errs = compare(got, dict(loss=loss, lse=lse, dH=dH, dW=dW), dtype, loss_tol=ltol,
                   grad_tol=TOL[dtype]["grad"] + (ltol - TOL[dtype]["loss"]))
    log("  errors", errs)
