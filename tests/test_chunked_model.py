"""The chunked method, checked on the CPU against the fp64 token-by-token oracle.

The HIP kernels evaluate the recurrence in 64-token chunks (intra-chunk UT/WY
solve, inter-chunk state pass).  The model in chunked_model.py writes that
algebra out in numpy: in fp64 it must equal the oracle to 1e-12 (the chunked
form is an identity, not an approximation), and its triangular solve must equal
numpy.linalg.solve.  With bf16 rounding injected where the kernels round, the
model predicts the kernels' error against the oracle; the precision of the
kernel design (U~ in fp32 through a bf16 hi/lo pair) is recorded here.
"""
import numpy as np
import pytest

from chunked_model import ALL_BF16, EXACT, KERNEL, KERNEL_F16, chunked_forward, f16_tiles, unit_lower_inverse
from oracle import Oracle, rel_l2
from workloads import custom_problem, make_problem


def test_unit_lower_inverse_equals_linalg_solve():
    rng = np.random.default_rng(0)
    for n in (1, 2, 17, 64):
        A = np.tril(rng.normal(size=(3, n, n)) * 0.3, -1)
        T = unit_lower_inverse(A)
        ref = np.linalg.solve(np.eye(n)[None] + A, np.broadcast_to(np.eye(n), (3, n, n)))
        assert np.max(np.abs(T - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))
        assert np.allclose(np.tril(T), T) and np.all(np.diagonal(T, axis1=1, axis2=2) == 1.0)


@pytest.mark.parametrize("lengths,hk,hv,dk,dv,l2norm,state", [
    ((1, 63, 64, 65, 130, 200), 2, 4, 64, 64, True, True),
    ((300,), 1, 2, 128, 128, True, False),
    ((129, 0, 70), 2, 2, 64, 128, False, True),
])
def test_exact_chunked_model_equals_the_token_recurrence(lengths, hk, hv, dk, dv, l2norm, state):
    p = custom_problem(lengths, hk=hk, hv=hv, dk=dk, dv=dv, seed=11, with_state=state, l2norm=l2norm)
    if not l2norm:
        import dataclasses
        p = dataclasses.replace(p, k=(p.k.float() / 8).bfloat16(), q=(p.q.float() / 8).bfloat16())
    o, fin = chunked_forward(p, EXACT)
    ref = Oracle(p).run_all()
    assert rel_l2(o, ref["o"]) <= 1e-12
    assert rel_l2(fin, ref["state"]) <= 1e-12


def test_exact_chunked_model_slow_decay_with_initial_state():
    # the slow-decay companion of the dense batch, cut to two sequences: the initial
    # state reaches o and the final state
    p = custom_problem((700, 64), hk=1, hv=4, dk=128, dv=128, seed=12, with_state=True, g_div=4096.0,
                       beta_div=64.0)
    o, fin = chunked_forward(p, EXACT)
    ref = Oracle(p).run_all()
    assert rel_l2(o, ref["o"]) <= 1e-12 and rel_l2(fin, ref["state"]) <= 1e-12


def test_planted_mistakes_in_the_model_are_caught():
    """The pin is not vacuous: the chunked algebra with a transposed triangular factor,
    or with the decays inside a chunk left out, is far from the oracle."""
    import chunked_model as cm
    p = custom_problem((130,), hk=1, hv=1, dk=64, dv=64, seed=13, with_state=True)
    ref = Oracle(p).run_all()
    orig_inv, orig_mask = cm.unit_lower_inverse, cm._masked_exp
    try:
        cm.unit_lower_inverse = lambda A: np.transpose(orig_inv(A), (0, 2, 1))
        o, fin = chunked_forward(p, EXACT)
        assert rel_l2(fin, ref["state"]) > 1e-2
        cm.unit_lower_inverse = orig_inv
        cm._masked_exp = lambda gam, strict: np.where(orig_mask(gam, strict) > 0, 1.0, 0.0)
        o, fin = chunked_forward(p, EXACT)
        assert rel_l2(o, ref["o"]) > 1e-2
    finally:
        cm.unit_lower_inverse, cm._masked_exp = orig_inv, orig_mask
    o, fin = chunked_forward(p, EXACT)
    assert rel_l2(fin, ref["state"]) <= 1e-12


def test_kernel_rounding_plan_on_the_varlen_workload():
    """The kernels' rounding points on the varlen workload (T = 4096, H = 16,
    K = V = 128): final states and o well inside the tolerances (5e-3 and 1e-2).
    Recorded: kernel design about 1.8e-3 (final) and 2.9e-3 (o); U~ itself in bf16
    about twice the final-state error."""
    p = make_problem(2)
    ref = Oracle(p).run_all()
    o, fin = chunked_forward(p, KERNEL)
    es, eo = rel_l2(fin, ref["state"]), rel_l2(o, ref["o"])
    print(f"kernel rounding: final {es:.2e}, o {eo:.2e}")
    assert es <= 2.5e-3 and eo <= 4e-3
    o2, fin2 = chunked_forward(p, ALL_BF16)
    es2 = rel_l2(fin2, ref["state"])
    print(f"U~ in bf16: final {es2:.2e}, o {rel_l2(o2, ref['o']):.2e}")
    assert es2 > 1.3 * es
    # the kernels' fp16 hand-over of U~ (power-of-two scale per 32 x 32 tile) costs
    # under 2 % of the final-state error of the fp32 hand-over
    o3, fin3 = chunked_forward(p, KERNEL_F16)
    es3, eo3 = rel_l2(fin3, ref["state"]), rel_l2(o3, ref["o"])
    print(f"U~ in scaled fp16: final {es3:.2e}, o {eo3:.2e}")
    assert es3 <= 1.02 * es and eo3 <= 1.02 * eo


def test_f16_tiles_rounding():
    """The scaled fp16 tiles: every element within 2^-11 relative (fp16's unit roundoff)
    wherever it is within 2^28 of its tile's largest magnitude, powers of two and zero
    tiles exact, tiles independent, and values far above fp16's range kept."""
    rng = np.random.default_rng(5)
    x = rng.normal(size=(3, 64, 96)) * np.exp(rng.normal(size=(3, 64, 96)) * 3)
    x = x.astype(np.float32).astype(np.float64)
    x[0, :32, :32] = 0.0
    x[1, 32:, 32:64] = 2.0 ** rng.integers(-60, 60, size=(32, 32))
    x[2, :32, 64:] *= 1e30
    y = f16_tiles(x)
    for b in range(3):
        for r in range(0, 64, 32):
            for c in range(0, 96, 32):
                t, u = x[b, r:r + 32, c:c + 32], y[b, r:r + 32, c:c + 32]
                amax = np.max(np.abs(t))
                keep = np.abs(t) >= amax * 2.0 ** -28
                assert np.all(np.abs(u - t)[keep] <= 2.0 ** -11 * np.abs(t)[keep])
                assert np.all(np.abs(u - t) <= 2.0 ** -11 * amax)
    assert np.all(y[0, :32, :32] == 0.0)
    big = x[1, 32:, 32:64]
    exact = np.abs(big) >= np.max(np.abs(big)) * 2.0 ** -24
    assert np.array_equal(y[1, 32:, 32:64][exact], big[exact])
    assert np.isfinite(y).all() and np.max(np.abs(y[2, :32, 64:])) > 1e29


@pytest.mark.parametrize("lengths,hk,hv,dk,dv,l2norm", [
    ((1, 63, 64, 65, 130), 2, 4, 64, 64, True),
    ((200, 0, 70), 1, 1, 64, 128, False),
    ((129,), 2, 2, 128, 64, True),
])
def test_exact_chunked_backward_equals_the_oracle_backward(lengths, hk, hv, dk, dv, l2norm):
    """The chunked backward (reverse chunk pass for the state gradient, then every
    chunk's gradients through P, W, U~, T = (I + A)^-1 and the decays) equals the
    oracle's token-by-token backward, itself pinned by autograd and central differences."""
    import dataclasses

    import torch

    import oracle
    from chunked_model import chunked_backward
    p = custom_problem(lengths, hk=hk, hv=hv, dk=dk, dv=dv, seed=14, with_state=True, l2norm=l2norm)
    if not l2norm:
        p = dataclasses.replace(p, k=(p.k.float() / 8).bfloat16(), q=(p.q.float() / 8).bfloat16())
    gen = torch.Generator().manual_seed(15)
    dO = torch.randn((p.total_tokens, hv, dv), generator=gen).double().numpy()
    dF = torch.randn((p.num_seqs, hv, dk, dv), generator=gen).double().numpy()
    ref = oracle.backward(p, d_o=dO, d_final=dF)
    got = chunked_backward(p, dO, dF)
    for name in ("dq", "dk", "dv", "dg", "dbeta", "d_init"):
        assert rel_l2(got[name], ref[name]) <= 1e-12, name
