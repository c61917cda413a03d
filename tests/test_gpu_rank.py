"""GPU parity of entropy-driven rank allocation (milo_rank_allocate) against
the fp64 greedy oracle.

Ranks are integers decided by comparing gains, so they must match the
oracle's exactly, except where two units' gains tie to within the
precision the two sides compute them in: then either pick is the greedy's
answer.  check_allocation accepts a difference only between units whose
fp64 gains lie within rtol of the selection threshold (the K-th largest
gain), with the budget kept and every rank in bounds.  Same spectra on both
sides: fp32 versus fp64 gains, rtol 1e-5.  Spectra from the GPU encode
against the fp64 SVD: the fp32 Gram eigenvalues carry absolute errors of
about 1e-7 of a block's energy, so a gain (H <= ln d times an energy
fraction) is known to rtol 5e-3 plus atol 1e-6; below that the order of
units is not determined by the data."""
import numpy as np
import pytest

import synth
from oracle import encode as oenc
from oracle import rank_alloc as oalloc
from tests.gpu_util import note

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def unit_gains(sig_b, r_min, unit):
    H, p = oalloc.block_distribution(sig_b)
    d = sig_b.shape[-1]
    return np.array([oalloc.unit_gain(H, p, r, unit) for r in range(r_min, r_min + unit * ((d - r_min) // unit),
                                                                        unit)])


def check_allocation(got, sig, budget, r_min, unit, rtol, name, atol=0.0):
    want = oalloc.allocate(sig, budget, r_min, unit)
    d = sig.shape[-1]
    assert got.sum() == budget, f"{name}: budget {got.sum()} != {budget}"
    assert got.min() >= r_min and got.max() <= d and np.all((got - r_min) % unit == 0)
    if np.array_equal(got, want):
        return 0
    gains = [unit_gains(sig[b], r_min, unit) for b in range(len(got))]
    allg = np.sort(np.concatenate(gains))[::-1]
    K = (budget - len(got) * r_min) // unit
    tau = allg[K - 1]
    diff = 0
    for b in np.nonzero(got != want)[0]:
        lo, hi = sorted((int(got[b]), int(want[b])))
        for r in range(lo, hi, unit):
            g = gains[b][(r - r_min) // unit]
            assert abs(g - tau) <= rtol * tau + atol, (f"{name}: block {b} differs at rank {r}: gain {g:.6e} "
                                                f"is not a near-tie of the threshold {tau:.6e}")
            diff += 1
    note(f"{name}: {diff} units swapped at near-ties")
    return diff


def run_alloc(sigma_np, bk, bv, r_min, unit):
    import torch
    from rank_attention_amd.encode import allocate_ranks
    s = torch.from_numpy(np.ascontiguousarray(sigma_np, np.float32)).to("cuda")
    ranks, ent = allocate_ranks(s, bk, bv, r_min, unit)
    torch.cuda.synchronize()
    return ranks.cpu().numpy().astype(np.int64), ent.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("nb,h,d,r_min,unit,frac", [
    (64, 4, 128, 8, 1, 0.5), (64, 4, 128, 16, 16, 0.25), (7, 2, 64, 0, 1, 0.3),
    (300, 1, 128, 1, 1, 0.7), (5, 3, 64, 64, 1, 1.0), (9, 2, 128, 0, 1, 0.0),
    (1100, 2, 128, 4, 16, 0.4)])
def test_allocation_matches_greedy(nb, h, d, r_min, unit, frac):
    sig = synth.make_spectra(nb, h, d, seed=nb + d)
    per = (d - r_min) // unit
    note(f"rank alloc nb={nb} Hkv={h} d={d} r_min={r_min} unit={unit} frac={frac}")
    budgets = []
    for kv, f in enumerate((frac, frac * 0.6)):
        units = int(round(f * nb * per))
        budgets.append(nb * r_min + unit * units)
    ranks, ent = run_alloc(sig, budgets[0], budgets[1], r_min, unit)
    sig64 = sig.astype(np.float64)
    for kv in range(2):
        s = sig64[:, :, kv, :]
        check_allocation(ranks[:, kv], s, budgets[kv], r_min, unit, 1e-5, f"kv{kv}")
        H = np.array([oalloc.block_distribution(s[b])[0] for b in range(nb)])
        np.testing.assert_allclose(ent[:, kv], H, rtol=1e-5, atol=1e-6)


def test_worked_example_exact():
    """The hand-worked case of the oracle's pins, on the GPU: B fills before A."""
    sig = np.zeros((2, 1, 2, 64), np.float32)
    sig[0, 0, :, :4] = [3.0, 1.0, 0.0, 0.0]
    sig[1, 0, :, :4] = [1.0, 1.0, 1.0, 1.0]
    for budget, want in [(1, [0, 1]), (4, [0, 4]), (5, [1, 4]), (8, [4, 4])]:
        ranks, _ = run_alloc(sig, budget, budget, 0, 1)
        assert list(ranks[:, 0]) == want and list(ranks[:, 1]) == want, budget


@pytest.mark.parametrize("frac", [0.2, 0.5])
def test_encode_spectrum_then_allocate_then_factors(frac):
    """The encode workflow on the GPU: spectra, ranks at a 20% / 50% budget,
    then factors at those ranks; against the oracle's SVD spectra and greedy."""
    import torch
    from rank_attention_amd.encode import DeviceContext, allocate_ranks
    cfg = synth.get_encode_config("enc_small").with_(n_blocks=12, block_tokens=384, seed=46)
    ctx = synth.make_dense_context(cfg)
    dc = DeviceContext(ctx.k, ctx.v, ctx.tok_start, ctx.n_tok, dtype=cfg.dtype)
    sigma, _ = dc.spectrum()
    nb, d, r_min = cfg.n_blocks, cfg.head_dim, 4
    budget = int(nb * d * frac)
    ranks, _ = allocate_ranks(sigma, budget, budget, r_min, 1)
    torch.cuda.synchronize()
    rk = ranks.cpu().numpy().astype(np.int64)
    ref_sig = oenc.context_spectra(ctx)                    # fp64 [nb][Hkv][2][d]
    for kv in range(2):
        check_allocation(rk[:, kv], ref_sig[:, :, kv, :], budget, r_min, 1, 5e-3, f"encode kv{kv}", atol=1e-6)
    pool, _, blocks = dc.factors(rk[:, 0], rk[:, 1])
    torch.cuda.synchronize()
    assert list(blocks["rank_k"]) == list(rk[:, 0]) and list(blocks["rank_v"]) == list(rk[:, 1])
    assert int(pool.numel()) >= int(blocks["off"][-1])
