"""Device numerics of the SiTU-GLU factors against the fp64 oracle, over the
whole input range the layer can see, out to |x| = 1e4 where both factors sit
on their caps (tech.news18a.com "KimiK3的StableLatentMoE架构解析", first
technique: the output range is strictly bounded, beta = 4, beta_u = 25).
moe_situ_eval runs the same inline device functions as the GEMM epilogues.

Error bound: each factor is an fp32 product of sigmoid and tanh built from
the hardware exp2 and reciprocal (about one ulp each); tanh(x) = (1 - e) /
(1 + e) with e = exp(-2|x|) loses relative accuracy for tiny |x| but keeps an
absolute error of a few ulp of 1.  So every output must be within
16 * 2^-24 * (cap + |exact|) of the fp64 value, cap = beta, beta_u and
beta * beta_u for phi, psi and h."""
import numpy as np
import pytest

import oracle

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

BETA, BETA_U = 4.0, 25.0
U32 = 2.0 ** -24


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _inputs():
    mags = np.logspace(-8, 4, 3000)
    specials = np.array([0.0, 1e-30, 1e-20, 0.5, 1.0, 1.2187, 2.0, 4.0, 8.0, 12.5, 25.0, 50.0,
                         88.0, 89.0, 100.0, 1000.0, 9999.0, 1e4])
    rng = np.random.default_rng(60)
    v = np.concatenate([mags, -mags, specials, -specials, rng.normal(0, 1, 4000),
                        rng.normal(0, 30, 4000)])
    return v.astype(np.float32)


def test_situ_factors_match_fp64_up_to_1e4():
    import sparse_moe_layer_quantile_amd as moe
    v = _inputs()
    rng = np.random.default_rng(61)
    g = v
    u = rng.permutation(v)  # pair the values differently for h
    phi, psi, h = (t.cpu().numpy().astype(np.float64) for t in
                   moe.situ_eval(torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda(),
                                 BETA, BETA_U))
    ref_phi = np.array([oracle.phi(float(a), BETA) for a in g])
    ref_psi = np.array([oracle.psi(float(b), BETA_U) for b in u])
    ref_h = ref_phi * ref_psi
    for name, got, ref, cap in (("phi", phi, ref_phi, BETA), ("psi", psi, ref_psi, BETA_U),
                                ("h", h, ref_h, BETA * BETA_U)):
        err = np.abs(got - ref)
        bound = 16 * U32 * (cap + np.abs(ref))
        worst = int(np.argmax(err / bound))
        print(f"  {name}: max |err| {err.max():.3e}, worst err/bound {err[worst] / bound[worst]:.3f} "
              f"at input {g[worst] if name != 'psi' else u[worst]:.6g}", flush=True)
        assert (err <= bound).all(), name
    # the caps hold in fp32 for every input: phi <= beta with its minimum
    # near -0.2698, |psi| <= beta_u, |h| <= beta beta_u
    assert phi.max() <= BETA and phi.min() >= -0.26977
    assert np.abs(psi).max() <= BETA_U and np.abs(h).max() <= BETA * BETA_U


def test_situ_saturates_exactly_at_the_caps():
    import sparse_moe_layer_quantile_amd as moe
    big = np.array([100.0, 200.0, 1000.0, 1e4], np.float32)
    g = np.concatenate([big, -big])
    u = np.concatenate([big * 4, -big * 4])
    phi, psi, h = (t.cpu().numpy() for t in
                   moe.situ_eval(torch.from_numpy(g).cuda(), torch.from_numpy(u).cuda(),
                                 BETA, BETA_U))
    np.testing.assert_array_equal(phi[:4], BETA)            # sigmoid -> 1, tanh -> 1
    # sigmoid(g) < 4e-44 for g <= -100: phi is below the least normal fp32 value
    assert (np.abs(phi[4:]) < 2.0 ** -126).all()
    np.testing.assert_array_equal(psi, np.sign(u) * BETA_U)
    np.testing.assert_array_equal(h[:4], BETA * BETA_U)
    # psi is odd, exactly: tanh is formed on |u| and signed afterwards
    v = _inputs()
    _, p1, _ = moe.situ_eval(torch.from_numpy(v).cuda(), torch.from_numpy(v).cuda())
    _, p2, _ = moe.situ_eval(torch.from_numpy(-v).cuda(), torch.from_numpy(-v).cuda())
    np.testing.assert_array_equal(p1.cpu().numpy(), -p2.cpu().numpy())


def test_situ_eval_partial_outputs_and_errors():
    import sparse_moe_layer_quantile_amd as moe
    g = torch.linspace(-10, 10, 1000, device="cuda")
    h = torch.empty_like(g)
    st = moe.moe_situ_eval(g.data_ptr(), g.data_ptr(), g.numel(), 4.0, 25.0, 0, 0, h.data_ptr(),
                           torch.cuda.current_stream().cuda_stream)
    assert st == 0
    _, _, h2 = moe.situ_eval(g, g)
    assert torch.equal(h, h2)
    assert moe.moe_situ_eval(g.data_ptr(), 0, 10, 4.0, 25.0, h.data_ptr(), 0, 0, 0) == -1
