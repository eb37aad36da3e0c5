"""The GEMM engine's layouts for the backward pass, through moe_gemm_bf16,
against numpy fp64 products of the same bf16 values: A and B as stored by the
forward ([M][K] x [N][K]), the weight operand K-outer ([K][N]), both operands
K-outer (K = tokens, with a partial last K tile), and one output per expert
over its pair rows (empty experts, ragged row counts)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _bf16(rng, *shape, scale=1.0):
    t = torch.from_numpy((rng.standard_normal(shape) * scale).astype(np.float32))
    return t.to(torch.bfloat16).cuda()


def _f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, want, what):
    err = np.abs(got.cpu().numpy() - want).max() / max(np.abs(want).max(), 1e-30)
    print(f"  {what}: normwise {err:.2e}", flush=True)
    assert err < 1e-5, what  # fp32 accumulation of exact bf16 products


@pytest.mark.parametrize("M,N,K", [(300, 200, 128), (40, 520, 192), (256, 256, 64)])
def test_stored_layout(M, N, K):
    import sparse_moe_layer_quantile_amd as moe
    rng = np.random.default_rng(1)
    a, b = _bf16(rng, M, K), _bf16(rng, N, K)
    _check(moe.gemm_bf16(a, b), _f64(a) @ _f64(b).T, f"A B^T {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(300, 264, 192), (40, 512, 128), (64, 3584, 448),
                                   (512, 72, 64)])
def test_weight_operand_k_outer(M, N, K):
    """dx = dy W with W stored [K][N]: partial M and N tiles, short batches."""
    import sparse_moe_layer_quantile_amd as moe
    rng = np.random.default_rng(2)
    a, b = _bf16(rng, M, K), _bf16(rng, K, N)
    c0 = torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda()
    _check(moe.gemm_bf16(a, b, b_kouter=True), _f64(a) @ _f64(b), f"A B {M}x{N}x{K}")
    _check(moe.gemm_bf16(a, b, b_kouter=True, c_in=c0), c0.cpu().numpy() + _f64(a) @ _f64(b),
           "C + A B")


@pytest.mark.parametrize("M,N,K", [(264, 200, 100), (256, 136, 1), (520, 264, 130),
                                   (128, 3072, 256)])
def test_both_operands_k_outer(M, N, K):
    """dW = dy^T n with K = tokens: a partial last K tile (masked), K = 1."""
    import sparse_moe_layer_quantile_amd as moe
    rng = np.random.default_rng(3)
    a, b = _bf16(rng, K, M), _bf16(rng, K, N)
    _check(moe.gemm_bf16(a, b, a_kouter=True, b_kouter=True), _f64(a).T @ _f64(b),
           f"A^T B {M}x{N}x{K}")


@pytest.mark.parametrize("N", [136, 768])
def test_expert_batched_k_ranges(N):
    """One output per expert over its rows: empty experts, 1 row, ragged tails,
    several K tiles; N in whole N tiles (one workgroup walks them all) or not."""
    import sparse_moe_layer_quantile_amd as moe
    rng = np.random.default_rng(4)
    M = 264
    off = np.array([0, 0, 3, 70, 70, 71, 200, 200], np.int32)
    P = int(off[-1])
    a, b = _bf16(rng, P + 8, M), _bf16(rng, P + 8, N)  # rows past P: never read
    c = moe.gemm_bf16(a, b, a_kouter=True, b_kouter=True,
                      k_offsets=torch.from_numpy(off).cuda())
    fa, fb = _f64(a), _f64(b)
    for e in range(len(off) - 1):
        want = fa[off[e]:off[e + 1]].T @ fb[off[e]:off[e + 1]]
        if off[e + 1] == off[e]:
            assert (c[e] == 0).all(), f"expert {e} without rows"
        else:
            _check(c[e], want, f"expert {e} ({off[e + 1] - off[e]} rows)")
