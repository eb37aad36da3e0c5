"""moe_forward_noalloc (the library-held workspace) against moe_forward with
a caller workspace, through the C ABI: two calls in a row, the second with a
smaller batch, must give the same output, routing and dispatch bit for bit
(same kernels on the same inputs); a batch needing more workspace than the
library holds is rejected before anything runs."""
import numpy as np
import pytest

import synth
from tests import parity

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


def say(*a):
    print(*a, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _outputs(cfg, bt):
    E, k = cfg.n_experts, cfg.top_k  # (an ABI config)
    z = lambda *s, dt=torch.int32: torch.full(s, -7, dtype=dt, device="cuda")
    return dict(idx=z(bt, k), w=z(bt, k, dt=torch.float32), cutoff=z(E, dt=torch.float32),
                logits=z(bt, E, dt=torch.float32), counts=z(E), offsets=z(E + 1),
                perm=z(bt * k), inv_perm=z(bt * k))


def _call(moe, layer, x, noalloc, side=None):
    bt = x.shape[0]
    cfg = layer.cfg
    out = _outputs(cfg, bt)
    route = moe.MoeRouteOut(*(out[n].data_ptr() for n in ("idx", "w", "cutoff", "logits")))
    disp = moe.MoeDispatchOut(*(out[n].data_ptr() for n in ("counts", "offsets", "perm",
                                                            "inv_perm")))
    y = torch.full((bt, cfg.d), 3.0, dtype=x.dtype, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    ss = side.cuda_stream if side is not None else 0
    if noalloc:
        st = moe.moe_forward_noalloc(cfg, layer.w, x.data_ptr(), bt, y.data_ptr(), route, disp,
                                     stream, ss)
    else:
        ws = layer.workspace(bt)
        st = moe.moe_forward(cfg, layer.w, x.data_ptr(), bt, y.data_ptr(), route, disp,
                             ws.data_ptr(), ws.numel(), stream, ss)
    assert st == 0, moe.status_str(st)
    torch.cuda.synchronize()
    out["y"] = y
    return {n: v.cpu() for n, v in out.items()}


@pytest.mark.parametrize("name,bts", [("k3_decode_bf16", (64, 16)), ("mid_bf16", (200, 37)),
                                      ("k3_decode_mxfp4_a8", (64, 5)), ("tiny_fp32", (64, 3))])
def test_noalloc_forward_equals_forward(name, bts):
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS[name]
    layer, x = parity.device_layer(cfg, seed=0)
    for i, bt in enumerate(bts):
        say(f"noalloc {name} call {i} bt {bt}: workspace {moe.workspace_bytes(layer.cfg, bt)} B")
        assert moe.workspace_bytes(layer.cfg, bt) <= moe.NOALLOC_SCRATCH_BYTES
        xs = x[:bt].contiguous()
        side = torch.cuda.Stream() if i == 1 else None
        a = _call(moe, layer, xs, noalloc=True, side=side)
        b = _call(moe, layer, xs, noalloc=False, side=side)
        for n in a:
            va, vb = a[n], b[n]
            if va.dtype == torch.bfloat16:
                va, vb = va.view(torch.int16), vb.view(torch.int16)
            assert torch.equal(va, vb), f"{name} bt {bt}: {n} differs"
    del layer, x


def test_noalloc_rejects_batches_beyond_its_scratch():
    import sparse_moe_layer_quantile_amd as moe
    cfg = synth.CONFIGS["k3_decode_bf16"]
    layer, x = parity.device_layer(cfg, seed=0, names=["x", "w_router"])
    bt = 128  # needs more than the 128 MiB the library holds
    assert moe.workspace_bytes(layer.cfg, bt) > moe.NOALLOC_SCRATCH_BYTES
    xb = torch.zeros((bt, cfg.d), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((bt, cfg.d), dtype=torch.bfloat16, device="cuda")
    st = moe.moe_forward_noalloc(layer.cfg, layer.w, xb.data_ptr(), bt, y.data_ptr(), None, None,
                                 torch.cuda.current_stream().cuda_stream, 0)
    assert st == -3  # MOE_ERR_WORKSPACE, nothing enqueued
