"""The allocation-free layer call against moe_layer_forward (GPU).

moe_layer_forward_noalloc runs the same kernels with its workspace in the
library's device array, so its outputs must equal the workspace call's bit
for bit.  Two calls in a row on the shared array, the second with fewer
tokens; then a problem too large for the array is refused."""
import numpy as np
import pytest
import torch

import sparse_moe_layer_amd as lib
from oracle import adapter
from sparse_moe_layer_amd.tensors import structs
from synthetic import CONFIGS, make_problem

pytestmark = pytest.mark.gpu


def _layer(p, T, noalloc):
    c = p.cfg
    P, W = structs(p, T=T)
    x = p.x[:T].contiguous()
    out = torch.full((T, c.H), float("nan"), dtype=p.x.dtype, device="cuda")
    ids = torch.full((T, c.k), -1, dtype=torch.int32, device="cuda")
    w = torch.full((T, c.k), float("nan"), dtype=torch.float32, device="cuda")
    if noalloc:
        lib.moe_layer_forward_noalloc(P, W, x, out, ids, w)
    else:
        lib.moe_layer_forward(P, W, x, out, ids, w, lib.workspace(P))
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), ids.cpu().numpy(), w.cpu().numpy()


@pytest.mark.parametrize("name", ["flash_prefill", "max_fp8"])
def test_noalloc_matches_workspace_call(name):
    shared = 128 if name == "flash_prefill" else 0
    cfg = CONFIGS[name].with_(name="noalloc_" + name, T=40, H=256, E=32, k=4, I=128, I_shared=shared, zipf_s=0.0)
    print(f"[no-alloc] {cfg.name} T=40 then T=12", flush=True)
    p = make_problem(cfg, 31, device="cuda")
    adapter.ensure_margin(p, 1e-3)
    for T in (40, 12):  # the second call with a smaller input, on the same device array
        ref = _layer(p, T, noalloc=False)
        got = _layer(p, T, noalloc=True)
        for a, b, what in zip(got, ref, ("out", "ids", "w")):
            assert np.array_equal(a, b, equal_nan=False), f"{what} differs at T={T}"


def test_noalloc_refuses_a_problem_beyond_its_array():
    cfg = CONFIGS["flash_prefill"].with_(name="noalloc_big", T=4096, H=256, E=32, k=4, I=128, I_shared=128)
    p = make_problem(cfg, 32, device="cuda")
    P, W = structs(p)
    big = lib.problem(4096, 2560, 512, 10, 640, 640)
    assert lib.moe_workspace_bytes(big) > lib.MOE_NOALLOC_SCRATCH_BYTES
    out = torch.empty((4096, 256), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(lib.MoEError) as e:
        lib.moe_layer_forward_noalloc(big, W, p.x, out, None, None)
    assert e.value.status == 5  # MOE_ERR_WORKSPACE
