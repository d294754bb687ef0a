"""The measurement helpers behind bench.py's ceilings (GPU): they run through
the C ABI, write nothing, and the MFMA probe's rate lies between half and all
of the chip's bf16 peak (an MFMA loop the compiler had dropped would read far
above it)."""
import pytest
import torch

import sparse_moe_layer_amd as lib

pytestmark = pytest.mark.gpu


def test_hbm_read_probe_reads_and_writes_nothing():
    src = torch.full((64 << 20,), 3, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    lib.moe_hbm_read_probe(src, sink)
    torch.cuda.synchronize()
    assert int(sink.item()) == 0


def test_mfma_pipe_probe_variants():
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.zeros(4 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.float32, device="cuda")
    for v in range(6):
        lib.moe_mfma_pipe_probe(v, 100, src, sink)
    torch.cuda.synchronize()
    assert float(sink.item()) == 0.0
    # MFMAs alone, timed: 8 waves per CU x steps x 16 MFMAs of 32x32x16
    steps = 20000
    lib.moe_mfma_pipe_probe(0, steps // 10, None, sink)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    lib.moe_mfma_pipe_probe(0, steps, None, sink)
    b.record()
    torch.cuda.synchronize()
    tflops = cus * 8 * steps * 16 * 32768 / (a.elapsed_time(b) * 1e-3) / 1e12
    print(f"[probe] MFMA-only rate {tflops:.0f} TFLOP/s", flush=True)
    assert 1250.0 < tflops < 2600.0
