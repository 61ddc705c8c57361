"""GPU checks of the Python binding's stream and device handling.

The allocating helpers put their outputs and temporaries on the stream the
library call runs on, so a block freed after a call is handed only to later
work on that stream.  A layer run on a side stream (a torch stream, and the
same stream passed as a raw hipStream_t handle) must give the default-stream
result bit for bit, even while the current stream allocates and writes new
tensors at once; tensors on the CPU and the GPU in one call are refused.
"""
import numpy as np
import pytest

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sq():
    import torch
    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    import w8a8_post_quantization_sq_amd as m
    m.lib()
    return m


def _layer_inputs(sq, dev):
    import torch
    wl = W.WORKLOADS["qkv4096"]
    inp = W.generate(wl, m=512)
    x = torch.from_numpy(inp.x).to(dev)
    ax = sq.calibrate(torch.from_numpy(inp.x_cal).to(dev))
    f = sq.fold(torch.from_numpy(inp.w).to(dev), ax, wl.alpha)
    torch.cuda.synchronize()
    return x, f


@pytest.mark.parametrize("handle", [False, True])
def test_smoothed_linear_on_a_side_stream(sq, handle):
    import torch
    dev = torch.device("cuda:0")
    print(f"[binding] side stream, raw handle={handle}", flush=True)
    x, f = _layer_inputs(sq, dev)
    ref = sq.smoothed_linear(x, f)
    torch.cuda.synchronize()
    ref = ref.cpu().numpy()
    side = torch.cuda.Stream(device=dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    outs = []
    for _ in range(4):
        y = sq.smoothed_linear(x, f, stream=side.cuda_stream if handle else side)
        # the current stream allocates and fills blocks of the freed
        # temporaries' sizes right away; with stream-ordered reuse they cannot
        # be the side stream's codes still being read
        junk = [torch.full((sq.packed_bytes(x.shape[0], x.shape[1]),), 77, dtype=torch.int8,
                           device=dev),
                torch.full((x.shape[0],), -1.0, device=dev)]
        outs.append((y, junk))
    torch.cuda.synchronize()
    for y, _ in outs:
        assert np.array_equal(y.cpu().numpy().view(np.uint16), ref.view(np.uint16))


def test_binding_refuses_mixed_devices(sq):
    import torch
    dev = torch.device("cuda:0")
    x = torch.zeros(4, 64, dtype=torch.float16, device=dev)
    inv = torch.ones(64, dtype=torch.float32)                     # on the CPU
    xq = torch.zeros(sq.packed_bytes(4, 64), dtype=torch.int8, device=dev)
    xs = torch.zeros(4, dtype=torch.float32, device=dev)
    with pytest.raises(ValueError, match="inv_smooth: expected a GPU tensor"):
        sq.sq_quant_act_per_token(x, inv, xq, xs)
