"""Host checks of the Python binding's output validation (no GPU, no library call).

The C ABI receives no output sizes, so the binding is the only guard against an
output buffer that is too small, of the wrong dtype, on another device or not
contiguous.  These tests call its validators directly with CPU tensors.
"""

import pytest
import torch

import block_scaled_fp8_x128_amd as fp8bs

CPU = torch.device("cpu")


def test_out_accepts_exact_match():
    t = torch.empty((4, 256), dtype=torch.uint8)
    assert fp8bs._out(t, (4, 256), fp8bs._CODE_DTYPES, CPU, "t") is t
    t8 = torch.empty((4, 256), dtype=torch.float8_e4m3fn)
    assert fp8bs._out(t8, (4, 256), fp8bs._CODE_DTYPES, CPU, "t") is t8


@pytest.mark.parametrize("bad", [
    torch.empty((3, 256), dtype=torch.uint8),            # too few rows
    torch.empty((4, 128), dtype=torch.uint8),            # too few columns
    torch.empty((4 * 256,), dtype=torch.uint8),          # right size, wrong shape
    torch.empty((4, 256), dtype=torch.int8),             # wrong dtype
    torch.empty((256, 4), dtype=torch.uint8).t(),        # not contiguous
    "not a tensor",
])
def test_out_rejects(bad):
    with pytest.raises(ValueError):
        fp8bs._out(bad, (4, 256), fp8bs._CODE_DTYPES, CPU, "t")


def test_out_rejects_other_device():
    t = torch.empty((4, 256), dtype=torch.uint8, device="meta")
    with pytest.raises(ValueError):
        fp8bs._out(t, (4, 256), fp8bs._CODE_DTYPES, CPU, "t")


def test_pair_out():
    q, s = fp8bs._pair_out(None, 5, 384, CPU)
    assert q.shape == (5, 384) and q.dtype == torch.uint8 and s.shape == (5, 3) and s.dtype == torch.float32
    good = (torch.empty((5, 384), dtype=torch.uint8), torch.empty((5, 3), dtype=torch.float32))
    assert fp8bs._pair_out(good, 5, 384, CPU) == good
    for bad in [(good[0],), (good[0], torch.empty((5, 2), dtype=torch.float32)),
                (good[0], torch.empty((5, 3), dtype=torch.bfloat16)),
                (torch.empty((5, 256), dtype=torch.uint8), good[1])]:
        with pytest.raises(ValueError):
            fp8bs._pair_out(bad, 5, 384, CPU)


def test_out_error_names_the_buffer():
    good = torch.empty((5, 384), dtype=torch.uint8)
    with pytest.raises(ValueError, match=r"out\[1\] \(xs\) must have shape \(5, 3\)"):
        fp8bs._pair_out((good, torch.empty((5, 2), dtype=torch.float32)), 5, 384, CPU)
    with pytest.raises(ValueError, match=r"out\[0\] \(hq\) must have dtype"):
        fp8bs._pair_out((torch.empty((5, 384), dtype=torch.int8), torch.empty((5, 3))), 5, 384, CPU, "hq", "hs")
    with pytest.raises(ValueError, match=r"^t must be contiguous$"):
        fp8bs._out(torch.empty((256, 4), dtype=torch.uint8).t(), (4, 256), fp8bs._CODE_DTYPES, CPU, "t")


def test_pointer_arguments_are_plain_ints():
    t = torch.empty(16, dtype=torch.uint8)
    assert fp8bs._ptr(t) == t.data_ptr() and fp8bs._ptr(None) is None


def test_w_and_dual_outs():
    w = torch.empty((256, 384), dtype=torch.bfloat16)
    wq, ws = fp8bs._w_out(None, w)
    assert wq.shape == (256, 384) and ws.shape == (2, 3)
    d = fp8bs._dual_outs(w)
    assert [tuple(t.shape) for t in d] == [(256, 384), (2, 3), (384, 256), (3, 2)]
    assert fp8bs._dual_outs(w, d) == d
    with pytest.raises(ValueError):   # W^T codes with W's shape
        fp8bs._dual_outs(w, (d[0], d[1], torch.empty((256, 384), dtype=torch.uint8), d[3]))
    with pytest.raises(ValueError):
        fp8bs._dual_outs(w, d[:3])
    with pytest.raises(ValueError):
        fp8bs._w_out((wq, torch.empty((3, 2), dtype=torch.float32)), w)


def test_y_out_dtype_follows_out_dtype():
    y = fp8bs._y_out(None, 3, 128, fp8bs.OUT_FP32, CPU)
    assert y.dtype == torch.float32 and y.shape == (3, 128)
    assert fp8bs._y_out(y, 3, 128, fp8bs.OUT_FP32, CPU) is y
    # a bf16 buffer with fp32 output requested would be written past its end
    with pytest.raises(ValueError):
        fp8bs._y_out(torch.empty((3, 128), dtype=torch.bfloat16), 3, 128, fp8bs.OUT_FP32, CPU)
    with pytest.raises(ValueError):
        fp8bs._y_out(torch.empty((2, 128), dtype=torch.bfloat16), 3, 128, fp8bs.OUT_BF16, CPU)


def test_workspace():
    assert fp8bs._workspace(None, 0, CPU) is None
    assert fp8bs._workspace(None, 64, CPU).numel() == 64
    with pytest.raises(ValueError):
        fp8bs._workspace(torch.empty((8, 8), dtype=torch.uint8).t(), 64, CPU)
    with pytest.raises(ValueError):
        fp8bs._workspace(torch.empty(64, dtype=torch.uint8, device="meta"), 64, CPU)


def test_same_device():
    a = torch.empty(1)
    fp8bs._same_device(CPU, ("a", a))
    with pytest.raises(ValueError):
        fp8bs._same_device(CPU, ("a", torch.empty(1, device="meta")))


def test_wrappers_reject_host_inputs():
    """Public wrappers refuse host tensors before anything reaches the library."""
    x = torch.zeros((4, 256), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fp8bs.quant_act_1x128(x)
    with pytest.raises(ValueError):
        fp8bs.fp8_block_gemm(torch.zeros((4, 256), dtype=torch.uint8), torch.ones((4, 2)),
                             torch.zeros((128, 256), dtype=torch.uint8), torch.ones((1, 2)))
