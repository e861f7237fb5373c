"""librr narrows float32 to bfloat16 with gfx950's conversion instruction
(one value, or two packed).  This checks it against the rounding rule the
oracle uses (round to nearest even on the bit pattern; NaN keeps sign and top
payload, quiet bit set) for all 2^32 float32 inputs, through the library's
own device functions (tests/hw/bf16_narrow_check.hip)."""

import ctypes
import os

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libbf16_narrow_check.so")


def test_bf16_narrowing_exhaustive():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.bf16_narrow_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.bf16_narrow_check.restype = ctypes.c_int
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(64, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    assert L.bf16_narrow_check(count.data_ptr(), first.data_ptr(), stream.cuda_stream) == 0
    torch.cuda.synchronize()
    n = int(count.item())
    rows = first.view(16, 4).cpu().tolist()[:min(n, 16)]
    forms = ("single", "packed low", "packed high")
    detail = [f"in 0x{r[0] & 0xFFFFFFFF:08x}: got 0x{r[1] & 0xFFFF:04x} want 0x{r[2] & 0xFFFF:04x} ({forms[r[3]]})"
              for r in rows]
    assert n == 0, f"{n} mismatches; first: {detail}"
