"""librr narrows float32 to bfloat16 and binary16 with gfx950's conversion
instructions (one value, or two packed).  This checks them against the
rounding rules the oracle uses, written out on the bit pattern in
tests/hw/narrow16_check.hip, for all 2^32 float32 inputs, through the
library's own device functions.  The binary16 rule there was itself checked
against oracle.fp16.narrow over all 2^32 inputs on the CPU."""

import ctypes
import os

import pytest

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

LIB = os.path.join(os.path.dirname(os.path.abspath(__file__)), "hw", "libnarrow16_check.so")
FORMS = ("bfloat16 single", "bfloat16 packed low", "bfloat16 packed high", "binary16 single",
         "binary16 packed low", "binary16 packed high")


def test_narrowing_exhaustive():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    if not os.path.exists(LIB):
        pytest.fail(f"{LIB} is not built (run __graft_entry__.build())")
    L = ctypes.CDLL(LIB)
    L.narrow16_check.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.narrow16_check.restype = ctypes.c_int
    count = torch.zeros(1, dtype=torch.int64, device="cuda")
    first = torch.zeros(64, dtype=torch.int32, device="cuda")
    assert L.narrow16_check(count.data_ptr(), first.data_ptr(), torch.cuda.current_stream().cuda_stream) == 0
    torch.cuda.synchronize()
    n = int(count.item())
    rows = first.view(16, 4).cpu().tolist()[:min(n, 16)]
    detail = [f"in 0x{r[0] & 0xFFFFFFFF:08x}: got 0x{r[1] & 0xFFFF:04x} want 0x{r[2] & 0xFFFF:04x} ({FORMS[r[3]]})"
              for r in rows]
    assert n == 0, f"{n} mismatches; first: {detail}"
