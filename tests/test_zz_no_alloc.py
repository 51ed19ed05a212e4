"""dory_sample_static (no allocation: scratch in the library's fixed device array) against
dory_sample (library-allocated scratch) through the C ABI: the same ids (integer results, bit-exact)
on two calls in a row, the second smaller, and both against the oracle's sampler."""
import ctypes as C
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

from looped_ngpt_language_amd import dory  # noqa: E402
from oracle.sampling import sample_row  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def call(fn, logits, us, t, p):
    rows, v = logits.shape
    ids = torch.full((rows,), -1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    r = fn(logits.data_ptr(), rows, v, C.c_float(t), C.c_float(p), us.data_ptr(), ids.data_ptr(),
           C.c_void_p(st.cuda_stream))
    assert r == dory.DORY_OK
    torch.cuda.synchronize()
    return ids.cpu().numpy()


@pytest.mark.parametrize("t,p", [(1.0, 0.95), (0.7, 1.0), (0.0, 0.95)])
def test_static_scratch_matches_allocating_sampler(t, p):
    lib = dory.lib()
    g = torch.Generator(device="cuda:0").manual_seed(17)
    for rows, v in ((96, 131072), (5, 32768)):    # two calls in a row, the second smaller
        logits = (torch.randn(rows, v, device="cuda:0", generator=g) * 2).contiguous()
        us = torch.rand(rows, device="cuda:0", generator=g)
        a = call(lib.dory_sample, logits, us, t, p)
        b = call(lib.dory_sample_static, logits, us, t, p)
        say(f"[sample static] rows={rows} V={v} T={t} p={p}: ids equal {int(np.sum(a == b))}/{rows}")
        np.testing.assert_array_equal(a, b)
        host = logits.double().cpu().numpy()
        uh = us.double().cpu().numpy()
        for r in range(0, rows, max(1, rows // 8)):
            assert b[r] == sample_row(host[r], t, p, float(uh[r]))
