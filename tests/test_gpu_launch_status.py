"""A call's status is its own launch's status.

The library takes each launch's status from hipLaunchKernel's return value.
An error that an earlier, unrelated HIP call left on the host thread must
neither come back as PA_ERR_HIP from a call that launched fine nor be
cleared by it: the caller still finds it with hipGetLastError afterwards
(fail early and surface asynchronous errors where they belong -- "Hardware
abstraction and portability", §六 and §九).  The planted error is an invalid
device ordinal passed to hipSetDevice, which touches no GPU state.
"""

import ctypes
import math

import numpy as np
import pytest
import torch

from gpu_helpers import DecodeOnGPU, require_gpu
from workloads import make_decode_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hip():
    require_gpu()
    # the runtime torch loaded (libpa.so resolves to the same SONAME)
    rt = ctypes.CDLL("libamdhip64.so.7")
    rt.hipSetDevice.argtypes = [ctypes.c_int]
    rt.hipSetDevice.restype = ctypes.c_int
    rt.hipGetLastError.restype = ctypes.c_int
    rt.hipGetDevice.argtypes = [ctypes.POINTER(ctypes.c_int)]
    rt.hipGetDevice.restype = ctypes.c_int
    return rt


def _plant(rt):
    err = rt.hipSetDevice(9999)
    assert err != 0, "hipSetDevice accepted an invalid ordinal"
    return err


@pytest.mark.parametrize("part", [0, 64])
def test_earlier_error_is_neither_reported_nor_cleared(hip, part):
    import paged_kv_cache_24_amd as pa
    c = make_decode_case(name="status", seed=61, dtype="f16", num_q_heads=8, num_kv_heads=2,
                         head_dim=128, seq_lens=[300, 17, 5], num_blocks=32, max_blocks_per_seq=20,
                         scale=1 / math.sqrt(128), write_last=True)
    g = DecodeOnGPU(c)
    need = pa.pa_decode_workspace_size(c.num_seqs, 8, 2, 128, 16, c.max_blocks_per_seq, part)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    torch.cuda.synchronize()

    # the runtime must keep an error across a successful call, or there is nothing to test
    planted = _plant(hip)
    dev = ctypes.c_int(-1)
    assert hip.hipGetDevice(ctypes.byref(dev)) == 0
    kept = hip.hipGetLastError()
    if kept != planted:
        pytest.skip(f"this HIP runtime does not keep an earlier error ({kept} after {planted})")

    planted = _plant(hip)
    status = pa.lib.pa_reshape_and_cache(g.key.data_ptr(), g.value.data_ptr(), g.k_cache.data_ptr(),
                                         g.v_cache.data_ptr(), g.slots.data_ptr(),
                                         len(c.slot_mapping), 2, 128, 16, c.num_blocks, 0, stream)
    assert status == 0 and hip.hipGetLastError() == planted

    args = (g.out.data_ptr(), g.q.data_ptr(), g.k_cache.data_ptr(), g.v_cache.data_ptr(),
            g.tables.data_ptr(), g.lens.data_ptr(), c.num_seqs, 8, 2, 128, 16,
            c.max_blocks_per_seq, c.num_blocks, c.scale, 0, part, 0, ws.data_ptr(), ws.numel(),
            stream)
    planted = _plant(hip)
    status = pa.lib.pa_decode(*args)                # partitions, then merge when it splits
    after = hip.hipGetLastError()
    assert status == 0, f"a launch that succeeded reported {status} ({pa.pa_status_string(status)})"
    assert after == planted, f"the earlier error was cleared ({after} instead of {planted})"
    assert hip.hipGetLastError() == 0
    torch.cuda.synchronize()
    assert np.isfinite(g.out.float().cpu().numpy()).all()
