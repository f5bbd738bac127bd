"""pa_decode_noalloc (the library's own per-GPU workspace, no allocation)
against pa_decode with a workspace, through the C ABI (needs a gfx950 GPU).

Two calls in a row on the same GPU array, the second with a smaller batch:
both must equal pa_decode bit for bit (same kernels, same grid) and match
the oracle within the attention tolerance; a shape whose workspace exceeds
the array is rejected."""

import numpy as np
import pytest

import parity_log
import workloads as W
from oracle_driver import OracleCache

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2, "f16": 6e-3}


def _case(w):
    import torch
    import gpu_driver as gd
    oc = OracleCache(w).run()
    gc = gd.GpuCache(w).run()
    tables, lens = gc.tables()
    q = gd.to_torch(w.q, w.dtype, gc.device)
    return oc, gc, q, torch.from_numpy(tables).to(gc.device), torch.from_numpy(lens).to(gc.device)


def _check(w, sl):
    """Decodes sequences sl of w both ways; returns the max-abs error vs the oracle."""
    import torch
    import gpu_driver as gd
    import paged_kv_cache_338_amd as pa
    oc, gc, q, td, ld = _case(w)
    q, td, ld = q[sl].contiguous(), td[sl].contiguous(), ld[sl].contiguous()
    want_ws = torch.empty_like(q)
    pa.pa_decode(q, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, want_ws)
    got = torch.full_like(q, float("nan"))
    pa.pa_decode_noalloc(q, gc.k_cache, gc.v_cache, td, ld, w.block_size, w.scale, got)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int16), want_ws.view(torch.int16))
    want = oc.decode()[sl]
    err = parity_log.within(gd.widen_out(got, w.dtype), want, TOL[w.dtype], w.dtype)
    return err


def test_noalloc_two_calls_second_smaller():
    w = W.llama3_8b_decode()
    e1 = _check(w, slice(0, 8))  # the worked batch: cut segments merge in the array
    e2 = _check(w, slice(2, 5))  # then a smaller batch on the same array
    print(f"max-abs error vs oracle: {e1:.3g} (8 sequences), {e2:.3g} (3 sequences)")


def test_noalloc_serving_then_tiny():
    w = W.serving_batch()
    _check(w, slice(0, 256))
    _check(W.tiny_ref(), slice(0, 4))


def test_noalloc_rejects_a_workspace_beyond_its_array():
    # 8192 sequences x 1024 KV heads need 64 MiB of arrival counters, more
    # than the array's 4 MiB counter region: the call is refused on the host
    # before any pointer is used, so placeholder addresses serve.
    import ctypes
    import paged_kv_cache_338_amd as pa
    lib = pa.load_library()
    d = pa.CacheDesc(4, 16, 1024, 64, pa.PA_BF16)
    assert pa.pa_decode_workspace_size(d, 8192, 1024, 1) > 64 << 20
    fake = ctypes.c_void_p(4096)
    st = lib.pa_decode_noalloc(fake, fake, fake, fake, 1, fake, 8192, 16, 0.125, fake, 1024,
                               ctypes.byref(d), None)
    assert st == pa.PA_ERR_UNSUPPORTED
    assert b"device array" in lib.pa_last_error()
