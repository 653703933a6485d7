"""GPU check of flashbob_bob_noalloc (the entry point that allocates nothing:
its row scalars live in a static device buffer of the library) against
flashbob_bob, through the C ABI: bitwise equal outputs on two calls in a row,
the second one smaller, for both input dtypes."""

import ctypes
import math

import pytest
import torch

from exact_second_order_amd import flashbob as fb
from exact_second_order_amd.inputs import NAMES, make_inputs

from helpers import say

pytestmark = pytest.mark.gpu


def _ptrs(ts):
    return [ctypes.c_void_p(t.data_ptr()) for t in ts]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_noalloc_matches_flashbob_bob_two_calls(dtype):
    lib = fb.load_library()
    dt = fb.FLASHBOB_BF16 if dtype == torch.bfloat16 else fb.FLASHBOB_F32
    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    # the second call is smaller and ragged: it must not see the first one's
    # row scalars (the static buffer keeps the last call's contents)
    for (B, H, N, d, seed) in ((2, 3, 777, 64, 11), (1, 2, 130, 64, 12)):
        say(f"[noalloc] {dtype} B={B} H={H} N={N} d={d}")
        ins = make_inputs(B, H, N, d, dtype, seed=seed)
        x = [ins[k].cuda() for k in NAMES]
        scale = 1.0 / math.sqrt(d)
        ref = [torch.empty(x[0].shape, dtype=torch.float32, device="cuda") for _ in range(4)]
        got = [torch.full(x[0].shape, float("nan"), dtype=torch.float32, device="cuda") for _ in range(4)]
        ws = torch.empty(lib.flashbob_workspace_bytes(B, H, N, d), dtype=torch.uint8, device="cuda")
        rc = lib.flashbob_bob(*_ptrs(x), *_ptrs(ref), B, H, N, d, ctypes.c_float(scale), dt,
                              ctypes.c_void_p(ws.data_ptr()), ctypes.c_size_t(ws.numel()), sh)
        assert rc == 0, rc
        rc = lib.flashbob_bob_noalloc(*_ptrs(x), *_ptrs(got), B, H, N, d, ctypes.c_float(scale), dt, sh)
        assert rc == 0, rc
        torch.cuda.synchronize()
        for g, r in zip(got, ref):
            assert torch.equal(g, r)
    # the Python wrapper goes through the same entry point
    out = fb.bob_noalloc(*x, scale=scale)
    torch.cuda.synchronize()
    for g, r in zip(out, ref):
        assert torch.equal(g, r)
