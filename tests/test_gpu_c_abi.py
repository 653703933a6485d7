"""The C ABI driven from a plain C program (tests/c_abi_check.c, built by
exact_second_order_amd.build with gcc against include/flashbob.h and
libflashbob.so): device memory from hipMalloc, no torch on the GPU side. Its
outputs are compared with the fp64 oracle on seeded inputs, both dtypes, with
and without the causal mask (ragged N)."""

import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from exact_second_order_amd import build
from helpers import NAMES, TOL, make_inputs, rel_fro, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("causal", [0, 1], ids=["full", "causal"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["f32", "bf16"])
def test_plain_c_caller(tmp_path, dtype, causal):
    if not os.path.exists(build.C_CHECK):
        pytest.fail(f"{build.C_CHECK} is missing: run python -m exact_second_order_amd.build")
    B, H, N, d, s = 1, 2, 300, 64, 0.125
    say(f"[c-abi] {dtype} causal={causal}")
    ins = make_inputs(B, H, N, d, dtype, seed=1900 + causal)
    for k in NAMES:  # raw little-endian bits, as the C program reads them
        raw = ins[k].contiguous().view(torch.int16 if dtype == torch.bfloat16 else torch.int32).numpy()
        raw.tofile(str(tmp_path / f"{k}.bin"))
    code = 1 if dtype == torch.bfloat16 else 0
    r = subprocess.run([build.C_CHECK, str(B), str(H), str(N), str(d), str(code), repr(s), str(causal),
                        str(tmp_path), str(tmp_path)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    xs = [ins[k].to(torch.float64).numpy() for k in NAMES]
    ref = oracle.bob(*xs, s, causal=bool(causal))
    for k, name in enumerate(("gradQ", "gradK", "gradV", "graddO")):
        got = np.fromfile(str(tmp_path / f"{name}.bin"), dtype=np.float32).reshape(B, H, N, d)
        assert rel_fro(got, ref[k]) <= TOL[dtype], name
