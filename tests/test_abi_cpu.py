"""C-ABI checks that need no GPU: the library loads, exports every function
that include/flashbob.h declares, and rejects bad arguments with the documented
error codes before making any HIP call (fake, never-dereferenced pointers)."""

import ctypes
import os
import re

import pytest

from exact_second_order_amd import flashbob as fb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "flashbob.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fb.LIB_PATH), reason="libflashbob.so not built")

F32, BF16 = fb.FLASHBOB_F32, fb.FLASHBOB_BF16
OK, NULL, SHAPE, UD, DT, ALIGN, WS, ALIAS, SCALE = 0, -1, -2, -3, -5, -6, -7, -8, -9


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(flashbob_\w+)\s*\(", text)))


def test_noalloc_limits_match_the_header():
    text = open(HEADER).read()
    for name in ("FLASHBOB_NOALLOC_MAX_ROWS", "FLASHBOB_NOALLOC_SCRATCH_BYTES"):
        m = re.search(r"#define\s+%s\s+\((\d+)u?\s*<<\s*(\d+)\)" % name, text)
        assert m, name
        assert int(m.group(1)) << int(m.group(2)) == getattr(fb, name)


def test_header_declares_expected_entry_points():
    assert header_functions() == sorted(fb.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(fb.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_library_exports_nothing_else():
    """The dynamic symbol table holds exactly the header's entry points (the
    build hides everything else: kernels, helpers, compiler globals)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--defined-only", fb.LIB_PATH], capture_output=True, text=True, check=True).stdout
    names = sorted({ln.split()[-1] for ln in out.splitlines() if ln.strip()})
    assert names == header_functions()


def test_version_and_strerror():
    lib = fb.load_library()
    assert lib.flashbob_version() == 104
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -9, -10, -11, -100, 12345):
        s = lib.flashbob_strerror(code)
        assert isinstance(s, bytes) and len(s) > 0


def test_workspace_bytes():
    lib = fb.load_library()
    assert lib.flashbob_workspace_bytes(1, 1, 128, 64) == 2048
    assert lib.flashbob_workspace_bytes(1, 4, 65536, 64) == 4 * 4 * 4 * 65536
    assert lib.flashbob_workspace_bytes(1, 1, 3, 64) == 256  # rounded up
    assert lib.flashbob_workspace_bytes(0, 1, 128, 64) == 0
    assert lib.flashbob_workspace_bytes(1, 1, -1, 64) == 0


# fake device addresses: 16-byte aligned, disjoint, never dereferenced
BASE = 1 << 40
STRIDE = 1 << 32


def fake_args(B=1, H=1, N=128, d=64, dtype=F32, scale=0.125, ws=None):
    ins = [BASE + i * STRIDE for i in range(7)]
    outs = [BASE + (7 + i) * STRIDE for i in range(4)]
    wsp = BASE + 11 * STRIDE
    nws = fb.load_library().flashbob_workspace_bytes(B, H, N, d) if ws is None else ws
    return ins, outs, B, H, N, d, scale, dtype, wsp, nws


def call(ins, outs, B, H, N, d, scale, dtype, wsp, nws):
    return fb.raw_bob(ins, outs, B, H, N, d, scale, dtype, wsp, nws)


@pytest.mark.parametrize("d", [0, 16, 48, 63, 100, 160, 256])
def test_rejects_unsupported_d(d):
    a = list(fake_args())
    a[5] = d
    assert call(*a) == UD


def test_head_dim_256_bf16_only():
    # bf16 at d = 256 passes the head-dim check (and stops at the missing
    # workspace); fp32 at d = 256 is refused
    assert call(*fake_args(d=256, dtype=BF16, ws=0)) == WS
    assert call(*fake_args(d=256, dtype=F32, ws=0)) == UD


def test_rejects_negative_sizes_and_overflow():
    for idx in (2, 3, 4):
        a = list(fake_args())
        a[idx] = -1
        assert call(*a) == SHAPE
    a = list(fake_args(B=1 << 20, H=1 << 10, N=1 << 20, d=128))
    assert call(*a) == SHAPE


def test_rejects_bad_dtype_and_scale():
    a = list(fake_args())
    a[7] = 7
    assert call(*a) == DT
    # the dtype is checked before the head dim (which head dims exist depends
    # on it): an unknown dtype reports the dtype, whatever d is
    for d in (256, 48):
        a = list(fake_args(d=d))
        a[7] = 7
        assert call(*a) == DT
    for bad in (float("nan"), float("inf"), -float("inf")):
        a = list(fake_args())
        a[6] = bad
        assert call(*a) == SCALE


def test_rejects_null_pointers():
    for k in range(7):
        a = list(fake_args())
        a[0] = list(a[0])
        a[0][k] = 0
        assert call(*a) == NULL
    for k in range(4):
        a = list(fake_args())
        a[1] = list(a[1])
        a[1][k] = 0
        assert call(*a) == NULL
    a = list(fake_args())
    a[8] = 0
    assert call(*a) == NULL


def test_rejects_misaligned_pointers():
    a = list(fake_args())
    a[0] = list(a[0])
    a[0][3] += 8
    assert call(*a) == ALIGN
    a = list(fake_args())
    a[1] = list(a[1])
    a[1][2] += 4
    assert call(*a) == ALIGN


def test_rejects_small_workspace():
    a = fake_args(ws=1024)
    assert call(*a) == WS


def test_rejects_aliasing_outputs():
    a = list(fake_args())
    a[1] = list(a[1])
    a[1][0] = a[0][0]  # gradQ on top of Q
    assert call(*a) == ALIAS
    a = list(fake_args())
    a[1] = list(a[1])
    a[1][1] = a[1][0] + 64  # gradK overlaps gradQ
    assert call(*a) == ALIAS
    a = list(fake_args())
    a[8] = a[1][3] + 16  # workspace inside graddO
    assert call(*a) == ALIAS


def test_inputs_may_alias_each_other():
    # read-only inputs may share memory; the call then fails only because
    # there is no device here, which must surface as ERR_HIP, not as a
    # validation error. Skipped when a GPU is present (it would launch).
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on a real device with fake pointers")
    a = list(fake_args())
    a[0] = [a[0][0]] * 7
    rc = call(*a)
    assert rc == -100


def test_empty_problem_is_a_noop():
    for B, H, N in ((0, 1, 128), (1, 0, 128), (1, 1, 0)):
        a = list(fake_args(B=B, H=H, N=N))
        a[0] = [0] * 7  # even NULL pointers are fine when there is nothing to do
        a[1] = [0] * 4
        a[8] = 0
        assert call(*a) == OK


def test_rowstats_validation():
    lib = fb.load_library()
    vp = ctypes.c_void_p
    ins = [vp(BASE + i * STRIDE) for i in range(7)]
    outs = [vp(BASE + (7 + i) * STRIDE) for i in range(4)]
    assert lib.flashbob_rowstats(*ins, *outs, 1, 1, 128, 80, ctypes.c_float(0.1), F32, vp(0)) == UD
    bad = list(outs)
    bad[2] = vp(0)
    assert lib.flashbob_rowstats(*ins, *bad, 1, 1, 128, 64, ctypes.c_float(0.1), F32, vp(0)) == NULL
    bad = list(outs)
    bad[1] = vp(BASE + 7 * STRIDE + 4)
    assert lib.flashbob_rowstats(*ins, *bad, 1, 1, 128, 64, ctypes.c_float(0.1), F32, vp(0)) == ALIGN


# fake dQ, dK, dV (first backward outputs) past the workspace slot
FIRST = [BASE + (12 + i) * STRIDE for i in range(3)]


# a fake saved log-sum-exp input after those
LSE = BASE + 15 * STRIDE


def call_ex(ins, outs, B, H, N, d, scale, dtype, wsp, nws, flags=0, stages=7, hkv=None, first=(0, 0, 0), lse=0):
    lib = fb.load_library()
    vp = ctypes.c_void_p
    return lib.flashbob_bob_ex(*[vp(p) for p in ins], *[vp(p) for p in outs], *[vp(p) for p in first], vp(lse),
                               B, H, H if hkv is None else hkv, N, d, ctypes.c_float(scale), dtype, flags, stages,
                               vp(wsp), ctypes.c_size_t(nws), vp(0))


def test_ex_rejects_unknown_flags_and_stage_sets():
    FLAGS = -10
    for flags in (16, 17, 32, -1, 1 << 20):
        assert call_ex(*fake_args(), flags=flags, first=FIRST, lse=LSE) == FLAGS
    for stages in (0, 8, 9, -1, 16):
        assert call_ex(*fake_args(), stages=stages) == FLAGS
    # the flags check comes first, the shape checks still apply after it
    a = list(fake_args())
    a[5] = 80
    assert call_ex(*a, flags=1, stages=7) == UD
    lib = fb.load_library()
    vp = ctypes.c_void_p
    ins = [vp(BASE + i * STRIDE) for i in range(7)]
    outs = [vp(BASE + (7 + i) * STRIDE) for i in range(4)]
    assert lib.flashbob_rowstats_ex(*ins, *outs, 1, 1, 1, 128, 64, ctypes.c_float(0.1), F32, 2, vp(0)) == FLAGS


def test_ex_empty_problem_is_a_noop():
    # B*H*N == 0 returns OK before any HIP call, with or without the mask
    for flags in range(16):
        assert call_ex(*fake_args(B=0), flags=flags) == 0


def test_ex_first_backward_output_checks():
    # with FLASHBOB_FIRST_BACKWARD the dQ, dK, dV pointers are outputs like
    # the others: NULL, misaligned and aliased ones are rejected; without it
    # they are ignored, so NULL passes the checks (the call then fails only
    # for want of a device)
    import torch
    FB = fb.FLASHBOB_FIRST_BACKWARD
    for k in range(3):
        first = list(FIRST)
        first[k] = 0
        assert call_ex(*fake_args(), flags=FB, first=first) == NULL
        first[k] = FIRST[k] + 4
        assert call_ex(*fake_args(), flags=FB | 1, first=first) == ALIGN
        a = fake_args()
        first[k] = a[0][3] + 16          # inside dO
        assert call_ex(*a, flags=FB, first=first) == ALIAS
        first[k] = a[1][k]               # on top of gradQ / gradK / gradV
        assert call_ex(*a, flags=FB, first=first) == ALIAS
    a = fake_args()
    assert call_ex(*a, flags=FB, first=(FIRST[0], FIRST[0], FIRST[2])) == ALIAS
    assert call_ex(*a, flags=FB, first=(a[8], FIRST[1], FIRST[2])) == ALIAS  # on the workspace
    if torch.cuda.is_available():
        return  # the calls below would launch kernels on fake pointers
    assert call_ex(*fake_args(), flags=FB, first=FIRST) == -100
    assert call_ex(*fake_args(), flags=0, first=(0, 0, 0)) == -100


def test_ex_rejects_bad_kv_head_counts():
    for H, hkv in ((4, 0), (4, 3), (4, 5), (4, -1), (6, 4)):
        assert call_ex(*fake_args(H=H), hkv=hkv) == SHAPE, (H, hkv)
    lib = fb.load_library()
    vp = ctypes.c_void_p
    ins = [vp(BASE + i * STRIDE) for i in range(7)]
    outs = [vp(BASE + (7 + i) * STRIDE) for i in range(4)]
    assert lib.flashbob_rowstats_ex(*ins, *outs, 1, 4, 3, 128, 64, ctypes.c_float(0.1), F32, 0, vp(0)) == SHAPE


def test_ex_alias_check_uses_kv_sizes():
    # with H = 4, H_kv = 1 the key/value tensors are a quarter of the query
    # ones: gradK placed right after K's (smaller) extent is legal (the call
    # then fails only for want of a device: skipped where one exists, as it
    # would launch on fake pointers), and overlapping it is caught
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on a real device with fake pointers")
    B, H, N, d = 1, 4, 128, 64
    ins, outs, *_ = fake_args(B=B, H=H, N=N, d=d)
    nws = fb.load_library().flashbob_workspace_bytes(B, H, N, d)
    kv_bytes = B * 1 * N * d * 4
    ins = list(ins)
    outs = list(outs)
    outs[1] = ins[1] + kv_bytes            # gradK starts where K ends
    assert call_ex(ins, outs, B, H, N, d, 0.1, F32, BASE + 11 * STRIDE, nws, hkv=1) == -100
    outs[1] = ins[1] + kv_bytes - 16       # one chunk of overlap
    assert call_ex(ins, outs, B, H, N, d, 0.1, F32, BASE + 11 * STRIDE, nws, hkv=1) == -8


def test_ex_saved_lse_checks():
    # FLASHBOB_SAVED_LSE makes lse_in an input: NULL, misaligned (it is read
    # as 4-byte scalars) and overlapping an output are rejected; without the
    # flag it is ignored
    import torch
    SV = fb.FLASHBOB_SAVED_LSE
    a = fake_args()
    assert call_ex(*a, flags=SV, lse=0) == NULL
    assert call_ex(*a, flags=SV | 1, lse=LSE + 2) == ALIGN
    assert call_ex(*a, flags=SV, lse=a[1][0] + 64) == ALIAS      # inside gradQ
    assert call_ex(*a, flags=SV, lse=a[8]) == ALIAS              # on the workspace
    assert call_ex(*a, flags=SV | 2, lse=FIRST[1] + 4, first=FIRST) == ALIAS  # inside dK
    if torch.cuda.is_available():
        return  # the calls below would launch kernels on fake pointers
    assert call_ex(*a, flags=SV, lse=LSE + 4) == -100   # 4-byte aligned is enough
    assert call_ex(*a, flags=SV, lse=a[0][0]) == -100   # reading an input's memory is no hazard
    assert call_ex(*a, flags=0, lse=LSE + 1) == -100    # ignored without the flag


def test_ex_bf16_outputs_use_two_byte_sizes():
    # with FLASHBOB_BF16_OUTPUTS every output is half as large: an output
    # placed right after another's bf16 extent is legal (the call then fails
    # only for want of a device), the same placement overlaps float32 outputs
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch kernels on a real device with fake pointers")
    B, H, N, d = 1, 1, 128, 64
    ins, outs, *rest = fake_args(B=B, H=H, N=N, d=d)
    outs = list(outs)
    outs[1] = outs[0] + B * H * N * d * 2   # gradK right after a bf16 gradQ
    a = (ins, outs, *rest)
    assert call_ex(*a, flags=fb.FLASHBOB_BF16_OUTPUTS) == -100
    assert call_ex(*a, flags=0) == ALIAS


def test_plain_c_caller_is_built_and_checks_its_arguments():
    # the C program of tests/c_abi_check.c (built with the library) refuses a
    # bad command line before making any HIP call
    import subprocess
    from exact_second_order_amd import build
    assert os.path.exists(build.C_CHECK), "run python -m exact_second_order_amd.build"
    r = subprocess.run([build.C_CHECK], capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "usage" in r.stderr
    r = subprocess.run([build.C_CHECK, "1", "1", "0", "64", "0", "0.1", "0", "/nonexistent", "/nonexistent"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2 and "bad arguments" in r.stderr


def test_noalloc_checks_arguments_and_its_limit_before_any_hip_call():
    """flashbob_bob_noalloc rejects bad arguments, and problems larger than
    its static buffer, with error codes and without touching the device
    (fake pointers, no GPU here)."""
    lib = fb.load_library()
    ins = [BASE + i * STRIDE for i in range(7)]
    outs = [BASE + (7 + i) * STRIDE for i in range(4)]

    def noalloc(B, H, N, d, scale=0.125, dtype=F32, outs=outs, ins=ins):
        return lib.flashbob_bob_noalloc(*[ctypes.c_void_p(p) for p in ins], *[ctypes.c_void_p(p) for p in outs],
                                        B, H, N, d, ctypes.c_float(scale), dtype, None)
    limit = fb.FLASHBOB_NOALLOC_MAX_ROWS
    assert noalloc(1, 1, limit + 1, 64) == -11        # FLASHBOB_ERR_SCRATCH
    assert noalloc(2, 4, limit // 8 + 1, 64) == -11
    assert noalloc(1, 1, 128, 48) == UD
    assert noalloc(1, 1, 128, 64, dtype=7) == DT
    assert noalloc(1, 1, 128, 64, scale=float("nan")) == SCALE
    assert noalloc(1, 1, 128, 64, outs=[outs[0], outs[0], outs[2], outs[3]]) == ALIAS
    assert noalloc(1, 1, 128, 64, outs=[outs[0], 0, outs[2], outs[3]]) == NULL
    assert noalloc(1, 1, 128, 64, ins=[ins[0] + 8] + ins[1:]) == ALIGN
    assert noalloc(0, 1, 128, 64) == OK               # empty problem: nothing to do
    assert b"1048576" in lib.flashbob_strerror(-11)
