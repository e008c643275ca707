"""The C-ABI library loads, exports what include/fa.h declares, and rejects bad arguments
before touching the GPU (CPU only: no call here reaches a kernel launch)."""
import ctypes
import os
import re
import subprocess

import pytest

import exact_attention_126_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

# Fake device addresses: validation fails before any of these could be dereferenced.
P = 0x100000
P_MIS = 0x100008  # 8-byte aligned only
BF16, F32 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F32


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:fa_status_t|size_t|const char\*)\s+(fa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    # FA_ABI_TEST_LIB: another build of the same C ABI to run these cases against (the host-only
    # sanitizer build of tests/test_host_sanitizer.py)
    other = os.environ.get("FA_ABI_TEST_LIB")
    if other:
        fa._lib = None
        fa.LIB_PATH = other
    if not os.path.exists(fa.LIB_PATH):
        pytest.fail("libfa.so is not built (python -m exact_attention_126_amd.build)")
    return fa.lib()


def test_exports_every_declared_symbol(L):
    declared = _declared()
    assert declared == sorted(fa.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", fa.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\sT\s(fa_\w+)$", out, re.M))
    assert set(declared) <= exported
    for name in declared:
        assert hasattr(L, name)


def test_single_hip_runtime_mapped(L):
    maps = open("/proc/self/maps").read()
    hip = {ln.split()[-1] for ln in maps.splitlines() if "libamdhip64" in ln}
    assert len(hip) == 1, hip


def test_status_strings(L):
    for code in range(9):
        s = fa.fa_status_string(code)
        assert s and s != "unknown status"
    assert fa.fa_status_string(99) == "unknown status"


def fwd(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=1, Nq=128, Nk=128, d=64, causal=0, scale=0.125, dtype=BF16):
    vp = ctypes.c_void_p
    return L.fa_fwd(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None, vp(o) if o else None,
                    vp(lse) if lse else None, B, H, Nq, Nk, d, causal, scale, dtype, None)


def test_fwd_validation(L):
    assert fwd(L, q=0) == 1 and fwd(L, lse=0) == 1
    assert fwd(L, d=96) == 4 and fwd(L, d=256) == 4 and fwd(L, dtype=7) == 4
    assert fwd(L, k=P_MIS) == 2 and fwd(L, o=P + 4) == 2 and fwd(L, lse=P + 2) == 2
    assert fwd(L, lse=P + 4, scale=0.0) == 7  # a 4-byte aligned lse passes the alignment check
    assert fwd(L, B=0) == 3 and fwd(L, H=-1) == 3 and fwd(L, Nq=0) == 3 and fwd(L, Nk=0) == 3
    assert fwd(L, causal=1, Nq=128, Nk=256) == 3
    assert fwd(L, Nq=2**31 // 128, d=128) == 3  # one head beyond 2^31 bytes
    assert fwd(L, B=2**20, H=2**20) == 3
    assert fwd(L, scale=0.0) == 7 and fwd(L, scale=-1.0) == 7 and fwd(L, scale=float("inf")) == 7
    assert fwd(L, scale=float("nan")) == 7


def fwd_ex(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=4, H_kv=2, Nq=128, Nk=256, d=64, mask=1, scale=0.125, dtype=BF16):
    vp = ctypes.c_void_p
    return L.fa_fwd_ex(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None, vp(o) if o else None,
                       vp(lse) if lse else None, B, H, H_kv, Nq, Nk, d, mask, scale, dtype, None)


def test_fwd_ex_validation(L):
    assert fwd_ex(L, k=0) == 1
    assert fwd_ex(L, d=80) == 4 and fwd_ex(L, dtype=5) == 4
    assert fwd_ex(L, v=P_MIS) == 2
    assert fwd_ex(L, H_kv=0) == 3 and fwd_ex(L, H_kv=3) == 3 and fwd_ex(L, H_kv=8) == 3  # must divide H
    assert fwd_ex(L, mask=2, Nq=300, Nk=200) == 3  # bottom-right: the first rows would see no key
    assert fwd_ex(L, mask=3) == 7 and fwd_ex(L, mask=-1) == 7
    assert fwd_ex(L, scale=0.0) == 7
    assert fwd_ex(L, B=2**20, H=2**20, H_kv=2**20) == 3
    # shapes fa_fwd rejects but fa_fwd_ex accepts: validation passes, and with no GPU in this
    # process the device query then fails (FA_ERR_HIP) before anything could be launched
    no_gpu = 6
    assert fwd(L, causal=1, Nq=128, Nk=256) == 3
    assert fwd_ex(L, mask=1, Nq=128, Nk=256) in (0, no_gpu)
    assert fwd_ex(L, mask=1, Nq=300, Nk=200) in (0, no_gpu)
    assert fwd_ex(L, mask=2, Nq=200, Nk=300) in (0, no_gpu)
    assert fwd_ex(L, H_kv=1, mask=0) in (0, no_gpu) and fwd_ex(L, H_kv=4, mask=0) in (0, no_gpu)


def split_ex(L, q=P, k=P, v=P, ws=P, wsb=None, B=2, H=4, H_kv=2, Nk=100, d=128, scale=0.1, S=4, dtype=BF16):
    vp = ctypes.c_void_p
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(B, H, d, S) if S > 0 else 0
    return L.fa_decode_split_ex(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None,
                                vp(ws) if ws else None, wsb, B, H, H_kv, Nk, d, scale, S, dtype, None)


def test_decode_split_ex_validation(L):
    assert split_ex(L, ws=0) == 1
    assert split_ex(L, d=32) == 4
    assert split_ex(L, k=P_MIS) == 2
    assert split_ex(L, H_kv=0) == 3 and split_ex(L, H_kv=3) == 3 and split_ex(L, H_kv=8) == 3
    assert split_ex(L, S=0, wsb=1 << 20) == 7 and split_ex(L, S=101) == 7
    assert split_ex(L, wsb=fa.fa_decode_workspace_bytes(2, 4, 128, 4) - 1) == 5


def split_fp8(L, q=P, k=P, v=P, ks=P, vs=P, ws=P, wsb=None, B=2, H=4, H_kv=2, Nk=100, d=128, scale=0.1, S=4):
    vp = ctypes.c_void_p
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(B, H, d, S) if S > 0 else 0
    ptr = lambda x: vp(x) if x else None  # noqa: E731
    return L.fa_decode_split_fp8kv(ptr(q), ptr(k), ptr(v), ptr(ks), ptr(vs), ptr(ws), wsb, B, H, H_kv, Nk, d, scale,
                                   S, None)


def test_decode_split_fp8kv_validation(L):
    assert split_fp8(L, ks=0) == 1 and split_fp8(L, vs=0) == 1 and split_fp8(L, k=0) == 1
    assert split_fp8(L, d=96) == 4
    assert split_fp8(L, v=P_MIS) == 2 and split_fp8(L, ks=P + 2) == 2
    assert split_fp8(L, H_kv=0) == 3 and split_fp8(L, H_kv=3) == 3 and split_fp8(L, Nk=0) == 3
    assert split_fp8(L, S=0, wsb=1 << 20) == 7 and split_fp8(L, S=101) == 7
    assert split_fp8(L, scale=float("nan")) == 7
    assert split_fp8(L, wsb=fa.fa_decode_workspace_bytes(2, 4, 128, 4) - 1) == 5


def fwd_fp8(L, q=P, k=P, v=P, qs=P, ks=P, vs=P, o=P, lse=P, B=2, H=4, H_kv=2, Nq=100, Nk=100, d=128, mask=0,
            scale=0.1):
    vp = ctypes.c_void_p
    ptr = lambda x: vp(x) if x else None  # noqa: E731
    return L.fa_fwd_fp8(ptr(q), ptr(k), ptr(v), ptr(qs), ptr(ks), ptr(vs), ptr(o), ptr(lse), B, H, H_kv, Nq, Nk, d,
                        mask, scale, None)


def test_fwd_fp8_validation(L):
    assert fwd_fp8(L, qs=0) == 1 and fwd_fp8(L, vs=0) == 1 and fwd_fp8(L, lse=0) == 1
    assert fwd_fp8(L, mask=3) == 7 and fwd_fp8(L, scale=0.0) == 7
    assert fwd_fp8(L, d=32) == 4
    assert fwd_fp8(L, o=P_MIS) == 2 and fwd_fp8(L, ks=P + 1) == 2
    assert fwd_fp8(L, H_kv=3) == 3 and fwd_fp8(L, Nq=0) == 3
    assert fwd_fp8(L, mask=2, Nq=200, Nk=100) == 3
    assert fwd_fp8(L, Nk=(1 << 31) // 128 + 1) == 3


def test_decode_workspace_bytes(L):
    assert fa.fa_decode_workspace_bytes(16, 32, 128, 64) == 16 * 32 * 64 * 130 * 4
    assert fa.fa_decode_workspace_bytes(0, 32, 128, 64) == 0
    assert fa.fa_decode_workspace_bytes(1, 1, 64, 0) == 0


def split(L, q=P, k=P, v=P, ws=P, wsb=None, B=2, H=3, Nk=100, d=128, scale=0.1, S=4, dtype=BF16):
    vp = ctypes.c_void_p
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(B, H, d, S) if S > 0 else 0
    return L.fa_decode_split(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None,
                             vp(ws) if ws else None, wsb, B, H, Nk, d, scale, S, dtype, None)


def test_decode_split_validation(L):
    assert split(L, ws=0) == 1 and split(L, q=0) == 1
    assert split(L, d=32) == 4 and split(L, dtype=3) == 4
    assert split(L, ws=P + 8) == 2 and split(L, v=P_MIS) == 2
    assert split(L, Nk=0) == 3 and split(L, B=0) == 3
    assert split(L, S=0, wsb=1 << 20) == 7 and split(L, S=101) == 7 and split(L, scale=0.0) == 7
    need = fa.fa_decode_workspace_bytes(2, 3, 128, 4)
    assert split(L, wsb=need - 1) == 5


def combine(L, ws=P, wsb=None, o=P, lse=P, B=2, H=3, d=64, S=4, dtype=F32):
    vp = ctypes.c_void_p
    if wsb is None:
        wsb = fa.fa_decode_workspace_bytes(B, H, d, S) if S > 0 else 0
    return L.fa_decode_combine(vp(ws) if ws else None, wsb, vp(o) if o else None, vp(lse) if lse else None,
                               B, H, d, S, dtype, None)


def test_decode_combine_validation(L):
    assert combine(L, o=0) == 1 and combine(L, lse=0) == 1
    assert combine(L, d=100) == 4
    assert combine(L, o=P + 8) == 2
    assert combine(L, H=0) == 3
    assert combine(L, S=0, wsb=1 << 20) == 7
    assert combine(L, wsb=fa.fa_decode_workspace_bytes(2, 3, 64, 4) - 4) == 5


def noalloc(L, q=P, k=P, v=P, o=P, lse=P, B=2, H=4, H_kv=2, Nk=1000, d=128, scale=0.125, S=16, dtype=BF16):
    vp = ctypes.c_void_p
    return L.fa_decode_noalloc(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None,
                               vp(o) if o else None, vp(lse) if lse else None, B, H, H_kv, Nk, d, scale, S, dtype,
                               None)


def test_decode_noalloc_validation(L):
    """Every check, the scratch limit included, is taken before the first HIP call."""
    assert noalloc(L, q=0) == 1 and noalloc(L, o=0) == 1 and noalloc(L, lse=0) == 1
    assert noalloc(L, d=96) == 4 and noalloc(L, dtype=3) == 4
    assert noalloc(L, o=P + 8) == 2 and noalloc(L, lse=P + 2) == 2 and noalloc(L, k=P_MIS) == 2
    assert noalloc(L, H=3) == 3 and noalloc(L, B=0) == 3 and noalloc(L, Nk=0) == 3
    assert noalloc(L, S=0) == 7 and noalloc(L, S=1001) == 7 and noalloc(L, scale=float("nan")) == 7
    # the largest split count whose partials fit the 32 MiB scratch, and one more
    B, H, d = 16, 32, 128
    s_max = fa.DECODE_NOALLOC_SCRATCH_BYTES // (B * H * (d + 2) * 4)
    assert fa.fa_decode_workspace_bytes(B, H, d, s_max) <= fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert fa.fa_decode_workspace_bytes(B, H, d, s_max + 1) > fa.DECODE_NOALLOC_SCRATCH_BYTES
    assert noalloc(L, B=B, H=H, H_kv=H, Nk=32768, d=d, S=s_max + 1) == 8
    assert noalloc(L, B=1024, H=64, H_kv=8, Nk=32768, d=128, S=64) == 8


def masked(L, q=P, k=P, v=P, o=P, lse=P, B=1, H=4, H_kv=2, Nq=300, Nk=500, d=128, mask=P, ws=P, wsb=1 << 20,
           scale=0.125, dtype=BF16):
    vp = ctypes.c_void_p
    return L.fa_fwd_masked(vp(q) if q else None, vp(k) if k else None, vp(v) if v else None, vp(o) if o else None,
                           vp(lse) if lse else None, B, H, H_kv, Nq, Nk, d, vp(mask) if mask else None,
                           vp(ws) if ws else None, wsb, scale, dtype, None)


def test_fwd_masked_validation(L):
    # two 256-row blocks of 8 tiles: counts (2 x 4 bytes, padded to 16), classes (2 x 8 bytes), lists
    # (2 x 8 x 2 bytes), the forward's claim counter (16 bytes)
    assert fa.fa_fwd_masked_workspace_bytes(300, 500) == 16 + 16 + 2 * 8 * 2 + 16
    # 3 blocks of 3 tiles: counts 12 -> 16, classes 9 -> 16, lists 18 -> 32, counter 16
    assert fa.fa_fwd_masked_workspace_bytes(700, 150) == 16 + 16 + 32 + 16
    assert fa.fa_fwd_masked_workspace_bytes(0, 500) == 0 and fa.fa_fwd_masked_workspace_bytes(10, 131073) == 0
    assert masked(L, mask=0) == 1 and masked(L, ws=0) == 1 and masked(L, q=0) == 1
    assert masked(L, dtype=F32) == 4 and masked(L, d=96) == 4
    assert masked(L, mask=P + 4) == 2 and masked(L, ws=P + 8) == 2 and masked(L, o=P + 8) == 2
    assert masked(L, mask=P + 8) in (0, 6)  # 8-byte aligned mask words are enough
    assert masked(L, H_kv=3) == 3 and masked(L, Nq=0) == 3 and masked(L, Nk=131073) == 3
    assert masked(L, scale=float("inf")) == 7
    assert masked(L, wsb=fa.fa_fwd_masked_workspace_bytes(300, 500) - 1) == 5


def test_binding_combine_checks_output_shapes():
    """The combine writes B*H LSE values and B*H*d outputs, with B, H and d taken from o: a short
    lse or an o that is not [B,H,1,d] is rejected before the library is called."""
    import torch
    ws = torch.zeros(fa.fa_decode_workspace_bytes(2, 3, 64, 4) // 4)
    o = torch.zeros(2, 3, 1, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_decode_combine(ws, o, torch.zeros(2, 2, 1), 4)
    with pytest.raises(ValueError, match="lse"):
        fa.fa_decode_combine(ws, o, torch.zeros(6), 4)
    with pytest.raises(ValueError, match="o "):
        fa.fa_decode_combine(ws, torch.zeros(2, 3, 2, 64, dtype=torch.bfloat16), torch.zeros(2, 3, 1), 4)
    with pytest.raises(ValueError, match="o "):
        fa.fa_decode_combine(ws, torch.zeros(6, 64, dtype=torch.bfloat16), torch.zeros(2, 3, 1), 4)
    with pytest.raises(ValueError, match="device"):  # right shapes, host memory
        fa.fa_decode_combine(ws, o, torch.zeros(2, 3, 1), 4)


def test_binding_rejects_host_tensors():
    import torch
    q = torch.zeros(1, 1, 8, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        fa.attention(q, q, q)


def test_calibration_library_loads_and_validates():
    """libfa_calib.so (the sustained MFMA-rate probe the benchmark reports beside the nominal
    peak) loads, sizes its buffers and rejects bad arguments without launching."""
    path = os.path.join(ROOT, "exact_attention_126_amd", "libfa_calib.so")
    if not os.path.exists(path):
        pytest.fail("libfa_calib.so is not built (python -m exact_attention_126_amd.build)")
    C = ctypes.CDLL(path)
    C.fa_calib_src_bytes.argtypes = [ctypes.c_int]
    C.fa_calib_src_bytes.restype = ctypes.c_size_t
    C.fa_calib_out_floats.argtypes = [ctypes.c_int]
    C.fa_calib_out_floats.restype = ctypes.c_size_t
    C.fa_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    C.fa_calib_mfma.restype = ctypes.c_int
    assert C.fa_calib_src_bytes(256) == 256 * 8 * 64 * 16
    assert C.fa_calib_out_floats(256) == 256 * 256
    assert C.fa_calib_src_bytes(0) == 0
    nb, nf = C.fa_calib_src_bytes(4), C.fa_calib_out_floats(4)
    assert C.fa_calib_mfma(None, nb, P, nf, P, 4, 8, None) == -1         # null operand buffer
    assert C.fa_calib_mfma(P, nb - 16, P, nf, P, 4, 8, None) == -1       # operand buffer too small
    assert C.fa_calib_mfma(P, nb, P, nf - 1, P, 4, 8, None) == -1        # output buffer too small
    assert C.fa_calib_mfma(P_MIS, nb, P, nf, P, 4, 8, None) == -1        # misaligned operands
    assert C.fa_calib_mfma(P, nb, P, nf, P, 4, 6, None) == -1            # niter not a multiple of 4
    assert C.fa_calib_mfma(P, nb, P, nf, P, 0, 8, None) == -1            # empty grid


def bwd(L, q=P, k=P, v=P, o=P, do=P, lse=P, dq=P, dk=P, dv=P, ws=P, wsb=None, B=1, H=4, H_kv=2, Nq=128, Nk=256, d=128,
        mask=1, scale=0.1, dtype=BF16):
    vp = ctypes.c_void_p
    if wsb is None:
        wsb = fa.fa_bwd_workspace_bytes(B, H, Nq) if B > 0 and H > 0 and Nq > 0 else 0
    ptr = lambda x: vp(x) if x else None
    return L.fa_bwd(ptr(q), ptr(k), ptr(v), ptr(o), ptr(do), ptr(lse), ptr(dq), ptr(dk), ptr(dv), ptr(ws), wsb, B, H,
                    H_kv, Nq, Nk, d, mask, scale, dtype, None)


def test_bwd_validation(L):
    assert fa.fa_bwd_workspace_bytes(2, 3, 100) == 2 * 3 * 100 * 2 * 4
    assert fa.fa_bwd_workspace_bytes(0, 3, 100) == 0
    assert bwd(L, do=0) == 1 and bwd(L, ws=0) == 1 and bwd(L, lse=0) == 1
    assert bwd(L, dtype=F32) == 4 and bwd(L, d=96) == 4
    assert bwd(L, dk=P_MIS) == 2 and bwd(L, lse=P + 2) == 2 and bwd(L, ws=P + 8) == 2
    assert bwd(L, mask=5) == 7 and bwd(L, scale=0.0) == 7
    assert bwd(L, H_kv=3) == 3 and bwd(L, Nq=0) == 3 and bwd(L, mask=2, Nq=300, Nk=200) == 3
    assert bwd(L, B=2**12, H=2**12, H_kv=2**12, Nq=2**10, wsb=1 << 40) == 3  # workspace offsets beyond 32 bits
    assert bwd(L, wsb=fa.fa_bwd_workspace_bytes(1, 4, 128) - 4) == 5
    assert bwd(L) in (0, 6)  # valid: with no GPU in this process the launch reports FA_ERR_HIP


def test_poisoned_build_loads_and_exports_the_same_abi():
    """libfa_poison.so (the FA_DEBUG_POISON_LDS=1 build) exports every declared entry point, and
    its argument checks answer like the normal library's without launching."""
    from exact_attention_126_amd import build as fa_build
    if not os.path.exists(fa_build.POISON_LIB):
        pytest.fail("libfa_poison.so is not built (python -m exact_attention_126_amd.build)")
    out = subprocess.run(["nm", "-D", "--defined-only", fa_build.POISON_LIB], capture_output=True,
                         text=True).stdout
    assert set(_declared()) <= set(re.findall(r"\sT\s(fa_\w+)$", out, re.M))
    Lp = fa.load_library(fa_build.POISON_LIB)
    i64 = ctypes.c_int64
    for args in ((None, P, P, P, P, 1, 2, 64, 64, 128, BF16, 0.1, 1, None),   # null q
                 (P, P, P, P, P, 1, 2, 64, 64, 96, BF16, 0.1, 1, None),       # unsupported head dim
                 (P_MIS, P, P, P, P, 1, 2, 64, 64, 128, BF16, 0.1, 1, None)):  # misaligned q
        assert Lp.fa_fwd(*args) == fa.lib().fa_fwd(*args) != fa.FA_OK
    assert Lp.fa_bwd_workspace_bytes(i64(2), i64(3), i64(100)) == fa.lib().fa_bwd_workspace_bytes(2, 3, 100)
