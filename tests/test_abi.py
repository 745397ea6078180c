"""The C ABI library loads, exports every function include/pn.h declares, and rejects bad
arguments with the documented status codes before touching the device (host logic only)."""
import ctypes as C
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(pn_\w+)\s*\(", text, flags=re.M)))


@pytest.fixture(scope="module")
def pn():
    import block_quantized_weight_pn3t_amd as pn
    return pn


def test_header_declares_the_entry_points():
    names = declared_functions()
    for must in ("pn_validate_row", "pn_dequantize_row", "pn_gemv", "pn_gemv_nvfp4",
                 "pn_quantize_rows", "pn_validate_rows", "pn_dequantize_rows"):
        assert must in names


def test_library_exports_every_declared_symbol(pn):
    lib = C.CDLL(pn.library_path)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_row_bytes(pn):
    assert pn.row_bytes(pn.PN3T, 5120) == 64 * 34
    assert pn.row_bytes(pn.PN4T, 17408) == 272 * 34
    assert pn.row_bytes(pn.PN3T, 6144) == 0
    assert pn.row_bytes(pn.PN4T, 0) == 0
    assert pn.row_bytes(7, 640) == 0


def test_argument_errors_are_reported_before_any_device_work(pn):
    L = pn.lib()
    P = C.c_void_p
    fake = P(0x1000)  # never dereferenced: every call below fails its argument checks
    assert L.pn_gemv(7, fake, 4, 640, fake, 1, fake, None) == -1          # PN_ERR_TYPE
    assert L.pn_gemv(124, fake, 4, 650, fake, 1, fake, None) == -2        # K not whole blocks
    assert L.pn_gemv(124, fake, 4, 0, fake, 1, fake, None) == -2          # K = 0
    assert L.pn_gemv(124, fake, -1, 640, fake, 1, fake, None) == -2       # negative N
    assert L.pn_gemv(124, fake, 4, 640, fake, 17, fake, None) == -3       # M > 16
    assert L.pn_gemv(124, fake, 4, 640, fake, -1, fake, None) == -3
    assert L.pn_gemv(124, fake, 0, 640, fake, 1, fake, None) == 0         # N = 0: no-op
    assert L.pn_gemv(124, fake, 4, 640, fake, 0, fake, None) == 0         # M = 0: no-op
    assert L.pn_gemv(124, None, 4, 640, fake, 1, fake, None) == -4        # NULL W
    assert L.pn_gemv(124, P(0x1001), 4, 640, fake, 1, fake, None) == -5   # W odd address
    assert L.pn_gemv(124, fake, 4, 640, P(0x1002), 1, fake, None) == -5   # x not 4-aligned
    assert L.pn_validate_rows(125, fake, 3, 100, fake, None) == -2
    assert L.pn_dequantize_rows(124, None, 3, 80, fake, None) == -4
    assert L.pn_quantize_rows(124, fake, 2, 81, fake, None, None) == -2
    assert L.pn_gemv_nvfp4(fake, fake, C.c_float(1.0), 4, 24, fake, 1, fake, None) == -2
    assert L.pn_gemv_nvfp4(fake, fake, C.c_float(1.0), 4, 32, fake, 9, fake, None) == -3
    assert L.pn_gemv_nvfp4(fake, fake, C.c_float(1.0), 4, 32, fake, 5, fake, None) == -3
    assert L.pn_gemv_fp8row(fake, fake, 4, 32, fake, 5, fake, None) == -3
    assert L.pn_gemv_nvfp4(P(0x1004), fake, C.c_float(1.0), 4, 32, fake, 1, fake, None) == -5
    assert L.pn_nvfp4_validate_rows(fake, C.c_float(1.0), 4, 8, fake, None) == -2
    # Hadamard rotation and the fused GEMV
    assert L.pn_hadamard_rows(fake, 1, 640, 3, fake, None) == -8       # B not a power of two
    assert L.pn_hadamard_rows(fake, 1, 640, 256, fake, None) == -8     # B does not divide K
    assert L.pn_hadamard_rows(fake, 1, 32768, 32768, fake, None) == -8  # B above 16384
    assert L.pn_hadamard_rows(fake, 1, 640, 1, fake, None) == -8       # B = 1
    assert L.pn_hadamard_rows(fake, 1, 6, 2, fake, None) == -2         # K not a multiple of 4
    assert L.pn_hadamard_rows(fake, -1, 640, 64, fake, None) == -2
    assert L.pn_hadamard_rows(fake, 0, 640, 64, fake, None) == 0       # M = 0: no-op
    assert L.pn_hadamard_rows(None, 1, 640, 64, fake, None) == -4
    assert L.pn_hadamard_rows(fake, 1, 640, 64, P(0x1002), None) == -5
    assert L.pn_gemv_hadamard(124, fake, 4, 640, fake, 5, 64, fake, None) == -3  # M above 4
    assert L.pn_gemv_hadamard(124, fake, 4, 640, fake, 1, 256, fake, None) == -8
    assert L.pn_gemv_hadamard(124, fake, 4, 650, fake, 1, 64, fake, None) == -2
    assert L.pn_gemv_hadamard(7, fake, 4, 640, fake, 1, 64, fake, None) == -1
    assert L.pn_gemv_hadamard(124, fake, 0, 640, fake, 1, 64, fake, None) == 0
    # the entry point that allocates nothing: the same checks, plus its array's size limit
    na = L.pn_gemv_hadamard_noalloc
    assert na(124, fake, 4, 640, fake, 5, 64, fake, None) == -3
    assert na(124, fake, 4, 640, fake, 1, 256, fake, None) == -8
    assert na(7, fake, 4, 640, fake, 1, 64, fake, None) == -1
    assert na(125, fake, 4, 65600, fake, 4, 64, fake, None) == -2      # M * K above 262,144
    assert na(125, fake, 4, 131136, fake, 2, 64, fake, None) == -2
    assert na(125, fake, 0, 65536, fake, 4, 1024, fake, None) == 0     # 262,144 floats: in range
    assert na(124, P(0x1001), 4, 640, fake, 1, 64, fake, None) == -5
    assert L.pn_gemv_hadamard(124, None, 4, 640, fake, 1, 64, fake, None) == -4
    # several GEMVs that share x
    Part = pn.GemvPart

    def group(parts, K=640, x=fake, M=1, count=None):
        arr = (Part * max(len(parts), 1))(*parts)
        return L.pn_gemv_group(arr if parts else None, len(parts) if count is None else count,
                               K, x, M, None)
    ok = Part(124, 0x1000, 4, 0x2000)
    assert group([ok], count=0) == -2                                  # no parts
    assert group([ok] * 5) == -2                                       # above the maximum
    assert group([]) == -2
    assert L.pn_gemv_group(None, 2, 640, fake, 1, None) == -4           # NULL parts
    assert group([ok, Part(7, 0x1000, 4, 0x2000)]) == -1               # a bad type
    assert group([ok, Part(125, 0x1000, 4, 0x2000)], K=560) == -2      # K not whole pn4t blocks
    assert group([ok, Part(124, 0x1000, -1, 0x2000)]) == -2            # negative N
    assert group([ok], M=17) == -3
    assert group([ok], M=0) == 0                                       # M = 0: no-op
    assert group([Part(124, 0, 0, 0), Part(125, 0, 0, 0)], K=320) == 0  # every N = 0: no-op
    assert group([ok, Part(124, 0, 4, 0x2000)]) == -4                  # NULL W
    assert group([ok, Part(124, 0x1001, 4, 0x2000)]) == -5             # W odd address
    assert group([ok, Part(124, 0x1000, 4, 0x2002)]) == -5             # y not 4-aligned
    assert group([ok], x=P(0x1002)) == -5                              # x not 4-aligned
    assert group([ok], x=None) == -4
    hg = lambda parts, B=64, M=1, K=640: L.pn_gemv_group_hadamard(
        (Part * len(parts))(*parts), len(parts), K, fake, M, B, None)
    assert hg([ok], B=3) == -8                                         # B not a power of two
    assert hg([ok], B=256) == -8                                       # B does not divide K
    assert hg([ok], M=5) == -3                                         # above 4 tokens
    assert hg([ok, Part(7, 0x1000, 4, 0x2000)]) == -1
    assert hg([ok], M=0) == 0
    assert L.pn_gemv_group_hadamard(None, 1, 640, fake, 1, 64, None) == -4
    for s in (0, -1, -2, -3, -4, -5, -6, -7, -8, -99):
        assert isinstance(pn.status_string(s), str)
