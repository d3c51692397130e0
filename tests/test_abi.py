"""Host-side checks of the C ABI (no GPU needed): libmxq.so loads, exports
every entry point include/mxq.h declares, validates arguments before touching
a device, and the Python binding fails loudly when the library is missing."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxq.h")
LIB = os.path.join(ROOT, "moe_grouped_gemm_mxq_amd", "libmxq.so")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        from moe_grouped_gemm_mxq_amd.build import build
        build()
    return ctypes.CDLL(LIB)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mxq_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["mxq_quantize", "mxq_quantize_grouped", "mxq_qdq_fp4", "mxq_gemm",
              "mxq_grouped_gemm", "mxq_validate_group_end", "mxq_last_error", "mxq_device_check"]:
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for n in declared_functions():
        assert hasattr(lib, n), f"libmxq.so does not export {n}"
    from moe_grouped_gemm_mxq_amd import mxq
    assert sorted(mxq.EXPORTED) == declared_functions()


def test_build_targets_gfx950_only():
    from moe_grouped_gemm_mxq_amd import build
    arch = [f for f in build.FLAGS if f.startswith("--offload-arch")]
    assert arch == ["--offload-arch=gfx950"]
    assert "-packed-fp32-ops" in build.FLAGS


def test_abi_version_and_pure_host_helpers(lib):
    lib.mxq_abi_version.restype = ctypes.c_int
    header = open(os.path.join(ROOT, "include", "mxq.h")).read()
    declared = int(re.search(r"#define MXQ_ABI_VERSION (\d+)", header).group(1))
    assert lib.mxq_abi_version() == declared
    from moe_grouped_gemm_mxq_amd import mxq
    assert mxq.ABI_VERSION == declared
    f = lib.mxq_grouped_cols_max
    f.restype = ctypes.c_int64
    f.argtypes = [ctypes.c_int64, ctypes.c_int32]
    # at least T + 31 G, an odd multiple of 256
    assert f(131072, 32) == 517 * 256
    assert f(1, 1) == 256
    assert f(0, 0) == 256
    for T, G in ((70, 6), (131072, 1), (256, 1), (513, 1024), (2 ** 31 - 1, 1024)):
        v = f(T, G)
        assert v >= T + 31 * G and v % 256 == 0 and (v // 256) % 2 == 1 and v - (T + 31 * G) < 512


def test_operand_sizes(lib):
    """Shape-only sizes of a quantised operand: codes rows x ceil32(K) bytes (E4M3)
    or half that (E2M1); scales ceil128(rows) x ceil32(K)/32 bytes, the binding's
    scale_shape; bad arguments are rejected."""
    from moe_grouped_gemm_mxq_amd import mxq
    fn = lib.mxq_operand_sizes
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    c, s = ctypes.c_int64(), ctypes.c_int64()
    for rows, K in [(1, 1), (33, 2), (128, 32), (129, 33), (131072, 7168), (7168, 131328)]:
        Kp = (K + 31) // 32 * 32
        sshape = mxq.scale_shape(rows, Kp // 32)
        for fmt, code in ((0, rows * Kp), (1, rows * Kp // 2)):
            assert fn(rows, K, fmt, ctypes.byref(c), ctypes.byref(s)) == 0
            assert c.value == code and s.value == sshape[0] * sshape[1] * sshape[2] * sshape[3]
        assert mxq.mxq_operand_sizes(rows, K) == (rows * Kp, s.value)
    assert fn(0, 32, 0, ctypes.byref(c), ctypes.byref(s)) == 1
    assert fn(4, 32, 7, ctypes.byref(c), ctypes.byref(s)) == 1
    assert fn(4, 32, 0, None, ctypes.byref(s)) == 1
    assert "NULL" in err(lib)


def call(lib, name, *args):
    fn = getattr(lib, name)
    fn.restype = ctypes.c_int
    return fn(*args)


def err(lib):
    lib.mxq_last_error.restype = ctypes.c_char_p
    return lib.mxq_last_error().decode()


P = ctypes.c_void_p
I64 = ctypes.c_int64
FAKE = P(0x1000)       # never dereferenced: validation fails before any device work


def test_invalid_arguments_are_rejected_on_the_host(lib):
    # NULL input
    assert call(lib, "mxq_quantize", P(0), I64(4), I64(32), I64(32), 1, FAKE, FAKE, P(0), P(0), P(0)) == 1
    assert "NULL" in err(lib)
    # bad sizes / axis / ldx
    assert call(lib, "mxq_quantize", FAKE, I64(0), I64(32), I64(32), 1, FAKE, FAKE, P(0), P(0), P(0)) == 1
    assert call(lib, "mxq_quantize", FAKE, I64(4), I64(32), I64(16), 1, FAKE, FAKE, P(0), P(0), P(0)) == 1
    assert call(lib, "mxq_quantize", FAKE, I64(4), I64(32), I64(32), 4, FAKE, FAKE, FAKE, FAKE, P(0)) == 1
    # misaligned code output
    assert call(lib, "mxq_quantize", FAKE, I64(4), I64(32), I64(32), 1, P(0x1001), FAKE, P(0), P(0), P(0)) == 1
    # misaligned row scales (the row quantiser stores them as dwords)
    assert call(lib, "mxq_quantize", FAKE, I64(4), I64(32), I64(32), 1, FAKE, P(0x1002), P(0), P(0), P(0)) == 1
    assert "s_row" in err(lib)
    assert call(lib, "mxq_quantize_batched", FAKE, I64(1), I64(4), I64(32), I64(32), I64(128), 1, FAKE,
                P(0x1001), P(0), P(0), P(0)) == 1
    assert call(lib, "mxq_quantize_grouped", FAKE, I64(64), I64(32), I64(32), FAKE, ctypes.c_int32(2),
                I64(64), 1, FAKE, P(0x1003), P(0), P(0), P(0)) == 1
    assert "s_row" in err(lib)
    # GEMM: K not a multiple of 32, ldc < N, bad format
    assert call(lib, "mxq_gemm", FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(4), I64(48), I64(4), 0, P(0)) == 1
    assert "multiple of 32" in err(lib)
    assert call(lib, "mxq_gemm", FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(8), I64(64), I64(4), 0, P(0)) == 1
    assert call(lib, "mxq_gemm", FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(4), I64(64), I64(4), 7, P(0)) == 2
    # code rows of 2^23 bytes or more (K >= 2^23 for E4M3, 2^24 for E2M1) are rejected
    for fmt, K in ((0, 1 << 23), (1, 1 << 24)):
        assert call(lib, "mxq_gemm", FAKE, FAKE, FAKE, FAKE, FAKE, I64(256), I64(256), I64(K), I64(256), fmt,
                    P(0)) == 1
        assert "MXQ_GEMM_MAX_ROW_BYTES" in err(lib)
        for mode in (0, 1):
            assert call(lib, "mxq_grouped_gemm", mode, FAKE, FAKE, FAKE, FAKE, FAKE, I64(256), I64(256), I64(K),
                        FAKE, ctypes.c_int32(2), fmt, P(0)) == 1
            assert "MXQ_GEMM_MAX_ROW_BYTES" in err(lib)
    # GEMM scale arrays are read as dwords
    assert call(lib, "mxq_gemm", FAKE, P(0x1002), FAKE, FAKE, FAKE, I64(4), I64(4), I64(64), I64(4), 0, P(0)) == 1
    assert "sA, sB" in err(lib)
    assert call(lib, "mxq_grouped_gemm", 0, FAKE, FAKE, FAKE, P(0x1001), FAKE, I64(4), I64(4), I64(64), FAKE,
                ctypes.c_int32(2), 0, P(0)) == 1
    assert "sA, sB" in err(lib)
    # grouped: G out of range, bad mode, ldq not a multiple of 32
    assert call(lib, "mxq_grouped_gemm", 0, FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(4), I64(64), FAKE,
                ctypes.c_int32(0), 0, P(0)) == 1
    assert call(lib, "mxq_grouped_gemm", 5, FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(4), I64(64), FAKE,
                ctypes.c_int32(2), 0, P(0)) == 1
    assert call(lib, "mxq_quantize_grouped", FAKE, I64(64), I64(32), I64(32), FAKE, ctypes.c_int32(2),
                I64(40), 2, P(0), P(0), FAKE, FAKE, P(0)) == 1
    assert call(lib, "mxq_qdq_fp4", FAKE, P(0), I64(2), I64(33), P(0), P(0), P(0)) == 1
    # batched: batch out of range, x_stride smaller than one matrix
    assert call(lib, "mxq_quantize_batched", FAKE, I64(0), I64(4), I64(32), I64(32), I64(128), 1, FAKE, FAKE,
                P(0), P(0), P(0)) == 1
    assert call(lib, "mxq_quantize_batched", FAKE, I64(70000), I64(4), I64(32), I64(32), I64(128), 1, FAKE,
                FAKE, P(0), P(0), P(0)) == 1
    assert call(lib, "mxq_quantize_batched", FAKE, I64(2), I64(4), I64(32), I64(32), I64(64), 1, FAKE, FAKE,
                P(0), P(0), P(0)) == 1
    assert "x_stride" in err(lib)
    assert call(lib, "mxq_validate_group_end", FAKE, ctypes.c_int32(2000), I64(5), FAKE, P(0)) == 1
    # MXFP4 with a scale factor: factor out of range, misaligned mask
    F32 = ctypes.c_float
    for sf in (0.0, -6.0, float("inf"), float("nan"), 2.0 ** 64, 2.0 ** -65, 1e-40):
        assert call(lib, "mxq_qdq_fp4_ex", FAKE, FAKE, I64(2), I64(64), F32(sf), P(0), P(0), P(0), P(0)) == 1
    assert "scale_factor" in err(lib)
    assert call(lib, "mxq_qdq_fp4_ex", FAKE, FAKE, I64(2), I64(64), F32(6.0), P(0), P(0), P(0x1002), P(0)) == 1
    # grouped token-axis MXFP4 operands: NULL, bad ldq, misaligned codes, bad factor, T >= 2^31
    assert call(lib, "mxq_quantize_fp4_grouped", P(0), I64(64), I64(8), I64(8), FAKE, ctypes.c_int32(2), I64(128),
                F32(6.0), FAKE, FAKE, P(0)) == 1
    assert call(lib, "mxq_quantize_fp4_grouped", FAKE, I64(64), I64(8), I64(8), FAKE, ctypes.c_int32(2), I64(100),
                F32(6.0), FAKE, FAKE, P(0)) == 1
    assert call(lib, "mxq_quantize_fp4_grouped", FAKE, I64(64), I64(8), I64(8), FAKE, ctypes.c_int32(2), I64(128),
                F32(6.0), P(0x1008), FAKE, P(0)) == 1
    assert call(lib, "mxq_quantize_fp4_grouped", FAKE, I64(64), I64(8), I64(8), FAKE, ctypes.c_int32(2), I64(128),
                F32(0.0), FAKE, FAKE, P(0)) == 1
    assert call(lib, "mxq_quantize_fp4_grouped", FAKE, I64(2 ** 31), I64(8), I64(8), FAKE, ctypes.c_int32(2),
                I64(128), F32(6.0), FAKE, FAKE, P(0)) == 1
    assert call(lib, "mxq_quantize_fp4", FAKE, I64(2), I64(64), F32(6.0), P(0x1008), FAKE, P(0)) == 1
    # STE backward: NULL mask, partial overlap of grad_x and grad_y
    assert call(lib, "mxq_ste_backward_fp4", FAKE, P(0), FAKE, I64(2), I64(64), P(0)) == 1
    assert call(lib, "mxq_ste_backward_fp4", P(0x1000), FAKE, P(0x1010), I64(2), I64(64), P(0)) == 1
    assert "overlap" in err(lib)


def _gpu_present():
    r = subprocess.run([sys.executable, "-c", "import torch; print(torch.cuda.device_count())"],
                       capture_output=True, text=True)
    return r.stdout.strip() not in ("", "0")


def test_valid_call_without_gfx950_reports_device_error(lib):
    if _gpu_present():
        pytest.skip("a GPU is present; this checks the no-device path")
    assert call(lib, "mxq_device_check", 0) == 3
    assert call(lib, "mxq_quantize", FAKE, I64(4), I64(32), I64(32), 1, FAKE, FAKE, P(0), P(0), P(0)) == 3
    assert err(lib)
    # E2M1 operands in both grouped modes and the grouped token-axis MXFP4
    # quantiser: well-formed, so they stop at the device gate
    assert call(lib, "mxq_grouped_gemm", 1, FAKE, FAKE, FAKE, FAKE, FAKE, I64(4), I64(4), I64(64), FAKE,
                ctypes.c_int32(2), 1, P(0)) == 3
    assert call(lib, "mxq_quantize_fp4_grouped", FAKE, I64(64), I64(8), I64(8), FAKE, ctypes.c_int32(2), I64(128),
                ctypes.c_float(6.0), FAKE, FAKE, P(0)) == 3
    # the largest K of each format passes the host checks
    for fmt, K in ((0, (1 << 23) - 32), (1, (1 << 24) - 32)):
        assert call(lib, "mxq_gemm", FAKE, FAKE, FAKE, FAKE, FAKE, I64(256), I64(256), I64(K), I64(256), fmt,
                    P(0)) == 3


def test_binding_fails_loudly_without_the_library(tmp_path):
    env = dict(os.environ, MXQ_LIB_PATH=str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", "import moe_grouped_gemm_mxq_amd.mxq"], cwd=ROOT,
                       env=env, capture_output=True, text=True)
    assert r.returncode != 0
    assert "RuntimeError" in r.stderr and "libmxq.so not found" in r.stderr


def _threshold(lib, sf):
    F, T = ctypes.c_int32(), ctypes.c_uint32()
    rc = call(lib, "mxq_fp4_scale_threshold", ctypes.c_float(sf), ctypes.byref(F), ctypes.byref(T))
    return rc, F.value, T.value


def _exact_threshold(sf):
    """F = floor(log2(sf*sqrt2)), T = ceil((sf*sqrt2/2^F - 1) * 2^23), from
    rationals: 4^F <= 2 sf^2 < 4^(F+1); T is the least integer with
    ((2^23 + T) / 2^23)^2 >= 2 sf^2 / 4^F."""
    from fractions import Fraction
    q = 2 * Fraction(sf) ** 2
    F = 0
    while Fraction(4) ** F > q:
        F -= 1
    while Fraction(4) ** (F + 1) <= q:
        F += 1
    r = q / Fraction(4) ** F                   # (1 + t)^2 in [1, 4)
    lo, hi = 0, 1 << 23                        # least T in [0, 2^23] with ((2^23+T)/2^23)^2 >= r
    while lo < hi:
        mid = (lo + hi) // 2
        if Fraction((1 << 23) + mid, 1 << 23) ** 2 >= r:
            hi = mid
        else:
            lo = mid + 1
    return F, lo


def test_fp4_scale_threshold_matches_exact_rationals(lib):
    import numpy as np
    assert _threshold(lib, 6.0) == (0, 3, 0x7C3B7)
    rng = np.random.default_rng(1)
    sfs = [1.0, 2.0 ** -64, float(np.nextafter(np.float32(2.0 ** 64), np.float32(0))), 0.75, 7.25, 12.0,
           float(np.float32(2 ** 0.5)), float(np.nextafter(np.float32(2 ** 0.5), np.float32(2))),
           float(np.nextafter(np.float32(2 ** 0.5), np.float32(0)))]
    sfs += [float(v) for v in (2.0 ** rng.uniform(-60, 60, 40)).astype(np.float32)]
    for sf in sfs:
        rc, F, T = _threshold(lib, sf)
        assert rc == 0 and (F, T) == _exact_threshold(sf), sf
    for sf in (0.0, -1.0, float("inf"), float("nan"), 2.0 ** 64, 1e-30):
        assert _threshold(lib, sf)[0] == 1


def test_fp4_exponent_rule_from_threshold_matches_oracle(lib):
    """The kernels' exponent rule E - F + (mantissa >= T), clamped at -30,
    applied to the host helper's (F, T), gives the oracle's scale bytes."""
    import numpy as np
    import oracle
    rng = np.random.default_rng(4)
    for sf in (6.0, 5.0, 0.75, 13.5, 1.0):
        _, F, T = _threshold(lib, sf)
        x = (rng.standard_normal((64, 32)) * 2.0 ** rng.integers(-40, 40, (64, 1))).astype(np.float32)
        _, _, s, _ = oracle.mxfp4_qdq_ex(x, sf)
        amax = np.abs(x).max(axis=1).view(np.uint32).astype(np.int64)
        e = (amax >> 23) - 127 - F + ((amax & 0x7FFFFF) >= T)
        e = np.where(amax >> 23 == 0, -30, np.maximum(e, -30))
        assert np.array_equal(s[:, 0].astype(np.int64) - 127, e), sf


def test_binding_constants_match_the_header():
    """Constants the binding mirrors from include/mxq.h."""
    import re
    from moe_grouped_gemm_mxq_amd import mxq as m
    text = open(os.path.join(ROOT, "include", "mxq.h")).read()
    define = lambda name: eval(re.search(rf"#define {name} (.+?)(?:\s*/\*|\n)", text).group(1))
    assert define("MXQ_ABI_VERSION") == m.ABI_VERSION
    assert define("MXQ_MAX_GROUPS") == m.MAX_GROUPS
    assert define("MXQ_BLOCK") == m.BLOCK
    assert define("MXQ_GEMM_MAX_ROW_BYTES") == m.MAX_ROW_BYTES == 1 << 23
