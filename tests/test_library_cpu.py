"""CPU-side checks of libfp8bs.so: it loads, exports every symbol the header
declares, and rejects invalid arguments on the host before any launch.  Also
the exhaustive host proof of the quantizers' division shortcut.  No kernel is
launched here (there is no GPU in this tier).
"""
import ctypes
import os
import re
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]


@pytest.fixture(scope="module")
def lib():
    from fine_grained_fp8_amd import _lib, build
    sanitized = os.environ.get("FP8BS_SANITIZED_LIB")
    if sanitized:
        # the host-only sanitizer build of the same validation code (see
        # test_validation_layer_under_asan_ubsan)
        return _lib.load_library(sanitized)
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load_library()


def declared_functions():
    text = "".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("fp8_quant_act_1x128", "fp8_quant_weight_128x128", "fp8_block_gemm",
                     "fp8_block_gemm_grouped", "fp8_status_string", "fp8_abi_version"):
        assert required in names


def test_exports_every_declared_symbol(lib):
    from fine_grained_fp8_amd import _lib
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, f"binding does not declare {name}"
    nm = shutil.which("nm")
    if nm:
        out = subprocess.run([nm, "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                             text=True).stdout
        exported = set(re.findall(r"\bT (fp8_[a-z0-9_]+)", out))
        assert set(declared_functions()) <= exported


def test_abi_version_and_status_strings(lib):
    assert lib.fp8_abi_version() == 1
    for s in range(9):
        assert len(lib.fp8_status_string(s)) > 0
    assert lib.fp8_status_string(99) == b"unknown status"


# Fake, well-separated 16-byte-aligned "device" addresses: validation fails
# before any HIP call, so they are never dereferenced.
X, Q, S, S2, A, B, C = (0x10000000 * (i + 1) for i in range(7))
OK, NULL, SHAPE, LD, ALIGN, UNSUP, DEVICE, LAUNCH, ALIAS = range(9)


def qa(lib, x=X, rows=64, cols=256, ldx=256, d=0, q=Q, ldq=256, s=S, ld_s=64, s_in=None, amax=None,
       sat=None):
    return lib.fp8_quant_act_1x128(x, rows, cols, ldx, d, q, ldq, s, ld_s, s_in, amax, sat, None)


def test_quant_act_validation(lib):
    assert qa(lib, x=None) == NULL
    assert qa(lib, q=None) == NULL
    assert qa(lib, s=None) == NULL
    assert qa(lib, cols=200, ldx=256) == SHAPE
    assert qa(lib, rows=-1) == SHAPE
    assert qa(lib, d=7) == UNSUP
    assert qa(lib, d=1, rows=100) == SHAPE                    # COL needs rows % 128
    assert qa(lib, d=1, rows=128, s_in=S2) == UNSUP            # caller scales: ROW only
    assert qa(lib, ldx=128) == LD
    assert qa(lib, ldq=128) == LD
    assert qa(lib, ld_s=32) == LD
    assert qa(lib, x=X + 8) == ALIGN
    assert qa(lib, ldq=264) == ALIGN
    assert qa(lib, q=X) == ALIAS
    assert qa(lib, s=X + 64) == ALIAS
    assert qa(lib, rows=0, x=None) == OK                       # empty: no-op
    assert qa(lib, cols=0, x=None) == OK


def test_quant_weight_validation(lib):
    f = lib.fp8_quant_weight_128x128
    assert f(X, 256, 256, 256, Q, 256, None, 0, S, 2, None) in (DEVICE, OK)
    assert f(X, 200, 256, 256, Q, 256, None, 0, S, 2, None) == SHAPE
    assert f(None, 256, 256, 256, Q, 256, None, 0, S, 2, None) == NULL
    assert f(X, 256, 256, 256, Q, 256, A, 128, S, 2, None) == LD
    assert f(X, 256, 256, 256, Q, 256, None, 0, S, 1, None) == LD
    assert f(X, 256, 256, 256, X + 1024, 256, None, 0, S, 2, None) == ALIAS


def gemm(lib, layout=0, M=256, N=256, K=512, a=A, lda=512, sa=S, ld_sa=256, b=B, ldb=512, sb=S2,
         ld_sb=4, c=C, dt=0, ldc=256):
    return lib.fp8_block_gemm(layout, M, N, K, a, lda, sa, ld_sa, b, ldb, sb, ld_sb, c, dt, ldc, None)


def test_gemm_validation(lib):
    assert gemm(lib, layout=7) == UNSUP
    assert gemm(lib, layout=-1) == UNSUP
    assert gemm(lib, dt=5) == UNSUP
    assert gemm(lib, K=200, lda=256) == SHAPE
    assert gemm(lib, K=0) == SHAPE
    assert gemm(lib, N=200, ldc=256) == SHAPE                 # FPROP weights need N % 128
    assert gemm(lib, M=0, a=None) == OK
    assert gemm(lib, a=None) == NULL
    assert gemm(lib, lda=256) == LD
    assert gemm(lib, ld_sa=100) == LD
    assert gemm(lib, ld_sb=2) == LD
    assert gemm(lib, c=C + 4) == ALIGN
    assert gemm(lib, ldc=260) == ALIGN                        # bf16 row stride not 16-byte aligned
    assert gemm(lib, c=A + 4096) == ALIAS
    # DGRAD: B stored [K][N], block scales [K/128][N/128]
    assert gemm(lib, layout=1, ldb=128, ld_sb=2) == LD
    assert gemm(lib, layout=1, ldb=256, ld_sb=1) == LD
    # DGRAD_T: B = W_q^T [N][K], the forward block scales [K/128][N/128]
    assert gemm(lib, layout=3, N=200, ldc=256) == SHAPE
    assert gemm(lib, layout=3, ldb=256) == LD
    assert gemm(lib, layout=3, ld_sb=1) == LD
    assert gemm(lib, layout=3, ld_sb=2) in (DEVICE, OK)
    # *_TILED: B holds dense tiles, so ldb must equal K
    assert gemm(lib, layout=4, ldb=528) == LD
    assert gemm(lib, layout=4, N=200, ldc=256) == SHAPE
    assert gemm(lib, layout=4) in (DEVICE, OK)
    assert gemm(lib, layout=5, ldb=528, ld_sb=2) == LD
    assert gemm(lib, layout=5, ld_sb=2) in (DEVICE, OK)
    assert gemm(lib, layout=6, N=200, ldc=208, ld_sb=200, dt=1) == SHAPE   # tiled B: N % 128
    assert gemm(lib, layout=6, ldb=528, ld_sb=256, dt=1) == LD
    assert gemm(lib, layout=6, ld_sb=256, dt=1) in (DEVICE, OK)
    # WGRAD: any N, column scales [K/128][N]
    assert gemm(lib, layout=2, N=200, ldc=208, ld_sb=150) == LD
    assert gemm(lib, layout=2, N=200, ldc=208, ld_sb=200, dt=1) in (DEVICE, OK)
    # scale tables of 2 GiB or more are not addressable with 32-bit offsets
    assert gemm(lib, ld_sa=1 << 28) == UNSUP                  # 4 K blocks x 2^28 floats
    assert gemm(lib, layout=2, ld_sb=1 << 28, dt=1) == UNSUP
    # the kernels number output tiles in 32 bits: 2^21 x 2^10 tiles is refused
    # before any other check looks at the (fake) buffers
    big_m, big_n = 1 << 28, 1 << 18
    assert gemm(lib, M=big_m, N=big_n, K=128, lda=128, ld_sa=big_m, ldb=128, ld_sb=1, ldc=big_n) == UNSUP
    assert gemm(lib, M=big_m, N=big_n - 256, K=128, lda=128, ld_sa=big_m, ldb=128, ld_sb=1,
                ldc=big_n) != UNSUP                                # 2^31 - 2^21 tiles pass this check


def fused(lib, M=256, N=256, K=512, x=X, ldx=512, w=B, ldw=512, sw=S2, ld_sw=4, c=C, dt=0, ldc=256,
          q=None, ldq=0, s=None, ld_s=0):
    return lib.fp8_block_gemm_fused_quant(M, N, K, x, ldx, w, ldw, sw, ld_sw, c, dt, ldc, q, ldq, s, ld_s,
                                          None)


def test_fused_quant_gemm_validation(lib):
    assert fused(lib, dt=5) == UNSUP
    assert fused(lib, K=200, ldx=256, ldw=256) == SHAPE
    assert fused(lib, N=200, ldc=256) == SHAPE
    assert fused(lib, M=-1) == SHAPE
    assert fused(lib, M=0, x=None) == OK
    assert fused(lib, x=None) == NULL
    assert fused(lib, q=Q, ldq=512) == NULL                   # codes without scales
    assert fused(lib, ldx=256) == LD
    assert fused(lib, ld_sw=2) == LD
    assert fused(lib, q=Q, ldq=256, s=S, ld_s=256) == LD
    assert fused(lib, q=Q, ldq=512, s=S, ld_s=100) == LD
    assert fused(lib, ldx=516) == ALIGN                        # BF16 rows not 16-byte aligned
    assert fused(lib, x=X + 8) == ALIGN
    assert fused(lib, q=Q + 4, ldq=512, s=S, ld_s=256) == ALIGN
    assert fused(lib, ldx=(1 << 22) + 8) == UNSUP
    assert fused(lib, c=X + 4096) == ALIAS
    assert fused(lib, q=C, ldq=512, s=S, ld_s=256) == ALIAS
    assert fused(lib, q=Q, ldq=512, s=X + 1024, ld_s=256) == ALIAS
    assert fused(lib) in (DEVICE, OK)
    assert fused(lib, q=Q, ldq=512, s=S, ld_s=256, dt=1) in (DEVICE, OK)


def test_quant_dual_validation(lib):
    f = lib.fp8_quant_act_dual
    base = dict(x=X, rows=256, cols=384, ldx=384, qr=A, ldqr=384, sr=S, ldsr=256, qc=B, ldqc=256,
                sc=S2, ldsc=384)

    def call(**kw):
        a = dict(base, **kw)
        return f(a["x"], a["rows"], a["cols"], a["ldx"], a["qr"], a["ldqr"], a["sr"], a["ldsr"],
                 a["qc"], a["ldqc"], a["sc"], a["ldsc"], None)
    assert call(rows=200) == SHAPE
    assert call(cols=200, ldx=208, ldqr=208, ldsc=208) == SHAPE
    assert call(rows=0, x=None) == OK
    assert call(qc=None) == NULL
    assert call(sr=None) == NULL
    assert call(ldx=256) == LD
    assert call(ldqc=128) == LD
    assert call(ldsr=128) == LD
    assert call(ldsc=256) == LD
    assert call(qr=A + 8) == ALIGN
    assert call(ldqc=264) == ALIGN
    assert call(qc=X) == ALIAS
    assert call(qc=A) == ALIAS
    assert call() in (DEVICE, OK)


def test_payload_validation(lib):
    # H = 256: message 264 bytes, stride 272
    pack = lambda x=X, rows=64, H=256, ldx=256, src=None, T=64, msg=Q, stride=272: \
        lib.fp8_pack_tokens(x, rows, H, ldx, src, T, msg, stride, None)
    assert pack(H=200, ldx=200) == SHAPE
    assert pack(T=65) == SHAPE                   # no src_rows: T <= rows
    assert pack(T=-1) == SHAPE
    assert pack(T=0, msg=None) == OK
    assert pack(msg=None) == NULL
    assert pack(x=None) == NULL
    assert pack(ldx=128) == LD
    assert pack(stride=256) == LD                # < 264
    assert pack(stride=264) == ALIGN             # not a multiple of 16
    assert pack(x=X + 8) == ALIGN
    assert pack(src=A + 2, T=100) == ALIGN
    assert pack(msg=X) == ALIAS
    assert pack(src=Q + 64, T=100) == ALIAS      # src_rows inside the messages
    assert pack(src=A, T=100) in (DEVICE, OK)    # gathering: T may exceed rows
    assert pack() in (DEVICE, OK)

    unpack = lambda msg=Q, T=64, H=256, stride=272, q=A, ldq=256, s=S, lds=64: \
        lib.fp8_unpack_tokens(msg, T, H, stride, q, ldq, s, lds, None)
    assert unpack(H=100) == SHAPE
    assert unpack(q=None) == NULL
    assert unpack(lds=60) == LD
    assert unpack(ldq=128) == LD
    assert unpack(stride=200) == LD
    assert unpack(ldq=264) == ALIGN
    assert unpack(s=S + 2) == ALIGN
    assert unpack(q=Q + 16) == ALIAS
    assert unpack(s=A + 64) == ALIAS
    assert unpack() in (DEVICE, OK)

    deq = lambda msg=Q, T=64, H=256, stride=272, y=A, ldy=256: \
        lib.fp8_dequant_tokens(msg, T, H, stride, y, ldy, None)
    assert deq(H=-128) == SHAPE
    assert deq(y=None) == NULL
    assert deq(ldy=128) == LD
    assert deq(ldy=260) == ALIGN
    assert deq(y=Q + 256) == ALIAS
    assert deq(T=0, y=None) == OK
    assert deq() in (DEVICE, OK)


def test_quant_tiles_validation(lib):
    f = lambda x=X, rows=64, cols=2048, ldx=2048, tile=128, rank=1, q=Q, ldq=2048, s=S, lds=64, sat=None: \
        lib.fp8_quant_act_tiles(x, rows, cols, ldx, tile, rank, q, ldq, s, lds, sat, None)
    for tile in (0, 16, 100, 2048):
        assert f(tile=tile) == UNSUP
    for rank in (0, 9, -1):
        assert f(rank=rank) == UNSUP
    assert f(cols=2048 + 32, ldx=2080, ldq=2080) == SHAPE     # not a multiple of 128
    assert f(tile=32, cols=2080, ldx=2080, ldq=2080) in (DEVICE, OK)
    assert f(rows=0, x=None) == OK
    assert f(q=None) == NULL
    assert f(lds=60) == LD
    assert f(ldq=1024) == LD
    assert f(ldq=2056) == ALIGN
    assert f(sat=A + 2) == ALIGN
    assert f(q=X + 64) == ALIAS
    assert f(sat=Q) == ALIAS
    for tile in (32, 64, 128, 256, 512, 1024):
        assert f(tile=tile, rank=8) in (DEVICE, OK)


def test_probe_recip_validation(lib):
    f = lambda s=A, r=C, n=64: lib.fp8_probe_recip_online(s, r, n, None)
    assert f(n=-1) == SHAPE
    assert f(n=0, s=None) == OK
    assert f(s=None) == NULL
    assert f(r=A + 2) == ALIGN
    assert f(r=A + 128) == ALIAS
    assert f() in (DEVICE, OK)


def test_probe_mfma_validation(lib):
    f = lambda wg=4, it=2, mode=0, codes=A, out=C: lib.fp8_probe_mfma(wg, it, mode, codes, out, None)
    assert f(wg=0) == SHAPE
    assert f(it=0) == SHAPE
    assert f(mode=3) == SHAPE
    assert f(mode=-1) == SHAPE
    assert f(codes=None) == NULL
    assert f(out=None) == NULL
    assert f(codes=A + 8) == ALIGN
    assert f(out=A + 1024) == ALIAS
    assert f() in (DEVICE, OK)


def test_probe_gemm_split_validation(lib):
    import ctypes
    n, k = ctypes.c_int64(-5), ctypes.c_int32(-5)
    f = lambda tiles=300, K=1024, a=ctypes.byref(n), b=ctypes.byref(k): lib.fp8_probe_gemm_split(tiles, K, None, a, b)
    assert f(tiles=-1) == SHAPE
    assert f(K=0) == SHAPE
    assert f(K=1000) == SHAPE
    assert f(a=None) == NULL
    assert f(b=None) == NULL
    st = f()
    assert st in (DEVICE, OK)
    if st == OK:   # no GEMM ran on this stream: no split workspace, whole tiles only
        assert (n.value, k.value) == (0, 1)


def test_gemm_promotion_validation(lib):
    f = lambda A_=A, M=64, K=256, lda=256, B_=B, N=48, ldb=256, pk=128, C_=C, ldc=48: \
        lib.fp8_gemm_promotion(A_, M, K, lda, B_, N, ldb, pk, C_, ldc, None)
    assert f(K=200, lda=208, ldb=208) == SHAPE
    assert f(M=-1) == SHAPE
    for pk in (0, 16, 96, 200, -128):
        assert f(pk=pk) == UNSUP
    assert f(M=0, C_=None) == OK
    assert f(C_=None) == NULL
    assert f(A_=None) == NULL
    assert f(lda=128) == LD
    assert f(ldc=32) == LD
    assert f(lda=264) == ALIGN
    assert f(A_=A + 4) == ALIGN
    assert f(C_=A + 1024) == ALIAS
    for pk in (32, 64, 128, 384, 1 << 20):
        assert f(pk=pk) in (DEVICE, OK)


def test_tiled_column_codes_validation(lib):
    f = lambda x=X, rows=256, cols=384, ldx=384, d=2, q=Q, ldq=256, s=S, lds=384: \
        lib.fp8_quant_act_1x128(x, rows, cols, ldx, d, q, ldq, s, lds, None, None, None, None)
    assert f() in (DEVICE, OK)
    assert f(cols=200, ldx=208, lds=208) == SHAPE       # tiled: cols % 128
    assert f(ldq=272) == LD                              # dense: ldq == rows
    assert f(d=1, cols=200, ldx=208, lds=208) in (DEVICE, OK)   # the row-major COL keeps ragged cols
    g = lambda qc=B, sc=S2: lib.fp8_quant_act_dual_tiled(X, 256, 384, 384, A, 384, S, 256, qc, sc, 384, None)
    assert g() in (DEVICE, OK)
    assert g(qc=None) == NULL
    assert g(qc=A + 1024) == ALIAS


def test_tiled_weight_and_grouped_validation(lib):
    f = lambda w=X, rows=256, cols=512, ldw=512, q=Q, qt=None, s=S, lds=4: \
        lib.fp8_quant_weight_128x128_tiled(w, rows, cols, ldw, q, qt, s, lds, None)
    assert f(rows=200) == SHAPE
    assert f(q=None) == NULL
    assert f(ldw=256) == LD
    assert f(lds=2) == LD
    assert f(q=Q + 8) == ALIGN
    assert f(q=X + 256) == ALIAS
    assert f(qt=Q + 4096) == ALIAS                  # q_t overlaps the dense 256*512 q
    assert f(qt=A) in (DEVICE, OK)
    g = lib.fp8_block_gemm_grouped_tiled
    args = [8, X, 1024, 256, 512, A, 512, S, 1024, B, S2, C, 0, 256, None]
    assert g(*args) in (DEVICE, OK)
    bad = list(args); bad[3] = 200
    assert g(*bad) == SHAPE
    bad = list(args); bad[0] = 0
    assert g(*bad) == SHAPE


def test_grouped_validation(lib):
    f = lib.fp8_block_gemm_grouped
    args = [8, X, 1024, 256, 512, A, 512, S, 1024, B, 512, S2, C, 0, 256, None]
    assert f(*args) in (DEVICE, OK)
    bad = list(args); bad[0] = 0
    assert f(*bad) == SHAPE
    bad = list(args); bad[1] = None
    assert f(*bad) == NULL
    bad = list(args); bad[3] = 200
    assert f(*bad) == SHAPE
    bad = list(args); bad[10] = 256
    assert f(*bad) == LD
    # tile bound with one ragged tile per group: (2^21 + 8) x 2^10 >= 2^31
    big = [8, X, 1 << 28, 1 << 18, 128, A, 128, S, 1 << 28, B, 128, S2, C, 0, 1 << 18, None]
    assert f(*big) == UNSUP


def test_no_device_reported_without_gpu(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert qa(lib) == DEVICE
    assert gemm(lib) == DEVICE
    assert lib.fp8_cast_e4m3(X, 16, Q, None) == DEVICE


def test_division_shortcut_exhaustive(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "check_div")
    src = os.path.join(ROOT, "tests", "c", "check_div.c")
    flags = ["-O2", "-ffp-contract=off", "-fopenmp"]
    if "fma" in open("/proc/cpuinfo").read():
        flags.append("-mfma")
    subprocess.run([gcc, *flags, "-o", exe, src, "-lm"], check=True)
    res = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert res.returncode == 0, res.stdout
    assert "mismatches=0" in res.stdout
    assert "pairs=1065402240" in res.stdout
    assert "scales=32640 scale_mismatches=0" in res.stdout


def test_split_schedule_rule(tmp_path):
    """split_plan / split_range (kernels.hpp) built on the host: every plan of
    a grid of launches equals the rule stated in tests/split_rule.py, and the
    program's invariant checks (pieces tile [0, K) in order, boundaries on
    whole 4-block rounds, the pieces fit grid and workspace) all hold."""
    from split_rule import split_rule
    gxx = shutil.which("g++")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not gxx or not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    exe = str(tmp_path / "check_split_plan")
    csrc = os.path.join(ROOT, "fine_grained_fp8_amd", "csrc")
    r = subprocess.run([gxx, "-std=c++17", "-O1", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
                        "-I", csrc, os.path.join(ROOT, "tests", "c", "check_split_plan.cpp"), "-o", exe],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    res = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    lines = res.stdout.strip().splitlines()
    assert res.returncode == 0 and lines[-1].endswith("violations=0"), lines[-1]
    splits = 0
    for ln in lines[:-1]:
        tiles, grid, kb, slots, dp, st, pieces, rounds = map(int, ln.split())
        assert (st, pieces) == split_rule(tiles, grid, kb, slots), ln
        assert dp == tiles - st and rounds == (kb + 3) // 4, ln
        splits += pieces > 1
    assert splits > 100          # the grid exercises the split in many shapes


def test_validation_layer_under_asan_ubsan(tmp_path):
    """The C-ABI layer (api.cpp: argument checks, range and alias
    arithmetic, device query) built on the host with g++
    -fsanitize=address,undefined, the kernel launchers replaced by host stubs
    (tests/c/launch_stubs.cpp), runs every validation test of this file in a
    child process without a sanitizer report.  No device code is built or
    run here."""
    if os.environ.get("FP8BS_SANITIZED_LIB"):
        pytest.skip("already the sanitized child run")
    gxx = shutil.which("g++")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not gxx or not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("g++ or the HIP headers are not available")
    lib_path = str(tmp_path / "libfp8bs_san.so")
    csrc = os.path.join(ROOT, "fine_grained_fp8_amd", "csrc")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-fPIC", "-shared", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"), "-I", csrc,
           os.path.join(csrc, "api.cpp"), os.path.join(ROOT, "tests", "c", "launch_stubs.cpp"),
           "-L", os.path.join(rocm, "lib"), "-Wl,-rpath," + os.path.join(rocm, "lib"), "-lamdhip64",
           "-o", lib_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    asan = subprocess.run([gxx, "-print-file-name=libasan.so"], capture_output=True, text=True).stdout.strip()
    env = dict(os.environ, LD_PRELOAD=asan, FP8BS_SANITIZED_LIB=lib_path,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    sel = "(validation or status_strings or no_device) and not asan"
    r = subprocess.run([sys.executable, "-m", "pytest", os.path.abspath(__file__), "-q", "-x",
                        "-p", "no:cacheprovider", "-k", sel], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    report = r.stdout[-3000:] + r.stderr[-3000:]
    assert r.returncode == 0, report
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, report
    assert " passed" in r.stdout, report
