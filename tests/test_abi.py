"""The C-ABI library on the host: it loads, exports what include/gemm_relu.h
declares, and rejects bad arguments before any HIP call (no GPU needed)."""
import ctypes
import os
import re
import subprocess
import sys

import pytest

import dense_tiled_gemm_relu_amd as gr
from tests.helpers import COMPARISON_CONFIGS, built_configs

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    names = []
    for fn in os.listdir(os.path.join(ROOT, "include")):
        if fn.endswith(".h"):
            text = open(os.path.join(ROOT, "include", fn)).read()
            text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
            names += re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary():
    assert header_functions() == sorted(gr.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(gr.LIB_PATH)
    for name in header_functions():
        assert hasattr(lib, name), name


def test_strerror():
    assert gr.gemm_relu_strerror(0) == "success"
    assert gr.gemm_relu_strerror(gr.EINVAL) == "invalid argument"
    assert gr.gemm_relu_strerror(gr.EUNSUPPORTED).startswith("unsupported")
    assert gr.gemm_relu_strerror(gr.EHIP).startswith("HIP")
    assert gr.gemm_relu_strerror(12345) == "unknown status"


# fake, well-aligned and disjoint addresses: validation inspects, never dereferences
A, B, C = 1 << 32, 2 << 32, 3 << 32


@pytest.mark.parametrize("args", [
    (A, B, C, -1, 4, 4, 0, 0, 0),            # negative M
    (A, B, C, 4, -1, 4, 0, 0, 0),            # negative N
    (A, B, C, 4, 4, -1, 0, 0, 0),            # negative K
    (A, B, C, 2 ** 31, 4, 4, 0, 0, 0),       # beyond INT32_MAX
    (A, B, C, 4, 4, 4, 2, 0, 0),             # fp32 input not supported
    (A, B, C, 4, 4, 4, 0, 3, 0),             # 8-bit output not supported
    (A, B, C, 4, 4, 4, 5, 0, 0),             # unknown input code
    (A, B, C, 4, 4, 4, 3, 4, 0),             # 8-bit output not supported
    (A, B, C, 4, 4, 4, 0, 0, 2),             # transB not in {0, 1}
    (0, B, C, 4, 4, 4, 0, 0, 0),             # NULL A with elements
    (A, 0, C, 4, 4, 4, 0, 0, 0),             # NULL B with elements
    (A, B, 0, 4, 4, 4, 0, 0, 0),             # NULL C
    (A + 1, B, C, 4, 4, 4, 0, 0, 0),         # A not 2-byte aligned
    (A, B, C + 2, 4, 4, 4, 0, 2, 0),         # fp32 C not 4-byte aligned
    (A, B, A + 16, 4, 4, 4, 0, 0, 0),        # C overlaps A
    (A, B, B + 30, 4, 4, 4, 0, 0, 1),        # C overlaps B
])
def test_invalid_arguments_fail_before_the_device(args):
    assert gr.gemm_relu_status(*args, stream=0) == gr.EINVAL
    assert gr.gemm_relu_plan(*args) is None


def test_empty_outputs_are_a_no_op():
    assert gr.gemm_relu_status(0, 0, 0, 0, 5, 7, 0, 0, 0, stream=0) == gr.OK
    assert gr.gemm_relu_status(0, 0, 0, 5, 0, 7, 1, 2, 1, stream=0) == gr.OK
    assert gr.gemm_relu_plan(0, 0, 0, 0, 5, 7, 0, 0, 0) == "none"


def test_null_operands_allowed_when_K_is_zero():
    # K = 0: A and B hold no elements, C gets +0 everywhere (plan only here)
    assert gr.gemm_relu_plan(0, 0, C, 64, 64, 0, 0, 0, 0) is not None


@pytest.mark.parametrize("M,N,K,transB,aligned,want", [
    (8192, 8192, 8192, 0, True, "d256x256x32_s4_i16w8"),
    (4096, 4096, 4096, 0, True, "d256x256x32_s4_i16w8"),
    (4096, 7168, 4096, 1, True, "d256x256x32_s4_i16+d256x192x32_s4_i16"),
    (256, 256, 256, 0, True, "d64x32x128_s4"),
    (64, 8192, 8192, 0, True, "d32x64x128_s4"),        # skinny: whole-line B rows, twice the workgroups of 64x64
    (32, 16384, 8192, 0, True, "d64x64x64_s4"),        # skinny, but 64x64 tiles fill the CUs
    (2048, 2048, 512, 0, True, "d128x128x64_s3"),
    (4096, 7168, 4096, 0, True, "d256x256x32_s4_i16w8"),
    (4097, 3001, 5003, 0, True, "d256x256x32_s4_i16w8"),  # ragged and 2-byte aligned rows
    (4096, 4096, 4096, 0, False, "d256x256x32_s4_i16w8"), # 2-byte aligned base pointer
    (100, 100, 100, 0, True, "d64x32x128_s4"),
    (100, 24, 100, 0, True, "g64x64x64"),              # fewer than 32 columns of (K,N) B
    (100, 24, 100, 1, True, "d64x32x128_s4"),          # transposed B rows are clamped
    (64, 64, 1 << 23, 0, True, "g64x64x64"),           # copy offsets would overflow 32 bits
])
def test_plan_selection(M, N, K, transB, aligned, want):
    off = 0 if aligned else 2
    assert gr.gemm_relu_plan(A + off, B, C, M, N, K, 0, 0, transB) == want


@pytest.mark.parametrize("M,N,K,transB,want", [
    (8192, 8192, 8192, 0, "d256x256x32_s4_i"),
    (4096, 7168, 4096, 1, "d256x256x32_s4_i"),
    (64, 8192, 8192, 0, "d32x64x128_s4"),
    (100, 16, 100, 0, "g64x64x64"),                   # fewer than 16 columns of (K,N) B
    (100, 16, 100, 1, "d64x32x128_s4"),
])
@pytest.mark.parametrize("in_code", [3, 4])
def test_plan_selection_fp8(M, N, K, transB, want, in_code):
    assert gr.gemm_relu_plan(A, B, C, M, N, K, in_code, 0, transB) == want
    # 8-bit operands may start at any byte
    assert gr.gemm_relu_plan(A + 1, B + 3, C, M, N, K, in_code, 0, transB) == want


def test_fp8_forced_comparison_configuration_falls_back(monkeypatch):
    # the 16-bit comparison variants are not built for 8-bit inputs
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_w8i")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 3, 0, 0) == "d256x256x32_s4_i"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "g128x128x64")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 3, 0, 0) == "g128x128x64"


def test_forced_configuration(monkeypatch):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "g64x64x64")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 0) == "g64x64x64"
    # a configuration that cannot serve the problem falls back to the automatic choice
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x64_s2")
    assert gr.gemm_relu_plan(A, B, C, 100, 100, 100, 0, 0, 0) == "d64x32x128_s4"


def test_missing_library_fails_loudly(tmp_path):
    code = ("import dense_tiled_gemm_relu_amd as gr\n"
            "gr.LIB_PATH = %r\n"
            "try:\n"
            "    gr.gemm_relu(0, 0, 0, 1, 1, 1, 0, 0, 0, stream=0)\n"
            "except RuntimeError as e:\n"
            "    print('raised', e)\n" % str(tmp_path / "missing.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True)
    assert "raised" in r.stdout and "not built" in r.stdout


def test_product_path_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "dense_tiled_gemm_relu_amd")
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".hpp", ".h", ".cpp")):
                text = open(os.path.join(dirpath, fn)).read()
                assert "import oracle" not in text and "from oracle" not in text, fn
                assert "oracle.c" not in text and "liboracle" not in text, fn


# ------------------------------------------------ block-scaled entry point
SA_, SB_ = 4 << 32, 5 << 32


@pytest.mark.parametrize("args", [
    (A, SA_, B, SB_, C, 4, 4, 48, 5, 0),      # K not a multiple of 32
    (A, SA_, B, SB_, C, 4, 4, 64, 3, 0),      # a plain FP8 code is not an MX format
    (A, SA_, B, SB_, C, 4, 4, 64, 8, 0),      # unknown format
    (A, SA_, B, SB_, C, 4, 4, 64, 5, 3),      # unknown output
    (A, 0, B, SB_, C, 4, 4, 64, 7, 0),        # NULL scales with elements
    (A, SA_, B, SB_, SA_, 4, 4, 64, 7, 0),    # C overlaps SA
    (A, SA_, B, SB_, C, -1, 4, 64, 7, 0),     # negative M
])
def test_mx_invalid_arguments(args):
    assert gr.gemm_relu_mx_status(*args, stream=0) == gr.EINVAL
    assert gr.gemm_relu_mx_plan(*args) is None


@pytest.mark.parametrize("M,N,K,want", [
    (8192, 8192, 8192, "d256x256x32_s4_i"),
    (4096, 4096, 4096, "d256x256x32_s4_i"),
    (1024, 1024, 4096, "d128x128x64_s2"),
    (8192, 8192, 480, "d128x128x64_s2"),       # fewer than 16 scale blocks per row
    (64, 64, 64, "d128x128x64_s2"),
])
@pytest.mark.parametrize("fmt", [5, 6, 7])
def test_mx_plan_selection(M, N, K, want, fmt):
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, M, N, K, fmt, 0) == want
    assert gr.gemm_relu_mx_plan(0, 0, 0, 0, C, 0, N, K, fmt, 0) == "none"


@pytest.mark.parametrize("name", built_configs(["d256x256x32_s4_i", "d256x256x64_s2",
                                                 "d256x128x64_s2", "d128x128x64_s2"]))
def test_mx_forced_configuration(monkeypatch, name):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", name)
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 8192, 8192, 8192, 7, 0) == name
    # a configuration not built for block-scaled inputs falls back
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d64x64x64_s4")
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 8192, 8192, 8192, 7, 0) == "d256x256x32_s4_i"


@pytest.mark.parametrize("fmt", [5, 7])
def test_mx_interleaved_needs_16_scale_blocks_per_row(monkeypatch, fmt):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_i")
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 1024, 1024, 512, fmt, 0) == "d256x256x32_s4_i"
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 1024, 1024, 480, fmt, 0) == "d128x128x64_s2"


@pytest.mark.parametrize("in_dtype,want", [(0, "d256x256x32_s4_i16w8"), (1, "d256x256x32_s4_i16w8"),
                                           (3, "d256x256x32_s4_i")])
def test_mx_only_configuration_not_used_for_other_inputs(monkeypatch, in_dtype, want):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x128x64_s2")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, in_dtype, 0, 1) == want


# ------------------------------------------------ 2:4 sparse entry point
E_ = 6 << 32


@pytest.mark.parametrize("args", [
    (A, E_, B, C, 4, 4, 6, 0, 0, 0),          # K not a multiple of 4
    (A, E_, B, C, 4, 4, 8, 3, 0, 0),          # FP8 inputs are not a sparse format here
    (A, E_, B, C, 4, 4, 8, 0, 3, 0),          # unknown output
    (A, E_, B, C, 4, 4, 8, 0, 0, 2),          # transB not in {0, 1}
    (A, 0, B, C, 4, 4, 8, 0, 0, 1),           # NULL metadata with elements
    (A + 1, E_, B, C, 4, 4, 8, 0, 0, 1),      # misaligned As
    (A, E_, B, E_, 4, 4, 8, 0, 0, 1),         # C overlaps E
    (A, E_, B, C, 4, -1, 8, 0, 0, 1),         # negative N
])
def test_sp_invalid_arguments(args):
    assert gr.gemm_relu_sp_status(*args, stream=0) == gr.EINVAL
    assert gr.gemm_relu_sp_plan(*args) is None


def test_sp_plan():
    assert gr.gemm_relu_sp_plan(A, E_, B, C, 8192, 8192, 8192, 0, 0, 0) == "sp256x256x64_s3_w8"
    assert gr.gemm_relu_sp_plan(A, E_, B, C, 1, 1, 4, 1, 2, 1) == "sp256x256x64_s3_w8"
    assert gr.gemm_relu_sp_plan(A, E_, B, C, 0, 8, 8, 0, 0, 0) == "none"
    # B stored (K, N) needs a full tile of columns
    assert gr.gemm_relu_sp_plan(A, E_, B, C, 64, 255, 64, 0, 0, 0) == "unsupported"
    assert gr.gemm_relu_sp_status(A, E_, B, C, 64, 255, 64, 0, 0, 0, stream=0) == gr.EUNSUPPORTED
    assert gr.gemm_relu_sp_plan(A, E_, B, C, 64, 8, (1 << 22) + 4, 0, 0, 1) == "unsupported"


@pytest.mark.parametrize("name", built_configs(["d256x256x32_s4_ip", "d256x256x32_s4_i"]))
def test_comparison_configurations_are_selectable(monkeypatch, name):
    """The persistent tile loop and the 32x32-block tile: forced by name for
    16-bit inputs, never chosen automatically for them (the 16x16-block tile
    is); 8-bit inputs have no persistent build and take the 32x32 tile."""
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 0) == "d256x256x32_s4_i16w8"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", name)
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 0) == name
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 1, 2, 1) == name
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 3, 0, 0) == "d256x256x32_s4_i"


def test_16x16_tile_not_built_for_8bit_inputs(monkeypatch):
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_i16")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 3, 0, 0) == "d256x256x32_s4_i"
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 4, 0, 1) == "d256x256x32_s4_i"


def test_configs_lists_the_plan_names():
    """gemm_relu_configs names every configuration plan selection can return
    (and, in a comparison build, the comparison ones too)."""
    names = gr.gemm_relu_configs()
    assert len(names) == len(set(names))
    for want in ("d256x256x32_s4_i16w8", "d256x256x32_s4_i16", "d256x192x32_s4_i16",
                 "d256x256x32_s4_i16+d256x192x32_s4_i16",
                 "d64x128x64_s4_splitk", "d256x256x32_s4_i", "d128x128x64_s3", "d64x64x64_s4",
                 "d64x32x128_s4", "d32x64x128_s4", "g128x128x64", "g64x64x64", "d128x128x64_s2",
                 "sp256x256x64_s3_w8"):
        assert want in names
    assert set(names) - set(COMPARISON_CONFIGS) <= set(names)


def test_comparison_configurations_only_in_a_comparison_build(monkeypatch):
    """Without the comparison configurations a forced one is not launched:
    plan selection chooses as if it had not been named (and with them, it is)."""
    names = set(gr.gemm_relu_configs())
    cmp_built = set(COMPARISON_CONFIGS) & names
    assert cmp_built in (set(), set(COMPARISON_CONFIGS))     # all or none
    for name in ("d256x256x32_s4_isk", "d256x256x32_s4_ip", "d256x256x64_s2"):
        monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", name)
        got = gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 0)
        assert got == (name if cmp_built else "d256x256x32_s4_i16w8")
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x128x64_s2")
    got = gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 8192, 8192, 8192, 7, 0)
    assert got == ("d256x128x64_s2" if cmp_built else "d256x256x32_s4_i")


@pytest.mark.skipif(not built_configs(["d256x256x32_s4_isk"]),
                    reason="stream-K is a comparison configuration, not in this build")
def test_streamk_selection(monkeypatch):
    """Stream-K (the 256x256 tile with its last round split along K) is
    selected by name only, for 16-bit and 8-bit inputs with at least two K
    steps a tile; never chosen automatically; not built for block-scaled inputs."""
    for shape in [(4096, 7168, 4096), (4097, 3001, 5003), (3000, 3000, 3000)]:
        assert gr.gemm_relu_plan(A, B, C, *shape, 0, 0, 0) != "d256x256x32_s4_isk"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_isk")
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 0) == "d256x256x32_s4_isk"
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d256x256x32_s4_isk"
    assert gr.gemm_relu_plan(A, B, C, 512, 512, 64, 0, 0, 0) == "d256x256x32_s4_isk"
    assert gr.gemm_relu_plan(A, B, C, 512, 512, 32, 0, 0, 0) != "d256x256x32_s4_isk"
    assert gr.gemm_relu_plan(A, B, C, 512, 512, 128, 3, 0, 0) == "d256x256x32_s4_isk"
    assert gr.gemm_relu_plan(A, B, C, 512, 512, 64, 3, 0, 0) != "d256x256x32_s4_isk"
    assert gr.gemm_relu_mx_plan(A, SA_, B, SB_, C, 8192, 8192, 8192, 7, 0) == "d256x256x32_s4_i"


SPLIT = "d256x256x32_s4_i16+d256x192x32_s4_i16"
SPLIT8 = "d256x256x32_s4_i16w8+d128x384x32_s4_i16w8"


def test_two_region_grid_selection(monkeypatch):
    """16-bit inputs with B stored (N,K): when whole rounds of 256x256 tiles
    leave a partial round, the tile columns past those rounds are cut into
    narrower tiles of 3/4 the area (one launch, one narrower last round):
    256x192 four-wave tiles behind the four-wave 256x256 tile, or, when the
    eight-wave 256x256 tile is forced, 128x384 eight-wave tiles behind it (a
    comparison configuration).  (K,N) B, whole rounds, 8-bit inputs and forced
    configurations keep plain tiles; GEMM_RELU_SPLIT_COLS forces or forbids
    the split."""
    eight = bool(built_configs([SPLIT8]))
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == SPLIT
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 0, 0, 1) == SPLIT
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 0) == "d256x256x32_s4_i16w8"
    assert gr.gemm_relu_plan(A, B, C, 8192, 8192, 8192, 0, 0, 1) == "d256x256x32_s4_i16w8"
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 3, 0, 1) == "d256x256x32_s4_i"
    monkeypatch.setenv("GEMM_RELU_SPLIT_COLS", "0")
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d256x256x32_s4_i16w8"
    monkeypatch.setenv("GEMM_RELU_SPLIT_COLS", "1")
    assert gr.gemm_relu_plan(A, B, C, 512, 520, 64, 0, 0, 1) == SPLIT
    assert gr.gemm_relu_plan(A, B, C, 512, 256, 64, 0, 0, 1) == "d256x256x32_s4_i16"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_i16w8")
    assert gr.gemm_relu_plan(A, B, C, 512, 520, 64, 0, 0, 1) == (SPLIT8 if eight else "d256x256x32_s4_i16w8")
    assert gr.gemm_relu_plan(A, B, C, 512, 256, 64, 0, 0, 1) == "d256x256x32_s4_i16w8"
    monkeypatch.delenv("GEMM_RELU_SPLIT_COLS")
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d256x256x32_s4_i16w8"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x256x32_s4_i16")
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d256x256x32_s4_i16"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x192x32_s4_i16")
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d256x192x32_s4_i16"
    if eight:
        monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d128x384x32_s4_i16w8")
        assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 1) == "d128x384x32_s4_i16w8"
        # the narrower tiles are built for B stored (N,K) only
        assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 0) == "d256x256x32_s4_i16w8"
    monkeypatch.setenv("GEMM_RELU_FORCE_CONFIG", "d256x192x32_s4_i16")
    # the 256x192 tile is built for B stored (N,K) only
    assert gr.gemm_relu_plan(A, B, C, 4096, 7168, 4096, 1, 2, 0) == "d256x256x32_s4_i16w8"
