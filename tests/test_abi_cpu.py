"""The C-ABI library on the host: it loads, exports every symbol that
include/gsr.h declares, describes its tile table, and rejects bad arguments
before touching any device.  No kernel is launched here."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gsr.h")

FAKE = 0x7F0000000000  # a 16-byte aligned address that is never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(n for n in names if n not in ("if", "while")))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gemm_scale_relu", "gemm_scale_relu_ex", "gemm_scale_bias_act", "gemm_scale_bias_act_ex",
              "gsr_select_config", "gsr_num_configs", "gsr_config_ids", "gsr_get_config", "gsr_status_string",
              "gsr_version"):
        assert n in names


def test_every_declared_symbol_is_exported(native):
    lib = ctypes.CDLL(native.LIBRARY)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in gsr.h but not exported"


def test_config_struct_layout(native):
    assert ctypes.sizeof(native.GsrConfig) == 40


# Ids of configurations dropped from the table; they are never reused.
RETIRED_IDS = (0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15, 19, 20, 23, 24, 26)


def test_config_table(native):
    n = native.num_configs()
    ids = native.config_ids()
    assert n >= 4 and len(ids) == n and ids == sorted(set(ids))
    assert not set(ids) & set(RETIRED_IDS)
    for i in ids:
        c = native.get_config(i)
        assert c["id"] == i
        assert c["block_k"] in (32, 64, 128)
        assert c["block_m"] % (32 * c["waves_m"]) == 0 and c["block_n"] % (32 * c["waves_n"]) == 0
        # stages == 0: register-staged kernel with two LDS buffers;
        # stages == 1: A copied to LDS, B transposed through registers, two
        # LDS buffers each; stages >= 2: ring of LDS buffers filled by copies
        buffers = 2 if c["stages"] in (0, 1) else c["stages"]
        lds = buffers * (c["block_m"] + c["block_n"]) * c["block_k"] * 2
        if i in (28, 29, 31):  # two A buffers and three B buffers
            lds = (2 * c["block_m"] + 3 * c["block_n"]) * c["block_k"] * 2
        assert c["lds_bytes"] == lds <= 163840
    for bad in (-1, max(ids) + 1) + RETIRED_IDS:
        with pytest.raises(native.GsrError):
            native.get_config(bad)
    # the id listing honours its capacity and rejects a bad one
    buf = (ctypes.c_int32 * 2)(-7, -7)
    assert native.lib().gsr_config_ids(buf, 1) == n and buf[0] == ids[0] and buf[1] == -7
    assert native.lib().gsr_config_ids(None, 0) == n
    assert native.lib().gsr_config_ids(None, 3) == -1
    assert native.lib().gsr_config_ids(buf, -1) == -1


def test_retired_ids_are_rejected_before_any_device_use(native):
    """A forced launch of a retired or unknown id fails with
    GSR_ERROR_INVALID_CONFIG from the host-side checks (no device needed)."""
    for bad in RETIRED_IDS + (27, 1000):
        st = native.gemm_scale_relu_ex(8, 8, 8, 0x1000, 0x2000, 0x3000, 1.0, 0, bad)
        assert st == native.GSR_ERROR_INVALID_CONFIG, (bad, st)


@pytest.mark.parametrize("shape", [(256, 256, 256), (1024, 1024, 1024), (4096, 4096, 4096),
                                   (4097, 11008, 4096), (16384, 16384, 16384), (16, 11008, 4096),
                                   (1, 1, 1), (0, 5, 5)])
def test_selector(native, shape):
    c = native.select_config(*shape)
    assert c["id"] in native.config_ids()
    M, N, _ = shape
    if M * N >= 256 * 256 * 256:
        # large problems use a tile that still yields one workgroup per CU
        assert -(-M // c["block_m"]) * -(-N // c["block_n"]) >= 256


def test_status_strings(native):
    assert native.status_string(0) == "success"
    for s in range(1, 7):
        assert native.status_string(s) not in ("", "success", "unknown status")
    assert native.status_string(99) == "unknown status"
    assert native.version() >= 100


@pytest.mark.parametrize("args,status", [
    ((-1, 4, 4, FAKE, FAKE + 4096, FAKE + 8192), 1),
    ((4, -1, 4, FAKE, FAKE + 4096, FAKE + 8192), 1),
    ((4, 4, -1, FAKE, FAKE + 4096, FAKE + 8192), 1),
    ((4, 4, 4, 0, FAKE + 4096, FAKE + 8192), 1),        # null A
    ((4, 4, 4, FAKE, 0, FAKE + 8192), 1),               # null B
    ((4, 4, 4, FAKE, FAKE + 4096, 0), 1),               # null C
    ((4, 4, 4, FAKE + 1, FAKE + 4096, FAKE + 8192), 1),  # odd A
    ((4, 4, 4, FAKE, FAKE + 4097, FAKE + 8192), 1),      # odd B
    ((4, 4, 4, FAKE, FAKE + 4096, FAKE + 8193), 1),      # odd C
    ((4, 4, 4, FAKE, FAKE + 4096, FAKE + 16), 1),        # C overlaps A
    ((4, 4, 4, FAKE, FAKE + 4096, FAKE + 4096 + 30), 1), # C overlaps B
    ((2 ** 31, 4, 4, FAKE, FAKE + 4096, FAKE + 8192), 2),
    ((40000, 40000, 8, FAKE, FAKE + 2 ** 32, FAKE + 2 ** 33), 2),  # C >= 2^31 bytes
])
def test_argument_errors(native, args, status):
    M, N, K, A, B, C = args
    assert native.gemm_scale_relu(M, N, K, A, B, C, 0.5, 0) == status


def test_nonfinite_alpha_and_bad_config(native):
    import math
    assert native.gemm_scale_relu(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, math.nan, 0) == 1
    assert native.gemm_scale_relu(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, math.inf, 0) == 1
    assert native.gemm_scale_relu_ex(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, 0.5, 0, 99) == 6
    assert native.gemm_scale_relu_ex(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, 0.5, 0, -2) == 6


@pytest.mark.parametrize("bias,act", [
    (FAKE + 12288, 3),          # unknown activation
    (FAKE + 12288, -1),
    (FAKE + 12289, 1),          # odd bias address
    (FAKE + 8192 + 8, 1),       # bias inside C (C is 4x4 fp16 = 32 bytes at FAKE+8192)
    (FAKE + 8192 - 4, 2),       # bias (4 values, 8 bytes) running into C's first bytes
])
def test_epilogue_argument_errors(native, bias, act):
    # every case is rejected on the host, before any device is touched
    assert native.gemm_scale_bias_act(4, 4, 4, FAKE, FAKE + 4096, bias, FAKE + 8192, 1.0, act, 0) == 1


def test_epilogue_variants_share_the_checks(native):
    import math
    # the same validation as the plain entry point, before any device work
    assert native.gemm_scale_bias_act(-1, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, 1.0, 1, 0) == 1
    assert native.gemm_scale_bias_act(4, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 16, 1.0, 1, 0) == 1
    assert native.gemm_scale_bias_act(4, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, math.nan, 1, 0) == 1
    assert native.gemm_scale_bias_act(4, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, 1.0, 1, 0, 99) == 6
    assert native.gemm_scale_bias_act(0, 4, 4, 0, 0, 0, 0, 1.0, 1, 0) == 0
    assert native.gemm_scale_bias_act(2 ** 31, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, 1.0, 1, 0) == 2


def test_empty_output_is_a_noop(native):
    # M == 0 or N == 0: success, nothing enqueued, no device needed
    assert native.gemm_scale_relu(0, 16, 16, 0, 0, 0, 0.5, 0) == 0
    assert native.gemm_scale_relu(16, 0, 16, 0, 0, 0, 0.5, 0) == 0


def test_no_device(native):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("a device is present")
    assert native.gemm_scale_relu(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, 0.5, 0) == 3


def test_missing_library_fails_loudly(monkeypatch):
    from tiled_dense_gemm_scale_amd import _native
    monkeypatch.setattr(_native, "_lib", None)
    monkeypatch.setattr(_native, "LIBRARY", "/nonexistent/libgsr.so")
    with pytest.raises(RuntimeError, match="not built"):
        _native.lib()


def test_tuning_table_host_side(native, tmp_path):
    """The tuning table is parsed and consulted on the host: select_config
    reports the tuned launch for an exact shape and the built-in choice
    otherwise; a malformed file is rejected and the previous table kept."""
    native.clear_tuning()
    base = native.select_config(1024, 1024, 1024)
    other = native.select_config(1024, 1024, 1025)
    good = tmp_path / "t.txt"
    good.write_text("# comment line\n\n1024 1024 1024 22 2 0   # trailing comment\n300 520 200 28 8 1\n")
    native.load_tuning(str(good))
    try:
        assert native.tuning_entries() == 2
        c = native.select_config(1024, 1024, 1024)
        assert (c["id"], c["group_m"], c["xcd_remap"]) == (22, 2, 0)
        c = native.select_config(300, 520, 200)
        assert (c["id"], c["group_m"], c["xcd_remap"]) == (28, 8, 1)
        assert native.select_config(1024, 1024, 1025) == other  # not in the table
        for bad in ("1024 1024 1024 99 1 0\n",      # unknown config id
                    "1024 1024 1024 9 1 0\n",       # a retired config id
                    "1024 1024 1024 21 0 0\n",      # group_m < 1
                    "1024 1024 1024 21 1 3\n",      # xcd_remap not 0, 1 or 2
                    "1024 1024 21 1 0\n",           # too few fields
                    "1024 1024 1024 21 1 0 5\n",    # too many fields
                    "-1 4 4 21 1 0\n",              # negative size
                    "hello\n"):
            p = tmp_path / "bad.txt"
            p.write_text(bad)
            with pytest.raises(native.GsrError):
                native.load_tuning(str(p))
            assert native.tuning_entries() == 2  # previous table kept
        with pytest.raises(native.GsrError):
            native.load_tuning(str(tmp_path / "missing.txt"))
    finally:
        native.clear_tuning()
    assert native.tuning_entries() == 0
    assert native.select_config(1024, 1024, 1024) == base


def test_launch_entry_point_checks(native):
    # explicit launches are validated on the host before any device work
    for cid, gm, xcd in ((99, 4, 1), (-1, 4, 1), (21, 0, 1), (21, 5000, 1), (21, 4, 3), (21, 4, -1), (9, 4, 1), (7, 4, 1), (23, 4, 1), (8, 4, 1)):
        st = native.gemm_scale_bias_act_cfg(4, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, 1.0, 0, 0, cid, gm, xcd)
        assert st == 6, (cid, gm, xcd, st)


class _DeviceTensorStandIn:
    """Carries only the attributes the binding's operand checks read, so the
    checks run without a GPU; no data is ever touched."""

    def __init__(self, shape, index):
        import torch

        self.shape, self.dtype, self.is_cuda = tuple(shape), torch.float16, True
        self.device = torch.device("cuda", index)

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return True


def test_binding_rejects_operands_on_different_devices():
    import tiled_dense_gemm_scale_amd as gsr

    T = _DeviceTensorStandIn
    with pytest.raises(ValueError, match="one device"):
        gsr.gemm_scale_relu(T((4, 8), 0), T((8, 4), 1), 0.5)
    with pytest.raises(ValueError, match="A's device"):
        gsr.gemm_scale_relu(T((4, 8), 0), T((8, 4), 0), 0.5, c=T((4, 4), 1))
    with pytest.raises(ValueError, match="A's device"):
        gsr.gemm_scale_bias_act(T((4, 8), 0), T((8, 4), 0), T((4,), 1), c=T((4, 4), 0))


# ---- the entry points with a workspace --------------------------------------

WS = FAKE + (1 << 20)  # a workspace address clear of A, B and C


@pytest.mark.parametrize("ws,nbytes,splits,status", [
    (WS + 8, 1 << 16, 0, 1),          # workspace not 16-byte aligned
    (WS, -1, 0, 1),                   # negative size
    (FAKE + 8192 - 64, 4096, 0, 1),   # workspace running into C (C: 32 bytes at FAKE + 8192)
    (FAKE, 4096, 0, 1),               # workspace over A
    (FAKE + 4096 - 16, 4096, 0, 1),   # ... and over B
    (WS, 1 << 16, -1, 1),             # splits outside 0..16
    (WS, 1 << 16, 17, 1),
])
def test_workspace_argument_errors(native, ws, nbytes, splits, status):
    st = native.gemm_scale_bias_act_ws(4, 4, 4, FAKE, FAKE + 4096, 0, FAKE + 8192, 1.0, 0, ws, nbytes, 0, -1,
                                       splits)
    assert st == status, (ws, nbytes, splits, st)


def test_workspace_entry_points_share_the_checks(native):
    import math
    args = (FAKE, FAKE + 4096, 0, FAKE + 8192)
    assert native.gemm_scale_bias_act_ws(-1, 4, 4, *args, 1.0, 0, WS, 4096, 0, -1, 0) == 1
    assert native.gemm_scale_bias_act_ws(4, 4, 4, *args, math.nan, 0, WS, 4096, 0, -1, 0) == 1
    assert native.gemm_scale_bias_act_ws(4, 4, 4, *args, 1.0, 3, WS, 4096, 0, -1, 0) == 1
    assert native.gemm_scale_bias_act_ws(4, 4, 4, *args, 1.0, 0, WS, 4096, 0, 99, 0) == 6
    assert native.gemm_scale_bias_act_ws(4, 4, 4, *args, 1.0, 0, WS, 4096, 0, 8, 0) == 6   # a retired id
    assert native.gemm_scale_bias_act_ws(4, 4, 4, *args, 1.0, 0, WS, 4096, 0, -2, 0) == 6
    assert native.gemm_scale_bias_act_ws(2 ** 31, 4, 4, *args, 1.0, 0, WS, 4096, 0, -1, 0) == 2
    assert native.gemm_scale_bias_act_ws(0, 4, 4, 0, 0, 0, 0, 1.0, 0, 0, 0, 0, -1, 0) == 0
    assert native.gemm_scale_relu_ws(4, 4, 4, FAKE, FAKE + 4096, FAKE + 16, 0.5, WS, 4096, 0) == 1  # C over A
    assert native.gemm_scale_relu_ws(4, 4, 4, FAKE, FAKE + 4096, FAKE + 8192, 0.5, WS + 4, 4096, 0) == 1
    assert native.gemm_scale_relu_ws(0, 16, 16, 0, 0, 0, 0.5, 0, 0, 0) == 0


def test_workspace_bytes(native):
    """The library's split (host only): a 32-bit counter per tile in a
    256-byte-rounded region, then parts x tiles fp32 partial tiles.  Decode
    shapes against a 4096-wide weight split in four (64 tiles of 32 x 64),
    two tile rows in two (128 tiles); too few K-steps, too many tiles, or an
    unsplit call near the read ceiling: none."""
    tile = 32 * 64 * 4
    assert native.workspace_bytes(1, 4096, 4096) == 256 + 4 * 64 * tile
    assert native.workspace_bytes(32, 4096, 11008) == 256 + 4 * 64 * tile
    assert native.workspace_bytes(64, 4096, 4096) == 512 + 2 * 128 * tile
    assert native.workspace_bytes(1, 1024, 4096) == 256 + 4 * 16 * tile
    assert native.workspace_bytes(1, 4096, 2048) == 0          # 16 K-steps
    assert native.workspace_bytes(1, 11008, 4096) == 0         # 172 tiles
    assert native.workspace_bytes(1, 8192, 8192) == 0          # unsplit already near the read ceiling
    assert native.workspace_bytes(1024, 1024, 1024) == 0
    assert native.workspace_bytes(4096, 4096, 4096) == 0
    assert native.workspace_bytes(0, 4096, 4096) == 0
    assert native.workspace_bytes(16, 4096, 0) == 0
    with pytest.raises(native.GsrError):
        native.workspace_bytes(-1, 4, 4)
    # never more than 4 MiB + 512 bytes (at most 256 workgroups of 64 x 64 fp32)
    worst = max(native.workspace_bytes(M, N, K) for M in (1, 7, 32, 33, 64, 100, 128, 200, 512)
                for N in (8, 64, 1000, 2048, 4096, 8192) for K in (4096, 8192, 11008, 65536))
    assert 0 < worst <= (4 << 20) + 512
