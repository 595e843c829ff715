"""The C ABI without a GPU: libs6.so loads, exports every function that
include/s6.h declares, and its argument checks (which run before any HIP
call) return the documented status codes.  No kernel is launched here:
every call either fails validation or has no work (batch or dim zero)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "s6.h")
LIB = os.path.join(ROOT, "selective_state_space_63_amd", "libs6.so")



@pytest.fixture(scope="module", autouse=True)
def built():
    """Build libs6.so (host cross-compile for gfx950) only if nothing is built."""
    if not os.path.exists(LIB):
        from selective_state_space_63_amd import build
        build.build(LIB)
    assert os.path.exists(LIB)


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(s6_\w+)\s*\(", text, flags=re.M)))


def header_macros():
    text = open(HEADER).read()
    return {m: int(v) for m, v in re.findall(r"#define\s+(S6_\w+)\s+\(?(-?\d+)\)?", text)}


@pytest.fixture(scope="module")
def lib():
    from selective_state_space_63_amd import s6
    return s6.load_library()


@pytest.fixture(scope="module")
def codes():
    return header_macros()


def test_header_declares_the_entry_points():
    assert header_functions() == ["s6_conv_scan_bwd", "s6_conv_scan_fwd", "s6_conv_state_update", "s6_last_state",
                                  "s6_last_state_ex", "s6_last_state_workspace_size",
                                  "s6_scan_bwd", "s6_scan_bwd_ckpt", "s6_scan_bwd_ex", "s6_scan_bwd_workspace_size",
                                  "s6_scan_fwd", "s6_scan_fwd_ckpt", "s6_scan_fwd_ex", "s6_scan_fwd_noalloc",
                                  "s6_scan_fwd_workspace_size",
                                  "s6_ssd_scan_fwd", "s6_ssd_scan_fwd_workspace_size",
                                  "s6_state_update", "s6_state_update_ex", "s6_status_str", "s6_version"]


def test_every_declared_symbol_is_exported():
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [f for f in header_functions() if f not in exported]
    assert not missing, f"declared but not exported: {missing}"


def test_version_and_status_strings(lib, codes):
    assert lib.s6_version() == 20000
    for name, v in codes.items():
        if name.startswith("S6_ERR_") or name == "S6_OK":
            s = lib.s6_status_str(v).decode()
            assert s and s != "unknown status", name
    assert lib.s6_status_str(12345).decode() == "unknown status"


# Fake, aligned, never-dereferenced addresses: validation must reject the
# call (or find no work) before anything touches them.
P = ctypes.c_void_p(1 << 20)
P_ODD = ctypes.c_void_p((1 << 20) + 2)


def scan(lib, b=2, d=64, L=32, n=16, dt=0, x=P, y=P, A=P, z=None, hl=None):
    return lib.s6_scan_fwd(b, d, L, n, dt, x, P, A, P, P, None, z, None, y, hl, None, 0, None)


def test_scan_validation(lib, codes):
    assert scan(lib, dt=2) == codes["S6_ERR_DTYPE"]
    assert scan(lib, dt=-1) == codes["S6_ERR_DTYPE"]
    assert scan(lib, b=-1) == codes["S6_ERR_SHAPE"]
    assert scan(lib, L=-5) == codes["S6_ERR_SHAPE"]
    assert scan(lib, n=0) == codes["S6_ERR_UNSUPPORTED"]
    assert scan(lib, n=33) == codes["S6_ERR_UNSUPPORTED"]
    assert scan(lib, b=1 << 40, d=1 << 20) == codes["S6_ERR_SHAPE"]  # element count overflows
    assert scan(lib, x=None) == codes["S6_ERR_NULL"]
    assert scan(lib, y=None) == codes["S6_ERR_NULL"]
    assert scan(lib, A=None) == codes["S6_ERR_NULL"]
    assert scan(lib, dt=0, x=P_ODD) == codes["S6_ERR_ALIGN"]  # fp32 needs 4 bytes
    assert scan(lib, dt=1, z=ctypes.c_void_p((1 << 20) + 1)) == codes["S6_ERR_ALIGN"]
    assert scan(lib, A=P_ODD) == codes["S6_ERR_ALIGN"]
    # no work: batch or dim zero returns OK without touching memory
    assert scan(lib, b=0) == codes["S6_OK"]
    assert scan(lib, d=0) == codes["S6_OK"]


def test_last_state_validation(lib, codes):
    f = lib.s6_last_state
    assert f(2, 64, 32, 16, 0, P, P, P, P, None, None, None, 0, None) == codes["S6_ERR_NULL"]  # no h_last
    assert f(2, 64, 32, 40, 0, P, P, P, P, None, P, None, 0, None) == codes["S6_ERR_UNSUPPORTED"]
    assert f(2, 64, 32, 16, 7, P, P, P, P, None, P, None, 0, None) == codes["S6_ERR_DTYPE"]
    assert f(2, 64, 32, 16, 0, None, P, P, P, None, P, None, 0, None) == codes["S6_ERR_NULL"]
    assert f(0, 64, 32, 16, 0, P, P, P, P, None, P, None, 0, None) == codes["S6_OK"]


def test_state_update_validation(lib, codes):
    f = lib.s6_state_update
    assert f(2, 64, 16, 0, None, P, P, P, P, P, None, None, P, None) == codes["S6_ERR_NULL"]
    assert f(2, 64, 16, 0, P, P, P, P, P, P, None, None, None, None) == codes["S6_ERR_NULL"]
    assert f(2, 64, 0, 0, P, P, P, P, P, P, None, None, P, None) == codes["S6_ERR_UNSUPPORTED"]
    assert f(2, 64, 16, 3, P, P, P, P, P, P, None, None, P, None) == codes["S6_ERR_DTYPE"]
    assert f(-2, 64, 16, 0, P, P, P, P, P, P, None, None, P, None) == codes["S6_ERR_SHAPE"]
    assert f(2, 0, 16, 0, P, P, P, P, P, P, None, None, P, None) == codes["S6_OK"]
    assert f(1 << 20, 1 << 20, 16, 0, P, P, P, P, P, P, None, None, P, None) == codes["S6_ERR_SHAPE"]


def test_option_entry_points_validation(lib, codes):
    """The _ex entry points: unknown flag bits, a misaligned bias, and the
    plain checks, all before any HIP call."""
    SP, ZOH = codes["S6_DELTA_SOFTPLUS"], codes["S6_ZOH_EXACT"]
    assert (SP, ZOH) == (1, 2)

    def scan_ex(flags=SP | ZOH, bias=P, b=2, n=16, dt=1, x=P, y=P):
        return lib.s6_scan_fwd_ex(b, 64, 32, n, dt, x, P, bias, flags, P, P, P, None, None, None, y, None,
                                  None, 0, None)

    assert scan_ex(flags=4) == codes["S6_ERR_FLAGS"]
    assert scan_ex(flags=-1) == codes["S6_ERR_FLAGS"]
    assert scan_ex(bias=P_ODD) == codes["S6_ERR_ALIGN"]
    assert scan_ex(n=0) == codes["S6_ERR_UNSUPPORTED"]
    assert scan_ex(dt=5) == codes["S6_ERR_DTYPE"]
    assert scan_ex(x=None) == codes["S6_ERR_NULL"]
    assert scan_ex(y=None) == codes["S6_ERR_NULL"]
    assert scan_ex(b=0) == codes["S6_OK"]
    assert scan_ex(b=0, bias=None, flags=0) == codes["S6_OK"]
    f = lib.s6_last_state_ex
    assert f(2, 64, 32, 16, 1, P, P, P, 8, P, P, None, P, None, 0, None) == codes["S6_ERR_FLAGS"]
    assert f(2, 64, 32, 16, 1, P, P, P_ODD, 1, P, P, None, P, None, 0, None) == codes["S6_ERR_ALIGN"]
    assert f(2, 64, 32, 16, 1, P, P, P, 1, P, P, None, None, None, 0, None) == codes["S6_ERR_NULL"]
    assert f(0, 64, 32, 16, 1, P, P, P, 3, P, P, None, P, None, 0, None) == codes["S6_OK"]
    g = lib.s6_state_update_ex
    assert g(2, 64, 16, 0, P, P, P, P, 16, P, P, P, None, None, P, None) == codes["S6_ERR_FLAGS"]
    assert g(2, 64, 16, 0, P, P, P, P_ODD, 1, P, P, P, None, None, P, None) == codes["S6_ERR_ALIGN"]
    assert g(2, 64, 16, 0, None, P, P, P, 1, P, P, P, None, None, P, None) == codes["S6_ERR_NULL"]
    assert g(2, 0, 16, 0, P, P, P, P, 3, P, P, P, None, None, P, None) == codes["S6_OK"]


def test_conv_entry_points_validation(lib, codes):
    """The convolution front's checks: width 1..4, a filter, a state for
    decode widths above 1, alignment, then the plain checks."""
    def scan(w=P, width=4, bias=None, state=None, flags=0, b=2, x=P, y=P):
        return lib.s6_conv_scan_fwd(b, 64, 32, 16, 1, x, w, bias, width, state, P, None, flags, P, P, P, None, None,
                                    None, y, None, None, 0, None)

    assert scan(width=0) == codes["S6_ERR_UNSUPPORTED"]
    assert scan(width=5) == codes["S6_ERR_UNSUPPORTED"]
    assert scan(width=-1) == codes["S6_ERR_UNSUPPORTED"]
    assert scan(w=None) == codes["S6_ERR_NULL"]
    assert scan(w=None, width=0) == codes["S6_ERR_NULL"]
    assert scan(w=P_ODD) == codes["S6_ERR_ALIGN"]
    assert scan(bias=P_ODD) == codes["S6_ERR_ALIGN"]
    assert scan(state=P_ODD) == codes["S6_ERR_ALIGN"]
    assert scan(flags=4) == codes["S6_ERR_FLAGS"]
    assert scan(x=None) == codes["S6_ERR_NULL"]
    assert scan(y=None) == codes["S6_ERR_NULL"]
    assert scan(b=0) == codes["S6_OK"]
    assert scan(b=0, width=1, state=None) == codes["S6_OK"]

    def step(w=P, width=4, state=P, bias=None, b=2, h=P):
        return lib.s6_conv_state_update(b, 64, 16, 1, h, state, P, w, bias, width, P, None, 0, P, P, P, None, None,
                                        P, None)

    assert step(width=5) == codes["S6_ERR_UNSUPPORTED"]
    assert step(width=0) == codes["S6_ERR_UNSUPPORTED"]
    assert step(w=None, width=0) == codes["S6_ERR_NULL"]
    assert step(state=None) == codes["S6_ERR_NULL"]
    assert step(state=P_ODD) == codes["S6_ERR_ALIGN"]
    assert step(bias=P_ODD) == codes["S6_ERR_ALIGN"]
    assert step(h=None) == codes["S6_ERR_NULL"]
    assert step(b=0) == codes["S6_OK"]
    assert step(b=0, width=1, state=None) == codes["S6_OK"]

    def bwd(w=P, width=4, dw=P, d=64, flags=0, bias=None):
        return lib.s6_conv_scan_bwd(2, d, 32, 16, 1, P, w, bias, width, None, P, None, flags, P, P, P, None, None,
                                    None, P, None, P, P, P, P, P, None, None, None, None, dw, None, None, None, 0,
                                    None)

    assert bwd(width=5) == codes["S6_ERR_UNSUPPORTED"]
    assert bwd(w=None) == codes["S6_ERR_NULL"]
    assert bwd(w=None, width=0) == codes["S6_ERR_NULL"]
    assert bwd(dw=None) == codes["S6_ERR_NULL"]
    assert bwd(bias=P_ODD) == codes["S6_ERR_ALIGN"]
    assert bwd(flags=8) == codes["S6_ERR_FLAGS"]
    assert bwd(flags=2) == codes["S6_ERR_UNSUPPORTED"]  # no exact hold with the front
    assert bwd(d=0, dw=None) == codes["S6_OK"]  # no channels: nothing to write


def test_checkpoint_entry_points_validation(lib, codes):
    """Checkpoints are required when there is work, 4-byte aligned; the
    other checks are those of the _ex entry points."""
    assert codes["S6_CKPT_TOKENS"] == 64

    def fwd(ck=P, b=2, L=32, flags=0):
        return lib.s6_scan_fwd_ckpt(b, 64, L, 16, 1, P, P, None, flags, P, P, P, None, None, None, P, None, ck, None,
                                    0, None)

    assert fwd(ck=None) == codes["S6_ERR_NULL"]
    assert fwd(ck=P_ODD) == codes["S6_ERR_ALIGN"]
    assert fwd(flags=8) == codes["S6_ERR_FLAGS"]
    assert fwd(ck=None, b=0) == codes["S6_OK"]
    assert fwd(ck=None, L=0, b=0) == codes["S6_OK"]

    def bwd(ck=P, flags=0, b=2):
        return lib.s6_scan_bwd_ckpt(b, 64, 32, 16, 1, P, P, None, flags, P, P, P, None, None, ck, P, None, P, P, P, P,
                                    P, None, None, None, None, None, 0, None)

    assert bwd(ck=None) == codes["S6_ERR_NULL"]
    assert bwd(ck=P_ODD) == codes["S6_ERR_ALIGN"]
    assert bwd(flags=8) == codes["S6_ERR_FLAGS"]


def test_backward_validation(lib, codes):
    f = lib.s6_scan_bwd

    def bwd(b=2, d=64, L=32, n=16, dt=1, x=P, dy=P, dA=P, dB=P, dz=None, dh0=None):
        return f(b, d, L, n, dt, x, P, P, P, P, None, None, None, dy, None, P, P, dA, dB, P, None, dz, dh0, None, 0,
                 None)

    assert bwd(dt=3) == codes["S6_ERR_DTYPE"]
    assert bwd(n=0) == codes["S6_ERR_UNSUPPORTED"]
    assert bwd(n=33) == codes["S6_ERR_UNSUPPORTED"]
    assert bwd(L=-1) == codes["S6_ERR_SHAPE"]
    assert bwd(x=None) == codes["S6_ERR_NULL"]
    assert bwd(dy=None) == codes["S6_ERR_NULL"]
    assert bwd(dA=None) == codes["S6_ERR_NULL"]
    assert bwd(dB=None) == codes["S6_ERR_NULL"]
    assert bwd(dz=P_ODD) == codes["S6_ERR_ALIGN"]
    assert bwd(dh0=P_ODD) == codes["S6_ERR_ALIGN"]
    assert bwd(d=0, dA=None) == codes["S6_OK"]  # no channels: nothing to write
    g = lib.s6_scan_bwd_ex

    def bwd_ex(flags=1, bias=P, dbias=P, d=64):
        return g(2, d, 32, 16, 1, P, P, bias, flags, P, P, P, None, None, None, P, None, P, P, P, P, P, None, None,
                 None, dbias, None, 0, None)

    # (dim 0: the checks pass and nothing is launched on these placeholder pointers)
    assert bwd_ex(flags=2, d=0) == codes["S6_OK"]  # the exact hold has a backward
    assert bwd_ex(flags=3, d=0) == codes["S6_OK"]
    assert bwd_ex(flags=8) == codes["S6_ERR_FLAGS"]
    assert bwd_ex(bias=P_ODD) == codes["S6_ERR_ALIGN"]
    assert bwd_ex(dbias=P_ODD) == codes["S6_ERR_ALIGN"]


def test_binding_refuses_host_tensors():
    torch = pytest.importorskip("torch")
    from selective_state_space_63_amd import s6
    x = torch.zeros(1, 4, 8)
    with pytest.raises(ValueError):
        s6.scan_fwd(x, x, torch.zeros(4, 2), torch.zeros(1, 2, 8), torch.zeros(1, 2, 8))


def test_binding_fails_loudly_without_library(tmp_path):
    from selective_state_space_63_amd import s6
    with pytest.raises(FileNotFoundError):
        s6.load_library(str(tmp_path / "missing.so"))


def _size(fn, *args):
    out = ctypes.c_size_t(12345)
    rc = fn(*args, ctypes.byref(out))
    return rc, out.value


def test_workspace_size_queries(lib, codes):
    """Sizes from the launch plan on a 256-CU device (the count the library
    assumes when no device can be queried, and MI355X's): no workspace when
    the (row, 32-channel block) workgroups fill the GPU; for few long rows
    the segment carries.  The 1M-token sequence (1 x 1536 channels, 16
    states): 48 blocks, 5 workgroups of 4 waves per CU -> 26 segments of
    40384 tokens; 25 end states and summed deltas, 26 incoming states."""
    ok = codes["S6_OK"]
    assert _size(lib.s6_scan_fwd_workspace_size, 8, 5120, 2048, 16, 1) == (ok, 0)
    # 1M tokens, 48 channel blocks: 2 x 1280 slots / 48 -> 53 segments of
    # 19840 tokens; 52 end states and summed deltas, 53 incoming states
    nstate = 1536 * 16 * 4
    want = 52 * nstate + 52 * 1536 * 4 + 53 * nstate
    assert _size(lib.s6_scan_fwd_workspace_size, 1, 1536, 1 << 20, 16, 1) == (ok, want)
    assert _size(lib.s6_last_state_workspace_size, 1, 1536, 1 << 20, 16, 1) == (ok, 53 * nstate + 53 * 1536 * 4)
    assert _size(lib.s6_scan_fwd_workspace_size, 0, 1536, 1 << 20, 16, 1) == (ok, 0)
    assert _size(lib.s6_scan_fwd_workspace_size, 1, 1536, 0, 16, 1) == (ok, 0)
    assert _size(lib.s6_scan_fwd_workspace_size, 1, 64, 4096, 40, 1)[0] == codes["S6_ERR_UNSUPPORTED"]
    assert _size(lib.s6_scan_fwd_workspace_size, 1, 64, 4096, 16, 9)[0] == codes["S6_ERR_DTYPE"]
    assert lib.s6_scan_fwd_workspace_size(1, 64, 4096, 16, 1, None) == codes["S6_ERR_NULL"]
    # backward of the 3B layer (one part; the sequential state-only scan
    # fills the GPU): room for the state entering each of the 128 16-token
    # chunks (the exact hold stores them all; the other levels one per
    # 64-token segment), the per-row partials of dA, dD and the bias
    # gradient, and the per-16-channel-block dB/dC partials, which dominate
    rc, full = _size(lib.s6_scan_bwd_workspace_size, 8, 5120, 2048, 16, 1, 0, 0)
    assert rc == ok
    st = 8 * 5120 * 16 * 4
    bc = (5120 // 16) * 8 * 16 * 2048 * 4
    rest = st + 2 * 8 * 5120 * 4 + 2 * bc
    assert full == 128 * st + rest
    rc, ck = _size(lib.s6_scan_bwd_workspace_size, 8, 5120, 2048, 16, 1, 0, 1)
    assert rc == ok and ck == rest
    # with the convolution front: also the gradient of the filtered input and
    # the filter/bias partials
    rc, conv = _size(lib.s6_scan_bwd_workspace_size, 8, 5120, 2048, 16, 1, 4, 0)
    assert rc == ok and conv == full + 8 * 5120 * 2048 * 4 + 8 * 1 * 5120 * 5 * 4
    # a long row (batch 1, 1536 channels, 65536 tokens: the work runs in parts):
    # the 64-token segments' 1023 end states and summed deltas and 1024
    # incoming states stay
    rc, lng = _size(lib.s6_scan_bwd_workspace_size, 1, 1536, 65536, 16, 1, 0, 0)
    rc2, lck = _size(lib.s6_scan_bwd_workspace_size, 1, 1536, 65536, 16, 1, 0, 1)
    st1 = 1536 * 16 * 4
    seg = (1023 * st1 + 255) // 256 * 256 + (1023 * 1536 * 4 + 255) // 256 * 256 + 1024 * st1
    assert rc == ok and rc2 == ok and lng - lck == seg
    assert _size(lib.s6_scan_bwd_workspace_size, 8, 5120, 2048, 16, 1, 5, 0)[0] == codes["S6_ERR_UNSUPPORTED"]
    assert _size(lib.s6_scan_bwd_workspace_size, 8, 5120, 0, 16, 1, 0, 0) == (ok, 0)


def test_workspace_required(lib, codes):
    """A call that needs a workspace fails with S6_ERR_WORKSPACE (NULL or
    too small) or S6_ERR_ALIGN (not 256-byte aligned) before any HIP call;
    one that needs none accepts NULL (checked above with batch or dim 0)."""
    rc, need = _size(lib.s6_scan_fwd_workspace_size, 1, 64, 4096, 16, 1)
    assert rc == codes["S6_OK"] and need > 0  # 2 blocks: cut into segments

    def fwd(ws, nbytes):
        return lib.s6_scan_fwd(1, 64, 4096, 16, 1, P, P, P, P, P, None, None, None, P, None, ws, nbytes, None)

    assert fwd(None, 0) == codes["S6_ERR_WORKSPACE"]
    assert fwd(None, need) == codes["S6_ERR_WORKSPACE"]
    assert fwd(P, need - 1) == codes["S6_ERR_WORKSPACE"]
    assert fwd(ctypes.c_void_p((1 << 20) + 128), need) == codes["S6_ERR_ALIGN"]
    f = lib.s6_last_state
    assert f(1, 64, 4096, 16, 1, P, P, P, P, None, P, None, 0, None) == codes["S6_ERR_WORKSPACE"]
    g = lib.s6_scan_bwd
    assert g(2, 64, 32, 16, 1, P, P, P, P, P, None, None, None, P, None, P, P, P, P, P, None, None, None,
             None, 0, None) == codes["S6_ERR_WORKSPACE"]
    rc, bneed = _size(lib.s6_scan_bwd_workspace_size, 2, 64, 32, 16, 1, 0, 0)
    assert rc == codes["S6_OK"] and bneed > 0
    assert g(2, 64, 32, 16, 1, P, P, P, P, P, None, None, None, P, None, P, P, P, P, P, None, None, None,
             P, bneed - 4, None) == codes["S6_ERR_WORKSPACE"]


def test_library_source_allocates_nothing():
    """No device allocation or release anywhere in the library's sources."""
    import glob
    for f in glob.glob(os.path.join(ROOT, "selective_state_space_63_amd", "csrc", "*")):
        text = open(f).read()
        for word in ("hipMalloc", "hipFree", "hipHostMalloc", "hipMallocAsync"):
            assert word not in text, (f, word)


def test_ssd_validation(lib, codes):
    """The scalar-A chunked scan: dstate up to 16, the common checks; a
    workspace only when few long rows are cut into segments."""
    def f(b=2, d=64, L=32, n=16, dt=1, x=P, y=P, A=P, z=None):
        return lib.s6_ssd_scan_fwd(b, d, L, n, dt, x, P, A, P, P, None, z, None, y, None, None, 0, None)

    assert f(n=17) == codes["S6_ERR_UNSUPPORTED"]
    assert f(n=0) == codes["S6_ERR_UNSUPPORTED"]
    assert f(dt=4) == codes["S6_ERR_DTYPE"]
    assert f(L=-1) == codes["S6_ERR_SHAPE"]
    assert f(x=None) == codes["S6_ERR_NULL"]
    assert f(y=None) == codes["S6_ERR_NULL"]
    assert f(A=None) == codes["S6_ERR_NULL"]
    assert f(A=P_ODD) == codes["S6_ERR_ALIGN"]
    assert f(dt=1, z=ctypes.c_void_p((1 << 20) + 1)) == codes["S6_ERR_ALIGN"]
    assert f(b=0) == codes["S6_OK"]
    # the 3B layer's 2560 waves fill the slots: one segment, no workspace
    assert _size(lib.s6_ssd_scan_fwd_workspace_size, 8, 5120, 2048, 16, 1) == (codes["S6_OK"], 0)
    # 1M tokens of 1536 channels (96 waves): 2 x 3072 slots / 96 = 64 segments
    # of 16384 tokens; 63 end states and summed steps, 64 incoming states
    st = 1536 * 16 * 4
    want = 63 * st + (63 * 1536 * 4 + 255) // 256 * 256 + 64 * st
    assert _size(lib.s6_ssd_scan_fwd_workspace_size, 1, 1536, 1 << 20, 16, 1) == (codes["S6_OK"], want)
    # one 16-channel tile of 256 tokens: 8 segments of 32 tokens
    assert _size(lib.s6_ssd_scan_fwd_workspace_size, 1, 16, 256, 4, 1) == (codes["S6_OK"], 1792 + 512 + 2048)
    assert f(b=1, d=16, L=256, n=4) == codes["S6_ERR_WORKSPACE"]
    assert _size(lib.s6_ssd_scan_fwd_workspace_size, 1, 16, 256, 32, 1)[0] == codes["S6_ERR_UNSUPPORTED"]


def test_noalloc_validation(lib, codes):
    """The static-scratch forward checks its arguments like s6_scan_fwd,
    before any HIP call."""
    def f(b=2, d=64, L=32, n=16, dt=1, x=P, y=P):
        return lib.s6_scan_fwd_noalloc(b, d, L, n, dt, x, P, P, P, P, None, None, None, y, None, None)

    assert f(dt=3) == codes["S6_ERR_DTYPE"]
    assert f(n=40) == codes["S6_ERR_UNSUPPORTED"]
    assert f(L=-2) == codes["S6_ERR_SHAPE"]
    assert f(x=None) == codes["S6_ERR_NULL"]
    assert f(y=None) == codes["S6_ERR_NULL"]
    assert f(b=0) == codes["S6_OK"]


def test_noalloc_scratch_bound():
    """A segmented forward's carries need at most about 2 * slots * 128 *
    (2N + 1) bytes (slots: the workgroup slots of the launch plan on 256 CUs,
    filled twice), i.e. below 12 MB for every state count and sequence
    length, so the 16 MiB static scratch of s6_scan_fwd_noalloc covers every
    call on a 256-CU device."""
    from selective_state_space_63_amd import s6
    worst = 0
    for n in (1, 4, 5, 8, 9, 16, 17, 32):
        for d in (32, 64, 96, 160, 1536):
            for L in (1 << 12, 1 << 16, 1 << 20):
                worst = max(worst, s6.workspace_size("scan_fwd", 1, d, L, n))
    assert 0 < worst <= 12_000_000 < (16 << 20), worst
