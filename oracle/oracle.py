"""ctypes wrapper around the fp64 C oracle (s6_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
bench's CPU-baseline leg.  The HIP library and its Python binding never import
this module, and this module imports nothing from them.

Inputs are numpy arrays of any float dtype; they are converted to fp64
exactly (every fp32 or bf16 value is an fp64 value), so the oracle sees the
very values the GPU reads.  Outputs are fp64.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "s6_oracle.c")
LIB = os.path.join(HERE, "liboracle_s6.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", "-fno-fast-math", "-ffp-contract=off"]


def build(out: str = LIB, src: str = SRC) -> str:
    """Compile the oracle with gcc.  -ffp-contract=off keeps every product
    and sum a separately rounded fp64 operation, exactly as written."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build_from_text(text: str) -> str:
    """Compile an oracle from source text into a fresh temporary library
    (used by the tests that plant deliberate mistakes)."""
    d = tempfile.mkdtemp(prefix="s6oracle_")
    src = os.path.join(d, "s6_oracle_variant.c")
    with open(src, "w") as f:
        f.write(text)
    return build(os.path.join(d, "liboracle_variant.so"), src)


_P = ctypes.POINTER(ctypes.c_double)
SOFTPLUS, ZOH_EXACT = 1, 2  # option bits of oracle_scan_ex / oracle_step_ex
_I = ctypes.c_int64


class Oracle:
    def __init__(self, path: str | None = None):
        path = path or LIB
        if not os.path.exists(path) or (path == LIB and os.path.getmtime(path) < os.path.getmtime(SRC)):
            if path != LIB:
                raise FileNotFoundError(path)
            build()
        self.lib = ctypes.CDLL(path)
        self.lib.oracle_scan.argtypes = [_I, _I, _I, _I] + [_P] * 12
        self.lib.oracle_scan.restype = None
        self.lib.oracle_step.argtypes = [_I, _I, _I] + [_P] * 11
        self.lib.oracle_step.restype = None
        self.lib.oracle_scan_ex.argtypes = [_I, _I, _I, _I, _P, _P, _P, ctypes.c_int] + [_P] * 10
        self.lib.oracle_scan_ex.restype = None
        self.lib.oracle_step_ex.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, ctypes.c_int] + [_P] * 7
        self.lib.oracle_step_ex.restype = None
        self.lib.oracle_scan_bwd.argtypes = [_I, _I, _I, _I] + [_P] * 26
        self.lib.oracle_scan_bwd.restype = ctypes.c_int
        self.lib.oracle_scan_bwd_ex.argtypes = [_I, _I, _I, _I, _P, _P, _P, ctypes.c_int] + [_P] * 26
        self.lib.oracle_scan_bwd_ex.restype = ctypes.c_int
        self.lib.oracle_scan_xm.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, ctypes.c_int] + [_P] * 10
        self.lib.oracle_scan_xm.restype = None
        self.lib.oracle_step_xm.argtypes = [_I, _I, _I, _P, _P, _P, _P, _P, _P, ctypes.c_int] + [_P] * 7
        self.lib.oracle_step_xm.restype = None
        self.lib.oracle_conv_silu.argtypes = [_I, _I, _I, _I] + [_P] * 6
        self.lib.oracle_conv_silu.restype = ctypes.c_int
        self.lib.oracle_conv_silu_bwd.argtypes = [_I, _I, _I, _I] + [_P] * 14
        self.lib.oracle_conv_silu_bwd.restype = ctypes.c_int
        self.lib.oracle_scan_bwd_xm.argtypes = [_I, _I, _I, _I, _P, _P, _P, _P, ctypes.c_int] + [_P] * 26
        self.lib.oracle_scan_bwd_xm.restype = ctypes.c_int
        self.lib.oracle_num_threads.restype = ctypes.c_int
        self.path = path

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    @staticmethod
    def _in(a, shape):
        if a is None:
            return None, None
        arr = np.ascontiguousarray(np.asarray(a, dtype=np.float64))
        if arr.shape != tuple(shape):
            raise ValueError(f"shape {arr.shape} != {tuple(shape)}")
        return arr, arr.ctypes.data_as(_P)

    @staticmethod
    def _flags(softplus, zoh):
        return (SOFTPLUS if softplus else 0) | (ZOH_EXACT if zoh else 0)

    def scan(self, x, delta, A, Bm, Cm, Dskip=None, z=None, h0=None, delta_bias=None,
             softplus=False, zoh=False, xmag=None):
        """Full scan.  x, delta, z: (batch, D, L); Bm, Cm: (batch, N, L);
        A: (D, N); Dskip: (D,); h0: (batch, D, N); delta_bias: (D,), added
        to delta.  softplus: the step is softplus(delta + delta_bias); zoh:
        exact zero-order-hold input coefficient (exp(Delta A) - 1) / A.
        xmag: (batch, D, L) magnitudes taken for x in m (|x| when None; the
        xm of conv_silu when x is its output).  Returns a dict with y and m
        (batch, D, L), h_last and H_last (batch, D, N), all fp64."""
        x = np.asarray(x)
        Bsz, D, L = x.shape
        N = np.asarray(A).shape[1]
        if N > 256:
            raise ValueError("oracle supports N <= 256")
        keep = []
        args = []
        for a, shp in ((x, (Bsz, D, L)), (delta, (Bsz, D, L)), (A, (D, N)), (Bm, (Bsz, N, L)),
                       (Cm, (Bsz, N, L)), (Dskip, (D,)), (z, (Bsz, D, L)), (h0, (Bsz, D, N))):
            arr, ptr = self._in(a, shp)
            keep.append(arr)
            args.append(ptr)
        y = np.empty((Bsz, D, L))
        m = np.empty((Bsz, D, L))
        hl = np.empty((Bsz, D, N))
        Hl = np.empty((Bsz, D, N))
        outs = [o.ctypes.data_as(_P) for o in (y, m, hl, Hl)]
        flags = self._flags(softplus, zoh)
        if xmag is not None:
            xm, xptr = self._in(xmag, (Bsz, D, L))
            bias, bptr = self._in(delta_bias, (D,))
            self.lib.oracle_scan_xm(Bsz, D, L, N, args[0], xptr, args[1], bptr, flags, *args[2:], *outs)
        elif delta_bias is None and flags == 0:
            self.lib.oracle_scan(Bsz, D, L, N, *args, *outs)
        else:
            bias, bptr = self._in(delta_bias, (D,))
            self.lib.oracle_scan_ex(Bsz, D, L, N, args[0], args[1], bptr, flags, *args[2:], *outs)
        return {"y": y, "m": m, "h_last": hl, "H_last": Hl}

    def step(self, h, H, x, delta, A, Bm, Cm, Dskip=None, z=None, delta_bias=None, softplus=False,
             zoh=False, xmag=None):
        """One decode token.  h, H: (batch, D, N) fp64 arrays updated in place;
        x, delta, z: (batch, D); Bm, Cm: (batch, N); options and xmag as in
        scan.  Returns (y, m)."""
        if h.dtype != np.float64 or not h.flags.c_contiguous or H.dtype != np.float64:
            raise ValueError("h and H must be contiguous float64 arrays")
        Bsz, D, N = h.shape
        keep = []
        args = []
        for a, shp in ((x, (Bsz, D)), (delta, (Bsz, D)), (A, (D, N)), (Bm, (Bsz, N)),
                       (Cm, (Bsz, N)), (Dskip, (D,)), (z, (Bsz, D))):
            arr, ptr = self._in(a, shp)
            keep.append(arr)
            args.append(ptr)
        y = np.empty((Bsz, D))
        m = np.empty((Bsz, D))
        flags = self._flags(softplus, zoh)
        if xmag is not None:
            xm, xptr = self._in(xmag, (Bsz, D))
            bias, bptr = self._in(delta_bias, (D,))
            self.lib.oracle_step_xm(Bsz, D, N, h.ctypes.data_as(_P), H.ctypes.data_as(_P), args[0], xptr,
                                    args[1], bptr, flags, *args[2:], y.ctypes.data_as(_P),
                                    m.ctypes.data_as(_P))
        elif delta_bias is None and flags == 0:
            self.lib.oracle_step(Bsz, D, N, h.ctypes.data_as(_P), H.ctypes.data_as(_P), *args,
                                 y.ctypes.data_as(_P), m.ctypes.data_as(_P))
        else:
            bias, bptr = self._in(delta_bias, (D,))
            self.lib.oracle_step_ex(Bsz, D, N, h.ctypes.data_as(_P), H.ctypes.data_as(_P), args[0],
                                    args[1], bptr, flags, *args[2:], y.ctypes.data_as(_P),
                                    m.ctypes.data_as(_P))
        return y, m

    def conv_silu(self, x, w, bias=None, state=None):
        """The convolution front: x' = SiLU(bias[d] + sum_k w[d, k]
        x_{t-K+1+k}) along the tokens of each (batch, channel) row, inputs
        before the sequence from state (batch, D, K-1) (oldest first) or 0.
        x: (batch, D, L); w: (D, K); bias: (D,).  Returns (x', xm), both
        (batch, D, L) fp64; xm is the magnitude the error metric takes for
        x' (pass it to scan / step as xmag)."""
        x = np.asarray(x)
        Bsz, D, L = x.shape
        K = np.asarray(w).shape[1]
        xa, xp = self._in(x, (Bsz, D, L))
        wa, wp = self._in(w, (D, K))
        ba, bp = self._in(bias, (D,))
        sa, sp = self._in(state, (Bsz, D, K - 1)) if state is not None else (None, None)
        xo = np.empty((Bsz, D, L))
        xm = np.empty((Bsz, D, L))
        rc = self.lib.oracle_conv_silu(Bsz, D, L, K, xp, wp, bp, sp, xo.ctypes.data_as(_P),
                                       xm.ctypes.data_as(_P))
        if rc != 0:
            raise ValueError("conv_silu: width must be >= 1")
        return xo, xm

    def conv_silu_bwd(self, x, w, dxo, mdxo=None, bias=None, state=None):
        """Gradients through the convolution front from dxo, the gradient
        with respect to its output (and mdxo, that gradient's magnitude).
        Returns a dict: dx (batch, D, L), dw (D, K), dbias (D,), dstate
        (batch, D, K-1), and their magnitudes under the keys prefixed with
        "m"."""
        x = np.asarray(x)
        Bsz, D, L = x.shape
        K = np.asarray(w).shape[1]
        keep = []
        ptrs = []
        for a, shp in ((x, (Bsz, D, L)), (w, (D, K)), (bias, (D,)), (state, (Bsz, D, K - 1)),
                       (dxo, (Bsz, D, L)), (mdxo, (Bsz, D, L))):
            arr, ptr = self._in(a, shp) if a is not None else (None, None)
            keep.append(arr)
            ptrs.append(ptr)
        shapes = {"dx": (Bsz, D, L), "dw": (D, K), "dbias": (D,), "dstate": (Bsz, D, K - 1)}
        out = {k: np.empty(v) for k, v in shapes.items()}
        out.update({"m" + k: np.empty(v) for k, v in shapes.items()})
        order = ["dx", "dw", "dbias", "dstate"]
        optr = [out[k].ctypes.data_as(_P) for k in order] + [out["m" + k].ctypes.data_as(_P) for k in order]
        rc = self.lib.oracle_conv_silu_bwd(Bsz, D, L, K, *ptrs, *optr)
        if rc != 0:
            raise ValueError(f"conv_silu_bwd failed ({rc})")
        return out

    def scan_bwd(self, x, delta, A, Bm, Cm, dy, Dskip=None, z=None, h0=None, dh_last=None,
                 delta_bias=None, softplus=False, zoh=False, xmag=None):
        """Gradients of <dy, y> + <dh_last, h_last> for the scan (with the
        step bias, softplus and exact hold of scan(); xmag as in scan).  Returns a
        dict: dx, ddelta (of the stored delta), dz (batch, D, L); dA (D, N);
        dBm, dCm (batch, N, L); dDskip (D,); dh0 (batch, D, N); ddelta_bias
        (D,); and for each the magnitude under the key prefixed with "m"
        (mdx, mddelta, ...).  dz is zero without a gate."""
        x = np.asarray(x)
        Bsz, D, L = x.shape
        N = np.asarray(A).shape[1]
        if N > 256:
            raise ValueError("oracle supports N <= 256")
        keep = []
        args = []
        for a, shp in ((x, (Bsz, D, L)), (delta, (Bsz, D, L)), (A, (D, N)), (Bm, (Bsz, N, L)),
                       (Cm, (Bsz, N, L)), (Dskip, (D,)), (z, (Bsz, D, L)), (h0, (Bsz, D, N)),
                       (dy, (Bsz, D, L)), (dh_last, (Bsz, D, N))):
            arr, ptr = self._in(a, shp)
            keep.append(arr)
            args.append(ptr)
        shapes = {"dx": (Bsz, D, L), "ddelta": (Bsz, D, L), "dA": (D, N), "dBm": (Bsz, N, L),
                  "dCm": (Bsz, N, L), "dDskip": (D,), "dz": (Bsz, D, L), "dh0": (Bsz, D, N),
                  "ddelta_bias": (D,)}
        out = {k: np.empty(v) for k, v in shapes.items()}
        out.update({"m" + k: np.empty(v) for k, v in shapes.items()})
        order = ["dx", "ddelta", "dA", "dBm", "dCm", "dDskip", "dz", "dh0", "ddelta_bias"]
        ptrs = [out[k].ctypes.data_as(_P) for k in order] + [out["m" + k].ctypes.data_as(_P) for k in order]
        bias, bptr = self._in(delta_bias, (D,))
        xm, xptr = self._in(xmag, (Bsz, D, L))
        rc = self.lib.oracle_scan_bwd_xm(Bsz, D, L, N, args[0], xptr, args[1], bptr, self._flags(softplus, zoh),
                                         *args[2:], *ptrs)
        if rc == -2:
            raise ValueError("oracle_scan_bwd: unsupported option")
        if rc != 0:
            raise MemoryError("oracle_scan_bwd: out of memory")
        return out


_default = None


def default() -> Oracle:
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def scaled_error(got, ref, mag) -> float:
    """Largest componentwise error |got - ref| / mag, where mag is the
    oracle's absolute-value magnitude of the same element (mag >= |ref|).
    0/0 counts as 0; x/0 with x > 0 as infinity.  Non-finite got -> inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    mag = np.asarray(mag, dtype=np.float64)
    if got.size == 0:
        return 0.0
    if not np.all(np.isfinite(got)):
        return float("inf")
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        e = np.where(diff == 0.0, 0.0, diff / mag)
    return float(np.max(e))


def relative_error(got, ref, floor_frac=1e-3) -> float:
    """Plain max |got - ref| / |ref| over elements with |ref| >= floor_frac *
    max|ref| (reported beside the scaled error; it is unbounded near zero
    crossings, so elements close to zero are left out)."""
    got = np.asarray(got, dtype=np.float64).ravel()
    ref = np.asarray(ref, dtype=np.float64).ravel()
    if ref.size == 0:
        return 0.0
    big = np.abs(ref) >= floor_frac * np.max(np.abs(ref))
    if not np.any(big):
        return 0.0
    return float(np.max(np.abs(got[big] - ref[big]) / np.abs(ref[big])))
