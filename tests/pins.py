"""Pins for the fp64 oracle: checks against facts that do not come from the
oracle itself -- hand-derived values (tests/golden), closed forms, a brute
force in 50-digit arithmetic over the materialised (all pairs of tokens) form,
a tree-order scan, and structural invariants.

Each pin is a function taking an oracle object and raising AssertionError on
failure.  test_oracle_pins.py runs them on the real oracle;
test_oracle_mutants.py runs them on copies of the oracle with one deliberate
mistake planted and requires that some pin rejects every copy.

Sources: "【LLM】Mamba和State Space Models详解", sections cited per pin.
"""
from __future__ import annotations

import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand_problem(seed, Bsz=2, D=3, L=40, N=5, gate=True, h0=True, dmin=1e-3, dmax=0.3):
    g = _rng(seed)
    A = -np.exp(g.uniform(np.log(0.3), np.log(8.0), size=(D, N)))
    return dict(
        x=g.standard_normal((Bsz, D, L)),
        delta=np.exp(g.uniform(np.log(dmin), np.log(dmax), size=(Bsz, D, L))),
        A=A,
        Bm=g.standard_normal((Bsz, N, L)),
        Cm=g.standard_normal((Bsz, N, L)),
        Dskip=g.standard_normal(D),
        z=g.standard_normal((Bsz, D, L)) if gate else None,
        h0=g.standard_normal((Bsz, D, N)) if h0 else None,
    )


def _silu(z):
    return z / (1.0 + np.exp(-z))


def _read_golden(name):
    rows = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            rows[" ".join(p for p in parts if not _isnum(p))] = [float(p) for p in parts if _isnum(p)]
    return rows


def _isnum(s):
    try:
        float(s)
        return True
    except ValueError:
        return False


# --------------------------------------------------------------------------
def pin_zero_step_hand(o):
    """Delta = 0: the state never moves, y = C.h0 + D x exactly (§3.2, §2.2).
    Hand values from tests/golden/zero_step_hand.txt."""
    g = _read_golden("zero_step_hand.txt")
    A = np.array([g["A"]])
    h0 = np.array([[g["h0"]]])
    Bv = np.array(g["B"])
    C = np.array([g["C0"], g["C1"], g["C2"]]).T  # (N, L)
    x = np.array([[g["x"]]])
    L = x.shape[-1]
    Bm = np.repeat(Bv[:, None], L, axis=1)[None]
    r = o.scan(x, np.zeros_like(x), A, Bm, C[None], Dskip=np.array(g["D"]), h0=h0)
    assert np.array_equal(r["y"][0, 0], np.array(g["y"])), r["y"]
    assert np.array_equal(r["h_last"], h0)


def pin_scalar_hand(o):
    """Scalar and two-state recurrences worked by hand (§2.3, §2.4); values
    from tests/golden/scalar_hand.txt."""
    g = _read_golden("scalar_hand.txt")
    ln2 = math.log(2.0)
    x = np.array([[[1.0, 2.0, 0.0, -1.0]]])
    dl = np.full_like(x, ln2)
    ones = np.ones((1, 1, 4))
    # case 1
    r = o.scan(x, dl, np.array([[-1.0]]), ones, ones)
    want = np.array(g["case1 y_over_ln2"]) * ln2
    assert np.allclose(r["y"][0, 0], want, rtol=1e-15, atol=1e-15), (r["y"], want)
    # case 2: skip + gate
    z = np.array([[[0.0, 1.0, -1.0, 2.0]]])
    r = o.scan(x, dl, np.array([[-1.0]]), ones, ones, Dskip=np.array([0.5]), z=z)
    want = np.array(g["case2 y"])
    assert np.allclose(r["y"][0, 0], want, rtol=2e-11, atol=1e-11), (r["y"], want)
    # case 3: two states
    x3 = np.array([[[1.0, 0.0, 0.0, 0.0]]])
    Bm = np.ones((1, 2, 4))
    Cm = np.array([[[1.0] * 4, [-1.0] * 4]])
    r = o.scan(x3, np.full_like(x3, ln2), np.array([[-1.0, -2.0]]), Bm, Cm)
    want = np.array(g["case3 y_over_ln2"]) * ln2
    assert np.allclose(r["y"][0, 0], want, rtol=1e-15, atol=1e-15), (r["y"], want)


def pin_lti_convolution(o):
    """Time-invariant Delta, B, C: the recurrence equals a causal convolution
    of x with the kernel K_k = sum_n C[n] exp(k Delta A[n]) Delta B[n], plus
    the skip term and the decayed initial state (§2.5 convolutional form,
    §2.7 time invariance).  The kernel uses exp of k*Delta*A, not powers, and
    numpy.convolve, so it is a different evaluation of the same definition."""
    g = _rng(11)
    Bsz, D, L, N = 2, 3, 96, 4
    A = -np.exp(g.uniform(np.log(0.2), np.log(6.0), size=(D, N)))
    dconst = np.exp(g.uniform(np.log(1e-2), np.log(0.5), size=(Bsz, D)))
    Bc = g.standard_normal((Bsz, N))
    Cc = g.standard_normal((Bsz, N))
    x = g.standard_normal((Bsz, D, L))
    z = g.standard_normal((Bsz, D, L))
    Dsk = g.standard_normal(D)
    h0 = g.standard_normal((Bsz, D, N))
    delta = np.repeat(dconst[:, :, None], L, axis=2)
    Bm = np.repeat(Bc[:, :, None], L, axis=2)
    Cm = np.repeat(Cc[:, :, None], L, axis=2)
    r = o.scan(x, delta, A, Bm, Cm, Dskip=Dsk, z=z, h0=h0)
    k = np.arange(L)
    for b in range(Bsz):
        for d in range(D):
            dt = dconst[b, d]
            K = np.zeros(L)
            init = np.zeros(L)
            for n in range(N):
                K += Cc[b, n] * np.exp(k * dt * A[d, n]) * dt * Bc[b, n]
                init += Cc[b, n] * np.exp((k + 1) * dt * A[d, n]) * h0[b, d, n]
            pre = np.convolve(x[b, d], K)[:L] + Dsk[d] * x[b, d] + init
            want = pre * _silu(z[b, d])
            err = np.max(np.abs(r["y"][b, d] - want) / r["m"][b, d])
            assert err < 1e-12, err


def pin_step_response(o):
    """Constant x, Delta, B: the state is a geometric series,
    h_t = dBx (1 - dA^(t+1)) / (1 - dA) (§2.4 unrolled recurrence)."""
    g = _rng(12)
    D, N, L = 2, 3, 200
    A = -np.array([[0.5, 2.0, 7.0], [1.0, 3.0, 0.1]])
    dt = np.array([0.05, 0.3])
    Bv = g.standard_normal(N)
    Cv = g.standard_normal(N)
    xv = np.array([0.7, -1.3])
    x = np.repeat(xv[None, :, None], L, axis=2)
    delta = np.repeat(dt[None, :, None], L, axis=2)
    Bm = np.repeat(Bv[None, :, None], L, axis=2)
    Cm = np.repeat(Cv[None, :, None], L, axis=2)
    r = o.scan(x, delta, A, Bm, Cm)
    t = np.arange(L)
    for d in range(D):
        y = np.zeros(L)
        for n in range(N):
            dA = math.exp(dt[d] * A[d, n])
            h = dt[d] * Bv[n] * xv[d] * (1.0 - dA ** (t + 1)) / (1.0 - dA)
            y += Cv[n] * h
            assert abs(r["h_last"][0, d, n] - h[-1]) <= 1e-12 * abs(h[-1]) + 1e-300
        err = np.max(np.abs(r["y"][0, d] - y) / r["m"][0, d])
        assert err < 1e-12, err


def brute_force_y(p, dps=50):
    """Materialised form in 50-digit arithmetic: for every pair of tokens
    s <= t, the contribution of x_s to y_t is
      sum_n C_t[n] exp(A[n] * sum_{u=s+1..t} Delta_u) Delta_s B_s[n] x_s,
    the initial state contributes sum_n C_t[n] exp(A[n] sum_{u<=t} Delta_u) h0[n],
    then + D x_t and times SiLU(z_t).  Exponentials of sums, not products of
    exponentials: a different algorithm for the same definition (§3.3)."""
    import mpmath as mp
    mp.mp.dps = dps
    x, dl, A, Bm, Cm = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"]
    Bsz, D, L = x.shape
    N = A.shape[1]
    out = np.zeros((Bsz, D, L))
    for b in range(Bsz):
        for d in range(D):
            cum = [mp.mpf(0)]
            for t in range(L):
                cum.append(cum[-1] + mp.mpf(float(dl[b, d, t])))
            for t in range(L):
                acc = mp.mpf(0)
                for n in range(N):
                    An = mp.mpf(float(A[d, n]))
                    Ct = mp.mpf(float(Cm[b, n, t]))
                    for s in range(t + 1):
                        acc += Ct * mp.exp(An * (cum[t + 1] - cum[s + 1])) * mp.mpf(float(dl[b, d, s])) \
                            * mp.mpf(float(Bm[b, n, s])) * mp.mpf(float(x[b, d, s]))
                    if p.get("h0") is not None:
                        acc += Ct * mp.exp(An * cum[t + 1]) * mp.mpf(float(p["h0"][b, d, n]))
                if p.get("Dskip") is not None:
                    acc += mp.mpf(float(p["Dskip"][d])) * mp.mpf(float(x[b, d, t]))
                if p.get("z") is not None:
                    zz = mp.mpf(float(p["z"][b, d, t]))
                    acc *= zz / (1 + mp.exp(-zz))
                out[b, d, t] = float(acc)
    return out


def pin_brute_force(o):
    """Whole oracle against the 50-digit materialised form on tiny random
    problems with time-varying Delta, B, C, with and without h0 and gate."""
    for seed, kw in ((21, dict(gate=True, h0=True)), (22, dict(gate=False, h0=False)),
                     (23, dict(gate=True, h0=False, Bsz=1, D=2, N=3, L=24))):
        base = dict(Bsz=2, D=3, L=20, N=4)
        base.update(kw)
        p = _rand_problem(seed, **base)
        r = o.scan(**p)
        want = brute_force_y(p)
        err = np.max(np.abs(r["y"] - want) / r["m"])
        assert err < 1e-13, (seed, err)


def pin_tree_scan(o):
    """Associativity (§3.3): the pairs (a, b) with h_t = a_t h_{t-1} + b_t
    combine as (a1, b1) then (a2, b2) -> (a1 a2, a2 b1 + b2).  An inclusive
    Hillis-Steele scan in that combine order must give the oracle's final
    state and outputs."""
    p = _rand_problem(31, Bsz=2, D=2, L=37, N=3)
    r = o.scan(**p)
    x, dl, A, Bm, Cm = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"]
    Bsz, D, L = x.shape
    N = A.shape[1]
    for b in range(Bsz):
        for d in range(D):
            y = np.zeros(L)
            for n in range(N):
                a = np.exp(dl[b, d] * A[d, n])
                bb = dl[b, d] * Bm[b, n] * x[b, d]
                bb = bb.copy()
                bb[0] += a[0] * p["h0"][b, d, n]
                a = a.copy()
                step = 1
                while step < L:
                    a_prev = np.concatenate([np.ones(step), a[:-step]])
                    b_prev = np.concatenate([np.zeros(step), bb[:-step]])
                    bb = a * b_prev + bb
                    a = a_prev * a
                    step *= 2
                y += Cm[b, n] * bb
                assert abs(bb[-1] - r["h_last"][b, d, n]) <= 1e-12 * r["H_last"][b, d, n]
            y = (y + p["Dskip"][d] * x[b, d]) * _silu(p["z"][b, d])
            err = np.max(np.abs(y - r["y"][b, d]) / r["m"][b, d])
            assert err < 1e-13, err


def pin_split_resume(o):
    """Carry semantics: scanning [0, L) equals scanning [0, L1) and then
    [L1, L) from the final state of the first part (the finite state is the
    whole context, §2.4).  Checked at several cut points, including 1 and
    L-1."""
    p = _rand_problem(41, Bsz=2, D=3, L=50, N=4)
    full = o.scan(**p)
    for L1 in (1, 17, 32, 49):
        s1 = {k: (v[..., :L1] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
        s2 = {k: (v[..., L1:] if k in ("x", "delta", "Bm", "Cm", "z") else v) for k, v in p.items()}
        r1 = o.scan(**s1)
        s2["h0"] = r1["h_last"]
        r2 = o.scan(**s2)
        y = np.concatenate([r1["y"], r2["y"]], axis=-1)
        assert np.max(np.abs(y - full["y"]) / full["m"]) < 1e-13
        assert np.max(np.abs(r2["h_last"] - full["h_last"]) / full["H_last"]) < 1e-13


def pin_linearity_and_permutation(o):
    """With h0 = 0 the output is linear in x for fixed Delta, B, C, z; pairs
    are independent, so permuting channels (with their A, D rows) permutes
    the outputs, and each batch row uses only its own B and C (§3.2)."""
    p = _rand_problem(51, Bsz=2, D=4, L=30, N=3, h0=False)
    g = _rng(52)
    x2 = g.standard_normal(p["x"].shape)
    r1 = o.scan(**p)
    q = dict(p, x=x2)
    r2 = o.scan(**q)
    q = dict(p, x=2.5 * p["x"] - 0.75 * x2)
    r3 = o.scan(**q)
    lin = 2.5 * r1["y"] - 0.75 * r2["y"]
    assert np.max(np.abs(r3["y"] - lin) / (2.5 * r1["m"] + 0.75 * r2["m"])) < 1e-13
    perm = np.array([2, 0, 3, 1])
    q = dict(p, x=p["x"][:, perm], delta=p["delta"][:, perm], z=p["z"][:, perm], A=p["A"][perm],
             Dskip=p["Dskip"][perm])
    r4 = o.scan(**q)
    assert np.array_equal(r4["y"], r1["y"][:, perm])
    bperm = np.array([1, 0])
    q = {k: (v[bperm] if k in ("x", "delta", "z", "Bm", "Cm") else v) for k, v in p.items()}
    r5 = o.scan(**q)
    assert np.array_equal(r5["y"], r1["y"][bperm])


def pin_gate_limits(o):
    """SiLU gate: z = 0 gives y = 0 exactly; z = 40 passes (Ch + Dx) times 40
    (to 1e-15 relative); z = -40 gives |y| below 1e-15 |Ch + Dx| * 40."""
    p = _rand_problem(61, Bsz=1, D=2, L=16, N=3)
    ungated = o.scan(**dict(p, z=None))["y"]
    r = o.scan(**dict(p, z=np.zeros_like(p["x"])))
    assert np.all(r["y"] == 0.0)
    r = o.scan(**dict(p, z=np.full_like(p["x"], 40.0)))
    assert np.allclose(r["y"], 40.0 * ungated, rtol=1e-14, atol=0)
    r = o.scan(**dict(p, z=np.full_like(p["x"], -40.0)))
    assert np.all(np.abs(r["y"]) <= 1e-15 * 40.0 * np.abs(ungated) + 1e-300)


def pin_decode_equals_scan(o):
    """S single-token steps from h0 equal one scan over the same S tokens:
    the recurrent form needs only the previous state (§2.4)."""
    p = _rand_problem(71, Bsz=2, D=3, L=12, N=4)
    r = o.scan(**p)
    h = p["h0"].copy()
    H = np.abs(h)
    for s in range(p["x"].shape[-1]):
        y, m = o.step(h, H, p["x"][..., s], p["delta"][..., s], p["A"], p["Bm"][..., s],
                      p["Cm"][..., s], Dskip=p["Dskip"], z=p["z"][..., s])
        assert np.array_equal(y, r["y"][..., s]) and np.array_equal(m, r["m"][..., s])
    assert np.array_equal(h, r["h_last"]) and np.array_equal(H, r["H_last"])


def pin_magnitude_bounds(o):
    """The magnitude m bounds |y| and equals |y| when every term is >= 0."""
    p = _rand_problem(81, Bsz=2, D=2, L=25, N=3)
    r = o.scan(**p)
    assert np.all(r["m"] >= np.abs(r["y"]) * (1 - 1e-15))
    q = dict(p, x=np.abs(p["x"]), Bm=np.abs(p["Bm"]), Cm=np.abs(p["Cm"]), Dskip=np.abs(p["Dskip"]),
             z=None, h0=np.abs(p["h0"]))
    r = o.scan(**q)
    assert np.allclose(r["m"], r["y"], rtol=1e-14, atol=0)


# ----------------------------------------------- discretisation options --
def pin_softplus_hand(o):
    """Step softplus(delta + bias[d]) with a per-channel bias (§3.2, §2.3):
    three channels whose v = delta + bias are 0, ln 3 and -ln 3, worked by
    hand in tests/golden/softplus_hand.txt.  Run as a scan and as decode
    steps."""
    g = _read_golden("softplus_hand.txt")
    v = np.array(g["v"])
    bias = np.array(g["bias"])
    xv = np.array(g["x"])
    L = xv.size
    D = v.size
    steps = np.array([math.log(2.0), math.log(4.0), math.log(4.0 / 3.0)])
    want = np.array([g[f"ch{d} y_over_delta"] for d in range(D)]) * steps[:, None]
    x = np.repeat(xv[None, None, :], D, axis=1)
    raw = np.repeat((v - bias)[None, :, None], L, axis=2)
    ones = np.ones((1, 1, L))
    A = -np.ones((D, 1))
    r = o.scan(x, raw, A, ones, ones, delta_bias=bias, softplus=True)
    assert np.allclose(r["y"][0], want, rtol=1e-14, atol=1e-15), (r["y"], want)
    h = np.zeros((1, D, 1))
    H = np.zeros((1, D, 1))
    for t in range(L):
        y, _ = o.step(h, H, x[..., t], raw[..., t], A, ones[..., t], ones[..., t], delta_bias=bias,
                      softplus=True)
        assert np.allclose(y[0], want[:, t], rtol=1e-14, atol=1e-15), (t, y, want[:, t])


def pin_softplus_limits(o):
    """softplus(v) -> v for large v and -> e^v for very negative v: a scan
    with v = 40 equals the plain scan with Delta = 40, and v = -40 the plain
    scan with Delta = e^-40 (to 1e-15 of the magnitude)."""
    p = _rand_problem(91, Bsz=1, D=2, L=12, N=3)
    bias = np.array([0.75, -1.5])
    for vv, dl in ((40.0, 40.0), (-40.0, math.exp(-40.0))):
        raw = np.full_like(p["delta"], vv) - bias[None, :, None]
        got = o.scan(**dict(p, delta=raw), delta_bias=bias, softplus=True)
        ref = o.scan(**dict(p, delta=np.full_like(p["delta"], dl)))
        assert np.max(np.abs(got["y"] - ref["y"]) / ref["m"]) < 1e-15, vv


def pin_zoh_hand(o):
    """Exact zero-order hold of the input term (§2.3): scalar, two-state and
    A = 0 cases worked by hand in tests/golden/zoh_hand.txt; scan and decode
    steps."""
    g = _read_golden("zoh_hand.txt")
    ln2 = math.log(2.0)
    x = np.array([[g["x"]]])
    L = x.shape[-1]
    ones = np.ones((1, 1, L))
    cases = [
        (x, np.full_like(x, ln2), np.array([[-1.0]]), ones, ones, g["case1 y"]),
        (np.array([[[1.0, 0.0, 0.0, 0.0]]]), np.full_like(x, ln2), np.array([[-1.0, -2.0]]),
         np.ones((1, 2, L)), np.array([[[1.0] * L, [-1.0] * L]]), g["case2 y"]),
        (x, np.full_like(x, 0.25), np.array([[0.0]]), ones, ones, g["case3 y"]),
    ]
    for xc, dl, A, Bm, Cm, want in cases:
        r = o.scan(xc, dl, A, Bm, Cm, zoh=True)
        assert np.allclose(r["y"][0, 0], want, rtol=1e-15, atol=1e-15), (r["y"], want)
        N = A.shape[1]
        h = np.zeros((1, 1, N))
        H = np.zeros((1, 1, N))
        for t in range(L):
            y, _ = o.step(h, H, xc[..., t], dl[..., t], A, Bm[..., t], Cm[..., t], zoh=True)
            assert abs(y[0, 0] - want[t]) <= 1e-15, (t, y, want[t])


def pin_zoh_limits(o):
    """Exact hold against its limits: |Delta A| -> 0 gives the plain step
    Delta B (relative gap about |Delta A| / 2); Delta |A| -> infinity gives
    the coefficient 1 / |A|, so one token from h = 0 leaves h = B x / |A|."""
    p = _rand_problem(92, Bsz=1, D=2, L=20, N=3, h0=False, gate=False)
    tiny = dict(p, A=-np.full_like(p["A"], 1e-9))
    a = o.scan(**tiny, zoh=True)
    b = o.scan(**tiny)
    assert np.max(np.abs(a["y"] - b["y"]) / b["m"]) < 1e-9
    A = -np.array([[2.0, 5.0, 0.5], [1.0, 4.0, 8.0]])
    x = p["x"][..., :1]
    Bm = p["Bm"][..., :1]
    r = o.scan(x, np.full_like(x, 200.0), A, Bm, np.ones_like(Bm), zoh=True)
    want = Bm[0, None, :, 0] * x[0, :, 0, None] / np.abs(A)
    assert np.allclose(r["h_last"][0], want, rtol=1e-15, atol=0), (r["h_last"], want)


def brute_force_options(p, dps=30):
    """Materialised form with both options, in multi-digit arithmetic: the
    step Delta = ln(1 + e^(delta + bias)) straight from the definition, and
    the input coefficient as the hold integral of exp(s A) over [0, Delta]
    by numerical quadrature (not the closed form).  Otherwise as
    brute_force_y."""
    import mpmath as mp
    mp.mp.dps = dps
    x, raw, A, Bm, Cm, bias = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], p["delta_bias"]
    Bsz, D, L = x.shape
    N = A.shape[1]
    out = np.zeros((Bsz, D, L))
    for b in range(Bsz):
        for d in range(D):
            dl = [mp.log(1 + mp.exp(mp.mpf(float(raw[b, d, t])) + mp.mpf(float(bias[d])))) for t in range(L)]
            cum = [mp.mpf(0)]
            for t in range(L):
                cum.append(cum[-1] + dl[t])
            hold = [[mp.quad(lambda s, An=mp.mpf(float(A[d, n])): mp.exp(s * An), [0, dl[t]])
                     for n in range(N)] for t in range(L)]
            for t in range(L):
                acc = mp.mpf(0)
                for n in range(N):
                    An = mp.mpf(float(A[d, n]))
                    Ct = mp.mpf(float(Cm[b, n, t]))
                    for s in range(t + 1):
                        acc += Ct * mp.exp(An * (cum[t + 1] - cum[s + 1])) * hold[s][n] \
                            * mp.mpf(float(Bm[b, n, s])) * mp.mpf(float(x[b, d, s]))
                    if p.get("h0") is not None:
                        acc += Ct * mp.exp(An * cum[t + 1]) * mp.mpf(float(p["h0"][b, d, n]))
                if p.get("Dskip") is not None:
                    acc += mp.mpf(float(p["Dskip"][d])) * mp.mpf(float(x[b, d, t]))
                if p.get("z") is not None:
                    zz = mp.mpf(float(p["z"][b, d, t]))
                    acc *= zz / (1 + mp.exp(-zz))
                out[b, d, t] = float(acc)
    return out


def pin_options_brute_force(o):
    """Softplus step with bias and exact hold together, against the
    quadrature-based materialised form, on tiny random problems with
    time-varying delta, B, C, an initial state and a gate."""
    for seed in (93, 94):
        p = _rand_problem(seed, Bsz=1, D=2, L=10, N=3)
        g = _rng(seed + 100)
        p["delta"] = g.normal(-2.0, 1.5, size=p["delta"].shape)  # raw values, any sign
        p["delta_bias"] = g.normal(0.0, 1.0, size=p["x"].shape[1])
        r = o.scan(**p, softplus=True, zoh=True)
        want = brute_force_options(p)
        err = np.max(np.abs(r["y"] - want) / r["m"])
        assert err < 1e-13, (seed, err)


# --------------------------------------------------------------- backward --
BWD_INPUTS = (("x", "dx"), ("delta", "ddelta"), ("A", "dA"), ("Bm", "dBm"), ("Cm", "dCm"),
              ("Dskip", "dDskip"), ("z", "dz"), ("h0", "dh0"))


def _bwd_problem(seed, **kw):
    p = _rand_problem(seed, **kw)
    g = _rng(seed + 500)
    dy = g.standard_normal(p["x"].shape)
    dhl = g.standard_normal(p["h0"].shape) if p.get("h0") is not None else None
    return p, dy, dhl


def _bwd(o, p, dy, dhl):
    return o.scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p.get("Dskip"), z=p.get("z"),
                      h0=p.get("h0"), dh_last=dhl)


def brute_force_loss(p, dy, dhl, dps=50, bias=None, softplus=False, zoh=False):
    """<dy, y> + <dh_last, h_last> in multi-digit arithmetic from the
    materialised form (exponentials of sums of Delta, as in brute_force_y),
    returned as an mpmath number.  With bias / softplus the step is
    delta + bias[d], or ln(1 + e^(delta + bias[d])) from the definition;
    zoh: token s enters with the hold's integral of e^(rA) over r in
    [0, Delta_s], (e^(Delta_s A) - 1) / A, in place of Delta_s."""
    import mpmath as mp
    mp.mp.dps = dps
    f = lambda v: mp.mpf(v) if not isinstance(v, mp.mpf) else v  # noqa: E731
    x, A, Bm, Cm = p["x"], p["A"], p["Bm"], p["Cm"]
    Bsz, D, L = x.shape
    N = A.shape[1]
    dl = np.empty(p["delta"].shape, dtype=object)
    for idx in np.ndindex(dl.shape):
        v = f(p["delta"][idx]) + (f(bias[idx[1]]) if bias is not None else 0)
        dl[idx] = mp.log(1 + mp.exp(v)) if softplus else v
    total = mp.mpf(0)
    for b in range(Bsz):
        for d in range(D):
            cum = [mp.mpf(0)]
            for t in range(L):
                cum.append(cum[-1] + f(dl[b, d, t]))
            for t in range(L + 1):  # t = L: the final state
                for n in range(N):
                    An = f(A[d, n])
                    last = t == L
                    tt = L - 1 if last else t
                    hn = mp.mpf(0)
                    for s in range(tt + 1):
                        cs = (mp.expm1(An * f(dl[b, d, s])) / An if An != 0 else f(dl[b, d, s])) if zoh \
                            else f(dl[b, d, s])
                        hn += mp.exp(An * (cum[tt + 1] - cum[s + 1])) * cs * f(Bm[b, n, s]) * f(x[b, d, s])
                    if p.get("h0") is not None:
                        hn += mp.exp(An * cum[tt + 1]) * f(p["h0"][b, d, n])
                    if last:
                        if dhl is not None:
                            total += f(dhl[b, d, n]) * hn
                    else:
                        yc_n = f(Cm[b, n, t]) * hn
                        g = mp.mpf(1)
                        if p.get("z") is not None:
                            zz = f(p["z"][b, d, t])
                            g = zz / (1 + mp.exp(-zz))
                        total += f(dy[b, d, t]) * yc_n * g
            if p.get("Dskip") is not None:
                for t in range(L):
                    g = mp.mpf(1)
                    if p.get("z") is not None:
                        zz = f(p["z"][b, d, t])
                        g = zz / (1 + mp.exp(-zz))
                    total += f(dy[b, d, t]) * f(p["Dskip"][d]) * f(x[b, d, t]) * g
    return total


def pin_bwd_directional_brute_force(o):
    """Every gradient of the backward oracle against a directional derivative
    of the 50-digit materialised loss by central differences (step 1e-15,
    truncation far below fp64): an evaluation that shares neither the
    recurrence nor the adjoint formulas (§3.3, §3.4 recomputation)."""
    import mpmath as mp
    p, dy, dhl = _bwd_problem(101, Bsz=2, D=2, L=7, N=3)
    r = _bwd(o, p, dy, dhl)
    g = _rng(102)
    eps = mp.mpf("1e-15")
    for key, gk in BWD_INPUTS:
        v = g.standard_normal(p[key].shape)
        mp.mp.dps = 50
        qp = dict(p)
        qm = dict(p)
        qp[key] = np.array([mp.mpf(float(a)) + eps * mp.mpf(float(b)) for a, b in
                            zip(p[key].ravel(), v.ravel())], dtype=object).reshape(p[key].shape)
        qm[key] = np.array([mp.mpf(float(a)) - eps * mp.mpf(float(b)) for a, b in
                            zip(p[key].ravel(), v.ravel())], dtype=object).reshape(p[key].shape)
        fd = (brute_force_loss(qp, dy, dhl) - brute_force_loss(qm, dy, dhl)) / (2 * eps)
        an = float(np.sum(r[gk] * v))
        scale = float(np.sum(r["m" + gk] * np.abs(v)))
        assert abs(float(fd) - an) <= 1e-13 * scale, (key, float(fd), an, scale)


def pin_bwd_elementwise_fd(o):
    """Every element of every gradient against a central difference of the
    forward oracle (step 1e-6, fp64) on a tiny problem: catches a wrong index
    or layout that a directional check could average out."""
    p, dy, dhl = _bwd_problem(103, Bsz=2, D=2, L=5, N=2)
    r = _bwd(o, p, dy, dhl)

    def loss(q):
        f = o.scan(**q)
        return np.sum(dy * f["y"]) + np.sum(dhl * f["h_last"])

    eps = 1e-6
    for key, gk in BWD_INPUTS:
        fd = np.zeros(p[key].shape)
        for idx in np.ndindex(p[key].shape):
            qp = dict(p)
            qm = dict(p)
            qp[key] = p[key].copy()
            qm[key] = p[key].copy()
            qp[key][idx] += eps
            qm[key][idx] -= eps
            fd[idx] = (loss(qp) - loss(qm)) / (2 * eps)
        err = np.abs(fd - r[gk]) / np.maximum(r["m" + gk], 1e-300)
        assert np.all(err < 1e-6), (key, np.max(err))


def pin_bwd_linear_in_cotangent(o):
    """The gradients are linear in (dy, dh_last) for fixed inputs."""
    p, dy, dhl = _bwd_problem(104, Bsz=1, D=3, L=9, N=3)
    g = _rng(105)
    dy2 = g.standard_normal(dy.shape)
    dhl2 = g.standard_normal(dhl.shape)
    r1 = _bwd(o, p, dy, dhl)
    r2 = _bwd(o, p, dy2, dhl2)
    r3 = _bwd(o, p, 1.5 * dy - 0.5 * dy2, 1.5 * dhl - 0.5 * dhl2)
    for _, gk in BWD_INPUTS:
        want = 1.5 * r1[gk] - 0.5 * r2[gk]
        scale = 1.5 * r1["m" + gk] + 0.5 * r2["m" + gk]
        assert np.all(np.abs(r3[gk] - want) <= 1e-13 * scale + 1e-300), gk


def pin_bwd_no_input_coupling(o):
    """B = 0 and h0 = 0: the state stays 0 and y = D x SiLU(z), so
    dx = dy SiLU(z) D, dD = sum dy SiLU(z) x, dz = dy D x SiLU'(z), and the
    gradients of delta, A and C vanish.  The adjoint is then the
    anti-causal sum lambda_t = sum_{s >= t} exp(A sum_{u=t+1..s} Delta_u)
    dyc_s C_s, evaluated directly (exponentials of sums), which gives
    dB = sum_d lambda Delta x and dh0 = exp(A Delta_0) lambda_0."""
    p, dy, _ = _bwd_problem(106, Bsz=2, D=2, L=6, N=3, h0=False)
    p["Bm"] = np.zeros_like(p["Bm"])
    r = _bwd(o, p, dy, None)
    zz = p["z"]
    s = 1.0 / (1.0 + np.exp(-zz))
    g = zz * s
    dsilu = s * (1.0 + zz * (1.0 - s))
    Dk = p["Dskip"][None, :, None]
    assert np.allclose(r["dx"], dy * g * Dk, rtol=1e-14, atol=0)
    assert np.allclose(r["dDskip"], np.sum(dy * g * p["x"], axis=(0, 2)), rtol=1e-13, atol=0)
    assert np.allclose(r["dz"], dy * Dk * p["x"] * dsilu, rtol=1e-14, atol=0)
    for gk in ("ddelta", "dA", "dCm"):
        assert np.all(r[gk] == 0.0), gk
    Bsz, D, L = p["x"].shape
    N = p["A"].shape[1]
    dB = np.zeros((Bsz, N, L))
    dh0 = np.zeros((Bsz, D, N))
    for b in range(Bsz):
        for d in range(D):
            dl = p["delta"][b, d]
            cum = np.concatenate([[0.0], np.cumsum(dl)])
            dyc = dy[b, d] * g[b, d]
            for n in range(N):
                An = p["A"][d, n]
                lam = np.array([sum(math.exp(An * (cum[s_ + 1] - cum[t + 1])) * dyc[s_] * p["Cm"][b, n, s_]
                                    for s_ in range(t, L)) for t in range(L)])
                dB[b, n] += lam * dl * p["x"][b, d]
                dh0[b, d, n] = math.exp(An * dl[0]) * lam[0]
    assert np.all(np.abs(r["dBm"] - dB) <= 1e-13 * r["mdBm"]), np.max(np.abs(r["dBm"] - dB))
    assert np.all(np.abs(r["dh0"] - dh0) <= 1e-13 * r["mdh0"]), np.max(np.abs(r["dh0"] - dh0))


def pin_bwd_options_directional_brute_force(o):
    """The backward with a step bias and softplus against a directional
    derivative of the 50-digit materialised loss whose step is
    ln(1 + e^(delta + bias)) from the definition: the gradients of the
    stored delta and of the bias (and of every other input)."""
    import mpmath as mp
    p, dy, dhl = _bwd_problem(107, Bsz=2, D=2, L=6, N=3)
    g = _rng(108)
    p["delta"] = g.normal(-1.5, 1.0, size=p["delta"].shape)
    bias = g.normal(0.0, 0.7, size=p["x"].shape[1])
    r = o.scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                   dh_last=dhl, delta_bias=bias, softplus=True)
    eps = mp.mpf("1e-15")
    for key, gk in BWD_INPUTS + (("bias", "ddelta_bias"),):
        base = bias if key == "bias" else p[key]
        v = g.standard_normal(base.shape)
        mp.mp.dps = 50
        plus = np.array([mp.mpf(float(a)) + eps * mp.mpf(float(c)) for a, c in zip(base.ravel(), v.ravel())],
                        dtype=object).reshape(base.shape)
        minus = np.array([mp.mpf(float(a)) - eps * mp.mpf(float(c)) for a, c in zip(base.ravel(), v.ravel())],
                         dtype=object).reshape(base.shape)
        if key == "bias":
            fp = brute_force_loss(p, dy, dhl, bias=plus, softplus=True)
            fm = brute_force_loss(p, dy, dhl, bias=minus, softplus=True)
        else:
            fp = brute_force_loss(dict(p, **{key: plus}), dy, dhl, bias=bias, softplus=True)
            fm = brute_force_loss(dict(p, **{key: minus}), dy, dhl, bias=bias, softplus=True)
        fd = (fp - fm) / (2 * eps)
        an = float(np.sum(r[gk] * v))
        scale = float(np.sum(r["m" + gk] * np.abs(v)))
        assert abs(float(fd) - an) <= 1e-13 * scale, (key, float(fd), an, scale)


def pin_bwd_options_elementwise_fd(o):
    """Every element of the gradients of the stored delta and of the bias
    against central differences of the forward oracle with the same options
    (bias alone, and bias with softplus)."""
    p, dy, dhl = _bwd_problem(109, Bsz=2, D=2, L=5, N=2)
    g = _rng(110)
    p["delta"] = g.normal(-1.0, 1.0, size=p["delta"].shape)
    bias = g.normal(0.5, 0.5, size=p["x"].shape[1])
    for softplus in (False, True):
        q = dict(p)
        if not softplus:
            q["delta"] = np.abs(p["delta"]) * 0.2  # keep the step positive without softplus
        r = o.scan_bwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], dy, Dskip=q["Dskip"], z=q["z"], h0=q["h0"],
                       dh_last=dhl, delta_bias=bias, softplus=softplus)

        def loss(dl, bs):
            f = o.scan(**dict(q, delta=dl), delta_bias=bs, softplus=softplus)
            return np.sum(dy * f["y"]) + np.sum(dhl * f["h_last"])

        eps = 1e-6
        for key, gk in (("delta", "ddelta"), ("bias", "ddelta_bias")):
            base = q["delta"] if key == "delta" else bias
            fd = np.zeros(base.shape)
            for idx in np.ndindex(base.shape):
                bp, bm = base.copy(), base.copy()
                bp[idx] += eps
                bm[idx] -= eps
                fd[idx] = ((loss(bp, bias) - loss(bm, bias)) if key == "delta"
                           else (loss(q["delta"], bp) - loss(q["delta"], bm))) / (2 * eps)
            err = np.abs(fd - r[gk]) / np.maximum(r["m" + gk], 1e-300)
            assert np.all(err < 1e-6), (softplus, key, np.max(err))


def pin_bwd_zoh_directional_brute_force(o):
    """The backward with the exact hold (and softplus with a bias) against a
    directional derivative of the 50-digit materialised loss whose input
    coefficient is (e^(Delta A) - 1) / A: every gradient, including dA
    (through the coefficient) and the stored delta."""
    import mpmath as mp
    p, dy, dhl = _bwd_problem(131, Bsz=2, D=2, L=6, N=3)
    g = _rng(132)
    p["delta"] = g.normal(-1.5, 1.0, size=p["delta"].shape)
    bias = g.normal(0.0, 0.7, size=p["x"].shape[1])
    r = o.scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                   dh_last=dhl, delta_bias=bias, softplus=True, zoh=True)
    eps = mp.mpf("1e-15")
    for key, gk in BWD_INPUTS + (("bias", "ddelta_bias"),):
        base = bias if key == "bias" else p[key]
        v = g.standard_normal(base.shape)
        mp.mp.dps = 50
        plus = np.array([mp.mpf(float(a)) + eps * mp.mpf(float(c)) for a, c in zip(base.ravel(), v.ravel())],
                        dtype=object).reshape(base.shape)
        minus = np.array([mp.mpf(float(a)) - eps * mp.mpf(float(c)) for a, c in zip(base.ravel(), v.ravel())],
                         dtype=object).reshape(base.shape)
        if key == "bias":
            fp = brute_force_loss(p, dy, dhl, bias=plus, softplus=True, zoh=True)
            fm = brute_force_loss(p, dy, dhl, bias=minus, softplus=True, zoh=True)
        else:
            fp = brute_force_loss(dict(p, **{key: plus}), dy, dhl, bias=bias, softplus=True, zoh=True)
            fm = brute_force_loss(dict(p, **{key: minus}), dy, dhl, bias=bias, softplus=True, zoh=True)
        fd = (fp - fm) / (2 * eps)
        an = float(np.sum(r[gk] * v))
        scale = float(np.sum(r["m" + gk] * np.abs(v)))
        assert abs(float(fd) - an) <= 1e-13 * scale, (key, float(fd), an, scale)


def pin_bwd_zoh_elementwise_fd(o):
    """Every element of the gradients of delta and of A with the exact hold
    against central differences of the forward oracle, with steps from 1e-4
    to 0.1 so that Delta A spans both evaluations of dc/dA (its series below
    |Delta A| = 1e-2 and the closed form above)."""
    p, dy, dhl = _bwd_problem(133, Bsz=2, D=2, L=5, N=3)
    g = _rng(134)
    p["delta"] = np.exp(g.uniform(np.log(1e-4), np.log(0.1), size=p["delta"].shape))
    r = o.scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                   dh_last=dhl, zoh=True)
    u = np.abs(p["delta"][:, :, :, None] * p["A"][None, :, None, :])
    assert u.min() < 1e-2 < u.max()

    def loss(q):
        f = o.scan(**q, zoh=True)
        return np.sum(dy * f["y"]) + np.sum(dhl * f["h_last"])

    for key, gk, eps in (("delta", "ddelta", 1e-9), ("A", "dA", 1e-7)):
        base = p[key]
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            bp, bm = base.copy(), base.copy()
            bp[idx] += eps
            bm[idx] -= eps
            fd[idx] = (loss(dict(p, **{key: bp})) - loss(dict(p, **{key: bm}))) / (2 * eps)
        err = np.abs(fd - r[gk]) / np.maximum(r["m" + gk], 1e-300)
        assert np.all(err < 1e-5), (key, np.max(err))


def pin_bwd_zoh_single_token(o):
    """One token from a zero state, loss <dh_last, h_last> = sum_n
    dh_n c(Delta, A_n) B_n x: the gradients are closed forms in the hold's
    coefficient c(Delta, A) = (e^(Delta A) - 1) / A and its derivatives,
    taken here in 50-digit arithmetic (dc/dA by mpmath's numerical
    differentiation) for Delta A from -1e-5 to -3, across the oracle's switch
    between the series and the closed form of dc/dA."""
    import mpmath as mp
    mp.mp.dps = 50
    A = -np.array([[1e-5, 3e-4, 2e-3, 9e-3, 1.1e-2, 0.05, 0.4, 3.0]])
    N = A.shape[1]
    g = _rng(135)
    dt, x = 1.0, 0.75
    Bm = g.standard_normal((1, N, 1))
    dhl = g.standard_normal((1, 1, N))
    r = o.scan_bwd(np.array([[[x]]]), np.array([[[dt]]]), A, Bm, np.zeros((1, N, 1)), np.zeros((1, 1, 1)),
                   dh_last=dhl, zoh=True)

    def c(a, d=mp.mpf(dt)):
        return mp.expm1(d * a) / a

    dA_want = np.array([float(dhl[0, 0, n] * Bm[0, n, 0] * x * mp.diff(c, mp.mpf(A[0, n]))) for n in range(N)])
    assert np.allclose(r["dA"][0], dA_want, rtol=1e-13, atol=0), (r["dA"][0], dA_want)
    ddt_want = sum(float(dhl[0, 0, n] * Bm[0, n, 0] * x * mp.exp(dt * mp.mpf(A[0, n]))) for n in range(N))
    assert abs(r["ddelta"][0, 0, 0] - ddt_want) <= 1e-13 * r["mddelta"][0, 0, 0]
    dx_want = sum(float(dhl[0, 0, n] * Bm[0, n, 0] * c(mp.mpf(A[0, n]))) for n in range(N))
    assert abs(r["dx"][0, 0, 0] - dx_want) <= 1e-13 * r["mdx"][0, 0, 0]
    dB_want = np.array([float(dhl[0, 0, n] * x * c(mp.mpf(A[0, n]))) for n in range(N)])
    assert np.allclose(r["dBm"][0, :, 0], dB_want, rtol=1e-13, atol=0)


# ------------------------------------------------------ convolution front --
def _conv_problem(seed, Bsz=2, D=3, L=30, K=4, bias=True, state=True):
    g = _rng(seed)
    return dict(x=g.standard_normal((Bsz, D, L)), w=g.standard_normal((D, K)) * 0.6,
                bias=g.standard_normal(D) if bias else None,
                state=g.standard_normal((Bsz, D, K - 1)) if state and K > 1 else None)


def pin_conv_hand(o):
    """The convolution front on a hand-worked channel (tests/golden/
    conv_hand.txt; §3.5 "Mamba Block"): taps, their order, the bias and the
    inputs taken from the state before the sequence."""
    g = _read_golden("conv_hand.txt")
    x = np.array(g["x"])[None, None, :]
    w = np.array(g["w"])[None, :]
    bias = np.array(g["bias"])
    state = np.array(g["state"])[None, None, :]
    for key, st in (("xc_state", state), ("xc_nostate", None)):
        xo, _ = o.conv_silu(x, w, bias, st)
        want = _silu(np.array(g[key]))
        assert np.allclose(xo[0, 0], want, rtol=1e-15, atol=0), (key, xo[0, 0], want)


def pin_conv_numpy(o):
    """Against numpy's convolution (a library routine): x' = SiLU(bias +
    (x_ext * reversed w)), x_ext = state ++ x, every width 1..4, with and
    without bias and state."""
    for K in (1, 2, 3, 4):
        for seed, kw in ((90 + K, dict(bias=True, state=True)), (95 + K, dict(bias=False, state=False))):
            p = _conv_problem(seed, K=K, **kw)
            xo, _ = o.conv_silu(**p)
            Bsz, D, L = p["x"].shape
            st = p["state"] if p["state"] is not None else np.zeros((Bsz, D, K - 1))
            full = np.concatenate([st, p["x"]], axis=-1)
            for b in range(Bsz):
                for d in range(D):
                    c = np.convolve(full[b, d], p["w"][d][::-1], mode="valid")
                    if p["bias"] is not None:
                        c = c + p["bias"][d]
                    assert np.allclose(xo[b, d], _silu(c), rtol=1e-13, atol=1e-15), (K, b, d)


def pin_conv_split_resume(o):
    """A sequence cut in two: the second part with the last K-1 inputs of
    the first as its state gives the same output as the whole sequence."""
    p = _conv_problem(101, L=37, K=4)
    whole, _ = o.conv_silu(**p)
    for cut in (1, 2, 3, 17):
        a, _ = o.conv_silu(p["x"][..., :cut], p["w"], p["bias"], p["state"])
        ext = np.concatenate([p["state"], p["x"][..., :cut]], axis=-1)[..., -3:]
        b, _ = o.conv_silu(p["x"][..., cut:], p["w"], p["bias"], ext)
        assert np.allclose(np.concatenate([a, b], axis=-1), whole, rtol=0, atol=0), cut


def pin_conv_magnitude(o):
    """xm bounds the first-order effect of relative perturbations of size
    eps of every term of the convolution's sum (and of x' itself), and is
    >= |x'|; the scan's magnitude is linear in the x magnitudes it is given
    (with no initial state), so doubling xmag doubles m."""
    p = _conv_problem(111, Bsz=1, D=2, L=25, K=4)
    xo, xm = o.conv_silu(**p)
    assert np.all(xm >= np.abs(xo))
    g = _rng(112)
    eps = 1e-7
    K = p["w"].shape[1]
    full = np.concatenate([p["state"], p["x"]], axis=-1)
    worst = 0.0
    for trial in range(20):
        for d in range(2):
            for t in range(25):
                terms = p["w"][d] * full[0, d, t:t + K]
                pert = np.concatenate([[p["bias"][d]], terms])
                pert = pert * (1 + eps * g.choice([-1.0, 1.0], size=pert.size))
                c = pert.sum()
                dev = abs(_silu(c) * (1 + eps * g.choice([-1.0, 1.0])) - xo[0, d, t])
                worst = max(worst, dev / (eps * xm[0, d, t]))
    assert worst <= 1.0 + 1e-3, worst
    # tight somewhere: the bound is not loose by a large factor everywhere
    assert worst >= 0.2, worst
    q = _rand_problem(113, Bsz=1, D=2, L=20, N=3, h0=False)
    r1 = o.scan(**q)
    r2 = o.scan(**q, xmag=2 * np.abs(q["x"]))
    assert np.allclose(r2["m"], 2 * r1["m"], rtol=1e-14, atol=0)
    assert np.array_equal(r2["y"], r1["y"])


def _mp_conv_silu(p, dps=50):
    import mpmath as mp
    mp.mp.dps = dps
    x, w = p["x"], p["w"]
    Bsz, D, L = x.shape
    K = w.shape[1]
    out = np.zeros(x.shape)
    for b in range(Bsz):
        for d in range(D):
            for t in range(L):
                acc = mp.mpf(float(p["bias"][d])) if p["bias"] is not None else mp.mpf(0)
                for k in range(K):
                    s = t - (K - 1) + k
                    if s >= 0:
                        xs = float(x[b, d, s])
                    elif p["state"] is not None:
                        xs = float(p["state"][b, d, K - 1 + s])
                    else:
                        xs = 0.0
                    acc += mp.mpf(float(w[d, k])) * mp.mpf(xs)
                out[b, d, t] = float(acc / (1 + mp.exp(-acc)))
    return out


def pin_conv_scan_brute_force(o):
    """The scan of the convolution front's output against the 50-digit
    materialised form fed with a 50-digit convolution front."""
    p = _rand_problem(121, Bsz=1, D=2, L=16, N=3)
    c = _conv_problem(122, Bsz=1, D=2, L=16, K=4)
    xo, xm = o.conv_silu(**c)
    r = o.scan(**dict(p, x=xo), xmag=xm)
    want = brute_force_y(dict(p, x=_mp_conv_silu(c)))
    err = np.max(np.abs(r["y"] - want) / r["m"])
    assert err < 1e-13, err



def _conv_chain_loss(o, p, c, dy, dhl):
    xo, _ = o.conv_silu(**c)
    f = o.scan(**dict(p, x=xo))
    return np.sum(dy * f["y"]) + np.sum(dhl * f["h_last"])


def _conv_chain_grads(o, p, c, dy, dhl):
    xo, xm = o.conv_silu(**c)
    r = o.scan_bwd(xo, p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p["Dskip"], z=p["z"], h0=p["h0"],
                   dh_last=dhl, xmag=xm)
    cb = o.conv_silu_bwd(c["x"], c["w"], r["dx"], mdxo=r["mdx"], bias=c["bias"], state=c["state"])
    return r, cb


def pin_conv_bwd_chain_fd(o):
    """Gradients through the convolution front and the scan (the oracle's
    scan backward on the front's output, then the front's backward) against
    central differences of the composed forward oracle, for every element of
    x, the filter, the bias and the state."""
    p, dy, dhl = _bwd_problem(141, Bsz=2, D=2, L=9, N=3)
    c = _conv_problem(142, Bsz=2, D=2, L=9, K=3)
    c["x"] = p["x"]
    r, cb = _conv_chain_grads(o, p, c, dy, dhl)
    eps = 1e-6
    for key, gk in (("x", "dx"), ("w", "dw"), ("bias", "dbias"), ("state", "dstate")):
        base = c[key]
        fd = np.zeros(base.shape)
        for idx in np.ndindex(base.shape):
            bp, bm = base.copy(), base.copy()
            bp[idx] += eps
            bm[idx] -= eps
            fd[idx] = (_conv_chain_loss(o, p, dict(c, **{key: bp}), dy, dhl)
                       - _conv_chain_loss(o, p, dict(c, **{key: bm}), dy, dhl)) / (2 * eps)
        err = np.abs(fd - cb[gk]) / np.maximum(cb["m" + gk], 1e-300)
        assert np.all(err < 1e-6), (key, np.max(err))


def pin_conv_bwd_numpy(o):
    """The front's backward against numpy routines: with dxc = dxo SiLU'(xc)
    (xc by numpy's convolution), dx and the state's gradient are the full
    correlation of dxc with the filter, dw the correlation of x (with the
    state before it) with dxc, dbias the sum of dxc; widths 1..4."""
    for K in (1, 2, 3, 4):
        c = _conv_problem(150 + K, Bsz=2, D=3, L=11, K=K)
        g = _rng(160 + K)
        dxo = g.standard_normal(c["x"].shape)
        cb = o.conv_silu_bwd(c["x"], c["w"], dxo, bias=c["bias"], state=c["state"])
        Bsz, D, L = c["x"].shape
        st = c["state"] if c["state"] is not None else np.zeros((Bsz, D, K - 1))
        for b in range(Bsz):
            for d in range(D):
                full = np.concatenate([st[b, d], c["x"][b, d]])
                xc = np.convolve(full, c["w"][d][::-1], mode="valid") + c["bias"][d]
                s = 1.0 / (1.0 + np.exp(-xc))
                dxc = dxo[b, d] * s * (1.0 + xc * (1.0 - s))
                back = np.convolve(dxc, c["w"][d], mode="full")  # gradient of every input of `full`
                assert np.allclose(cb["dx"][b, d], back[K - 1:], rtol=1e-12, atol=1e-14)
                if K > 1:
                    assert np.allclose(cb["dstate"][b, d], back[:K - 1], rtol=1e-12, atol=1e-14)
        for d in range(D):
            dw = np.zeros(K)
            db = 0.0
            for b in range(Bsz):
                full = np.concatenate([st[b, d], c["x"][b, d]])
                xc = np.convolve(full, c["w"][d][::-1], mode="valid") + c["bias"][d]
                s = 1.0 / (1.0 + np.exp(-xc))
                dxc = dxo[b, d] * s * (1.0 + xc * (1.0 - s))
                dw += np.correlate(full, dxc, mode="valid")
                db += dxc.sum()
            assert np.allclose(cb["dw"][d], dw, rtol=1e-12, atol=1e-14), (K, d)
            assert np.isclose(cb["dbias"][d], db, rtol=1e-12, atol=1e-14)


def pin_conv_bwd_magnitude(o):
    """Width 1 and weight 1 make dx = dxc: its magnitude minus mdxo |SiLU'|
    bounds (and is within 5x of) the change of dxc under relative
    perturbations of size eps of the filter's terms; with the backward's
    magnitudes m(2|x'|) for the scan, dB's and dD's magnitudes double."""
    g = _rng(171)
    x = g.standard_normal((1, 2, 30)) * 2
    w = np.ones((2, 1))
    bias = g.standard_normal(2)
    dxo = g.standard_normal(x.shape)
    cb = o.conv_silu_bwd(x, w, dxo, mdxo=np.abs(dxo), bias=bias)
    xc = x + bias[None, :, None]
    s = 1.0 / (1.0 + np.exp(-xc))
    first = np.abs(dxo) * np.abs(s * (1.0 + xc * (1.0 - s)))
    second = cb["mdx"] - first
    eps = 1e-7
    worst = np.zeros(x.shape)
    for trial in range(40):
        tx = x * (1 + eps * g.choice([-1.0, 1.0], size=x.shape))
        tb = bias * (1 + eps * g.choice([-1.0, 1.0], size=bias.shape))
        pert = o.conv_silu_bwd(tx, w, dxo, bias=tb)["dx"]
        worst = np.maximum(worst, np.abs(pert - cb["dx"]) / eps)
    assert np.all(worst <= second * (1 + 1e-3) + 1e-12)
    assert np.max(worst / np.maximum(second, 1e-300)) >= 0.2
    q = _rand_problem(172, Bsz=1, D=2, L=15, N=3, h0=False)
    dy = g.standard_normal(q["x"].shape)
    r1 = o.scan_bwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], dy, Dskip=q["Dskip"], z=q["z"])
    r2 = o.scan_bwd(q["x"], q["delta"], q["A"], q["Bm"], q["Cm"], dy, Dskip=q["Dskip"], z=q["z"],
                    xmag=2 * np.abs(q["x"]))
    assert np.allclose(r2["mdBm"], 2 * r1["mdBm"], rtol=1e-14, atol=0)
    assert np.allclose(r2["mdDskip"], 2 * r1["mdDskip"], rtol=1e-14, atol=0)
    assert np.array_equal(r2["dBm"], r1["dBm"])


# ---------------------------------------------- magnitudes of the backward --
BWD_GRADS = ("dx", "ddelta", "dA", "dBm", "dCm", "dDskip", "dz", "dh0", "ddelta_bias")


def _sign_uniform_bwd(seed, Bsz=2, D=3, L=24, N=4):
    """A backward problem on which every factor of every gradient's sum is
    >= 0: positive x, B, C, D, h0, dy, dh_last and step; z > 0 (SiLU and
    SiLU' positive there); A > 0 (transitions e^(Delta A) > 0, and the
    A-terms of dDelta and dA positive).  The hold's coefficient and its
    derivatives in Delta and A are positive for every A."""
    g = _rng(seed)
    return dict(
        x=g.uniform(0.1, 1.5, (Bsz, D, L)), delta=g.uniform(0.01, 0.3, (Bsz, D, L)),
        A=g.uniform(0.05, 0.6, (D, N)), Bm=g.uniform(0.1, 1.5, (Bsz, N, L)),
        Cm=g.uniform(0.1, 1.5, (Bsz, N, L)), Dskip=g.uniform(0.1, 1.5, D),
        z=g.uniform(0.05, 3.0, (Bsz, D, L)), h0=g.uniform(0.1, 1.5, (Bsz, D, N)),
        dy=g.uniform(0.1, 1.5, (Bsz, D, L)), dh_last=g.uniform(0.1, 1.5, (Bsz, D, N)),
        delta_bias=g.uniform(-0.5, 0.5, D))


def pin_bwd_magnitudes(o):
    """Every magnitude the backward returns is the same sum as its gradient
    over the absolute value of every factor.  So (a) where every factor is
    >= 0 it equals the gradient itself, element by element -- with the
    plain step, with the bias and softplus, with the exact hold and with
    x magnitudes |x| passed in explicitly; and (b) on random inputs it is
    never below |gradient|.  A magnitude scaled by any constant other than
    1 fails (a); a dropped term fails (a) or (b).  These magnitudes are the
    scale of every gradient comparison, so they are pinned here rather than
    through the comparisons that divide by them."""
    base = _sign_uniform_bwd(191)
    cases = [dict(), dict(delta_bias=base["delta_bias"], softplus=True), dict(zoh=True),
             dict(delta_bias=base["delta_bias"], softplus=True, zoh=True), dict(xmag=np.abs(base["x"]))]
    for opt in cases:
        r = o.scan_bwd(base["x"], base["delta"], base["A"], base["Bm"], base["Cm"], base["dy"],
                       Dskip=base["Dskip"], z=base["z"], h0=base["h0"], dh_last=base["dh_last"], **opt)
        for k in BWD_GRADS:
            if k == "ddelta_bias" and "delta_bias" not in opt:
                continue
            assert np.all(r[k] > 0), (k, opt.keys())
            assert np.allclose(r["m" + k], r[k], rtol=1e-13, atol=0), (k, list(opt.keys()),
                                                                       np.max(np.abs(r["m" + k] / r[k] - 1)))
    p, dy, dhl = _bwd_problem(192, Bsz=2, D=3, L=30, N=4)
    g = _rng(193)
    bias = g.standard_normal(3) * 0.5
    for opt in (dict(), dict(delta_bias=bias, softplus=True), dict(zoh=True)):
        r = o.scan_bwd(p["x"], p["delta"], p["A"], p["Bm"], p["Cm"], dy, Dskip=p["Dskip"], z=p["z"],
                       h0=p["h0"], dh_last=dhl, **opt)
        for k in BWD_GRADS:
            if k == "ddelta_bias" and "delta_bias" not in opt:
                continue
            assert np.all(r["m" + k] >= np.abs(r[k]) * (1 - 1e-13)), (k, list(opt.keys()))
            # not a trivial bound: on random signs the sums cancel, but not by orders of magnitude
            assert np.max(np.abs(r[k]) / r["m" + k]) > 0.05, (k, list(opt.keys()))


def pin_conv_bwd_magnitude_bracket(o):
    """The front's backward magnitudes (input, filter, bias, state) on inputs
    where every factor is >= 0 and the filter's output xc lies in (0, 0.3]:
    there they are the gradient itself plus the second-derivative term
    |dxo| |SiLU''(xc)| (|bias| + sum |w x|), which adds at most 30% (on
    that range |SiLU''| <= 0.5, SiLU' >= 0.5 and the sum of terms is xc
    itself).  So gradient <= magnitude <= 1.3 gradient element by element;
    a magnitude off by a constant factor fails one side."""
    g = _rng(194)
    Bsz, D, L, K = 2, 3, 20, 4
    x = g.uniform(0.0, 0.1, (Bsz, D, L))
    w = g.uniform(0.05, 0.5, (D, K))
    bias = g.uniform(0.0, 0.05, D)
    state = g.uniform(0.0, 0.1, (Bsz, D, K - 1))
    dxo = g.uniform(0.1, 1.5, (Bsz, D, L))
    xo, _ = o.conv_silu(x, w, bias, state)
    full = np.concatenate([state, x], axis=-1)
    xc = bias[None, :, None] + sum(w[None, :, k, None] * full[..., k:k + L] for k in range(K))
    assert np.all(xc > 0) and np.all(xc <= 0.3)
    cb = o.conv_silu_bwd(x, w, dxo, mdxo=dxo, bias=bias, state=state)
    for k in ("dx", "dw", "dbias", "dstate"):
        assert np.all(cb[k] > 0), k
        assert np.all(cb["m" + k] >= cb[k] * (1 - 1e-14)), k
        assert np.all(cb["m" + k] <= 1.3 * cb[k]), (k, np.max(cb["m" + k] / cb[k]))


# ---------------------------------------------- scalar A: the matrix form --
def semiseparable_scalar_a(p):
    """The scan with one A value per channel (A[d, n] = a_d), evaluated as a
    matrix: per batch row the Gram matrix G[t, s] = sum_n C_t[n] B_s[n] of
    the shared B and C (L x L, one numpy product), and per channel the
    lower-triangular (semiseparable) mask M[t, s] = exp(a_d (cum_t - cum_s))
    for s <= t from the cumulative step cum_t = sum_{u <= t} Delta_u, so
    y = (G o M) (Delta x) + exp(a_d cum_t) C_t . h0 + D x, then the gate;
    the final state sum_s exp(a_d (cum_L - cum_s)) Delta_s x_s B_s +
    exp(a_d cum_L) h0.  The structured-matrix view of the Mamba-2 abstract
    on the paper-list page, written out densely in fp64."""
    x, dl, A, Bm, Cm = p["x"], p["delta"], p["A"], p["Bm"], p["Cm"]
    Bsz, D, L = x.shape
    y = np.empty((Bsz, D, L))
    hl = np.empty((Bsz, D, Bm.shape[1]))
    tri = np.tril(np.ones((L, L), dtype=bool))
    for b in range(Bsz):
        G = Cm[b].T @ Bm[b]  # (L, L)
        for d in range(D):
            a = A[d, 0]
            cum = np.cumsum(dl[b, d])
            M = np.where(tri, np.exp(a * np.subtract.outer(cum, cum)), 0.0)
            v = dl[b, d] * x[b, d]
            yy = (G * M) @ v
            if p.get("h0") is not None:
                yy += np.exp(a * cum) * (Cm[b].T @ p["h0"][b, d])
            if p.get("Dskip") is not None:
                yy += p["Dskip"][d] * x[b, d]
            if p.get("z") is not None:
                yy *= _silu(p["z"][b, d])
            y[b, d] = yy
            h = Bm[b] @ (np.exp(a * (cum[-1] - cum)) * v)
            if p.get("h0") is not None:
                h += np.exp(a * cum[-1]) * p["h0"][b, d]
            hl[b, d] = h
    return y, hl


def pin_scalar_a_semiseparable(o):
    """With A[d, n] = a_d the oracle's recurrence equals the semiseparable
    matrix form built from the shared Gram matrix of B and C (a different
    evaluation: a matrix product over all pairs of tokens, decays as
    exponentials of differences of cumulative steps).  Several channels with
    different a_d (including a_d = 0 and a strongly decaying one), h0, skip
    and gate."""
    g = _rng(201)
    Bsz, D, L, N = 2, 4, 50, 6
    a = np.array([-0.5, -3.0, 0.0, -12.0])
    p = dict(x=g.standard_normal((Bsz, D, L)), delta=np.exp(g.uniform(np.log(1e-3), np.log(0.5), (Bsz, D, L))),
             A=np.repeat(a[:, None], N, axis=1), Bm=g.standard_normal((Bsz, N, L)), Cm=g.standard_normal((Bsz, N, L)),
             Dskip=g.standard_normal(D), z=g.standard_normal((Bsz, D, L)), h0=g.standard_normal((Bsz, D, N)))
    r = o.scan(**p)
    y, hl = semiseparable_scalar_a(p)
    assert np.max(np.abs(r["y"] - y) / r["m"]) < 1e-12, np.max(np.abs(r["y"] - y) / r["m"])
    assert np.max(np.abs(r["h_last"] - hl) / r["H_last"]) < 1e-12


PINS = [pin_zero_step_hand, pin_scalar_hand, pin_lti_convolution, pin_step_response,
        pin_brute_force, pin_tree_scan, pin_split_resume, pin_linearity_and_permutation,
        pin_gate_limits, pin_decode_equals_scan, pin_magnitude_bounds, pin_softplus_hand,
        pin_softplus_limits, pin_zoh_hand, pin_zoh_limits, pin_options_brute_force,
        pin_bwd_directional_brute_force, pin_bwd_elementwise_fd, pin_bwd_linear_in_cotangent,
        pin_bwd_no_input_coupling, pin_bwd_options_directional_brute_force, pin_bwd_options_elementwise_fd,
        pin_bwd_zoh_directional_brute_force, pin_bwd_zoh_elementwise_fd, pin_bwd_zoh_single_token,
        pin_conv_hand, pin_conv_numpy, pin_conv_split_resume, pin_conv_magnitude,
        pin_conv_scan_brute_force, pin_conv_bwd_chain_fd, pin_conv_bwd_numpy, pin_conv_bwd_magnitude,
        pin_bwd_magnitudes, pin_conv_bwd_magnitude_bracket,
        pin_scalar_a_semiseparable]
