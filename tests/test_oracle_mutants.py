"""Plant one plausible mistake at a time in a copy of the oracle's source,
build it, and require that at least one pin rejects it.  This shows that the
pins constrain every part of the oracle: dropped terms, wrong signs, wrong
indices, swapped operands, a wrong update order, the other reading of the
discretisation.  The real oracle file is never modified."""
import os

import pytest

import pins
from oracle import oracle as O

SRC = open(O.SRC).read()

# (name, [(old, new), ...]) -- each `old` must occur exactly once.
MUTANTS = [
    ("skip_dropped", [("double skip = dskip * xt;", "double skip = 0.0 * dskip * xt;")]),
    ("output_before_update", [
        ("h[n] = a * h[n] + bx;               /* update first ... */",
         "double hp_ = h[n]; h[n] = a * h[n] + bx;"),
        ("acc += Ct[n * bstride] * h[n];      /* ... then read the output from the new state */",
         "acc += Ct[n * bstride] * hp_;")]),
    ("B_C_swapped", [
        ("* Bt[n * bstride];", "* Ct[n * bstride];"),
        ("acc += Ct[n * bstride] * h[n];      /*", "acc += Bt[n * bstride] * h[n];      /*")]),
    ("exp_sign", [("double a = exp(dt * Ad[n]);         /*", "double a = exp(-dt * Ad[n]);         /*")]),
    ("dt_dropped_from_input", [("(zoh ? zoh_coef(dt, Ad[n]) : dt) * Bt",
                                "(zoh ? zoh_coef(dt, Ad[n]) : 1.0) * Bt")]),
    ("gate_before_skip", [("        yt *= g;\n        mag *= fabs(g);\n      }\n      y[p * L + t] = yt;",
                           "        yt = (yt - dsk * x[p * L + t]) * g + dsk * x[p * L + t];\n"
                           "        mag *= fabs(g);\n      }\n      y[p * L + t] = yt;")]),
    ("h0_ignored", [("h[n] = h0 ? h0[p * N + n] : 0.0;", "h[n] = 0.0;")]),
    ("exact_zoh_for_B", [("(zoh ? zoh_coef(dt, Ad[n]) : dt) * Bt", "zoh_coef(dt, Ad[n]) * Bt")]),
    ("zoh_never", [("(zoh ? zoh_coef(dt, Ad[n]) : dt) * Bt", "dt * Bt")]),
    ("zoh_sign", [("return a != 0.0 ? expm1(dt * a) / a : dt;", "return a != 0.0 ? -expm1(dt * a) / a : dt;")]),
    ("zoh_extra_step", [("return a != 0.0 ? expm1(dt * a) / a : dt;",
                         "return a != 0.0 ? dt * expm1(dt * a) / a : dt;")]),
    ("zoh_limit_at_zero", [("return a != 0.0 ? expm1(dt * a) / a : dt;", "return a != 0.0 ? expm1(dt * a) / a : 0.0;")]),
    ("softplus_no_abs", [("log1p(exp(-fabs(v)))", "log1p(exp(-v))")]),
    ("softplus_is_exp", [("return (v > 0.0 ? v : 0.0) + log1p(exp(-fabs(v)));", "return exp(v);")]),
    ("bias_dropped", [("double v = dbias ? raw + dbias[d] : raw;", "double v = raw;")]),
    ("bias_channel", [("raw + dbias[d]", "raw + dbias[0]")]),
    ("bias_after_softplus", [("double v = dbias ? raw + dbias[d] : raw;\n  return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;",
                              "return ((flags & ORACLE_DELTA_SOFTPLUS) ? softplus(raw) : raw) + (dbias ? dbias[d] : 0.0);")]),
    ("softplus_always", [("return (flags & ORACLE_DELTA_SOFTPLUS) ? softplus(v) : v;", "return softplus(v);")]),
    # backward
    ("bwd_decay_same_step", [("const double l = dyc * Ct + lam[n];", "const double l = a * (dyc * Ct + lam[n]);")]),
    ("bwd_carry_without_decay", [("lam[n] = a * l; /* carried", "lam[n] = l; /* carried")]),
    ("bwd_ddelta_no_input_term", [("gd += l * (Ad[n] * a * hp + cfd * Bt * xt);", "gd += l * (Ad[n] * a * hp);")]),
    ("bwd_ddelta_new_state", [("gd += l * (Ad[n] * a * hp + cfd * Bt * xt);", "gd += l * (Ad[n] * a * ht + cfd * Bt * xt);")]),
    ("bwd_dA_no_step", [("dA_b[p * N + n] += l * dt * a * hp + l * cfa * Bt * xt;",
                         "dA_b[p * N + n] += l * a * hp + l * cfa * Bt * xt;")]),
    ("bwd_dB_no_x", [("dBm[b * N * L + n * L + t] += l * cf * xt;", "dBm[b * N * L + n * L + t] += l * cf;")]),
    ("bwd_dC_prev_state", [("dCm[b * N * L + n * L + t] += dyc * ht;", "dCm[b * N * L + n * L + t] += dyc * hp;")]),
    ("bwd_dz_silu_not_derivative", [("dz[p * L + t] = z ? dy[p * L + t] * yc * dsilu : 0.0;",
                                     "dz[p * L + t] = z ? dy[p * L + t] * yc * g : 0.0;")]),
    ("bwd_gate_ignored", [("const double dyc = dy[p * L + t] * g;", "const double dyc = dy[p * L + t];")]),
    ("bwd_dh_last_ignored", [("lam[n] = dh_last ? dh_last[p * N + n] : 0.0;", "lam[n] = 0.0;")]),
    ("bwd_dx_no_skip", [("dx[p * L + t] = dyc * dsk + gx;", "dx[p * L + t] = gx;")]),
    ("bwd_dD_ungated", [("dD_b[p] += dyc * xt;", "dD_b[p] += dy[p * L + t] * xt;")]),
    ("bwd_dx_B_of_next_state", [("gx += l * cf * Bt;", "gx += l * cf * Bb[((n + 1) % N) * L + t];")]),
    # backward of the exact hold
    ("bwd_zoh_coef_is_step", [("const double cf = zoh ? zoh_coef(dt, Ad[n]) : dt;", "const double cf = dt;")]),
    ("bwd_zoh_dstep_is_one", [("const double cfd = zoh ? a : 1.0;", "const double cfd = 1.0;")]),
    ("bwd_zoh_no_dA_term", [("const double cfa = zoh ? zoh_dcoef_da(dt, Ad[n]) : 0.0;", "const double cfa = 0.0;")]),
    ("bwd_zoh_dA_sign", [("q = (u * exp(u) - expm1(u)) / (u * u);", "q = (expm1(u) - u * exp(u)) / (u * u);")]),
    ("bwd_zoh_series_term", [("(1.0 / 3 + u * (1.0 / 8", "(1.0 / 6 + u * (1.0 / 8")]),
    ("bwd_zoh_forward_plain", [("const double cb = (zoh ? zoh_coef(dt, Ad[n]) : dt) * Bb[n * L + t];",
                                "const double cb = dt * Bb[n * L + t];")]),
    ("bwd_softplus_chain_missing", [("const double js = sp ? sigmoid(v) : 1.0;", "const double js = 1.0;")]),
    ("bwd_softplus_chain_of_step", [("const double js = sp ? sigmoid(v) : 1.0;", "const double js = sp ? sigmoid(dt) : 1.0;")]),
    ("bwd_bias_grad_dropped", [("db_b[p] += gd * js;", "db_b[p] += 0.0 * gd * js;")]),
    ("bwd_reverse_step_without_options", [
        ("const double dt = step_of(delta[p * L + t], dbias, d, flags), xt = x[p * L + t];\n"
         "        const double xm = xmag ? xmag[p * L + t] : fabs(xt);\n        const double g",
         "const double dt = delta[p * L + t], xt = x[p * L + t];\n"
         "        const double xm = xmag ? xmag[p * L + t] : fabs(xt);\n        const double g")]),
    ("delta_index_shift", [("double dt = step_of(delta[p * L + t], dbias, d, flags);",
                            "double dt = step_of(delta[p * L + (t > 0 ? t - 1 : 0)], dbias, d, flags);")]),
    ("A_state_index", [("double a = exp(dt * Ad[n]);         /*", "double a = exp(dt * Ad[(n + 1) % N]);         /*")]),
    ("B_batch_index", [("const double* Bb = Bm + b * N * L;\n    const double* Cb = Cm + b * N * L;\n    double dsk",
                        "const double* Bb = Bm;\n    const double* Cb = Cm + b * N * L;\n    double dsk")]),
    ("BC_layout_transposed", [("Bb + t, Cb + t,\n                               L,",
                               "Bb + t * N, Cb + t * N,\n                               1,")]),
    ("skip_channel_index", [("double dsk = Dskip ? Dskip[d] : 0.0;\n    for (int64_t t",
                             "double dsk = Dskip ? Dskip[0] : 0.0;\n    for (int64_t t")]),
    ("sigmoid_sign", [("return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));")]),
    ("input_decayed_same_step", [("h[n] = a * h[n] + bx;", "h[n] = a * (h[n] + bx);")]),
    ("magnitude_drops_input", [("H[n] = fabs(a) * H[n] + fabs(cb) * xm;", "H[n] = fabs(a) * H[n];")]),
    # convolution front
    ("conv_tap_shift", [("int64_t s = t - (K - 1) + k;  /* token of tap k */", "int64_t s = t - K + k;")]),
    ("conv_taps_reversed", [("acc += w[d * K + k] * xs;", "acc += w[d * K + (K - 1 - k)] * xs;")]),
    ("conv_weight_channel", [("acc += w[d * K + k] * xs;", "acc += w[k] * xs;")]),
    ("conv_state_ignored", [("(state ? state[p * (K - 1) + (K - 1) + s] : 0.0)", "0.0")]),
    ("conv_state_order", [("? state[p * (K - 1) + (K - 1) + s]", "? state[p * (K - 1) - 1 - s]")]),
    ("conv_bias_dropped", [("double b0 = bias ? bias[d] : 0.0;", "double b0 = 0.0;")]),
    ("conv_no_silu", [("xo[p * L + t] = acc * sg;", "xo[p * L + t] = acc;")]),
    ("scan_xmag_ignored", [("double xm = xmag ? xmag[p * L + t] : fabs(x[p * L + t]);",
                           "double xm = fabs(x[p * L + t]);")]),
    ("conv_bwd_taps_reversed", [("        g += w[d * K + k] * dxc[p * L + t];", "        g += w[d * K + (K - 1 - k)] * dxc[p * L + t];")]),
    ("conv_bwd_silu_prime", [("const double d1 = sg * (1.0 + acc * (1.0 - sg));", "const double d1 = sg;")]),
    ("conv_bwd_dw_shift", [("xs = conv_input(p, t + k - (K - 1), L, K, x, state);",
                            "xs = conv_input(p, t + k - K, L, K, x, state);")]),
    ("conv_bwd_state_index", [("if (dstate) dstate[p * (K - 1) + (K - 1) + s] = g;", "if (dstate) dstate[p * (K - 1) - 1 - s] = g;")]),
    ("conv_bwd_bias_grad", [("          double xs = 1.0;\n", "          double xs = 0.0;\n")]),
    ("conv_bwd_no_second_derivative", [("fabs(dxo[p * L + t]) * fabs(d2) * mag;", "0.0 * mag;")]),
    ("scan_bwd_xmag_ignored", [("        const double xm = xmag ? xmag[p * L + t] : fabs(xt);\n        const double g",
                                "        const double xm = fabs(xt);\n        const double g")]),
    ("conv_magnitude_no_sum", [("fabs(sg * (1.0 + acc * (1.0 - sg))) * mag;", "0.0 * mag;")]),
    # backward magnitudes scaled by a constant (the scale of every gradient comparison)
    ("bwd_magnitude_mdx_x100", [('if (mdx) mdx[p * L + t] = fabs(dyc * dsk) + mgx;', 'if (mdx) mdx[p * L + t] = 100.0 * (fabs(dyc * dsk) + mgx);')]),
    ("bwd_magnitude_mdx_x0.01", [('if (mdx) mdx[p * L + t] = fabs(dyc * dsk) + mgx;', 'if (mdx) mdx[p * L + t] = 0.01 * (fabs(dyc * dsk) + mgx);')]),
    ("bwd_magnitude_mddelta_x100", [('if (mddelta) mddelta[p * L + t] = mgd * js;', 'if (mddelta) mddelta[p * L + t] = 100.0 * mgd * js;')]),
    ("bwd_magnitude_mddelta_x0.01", [('if (mddelta) mddelta[p * L + t] = mgd * js;', 'if (mddelta) mddelta[p * L + t] = 0.01 * mgd * js;')]),
    ("bwd_magnitude_mdA_x100", [('if (mdA) mdA[i] = ms;', 'if (mdA) mdA[i] = 100.0 * ms;')]),
    ("bwd_magnitude_mdA_x0.01", [('if (mdA) mdA[i] = ms;', 'if (mdA) mdA[i] = 0.01 * ms;')]),
    ("bwd_magnitude_mdB_x100", [('if (mdB) mdB[b * N * L + n * L + t] += ml * fabs(cf) * xm;', 'if (mdB) mdB[b * N * L + n * L + t] += 100.0 * ml * fabs(cf) * xm;')]),
    ("bwd_magnitude_mdB_x0.01", [('if (mdB) mdB[b * N * L + n * L + t] += ml * fabs(cf) * xm;', 'if (mdB) mdB[b * N * L + n * L + t] += 0.01 * ml * fabs(cf) * xm;')]),
    ("bwd_magnitude_mdC_x100", [('if (mdC) mdC[b * N * L + n * L + t] += fabs(dyc) * Ht;', 'if (mdC) mdC[b * N * L + n * L + t] += 100.0 * fabs(dyc) * Ht;')]),
    ("bwd_magnitude_mdC_x0.01", [('if (mdC) mdC[b * N * L + n * L + t] += fabs(dyc) * Ht;', 'if (mdC) mdC[b * N * L + n * L + t] += 0.01 * fabs(dyc) * Ht;')]),
    ("bwd_magnitude_mdD_x100", [('if (mdD) mdD[d] = ms;', 'if (mdD) mdD[d] = 100.0 * ms;')]),
    ("bwd_magnitude_mdD_x0.01", [('if (mdD) mdD[d] = ms;', 'if (mdD) mdD[d] = 0.01 * ms;')]),
    ("bwd_magnitude_mdz_x100", [('if (mdz) mdz[p * L + t] = z ? fabs(dy[p * L + t]) * mdsilu * myc : 0.0;', 'if (mdz) mdz[p * L + t] = z ? 100.0 * fabs(dy[p * L + t]) * mdsilu * myc : 0.0;')]),
    ("bwd_magnitude_mdz_x0.01", [('if (mdz) mdz[p * L + t] = z ? fabs(dy[p * L + t]) * mdsilu * myc : 0.0;', 'if (mdz) mdz[p * L + t] = z ? 0.01 * fabs(dy[p * L + t]) * mdsilu * myc : 0.0;')]),
    ("bwd_magnitude_mdh0_x100", [('if (mdh0) mdh0[p * N + n] = Lam[n];', 'if (mdh0) mdh0[p * N + n] = 100.0 * Lam[n];')]),
    ("bwd_magnitude_mdh0_x0.01", [('if (mdh0) mdh0[p * N + n] = Lam[n];', 'if (mdh0) mdh0[p * N + n] = 0.01 * Lam[n];')]),
    ("bwd_magnitude_mddbias_x100", [('if (mddbias) mddbias[d] = msb;', 'if (mddbias) mddbias[d] = 100.0 * msb;')]),
    ("bwd_magnitude_mddbias_x0.01", [('if (mddbias) mddbias[d] = msb;', 'if (mddbias) mddbias[d] = 0.01 * msb;')]),
    ("bwd_magnitude_conv_mdx_x100", [('if (mdx) mdx[p * L + s] = mg;', 'if (mdx) mdx[p * L + s] = 100.0 * mg;')]),
    ("bwd_magnitude_conv_mdx_x0.01", [('if (mdx) mdx[p * L + s] = mg;', 'if (mdx) mdx[p * L + s] = 0.01 * mg;')]),
    ("bwd_magnitude_conv_mdstate_x100", [('if (mdstate) mdstate[p * (K - 1) + (K - 1) + s] = mg;', 'if (mdstate) mdstate[p * (K - 1) + (K - 1) + s] = 100.0 * mg;')]),
    ("bwd_magnitude_conv_mdstate_x0.01", [('if (mdstate) mdstate[p * (K - 1) + (K - 1) + s] = mg;', 'if (mdstate) mdstate[p * (K - 1) + (K - 1) + s] = 0.01 * mg;')]),
    ("bwd_magnitude_conv_mdw_x100", [('if (mdw) mdw[d * K + k] = mg;', 'if (mdw) mdw[d * K + k] = 100.0 * mg;')]),
    ("bwd_magnitude_conv_mdw_x0.01", [('if (mdw) mdw[d * K + k] = mg;', 'if (mdw) mdw[d * K + k] = 0.01 * mg;')]),
    ("bwd_magnitude_conv_mdbias_x100", [('if (mdbias) mdbias[d] = mg;', 'if (mdbias) mdbias[d] = 100.0 * mg;')]),
    ("bwd_magnitude_conv_mdbias_x0.01", [('if (mdbias) mdbias[d] = mg;', 'if (mdbias) mdbias[d] = 0.01 * mg;')]),
]


def _mutate(text, subs):
    for old, new in subs:
        assert text.count(old) == 1, f"mutation anchor not unique/found: {old!r}"
        text = text.replace(old, new)
    return text


@pytest.mark.parametrize("name,subs", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, subs):
    lib = O.build_from_text(_mutate(SRC, subs))
    o = O.Oracle(lib)
    for pin in pins.PINS:
        try:
            pin(o)
        except AssertionError:
            return  # rejected by this pin
    pytest.fail(f"mutant {name} passed every pin")
