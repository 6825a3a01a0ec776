"""The oracle's pins must reject plausible mistakes.

Each case below plants one mistake in a temporary copy of ``oracle/kda_oracle.c``
(on the CPU; nothing here touches the GPU path), builds it, routes the oracle
through it, and checks that at least one pin from ``test_oracle_pins`` fails.
"""
import os
import subprocess

import pytest

import test_oracle_pins as P

ORACLE_C = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "oracle", "kda_oracle.c")

DECAY = """        /* decay: row c of S scales by exp(g_t[c]) */
        for (int32_t c = 0; c < dk; ++c) {
            const double gc = gate_scalar ? g[(size_t)t * hv + h]
                                          : g[((size_t)t * hv + h) * dk + c];
            const double a = exp(gc);
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] *= a;
        }
"""
PRED = """        /* prediction S'^T k */"""
READOUT = """        /* read out after the write */"""

MUTANTS = {
    # decay applied after the rank-1 write instead of before the prediction
    "decay_after_write": [(DECAY, ""), (READOUT, DECAY + READOUT)],
    # residual without beta
    "no_beta": [("u[j] = bt * ((double)vt[j] - pred[j]);", "u[j] = ((double)vt[j] - pred[j]);")],
    # sign slip in the residual
    "residual_sign": [("u[j] = bt * ((double)vt[j] - pred[j]);", "u[j] = bt * ((double)vt[j] + pred[j]);")],
    # read-out from the state before the write (move the write after the read-out)
    "readout_before_write": [
        ("""        for (int32_t c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] += kc * u[j];
        }
""", ""),
        ("""        for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;
""", """        for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;
        for (int32_t c = 0; c < dk; ++c) {
            const double kc = (double)kt[c];
            double *row = S + (size_t)c * dv;
            for (int32_t j = 0; j < dv; ++j) row[j] += kc * u[j];
        }
""")],
    # the gate indexed by the value channel (decay along V instead of K)
    "decay_along_v": [("for (int32_t j = 0; j < dv; ++j) row[j] *= a;",
                       "for (int32_t j = 0; j < dv; ++j) row[j] *= exp(gate_scalar ? gc : "
                       "g[((size_t)t * hv + h) * dk + (j % dk)]);")],
    # final state written in math orientation instead of [V, K]
    "state_transposed": [("ht_unit[(size_t)j * dk + c] = S[(size_t)c * dv + j];",
                          "ht_unit[(size_t)c * dv + j] = S[(size_t)c * dv + j];")],
    # initial state read in the wrong orientation
    "h0_transposed": [("(double)h0_unit[(size_t)j * dk + c]", "(double)h0_unit[(size_t)c * dv + j]")],
    # key head chosen as h % hk instead of h / (hv / hk)
    "gqa_modulo": [("h / group,", "h % hk,")],
    # scale never applied
    "no_scale": [("for (int32_t j = 0; j < dv; ++j) ot[j] *= scale;", "")],
    # exp(-g): growth instead of decay
    "gate_sign": [("const double a = exp(gc);", "const double a = exp(-gc);")],
    # the prediction uses q instead of k
    "pred_uses_q": [("const double kc = (double)kt[c];\n            const double *row = S + (size_t)c * dv;\n"
                     "            for (int32_t j = 0; j < dv; ++j) pred[j] += row[j] * kc;",
                     "const double kc = (double)qt[c];\n            const double *row = S + (size_t)c * dv;\n"
                     "            for (int32_t j = 0; j < dv; ++j) pred[j] += row[j] * kc;")],
}

PINS = [
    lambda O: P.test_golden_handworked(O),
    lambda O: P.test_single_token_zero_state_closed_form(O),
    lambda O: P.test_beta_zero_is_pure_per_channel_decay(O),
    lambda O: P.test_zero_gate_zero_beta_is_identity(O),
    lambda O: P.test_delta_write_invariant(O, "moderate"),
    lambda O: P.test_orthonormal_keys_decouple_channels(O),
    lambda O: P.test_transition_matrix_brute_force(O, 32, [17, 3, 9], 1, 2, 8, 8, False),
    lambda O: P.test_transition_matrix_brute_force(O, 33, [12], 2, 4, 6, 5, True),
    lambda O: P.test_chunked_equals_recurrent(O, 16, "moderate"),
    lambda O: P.test_gqa_head_map(O),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(oracle, tmp_path, name):
    src = open(ORACLE_C).read()
    for old, new in MUTANTS[name]:
        assert old in src, (name, old[:60])
        src = src.replace(old, new, 1)
    c_path = tmp_path / ("kda_oracle_%s.c" % name)
    so_path = tmp_path / ("libkda_oracle_%s.so" % name)
    c_path.write_text(src)
    subprocess.run(["gcc", "-O1", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-o", str(so_path),
                    str(c_path), "-lm"], check=True)
    caught = []
    with oracle.use_library(str(so_path)):
        for i, pin in enumerate(PINS):
            try:
                pin(oracle)
            except AssertionError:
                caught.append(i)
    assert caught, "mutant %s passed every pin" % name
