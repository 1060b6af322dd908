"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
the pins catch every one of them.  Each mutant is compiled from a patched copy of
oracle/oracle.c into a temporary directory and checked in a child process, so a
mutant that crashes counts as caught without taking the test run down."""
import json
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(os.path.dirname(HERE), "oracle", "oracle.c")

# name -> list of (original text, replacement); every original must occur in oracle.c
MUTANTS = {
    "drop_scale": [("const double sj = p->scale * dot;", "const double sj = dot;")],
    "query_block_uses_block_k": [("const int64_t qi = s / p->block_q;",
                                  "const int64_t qi = s / p->block_k;")],
    "no_max_subtraction": [("sbuf[t] = exp(sbuf[t] - m);", "sbuf[t] = exp(sbuf[t]);"),
                           ("*lse_out = m + log(l);", "*lse_out = log(l);")],
    "lse_drops_max": [("*lse_out = m + log(l);", "*lse_out = log(l);")],
    "key_block_short_by_one": [("for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {\n"
                                "            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;\n"
                                "            const int64_t kbase",
                                "for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k - 1; ++j) {\n"
                                "            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;\n"
                                "            const int64_t kbase"),
                               ("for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k; ++j) {\n"
                                "            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;\n"
                                "            const int64_t vbase",
                                "for (int64_t j = kj * p->block_k; j < (kj + 1) * p->block_k - 1; ++j) {\n"
                                "            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;\n"
                                "            const int64_t vbase")],
    "v_row_is_query_row": [("const int64_t vbase = (bh * p->S + j) * D;",
                            "const int64_t vbase = (bh * p->S + s) * D;")],
    "empty_row_lse_zero": [("*lse_out = -INFINITY;\n        return;", "*lse_out = 0.0;\n        return;")],
    "dot_uses_k_twice": [("dot += widen(p->q, p->dtype, qbase + d) * widen(p->k, p->dtype, kbase + d);",
                          "dot += widen(p->k, p->dtype, qbase + d) * widen(p->k, p->dtype, kbase + d);")],
    "no_normalisation": [("out_row[d] = acc[d] / l;", "out_row[d] = acc[d];")],
    "k_ignores_head": [("const int64_t kbase = (bh * p->S + j) * D;\n            double dot = 0.0;\n"
                        "            for (int64_t d = 0; d < D; ++d)\n                dot += widen(p->q",
                        "const int64_t kbase = (j) * D;\n            double dot = 0.0;\n"
                        "            for (int64_t d = 0; d < D; ++d)\n                dot += widen(p->q")],
    # the block mask read transposed (mask[kj][qi] instead of mask[qi][kj])
    "mask_transposed": [("const uint8_t* mrow = p->mask + (bh * p->n_q + qi) * p->n_k;",
                         "uint8_t mrow_t[4096];\n"
                         "    for (int64_t c = 0; c < p->n_k && c < 4096; ++c)\n"
                         "        mrow_t[c] = (c < p->n_q && qi < p->n_k) ? p->mask[(bh * p->n_q + c) * p->n_k + qi] : 0;\n"
                         "    const uint8_t* mrow = mrow_t;")],
    "bf16_wrong_shift": [("((uint32_t)((const uint16_t*)base)[idx]) << 16;",
                          "((uint32_t)((const uint16_t*)base)[idx]) << 15;")],
    "elem_partial_ignores_bits": [("if (!p->pidx || blk == 1) return 1;", "return 1;")],
    "elem_bit_order_reversed": [("return (int)((w >> (c % 32)) & 1u);", "return (int)((w >> (31 - c % 32)) & 1u);")],
    "elem_tile_row_from_key": [("const int64_t i = s % p->block_q, c = j % p->block_k;",
                                "const int64_t i = j % p->block_q, c = j % p->block_k;")],
    "elem_tile_index_ignored": [("(int64_t)p->pidx[bi] * p->block_q", "(int64_t)0 * p->block_q")],
    # backward with element masks: dk/dv or dq summed over every key of an active block
    "bwd_dkdv_ignores_element_bits": [("            if (!kept(p, p->mask[bi], bi, r, j)) continue;\n", "")],
    "bwd_dq_ignores_element_bits": [("            if (!kept(p, mrow[kj], brow + kj, s, j)) continue;\n"
                                     "            const int64_t kbase = (bh * p->S + j) * D;\n"
                                     "            const double ds",
                                     "            const int64_t kbase = (bh * p->S + j) * D;\n"
                                     "            const double ds")],
    "elem_partial_as_empty": [("if (!p->pidx || blk == 1) return 1;", "if (!p->pidx || blk == 1) return 1;\n    if (blk > 1) return 0;")],
    "ragged_group_start_late": [("const int64_t end = start + rows;",
                                 "const int64_t end = start + rows;\n        const int64_t start1 = start + (rows > 0);"),
                                ("for (int64_t i = start; i < end; ++i)\n            for (int64_t n = 0; n < N; ++n) {",
                                 "for (int64_t i = start1; i < end; ++i)\n            for (int64_t n = 0; n < N; ++n) {")],
    "ragged_next_expert": [("widen(rhs, dtype, (g * K + k) * N + n)",
                            "widen(rhs, dtype, (((g + 1) % G) * K + k) * N + n)")],
    "ragged_rhs_transposed": [("widen(rhs, dtype, (g * K + k) * N + n)",
                               "widen(rhs, dtype, (g * K + (n % K)) * N + (k % N))")],
    "ragged_tail_not_zeroed": [("for (int64_t i = start; i < M; ++i)\n        for (int64_t n = 0; n < N; ++n) out[i * N + n] = 0.0;",
                                "for (int64_t i = start; i < M; ++i)\n        for (int64_t n = 0; n < N; ++n) out[i * N + n] = 1.0;")],
    # group sizes outside [0, rows left]: a negative size taken by magnitude, the
    # last group clamped one row short
    "ragged_negative_size_abs": [("int64_t rows = group_sizes[g] < 0 ? 0 : (int64_t)group_sizes[g];",
                                  "int64_t rows = group_sizes[g] < 0 ? -(int64_t)group_sizes[g] : (int64_t)group_sizes[g];")],
    "ragged_clamp_short": [("if (rows > M - start) rows = M - start;", "if (rows > M - start) rows = M - start - 1;")],
    "bwd_no_delta": [("const double ds = sbuf[t] * (pbuf[t] - delta);", "const double ds = sbuf[t] * pbuf[t];"),
                     ("const double ds = P * (dp - delta[r]);", "const double ds = P * dp;")],
    "bwd_delta_unweighted": [("delta += sbuf[t] * dp;", "delta += dp;")],
    "bwd_dk_no_scale": [("for (int64_t d = 0; d < D; ++d) dk_row[d] *= p->scale;", "")],
    "bwd_dq_no_scale": [("for (int64_t d = 0; d < D; ++d) dq_row[d] *= p->scale;", "")],
    "bwd_dv_uses_ds": [("dv_row[d] += P * widen(dout, p->dtype, qbase + d);",
                        "dv_row[d] += ds * widen(dout, p->dtype, qbase + d);")],
    "bwd_dq_uses_v": [("dq_row[d] += ds * widen(p->k, p->dtype, kbase + d);",
                       "dq_row[d] += ds * widen(p->v, p->dtype, kbase + d);")],
    "bwd_dk_uses_dout": [("dk_row[d] += ds * widen(p->q, p->dtype, qbase + d);",
                          "dk_row[d] += ds * widen(dout, p->dtype, qbase + d);")],
    "bwd_lse_drops_max": [("const double lse = m + log(l);", "const double lse = log(l);")],
    "bwd_key_sees_next_block": [("const int64_t bi = (bh * p->n_q + qi) * p->n_k + kj;",
                                 "const int64_t bi = (bh * p->n_q + qi) * p->n_k + (kj + 1) % p->n_k;")],
    "bwd_dp_sign": [("dp += widen(dout, p->dtype, qbase + d) * widen(p->v, p->dtype, kbase + d);",
                     "dp -= widen(dout, p->dtype, qbase + d) * widen(p->v, p->dtype, kbase + d);")],
    "fp8_bias_8": [("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)")],
    "fp8_subnormal_as_normal": [("e == 0 ? ldexp((double)m / 8.0, -6)", "e == 0 ? ldexp(1.0 + (double)m / 8.0, -7)")],
    "fp8_sign_dropped": [("return sgn ? -mag : mag;", "return mag;")],
    "compact_skips_last_column": [("for (int64_t kj = 0; kj < n_k; ++kj)\n            if (mask[r * n_k + kj])",
                                   "for (int64_t kj = 0; kj < n_k - 1; ++kj)\n            if (mask[r * n_k + kj])")],
}


def _build(tmp_path, name, patches):
    src = open(SRC).read()
    for old, new in patches:
        assert old in src, "patch for %s no longer applies: %r" % (name, old[:60])
        src = src.replace(old, new)
    c = tmp_path / ("%s.c" % name)
    c.write_text(src)
    so = tmp_path / ("lib%s.so" % name)
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-o", str(so), str(c), "-lm"],
                   check=True)
    return so


def _run_checks(so):
    env = dict(os.environ, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, os.path.join(HERE, "oracle_checks.py"), str(so)],
                       capture_output=True, text=True, env=env, cwd=HERE, timeout=300)
    if r.returncode != 0:
        return ["<crashed rc=%d>" % r.returncode]
    return json.loads(r.stdout.strip().splitlines()[-1])


def test_unmutated_copy_passes(tmp_path):
    so = _build(tmp_path, "clean", [])
    assert _run_checks(so) == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    so = _build(tmp_path, name, MUTANTS[name])
    failed = _run_checks(so)
    assert failed, "mutant %s passed every pin" % name
