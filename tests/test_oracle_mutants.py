"""Plant plausible mistakes in a copy of the oracle and check that the pins see them.

Each mutant is a one-place textual edit of oracle/oracle.c (a dropped term, a
wrong sign, index or offset, a transposed operand, a lost subnormal...). It is
compiled into a temporary library on the CPU and the pins run against it in a
child process (some mutants index out of bounds, so a crash of the child also
counts as the mutant being caught); at least one pin must fail on it.
"""
import json
import os
import subprocess
import sys

import pytest

import oracle as O

SRC = os.path.join(os.path.dirname(O.__file__), "oracle.c")

MUTANTS = {
    "q4_interleaved_nibbles": ("(i < 16) ? (qs[i] & 0x0f) : (qs[i - 16] >> 4)",
                               "(qs[i / 2] >> (4 * (i % 2))) & 0x0f"),
    "q4_offset_sign": ("(double)(nib - 8)", "(double)(nib + 8)"),
    "q4_no_offset": ("(double)(nib - 8)", "(double)(nib)"),
    "subnormal_flushed": ("v = ldexp((double)m, -24);", "v = 0.0;"),
    "exponent_bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "hidden_bit_dropped": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(m), e - 25)"),
    "q8_unsigned": ("(int)(int8_t)blk[2 + i]", "(int)blk[2 + i]"),
    "last_weight_dropped": ("for (int64_t k = 0; k < K; ++k) {", "for (int64_t k = 0; k + 1 < K; ++k) {"),
    "q8_row_transposed": ("w + (n * (K / 32) + k / 32) * 34", "w + ((k / 32) * 1 + n * 0) * 34"),
    "q4_block_stride": ("w + (n * (K / 32) + k / 32) * 18", "w + (n * (K / 32) + k / 32) * 16"),
    "f16_transposed": ("w + (n * K + k) * 2", "w + (k * K + n) * 2"),
    "abs_dropped": ("asum += fabs(p);", "asum += p;"),
    "silu_sign": ("g / (1.0 + exp(-g))", "g / (1.0 + exp(g))"),
    "gateup_swapped": ("out[n] = oracle_silu(gg[n]) * uu[n]", "out[n] = oracle_silu(uu[n]) * gg[n]"),
    "x_index_shifted": ("double p = wk * (double)x[k];", "double p = wk * (double)x[(k + 1) % K];"),
    "sign_bit_ignored": ("return sign ? -v : v;", "return v;"),
    "scale_byte_order": ("(uint16_t)(p[0] | (p[1] << 8))", "(uint16_t)(p[1] | (p[0] << 8))"),
    "bias_dropped": ("out[n] += (double)bias[n];", "out[n] += 0.0;"),
    "residual_subtracted": ("out[n] += (double)residual[n];", "out[n] -= (double)residual[n];"),
    "residual_for_bias": ("out[n] += (double)bias[n];", "out[n] += (double)residual[n];"),
    "rms_eps_dropped": ("sqrt(ss / (double)K + eps)", "sqrt(ss / (double)K)"),
    "rms_sum_not_mean": ("sqrt(ss / (double)K + eps)", "sqrt(ss + eps)"),
    "rms_sqrt_dropped": ("double rms = sqrt(ss / (double)K + eps);", "double rms = ss / (double)K + eps;"),
    "rms_gamma_shifted": ("out[k] = (double)gamma[k] * (double)x[k] / rms;",
                          "out[k] = (double)gamma[(k + 1) % K] * (double)x[k] / rms;"),
    "rms_gamma_dropped": ("out[k] = (double)gamma[k] * (double)x[k] / rms;", "out[k] = (double)x[k] / rms;"),
    "rms_product_unnormalised": ("double p = wk * xn[k];", "double p = wk * (double)x[k];"),
    "q4k_scale_from_min_byte": ("*sc = u[j] & 63;", "*sc = u[j + 4] & 63;"),
    "q4k_upper_scale_bits_wrong_byte": ("*sc = (u[j + 4] & 15) | ((u[j - 4] >> 6) << 4);",
                                        "*sc = (u[j + 4] & 15) | ((u[j] >> 6) << 4);"),
    "q4k_upper_min_bits_wrong_byte": ("*mn = (u[j + 4] >> 4) | ((u[j] >> 6) << 4);",
                                      "*mn = (u[j + 4] >> 4) | ((u[j - 4] >> 6) << 4);"),
    "q4k_min_added": ("return d * (double)sc * (double)q - dmin * (double)mn;",
                      "return d * (double)sc * (double)q + dmin * (double)mn;"),
    "q4k_nibbles_interleaved": ("int q = (l < 32) ? (qs[32 * g + l] & 15) : (qs[32 * g + l - 32] >> 4);",
                                "int q = (qs[32 * g + l / 2] >> (4 * (l % 2))) & 15;"),
    "q4k_dmin_read_as_d": ("double dmin = oracle_half_to_double(read_le16(blk + 2));",
                           "double dmin = oracle_half_to_double(read_le16(blk));"),
    "q4k_superblock_stride": ("w + (n * (K / 256) + k / 256) * 144", "w + (n * (K / 256) + k / 256) * 128"),
    "q6k_nibble_halves_swapped": ("lo = (g < 2) ? (lo & 15) : (lo >> 4);", "lo = (g < 2) ? (lo >> 4) : (lo & 15);"),
    "q6k_ql_group_offset": ("ql[64 * h + 32 * (g % 2) + l]", "ql[64 * h + 32 * (g / 2) + l]"),
    "q6k_ql_half_stride": ("ql[64 * h + 32 * (g % 2) + l]", "ql[32 * h + 32 * (g % 2) + l]"),
    "q6k_qh_half_stride": ("qh[32 * h + l]", "qh[16 * h + l]"),
    "q6k_qh_bit_order": ("(qh[32 * h + l] >> (2 * g)) & 3", "(qh[32 * h + l] >> (6 - 2 * g)) & 3"),
    "q6k_fields_swapped": ("int q = lo | (hi << 4);", "int q = (lo << 2) | hi;"),
    "q6k_scale_per_32": ("(double)sc[i / 16]", "(double)sc[i / 32]"),
    "q6k_scale_unsigned": ("(double)sc[i / 16]", "(double)(uint8_t)sc[i / 16]"),
    "q6k_offset_31": ("(double)(q - 32)", "(double)(q - 31)"),
    "q6k_no_offset": ("(double)(q - 32)", "(double)(q)"),
    "q6k_d_first": ("read_le16(blk + 208)", "read_le16(blk)"),
    "q6k_superblock_stride": ("w + (n * (K / 256) + k / 256) * 210", "w + (n * (K / 256) + k / 256) * 208"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site for {name} no longer exists in oracle.c"
    mutated = src.replace(old, new, 1)
    c_path = tmp_path / "mutant.c"
    so_path = tmp_path / "libmutant.so"
    c_path.write_text(mutated)
    subprocess.check_call(["gcc", "-std=c11", "-O1", "-fPIC", "-shared", "-ffp-contract=off",
                           "-o", str(so_path), str(c_path), "-lm", "-lpthread"])
    here = os.path.dirname(os.path.abspath(__file__))
    proc = subprocess.run([sys.executable, os.path.join(here, "oracle_pins.py"), str(so_path)],
                          capture_output=True, text=True, timeout=300,
                          env={**os.environ, "PYTHONPATH": os.pathsep.join([os.path.dirname(here), here])})
    if proc.returncode != 0:
        return  # the mutant crashed the pins' process: caught
    caught = json.loads(proc.stdout.strip().splitlines()[-1])
    assert caught, f"mutant {name} passed every pin"
