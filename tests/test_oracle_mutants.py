"""Planted mistakes in a copy of the oracle's C source must fail a pin.

Each case edits one plausible slip into a temporary copy of
oracle/hqmq_oracle.c (a dropped term, a flipped sign, a transposed operand, an
off-by-one, a wrong comparison), builds it with gcc, routes the oracle
wrappers to that build and runs the pin that should catch it.  The real
oracle is untouched.  CPU only.
"""
import os
import subprocess
import tempfile

import numpy as np
import pytest

import oracle as O
from tests import test_oracle_algebra as A
from tests import test_oracle_attend as T
from tests import test_oracle_compact_norm as CN
from tests import test_oracle_exact as EX
from tests import test_oracle_f16_codebook as F
from tests import test_oracle_med3_codec as M
from tests import test_oracle_quantizer as Q

SRC = os.path.join(os.path.dirname(O.__file__), "hqmq_oracle.c")

MUTANTS = [
    # (name, original text, planted text, pin that must fail)
    ("product-order-swapped",
     "or_qmul(a, b, out);\n}", "or_qmul(b, a, out);\n}",
     lambda: Q.test_nearest_matches_kdtree(8)),
    ("hamilton-sign",
     "a[0] * b[1] + a[1] * b[0] + a[2] * b[3] - a[3] * b[2]",
     "a[0] * b[1] + a[1] * b[0] - a[2] * b[3] + a[3] * b[2]",
     A.test_qmul_matches_matrix_representation),
    ("t2-unit-sign",
     "(p % 2 == 0) ? 1.0 : -1.0", "(p % 2 == 0) ? -1.0 : 1.0",
     Q.test_deep_hole_six_way_tie_takes_smallest_code),
    ("t2-half-sign-bit",
     "((bits >> m) & 1) ? -0.5 : 0.5", "((bits >> (3 - m)) & 1) ? -0.5 : 0.5",
     A.test_t2_canonical_order),
    ("norm-dropped-term",
     "    s2 = fmaf(v[3], v[3], s2);\n", "",
     Q.test_norm2_is_the_declared_fp32_chain),
    ("norm-code-no-half",
     "float h = r * 0.5f;", "float h = r;",
     Q.test_half_norm_code_matches_numpy),
    ("argmax-ties-to-largest",
     "if (sc > best) {", "if (sc >= best) {",
     Q.test_deep_hole_six_way_tie_takes_smallest_code),
    ("median-upper",
     "float m = tmp[(n - 1) / 2];", "float m = tmp[n / 2];",
     lambda: M.test_lower_median_matches_partition(4)),
    ("threshold-ge",
     "if (s2[i] > thr) {", "if (s2[i] >= thr) {",
     M.test_strict_greater_boundary),
    ("threshold-C-not-squared",
     "float cc = C * C;", "float cc = C;",
     M.test_designed_batch_exact_outliers),
    ("f16-truncates",
     "double r = nearbyint(ldexp(a, 10 - E));", "double r = floor(ldexp(a, 10 - E));",
     F.test_f16_bits_against_numpy),
    ("philox-constant",
     "M0 = 0xD2E7470EE14C6C93ull", "M0 = 0xD2E7470EE14C6C95ull",
     lambda: F.test_philox_matches_numpy((5, 77), 1)),
    ("codebook-no-rejection",
     "if (!(n2 <= 1.0))", "if (!(n2 <= 4.0))",
     F.test_codebook_is_uniform_on_s3),
    ("pack-bit-order",
     "long bit = (long)c * b + i;\n                words", "long bit = (long)c * b + (b - 1 - i);\n                words",
     lambda: M.test_pack_row_bit_layout(8, 128)),
    ("decode-norm-factor",
     "double r = 2.0 * or_f16_value(hnorm[i]);", "double r = or_f16_value(hnorm[i]);",
     M.test_decode_closed_form_and_round_trip),
    ("attend-no-scale",
     "s[t] = scale * acc;", "s[t] = acc;",
     lambda: T.test_attend_matches_scipy_softmax(7, 64, 4, 0.125)),
    ("attend-skips-first-token",
     "for (int64_t t = 0; t < T; ++t)\n            for (int d = 0; d < D; ++d)\n                og[d] += s[t] * v[t * D + d];",
     "for (int64_t t = 1; t < T; ++t)\n            for (int d = 0; d < D; ++d)\n                og[d] += s[t] * v[t * D + d];",
     T.test_one_token_gives_its_value),
    ("attend-normalises-by-count",
     "og[d] /= z;", "og[d] /= (double)T;",
     T.test_dominant_key_gives_its_value),
    ("attend-values-from-keys",
     "og[d] += s[t] * v[t * D + d];", "og[d] += s[t] * k[t * D + d];",
     T.test_uniform_scores_give_the_mean_of_v),
    ("compact-norm-truncates",
     "    if (t - f < 0.5)\n        return clo;", "    if (t - f < 1.0)\n        return clo;",
     lambda: CN.test_rounds_to_the_nearest_value_ties_to_even(10)),
    ("compact-norm-ties-odd",
     "return (clo & 1u) ? chi : clo;", "return (clo & 1u) ? clo : chi;",
     lambda: CN.test_rounds_to_the_nearest_value_ties_to_even(8)),
    ("compact-norm-no-cap",
     "    const double hi = (f + 1.0) * q < vmax ? (f + 1.0) * q : vmax;", "    const double hi = (f + 1.0) * q;",
     lambda: CN.test_monotone_bounded_and_flagged(8)),
    ("exact-digit-weight",
     "                    weight *= 3u;", "                    weight *= 4u;",
     lambda: EX.test_pack_exact_round_trips_through_an_independent_unpacker(8, 32, 9)),
    ("exact-digit-field-order",
     "const long base = (long)OR_FIELD_BITS * (2 * fh * r + pl * fh + f);",
     "const long base = (long)OR_FIELD_BITS * (2 * fh * r + (1 - pl) * fh + f);",
     lambda: EX.test_pack_exact_round_trips_through_an_independent_unpacker(32, 32, 4)),
    ("exact-planes-interleaved",
     "            uint32_t *plane = words + (pl * 4 + r) * wl;\n            for (int c = 0; c < cpt; ++c) {\n                const uint32_t low",
     "            uint32_t *plane = words + (r * 2 + pl) * wl;\n            for (int c = 0; c < cpt; ++c) {\n                const uint32_t low",
     lambda: EX.test_pack_exact_round_trips_through_an_independent_unpacker(8, 32, 9)),
    ("exact-grid-rounds-down",
     "return (uint32_t)((2u * (uint64_t)n * 32768u + R) / (2u * R));",
     "return (uint32_t)((2u * (uint64_t)n * 32768u) / (2u * R));",
     lambda: EX.test_level_grid_divides_the_binades_evenly(8)),
    ("exact-norm-ties-odd",
     "if (d < bd || (d == bd && (n & 1u) == 0u)) {", "if (d < bd || (d == bd && (n & 1u) == 1u)) {",
     lambda: EX.test_exact_norm_is_the_nearest_level_for_every_binary16_input(8)),
    ("exact-norm-flag-level",
     "    if (h16 & 0x8000u)\n        return R - 1u;", "    if (h16 & 0x8000u)\n        return R - 2u;",
     lambda: EX.test_exact_norm_is_the_nearest_level_for_every_binary16_input(32)),
    ("side-pos-drops-offset",
     "side_pos[n_out] = (uint32_t)((t0 + t) * cpt + c);", "side_pos[n_out] = (uint32_t)(t * cpt + c);",
     M.test_batches_and_partial_tail),
]


@pytest.fixture(scope="module")
def src_text():
    return open(SRC).read()


@pytest.mark.parametrize("name,old,new,pin", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(src_text, name, old, new, pin):
    assert src_text.count(old) == 1, f"mutation site for {name} not unique"
    # the pin passes on the real oracle
    pin()
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "m.c")
        so = os.path.join(d, "m.so")
        open(c, "w").write(src_text.replace(old, new))
        subprocess.run(["gcc", "-O2", "-std=gnu11", "-ffp-contract=off", "-fopenmp",
                        "-shared", "-fPIC", c, "-o", so, "-lm"], check=True)
        with O.use_library(so):
            with pytest.raises((AssertionError, ValueError)):
                pin()
    np.testing.assert_array_equal(O.t2_elements()[0], [1, 0, 0, 0])
