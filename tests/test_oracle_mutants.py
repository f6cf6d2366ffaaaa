"""The pins are sensitive: a copy of the oracle with one plausible mistake planted in its C source
(compiled here, on the CPU) must fail at least one pin.  Mistakes cover a dropped term, a sign, an
index/transposition, the rounding rule, dispatch stability and range checks, the gathered row,
the expert weight choice, the destination term of the reduction, and the gate, token and
accumulation of the combine, and the
scale, max shift, key index and merge of the attention."""
import os

import pytest

import _pins
import oracle

# (name, text in pk_oracle.c, replacement, pins expected to catch it)
MUTANTS = [
    ("drop_last_k", "for (int64_t k = 0; k < g->K; ++k) {", "for (int64_t k = 0; k < g->K - 1; ++k) {",
     _pins.GEMM_PINS),
    ("flip_sign", "r[j] += a * b[j];", "r[j] -= a * b[j];", _pins.GEMM_PINS),
    ("transpose_b", "r[j] += a * b[j];",
     "r[j] += a * g->Bd[(j % g->K) * g->N + (k % g->N)];", _pins.GEMM_PINS),
    ("ties_away", "double n = nearbyint(a / quantum);", "double n = round(a / quantum);",
     _pins.BF16_PINS),
    ("truncate", "double n = nearbyint(a / quantum);", "double n = trunc(a / quantum);",
     _pins.BF16_PINS),
    ("unstable_scatter",
     "    for (int64_t f = 0; f < slots; ++f) {\n        int32_t id = topk_ids[f];\n        if (id < 0 || id >= num_experts) continue;\n        if (id >= expert_begin && id < expert_begin + num_local)\n            perm[",
     "    for (int64_t f = slots - 1; f >= 0; --f) {\n        int32_t id = topk_ids[f];\n        if (id < 0 || id >= num_experts) continue;\n        if (id >= expert_begin && id < expert_begin + num_local)\n            perm[",
     _pins.DISPATCH_PINS),
    ("no_id_range_check", "if (id < 0 || id >= num_experts) continue;", "if (id < 0) continue;",
     _pins.DISPATCH_PINS),
    ("wrong_token", "int64_t token = perm[r0 + j] / top_k;", "int64_t token = perm[r0 + j] % top_k;",
     _pins.GROUPED_PINS),
    ("wrong_expert_weight", "W + (int64_t)e * K * N", "W + (int64_t)(num_local - 1 - e) * K * N",
     _pins.GROUPED_PINS),
    ("drop_destination", "R[i * ldr + j] = D0 ? (double)D0[i * ldd + j] : 0.0;",
     "R[i * ldr + j] = 0.0;", _pins.REDUCE_PINS),
    ("drop_last_producer", "for (int p = 0; p < num_producers; ++p) {",
     "for (int p = 0; p < num_producers - 1; ++p) {", _pins.REDUCE_PINS),
    ("combine_drop_gate", "for (int64_t c = 0; c < N; ++c) o[c] += g * z[c];",
     "for (int64_t c = 0; c < N; ++c) o[c] += z[c];", _pins.COMBINE_PINS),
    ("combine_wrong_token", "double* o = out + t * ldo;", "double* o = out + (f % T) * ldo;",
     _pins.COMBINE_PINS),
    ("combine_gate_of_row", "const double g = (double)gates[f];",
     "const double g = (double)gates[sel[i]];", _pins.COMBINE_PINS),
    ("combine_overwrite", "for (int64_t c = 0; c < N; ++c) o[c] += g * z[c];",
     "for (int64_t c = 0; c < N; ++c) o[c] = g * z[c];", _pins.COMBINE_PINS),
    ("attn_no_rescale", "for (int64_t d = 0; d < D; ++d) o[d] = a * o[d] + b * oc[d];",
     "for (int64_t d = 0; d < D; ++d) o[d] = o[d] + b * oc[d];", _pins.ATTENTION_PINS),
    ("attn_drop_scale", "s[j] = scale * acc;", "s[j] = acc;", _pins.ATTENTION_PINS),
    ("attn_no_max_shift", "for (int64_t j = 0; j < Sk; ++j) sum += exp(s[j] - m);\n        const double lse_c = m + log(sum);",
     "for (int64_t j = 0; j < Sk; ++j) sum += exp(s[j]);\n        const double lse_c = log(sum);",
     _pins.ATTENTION_PINS),
    ("attn_transposed_k", "pk_oracle_bf16_to_f64(K[j * ldk + d])", "pk_oracle_bf16_to_f64(K[(d % Sk) * ldk + (j % D)])",
     _pins.ATTENTION_PINS),
    ("attn_merge_weight", "const double a = exp(lse[i] - merged), b = exp(lse_c - merged);",
     "const double a = exp(lse[i] - merged), b = exp(lse_c - lse[i]);", _pins.ATTENTION_PINS),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(tmp_path, name, old, new, pins):
    src = open(oracle.SOURCE).read()
    count = src.count(old)
    assert count >= 1, "mutation anchor not found for %s" % name
    mutated = src.replace(old, new, 1) if name != "unstable_scatter" else src.replace(old, new)
    path = tmp_path / ("mut_%s.c" % name)
    path.write_text(mutated)
    lib = oracle.compile_library(str(path), str(tmp_path / ("mut_%s.so" % name)))
    mutant = oracle.Oracle(lib)
    caught = []
    for pin in pins:
        try:
            pin(mutant)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "mutant %s passed every pin" % name
