"""Plant a plausible mistake in a copy of the oracle's C source, on the CPU,
and check that at least one pin catches it.  This is evidence that the pins
constrain every step of the oracle, not only that the oracle passes them."""
import os

import pytest

import oracle
from test_oracle_pins import PINS

# (name, exact text in the oracle source, replacement)
MUTATIONS = [
    ("router_transposed_w", "bf16_to_double(w[(size_t)e * H + h]);",
     "bf16_to_double(w[(size_t)h * E + e]);"),
    ("router_dropped_term", "for (int h = 0; h < H; ++h)\n        s += bf16_to_double(x[",
     "for (int h = 1; h < H; ++h)\n        s += bf16_to_double(x["),
    ("tie_to_higher_id", "if (best < 0 || l[e] > l[best]) best = e;",
     "if (best < 0 || l[e] >= l[best]) best = e;"),
    ("softmax_sign", "z += exp((double)l[idx[(size_t)t * k + j]] - m);",
     "z += exp(m - (double)l[idx[(size_t)t * k + j]]);"),
    ("no_padding_roundup", "int padded = ((counts[e] + ROW_BLOCK - 1) / ROW_BLOCK) * ROW_BLOCK;",
     "int padded = (counts[e] / ROW_BLOCK) * ROW_BLOCK + ROW_BLOCK;"),
    ("unstable_rows", "for (long p = 0; p < R; ++p) {\n    int e = idx[p];",
     "for (long p = R - 1; p >= 0; --p) {\n    int e = idx[p];"),
    ("gather_wrong_token", "memcpy(x_perm + (size_t)r * H, x + (size_t)(p / k) * H,",
     "memcpy(x_perm + (size_t)r * H, x + (size_t)(p % k) * H,"),
    ("transposed_b", "size_t off = layout == 0 ? (size_t)kk * N + n : (size_t)n * K + kk;",
     "size_t off = layout == 0 ? (size_t)n * K + kk : (size_t)n * K + kk;"),
    ("dropped_k_term", "      for (int kk = 0; kk < K; ++kk)\n        acc +=",
     "      for (int kk = 1; kk < K; ++kk)\n        acc +="),
    ("silu_sign", "return z / (1.0 + exp(-z));", "return z / (1.0 + exp(z));"),
    ("gate_up_swapped", "acc = silu(acc) * up;", "acc = silu(up) * acc;"),
    ("combine_wrong_pair", "long p = (long)t * k + j;\n      const uint16_t *yr",
     "long p = (long)j * T + t;\n      const uint16_t *yr"),
    ("down_transposed", "y[n] += a * bf16_to_double(wd[(size_t)c * H + n]);",
     "y[n] += a * bf16_to_double(wd[(size_t)n * I + c]);"),
    ("combine_weight_dropped", "for (int n = 0; n < H; ++n) o[n] += wj * y[n];",
     "for (int n = 0; n < H; ++n) o[n] += y[n];"),
    ("fp16_exponent", "v = ldexp((double)(fr | 0x400), ex - 25);",
     "v = ldexp((double)(fr | 0x400), ex - 24);"),
    ("bf16_shift", "uint32_t u = ((uint32_t)b) << 16;", "uint32_t u = ((uint32_t)b) << 15;"),
    ("block_expert_off_by_one", "block_expert[r / ROW_BLOCK] = e;",
     "block_expert[r / ROW_BLOCK + 1 < nblk ? r / ROW_BLOCK + 1 : r / ROW_BLOCK] = e;"),
    ("scatter_wrong_token", "double *o = out + (size_t)(p / k) * N;",
     "double *o = out + (size_t)(p % T) * N;"),
    ("scatter_weight_dropped", "for (int n = 0; n < N; ++n) o[n] += wp * yr[n];",
     "for (int n = 0; n < N; ++n) o[n] += yr[n];"),
]


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_pins_catch_planted_mistake(name, old, new, tmp_path):
    src = oracle.source_text()
    assert src.count(old) == 1, "mutation target not unique: %s" % name
    variant = oracle.compile_variant(src.replace(old, new), str(tmp_path / ("v_%s.so" % name)))
    caught = []
    for pin in PINS:
        try:
            pin(variant)
        except Exception as e:  # an assertion or a crash-free error both count
            caught.append((pin.__name__, type(e).__name__))
    assert caught, "no pin caught the planted mistake %s" % name
