"""The oracle's pins catch plausible mistakes (CPU only).

Each mutant below is a copy of paged_attention_ref.c with one planted slip of
the kind a hand-written attention reference can plausibly contain: a wrong
page or slot index, the wrong KV head for a query head, K and V swapped, the
softmax scale dropped, a base-2 log-sum-exp, a wrong merge weight, a wrong
split boundary, a wrong FP8 exponent bias, a wrong cache layout, a causal
mask off by one or aligned to the wrong end, a window or sink slip; in the KV
append a RoPE sign, pairing or cos/sin swap, a wrong scale, rounding ties or
slot; in the decode metadata a prefix sum, gather stride, page divide,
extension, request row or window page slip; in the contiguous layout a
stride slip.  The copy is compiled with the oracle's own build command and
the pin suite (test_oracle_pins.py) is run against it in a child process
through PKD_ORACLE_LIB; every mutant must make at least one pin fail.  A control copy
with no change must pass, which shows that the child really loads the copy.

The mistakes are planted in the oracle only, on the CPU; nothing here touches
the GPU library.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

from oracle import build as oracle_build

REPO = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(REPO, "tests", "test_oracle_pins.py")

# (name, text in paged_attention_ref.c, replacement).  Each text occurs exactly once.
MUTANTS = [
    ("block_table_ignored",
     "int32_t page = P->block_table[(int64_t)b * P->max_pages + t / P->page_size];",
     "int32_t page = t / P->page_size;"),
    ("block_table_row_of_sequence_zero",
     "int32_t page = P->block_table[(int64_t)b * P->max_pages + t / P->page_size];",
     "int32_t page = P->block_table[t / P->page_size];"),
    ("slot_off_by_one",
     "int slot = t % P->page_size;", "int slot = (t + 1) % P->page_size;"),
    ("head_major_page_layout",
     "(((int64_t)page * P->page_size + slot) * P->hkv + g) * P->head_dim + d",
     "(((int64_t)page * P->hkv + g) * P->page_size + slot) * P->head_dim + d"),
    ("gqa_interleaved_head_map",
     "const int g = h / G;", "const int g = h % P->hkv;"),
    ("query_rows_transposed",
     "P->q + (((int64_t)b * P->q_len + qi) * P->hq + h) * D;",
     "P->q + (((int64_t)h * P->q_len + qi) * P->batch + b) * D;"),
    ("query_token_major_over_batch",
     "P->q + (((int64_t)b * P->q_len + qi) * P->hq + h) * D;",
     "P->q + (((int64_t)qi * P->batch + b) * P->hq + h) * D;"),
    ("output_rows_head_major",
     "const int64_t row = ((int64_t)b * P->q_len + qi) * P->hq + h;",
     "const int64_t row = ((int64_t)b * P->hq + h) * P->q_len + qi;"),
    ("causal_limit_off_by_one",
     "const int v = L - P->q_len + qi + 1;", "const int v = L - P->q_len + qi;"),
    ("causal_mask_top_left_aligned",
     "const int v = L - P->q_len + qi + 1;", "const int v = qi + 1;"),
    ("causal_flag_ignored",
     "if (!P->causal) return L;", "if (P->causal < 2) return L;"),
    ("scale_dropped",
     "s[t - t0] = P->scale * acc;", "s[t - t0] = acc;"),
    ("values_read_from_keys",
     "o[d] += w * kv_elem(P, 1, b, t, g, d);", "o[d] += w * kv_elem(P, 0, b, t, g, d);"),
    ("softmax_exponent_sign",
     "double w = exp(s[t - t0] - m);", "double w = exp(m - s[t - t0]);"),
    ("output_not_normalised",
     "for (int d = 0; d < D; ++d) o[d] /= z;", "for (int d = 0; d < D; ++d) o[d] /= 1.0;"),
    ("lse_base_two",
     "return m + log(z);", "return m + log2(z);"),
    ("lse_missing_max",
     "return m + log(z);", "return log(z);"),
    ("empty_range_lse_zero",
     "if (t1 <= t0) return -INFINITY;", "if (t1 <= t0) return 0.0;"),
    ("merge_weight_against_max",
     "double w = exp(lse_part[j] - lse);", "double w = exp(lse_part[j] - M);"),
    ("merge_lse_missing_max",
     "double lse = M + log(z);", "double lse = log(z);"),
    ("split_chunk_rounds_down",
     "int c = (V - lo + S - 1) / S;", "int c = (V - lo) / S > 0 ? (V - lo) / S : 1;"),
    ("fp8_subnormal_exponent",
     "mag = ldexp((double)m / 8.0, 1 - 7);", "mag = ldexp((double)m / 8.0, -7);"),
    ("fp8_exponent_bias_eight",
     "mag = ldexp(1.0 + (double)m / 8.0, e - 7);", "mag = ldexp(1.0 + (double)m / 8.0, e - 8);"),
    ("fp8_scales_swapped",
     "is_v ? P->v_scale : P->k_scale;", "is_v ? P->k_scale : P->v_scale;"),
    ("fp8_scale_of_head_zero",
     "* (double)sc[g];", "* (double)sc[0];"),
    ("bf16_bits_shifted",
     "((uint32_t)bits) << 16;", "((uint32_t)bits) << 15;"),
    ("page_bound_off_by_one",
     "if (p < 0 || p >= P->num_pages)", "if (p < 0 || p > P->num_pages)"),
    ("window_off_by_one",
     "int lo = p - P->window + 1;", "int lo = p - P->window;"),
    ("window_from_last_position",
     "const int p = P->seq_lens[b] - P->q_len + qi;  /* the query token's position */",
     "const int p = P->seq_lens[b] - 1;  /* the query token's position */"),
    ("sink_of_head_zero",
     "const double sk = (double)P->sinks[h];", "const double sk = (double)P->sinks[0];"),
    ("sink_only_in_lse",
     "const double f = exp(lse - l2);", "const double f = 1.0;"),
    ("append_rope_sign",
     "y[d] = fmaf(x0, c, -t0);", "y[d] = fmaf(x0, c, t0);"),
    ("append_rope_adjacent_pairs",
     "const float x0 = bf16_float(k_new[src + d]), x1 = bf16_float(k_new[src + d + D / 2]);",
     "const float x0 = bf16_float(k_new[src + d]), x1 = bf16_float(k_new[src + (d ^ 1)]);"),
    ("append_cos_sin_swapped",
     "const float c = cs[d], s = cs[D / 2 + d];", "const float c = cs[D / 2 + d], s = cs[d];"),
    ("append_scale_of_head_zero",
     "store_row(kv_fp8, k_cache, dst, y, D, kv_fp8 ? k_scale[h] : 1.0f);",
     "store_row(kv_fp8, k_cache, dst, y, D, kv_fp8 ? k_scale[0] : 1.0f);"),
    ("fp8_ties_to_odd",
     "(err == best_err && (c & 1) == 0 && (best & 1) == 1)", "(err == best_err && (c & 1) == 1 && (best & 1) == 0)"),
    ("bf16_round_truncates",
     "u += 0x7FFFu + ((u >> 16) & 1u);", "u += 0u;"),
    ("append_writes_token_row_not_slot",
     "const int64_t dst = (slot * hkv + h) * (int64_t)D;", "const int64_t dst = ((n % capacity) * hkv + h) * (int64_t)D;"),
    ("metadata_prefix_sum_inclusive",
     "cu_seqlens_k[b + 1] = (int32_t)run;", "cu_seqlens_k[b] = (int32_t)run; cu_seqlens_k[b + 1] = (int32_t)run;"),
    ("metadata_gather_stride_one",
     "req_to_token[r * req_stride + (int64_t)j * page_size]", "req_to_token[r * req_stride + (int64_t)j]"),
    ("metadata_no_page_divide",
     "return slot >= 0 ? slot / page_size : -1;", "return slot >= 0 ? slot : -1;"),
    ("metadata_extend_ignored",
     "const int64_t L = seq_lens[b] + extend;", "const int64_t L = seq_lens[b];"),
    ("metadata_pool_index_ignored",
     "const int64_t r = req_pool_indices[b];", "const int64_t r = b;"),
    ("metadata_swa_first_page_off_by_one",
     "int64_t lo = len - q_len - window + 1;", "int64_t lo = len - q_len - window;"),
    ("contiguous_token_and_head_strides_swapped",
     "(int64_t)t * P->kv_strides[1] + (int64_t)g * P->kv_strides[2]",
     "(int64_t)t * P->kv_strides[2] + (int64_t)g * P->kv_strides[1]"),
    ("contiguous_batch_stride_dropped",
     "idx = (int64_t)b * P->kv_strides[0] + (int64_t)t", "idx = (int64_t)t"),
    ("contiguous_q_strides_ignored",
     "const uint16_t* qrow = P->q_strides ?", "const uint16_t* qrow = 0 ?"),
    ("metadata_swa_length_not_shifted",
     "swa_seqlens[b] = (int32_t)(len - f * page_size);", "swa_seqlens[b] = (int32_t)len;"),
]


def _run_pins(lib_path):
    env = dict(os.environ, PKD_ORACLE_LIB=lib_path, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", PINS, "-x", "-q", "-p", "no:cacheprovider"],
                       cwd=REPO, env=env, capture_output=True, text=True, timeout=600)
    return r.returncode, r.stdout[-3000:] + r.stderr[-2000:]


def _compile(src_text, directory, name):
    src = os.path.join(directory, name + ".c")
    lib = os.path.join(directory, "lib" + name + ".so")
    with open(src, "w") as f:
        f.write(src_text)
    oracle_build.build(src=src, lib=lib)
    return lib


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    """Compile the control and every mutant, then run the pin suite against each
    in parallel child processes.  Returns {name: (returncode, output tail)}."""
    d = str(tmp_path_factory.mktemp("oracle_mutants"))
    with open(oracle_build.SRC) as f:
        original = f.read()
    libs = {"control": _compile(original, d, "control")}
    for name, old, new in MUTANTS:
        assert original.count(old) == 1, f"{name}: the text to mutate must occur once"
        libs[name] = _compile(original.replace(old, new), d, name)
    workers = min(6, os.cpu_count() or 1)
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        futs = {name: ex.submit(_run_pins, lib) for name, lib in libs.items()}
        return {name: f.result() for name, f in futs.items()}


def test_unmutated_copy_passes_the_pins(outcomes):
    rc, tail = outcomes["control"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", [m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(outcomes, name):
    rc, tail = outcomes[name]
    # exit status 1: the suite ran and some test failed (not a crash or a usage error)
    assert rc == 1, f"mutant {name} survived the pins (exit {rc}):\n{tail}"
