"""The oracle's pins catch plausible mistakes.

Each case plants one mistake in a copy of the oracle's source (on the CPU),
compiles it, points the oracle wrapper at the mutant and runs the pins of
tests/test_oracle_pins.py in process: at least one pin must fail.  The
unmutated copy, compiled the same way, must pass all of them (so a failure
is the planted mistake's doing, not the harness's).
"""
import contextlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

import oracle
from oracle import build_oracle

import test_oracle_pins as P
from synth import workloads

SRC = os.path.join(os.path.dirname(oracle.__file__), "zero_oracle.cpp")

# (name, exact text in the oracle source, replacement, needs the exhaustive cast pin)
MUTATIONS = [
    ("first moment drops its history", "float m1 = k.B1 * m[i] + k.C1 * g;",
     "float m1 = k.C1 * g;", False),
    ("second moment uses g instead of g*g", "float v1 = k.B2 * v[i] + k.C2 * (g * g);",
     "float v1 = k.B2 * v[i] + k.C2 * g;", False),
    ("eps inside the square root", "float d = std::sqrt(v1) * k.rho + k.E;",
     "float d = std::sqrt(v1 * k.rho * k.rho + k.E);", False),
    ("update added instead of subtracted", "float th1 = k.a_wd * master[i] - k.s * (m1 / d);",
     "float th1 = k.a_wd * master[i] + k.s * (m1 / d);", False),
    ("weight decay applied after the update",
     "float th1 = k.a_wd * master[i] - k.s * (m1 / d);",
     "float th1 = k.a_wd * (master[i] - k.s * (m1 / d));", False),
    ("weight decay dropped", "k.a_wd = (float)(1.0 - lr * wd);", "k.a_wd = 1.0f;", False),
    ("no first-moment bias correction", "k.s = (float)(lr / bc1);", "k.s = (float)lr;", False),
    ("no second-moment bias correction", "k.rho = (float)(1.0 / std::sqrt(bc2));",
     "k.rho = 1.0f;", False),
    ("step index off by one", "double bc1 = 1.0 - std::pow(b1, (double)t);",
     "double bc1 = 1.0 - std::pow(b1, (double)(t + 1));", False),
    ("C2 from beta1", "k.C2 = (float)(1.0 - b2);", "k.C2 = (float)(1.0 - b1);", False),
    ("average divides by N_d + 1", "float g = a / nd;", "float g = a / (nd + 1.0f);", False),
    ("reduction in reverse rank order",
     "for (int32_t q = 1; q < n_d; ++q) a = a + contribution(G[q], i);",
     "for (int32_t q = n_d - 1; q >= 1; --q) a = a + contribution(G[q], i);", False),
    ("reduction starts from +0", "float a = contribution(G[0], i);",
     "float a = 0.0f + contribution(G[0], i);", False),
    ("bf16 ties toward zero", "if (dlo < dhi) return (uint16_t)(lo_bits >> 16);",
     "if (dlo <= dhi) return (uint16_t)(lo_bits >> 16);", True),
    ("bf16 truncation", "if (dhi < dlo) return (uint16_t)(hi_bits >> 16);",
     "if (false) return (uint16_t)(hi_bits >> 16);", True),
    ("rank owns the next slice",
     "shard_out[p.shard_off[b] + j] = flat[p.padded_off[b] + (int64_t)rank * sb + j];",
     "shard_out[p.shard_off[b] + j] = flat[p.padded_off[b] + (int64_t)((rank + 1) % n_d) * sb + j];",
     False),
    ("always at least one pad element",
     "add_bucket(p, pos, l, ((l + n_d - 1) / n_d) * n_d, n_d);",
     "add_bucket(p, pos, l, (l / n_d + 1) * n_d, n_d);", False),
    ("bucket capacity off by one", "int64_t c = (sp.cap <= 0) ? p.total : sp.cap;",
     "int64_t c = (sp.cap <= 0) ? p.total : sp.cap + 1;", False),
    ("FSDP2 chunk rows rounded wrongly", "const int64_t c = (r + n_d - 1) / n_d;",
     "const int64_t c = r / n_d + 1;", False),
    ("accumulate ignores overwrite", "float a = overwrite ? contrib : (acc[i] + contrib);",
     "float a = acc[i] + contrib;", False),
    ("accumulate drops the 1/n scale", "float contrib = scale * widen_bf16(g[i]);",
     "float contrib = widen_bf16(g[i]);", False),
    ("pack shifts elements by one",
     "flat_out[p.padded_off[b] + (x - p.stream_off[b])] = tensors[t][e];",
     "flat_out[p.padded_off[b] + (x - p.stream_off[b])] = tensors[t][e > 0 ? e - 1 : e];", False),
    ("gather takes the next rank's shard",
     "out[p.padded_off[b] + (int64_t)q * sb + j] = shards[q][p.shard_off[b] + j];",
     "out[p.padded_off[b] + (int64_t)q * sb + j] = shards[(q + 1) % n_d][p.shard_off[b] + j];",
     False),
    ("reshard leaves non-zero padding", "std::memset(d, 0, elem_bytes);",
     "std::memset(d, 1, elem_bytes);", False),
    ("ZeRO-1 state counted unsharded",
     "double state = (double)k_bytes * (double)((mode >= 1) ? S : P);",
     "double state = (double)k_bytes * (double)((mode >= 2) ? S : P);", False),
    ("ZeRO-3 counts one parameter All-Gather", "const int passes = mode >= 3 ? 3 : 2;",
     "const int passes = mode >= 3 ? 2 : 2;", False),
    ("ring pass without the (N_d - 1) / N_d factor",
     "const double pass = 2.0 * (double)P * (double)(n_d - 1) / (double)n_d;",
     "const double pass = 2.0 * (double)P;", False),
]


def pin_calls(with_exhaustive: bool):
    """The pins of test_oracle_pins.py with their parameters, cheap ones first."""
    calls = [
        (P.test_bf16_round_ties_and_overflow, {}),
        (P.test_reduce_rank_order_pin, {}),
        (P.test_reduce_negative_zero_start, {}),
        (P.test_adamw_zero_gradient_special_case, {}),
        (P.test_accumulate_four_quarter_micro_batches_equal_full_batch_mean, {}),
        (P.test_accumulate_skip_store_and_emit, {}),
        (P.test_layout_fsdp1_worked_example, {}),
        (P.test_fsdp2_worked_examples, {}),
        (P.test_reduce_exact_small_integers, {}),
        (P.test_reduce_post_divide_equals_pre_divide_pow2, {}),
        (P.test_f32_reduce_order_and_exact_sums, {}),
        (P.test_f32_contributions_equal_bf16_path_on_bf16_values, {}),
        (P.test_adamw_step1_closed_form, {}),
        (P.test_sharded_equals_unsharded, {}),
    ]
    calls += [(P.test_adamw_vs_torch_float64_within_rounding_bound, {"t": t})
              for t in (1, 2, 10, 101, 1001)]
    calls += [(P.test_adamw_ten_steps_vs_torch_normwise, {})]
    calls += [(P.test_layout_brute_force, {"seed": s}) for s in range(40)]
    calls += [(P.test_fsdp2_layout_brute_force, {"seed": s}) for s in range(25)]
    calls += [(P.test_fsdp2_slices_agree_with_torch_chunk, {"seed": s}) for s in range(20)]
    calls += [(P.test_gather_locate_reshard_brute_force, {"seed": s}) for s in range(25)]
    calls += [(P.test_layout_workload_sizes_closed_form, {"name": n}) for n in workloads.NAMES]
    calls += [(P.test_layout_padded_tail_workload, {})]
    calls += [(P.test_memory_formulas, {"name": n}) for n in workloads.NAMES]
    calls += [(P.test_comm_volume_ring_simulation, {"n_d": n}) for n in (1, 2, 3, 4, 5, 8)]
    calls += [(P.test_comm_volume_closed_forms, {"name": n}) for n in workloads.NAMES]
    if with_exhaustive:
        calls += [(P.test_bf16_round_exhaustive_vs_torch, {})]
    return calls


@contextlib.contextmanager
def oracle_library(path):
    saved = (oracle._LIB_PATH, oracle._lib)
    oracle._LIB_PATH, oracle._lib = path, None
    try:
        yield
    finally:
        oracle._LIB_PATH, oracle._lib = saved


def first_failing_pin(path, with_exhaustive):
    with oracle_library(path):
        for fn, kw in pin_calls(with_exhaustive):
            try:
                fn(**kw)
            except AssertionError:
                return f"{fn.__name__}{kw or ''}"
    return None


def compile_variant(src_text, out_path):
    c_path = out_path + ".cpp"
    with open(c_path, "w") as f:
        f.write(src_text)
    subprocess.run(["g++", *build_oracle.FLAGS, "-w", c_path, "-o", out_path], check=True)


@pytest.fixture(scope="module")
def variants(tmp_path_factory):
    """Compile the unmutated oracle and every mutant (in parallel)."""
    src = open(SRC).read()
    tmp = str(tmp_path_factory.mktemp("oracle_mut"))
    jobs = [("control", src, os.path.join(tmp, "control.so"))]
    for k, (name, old, new, _) in enumerate(MUTATIONS):
        assert src.count(old) == 1, f"mutation site not unique or missing: {name}"
        jobs.append((name, src.replace(old, new), os.path.join(tmp, f"m{k}.so")))
    with ThreadPoolExecutor(8) as ex:
        list(ex.map(lambda j: compile_variant(j[1], j[2]), jobs))
    return {name: path for name, _, path in jobs}


def test_unmutated_copy_passes_every_pin(variants):
    assert first_failing_pin(variants["control"], with_exhaustive=True) is None


@pytest.mark.parametrize("name,old,new,exhaustive", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_fails_a_pin(variants, name, old, new, exhaustive):
    caught = first_failing_pin(variants[name], with_exhaustive=exhaustive)
    assert caught is not None, f"no pin caught: {name}"
