"""Plant plausible mistakes in a copy of the oracle (on the CPU) and require
every one of them to fail at least one pin.  This shows the pins constrain
each part of the oracle rather than restating it."""
import os
import shutil

import pytest

import oracle
from oracle import build as obuild
from oracle_pins import ALL_PINS

SRC = os.path.join(os.path.dirname(obuild.__file__), "oracle.c")

MUTANTS = {
    "gate_up_halves_swapped": (
        "double g = dot_row(W_gate_up, dt, base + n, d, xt);\n"
        "    double u = dot_row(W_gate_up, dt, base + f + n, d, xt);",
        "double g = dot_row(W_gate_up, dt, base + f + n, d, xt);\n"
        "    double u = dot_row(W_gate_up, dt, base + n, d, xt);"),
    "no_renormalisation": (
        "w[j] = (exp(logit[idx[j]] - m) / z) / sel;",
        "w[j] = (exp(logit[idx[j]] - m) / z);"),
    "ties_to_higher_index": (
        "return (a->e > b->e) - (a->e < b->e);",
        "return (a->e < b->e) - (a->e > b->e);"),
    "rank_ascending": (
        "if (a->logit > b->logit) return -1;\n  if (a->logit < b->logit) return 1;",
        "if (a->logit > b->logit) return 1;\n  if (a->logit < b->logit) return -1;"),
    "shared_expert_dropped": (
        "for (int64_t sg = 0; sg < S; ++sg) {\n          expert_hidden",
        "for (int64_t sg = 0; sg < 0; ++sg) {\n          expert_hidden"),
    "down_proj_transposed": (
        "out[i] = dot_row(W_down, dt, e * d + i, f, act);",
        "{ double s_ = 0.0; for (int64_t n_ = 0; n_ < f; ++n_) "
        "s_ += elem(W_down, dt, e * d * f + n_ * d + i) * act[n_]; out[i] = s_; }"),
    "silu_sign": (
        "double silu = g / (1.0 + exp(-g));",
        "double silu = g / (1.0 + exp(g));"),
    "bias_ignored": (
        "if (bias) logit[e] += (double)bias[e];",
        "(void)bias;"),
    "unstable_scatter": (
        "for (int64_t s = 0; s < n; ++s) {\n    int32_t e = idx[s];",
        "for (int64_t s = n - 1; s >= 0; --s) {\n    int32_t e = idx[s];"),
    # capacity: the dropped rows listed in reverse
    "capacity_dropped_rows_reversed": (
        "pos = drop_base[e] + (r - cap);",
        "pos = (dropped - 1) - (drop_base[e] + (r - cap));"),
    # capacity: dropped rows not skipped by the group offsets
    "capacity_groups_start_at_zero": (
        "offsets[0] = (int32_t)dropped;", "offsets[0] = 0;"),
    # layer with capacity: dropped copies still contribute
    "capacity_ignored_in_layer": (
        "if (keep && !keep[t * k + j]) continue;", "(void)keep;"),
    # balance: sum over tokens instead of the mean
    "balance_sum_not_mean": (
        "importance[e] = s / (double)T;", "importance[e] = s;"),
    # balance: no batch-mean division of the KL sum
    "balance_no_batchmean": (
        "*loss = kl / (double)E;", "*loss = kl;"),
    # balance: the 1e-8 guard left out of the log
    "balance_no_guard": (
        "kl += u * (log(u) - log(importance[e] + 1e-8));",
        "kl += u * (log(u) - log(importance[e]));"),
    # balance: softmax without the bias
    "balance_bias_ignored": (
        "if (bias) pt[e] += (double)bias[e];", "(void)bias;"),
    # MXFP4: the odd element taken from the low nibble
    "mxfp4_nibbles_swapped": (
        "unsigned code = (i % 2 == 0) ? (byte & 15u) : (byte >> 4);",
        "unsigned code = (i % 2 == 0) ? (byte >> 4) : (byte & 15u);"),
    # MXFP4: the subnormal code read as m * 1 instead of m * 1/2
    "mxfp4_subnormal_wrong": (
        "double mag = e == 0 ? 0.5 * (double)m :", "double mag = e == 0 ? 1.0 * (double)m :"),
    # MXFP4: E8M0 bias off by one
    "mxfp4_scale_bias": (
        "ldexp(1.0, (int)x - 127);", "ldexp(1.0, (int)x - 126);"),
    # MXFP4: one scale per 16 elements instead of 32
    "mxfp4_block_16": (
        "uint8_t x = scales[r * (K / 32) + i / 32];", "uint8_t x = scales[r * (K / 32) + (i / 16) % (K / 32)];"),
    # backward: silu' without its g (1 - s) term
    "bwd_silu_prime": (
        "dg[n] = da[n] * u[n] * (sg * (1.0 + g[n] * (1.0 - sg)));",
        "dg[n] = da[n] * u[n] * sg;"),
    # backward: gate and up gradients fed to the wrong weight rows
    "bwd_gate_up_rows_swapped": [
        ("acc += elem(W_gate_up, dt, (base + n) * d + c) * dg[n];",
         "acc += elem(W_gate_up, dt, (base + n) * d + c) * du[n];"),
        ("acc += elem(W_gate_up, dt, (base + f + n) * d + c) * du[n];",
         "acc += elem(W_gate_up, dt, (base + f + n) * d + c) * dg[n];")],
    # backward: softmax Jacobian without the subtracted mean
    "bwd_router_jacobian": (
        "double dl = w[j] * (dwt[j] - sw);", "double dl = w[j] * dwt[j];"),
    # backward: expert output gradient not scaled by the routing weight
    "bwd_unweighted_dO": (
        "for (int64_t i = 0; i < d; ++i) dO[i] = wj * elem(dy, dt, t * d + i);",
        "for (int64_t i = 0; i < d; ++i) dO[i] = elem(dy, dt, t * d + i);"),
    # backward: down-weight gradient against the wrong activation column
    "bwd_dWd_misindexed": (
        "gd[i * f + n] += dO[i] * a[n];", "gd[i * f + n] += dO[i] * a[(n + 1) % f];"),
    # backward with a capacity: dropped copies still sent through their expert
    "bwd_capacity_ignored": (
        "if (routed && keep && !keep[t * k + j]) {", "if (routed && keep && 0) {"),
    # balance: KL with its arguments swapped
    "balance_kl_reversed": (
        "kl += u * (log(u) - log(importance[e] + 1e-8));",
        "kl += importance[e] * (log(importance[e] + 1e-8) - log(u));"),
    "bf16_shift_wrong": (
        "uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 16;",
        "uint32_t bits = (uint32_t)((const uint16_t*)p)[i] << 15;"),
    "combine_first_weight_only": (
        "acc += w[t * k + j] * elem(O, dt, row * d + i);",
        "acc += w[t * k] * elem(O, dt, row * d + i);"),
    "router_uses_wrong_row": (
        "logit[e] = dot_row(W_router, dt, e, d, xt);",
        "logit[e] = dot_row(W_router, dt, E - 1 - e, d, xt);"),
    "gate_up_expert_stride_wrong": (
        "int64_t base = e * 2 * f;",
        "int64_t base = e * f;"),
    "shared_rows_misplaced": (
        "int64_t row = T * k + sg * T + t;",
        "int64_t row = T * k + sg * T + (T - 1 - t);"),
    # with a forced selection, the weights renormalised over the natural
    # top-k instead of over the forced experts
    "forced_renormalised_over_natural_topk": [
        ("  if (forced) {\n    for (int64_t j = 0; j < k; ++j) idx[j] = forced[j];",
         "  for (int64_t e = 0; e < E; ++e) {\n"
         "    order[e].logit = logit[e];\n    order[e].e = (int32_t)e;\n  }\n"
         "  qsort(order, (size_t)E, sizeof(ranked), by_logit_then_index);\n"
         "  if (forced) {\n    for (int64_t j = 0; j < k; ++j) idx[j] = forced[j];"),
        ("sel += exp(logit[idx[j]] - m) / z;", "sel += exp(logit[order[j].e] - m) / z;"),
    ],
}


def _edits(name):
    spec = MUTANTS[name]
    return spec if isinstance(spec, list) else [spec]


def _apply(src, name):
    for old, new in _edits(name):
        assert src.count(old) == 1, f"mutation {name} no longer matches oracle.c"
        src = src.replace(old, new)
    return src


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_mutations_apply_to_current_source():
    src = open(SRC).read()
    for name in MUTANTS:
        _apply(src, name)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    src = _apply(open(SRC).read(), name)
    d = mutant_dir / name
    d.mkdir()
    shutil.copy(os.path.join(os.path.dirname(SRC), "oracle.h"), d / "oracle.h")
    (d / "oracle.c").write_text(src)
    lib = obuild.build(src=str(d / "oracle.c"), lib=str(d / "liboracle.so"))
    orc = oracle.Oracle(lib)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {name}"
