"""Planted mistakes in the oracle must be caught by its pins.

Each case copies the oracle's C source, plants one plausible mistake with a
textual replacement, compiles the copy on the CPU, and runs every pin in
test_oracle_pins.py against it: at least one pin has to fail.  This shows the
pins constrain every step of the computation (score, scale, columns, causal
limit, index filter, block mapping, shard rule, lse, merge weights).
"""
import inspect
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

MUTATIONS = {
    "drop_scale": ("s[j] = P->scale * dot;", "s[j] = dot;"),
    "dot_over_v_columns_only": ("for (int k = 0; k < D; ++k) dot", "for (int k = 0; k < DV; ++k) dot"),
    "v_from_wrong_columns": ("out[c] += w * latent_value(P, vrow, c);", "out[c] += w * latent_value(P, vrow, c + 64);"),
    "kv8_factor_dropped": ("return (double)P->kv_scale[row] * (double)P->kv8[row * P->d_qk + c];",
                           "return (double)P->kv8[row * P->d_qk + c];"),
    "kv8_codes_unsigned": ("(double)P->kv8[row * P->d_qk + c]", "(double)(uint8_t)P->kv8[row * P->d_qk + c]"),
    "kv8_factor_of_neighbour_row": ("P->kv_scale[row]", "P->kv_scale[row ^ 1]"),
    "kv8_factor_on_keys_only": ("out[c] += w * latent_value(P, vrow, c);",
                                "out[c] += w * (P->kv8 ? (double)P->kv8[vrow * D + c] : latent_value(P, vrow, c));"),
    "causal_off_by_one": ("for (int64_t p = 0; p <= last; ++p)", "for (int64_t p = 0; p < last; ++p)"),
    "sparse_no_causal_filter": ("if (i >= 0 && i <= last && (", "if (i >= 0 && i < P->seq_lens[b] && ("),
    "sparse_shard_rule_by_token": ("(i / interleave) % num_shards == shard_id", "i % num_shards == shard_id"),
    "sparse_shard_filter_dropped": ("(num_shards == 1 || (i / interleave)", "(1 || (i / interleave)"),
    "identity_block_mapping": ("return (int64_t)blk * P->block_size + p % P->block_size;",
                               "return (int64_t)b * P->max_blocks * P->block_size + p;"),
    "shard_rule_by_token": ("(p / interleave) % num_shards == shard_id", "p % num_shards == shard_id"),
    "lse_without_max": ("*lse = m + log(l);", "*lse = log(l);"),
    "weights_without_max": ("double w = exp(s[j] - m) / l;", "double w = exp(s[j]) / l;"),
    "merge_weight_sign": ("double w = exp(li - M);", "double w = exp(M - li);"),
    "merge_unnormalised": ("for (int32_t c = 0; c < d_v; ++c) o[c] /= W;", ""),
}


def _pin_cases():
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = getattr(fn, "pytestmark", [])
        params = [m for m in marks if m.name == "parametrize"]
        if not params:
            yield name, fn, {}
            continue
        argnames, values = params[0].args
        argnames = [a.strip() for a in argnames.split(",")]
        for v in values:
            v = v if isinstance(v, tuple) else (v,)
            yield name, fn, dict(zip(argnames, v))


@pytest.mark.parametrize("mutation", sorted(MUTATIONS))
def test_planted_mistake_is_caught(mutation, tmp_path, monkeypatch):
    src = open(oracle._SRC).read()
    old, new = MUTATIONS[mutation]
    assert src.count(old) == 1, "mutation anchor must exist exactly once"
    mutated = tmp_path / "mutated.c"
    mutated.write_text(src.replace(old, new))
    so = tmp_path / "libmutated.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-o", str(so),
                    str(mutated), "-lm"], check=True)
    monkeypatch.setattr(oracle, "_lib", None)
    monkeypatch.setattr(oracle, "_LIB_PATH", str(so))
    monkeypatch.setattr(oracle, "_SRC", str(mutated))
    caught = []
    for name, fn, kwargs in _pin_cases():
        try:
            fn(**kwargs)
        except Exception:  # an assertion or an oracle error both count as caught
            caught.append(name)
    monkeypatch.setattr(oracle, "_lib", None)
    assert caught, "no pin detects mutation %s" % mutation
