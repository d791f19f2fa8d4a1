"""Planted mistakes in the oracle must fail its pins.

The pins (tests/test_oracle_*.py) check the oracle against routes independent of it:
torch SDPA in fp64, closed forms, brute force, the fp8 format. This test shows that
they are sharp enough. Each mutant below is msa_oracle.c with one plausible mistake
written in: a wrong causal alignment or bound, a wrong GQA head map, a dropped scale or
max, set semantics broken, a wrong pool layout, a page out of range read instead of
dropped, a wrong CSR query id or slot order, a varlen offset from the wrong origin, the
temperature applied to the sum only, a wrong fp8 exponent bias or subnormal quantum,
ties rounded away from zero, the fp8 decode's row sum taken over rounded probabilities,
or its probabilities left unrounded. Every mutant is compiled on the CPU and the pin
files run against it (through MSA_ORACLE_LIB) in a subprocess; each must make a pin
fail. The unmutated source, compiled the same way, must pass them all (the control),
so a failure is the mutation's doing.
"""
import concurrent.futures
import os
import subprocess
import sys

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ORACLE = os.path.join(ROOT, "oracle")
PINS = [os.path.join(HERE, f) for f in (
    "test_oracle_pins.py", "test_oracle_csr.py", "test_oracle_varlen.py",
    "test_oracle_temperature.py", "test_oracle_fp8.py", "test_oracle_decode_fp8.py")]

# name -> (text in msa_oracle.c, replacement, occurrences replaced)
MUTANTS = {
    "causal_top_left": ("(int64_t)qpos + kvlen - Sq : INT64_MAX",
                        "(int64_t)qpos : INT64_MAX", 2),
    "causal_limit_exclusive": ("j > limit) continue;", "j >= limit) continue;", 2),
    "gqa_head_modulo": (
        "      const uint16_t* qh = qrow + (int64_t)h * D;\n"
        "      double* oh = o_row + (int64_t)h * D;",
        "      const int hx = (h % qpk) * Hkv + hkv;\n"
        "      const uint16_t* qh = qrow + (int64_t)hx * D;\n"
        "      double* oh = o_row + (int64_t)hx * D;", 1),
    "scale_dropped": (
        "          score[n++] = scale * dot;\n          if (scale * dot > m) m = scale * dot;",
        "          score[n++] = dot;\n          if (dot > m) m = dot;", 1),
    "lse_without_max": ("lse_row[h] = m + log(l);", "lse_row[h] = log(l);", 1),
    "unused_slot_as_block0": ("if (sel[t] >= 0 && sel[t] < nblk) mark[sel[t]] = 1;",
                              "if (sel[t] < nblk) mark[sel[t] < 0 ? 0 : sel[t]] = 1;", 1),
    "seqused_ignored": ("if (seqused_k && seqused_k[b] < kvlen) kvlen = seqused_k[b];",
                        "(void)seqused_k;", 1),
    "pool_layout_token_major": (
        "return ((page * s->Hkv + hkv) * s->page_size + j % s->page_size) * s->D;",
        "return ((page * s->page_size + j % s->page_size) * s->Hkv + hkv) * s->D;", 1),
    "page_out_of_pool_read": ("if (page < 0 || page >= s->num_pages) return -1;",
                              "if (page < 0 || page >= s->num_pages) page = 0;", 1),
    "csr_local_query_id": ("q_idx[hkv * cap + pos] = (int32_t)((int64_t)b * Sq + qpos);",
                           "q_idx[hkv * cap + pos] = (int32_t)qpos;", 1),
    "csr_slots_descending": (
        "        for (int t = 0; t < topk; ++t) {\n"
        "          if (sel[t] < 0 || sel[t] >= nblk) continue;",
        "        for (int t = topk - 1; t >= 0; --t) {\n"
        "          if (sel[t] < 0 || sel[t] >= nblk) continue;", 1),
    "varlen_keys_from_origin": (
        "const int64_t koff = (int64_t)cu_seqlens_k[b] * Hkv * D * (kv_fp8 ? 1 : 2);",
        "const int64_t koff = 0;", 1),
    "varlen_global_query_position": ("(int)(g - cu_seqlens_q[b]), Sq_b", "(int)g, Sq_b", 1),
    "temperature_on_sum_only": ("lset_row[h] = m / temp + log(lt);",
                                "lset_row[h] = m + log(lt);", 1),
    "fp8_exponent_bias": ("ldexp((double)(8 + m), e - 10)", "ldexp((double)(8 + m), e - 11)", 1),
    "fp8_subnormal_quantum": ("ldexp((double)m, -9)", "ldexp((double)m, -10)", 1),
    "e4m3_ties_away": ("r = ldexp(rint(ldexp(a, 4 - e)), e - 4);",
                       "r = ldexp(round(ldexp(a, 4 - e)), e - 4);", 1),
    "fp8_decode_rounded_row_sum": (
        "            l += p;\n            const double pq = fp8_round(p);",
        "            const double pq = fp8_round(p);\n            l += pq;", 1),
    "fp8_decode_unrounded_p": ("const double pq = fp8_round(p);", "const double pq = p;", 1),
    "fp8_decode_head_modulo": ("const int hkv = h / qpk;", "const int hkv = h % Hkv;", 1),
}


def _run_pins(name, text, tmp):
    """Compile `text` as the oracle and run the pins on it: (exit code, last lines)."""
    src = os.path.join(tmp, f"{name}.c")
    lib = os.path.join(tmp, f"lib_{name}.so")
    with open(src, "w") as fh:
        fh.write(text)
    subprocess.check_call(["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11",
                           "-fno-fast-math", "-I", ORACLE, "-o", lib, src, "-lm"])
    env = dict(os.environ, MSA_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        "-m", "not gpu", *PINS], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=600)
    return r.returncode, "\n".join(r.stdout.strip().splitlines()[-3:])


@pytest.fixture(scope="module")
def outcomes(tmp_path_factory):
    tmp = str(tmp_path_factory.mktemp("mutants"))
    with open(os.path.join(ORACLE, "msa_oracle.c")) as fh:
        base = fh.read()
    texts = {"control": base}
    for name, (old, new, count) in MUTANTS.items():
        assert base.count(old) == count, f"{name}: the oracle source changed; update the mutant"
        texts[name] = base.replace(old, new)
    with concurrent.futures.ThreadPoolExecutor(max_workers=4) as ex:
        futs = {n: ex.submit(_run_pins, n, t, tmp) for n, t in texts.items()}
        return {n: f.result() for n, f in futs.items()}


def test_control_passes(outcomes):
    rc, tail = outcomes["control"]
    assert rc == 0, tail


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_caught(outcomes, name):
    rc, tail = outcomes[name]
    # 1: some pin failed (not a collection or usage error, which would be 2 or more)
    assert rc == 1, f"{name} survived the pins (exit {rc}):\n{tail}"
