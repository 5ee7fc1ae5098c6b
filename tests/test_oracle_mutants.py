"""Mutation check of the oracle's pins (CPU only, oracle infrastructure).

Each case plants one plausible mistake in a copy of ``oracle/oracle.c`` (a
dropped term, a wrong sign, index or operand, a reversed tie rule), builds the
copy with the oracle's own gcc flags and runs ``tests/test_oracle_pins.py``
against it in a fresh process: at least one pin must fail. A control run with
an unmodified copy must pass, which shows that the pins really run on the copy.
The oracle source itself is never modified.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")
FP8_PINS = os.path.join(ROOT, "tests", "test_oracle_fp8.py")

# (name, text of oracle.c, the mistaken text)
ATTEND_CALL = "attend(qq, keys, vals, t + 1, d, scale, s, o, &lse[row]);"
SUFFIX_SRC = "const int64_t src = (((r * W + b) * Ls_cap + j) * nkv + g) * d + e;"
MUTANTS = [
    # prefill / the attention definition
    ("score scale dropped", "s[u] = scale * acc;", "s[u] = acc;"),
    ("score reads V rows", "acc += q[e] * keys[u * d + e];", "acc += q[e] * vals[u * d + e];"),
    ("softmax sign flipped", "double p = exp(s[u] - m);", "double p = exp(m - s[u]);"),
    ("output not normalised", "for (int32_t e = 0; e < d; ++e) o[e] /= l;",
     "for (int32_t e = 0; e < d; ++e) o[e] /= 1.0;"),
    ("lse without its max", "*lse = m + log(l);", "*lse = log(l);"),
    ("lse in base 2", "*lse = m + log(l);", "*lse = m + log2(l);"),
    ("causal mask dropped", ATTEND_CALL, "attend(qq, keys, vals, len, d, scale, s, o, &lse[row]);"),
    ("diagonal excluded", ATTEND_CALL, "attend(qq, keys, vals, t > 0 ? t : 1, d, scale, s, o, &lse[row]);"),
    ("kv heads interleaved", "g = h / group;", "g = h % nkv;"),
    ("sequence start ignored", "keys[u * d + e] = widen(k[((start + u) * nkv + g) * d + e]);",
     "keys[u * d + e] = widen(k[(u * nkv + g) * d + e]);"),
    ("bf16 read as an integer", "    memcpy(&f, &u, sizeof f);\n    return (double)f;", "    return (double)bits;"),
    # shared-prefix decode
    ("suffix of beam 0", SUFFIX_SRC, "const int64_t src = (((r * W + 0) * Ls_cap + j) * nkv + g) * d + e;"),
    ("suffix stride Ls", SUFFIX_SRC, "const int64_t src = (((r * W + b) * Ls + j) * nkv + g) * d + e;"),
    ("decode heads interleaved",
     "vc[(Lp + j) * d + e] = widen(sv[src]);\n            }\n        for (int32_t hg = 0; hg < group; ++hg) {\n"
     "            const int64_t row = (r * W + b) * nq + g * group + hg;",
     "vc[(Lp + j) * d + e] = widen(sv[src]);\n            }\n        for (int32_t hg = 0; hg < group; ++hg) {\n"
     "            const int64_t row = (r * W + b) * nq + hg * nkv + g;"),
    ("packed decode heads interleaved",
     "vc[(lp + j) * d + e] = widen(sv[at]);\n            }\n        for (int32_t hg = 0; hg < group; ++hg) {\n"
     "            const int64_t row = (r * W + b) * nq + g * group + hg;",
     "vc[(lp + j) * d + e] = widen(sv[at]);\n            }\n        for (int32_t hg = 0; hg < group; ++hg) {\n"
     "            const int64_t row = (r * W + b) * nq + hg * nkv + g;"),
    ("prompt of request 0", "kc[u * d + e] = widen(pk[((r * Lp + u) * nkv + g) * d + e]);",
     "kc[u * d + e] = widen(pk[((0 * Lp + u) * nkv + g) * d + e]);"),
    # shared-prefix decode over packed prompts of their own lengths
    ("packed prompt start ignored", "kc[u * d + e] = widen(pk[((p0 + u) * nkv + g) * d + e]);",
     "kc[u * d + e] = widen(pk[((u) * nkv + g) * d + e]);"),
    ("packed suffix over the prompt", "kc[(lp + j) * d + e] = widen(sk[at]);", "kc[(j) * d + e] = widen(sk[at]);"),
    # last-token gather
    ("first token instead of last", "const int64_t last = (int64_t)cu[i + 1] - 1;",
     "const int64_t last = (int64_t)cu[i];"),
    ("empty sequence not zeroed", "memset(dst + (int64_t)i * row_bytes, 0, (size_t)row_bytes);",
     "memset(dst + (int64_t)i * row_bytes, 1, (size_t)row_bytes);"),
    # selective FP8 requantisation
    ("E4M3 ties away from zero", "double q = rint(ldexp(a, 3 - e));", "double q = floor(ldexp(a, 3 - e) + 0.5);"),
    ("E4M3 exponent bias 8", "return sign | (uint8_t)(((e + 7) << 3) | ((int)q - 8));",
     "return sign | (uint8_t)(((e + 8) << 3) | ((int)q - 8));"),
    ("SiLU without the gate factor", "h[j] = g / (1.0 + exp(-g)) * u;", "h[j] = 1.0 / (1.0 + exp(-g)) * u;"),
    ("scale from the E5M2 maximum", "const double sc = (amax > 1e-12 ? amax : 1e-12) / 448.0;",
     "const double sc = (amax > 1e-12 ? amax : 1e-12) / 57344.0;"),
    # suffix reorder
    ("reorder scatters", "dst_k[((r * W + b) * Ls_cap + j) * row + e] = src_k[((r * W + p) * Ls_cap + j) * row + e];",
     "dst_k[((r * W + p) * Ls_cap + j) * row + e] = src_k[((r * W + b) * Ls_cap + j) * row + e];"),
    ("reorder V from K", "dst_v[((r * W + b) * Ls_cap + j) * row + e] = src_v[",
     "dst_v[((r * W + b) * Ls_cap + j) * row + e] = src_k["),
    ("tokens not gathered", "dst_tok[(r * W + b) * tok_cap + t] = src_tok[(r * W + p) * tok_cap + t];",
     "dst_tok[(r * W + b) * tok_cap + t] = src_tok[(r * W + b) * tok_cap + t];"),
    # beam top-K
    ("logit ties to the higher id", "return (p->id > q->id) - (p->id < q->id);",
     "return (p->id < q->id) - (p->id > q->id);"),
    ("score ties to the higher index", "return (p->f > q->f) - (p->f < q->f);",
     "return (p->f < q->f) - (p->f > q->f);"),
    ("candidates flattened beam-minor", "const int32_t parent = c[i].f / k_local, j = c[i].f % k_local;",
     "const int32_t parent = c[i].f % W_in, j = c[i].f / W_in;"),
    ("lse over half the vocabulary", "for (int32_t v = 0; v < V; ++v) l += exp(widen(x[v]) - m);",
     "for (int32_t v = 0; v < V / 2; ++v) l += exp(widen(x[v]) - m);"),
    ("cumulative score dropped", "volatile float s = c + lp;", "volatile float s = lp;"),
    ("log-probability from the fp64 lse", "volatile float lp = e[j].x - lse32;",
     "volatile float lp = (float)((double)e[j].x - lse64);"),
]


def run_pins(tmp_path, source_text):
    src = tmp_path / "oracle.c"
    src.write_text(source_text)
    so = oracle.build(src=str(src), out=str(tmp_path / "liboracle_copy.so"))
    env = dict(os.environ, BGA_ORACLE_LIB=so)
    return subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", "-m", "not gpu",
                           PINS, FP8_PINS], cwd=ROOT, env=env, capture_output=True, text=True, timeout=900)


def test_pins_pass_on_an_unmodified_copy(tmp_path):
    r = run_pins(tmp_path, open(oracle._SRC).read())
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(oracle._SRC).read()
    assert text.count(old) == 1, f"mutation site of '{name}' not unique"
    r = run_pins(tmp_path, text.replace(old, new))
    # exit status 1: some pin failed (not a crash, a collection error or an interrupt)
    assert r.returncode == 1, f"'{name}' survived the pins:\n" + r.stdout[-3000:] + r.stderr[-2000:]


LOOP_SRC = os.path.join(ROOT, "oracle", "beam_loop.py")
LOOP_PINS = os.path.join(ROOT, "tests", "test_oracle_beam_loop.py")
LOOP_MUTANTS = [
    ("stop-token candidates also continue", "        elif len(parents) < W:", "        if len(parents) < W:"),
    ("finished history of beam 0", "finished.append(Finished(float(sc), list(histories[par]) + [tok]))",
     "finished.append(Finished(float(sc), list(histories[0]) + [tok]))"),
    ("K/V copied from the slot, not the parent", "new_k.append([full_k[r][p].copy() for p in par])",
     "new_k.append([full_k[r][min(b, len(full_k[r]) - 1)].copy() for b in range(len(par))])"),
    ("final ranking ascending", "entries.sort(key=lambda e: (-e[0], e[1]))", "entries.sort(key=lambda e: (e[0], e[1]))"),
    ("current token's K not appended", "full_k[r][b] = np.concatenate([full_k[r][b], kn[r, b][None]])",
     "full_k[r][b] = full_k[r][b]"),
]


def test_loop_pins_pass_on_an_unmodified_copy(tmp_path):
    src = tmp_path / "beam_loop.py"
    src.write_text(open(LOOP_SRC).read())
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", LOOP_PINS], cwd=ROOT,
                       env=dict(os.environ, BGA_ORACLE_BEAM_LOOP=str(src)), capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-2000:]


@pytest.mark.parametrize("name,old,new", LOOP_MUTANTS, ids=[m[0] for m in LOOP_MUTANTS])
def test_loop_pins_catch_planted_mistake(tmp_path, name, old, new):
    text = open(LOOP_SRC).read()
    assert text.count(old) == 1, f"mutation site of '{name}' not unique"
    src = tmp_path / "beam_loop.py"
    src.write_text(text.replace(old, new))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", LOOP_PINS], cwd=ROOT,
                       env=dict(os.environ, BGA_ORACLE_BEAM_LOOP=str(src)), capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 1, f"'{name}' survived the pins:\n" + r.stdout[-3000:] + r.stderr[-2000:]
