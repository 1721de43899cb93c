"""Planted-mistake check of the oracle pins (CPU only; run by hand, not collected).

    python tests/oracle_mutations.py

Each mutation below is a plausible mistake (a sign, an index, an off-by-one, a
dropped term, a transposed operand).  It is applied to a temporary copy of
oracle/cp_oracle.c, built into a temporary library, and the pins in
tests/test_oracle_pins.py and tests/test_gdn_oracle_pins.py are run against it through
CP_ORACLE_LIB.  Every
mutation should make at least one pin fail.  The committed oracle is never
modified.
"""
import os
import subprocess
import sys
import tempfile

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "cp_oracle.c")

MUTATIONS = [
    ("RoPE lower half: sign of the sin term",
     "lo * (double)cosb[to + j] - hi * (double)sinb[to + j]",
     "lo * (double)cosb[to + j] + hi * (double)sinb[to + j]"),
    ("RoPE upper half: sign of the sin term",
     "hi * (double)cosb[to + j + h2] + lo * (double)sinb[to + j + h2]",
     "hi * (double)cosb[to + j + h2] - lo * (double)sinb[to + j + h2]"),
    ("GQA head map", "const int g = h / G;", "const int g = h % nKV;"),
    ("window edge", "if (window == 0 || qp - kp < window || kp < sink) return 1;",
     "if (window == 0 || qp - kp <= window || kp < sink) return 1;"),
    ("causal edge", "if (!key_is_real || kp > qp) return 0;",
     "if (!key_is_real || kp >= qp) return 0;"),
    ("pad keys attended", "if (!key_is_real || kp > qp) return 0;", "if (kp > qp) return 0;"),
    ("scale dropped", "s[c] = (double)scale * dot + add;", "s[c] = dot + add;"),
    ("normaliser dropped", "for (int d = 0; d < D; ++d) o[d] = acc[d] / l;",
     "for (int d = 0; d < D; ++d) o[d] = acc[d];"),
    ("ring slot offset", "return sink + (p - sink) % (cap - sink);",
     "return (p - sink) % (cap - sink);"),
    ("sink eviction", "while (k < n && pos_out[k] < sink) ++k;",
     "while (k < n && pos_out[k] < sink - 1) ++k;"),
    ("seen advance", "seen[b] = s0 + n;", "seen[b] = s0 + C;"),
    ("pad-key bound (equivalent on real rows)", "real = j < nv;", "real = j <= nv;"),
    ("chunk key position", "kp = (long)seen[b] + j;", "kp = (long)seen[b] + j + 1;"),
    ("query position", "const long qp = (long)seen[b] + i;\n        /* pass 1",
     "const long qp = (long)seen[b] + i + 1;\n        /* pass 1"),
    ("window guard", "if (cap <= C + sink) return ORC_EWINDOW;",
     "if (cap < C + sink) return ORC_EWINDOW;"),
    ("selected row", "x[(((size_t)b * H + h) * C + (size_t)r) * D + d] : 0.0;",
     "x[(((size_t)b * H + h) * C + (size_t)r - 1) * D + d] : 0.0;"),
    ("transposed operand", "dot += qv[d] * orc_load(ksrc, ko + d, dtype);",
     "dot += qv[d] * orc_load(ksrc, ko + (d ^ 1), dtype);"),
    ("mask column position", "a = orc_attend(qp, pos[c], 1, window, sink);",
     "a = orc_attend(qp, c, 1, window, sink);"),
    ("GDN: gate dropped", "for (long e = 0; e < (long)dk * dv; ++e) S[e] *= g;",
     "for (long e = 0; e < (long)dk * dv; ++e) S[e] *= 1.0;"),
    ("GDN: sign of the prediction", "const double delta = ((double)vt[j] - sum[j]) * bt;",
     "const double delta = ((double)vt[j] + sum[j]) * bt;"),
    ("GDN: beta dropped", "const double delta = ((double)vt[j] - sum[j]) * bt;",
     "const double delta = ((double)vt[j] - sum[j]);"),
    ("GDN: transposed state read", "for (int i = 0; i < dk; ++i) acc += S[(long)i * dv + j] * (double)kt[i];",
     "for (int i = 0; i < dk; ++i) acc += S[(long)(i % dv) * dv + (j % dk)] * (double)kt[i];"),
    ("GDN: read-out dropped",
     "      double *ot = out + row * dv;\n      for (int j = 0; j < dv; ++j) {",
     "      double *ot = out + row * dv;\n      for (int j = 0; j < dv && 0; ++j) {"),
    ("GDN: gate applied after the update",
     "      for (long e = 0; e < (long)dk * dv; ++e) S[e] *= g;\n      for (int j",
     "      for (int j = 0; j < dv && 0; ++j) {}\n      for (int j"),
]
# the second half of the last mutation: the decay moves to just before the read-out
MOVE_DECAY = ("      double *ot = out + row * dv;",
              "      for (long e = 0; e < (long)dk * dv; ++e) S[e] *= g;\n"
              "      double *ot = out + row * dv;")
MUTATIONS[-1] = (MUTATIONS[-1][0], MUTATIONS[-1][1], MUTATIONS[-1][2], MOVE_DECAY)
PIN_FILES = ("test_oracle_pins.py", "test_gdn_oracle_pins.py")


def main():
    orig = open(SRC).read()
    caught = 0
    with tempfile.TemporaryDirectory() as tmp:
        for name, a, b, *more in MUTATIONS:
            assert a in orig, name
            src = os.path.join(tmp, "m.c")
            lib = os.path.join(tmp, "libm.so")
            mutated = orig.replace(a, b, 1)
            for a2, b2 in more:
                assert a2 in mutated, name
                mutated = mutated.replace(a2, b2, 1)
            open(src, "w").write(mutated)
            subprocess.run(["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fPIC", "-shared",
                            "-o", lib, src, "-lm"], check=True)
            env = dict(os.environ, CP_ORACLE_LIB=lib)
            r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p",
                                "no:cacheprovider"] +
                               [os.path.join(ROOT, "tests", f) for f in PIN_FILES],
                               cwd=ROOT, env=env, capture_output=True, text=True)
            hit = r.returncode != 0
            caught += hit
            print(f"{'caught' if hit else 'MISSED'}: {name}", flush=True)
    print(f"{caught} / {len(MUTATIONS)} mutations caught")
    return 0


if __name__ == "__main__":
    sys.exit(main())
