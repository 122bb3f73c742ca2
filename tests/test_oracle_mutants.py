"""The oracle's pins against planted mistakes.  Each mutant is the oracle's
C source with one plausible mistake (a dropped term, a wrong sign, index or
operand, an off-by-one or a broken ordering on the graph side), compiled on
the CPU; the pin suite (test_oracle_pins.py) run against it must fail.  The
unchanged source, built the same way, must pass.  The mistakes are planted
in the oracle only, and only here."""
import concurrent.futures
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "gt_oracle.c")
PINS = os.path.join(ROOT, "tests", "test_oracle_pins.py")

# name: (text of the oracle source, its mutated form); each text occurs once
MUTANTS = {
    # scores and softmax
    "bias dropped": ("if (p->bias) s += p->bias[e * p->H + h];",
                     "if (p->bias) s += 0.0 * p->bias[e * p->H + h];"),
    "bias scaled with the dot product": (
        "double s = p->scale * z;\n  if (p->bias) s += p->bias[e * p->H + h];",
        "double s = z;\n  if (p->bias) s += p->bias[e * p->H + h];\n  s *= p->scale;"),
    "scale missing": ("double s = p->scale * z;", "double s = z;"),
    "K of head 0 for every head": (
        "p->K + j * D + (i64)h * p->dh, p->dh);", "p->K + j * D, p->dh);"),
    "K of the row instead of the column": (
        "p->K + j * D + (i64)h * p->dh, p->dh);", "p->K + (i % p->M) * D + (i64)h * p->dh, p->dh);"),
    "weights not normalised": ("U[k * H + h] = exp(U[k * H + h] - m) / l;",
                               "U[k * H + h] = exp(U[k * H + h] - m);"),
    "lse without the log": ("m + log(l) : -INFINITY", "m + l : -INFINITY"),
    "Y from K": ("double v = p->V[j * (i64)H * dh + (i64)h * dh + c];",
                 "double v = p->K[j * (i64)H * dh + (i64)h * dh + c];"),
    "masked row not empty": ("for (i64 k = 0; k < deg; ++k) U[k * H + h] = 0.0;",
                             "for (i64 k = 0; k < deg; ++k) U[k * H + h] = 1.0 / (double)deg;"),
    # row side of the backward
    "dU from K": ("dot_head(p->dY + i * D + (i64)h * dh, p->V + j * D + (i64)h * dh, dh);",
                  "dot_head(p->dY + i * D + (i64)h * dh, p->K + j * D + (i64)h * dh, dh);"),
    "dU from Q": ("dot_head(p->dY + i * D + (i64)h * dh, p->V + j * D + (i64)h * dh, dh);",
                  "dot_head(p->Q + i * D + (i64)h * dh, p->V + j * D + (i64)h * dh, dh);"),
    "dS sign": ("dS[k * H + h] = U[k * H + h] * (dU[k * H + h] - Ds);",
                "dS[k * H + h] = U[k * H + h] * (Ds - dU[k * H + h]);"),
    "row term D dropped": ("dS[k * H + h] = U[k * H + h] * (dU[k * H + h] - Ds);",
                           "dS[k * H + h] = U[k * H + h] * dU[k * H + h];"),
    "D without the weights": ("Ds += U[k * H + h] * dU[k * H + h];", "Ds += dU[k * H + h];"),
    "dbias is the weight": ("o->dB[k * H + h] = dS[k * H + h];", "o->dB[k * H + h] = U[k * H + h];"),
    "dQ from V": ("double kv = p->K[j * D + (i64)h * dh + c];",
                  "double kv = p->V[j * D + (i64)h * dh + c];"),
    "dQ scale missing": ("if (o->dQ) o->dQ[(i64)h * dh + c] = p->scale * g;",
                         "if (o->dQ) o->dQ[(i64)h * dh + c] = g;"),
    # column side of the backward
    "dV from dS": ("gv += Uall[e * H + h] * y;", "gv += dSall[e * H + h] * y;"),
    "dK from dY (operand swapped)": ("gk += dSall[e * H + h] * q;", "gk += dSall[e * H + h] * y;"),
    "dK from the weights": ("gk += dSall[e * H + h] * q;", "gk += Uall[e * H + h] * q;"),
    "dK scale missing": ("dK[j * D + (i64)h * dh + c] = scale * gk;", "dK[j * D + (i64)h * dh + c] = gk;"),
    "column side reads edges by transposed position": ("i64 i = src[t], e = perm[t];",
                                                       "i64 i = src[t], e = t;"),
    # graph side
    "transpose not stable": (
        "for (i64 r = 0; r < R; ++r) {\n    for (i64 e = indptr[r]; e < indptr[r + 1]; ++e) {\n      i64 t = next",
        "for (i64 r = R - 1; r >= 0; --r) {\n    for (i64 e = indptr[r]; e < indptr[r + 1]; ++e) {\n      i64 t = next"),
    "transpose perm is the position": ("perm[t] = (i32)e;", "perm[t] = (i32)t;"),
    "CSR check lets duplicates through": ("indices[e] <= indices[e - 1]", "indices[e] < indices[e - 1]"),
    "CSR check misses column M": ("(i64)indices[e] >= M", "(i64)indices[e] > M"),
    "schedule ties by descending id": ("return (x > y) - (x < y);", "return (x < y) - (x > y);"),
    "schedule ignores the small classes": ("return d <= g_sort_small ? d - d % g_sort_class : d;",
                                           "return d;"),
    "schedule big threshold off by one": ("if (d > t_mid) nb++;", "if (d >= t_mid) nb++;"),
    "pieces of fixed length": ("items[4 * ni + 1] = (i32)(ptr[s] + (c * d) / nch);",
                               "items[4 * ni + 1] = (i32)(ptr[s] + c * chunk);"),
    "pieces dealt by their index": ("q[i + c] = (64 * (2 * c + 1)) / (2 * nch);",
                                    "q[i + c] = (64 * c) / nch;"),
}


def _build(src_text, path):
    c = path + ".c"
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-w", c, "-o", path, "-lm"],
                   check=True, timeout=300)


def _pins(lib):
    env = dict(os.environ, GT_ORACLE_LIB=lib, OMP_NUM_THREADS="1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider", PINS],
                       capture_output=True, text=True, env=env, timeout=600, cwd=ROOT)
    failed = [ln.split()[1] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
    return r.returncode, failed


def test_every_planted_mistake_fails_a_pin(tmp_path):
    src = open(SRC).read()
    jobs = {"(unchanged)": src}
    for name, (old, new) in MUTANTS.items():
        assert src.count(old) == 1, name
        jobs[name] = src.replace(old, new)

    def run(item):
        k, (name, text) = item
        lib = str(tmp_path / f"m{k}.so")
        _build(text, lib)
        return name, _pins(lib)

    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        results = dict(ex.map(run, enumerate(jobs.items())))
    rc, failed = results.pop("(unchanged)")
    assert rc == 0, f"the unchanged oracle fails its pins: {failed}"
    survivors = [n for n, (rc, _) in results.items() if rc != 1]
    for n, (rc, failed) in sorted(results.items()):
        print(f"{n}: {failed[0] if failed else 'rc ' + str(rc)}")
    assert not survivors, f"planted mistakes no pin catches: {survivors}"


# the numpy parts of the oracle: (module, its pin file) -> mutants
PY_MUTANTS = {
    ("layer.py", "test_oracle_layer.py"): {
        "Z without the residual": ("return _f64(X) @ _f64(Wo) + _f64(Y)", "return _f64(X) @ _f64(Wo)"),
        "Q from W_K": ("return X @ _f64(Wq), X @ _f64(Wk)", "return X @ _f64(Wk), X @ _f64(Wk)"),
        "dX without the V term": ("\n            + _f64(dV) @ _f64(Wv).T)", ")"),
        "dX with W_o untransposed": ("_f64(dZ) @ _f64(Wo).T", "_f64(dZ) @ _f64(Wo)"),
        "dW_Q from dK": ("Xt @ _f64(dQ), Xt @ _f64(dK)", "Xt @ _f64(dK), Xt @ _f64(dK)"),
        "bf16 by truncation": ("u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "u = u >> 16"),
        "bf16 ties away from zero": ("u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16", "u = (u + 0x8000) >> 16"),
    },
    ("heads.py", "test_oracle_heads.py"): {
        "split interleaves heads": ("out[r] = x[:, r * hp:(r + 1) * hp]", "out[r] = x[:, r::parts]"),
        "merge in reverse order": ("np.concatenate([p[r] for r in range(p.shape[0])], axis=1)",
                                   "np.concatenate([p[r] for r in reversed(range(p.shape[0]))], axis=1)"),
        "exchange takes heads strided": ("o[n, j] = blocks[owner[n]][local[n], r * hp + j]",
                                         "o[n, j] = blocks[owner[n]][local[n], j * p + r]"),
        "reverse exchange ignores the block offset": ("o[m, r * hp + j] = slices[r][starts[k] + m, j]",
                                                      "o[m, r * hp + j] = slices[r][m, j]"),
    },
}


def _python_copy(dst, module, text, pin_file):
    import shutil
    for sub, names in (("oracle", ("__init__.py", "oracle.py", "layer.py", "heads.py")),
                       ("graph_transformer_sparse_amd", ("__init__.py", "inputs.py")),
                       ("tests", ("conftest.py", pin_file))):
        os.makedirs(os.path.join(dst, sub))
        for n in names:
            shutil.copy(os.path.join(ROOT, sub, n), os.path.join(dst, sub, n))
    with open(os.path.join(dst, "oracle", module), "w") as f:
        f.write(text)


def test_numpy_oracle_mistakes_fail_a_pin(tmp_path):
    from oracle import oracle as O
    clib = O.build(force=False)          # the C part stays as it is
    jobs = []
    for (module, pin_file), muts in PY_MUTANTS.items():
        src = open(os.path.join(ROOT, "oracle", module)).read()
        jobs.append((module, pin_file, "(unchanged)", src))
        for name, (old, new) in muts.items():
            assert src.count(old) == 1, name
            jobs.append((module, pin_file, name, src.replace(old, new)))

    def run(item):
        k, (module, pin_file, name, text) = item
        dst = str(tmp_path / f"t{k}")
        _python_copy(dst, module, text, pin_file)
        env = dict(os.environ, GT_ORACLE_LIB=clib, OMP_NUM_THREADS="1")
        env.pop("PYTHONPATH", None)
        r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                            os.path.join("tests", pin_file)],
                           capture_output=True, text=True, env=env, timeout=600, cwd=dst)
        failed = [ln.split()[1] for ln in r.stdout.splitlines() if ln.startswith("FAILED ")]
        return (module, name), (r.returncode, failed, r.stdout[-400:])

    with concurrent.futures.ThreadPoolExecutor(max_workers=6) as ex:
        results = dict(ex.map(run, enumerate(jobs)))
    for (module, name), (rc, failed, tail) in sorted(results.items()):
        print(f"{module} {name}: {failed[0] if failed else 'rc ' + str(rc)}")
        if name == "(unchanged)":
            assert rc == 0, f"the unchanged {module} fails its pins: {tail}"
    survivors = [k for k, (rc, _, _) in results.items() if k[1] != "(unchanged)" and rc != 1]
    assert not survivors, f"planted mistakes no pin catches: {survivors}"
