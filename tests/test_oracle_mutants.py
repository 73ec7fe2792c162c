"""The oracle's pins must catch plausible mistakes.

Each case plants one mistake (a dropped term, a wrong sign or index, a
swapped operand, a wrong tie rule) in a temporary copy of the oracle, on the
CPU, and runs the pin tests of test_oracle_ops / test_oracle_model /
test_oracle_formats / test_oracle_rounding against it.  At least one pin must fail for every
mutant, and all must pass for the unmodified copy."""
import importlib.util
import inspect
import os

import pytest

from tests import test_oracle_formats as F
from tests import test_oracle_model as M
from tests import test_oracle_ops as P
from tests import test_oracle_rounding as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

C_MUTANTS = {
    "rope-sign": ("u[i] = rbf(rbf(a * c[i], rnd) - rbf(b * s[i], rnd), rnd);",
                  "u[i] = rbf(rbf(a * c[i], rnd) + rbf(b * s[i], rnd), rnd);"),
    "rope-pairing": ("double a = u[i], b = u[i + h];", "double a = u[i], b = u[(i + 1) % h];"),
    "rope-frequency": ("pow(theta, -2.0 * (double)i / (double)d)", "pow(theta, -1.0 * (double)i / (double)d)"),
    "rmsnorm-no-eps": ("double v = r32(ms + r32(eps, rnd), rnd);", "double v = r32(ms, rnd);"),
    "rmsnorm-n-minus-1": ("double ms = r32(ss / (double)n, rnd);", "double ms = r32(ss / (double)(n - 1), rnd);"),
    "rmsnorm-no-weight": ("out[k] = rbf(wval(w, k) * xh, rnd);", "out[k] = rbf(xh, rnd);"),
    "attn-no-scale": ("scores[j] = rbf(rbf(acc, rnd) * sc, rnd);", "scores[j] = rbf(rbf(acc, rnd), rnd);"),
    "attn-pv-uses-k": ("acc += scores[j] * V[j * ld + i];", "acc += scores[j] * K[j * ld + i];"),
    "attn-no-normalise": ("scores[j] = rbf(r32(scores[j] / z, rnd), rnd);", "scores[j] = rbf(r32(scores[j], rnd), rnd);"),
    "dot-reversed-operand": ("acc += wval(w, k) * x[k];", "acc += wval(w, k) * x[K - 1 - k];"),
    "swiglu-silu-on-up": ("double z = rbf(g[i] / (1.0 + exp(-g[i])), rnd);\n        m[i] = rbf(z * u[i], rnd);",
                          "double z = rbf(u[i] / (1.0 + exp(-u[i])), rnd);\n        m[i] = rbf(z * g[i], rnd);"),
    "residual-dropped": ("x[i] = rbf(x[i] + y[i], rnd);", "x[i] = rbf(y[i], rnd);"),
    "argmax-last-tie": ("if (v[i] > v[best]) best = i;", "if (v[i] >= v[best]) best = i;"),
    "bf16-round-half-up": ("u += 0x7fffu + ((u >> 16) & 1u);", "u += 0x8000u;"),
    # the bf16 rounding points of the eager-bf16 reading
    "attn-score-single-rounding": ("scores[j] = rbf(rbf(acc, rnd) * sc, rnd);", "scores[j] = rbf(acc * sc, rnd);"),
    "attn-probs-fp32": ("scores[j] = rbf(r32(scores[j] / z, rnd), rnd);", "scores[j] = r32(scores[j] / z, rnd);"),
    "attn-output-fp32": ("o[i] = rbf(acc, rnd);", "o[i] = r32(acc, rnd);"),
    "rope-products-unrounded": ("u[i] = rbf(rbf(a * c[i], rnd) - rbf(b * s[i], rnd), rnd);\n"
                                "        u[i + h] = rbf(rbf(b * c[i], rnd) + rbf(a * s[i], rnd), rnd);",
                                "u[i] = rbf(a * c[i] - b * s[i], rnd);\n"
                                "        u[i + h] = rbf(b * c[i] + a * s[i], rnd);"),
    "swiglu-silu-unrounded": ("double z = rbf(g[i] / (1.0 + exp(-g[i])), rnd);",
                              "double z = r32(g[i] / (1.0 + exp(-g[i])), rnd);"),
    "rmsnorm-single-rounding": ("double xh = rbf(r32(x[k] * r, rnd), rnd);", "double xh = r32(x[k] * r, rnd);"),
    "residual-fp32": ("x[i] = rbf(x[i] + y[i], rnd);", "x[i] = r32(x[i] + y[i], rnd);"),
}

PY_MUTANTS = {
    "gqa-modulo-mapping": ("g = h // group", "g = h % Hkv"),
    "attend-excludes-current": ("self.K[seq][l][g, :pos + 1]", "self.K[seq][l][g, :max(pos, 1)]"),
    "rope-at-wrong-position": ("Kx[t, g] = rope(Kx[t, g], pos, s.rope_theta, rnd)",
                               "Kx[t, g] = rope(Kx[t, g], pos + 1, s.rope_theta, rnd)"),
    "final-norm-skipped": ("hf = rmsnorm(x, self.w[\"final_norm\"], self.s.rms_eps, self.rnd)",
                           "hf = x"),
    "logits-rounded-bf16": ("return linear(self.lm, hf, OUT_F32, self.rnd)",
                            "return linear(self.lm, hf, OUT_BF16, self.rnd)"),
    "q-projection-fp32": ("Q = linear(lw[\"wq\"], Hn, OUT_BF16, rnd)", "Q = linear(lw[\"wq\"], Hn, OUT_F32, rnd)"),
    "down-projection-fp32": ("D = linear(lw[\"w_down\"], M, OUT_BF16, rnd)", "D = linear(lw[\"w_down\"], M, OUT_F32, rnd)"),
    "qk-norm-after-rope": ("                if s.qk_norm:\n"
                           "                    Q[t, h] = rmsnorm(Q[t, h], lw[\"q_norm\"], s.rms_eps, rnd)\n"
                           "                Q[t, h] = rope(Q[t, h], pos, s.rope_theta, rnd)",
                           "                Q[t, h] = rope(Q[t, h], pos, s.rope_theta, rnd)\n"
                           "                if s.qk_norm:\n"
                           "                    Q[t, h] = rmsnorm(Q[t, h], lw[\"q_norm\"], s.rms_eps, rnd)"),
}


def _pins():
    pins = []
    for mod in (F, P, M, R):
        for name, fn in sorted(vars(mod).items()):
            if not name.startswith("test_") or not callable(fn):
                continue
            params = inspect.signature(fn).parameters
            if "tmp_path" in params:           # subprocess-based; not for mutants
                continue
            marks = getattr(fn, "pytestmark", [])
            cases = [{}]
            for m in marks:
                if m.name == "parametrize":
                    argname, values = m.args[0], m.args[1]
                    cases = [dict(c, **{argname: v}) for c in cases for v in values]
            for c in cases:
                pins.append((name, fn, c))
    return pins


def _load(tmp_path, tag, c_edit=None, py_edit=None):
    d = tmp_path / tag
    d.mkdir()
    c_src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    py_src = open(os.path.join(ROOT, "oracle", "oracle.py")).read()
    for src_name, edit in (("c", c_edit), ("py", py_edit)):
        if edit is None:
            continue
        old, new = edit
        src = c_src if src_name == "c" else py_src
        assert src.count(old) == 1, "mutation anchor not unique: %r" % old
        src = src.replace(old, new)
        if src_name == "c":
            c_src = src
        else:
            py_src = src
    (d / "oracle.c").write_text(c_src)
    (d / "oracle.py").write_text(py_src)
    spec = importlib.util.spec_from_file_location("oracle_mutant_" + tag.replace("-", "_"),
                                                  str(d / "oracle.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    mod.build()
    mod.lib()
    return mod


def _failures(mod):
    failed = []
    for name, fn, kw in _pins():
        try:
            fn(mod, **kw)
        except Exception:                       # a failed pin (or a crash it provokes)
            failed.append(name)
    return failed


@pytest.mark.slow
def test_unmodified_copy_passes_every_pin(tmp_path):
    assert _failures(_load(tmp_path, "clean")) == []


@pytest.mark.slow
@pytest.mark.parametrize("tag", sorted(C_MUTANTS) + sorted(PY_MUTANTS))
def test_planted_mistake_is_caught(tmp_path, tag):
    if tag in C_MUTANTS:
        mod = _load(tmp_path, tag, c_edit=C_MUTANTS[tag])
    else:
        mod = _load(tmp_path, tag, py_edit=PY_MUTANTS[tag])
    assert _failures(mod), "no pin caught mutant %s" % tag
