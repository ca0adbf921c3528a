"""Plant plausible mistakes in a copy of the oracle (on the CPU) and check that
the pins catch every one: a pin set that a dropped term, a wrong sign, a
transposed operand or a reversed path could slip through would not pin
anything."""
import os

import pytest

import pins
from oracle import Oracle
from oracle import build as obuild

MUTANTS = {
    "erase term dropped": ("row[j] = a * (row[j] - bx * kj) + bv * kj;", "row[j] = a * row[j] + bv * kj;"),
    "erase sign flipped": ("row[j] = a * (row[j] - bx * kj) + bv * kj;", "row[j] = a * (row[j] + bx * kj) + bv * kj;"),
    "decay skips the erase": ("row[j] = a * (row[j] - bx * kj) + bv * kj;", "row[j] = a * row[j] - bx * kj + bv * kj;"),
    "write not gated by beta": ("double bv = b * (double)v[i];", "double bv = (double)v[i];"),
    "state read transposed": ("for (int j = 0; j < dk; ++j) s += S[(size_t)i * dk + j] * (double)q[j];",
                              "for (int j = 0; j < dk; ++j) s += S[(size_t)j * dk + i] * (double)q[j];"),
    "path walked leaf first": ("for (int i = 0; i < len / 2; ++i) {", "for (int i = 0; i < 0; ++i) {"),
    "erase uses the value": ("double bx = b * x[i];", "double bx = b * (double)v[i];"),
    "chain parent off by one": (": n - 1;", ": n - 2;"),
    "gather copies the wrong head": ("const float* src = c->pool + ((size_t)s * c->H + h) * dd;",
                                     "const float* src = c->pool + ((size_t)s * c->H + (h + 1) % c->H) * dd;"),
    "block read at the parent's state": ("walk_to(w, b, h, n, S, x, path, NULL);",
                                         "walk_to(w, b, h, n >= 0 ? parent_of(w->parent, w->T, b, n) : n, S, x, path, NULL);"),
    "argmax keeps the last maximum": ("if (best < 0 || t > bv) {", "if (best < 0 || t >= bv) {"),
    "walk takes the last matching child": ("next = c;\n                    break;", "next = c;"),
    "bonus read one row early": ("if (bonus) bonus[b] = tg[cur + 1];", "if (bonus) bonus[b] = tg[cur < 0 ? 0 : cur];"),
    "commit at the node before the accepted one": (
        "walk_to(c, b, h, c->accepted[b], S, x, path, NULL);",
        "walk_to(c, b, h, c->accepted[b] > 0 ? c->accepted[b] - 1 : c->accepted[b], S, x, path, NULL);"),
    "gather reads the state transposed": ("acc += (double)src[(size_t)r * c->dk + j] * (double)qv[j];",
                                          "acc += (double)src[(size_t)j * c->dk + r] * (double)qv[j];"),
    "log decay leaves out the node's own gate": ("for (int i = 0; i < len; ++i) {\n                    int e;",
                                                 "for (int i = 0; i < len - 1; ++i) {\n                    int e;"),
    "log decay drops the exponent": ("logp[((size_t)b * T + n) * H + h] = log(P) + (double)e2 * log(2.0);",
                                     "logp[((size_t)b * T + n) * H + h] = log(P);"),
    "log decay walks a chain instead of the tree": ("int len = root_path(parent, T, b, n, path);",
                                                    "int len = root_path(NULL, T, b, n, path);"),
    "gather pairs an output with the next query": (
        "const float* qv = c->queries + (((size_t)bp * c->H + h) * c->Qn + i) * c->dk;",
        "const float* qv = c->queries + (((size_t)bp * c->H + h) * c->Qn + (i + 1) % c->Qn) * c->dk;"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    with open(obuild.SRC) as f:
        src = f.read()
    assert src.count(old) >= 1, "mutation site vanished from oracle.c"
    mpath = os.path.join(str(tmp_path), "mutant.c")
    with open(mpath, "w") as f:
        f.write(src.replace(old, new))
    lib = obuild.build(src=mpath, out=os.path.join(str(tmp_path), "libmutant.so"))
    m = Oracle(lib)
    caught = []
    for pin in pins.ALL_PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught: " + name
