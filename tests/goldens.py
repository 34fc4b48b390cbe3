"""Readers for the cited text fixtures under tests/golden/.

The fixtures hold index expressions exactly as the pages print them; they are
evaluated here with a tiny arithmetic-only evaluator (no names other than the
index variables, no calls).
"""

from __future__ import annotations

import ast
import operator
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_OPS = {
    ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
    ast.Mod: operator.mod, ast.FloorDiv: operator.floordiv, ast.BitXor: operator.xor,
    ast.BitAnd: operator.and_, ast.BitOr: operator.or_, ast.RShift: operator.rshift,
    ast.LShift: operator.lshift,
}


def eval_index(expr: str, **names: int) -> int:
    def ev(node):
        if isinstance(node, ast.Expression):
            return ev(node.body)
        if isinstance(node, ast.BinOp) and type(node.op) in _OPS:
            return _OPS[type(node.op)](ev(node.left), ev(node.right))
        if isinstance(node, ast.Constant) and isinstance(node.value, int):
            return node.value
        if isinstance(node, ast.Name) and node.id in names:
            return names[node.id]
        raise ValueError(f"unsupported expression element: {ast.dump(node)}")
    return ev(ast.parse(expr, mode="eval"))


def _lines(name):
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def ints(text: str):
    return tuple(int(x) for x in text.split(","))


def address_examples():
    out = []
    for line in _lines("buffers_address_examples.txt"):
        name, shape, strides, off, expr = [p.strip() for p in line.split("|")]
        out.append((name, ints(shape), ints(strides), int(off), expr))
    return out


def view_permute_examples():
    out = []
    for line in _lines("buffers_view_permute.txt"):
        name, idx, strides, expr = [p.strip() for p in line.split("|")]
        out.append((name, tuple(idx.split(",")), ints(strides), expr))
    return out


def sf_ir():
    d = {}
    for line in _lines("sf_generated_ir.txt"):
        key, val = [p.strip() for p in line.split("=", 1)]
        d[key] = val
    ranges = dict((k, int(v)) for k, v in (t.split(":") for t in d["ranges"].split()))
    return {
        "read": d["read"], "write": d["write"], "ranges": ranges,
        "P": int(d["P"]), "shift": int(d["shift"]), "mask": int(d["mask"]),
        "region_extents": ints(d["region_extents"]),
        "src_strides": ints(d["src_strides"]), "dst_strides": ints(d["dst_strides"]),
    }
