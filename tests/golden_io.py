"""Readers for the hand-derived fixtures in tests/golden (tiny restricted expression parser)."""
import ast
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _eval(node):
    if isinstance(node, ast.Expression):
        return _eval(node.body)
    if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
        return float(node.value)
    if isinstance(node, ast.List):
        return [_eval(e) for e in node.elts]
    if isinstance(node, ast.UnaryOp) and isinstance(node.op, (ast.USub, ast.UAdd)):
        x = _eval(node.operand)
        return -x if isinstance(node.op, ast.USub) else x
    if isinstance(node, ast.BinOp):
        a, b = _eval(node.left), _eval(node.right)
        ops = {ast.Add: lambda: a + b, ast.Sub: lambda: a - b, ast.Mult: lambda: a * b,
               ast.Div: lambda: a / b, ast.Pow: lambda: a ** b}
        return ops[type(node.op)]()
    if isinstance(node, ast.Call) and isinstance(node.func, ast.Name) and node.func.id == "ln" and len(node.args) == 1:
        return math.log(_eval(node.args[0]))
    raise ValueError(f"unsupported expression: {ast.dump(node)}")


def expr(text: str):
    return _eval(ast.parse(text.strip(), mode="eval"))


def read_assignments(name):
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, val = line.split("=", 1)
            out[key.strip()] = np.array(expr(val), dtype=np.float64)
    return out


def read_rows(name, prefix=None):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            parts = line.split()
            if prefix is None:
                rows.append([float(x) for x in parts])
            elif parts[0] == prefix:
                rows.append(parts[1:])
    return rows
