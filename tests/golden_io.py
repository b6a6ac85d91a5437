"""Reader for the hand-computed fixtures in tests/golden/ (plain text, one key per line)."""
import ast
import math
import operator
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_OPS = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv, ast.USub: operator.neg, ast.Pow: operator.pow}


def _eval(node):
    if isinstance(node, ast.Expression):
        return _eval(node.body)
    if isinstance(node, ast.Constant):
        return float(node.value)
    if isinstance(node, ast.Name) and node.id == "sqrt2":
        return math.sqrt(2.0)
    if isinstance(node, ast.BinOp):
        return _OPS[type(node.op)](_eval(node.left), _eval(node.right))
    if isinstance(node, ast.UnaryOp):
        return _OPS[type(node.op)](_eval(node.operand))
    raise ValueError(f"unsupported token in golden value: {ast.dump(node)}")


def value(tok: str) -> float:
    return _eval(ast.parse(tok, mode="eval"))


def load(name: str) -> dict:
    """Returns {key: list of rows (each a list of floats)}; rows are split by '|'."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            key, rest = line.split(None, 1) if not line.startswith("row ") else (
                line.split(":")[0], line.split(":", 1)[1])
            rows = [[value(t) for t in part.split()] for part in rest.split("|")]
            out[key.strip()] = rows
    return out
