"""Loader of the hand-worked fixtures under tests/golden/.

A fixture holds the inputs of a tiny case and its expected outputs, each
written as an arithmetic expression (numbers, + - * /, exp, tanh, and the
symbols the fixture defines, e.g. s2 = 1/(1+exp(-2))).  The expressions were derived by
hand; this module only evaluates them, with a parser that admits nothing
but that arithmetic.
"""
from __future__ import annotations

import ast
import json
import math
import os
import operator

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_BIN = {ast.Add: operator.add, ast.Sub: operator.sub, ast.Mult: operator.mul,
        ast.Div: operator.truediv}
_UN = {ast.USub: operator.neg, ast.UAdd: operator.pos}
_FUN = {"exp": math.exp, "tanh": math.tanh}


def _eval(node, env):
    if isinstance(node, ast.Expression):
        return _eval(node.body, env)
    if isinstance(node, ast.Constant) and isinstance(node.value, (int, float)):
        return float(node.value)
    if isinstance(node, ast.Name) and node.id in env:
        return env[node.id]
    if isinstance(node, ast.BinOp) and type(node.op) in _BIN:
        return _BIN[type(node.op)](_eval(node.left, env), _eval(node.right, env))
    if isinstance(node, ast.UnaryOp) and type(node.op) in _UN:
        return _UN[type(node.op)](_eval(node.operand, env))
    if (isinstance(node, ast.Call) and isinstance(node.func, ast.Name)
            and node.func.id in _FUN and len(node.args) == 1 and not node.keywords):
        return _FUN[node.func.id](_eval(node.args[0], env))
    raise ValueError(f"not plain arithmetic: {ast.dump(node)}")


def evaluate(expr: str, env) -> float:
    return _eval(ast.parse(expr, mode="eval"), env)


def _values(v, env):
    if isinstance(v, list):
        return [_values(u, env) for u in v]
    if isinstance(v, str):
        return evaluate(v, env)
    return v


def symbols(fx):
    """The fixture's symbols, evaluated in order (later ones may use earlier)."""
    env = {}
    for sym, expr in fx.get("symbols", {}).items():
        env[sym] = evaluate(expr, env)
    return env


def load_raw(name: str):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


def load(name: str):
    """(config dict, inputs as float32 arrays, expected values).

    Expected entries written as strings become float64 arrays; entries
    written as plain integers (indices, counts) become int64 arrays."""
    with open(os.path.join(GOLDEN, name)) as fh:
        fx = json.load(fh)
    env = {}
    for sym, expr in fx["symbols"].items():  # in order: later ones may use earlier ones
        env[sym] = evaluate(expr, env)
    inputs = {k: np.asarray(v, np.float32) for k, v in fx["inputs"].items()}
    expected = {}
    for k, v in fx["expected"].items():
        val = _values(v, env)
        arr = np.asarray(val)
        expected[k] = arr.astype(np.float64) if arr.dtype.kind == "f" else arr.astype(np.int64)
    return fx["config"], inputs, expected
