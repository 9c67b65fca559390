"""Reader for the closed-form fixtures under tests/golden/."""
import math
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

_MATH = {"sqrt": math.sqrt, "exp": math.exp, "cos": math.cos, "sin": math.sin, "pi": math.pi}


def evaluate(expr: str, **names) -> float:
    """Evaluate one closed-form expression with Python's math functions only."""
    return float(eval(expr, {"__builtins__": {}}, {**_MATH, **names}))  # noqa: S307 - fixture text


def cases(filename: str):
    """Yield each case of a fixture as a dict of field -> list of expression strings."""
    with open(os.path.join(GOLDEN, filename), encoding="utf-8") as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            case = {}
            for field in line.split(";"):
                key, value = field.split("=", 1)
                case[key.strip()] = [v.strip() for v in value.split(",")]
            yield case


def values(exprs, **names):
    return [evaluate(e, **names) for e in exprs]
