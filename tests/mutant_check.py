"""Run the quick oracle pins against one build of the oracle library.

Usage: python tests/mutant_check.py <path-to-liboracle.so>
Exit status 0 if every pin holds, 1 if one fails (its name is printed).
Used by the mutation test, which runs it in a child process so that a broken
build that reads out of bounds cannot take the test run down with it.
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(HERE))
sys.path.insert(0, HERE)

import oracle  # noqa: E402
import pins  # noqa: E402


def main(path: str) -> int:
    orc = oracle.load(path)
    with open(os.path.join(HERE, "golden", "printed_shapes.json")) as f:
        shapes = json.load(f)["cases"]
    checks = [lambda o: pins.check_printed_shapes(o, shapes)] + list(pins.QUICK_CHECKS)
    for chk in checks:
        try:
            chk(orc)
        except Exception as e:  # any failure kills the mutant
            print(f"FAILED {getattr(chk, '__name__', 'check')}: {type(e).__name__}: {str(e)[:200]}")
            return 1
    print("all pins hold")
    return 0


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
