"""Run every oracle pin against one oracle library and report the first that
fails.  Used in a child process by the mutation tests, so that a planted
mistake that corrupts memory cannot take the test process down.

usage: python tests/pin_runner.py <path to liboracle .so>
exit 0: some pin failed (the planted mistake was caught) and its name is printed
exit 1: every pin passed
"""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import oracle  # noqa: E402
from oracle_pins import ALL_PINS  # noqa: E402


def main(path):
    L = oracle.load_from(path)
    for pin in ALL_PINS:
        try:
            pin(L)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            print(f"caught by {pin.__name__}: {type(e).__name__}")
            return 0
    print("not caught")
    return 1


if __name__ == "__main__":
    sys.exit(main(sys.argv[1]))
