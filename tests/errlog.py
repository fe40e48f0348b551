"""Optional record of the errors the GPU parity tests measure.

With RN_TEST_ERROR_LOG set to a file name, every error a test computes is appended to
that file as one JSON line (test id, kind, value); the tolerances in the tests are set
from these records (about five times the largest error measured for each kind). Without
the variable nothing is written."""
import json
import os


def record(kind, value):
    path = os.environ.get("RN_TEST_ERROR_LOG")
    if path:
        test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
        with open(path, "a") as f:
            f.write(json.dumps({"test": test, "kind": kind, "value": float(value)}) + "\n")
