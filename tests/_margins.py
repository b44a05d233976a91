"""Records of the measured parity errors (test infrastructure).

When ``LOSA_PARITY_LOG`` names a file, each GPU parity check appends one JSON
line with the errors it measured (max-abs, mean-abs, per quantity), so that a
run leaves the actual margins next to the bounds the tests assert.  Without
the variable nothing is written.
"""

import json
import os
import threading

_lock = threading.Lock()


def record(test, case, **values):
    path = os.environ.get("LOSA_PARITY_LOG")
    if not path:
        return
    row = {"test": test, "case": case}
    for key, val in values.items():
        if isinstance(val, bool) or not hasattr(val, "__float__"):
            row[key] = val
        elif float(val).is_integer() and "int" in type(val).__name__:
            row[key] = int(val)
        else:
            row[key] = float(val)
    with _lock, open(path, "a") as fh:
        fh.write(json.dumps(row) + "\n")
