"""The oracle against its stored outputs (tests/golden/oracle_small.json)."""
import json
import sys
from pathlib import Path

import numpy as np

import oracle

GOLDEN = Path(__file__).parent / "golden"
sys.path.insert(0, str(GOLDEN))


def test_oracle_reproduces_stored_outputs():
    import make_golden
    doc = json.loads((GOLDEN / "oracle_small.json").read_text())
    p = {k: np.asarray(v) for k, v in doc["inputs"].items()}
    fresh = make_golden.outputs(oracle.default(), p)
    for name, group in doc["outputs"].items():
        for k, v in group.items():
            if v is None:
                assert fresh[name][k] is None
                continue
            np.testing.assert_allclose(fresh[name][k], np.asarray(v), rtol=1e-13, atol=1e-15, err_msg=name + "." + k)
