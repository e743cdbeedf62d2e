"""Without the built library the product path fails loudly: the binding
raises ZeroLibraryMissing at the first call, and a rank's step cannot be set
up on any other code path. Run in child processes that point the binding at
a library path that does not exist."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import sys
from fsdp_sharded_mixed_zero_amd import synth, zero
from fsdp_sharded_mixed_zero_amd.rank import RankShard
calls = [lambda: zero.zero_layout([8, 8], 2, 0, 1),
         lambda: zero.zero_sqnorm_workspace_bytes(100),
         lambda: RankShard(synth.WORKLOADS["tiny"], device="cpu", fill=False)]
for k, call in enumerate(calls):
    try:
        call()
    except zero.ZeroLibraryMissing as e:
        print(f"call {k}: missing: {e}")
    else:
        print(f"call {k}: ran without the library")
        sys.exit(1)
"""


def test_calls_raise_when_the_library_is_missing(tmp_path):
    env = dict(os.environ, ZERO_MI355X_LIB=str(tmp_path / "absent" / "libzero_mi355x.so"))
    r = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, env=env, capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    lines = r.stdout.strip().splitlines()
    assert len(lines) == 3 and all(": missing: " in ln and "absent" in ln for ln in lines), r.stdout
