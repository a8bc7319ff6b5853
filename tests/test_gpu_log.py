"""The launch log (PISA_LOG): a prefill run in a child process with the
variable set describes each of its kernel launches on stderr; without it the
library prints nothing."""

import os
import subprocess
import sys

import pytest

from parity import log

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CHILD = r"""
import sys
sys.path.insert(0, sys.argv[1])
sys.path.insert(0, sys.argv[1] + '/tests')
import torch
import gen
import block_sparse_long_pisa_amd as pisa
from parity import cprob, to_dev
p = gen.Problem(1, 4, 2, 1000, 128, 64, 4, 2, 3, 64, "bf16")
q, k, v, _ = gen.host_inputs(p, 5, 0.1, None)
cp = cprob(p)
qd, kd, vd = to_dev(q, p.dtype), to_dev(k, p.dtype), to_dev(v, p.dtype)
pyr = pisa.build_pyramid(cp, kd)
idx, cnt = pisa.select_topk(cp, qd, pyr)
out, lse = pisa.sparse_attn_fwd(cp, qd, kd, vd, idx, cnt, want_lse=True)
torch.cuda.synchronize()
print("child done", flush=True)
"""


def _run(env_value):
    env = dict(os.environ)
    env.pop("PISA_LOG", None)
    if env_value is not None:
        env["PISA_LOG"] = env_value
    r = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "child done" in r.stdout
    return [l for l in r.stderr.splitlines() if l.startswith("[pisa]")]


def test_launch_log_describes_every_launch():
    log("launch log: a small prefill with PISA_LOG=1 in a child process")
    lines = _run("1")
    kernels = " ".join(lines)
    for name in ("pool_leaf_kernel", "select_kernel", "attn_bf16_kernel"):
        assert name in kernels, (name, lines)
    for l in lines:
        assert "grid (" in l and "workgroup (" in l and "N 1000" in l and "bf16" in l, l
    attn = [l for l in lines if "attn_bf16_kernel" in l]
    assert any("D = 128" in l and "BS = 64" in l for l in attn), attn  # the launcher's template arguments
    log(f"  {len(lines)} launches logged")


def test_no_log_without_the_variable():
    log("launch log: the same prefill with PISA_LOG unset, then 0")
    assert _run(None) == []
    assert _run("0") == []
