"""KQ_LOG: with the variable set, plan creation, calls and errors print one "[kq]" line each
on stderr, naming the kernel variant chosen; without it, the library prints nothing. The
setting is read once per process, so each case runs in a fresh one."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

SNIPPET = r"""
import torch
from kronecker_factored_transforms_amd import binding as B, synth as S
import kqtest as K
inp = S.make("hidden_n8192", T=4096)
plan, X = K.make_plan(inp)
codes, scales = plan(X)
codes, scales = plan(X[:17])
P = torch.eye(64, dtype=torch.float32, device="cuda:0")
B.weight_factor(P)
try:
    B.kq_transform_quant(plan.handle, X, 5, 10, codes, scales)   # ldx < n
except B.KqError:
    pass
torch.cuda.synchronize()
print("done", flush=True)
"""


def _run(env_log):
    env = dict(os.environ)
    env.pop("KQ_LOG", None)
    if env_log is not None:
        env["KQ_LOG"] = env_log
    env["PYTHONPATH"] = os.pathsep.join([ROOT, os.path.join(ROOT, "tests"), env.get("PYTHONPATH", "")])
    return subprocess.run([sys.executable, "-c", SNIPPET], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_log_lines_name_the_kernels(gpu):
    r = _run("1")
    assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
    lines = [l for l in r.stderr.splitlines() if l.startswith("[kq] ")]
    print("\n".join(lines), flush=True)
    assert any(l.startswith("[kq] create 64x128 x=bf16") and "kernel fused_mfma_bf16_stream_64x128" in l
               and "fused_mfma_bf16_pair_64x128" in l for l in lines)
    assert any("transform T=4096" in l and "fused_mfma_bf16_stream_64x128" in l and l.endswith(": ok")
               for l in lines)
    assert any("transform T=17" in l and "fused_mfma_bf16_pair_64x128" in l for l in lines)
    assert any(l == "[kq] weight_factor m=64: ok" for l in lines)
    assert any("transform T=5 ldx=10" in l and l.endswith(": invalid argument") for l in lines)


def test_no_log_without_the_variable(gpu):
    for value in (None, "0", ""):
        r = _run(value)
        assert r.returncode == 0 and "done" in r.stdout, r.stderr[-2000:]
        assert "[kq]" not in r.stderr
