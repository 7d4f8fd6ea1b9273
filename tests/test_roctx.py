"""roctx ranges (MOE_ROCTX=1): the library finds the roctx library at run time and its entry points still
validate and reject as documented with the ranges on; without the variable nothing is looked up.  CPU
only: every call below is rejected before any HIP call."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

PROBE = r"""
import ctypes, sys
sys.path.insert(0, %r)
from sparse_moe_expert_sigmoid_amd import abi
import synth
dims = synth.CONFIGS["tiny"].dims
FAKE = 0x10000
# rejected on the host (missing routing workspace, NULL weights): range pushed and popped around the return
rc = abi.moe_route(dims, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 1 << 20, stream=0, check=False)
assert rc == abi.MOE_EINVAL, rc
rc = abi.moe_w4a8_forward(dims, FAKE, FAKE, FAKE, FAKE, {k: 0 for k in ("w13_codes", "w13_exps", "w2_codes",
                          "w2_exps", "s13_codes", "s13_exps", "s2_codes", "s2_exps")}, FAKE, FAKE, routing_bytes=1 << 20,
                          scratch_bytes=1 << 30, flags=abi.MOE_FLAG_FORCE_GROUPED, stream=0, check=False)
assert rc == abi.MOE_EINVAL, rc
maps = open("/proc/self/maps").read()
print("ROCTX_LOADED" if ("roctx" in maps) else "ROCTX_ABSENT")
""" % ROOT


def _run(env_extra):
    env = dict(os.environ)
    env.pop("MOE_ROCTX", None)
    env.update(env_extra)
    r = subprocess.run([sys.executable, "-c", PROBE], capture_output=True, text=True, env=env, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    return r.stdout


def test_ranges_on_with_moe_roctx():
    out = _run({"MOE_ROCTX": "1"})
    roctx_present = os.path.exists("/opt/rocm/lib/librocprofiler-sdk-roctx.so.1") or \
        os.path.exists("/opt/rocm/lib/libroctx64.so.4")
    assert ("ROCTX_LOADED" in out) == roctx_present, out


def test_nothing_looked_up_without_moe_roctx():
    assert "ROCTX_ABSENT" in _run({})
