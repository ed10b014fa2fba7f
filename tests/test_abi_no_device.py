"""Runs the C-ABI contract checks of test_abi.py in a child process that sees
no HIP device (HIP_VISIBLE_DEVICES=-1).  Those checks pass fake device
pointers that only host-side validation may look at; with no visible device,
a call that got past validation by mistake fails in the HIP runtime instead
of launching a kernel on a GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_contract_without_a_device():
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1")
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_abi.py")],
                         cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    print(res.stdout[-4000:], res.stderr[-2000:])
    assert res.returncode == 0, res.stdout[-4000:]
    assert " passed" in res.stdout and "skipped" not in res.stdout.split("\n")[-2]
