"""The C ABI used from C++ host code alone (HIP runtime + include/attn_fwd.h + libattn_fwd.so, no
Python in the process): closed-form results in every mask mode and the NULL-pointer error path.
The program is built next to the library by the package build and runs as a child process."""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROGRAM = os.path.join(ROOT, "attention_forward_06_amd", "c_abi_check")


@pytest.mark.gpu
def test_c_abi_from_cpp_host_code():
    if not os.path.exists(PROGRAM):
        pytest.skip("c_abi_check is not built (attention_forward_06_amd.build.build() builds it)")
    res = subprocess.run([PROGRAM], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0 and "ALL PASS" in res.stdout, res.stdout + res.stderr
    lines = res.stdout.splitlines()
    for mode in ("none", "causal", "block_diag"):
        for check in ("constant V", "Q = 0 log-normaliser"):
            line = [x for x in lines if x.startswith(f"{mode} {check}")]
            assert len(line) == 1 and line[0].endswith("PASS"), (mode, check, res.stdout)
