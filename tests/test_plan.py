"""Host planner of the C ABI (pure C++): workspace regions hold everything any launch plan writes (CPU only)."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sigmoid_routed_mixture_amd", "csrc")


def test_workspace_layout_invariants(tmp_path):
    exe = str(tmp_path / "plan_check")
    subprocess.run(["g++", "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
                    os.path.join(os.path.dirname(__file__), "plan_check.cpp"), os.path.join(CSRC, "plan.cpp"),
                    "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True)
    print(r.stdout[-2000:])
    assert r.returncode == 0, r.stdout[-4000:]
