"""The product builds from its sources alone: a copy of the repository's files
(what git tracks or would track, no built library) runs ``__graft_entry__.build()``,
then imports the package and passes the C-ABI checks, in a fresh process."""
import os
import shutil
import subprocess
import sys
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _source_files():
    try:
        out = subprocess.run(["git", "ls-files", "--cached", "--others", "--exclude-standard", "-z"],
                             cwd=ROOT, capture_output=True, check=True).stdout
    except (OSError, subprocess.CalledProcessError):
        return None
    files = [f for f in out.decode().split("\0") if f]
    return [f for f in files if os.path.isfile(os.path.join(ROOT, f))]


@pytest.mark.skipif(shutil.which("git") is None or not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs git and hipcc")
def test_build_from_a_clean_tree():
    files = _source_files()
    if files is None:
        pytest.skip("not a git checkout")
    assert not any(f.endswith(".so") for f in files), "built libraries are not sources"
    with tempfile.TemporaryDirectory() as td:
        for f in files:
            dst = os.path.join(td, f)
            os.makedirs(os.path.dirname(dst), exist_ok=True)
            shutil.copy2(os.path.join(ROOT, f), dst)
        assert not os.path.exists(os.path.join(td, "selective_state_space_mimo_amd", "libm3scan.so"))
        env = dict(os.environ, PYTHONDONTWRITEBYTECODE="1")
        # the package refuses to import before the build
        r = subprocess.run([sys.executable, "-c", "import selective_state_space_mimo_amd"], cwd=td,
                           capture_output=True, text=True, env=env)
        assert r.returncode != 0 and "not built" in r.stderr
        r = subprocess.run([sys.executable, "-c", "import __graft_entry__ as g; g.build()"], cwd=td,
                           capture_output=True, text=True, env=env, timeout=900)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert os.path.exists(os.path.join(td, "selective_state_space_mimo_amd", "libm3scan.so"))
        r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-m", "not gpu", "-p", "no:cacheprovider",
                            os.path.join("tests", "test_abi.py")], cwd=td, capture_output=True, text=True,
                           env=env, timeout=600)
        assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-2000:]
