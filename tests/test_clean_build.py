"""build() from a clean checkout (CPU only): the committed tree, extracted with
``git archive HEAD`` into a temporary directory that holds no built library,
builds libkda (hipcc cross-compiles for gfx950 without a GPU) and the oracle,
then imports the package and loads the library it built there."""
import os
import shutil
import subprocess
import sys
import tarfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("git") is None or not os.path.isdir(os.path.join(ROOT, ".git")),
                    reason="needs git and the repository")
@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="needs hipcc")
def test_build_from_a_clean_checkout(tmp_path):
    tar = tmp_path / "head.tar"
    subprocess.run(["git", "-C", ROOT, "archive", "--format=tar", "-o", str(tar), "HEAD"], check=True)
    dst = tmp_path / "tree"
    dst.mkdir()
    with tarfile.open(tar) as tf:
        tf.extractall(dst)
    assert not (dst / "gated_delta_rule_67_amd" / "libkda.so").exists()
    script = ("import __graft_entry__ as g; g.build(); "
              "import gated_delta_rule_67_amd as kda; "
              "assert os.path.dirname(kda.LIB_PATH) == os.path.join(os.getcwd(), 'gated_delta_rule_67_amd'); "
              "print('abi', kda.abi_version())")
    env = dict(os.environ, PYTHONPATH=str(dst))
    r = subprocess.run([sys.executable, "-c", "import os; " + script], cwd=dst, env=env,
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]
    assert "abi " in r.stdout
    assert (dst / "gated_delta_rule_67_amd" / "libkda.so").exists()
