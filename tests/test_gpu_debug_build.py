"""The debug build (device index checks, -DHA_DEBUG) on the GPU: a child
process loads libhybrid_attn_debug.so and runs the main-path entry points on
edge shapes; any failed check makes a call return HA_ERR_DEVICE."""
import os
import subprocess
import sys

import pytest

from video_dit_hybrid_amd import build as B

pytestmark = pytest.mark.gpu


def test_debug_build_index_checks_pass(repo_root):
    assert os.path.exists(B.DEBUG_LIB_PATH), "the debug library is built by __graft_entry__.build()"
    env = dict(os.environ, HYBRID_ATTN_LIBRARY="debug")
    p = subprocess.run([sys.executable, "-u", os.path.join(repo_root, "tests", "debug_build_child.py")], env=env,
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=240)
    print(p.stdout[-3000:])
    assert p.returncode == 0, p.stdout[-3000:]
    assert "all index checks passed" in p.stdout
    assert "[hybrid_attn debug]" not in p.stdout
