"""The library and torch share one HIP runtime, whatever the import order
(no GPU needed): importing the binding first must not leave two
libamdhip64 copies in the process."""
import subprocess
import sys

from tests.conftest import ROOT


def test_one_hip_runtime_when_the_binding_is_imported_first():
    code = ("from residual_stream_architecture_amd import xhc\n"
            "import torch\n"
            "maps = open('/proc/self/maps').read().split('\\n')\n"
            "paths = sorted({l.split()[-1] for l in maps if 'libamdhip64' in l})\n"
            "print(len(paths), paths)\n"
            "assert len(paths) == 1, paths\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
