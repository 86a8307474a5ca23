"""The binding must leave one HIP runtime in the process whatever the import
order (CPU check of the loaded shared objects)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_one_hip_runtime_when_package_is_imported_before_torch():
    code = ("import decode_attention_gqa_amd, torch\n"
            "maps = open('/proc/self/maps').read().splitlines()\n"
            "print(sorted({l.split()[-1] for l in maps if 'libamdhip64' in l}))\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    paths = eval(r.stdout.strip().splitlines()[-1])
    assert len(paths) == 1, paths
