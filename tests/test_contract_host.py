"""Host-side checks of the run contract: bench.py refuses more than one GPU, and the
binding raises when the compiled library is absent instead of computing anything
elsewhere.  No GPU is touched."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("argv,env", [
    (["--gpus", "2"], {}),
    (["--gpus", "8"], {}),
    (["--gpus", "1"], {"WORLD_SIZE": "4"}),
])
def test_bench_refuses_more_than_one_gpu(argv, env):
    e = dict(os.environ)
    e.update(env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *argv],
                       cwd=ROOT, env=e, capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_missing_library_raises(monkeypatch, tmp_path):
    from long_context_attention_rkv_amd import _lib
    monkeypatch.setattr(_lib, "LIB_PATH", str(tmp_path / "librkv.so"))
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        _lib.load()
