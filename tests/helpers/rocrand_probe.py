"""Builds and runs the host-side rocRAND Philox4x32-10 probe (a library cross-check)."""
import os
import shutil
import subprocess
import tempfile

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "rocrand_philox_probe.cpp")
_exe = None


def available() -> bool:
    return shutil.which("hipcc") is not None and os.path.exists("/opt/rocm/include/rocrand")


def _build() -> str:
    global _exe
    if _exe is None:
        d = tempfile.mkdtemp(prefix="rr_probe_")
        exe = os.path.join(d, "probe")
        subprocess.run(["hipcc", "-O1", "-o", exe, SRC], check=True, cwd=d,
                       stdout=subprocess.DEVNULL, stderr=subprocess.DEVNULL)
        _exe = exe
    return _exe


def philox_blocks(ctr: np.ndarray, key: np.ndarray) -> np.ndarray:
    """ctr [n, 4] uint32, key [n, 2] uint32 -> [n, 4] uint32 (rocRAND's ten_rounds)."""
    exe = _build()
    lines = "\n".join("%d %d %d %d %d %d" % (*c, *k) for c, k in zip(ctr.tolist(), key.tolist()))
    out = subprocess.run([exe], input=lines + "\n", capture_output=True, text=True, check=True).stdout
    return np.array([[int(x) for x in ln.split()] for ln in out.strip().splitlines()], dtype=np.uint64
                    ).astype(np.uint32)
