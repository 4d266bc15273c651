"""The streaming kernels under the LDS-poison debug build: every LDS buffer
is filled with 0xff bytes before each use, and the parity cases of
lds_poison_cases.py must still pass (a kernel that reads LDS it did not
write for the tile at hand fails them).  The debug library is built with
`python -m kv_cache_quantization_srft_amd.build --poison`; the cases run in
one child process that loads it through SRFTQ_LIBRARY."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
POISON_LIB = os.path.join(ROOT, "kv_cache_quantization_srft_amd", "libsrftq_poison.so")


@pytest.mark.skipif(not os.path.exists(POISON_LIB), reason="LDS-poison debug build not built (build.py --poison)")
def test_streaming_kernels_read_only_what_they_wrote():
    env = dict(os.environ, SRFTQ_LIBRARY=POISON_LIB)
    r = subprocess.run([sys.executable, "-u", os.path.join(ROOT, "tests", "lds_poison_cases.py")], env=env,
                       capture_output=True, text=True, timeout=600)
    print(r.stdout[-4000:])
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all cases passed" in r.stdout
