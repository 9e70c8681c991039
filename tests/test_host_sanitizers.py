"""The host C++ side (runtime, thread pool, host Adam, accumulation, init,
ABI validation) rebuilt with ThreadSanitizer and with AddressSanitizer and run
under the CPU host tests; any sanitizer report fails the test.  The GPU
kernels are linked in uninstrumented and are not called without a GPU."""
import os

import pytest

from layer_streaming_amd import sanitize

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("kind", sanitize.KINDS)
def test_host_tests_pass_clean_under_sanitizer(kind):
    status, out = sanitize.run_tests(kind, [os.path.join(ROOT, "tests", "test_host.py")])
    assert "Sanitizer" not in out, out[-8000:]
    assert status == 0, out[-8000:]
    assert " passed" in out
