"""pytest plugin for the sanitizer run (loaded with `-p sanitize_plugin` by
tests/test_sanitizers.py, never by the ordinary suite).

HA_SAN_HOST_LIB names an ASan/UBSan build of the library's host-only sources
(the step generator and the status strings); the binding is pointed at it
before any test loads the real library, so the scheduler tests run on the
sanitized code.  ORACLE_LIB (read by oracle/oracle.py) does the same for the
oracle.  At the end of the session the plugin writes which libraries were in
use to HA_SAN_REPORT."""
import ctypes
import os


def pytest_configure(config):
    from chunked_prefill_mixed_hybrid_amd import binding as B
    lib = ctypes.CDLL(os.environ["HA_SAN_HOST_LIB"])
    lib.ha_status_string.argtypes = [ctypes.c_int]
    lib.ha_status_string.restype = ctypes.c_char_p
    B._lib = lib


def pytest_sessionfinish(session, exitstatus):
    import oracle
    from chunked_prefill_mixed_hybrid_amd import binding as B
    with open(os.environ["HA_SAN_REPORT"], "w") as f:
        f.write(f"oracle {oracle.default().path}\n")
        f.write(f"host {B._lib._name}\n")
