import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # MUSE_SANITIZED=1 (set by tests/test_sanitizers.py for its child run):
    # load the ASan/UBSan builds of the HIP library and of the oracle
    if os.environ.get("MUSE_SANITIZED") == "1":
        import full_gqa_attention_amd as fa
        from full_gqa_attention_amd import build as fa_build
        import oracle
        fa.LIB_PATH = fa_build.SAN_LIB_PATH
        oracle.use_sanitized_build()


def pytest_sessionfinish(session, exitstatus):
    if os.environ.get("MUSE_SANITIZED") == "1":
        maps = open("/proc/self/maps").read()
        for name in ("libmuse_attn_san.so", "liboracle_san.so"):
            print(f"\nsanitized library {name} loaded: {name in maps}")
