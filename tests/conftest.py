import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: full-size parity cases")


def pytest_sessionstart(session):
    """State, in the run's log, which library the tests exercise: kvz.lib()
    refuses a libkvz.so whose build id differs from the digest of the sources
    in this checkout, so a passing check means the binary is HEAD's source."""
    from attention_score_reduction_amd import build, kvz
    tr = session.config.pluginmanager.get_plugin("terminalreporter")
    try:
        bid = kvz.kvz_build_id()
        line = f"libkvz build id {bid[:16]} matches the source digest {build.source_digest()[:16]}"
    except Exception as e:  # the GPU tests fail loudly on their own; say why here
        line = f"libkvz not loadable: {e}"
    if tr is not None:
        tr.write_line(line)
    else:
        sys.stderr.write(line + "\n")
