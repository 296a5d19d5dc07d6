import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


import shutil  # noqa: E402
import subprocess  # noqa: E402

import pytest  # noqa: E402


@pytest.fixture(scope="session")
def c_client(tmp_path_factory):
    """tests/c_abi_client.c compiled with gcc and linked against the built
    libzs.so and the HIP runtime (no torch, no Python in the client)."""
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lib_dir = os.path.join(ROOT, "edge_node_scatter_amd")
    if not os.path.exists(os.path.join(lib_dir, "libzs.so")):
        raise RuntimeError("libzs.so is not built (run __graft_entry__.build())")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    exe = str(tmp_path_factory.mktemp("c_client") / "c_abi_client")
    subprocess.check_call([gcc, "-std=c11", "-O2", "-Wall", "-Werror",
                           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"),
                           os.path.join(ROOT, "tests", "c_abi_client.c"), "-o", exe,
                           "-L", lib_dir, "-lzs", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
                           f"-Wl,-rpath,{lib_dir}", f"-Wl,-rpath,{os.path.join(rocm, 'lib')}"])
    return exe
