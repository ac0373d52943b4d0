"""The C ABI from C: tests/c_abi_client.c, compiled as C11 with gcc against
include/sv.h alone, links every entry point the header declares and drives
the host-only paths (version, error strings, workspace sizes, tree depths,
argument checks).  Its results must equal the ones the Python side gets
through ctypes; no GPU is needed."""
import os
import shutil
import subprocess

import pytest

from draft_token_verification_06_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "draft_token_verification_06_amd")
ROCM_INCLUDE = "/opt/rocm/include"


@pytest.fixture(scope="module")
def client_output(tmp_path_factory):
    gcc = shutil.which("gcc")
    lib = os.path.join(PKG, "libspecverify.so")
    if not gcc or not os.path.isdir(ROCM_INCLUDE) or not os.path.exists(lib):
        pytest.skip("needs gcc, the ROCm headers and the built library")
    exe = str(tmp_path_factory.mktemp("c_abi") / "client")
    cmd = [gcc, "-std=c11", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__", "-I", ROCM_INCLUDE,
           "-I", os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "c_abi_client.c"), "-o", exe,
           "-L", PKG, "-lspecverify", f"-Wl,-rpath,{PKG}"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    run = subprocess.run([exe], check=True, capture_output=True, text=True, timeout=120)
    out = {}
    for line in run.stdout.splitlines():
        key, _, val = line.partition(" ")
        out.setdefault(key, []).append(val)
    return out


def _header_functions():
    names = []
    for line in open(os.path.join(ROOT, "include", "sv.h")):
        for kind in ("int ", "size_t ", "const char *", "int32_t "):
            if line.startswith(kind + "sv_") or line.startswith(kind + "*sv_"):
                names.append(line[len(kind):].split("(")[0].lstrip("*"))
    return names


def test_every_declared_function_links_from_c(client_output):
    linked = {v.split()[0]: v.split()[1] for v in client_output["linked"]}
    assert sorted(linked) == sorted(_header_functions())
    assert set(linked.values()) == {"1"}


def test_host_paths_agree_with_ctypes(client_output):
    L = _lib.lib()
    assert int(client_output["version"][0]) == L.sv_version()
    for v in client_output["strerror"]:
        code, text = v.split(" ", 1)
        assert text == L.sv_strerror(int(code)).decode()
    sizes = {"ws_window": (0, 256, 8, 128256, 1), "ws_greedy": (1, 256, 8, 128256, 1),
             "ws_tree": (2, 4, 41, 50257, 2), "ws_lmhead": (3, 256, 8, 128256, 1), "ws_bad_dtype": (0, 4, 4, 1000, 7)}
    for key, args in sizes.items():
        assert int(client_output[key][0]) == L.sv_workspace_size(*args)
    assert int(client_output["ws_bad_dtype"][0]) == 0
    assert int(client_output["depth_chain"][0]) == 4 and int(client_output["depth_bushy"][0]) == 2
    assert int(client_output["depth_bad"][0]) == -4
    assert int(client_output["probe_blocks"][0]) == L.sv_probe_blocks(1 << 30)


def test_argument_checks_from_c(client_output):
    want = {"window_null": -1, "window_dtype": -2, "noalloc_null": -1, "part_bad": -1, "early_null": -1,
            "greedy_null": -1, "tree_bad_parent": -4, "rollback_null": -1, "probe_null": -1, "lmhead_null": -1}
    for key, status in want.items():
        assert int(client_output[key][0]) == status, key
