"""Loader of libspecverify.so (ctypes).  Fails loudly when the library is not
built: there is no fallback path."""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libspecverify.so")

_c = ctypes
_P = _c.c_void_p
_I32 = _c.c_int32
_I64 = _c.c_int64
_U64 = _c.c_uint64
_SZ = _c.c_size_t

_SIGNATURES = {
    "sv_version": (_c.c_int, []),
    "sv_strerror": (_c.c_char_p, [_c.c_int]),
    "sv_workspace_size": (_SZ, [_c.c_int, _I32, _I32, _I32, _c.c_int]),
    "sv_verify_window": (_c.c_int, [_P, _I64, _P, _I64, _c.c_int, _P, _P, _I32, _I32, _I32,
                                    _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sv_verify_window_noalloc": (_c.c_int, [_P, _I64, _P, _I64, _c.c_int, _P, _P, _I32, _I32, _I32,
                                            _U64, _U64, _P, _P, _P, _P, _P, _P, _P]),
    "sv_verify_window_early_exit": (_c.c_int, [_P, _I64, _P, _I64, _c.c_int, _P, _P, _I32, _I32, _I32,
                                               _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sv_verify_window_part": (_c.c_int, [_c.c_int, _P, _I64, _P, _I64, _c.c_int, _P, _P, _I32, _I32,
                                         _I32, _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sv_verify_greedy": (_c.c_int, [_P, _I64, _c.c_int, _P, _P, _I32, _I32, _I32, _P, _P,
                                    _P, _SZ, _P]),
    "sv_tree_max_depth": (_I32, [_P, _I32]),
    "sv_verify_tree": (_c.c_int, [_P, _P, _c.c_int, _P, _P, _I32, _I32, _I32, _c.c_int,
                                  _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sv_rollback": (_c.c_int, [_P, _P, _I32, _I32, _I32, _I32, _P, _I64, _P, _I32, _P]),
    "sv_verify_window_lmhead": (_c.c_int, [_P, _P, _I32, _P, _P, _I32, _P, _P, _I32, _I32, _I32,
                                           _U64, _U64, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]),
    "sv_probe_blocks": (_I32, [_SZ]),
    "sv_probe_read": (_c.c_int, [_P, _SZ, _P, _P]),
}

EXPORTED = tuple(_SIGNATURES)

_lib = None


def hip_runtime_paths():
    """Distinct libamdhip64 files mapped into this process."""
    paths = set()
    with open("/proc/self/maps") as f:
        for line in f:
            if "libamdhip64" in line:
                paths.add(os.path.realpath(line.split()[-1]))
    return paths


def lib():
    """The loaded library with argument types declared."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is not built; run `python -m draft_token_verification_06_amd.build` "
            "(there is no CPU fallback)")
    import torch  # noqa: F401  -- torch's HIP runtime must be the one the library binds to

    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = hip_runtime_paths()
    if len(runtimes) > 1:
        raise RuntimeError(f"two HIP runtimes are mapped into this process: {sorted(runtimes)}")
    _lib = handle
    return _lib
