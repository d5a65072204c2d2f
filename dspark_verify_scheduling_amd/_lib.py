"""ctypes loader for libdspark.so, with the C signatures of include/dspark.h.

Loading never touches a GPU, so the library can be loaded (and its host-side
argument checks exercised) on a machine without one. If the library has not
been built, ``lib()`` raises: there is no fallback implementation.
"""

from __future__ import annotations

import ctypes
from ctypes import c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p
from pathlib import Path

_PKG = Path(__file__).resolve().parent
LIB_PATH = _PKG / "libdspark.so"
HOSTCHECK_PATH = _PKG / "libdspark_hostcheck.so"

OK, E_INVALID, E_UNSUPPORTED, E_WORKSPACE, E_LAUNCH = 0, 1, 2, 3, 4
F32, BF16 = 0, 1
IN_CONF_LOGITS, IN_COND, IN_SURVIVAL = 0, 1, 2
DATA_BAD_COST, DATA_BAD_CONF, DATA_BAD_LENS, DATA_BAD_LOGITS = 1, 2, 4, 8
MAX_GAMMA, MAX_CANDIDATES, MAX_BATCH, MAX_TIERS, MAX_VOCAB = 64, 8192, 8192, 32, 262144
MAX_SPS_PROBES = 512
STS_MAX_GRID, STS_MAX_BINS, STS_MAX_RECORDS = 128, 64, 4194304
COST_ADDITIVE, COST_SPS1D = 0, 1


class PlanOptions(ctypes.Structure):
    """dspark_plan_options of include/dspark.h."""
    _fields_ = [("cost_mode", c_int), ("sps_m", c_void_p), ("sps", c_void_p),
                ("sps_len", c_int32), ("align_to_tier", c_int32)]


# name -> (restype, argtypes), mirroring include/dspark.h
SIGNATURES = {
    "dspark_plan": (c_int, [
        c_int32, c_int32, c_int, c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32,
        c_int32, c_float, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p]),
    "dspark_plan_pack": (c_int, [
        c_int32, c_int32, c_int, c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32,
        c_int32, c_float, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dspark_plan_pack_ex": (c_int, [
        c_int32, c_int32, c_int, c_void_p, c_void_p, c_int32, c_int32, c_float, c_int32,
        c_int32, c_float, c_void_p, c_int32, c_void_p, c_int32, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dspark_pack": (c_int, [
        c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "dspark_accept": (c_int, [
        c_int32, c_int32, c_int32, c_int, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_size_t, c_void_p]),
    "dspark_accept_noalloc": (c_int, [
        c_int32, c_int32, c_int32, c_int, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p]),
    "dspark_cap_accept": (c_int, [
        c_int32, c_int32, c_int32, c_int, c_void_p, c_int64, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_size_t, c_void_p]),
    "dspark_scatter_to_strided": (c_int, [
        c_int32, c_int32, c_void_p, c_int32, c_void_p, c_int64, c_void_p, c_int64, c_int64,
        c_void_p, c_void_p]),
    "dspark_accept_workspace_size": (c_size_t, [c_int32, c_int32, c_int]),
    "dspark_accept_sampling": (c_int, [
        c_int32, c_int32, c_int32, c_int, c_void_p, c_int64, c_int32, c_void_p, c_void_p,
        c_int64, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dspark_accept_sampling_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int]),
    "dspark_sts_fit": (c_int, [
        c_int32, c_int32, c_void_p, c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
        c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t, c_void_p]),
    "dspark_sts_workspace_size": (c_size_t, [c_int32, c_int32, c_int32, c_int32]),
    "dspark_tv_accept": (c_int, [
        c_int32, c_int32, c_int32, c_int, c_void_p, c_int64, c_void_p, c_int64, c_int32,
        c_void_p, c_void_p, c_void_p]),
    "dspark_status_str": (ctypes.c_char_p, [c_int]),
    "dspark_last_error": (ctypes.c_char_p, []),
    "dspark_version": (c_int32, []),
}

_lib = None
_hostcheck = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not LIB_PATH.exists():
            raise RuntimeError(
                f"{LIB_PATH} is not built; run `python -m dspark_verify_scheduling_amd.build` "
                "(or __graft_entry__.build())")
        handle = ctypes.CDLL(str(LIB_PATH))
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def hostcheck() -> ctypes.CDLL:
    """Host-only build of the device sigmoid (CPU tests of its logic)."""
    global _hostcheck
    if _hostcheck is None:
        if not HOSTCHECK_PATH.exists():
            raise RuntimeError(f"{HOSTCHECK_PATH} is not built")
        handle = ctypes.CDLL(str(HOSTCHECK_PATH))
        handle.dspark_hostcheck_sigmoid.restype = None
        handle.dspark_hostcheck_sigmoid.argtypes = [c_void_p, c_void_p, c_void_p, c_int64, c_int]
        _hostcheck = handle
    return _hostcheck


def last_error() -> str:
    return lib().dspark_last_error().decode()


def status_str(st: int) -> str:
    return lib().dspark_status_str(st).decode()


class DsparkError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} -> {status_str(status)}: {last_error()}")


def check(fn: str, status: int) -> None:
    if status != OK:
        raise DsparkError(fn, status)


__all__ = ["lib", "hostcheck", "check", "DsparkError", "SIGNATURES", "c_double"]
