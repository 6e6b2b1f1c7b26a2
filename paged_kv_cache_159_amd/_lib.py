"""Loader of libpaged_kv.so and ctypes signatures of its C ABI (include/paged_kv.h).

Fails loudly: there is no CPU or PyTorch fallback. torch is imported first so
that the library binds to the HIP runtime torch already loaded (one runtime per
process); the loader checks that only one copy is mapped.
"""

from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libpaged_kv.so")

# Names declared in include/paged_kv.h, in declaration order.
EXPORTS = (
    "pkv_version",
    "pkv_status_string",
    "paged_attention_workspace_size",
    "paged_attention_decode",
    "paged_attention_decode_noalloc",
    "paged_attention_decode_partitions",
    "paged_attention_decode_merge",
    "paged_attention_grouped_workspace_size",
    "paged_attention_decode_grouped",
    "paged_attention_prefill",
    "reshape_and_cache",
    "copy_blocks",
    "swap_blocks",
    "swap_blocks_dma",
    "swap_blocks_staged",
)

PKV_F16, PKV_BF16 = 0, 1
STATUS = {0: "PKV_OK", -1: "PKV_ERR_NULL", -2: "PKV_ERR_SHAPE", -3: "PKV_ERR_UNSUPPORTED",
          -4: "PKV_ERR_WORKSPACE", -5: "PKV_ERR_LAUNCH", -6: "PKV_ERR_ALIGN", -7: "PKV_ERR_MEMORY",
          -8: "PKV_ERR_DATA", -9: "PKV_ERR_SCRATCH"}
# Bytes of paged_attention_decode_noalloc's fixed per-device scratch array.
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None

_p = ctypes.c_void_p
_i = ctypes.c_int
_f = ctypes.c_float
_z = ctypes.c_size_t

_SIGNATURES = {
    "pkv_version": (_i, []),
    "pkv_status_string": (ctypes.c_char_p, [_i]),
    "paged_attention_workspace_size": (_z, [_i, _i, _i, _i, _i]),
    "paged_attention_decode": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _z, _p]),
    "paged_attention_decode_noalloc": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p]),
    "paged_attention_decode_partitions": (_i, [_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _f, _i,
                                               _p, _z, _p]),
    "paged_attention_decode_merge": (_i, [_p, _p, _i, _i, _i, _i, _i, _i, _p, _z, _p]),
    "paged_attention_grouped_workspace_size": (_z, [_i, _i, _i, _i, _i]),
    "paged_attention_decode_grouped": (_i, [_p, _p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i,
                                            _f, _i, _p, _z, _p]),
    "paged_attention_prefill": (_i, [_p, _p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _f,
                                     _i, _p]),
    "reshape_and_cache": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p]),
    "copy_blocks": (_i, [_p, _p, _p, _i, _i, _i, _i, _i, _i, _p]),
    "swap_blocks": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]),
    "swap_blocks_dma": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p]),
    "swap_blocks_staged": (_i, [_p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _i, _p, _z, _p]),
}


class PagedKVError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {STATUS.get(status, status)}: {status_string(status)}")


def _hip_runtimes_mapped() -> set:
    paths = set()
    try:
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    paths.add(os.path.realpath(line.split()[-1]))
    except OSError:
        pass
    return paths


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m paged_kv_cache_159_amd.build` "
                           "(or __graft_entry__.build()) first. There is no fallback path.")
    import torch  # noqa: F401  (binds the library to torch's HIP runtime)
    handle = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(handle, name)
        fn.restype = res
        fn.argtypes = args
    runtimes = _hip_runtimes_mapped()
    if len(runtimes) > 1:
        raise RuntimeError(f"more than one HIP runtime mapped in this process: {sorted(runtimes)}")
    _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().pkv_status_string(int(status)).decode()


def check(fn: str, status: int) -> None:
    if status != 0:
        raise PagedKVError(fn, status)
