"""tensor_all_reduce_amd -- one MI355X's share of a flash all-reduce, as hand-written HIP for gfx950.

The kernels live in ``libfc.so`` (C ABI: ``include/fc.h``); ``tensor_all_reduce_amd.fc_*`` are thin ctypes
bindings of the same names, loaded on first use.  ``datagen`` (seeded synthetic inputs and the five named
workloads), ``bytes_model``, ``schedule`` and ``selector`` import without loading the library.
"""
_BINDINGS = ("fc_quantize", "fc_reduce_shard", "fc_gather_dequant", "fc_reduce_rmsnorm", "fc_ll_unpack_reduce",
             "fc_ll_pack", "fc_ll_gather", "fc_ll_poll_unpack_reduce", "fc_flag_unpack_reduce", "fc_flag_pack",
             "fc_reduce_shard_norm", "fc_copy", "fc_abi_version", "FcError", "lib")


def __getattr__(name):
    if name in _BINDINGS:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
