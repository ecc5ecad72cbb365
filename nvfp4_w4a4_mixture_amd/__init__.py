"""MI355X-native routed-expert MoE layer with NVFP4 W4A4 experts.

The computation lives in the HIP library ``lib/libmoe_nvfp4.so`` (C ABI in
``include/moe_nvfp4.h``); ``ops`` binds each entry point under its own name,
``layer.NVFP4MoELayer`` composes them into one layer forward.  Build with
``python -m nvfp4_w4a4_mixture_amd.build``.

Importing ``ops``/``layer`` loads the library and fails loudly if it is not
built; there is no CPU path.
"""

__version__ = "0.1.0"


def __getattr__(name):
    if name in ("ops", "layer", "workload_io"):
        import importlib

        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
