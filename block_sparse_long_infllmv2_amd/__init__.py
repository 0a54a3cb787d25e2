"""InfLLM v2 block-sparse attention for MI355X (gfx950).

The compute path is libinfllmv2.so (hand-written HIP kernels behind a C ABI,
include/infllmv2.h).  `binding` wraps its calls for torch tensors, `pipeline`
strings them into prefill / decode / tree-verification steps, and `workloads`
draws seeded synthetic inputs.  Importing `binding` or `pipeline` loads the
library and raises if it has not been built.
"""
import importlib

__all__ = ["binding", "pipeline", "workloads", "build"]


def __getattr__(name):
    if name in __all__:
        return importlib.import_module(f".{name}", __name__)
    raise AttributeError(name)
