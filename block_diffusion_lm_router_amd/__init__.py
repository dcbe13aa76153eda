"""MI355X-native hot path of a block-diffusion LM denoising step (hand-written HIP, gfx950).

The compute lives in libbdstep.so (C ABI in include/bdstep.h).  ``binding`` marshals
torch GPU tensors to it; ``workloads`` makes seeded synthetic inputs.  Importing this
package loads nothing; the first call into the binding loads the library and fails
loudly if it has not been built.
"""

import importlib

__all__ = ["workloads", "binding"]


def __getattr__(name):
    if name == "binding":
        return importlib.import_module(__name__ + "._binding")
    if name == "workloads":
        return importlib.import_module(__name__ + ".workloads")
    raise AttributeError(name)
