"""MI355X (gfx950) q4 MoE-layer hot path.

``libtf.so`` (HIP kernels + C ABI, ``include/tf.h``) does all the work; this
package only builds it (``build.py``) and binds it (``_lib.py`` for ctypes
declarations, ``api.py`` for torch-tensor marshalling).
"""
import importlib

from ._lib import (TF_FLAG_ID_RANGE, TF_FLAG_ID_REPEAT, TF_GELU_ERF, TF_GELU_TANH,  # noqa: F401
                   TFError, exported_names, load)


def __getattr__(name):
    # the torch-dependent binding is imported on first use
    api = importlib.import_module(".api", __name__)
    return api if name == "api" else getattr(api, name)
