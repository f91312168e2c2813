"""MI355X-native (gfx950) DeepSeekMoE layer forward.

The compute path is the C-ABI library ``libmoe.so`` built from the HIP
sources under ``csrc/``; ``binding`` wraps its entry points with ctypes.
Importing the package does not load the library; ``binding.lib()`` does, and
raises if it has not been built.
"""
from .configs import CONFIGS, LayerConfig  # noqa: F401
