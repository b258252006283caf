"""MI355X-native (gfx950) TDP upscale step: C-ABI library libtdp.so + binding.

``tdp``   ctypes binding, one function per entry point of include/tdp.h
``step``  device-resident runner of a whole step (imports torch)
``_build`` in-tree build of libtdp.so with hipcc
"""
from . import tdp  # noqa: F401
