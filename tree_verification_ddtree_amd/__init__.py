"""MI355X-native DDTree tree-verify step: HIP kernels behind a C ABI
(include/ddtree.h, libddtree.so) and a thin ctypes binding."""
from .binding import *  # noqa: F401,F403
from .binding import lib, TreeBatch, layer_table, DDTError  # noqa: F401
