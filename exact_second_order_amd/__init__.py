"""MI355X (gfx950) exact backward-over-backward of softmax attention.

The compute path is the HIP library libflashbob.so behind the C ABI of
include/flashbob.h; `flashbob` is its thin ctypes binding. Importing the
package does not load the library; the first call does, and fails loudly if
it has not been built.
"""

from .flashbob import FlashBoBError, bob, rowstats, workspace_bytes, load_library  # noqa: F401
