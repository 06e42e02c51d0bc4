"""Refined low-bit decode step (nested refinement bits on selected channels and
tokens) for AMD MI355X (gfx950).

The compute lives in ``libstrataflux.so`` (hand-written HIP, C ABI declared in
``include/strataflux.h``); ``binding`` wraps it with ctypes.  Importing this
package loads nothing: ``binding.lib()`` loads the library on first use and raises
if it has not been built.
"""

__all__ = ["binding", "inputs"]
