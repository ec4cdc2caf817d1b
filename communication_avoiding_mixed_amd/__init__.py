"""MI355X-native mixed-precision communication-avoiding SGD for generalized
linear models (logistic, least-squares, Poisson regression).

The compute path is the HIP library ``libcasgd.so`` behind the C ABI declared
in ``include/casgd.h``; :mod:`.binding` marshals torch device tensors into it.
Importing the package loads nothing native: the library is opened on first
use of the binding and raises if it has not been built.
"""

__all__ = ["binding", "synth"]
