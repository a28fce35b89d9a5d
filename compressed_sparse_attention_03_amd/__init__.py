"""MI355X-native hybrid compressed attention (CSA / HCA) forward pass.

The compute path is the HIP/C-ABI library ``libcsa.so`` built from ``csrc/``; this package only
marshals torch tensors into its calls (``ops``).  Importing the package does not load the library;
the first op call does, and raises if the library is missing.
"""
__all__ = ["ops", "inputs"]
