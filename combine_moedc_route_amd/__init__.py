"""libmoedc: MoE token routing, INT8 dispatch and combine on AMD MI355X.

``combine_moedc_route_amd.moedc`` is the ctypes binding over the HIP
library (``libmoedc.so``, built from ``csrc/``); ``workloads`` draws the
seeded synthetic inputs.  The library is loaded on first use; a missing
library raises instead of falling back to anything else.
"""
from . import moedc, workloads  # noqa: F401

__all__ = ["moedc", "workloads"]
