"""Swimba (Switch Mamba) parameter-space-MoE selective scan for MI355X (gfx950).

The computation lives in libswimba.so (hand-written HIP, C ABI in
include/swimba.h); ``swimba`` is its thin torch binding.
"""
from .swimba import (route, scan, scan_separate, scan_workspace_bytes, status_string,  # noqa: F401
                     step, SwimbaError)
