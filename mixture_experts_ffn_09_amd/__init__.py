"""MI355X (gfx950) sparse-MoE FFN layer forward.

The compute path is the HIP library ``libmoe_ffn.so`` (C ABI declared in
``include/moe_ffn.h``); ``mixture_experts_ffn_09_amd.moe`` is its thin ctypes
binding.  Importing the package loads nothing: the library is opened on first
use of the binding and a missing library is an error, never a fallback.
"""
