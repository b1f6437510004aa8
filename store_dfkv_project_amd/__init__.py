"""libdfkv: the decode-step context-KV update of a DFlash / DSpark block drafter
on one MI355X (gfx950), behind a C ABI (include/dfkv.h).

``store_dfkv_project_amd.dfkv`` is the ctypes binding (same names as the C
entry points); ``store_dfkv_project_amd.build`` compiles ``libdfkv.so`` with
hipcc.  ``store_dfkv_project_amd.step`` sets up device buffers for a step from
host arrays (torch device memory only; all arithmetic runs in the kernels).
"""
__all__ = ["dfkv", "build", "step"]
