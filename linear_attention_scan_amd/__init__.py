"""libfwmem: the fast-weight matrix-memory scan on MI355X (gfx950).

Importing the package loads nothing; ``linear_attention_scan_amd.fwmem`` holds the
ctypes binding of the C-ABI library and loads it on first use.
"""
