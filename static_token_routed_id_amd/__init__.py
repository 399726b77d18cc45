"""libl3: the Large Lookup Layer (L3) forward / backward on MI355X (gfx950).

Submodules:
  workloads -- seeded synthetic inputs (no layer arithmetic)
  build     -- hipcc build of libl3.so
  _lib      -- ctypes binding of include/l3.h (raises if libl3.so is missing)
  layer     -- torch-owned workspaces and autograd glue around _lib
Importing the package itself loads nothing; import the submodule you need.
"""
