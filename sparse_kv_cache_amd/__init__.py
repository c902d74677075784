"""Fathom plane-prefix key scan for MI355X (gfx950).

Submodules:
  fathom  -- ctypes binding of libfathom.so (imports fail loudly if unbuilt)
  synth   -- seeded synthetic inputs
  build   -- hipcc build of libfathom.so
Importing the package itself loads nothing.
"""
