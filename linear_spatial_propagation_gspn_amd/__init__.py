"""MI355X-native GSPN 2D line-scan linear propagation.

`gspn` is the binding of libgspn (include/gspn.h): the C ABI's calls under
the same names, and `gspn4`, the four-direction propagation as a
differentiable op.  `build` compiles libgspn.so in-tree for gfx950;
`workloads` draws the seeded synthetic inputs.
"""
