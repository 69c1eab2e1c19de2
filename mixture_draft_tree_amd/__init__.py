"""MI355X-native mixture draft tree (Multi-Future Drafting) hot path.

The compute path lives in `libmfdtree.so` (HIP kernels for gfx950 behind a C
ABI, declared in include/mfdtree.h).  `mixture_draft_tree_amd.mfdtree` is the
thin ctypes binding; `mixture_draft_tree_amd.synth` draws seeded inputs.
Importing this package loads nothing; importing `.mfdtree` loads the library
and raises if it has not been built.
"""
