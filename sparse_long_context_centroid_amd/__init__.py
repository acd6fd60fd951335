"""CommunityKV sparse decode path for MI355X (gfx950).

`binding` wraps the C-ABI library libckv.so (HIP kernels); `inputs` draws the
seeded synthetic workloads.  Importing the package loads neither.
"""
