"""MI355X (gfx950) microscaled FP4 quantisation: a C-ABI HIP library (libmxq.so)
with a thin Python binding (``mxq``) and seeded synthetic workloads
(``workloads``). Importing the package loads nothing; the library is loaded on
first use of a binding function."""
