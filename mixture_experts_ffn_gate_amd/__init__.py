"""MI355X-native MoE FFN layer (Nemotron-H style): HIP kernels behind a C ABI.

``moe_layer`` holds the ctypes binding of ``libmoe_layer.so``; ``workloads``
draws seeded synthetic inputs. Importing the package loads nothing native;
the binding loads the library on first use and raises if it is missing.
"""
