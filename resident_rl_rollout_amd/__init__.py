"""GPU-resident PPO rollout hot path for AMD Instinct MI355X (gfx950).

The compute lives in librl.so (hand-written HIP kernels behind the C ABI of include/rl.h);
``binding`` marshals torch tensors into it, ``inputs`` draws the seeded synthetic workloads and
``build`` compiles the library. Importing the package loads nothing; the binding loads the library on
first use and raises if it is missing.
"""
