"""A checking emulator for the library's own gfx950 kernels, run on the CPU.

The library's host code (libqkmla.so, unchanged) is loaded against a small
stand-in for the HIP runtime (runtime.c) whose kernel launches are executed
instruction by instruction from the device assembly that the build leaves in
``mla_latent_decode_amd/_build`` (``-save-temps``; the code object in the
library is assembled from exactly these files).  Device memory is ordinary
process memory registered with the emulator.

What a run checks, beyond the numbers it produces:
  * every global, LDS, scratch and kernel-argument access lies inside the
    allocation it belongs to;
  * vector-memory, LDS and scalar-memory results land only at the
    ``s_waitcnt`` that retires them: reading or overwriting a destination
    register earlier is reported, as is touching LDS bytes that an in-flight
    direct global->LDS load will write;
  * LDS accesses of different wavefronts between two barriers do not race;
  * inside inline asm, a vector-memory instruction does not read an SGPR that
    a VALU instruction wrote fewer than five wait states before, and an
    LDS-DMA load is not issued in the wait state right after an M0 write
    (the compiler guarantees both for the code it schedules itself).

Fidelity: integer and bit operations are exact; fp32 add/mul round once in
fp32; fused operations and transcendental instructions are evaluated in
float64 and rounded to float32 (within one ulp of the hardware's), MFMA sums
in float64.  Results are compared with the fp64 oracle at the same tolerances
as the GPU tests.  It is a test instrument, never a fallback: nothing in the
library imports it.
"""
