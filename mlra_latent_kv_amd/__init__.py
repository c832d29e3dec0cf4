"""MI355X-native MLA / MLRA-4 latent-KV decode attention.

Submodules are imported on demand so that the seeded input generator
(``mlra_latent_kv_amd.inputs``, NumPy only) can be used without loading the
HIP library or torch:

* ``mlra_latent_kv_amd.inputs``  - workload table and seeded synthetic inputs.
* ``mlra_latent_kv_amd.binding`` - ctypes binding of ``libmla_decode.so``
  (argument marshalling only; every step of the decode runs in HIP kernels).
* ``mlra_latent_kv_amd.build``   - hipcc build of the shared library.
"""

__all__ = ["inputs", "binding", "build"]
