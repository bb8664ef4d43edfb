"""attnq: MI355X-native NVFP4 weight-only decode projections.

The compute path is the HIP library ``libattnq.so`` (built from ``csrc/``);
``nvfp4_weight_only_rtn_amd.attnq`` is its thin ctypes binding. Importing the
package itself loads nothing, so the seeded input generators in
``nvfp4_weight_only_rtn_amd.inputs`` can be used without the library.
"""
