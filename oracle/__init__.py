"""CPU oracle for the DFlash block-diffusion draft pass.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or
links anything in this directory; only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP path (the only common module is the seeded input generator, which
holds none of the method's arithmetic).

* ``dflash_oracle`` — the draft pass as a plain numpy float64 function.
* ``brute``         — an independent scalar-loop evaluation for tiny shapes,
                      used to pin ``dflash_oracle``.
* ``sampling``      — sampled drafts (temperature > 0) and lossless
                      verification, with the Philox4x64-10 generator both
                      sides implement.
"""
