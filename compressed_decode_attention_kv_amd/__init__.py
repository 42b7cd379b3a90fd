"""MI355X-native TurboQuant-style KV-cache compression: packed-cache write
(quantize) and decode attention straight from the packed cache.

Submodules:
  tq     -- ctypes binding of the C-ABI library libtq.so (loads it on import
            and raises if it is missing: there is no CPU fallback);
  synth  -- seeded synthetic workloads (inputs only, no method arithmetic);
  build  -- compiles libtq.so for gfx950 with hipcc.
"""
