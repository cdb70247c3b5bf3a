"""MI355X-native (gfx950) per-frame forward of the PersonaPlex/Moshi temporal transformer
and its depth transformer, behind the C-ABI library libpp.so.

Importing the package loads nothing; `personaplex_temporal_transformer_amd.pp` holds
the ctypes binding, which loads libpp.so and fails loudly if it is missing.
"""
