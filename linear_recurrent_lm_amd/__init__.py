"""MI355X-native WKV-7 recurrence (RWKV-7): a C-ABI HIP library for gfx950.

`linear_recurrent_lm_amd.wkv7` is the thin Python binding over libwkv7.so;
`linear_recurrent_lm_amd.synth` draws the seeded synthetic inputs. Importing
the package itself loads nothing.
"""

__all__ = ["wkv7", "synth"]
