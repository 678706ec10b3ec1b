"""MI355X-native batched speculative-decoding verification with a paged KV cache.

The compute path is a C-ABI HIP library (``libspecdec.so``, built for gfx950 from
``csrc/``); ``binding`` marshals torch tensors into it. ``synth`` draws seeded synthetic
inputs. Importing the package does not load the library; the first call into the binding
does, and raises if the library has not been built.
"""

__all__ = ["binding", "synth"]
