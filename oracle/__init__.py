"""Plain CPU oracle for quantized-KV decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute anything in this package: only the test suite, the smoke check of
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` use it.  It
shares no code with the HIP library (no kernels, headers, helpers, tables or
pre/post-processing); the only module both sides use is ``synth``, which holds
seeded input generators and none of the method's arithmetic.

Every function here is written out from the definitions on the pages, slowly
and in the pages' order:

* codec.py     symmetric absmax rule, grouping axes, bit packing, dequant,
               bf16 rounding
* salience.py  MixKVQ channel salience and precision classes
* cache.py     sink / quantized groups / full-precision residual tail
* attention.py float64 stable-softmax attention over dequantized K, V
* bytes_model.py  payload byte accounting
* rotation.py  key-only Walsh-Hadamard rotation (fast transform in float32)
* rope.py      rotary embedding of pre-RoPE cached keys at decode
* nuq.py       non-uniform (codebook) datatype with per-vector dense-and-sparse
               outliers
* qjl.py       value-side 1-bit residual sketch of the KQV scheme

Parity status: every function is pinned by ``tests/test_oracle_*.py`` against
values printed on the pages, closed forms, invariants, brute force or library
routines; none is "parity unpinned".
"""

from . import codec, salience, cache, attention, bytes_model, rotation, rope, nuq, qjl  # noqa: F401,E501
