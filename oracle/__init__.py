"""CPU oracle for the paged quantized-KV decode step.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(the C-ABI library and its Python binding) never calls it, and it shares no
code, tables or helpers with that path.

What it computes (mjolnir-kernel PyPI project page / sdist README, section
"What it does", steps 1-4; wheel listing mjolnir/runner.py,
``T5DecodeRunner.plan`` and ``T5DecodeRunner.run``):

* ``plan``      the split-KV plan (an integer schedule), written from its
                definition;
* ``qquant``    dynamic e4m3 quantization of Q per (sequence, KV head), in
                fp32 with IEEE round-to-nearest division, exactly as the pages
                define it;
* ``formats``   the e4m3 / e2m3 / e3m2 / e2m1 codecs and the 6- and 4-bit
                bitstream packers, each from the published format definition;
* ``attention`` exact attention over the gathered, dequantized pages in fp64
                (softmax(Q K^T * scale) V), its split partials and their
                log-sum-exp merge;
* ``kvwrite``   the KV-cache write of new rows through a slot mapping
                (wheel listing mjolnir/backend.py, ``do_kv_cache_update``);
* ``draft``     the draft-step advance (slots of the appended tokens, the
                lengths grown in place) of multi-step draft decoding.

Parity status of each function is stated in its docstring; every function
here is pinned by the ``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.
"""

from . import formats, plan, qquant, attention, kvwrite, draft  # noqa: F401
