"""MI355X-native causal-prefill sequence mixer (full, sliding-window, differential) with a
Latin-square layer scheduler, behind the C-ABI library ``libmixer.so``.

The binding in ``mixer`` loads the HIP library on first use and fails loudly when it is
missing; ``synth`` (seeded inputs) has no dependency on it.
"""
