"""MI355X-native forward pass of a Mixture-of-Transformers world action model.

Two transformer experts share attention: a video expert runs once per
observation and publishes a per-block key/value cache; an action expert
attends, in block i, over its own keys/values concatenated with video block
i's, and is integrated by a flow-matching Euler update.  The compute path is
a C-ABI HIP library (``libwam.so``, declared in ``include/wam.h``); the Python
side only marshals arguments (``binding``) and draws seeded synthetic inputs
(``workload``).

Importing this package loads nothing native; ``binding.load()`` does.
"""
__all__ = ["workload", "binding"]
