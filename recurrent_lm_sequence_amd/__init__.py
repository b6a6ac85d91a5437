"""MI355X-native causal Taylor linear attention (BASED prefill, JRT-RNN prefix
prefill, state-passing decode) behind a C-ABI HIP library.

Importing the package loads nothing; ``recurrent_lm_sequence_amd.based_la``
loads the compiled library (and fails loudly if it is missing).
"""
