"""MI355X-native DSA sparse attention for the MTP verify step.

The compute path is the HIP library ``libdsa.so`` (built from ``csrc/``); the
Python names in :mod:`dsa_sparse_attention_amd.api` marshal torch device
tensors into its C ABI and nothing else.
"""
