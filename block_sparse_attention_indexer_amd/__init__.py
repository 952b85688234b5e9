"""Block-sparse paged attention (indexer + sparse attention) for MI355X.

The compute lives in the HIP library ``lib/libmsa.so`` (entry points declared
in ``include/msa.h``); ``binding`` marshals torch tensors into its C ABI.
Importing this package does not load the library; the first call does.
"""
