"""KVarN KV-cache block quantisation and packed decode attention for MI355X (gfx950).

The compute path lives in the HIP library ``libkvarn.so`` (sources under
``csrc/``); ``kvarn`` is its thin ctypes binding.
"""
