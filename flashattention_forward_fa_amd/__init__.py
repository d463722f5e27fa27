"""MI355X-native FlashAttention forward: Python binding over the C-ABI library libfa.

The binding only marshals arguments; every step of the attention forward runs
in the HIP kernels of ``libfa.so``.  The library is loaded on first use and a
missing or unloadable library raises -- there is no CPU fallback.
"""
