"""GPT-2 training step on MI355X (gfx950): C-ABI library libgpt2.so with
hand-written HIP kernels, and its ctypes binding (decoder_only_transformer_03_amd.gpt2).

The binding loads the library lazily on first use and raises if it has not
been built (python -m decoder_only_transformer_03_amd.build)."""
