"""GPT-2 training step (forward, backward, AdamW) as hand-written HIP kernels for MI355X (gfx950).

The compute lives in libgpt2.so (C ABI in include/gpt2.h and include/gpt2_ops.h); `binding`
marshals arguments to it with ctypes. `synth` holds the seeded synthetic-input generators.
Nothing is imported eagerly, so importing the package never touches the GPU.
"""
