"""MI355X-native LLaMA pre-norm decoder block forward (HIP/gfx950).

The compute path is the C-ABI library libllama_mi355x.so built from csrc/;
`ops` marshals torch tensors into it. Importing the package loads nothing.
"""
