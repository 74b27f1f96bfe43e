"""MI355X-native backward pass of a GPT-2 linear layer.

``linear_layer_backward_amd.mmb`` binds the HIP library (``libmmb.so``) that
computes dinp += dout.W, dweight += dout^T.inp and dbias = column sums of
dout (optionally with stochastically rounded bf16 dweight/dbias), the forward
product out = inp.W^T + bias, and the LayerNorm backward of the same model;
``linear_layer_backward_amd.workloads`` generates seeded synthetic inputs.
Importing this package loads nothing: the binding loads the library when
``mmb`` is imported and raises if it is missing.
"""
