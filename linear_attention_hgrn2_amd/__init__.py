"""HGRN2 gated linear recurrence with outer-product state expansion, on AMD
MI355X (gfx950).

The computation lives in ``libhgrn2.so`` (C ABI in ``include/hgrn2.h``, HIP
kernels in ``csrc/``); this package is its thin Python binding:

  fwd(q, k, v, log_f, h0=None, chunk=64)        chunked forward
  bwd(q, k, v, log_f, dy, h0, dht, states)      chunked backward
  bwd_noalloc(...)                              the same without a workspace (the library's own scratch)
  fwd_chunk / bwd_adjoint / bwd_chunk           the single launches fwd and bwd are made of
  fwd_tied / bwd_tied / ... / decode_step_tied  the same with tied gates, k = 1 - exp(log_f)
  fwd_gate / bwd_gate / decode_step_gate        gate from its pre-activation z and a lower bound:
                                                f = lb + (1 - lb) sigmoid(z), k = 1 - f
  decode_step(q, k, v, log_f, state)            one recurrent step, in place
  fwd_scalar / bwd_scalar / decode_step_scalar  one decay per head, log_a [B, T, H]
  hgrn1_fwd / hgrn1_bwd                         the HGRN1 elementwise recurrence over [B, T, C]
  hgrn2_chunk(q, k, v, log_f, h0, chunk)        autograd wrapper

Every call with token outputs takes out_dtype: None keeps the input dtype;
torch.float32 with bfloat16 inputs writes y and the gradients as float32
(HGRN2_OUT_F32).
"""
from ._binding import (BF16, F32, OUT_F32, HGRN2Chunk, HGRN2Error, LIB_PATH, NOALLOC_SCRATCH_BYTES, adjoints_shape, bwd,
                       bwd_adjoint, bwd_noalloc,
                       bwd_chunk, bwd_chunk_tied, bwd_gate, bwd_scalar, bwd_tied, decode_step, decode_step_gate,
                       decode_step_scalar, decode_step_tied, fwd_scalar, fwd, fwd_chunk, fwd_chunk_tied, fwd_gate, fwd_tied, hgrn1_bwd, hgrn1_fwd,
                       hgrn1_states_shape, hgrn2_chunk, lib, num_chunks, states_shape, supported)

__all__ = ["fwd", "bwd", "bwd_noalloc", "NOALLOC_SCRATCH_BYTES", "fwd_chunk", "bwd_adjoint", "bwd_chunk", "adjoints_shape", "decode_step",
           "fwd_tied", "bwd_tied", "fwd_chunk_tied", "bwd_chunk_tied", "decode_step_tied",
           "fwd_gate", "bwd_gate", "decode_step_gate", "fwd_scalar", "bwd_scalar", "decode_step_scalar", "hgrn1_fwd", "hgrn1_bwd", "hgrn1_states_shape", "hgrn2_chunk", "HGRN2Chunk", "HGRN2Error", "supported",
           "num_chunks", "states_shape", "lib", "LIB_PATH", "F32", "BF16", "OUT_F32"]
