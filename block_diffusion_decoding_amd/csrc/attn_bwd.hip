// Block-causal attention backward on the gfx950 matrix cores (bf16).
#include "bd_device.hpp"
#include "bd_kernels.hpp"

namespace bd {

size_t attn_bwd_workspace_bytes(int batch, int seqlen, int n_q_heads) {
  return (size_t)batch * n_q_heads * seqlen * sizeof(float);
}

hipError_t launch_attn_bwd_bf16(const void*, const void*, const void*, const void*, const float*, const void*,
                                void*, void*, void*, void*, const AttnShape&, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace bd
