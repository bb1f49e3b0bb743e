// Block attention backward (bf16, float32 accumulation) -- launcher.
#include "ra_internal.h"

namespace ra {

hipError_t launch_attn_bwd_bf16(const AttnArgs& a, int dqk, int dv, bool causal,
                                hipStream_t st) {
  (void)a; (void)dqk; (void)dv; (void)causal; (void)st;
  return hipErrorInvalidValue;
}

}  // namespace ra
