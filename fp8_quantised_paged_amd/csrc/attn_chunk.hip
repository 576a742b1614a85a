// Query-tiled causal chunk attention (long q_len); see launch_attn_chunk.
#include "kvfp8_internal.h"

namespace kvfp8 {

hipError_t launch_attn_chunk(const AttnArgs&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kvfp8
