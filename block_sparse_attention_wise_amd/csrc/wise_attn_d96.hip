// Attention kernels for head_dim 96 (all block sizes and modes).
#include "wise_attn_kernel.h"

namespace wise {
hipError_t launch_attn_d96(int block, int mode, const AttnParams& p, hipStream_t stream) {
  return launch_attn_d<96>(block, mode, p, stream);
}
size_t attn_lds_bytes_d96(int block, int mode, int nblk) { return attn_lds_bytes_d<96>(block, mode, nblk); }
}  // namespace wise
