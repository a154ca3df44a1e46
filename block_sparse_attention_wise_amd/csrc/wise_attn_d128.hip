// Attention kernels for head_dim 128 (all block sizes and modes).
#include "wise_attn_kernel.h"

namespace wise {
hipError_t launch_attn_d128(int block, int mode, const AttnParams& p, hipStream_t stream) {
  return launch_attn_d<128>(block, mode, p, stream);
}
size_t attn_lds_bytes_d128(int block, int mode, int nblk) { return attn_lds_bytes_d<128>(block, mode, nblk); }
}  // namespace wise
