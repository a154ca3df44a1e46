// Working-set diagnostics ("Attention Routing Stabilizes Early: Working-Set
// Inference for Recurrent Language Models" (WISE), Section 7 "Evaluation
// metrics"; Appendix C.2, Eq. 23-25).
//
//  * Retained future attention mass: for a row r = (b, h, q) and an
//    unrestricted step's block masses r_qb (Eq. 5, rows summing to 1), the
//    mass inside the frozen support, sum over kb in W_q of r_qb.
//  * Working-set overlap: for two supports A and B of the same row,
//    |A intersect B| and |A union B|; summed over rows (and divided) they give
//    the Jaccard similarity of Eq. (24) and (25).
//
// One wavefront per row.  CSR rows are read as sets, as everywhere in the
// library: entries outside [0, q] are ignored and repeats count once.  Each
// lane owns blocks lane, lane + 64, ... and builds its own bits with no
// atomics; the mass sum is a float64 per-lane sum in block order, then a
// fixed butterfly, so it is deterministic.
#include "wise_internal.h"

namespace wise {

namespace {

constexpr int kDiagWaves = 4;
constexpr int kMaxWords = 32;   // 64 * 32 = 2048 blocks per row

// Bit j of the result: block 64*j + lane is listed in CSR row `row`.
__device__ __forceinline__ uint32_t row_bits(const int32_t* row_ptr, const int32_t* col_idx, int row, int q,
                                             int lane) {
  int e0 = row_ptr[row], e1 = row_ptr[row + 1];
  if (e0 < 0) e0 = 0;          // malformed pointers: read nothing before col_idx
  if (e1 < e0) e1 = e0;        // and a decreasing pair as an empty row
  uint32_t bits = 0;
  for (int base = e0; base < e1; base += 64) {
    const int idx = base + lane;
    const int c = idx < e1 ? col_idx[idx] : -1;
    const bool ok = c >= 0 && c <= q;
    // every lane learns every listed block of this chunk, one at a time
    uint64_t pending = __ballot(ok);
    while (pending != 0) {                        // wave-uniform
      const int src = __builtin_ctzll(pending);
      pending &= pending - 1;
      const int blk = __shfl(c, src);
      if ((blk & 63) == lane) bits |= 1u << (blk >> 6);
    }
  }
  return bits;
}

__device__ __forceinline__ int wave_isum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ double wave_dsum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__global__ void __launch_bounds__(64 * kDiagWaves) support_mass_kernel(const float* mass, const int32_t* row_ptr,
                                                                       const int32_t* col_idx, float* out,
                                                                       int n_rows, int nblk) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kDiagWaves + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int q = row % nblk;
  const uint32_t bits = row_bits(row_ptr, col_idx, row, q, lane);
  const float* mrow = mass + (size_t)row * nblk;
  double s = 0.0;
  for (int j = 0; j < kMaxWords; ++j)
    if ((bits >> j) & 1u) s += (double)mrow[64 * j + lane];
  s = wave_dsum(s);
  if (lane == 0) out[row] = (float)s;
}

__global__ void __launch_bounds__(64 * kDiagWaves) support_overlap_kernel(
    const int32_t* rp_a, const int32_t* ci_a, const int32_t* rp_b, const int32_t* ci_b, int32_t* inter,
    int32_t* uni, int n_rows, int nblk) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kDiagWaves + (threadIdx.x >> 6);
  if (row >= n_rows) return;
  const int q = row % nblk;
  const uint32_t a = row_bits(rp_a, ci_a, row, q, lane);
  const uint32_t b = row_bits(rp_b, ci_b, row, q, lane);
  const int ni = wave_isum(__popc(a & b));
  const int nu = wave_isum(__popc(a | b));
  if (lane == 0) {
    inter[row] = ni;
    uni[row] = nu;
  }
}

}  // namespace

hipError_t launch_support_mass(const float* mass, const int32_t* row_ptr, const int32_t* col_idx, float* out,
                               int n_rows, int nblk, hipStream_t stream) {
  if (nblk > 64 * kMaxWords) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((n_rows + kDiagWaves - 1) / kDiagWaves);
  if (trace_enabled()) trace_launch("support_mass_kernel", grid, 64 * kDiagWaves, 0, "rows=%d n_blocks=%d", n_rows, nblk);
  hipLaunchKernelGGL(support_mass_kernel, dim3(grid), dim3(64 * kDiagWaves), 0, stream, mass, row_ptr, col_idx,
                     out, n_rows, nblk);
  return hipGetLastError();
}

hipError_t launch_support_overlap(const int32_t* rp_a, const int32_t* ci_a, const int32_t* rp_b,
                                  const int32_t* ci_b, int32_t* inter, int32_t* uni, int n_rows, int nblk,
                                  hipStream_t stream) {
  if (nblk > 64 * kMaxWords) return hipErrorInvalidValue;
  const unsigned grid = (unsigned)((n_rows + kDiagWaves - 1) / kDiagWaves);
  if (trace_enabled())
    trace_launch("support_overlap_kernel", grid, 64 * kDiagWaves, 0, "rows=%d n_blocks=%d", n_rows, nblk);
  hipLaunchKernelGGL(support_overlap_kernel, dim3(grid), dim3(64 * kDiagWaves), 0, stream, rp_a, ci_a, rp_b,
                     ci_b, inter, uni, n_rows, nblk);
  return hipGetLastError();
}

}  // namespace wise
