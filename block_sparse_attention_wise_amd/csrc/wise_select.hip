// Working-set selection (WISE, Section 5.1, Eq. 6; Appendix A.1, Eq. 12).
//
// One wavefront per row (batch, head, query block q) chooses, among the
// admissible key blocks 0..q, the smallest set whose mean discovery mass
// reaches eta, ranked by mass (ties to the lower block index), optionally
// capped, and adds the sink block 0 and the diagonal block q.
//
// No sort is needed.  The k*-th largest mass t* is the largest value t for
// which the mass of all blocks >= t still reaches eta; because the masses
// are non-negative fp32 numbers, their bit patterns order like the values,
// so t* is found by a greedy 31-step search over the bits, each step one
// float64 wavefront sum.  The chosen set is every block above t* plus the
// first (in index order) blocks equal to t* until eta is reached; the cap is
// applied the same way with counts instead of masses.  Ballots give index
// order and the compacted, ascending CSR output.
//
// Three launches build the CSR without scratch memory: count (row lengths
// into row_ptr[1..]), an in-place scan of row_ptr, and fill (the same
// deterministic selection again, written at row_ptr[row]).
#include "wise_internal.h"

namespace wise {

namespace {

constexpr int kSelWaves = 4;  // rows per workgroup

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ int wave_isum(int x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ uint32_t lanes_below(uint64_t mask, int lane) {
  return (uint32_t)__popcll(mask & ((1ull << lane) - 1ull));
}

// Selection flags of one row; bit j of the result is set when element
// e = 64*j + lane is kept.  EPL = elements per lane (n_blocks <= 64*EPL).
template <int EPL>
__device__ uint32_t select_row(const SelectParams& p, int row, int lane) {
  const int q = row % p.nblk;
  const int n = q + 1;
  const float* mrow = p.mass + (size_t)row * p.nblk;

  uint32_t bits[EPL];
  double mbar[EPL];
  uint32_t valid = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = 64 * j + lane;
    const bool v = e < n;
    const float x = v ? mrow[e] : 0.f;
    bits[j] = __float_as_uint(x);
    mbar[j] = v ? (double)x / p.n_steps : 0.0;
    if (v) valid |= 1u << j;
  }

  auto mass_at_least = [&](uint32_t t) {
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (((valid >> j) & 1u) && bits[j] >= t) s += mbar[j];
    return wave_sum(s);
  };
  auto count_at_least = [&](uint32_t t) {
    int c = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
      if (((valid >> j) & 1u) && bits[j] >= t) ++c;
    return wave_isum(c);
  };
  // Keep-set {bits > t} plus the first `ties` elements (index order) with
  // bits == t.  ties < 0 means all of them.
  auto keep_flags = [&](uint32_t t, int ties) {
    uint32_t f = 0;
    int seen = 0;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      const bool v = (valid >> j) & 1u;
      const bool tie = v && bits[j] == t;
      const uint64_t tb = __ballot(tie);
      const int rank = seen + (int)lanes_below(tb, lane);
      if (v && (bits[j] > t || (tie && (ties < 0 || rank < ties)))) f |= 1u << j;
      seen += (int)__popcll(tb);
    }
    return f;
  };

  uint32_t flags;
  int k_star;
  if (mass_at_least(0u) < p.eta) {
    // Rounding left the total below eta: every admissible block is kept.
    flags = valid;
    k_star = n;
  } else {
    uint32_t t = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = t | (1u << bit);
      if (mass_at_least(cand) >= p.eta) t = cand;
    }
    // Mass strictly above t*, then ties in index order until eta is reached
    // (t* has bit 31 clear, so t* + 1 does not wrap).
    const double above = mass_at_least(t + 1u);
    const int n_above = count_at_least(t + 1u);
    const double tie_val = (double)__uint_as_float(t) / p.n_steps;
    int need = 0;
    double pref = above;
    bool done = false;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
      uint64_t tb = __ballot(((valid >> j) & 1u) && bits[j] == t);
      while (tb != 0 && !done) {  // wave-uniform
        tb &= tb - 1;
        pref += tie_val;
        ++need;
        if (pref >= p.eta) done = true;
      }
    }
    flags = keep_flags(t, need);
    k_star = n_above + need;
  }

  if (p.max_blocks > 0 && k_star > p.max_blocks) {
    // Top max_blocks by (mass desc, index asc): largest t2 with at least
    // max_blocks blocks >= t2, then ties at t2 in index order.
    uint32_t t2 = 0;
    for (int bit = 30; bit >= 0; --bit) {
      const uint32_t cand = t2 | (1u << bit);
      if (count_at_least(cand) >= p.max_blocks) t2 = cand;
    }
    const int n_above = count_at_least(t2 + 1u);
    flags = keep_flags(t2, p.max_blocks - n_above);
  }

  // Sink and diagonal blocks are always kept.
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = 64 * j + lane;
    if (e == 0 || e == q) flags |= 1u << j;
  }
  return flags;
}

template <int EPL>
__global__ void __launch_bounds__(64 * kSelWaves) select_count_kernel(SelectParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;
  const uint32_t f = select_row<EPL>(p, row, lane);
  const int cnt = wave_isum(__popc(f));
  if (lane == 0) p.row_ptr[row + 1] = cnt;
}

template <int EPL>
__global__ void __launch_bounds__(64 * kSelWaves) select_fill_kernel(SelectParams p) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * kSelWaves + (threadIdx.x >> 6);
  if (row >= p.n_rows) return;
  const uint32_t f = select_row<EPL>(p, row, lane);
  int out = p.row_ptr[row];
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool keep = (f >> j) & 1u;
    const uint64_t b = __ballot(keep);
    if (keep) p.col_idx[out + (int)lanes_below(b, lane)] = 64 * j + lane;
    out += (int)__popcll(b);
  }
}

// In-place inclusive scan of row_ptr[1..n] (row lengths) with row_ptr[0] = 0,
// by one workgroup of 1024 threads walking the rows in chunks.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;

__global__ void __launch_bounds__(kScanThreads) scan_rows_kernel(int32_t* row_ptr, int n) {
  __shared__ int wsum[kScanThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry = 0;
  if (tid == 0) row_ptr[0] = 0;
  for (int base = 0; base < n; base += kScanThreads * kScanItems) {
    int v[kScanItems];
    int local = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int idx = base + tid * kScanItems + i;
      v[i] = idx < n ? row_ptr[1 + idx] : 0;
      local += v[i];
    }
    // inclusive scan of `local` across the workgroup
    int x = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int y = __shfl_up(x, off);
      if (lane >= off) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    int wprefix = 0;
    for (int w = 0; w < wave; ++w) wprefix += wsum[w];
    int total = 0;
    for (int w = 0; w < kScanThreads / 64; ++w) total += wsum[w];
    __syncthreads();
    int run = carry + wprefix + x - local;  // exclusive prefix of this thread
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int idx = base + tid * kScanItems + i;
      run += v[i];
      if (idx < n) row_ptr[1 + idx] = run;
    }
    carry += total;
  }
}

template <int EPL>
hipError_t launch_select_t(const SelectParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((p.n_rows + kSelWaves - 1) / kSelWaves);
  hipLaunchKernelGGL(select_count_kernel<EPL>, dim3(grid), dim3(64 * kSelWaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_rows_kernel, dim3(1), dim3(kScanThreads), 0, stream, p.row_ptr, p.n_rows);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_fill_kernel<EPL>, dim3(grid), dim3(64 * kSelWaves), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_select(const SelectParams& p, hipStream_t stream) {
  const int epl = (p.nblk + 63) / 64;
  if (epl <= 1) return launch_select_t<1>(p, stream);
  if (epl <= 2) return launch_select_t<2>(p, stream);
  if (epl <= 4) return launch_select_t<4>(p, stream);
  if (epl <= 8) return launch_select_t<8>(p, stream);
  if (epl <= 16) return launch_select_t<16>(p, stream);
  if (epl <= 32) return launch_select_t<32>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace wise
