// Working-set selection ("Attention Routing Stabilizes Early: Working-Set
// Inference for Recurrent Language Models" (WISE), Section 5.1, Eq. 6;
// Appendix A.1, Eq. 12).
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
// Variants (same machinery): the temporal union of per-step supports
// (Eq. 6 left / Eq. 18), and the controls of Appendix B: Static-95 (Eq. 19),
// MassMatched (Eq. 20-21: the first step's mass covered by the union becomes
// the threshold of the first step's own ranking) and SizeMatched (Eq. 22:
// the union's size becomes a top-k count on the first step).
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

// One row's masses as held by a wavefront: element e = 64*j + lane in slot
// j; fp32 bit patterns (non-negative, so they order like the values) and
// the float64 values the sums use.
template <int EPL>
struct RowMass {
  uint32_t bits[EPL];
  double val[EPL];
  uint32_t valid;  // bit j: element 64*j + lane is admissible (e <= q)
  double div;      // val = fp32 value / div
};

template <int EPL>
__device__ __forceinline__ RowMass<EPL> load_row(const float* mrow, int n, double div, int lane) {
  RowMass<EPL> r;
  r.valid = 0;
  r.div = div;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const int e = 64 * j + lane;
    const bool v = e < n;
    const float x = v ? mrow[e] : 0.f;
    r.bits[j] = __float_as_uint(x);
    r.val[j] = v ? (double)x / div : 0.0;
    if (v) r.valid |= 1u << j;
  }
  return r;
}

template <int EPL>
__device__ __forceinline__ double mass_at_least(const RowMass<EPL>& r, uint32_t t) {
  double s = 0.0;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (((r.valid >> j) & 1u) && r.bits[j] >= t) s += r.val[j];
  return wave_sum(s);
}

template <int EPL>
__device__ __forceinline__ int count_at_least(const RowMass<EPL>& r, uint32_t t) {
  int c = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j)
    if (((r.valid >> j) & 1u) && r.bits[j] >= t) ++c;
  return wave_isum(c);
}

// Keep-set {bits > t} plus the first `ties` elements (index order) with
// bits == t.
template <int EPL>
__device__ __forceinline__ uint32_t keep_flags(const RowMass<EPL>& r, uint32_t t, int ties, int lane) {
  uint32_t f = 0;
  int seen = 0;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    const bool v = (r.valid >> j) & 1u;
    const bool tie = v && r.bits[j] == t;
    const uint64_t tb = __ballot(tie);
    const int rank = seen + (int)lanes_below(tb, lane);
    if (v && (r.bits[j] > t || (tie && rank < ties))) f |= 1u << j;
    seen += (int)__popcll(tb);
  }
  return f;
}

// The cumulative-eta support (Eq. 6 right / Eq. 12): the smallest set of
// highest-mass admissible blocks (ties to the lower index) whose float64
// mass reaches eta; every admissible block when the total stays below eta.
template <int EPL>
__device__ uint32_t eta_flags(const RowMass<EPL>& r, double eta, int lane) {
  if (mass_at_least(r, 0u) < eta) return r.valid;
  uint32_t t = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (mass_at_least(r, cand) >= eta) t = cand;
  }
  // Mass strictly above t*, then ties in index order until eta is reached
  // (t* has bit 31 clear, so t* + 1 does not wrap).
  const double above = mass_at_least(r, t + 1u);
  const double tie_val = (double)__uint_as_float(t) / r.div;   // the value of every tied element
  int need = 0;
  double pref = above;
  bool done = false;
#pragma unroll
  for (int j = 0; j < EPL; ++j) {
    uint64_t tb = __ballot(((r.valid >> j) & 1u) && r.bits[j] == t);
    while (tb != 0 && !done) {  // wave-uniform
      tb &= tb - 1;
      pref += tie_val;
      ++need;
      if (pref >= eta) done = true;
    }
  }
  return keep_flags(r, t, need, lane);
}

// The k highest-mass admissible blocks (ties to the lower index): largest
// t with at least k blocks >= t, then ties at t in index order.
template <int EPL>
__device__ uint32_t topk_flags(const RowMass<EPL>& r, int k, int lane) {
  uint32_t t = 0;
  for (int bit = 30; bit >= 0; --bit) {
    const uint32_t cand = t | (1u << bit);
    if (count_at_least(r, cand) >= k) t = cand;
  }
  return keep_flags(r, t, k - count_at_least(r, t + 1u), lane);
}

template <int EPL>
__device__ __forceinline__ int flag_count(uint32_t f) {
  return wave_isum(__popc(f));
}

// Selection flags of one row; bit j of the result is set when element
// e = 64*j + lane is kept.  EPL = elements per lane (n_blocks <= 64*EPL).
template <int EPL>
__device__ uint32_t select_row(const SelectParams& p, int row, int lane) {
  const int q = row % p.nblk;
  const int n = q + 1;
  auto step_row = [&](int w) { return p.mass + (size_t)w * p.mass_stride + (size_t)row * p.nblk; };

  uint32_t flags = 0;
  if (p.kind == kSelMean) {
    const RowMass<EPL> r = load_row<EPL>(step_row(0), n, p.n_steps, lane);
    flags = eta_flags(r, p.eta, lane);
    if (p.max_blocks > 0 && flag_count<EPL>(flags) > p.max_blocks) flags = topk_flags(r, p.max_blocks, lane);
  } else if (p.kind == kSelUnion || p.kind == kSelStatic) {
    // Eq. (6) left / Eq. (18): union of every given step's own eta-support
    // (Static-95, Eq. 19: the single first step).
    for (int w = 0; w < p.n_mass; ++w) flags |= eta_flags(load_row<EPL>(step_row(w), n, 1.0, lane), p.eta, lane);
  } else {
    // Controls of Eq. (20)-(22): the union W of steps 1..n_mass-1, then the
    // first step's own ranking (step 0).
    uint32_t u = 0;
    for (int w = 1; w < p.n_mass; ++w) u |= eta_flags(load_row<EPL>(step_row(w), n, 1.0, lane), p.eta, lane);
    const RowMass<EPL> a = load_row<EPL>(step_row(0), n, 1.0, lane);
    if (p.kind == kSelMassMatched) {
      double m = 0.0;
#pragma unroll
      for (int j = 0; j < EPL; ++j)
        if ((u >> j) & 1u) m += a.val[j];
      flags = eta_flags(a, wave_sum(m), lane);
    } else {
      flags = topk_flags(a, flag_count<EPL>(u), lane);
    }
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
// by one workgroup of 1024 threads walking the rows in chunks; the total
// goes to *nnz as well when nnz is given.
constexpr int kScanThreads = 1024;
constexpr int kScanItems = 8;

__global__ void __launch_bounds__(kScanThreads) scan_rows_kernel(int32_t* row_ptr, int n, int64_t* nnz) {
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
  if (nnz != nullptr && tid == 0) *nnz = carry;
}

template <int EPL>
hipError_t launch_select_t(const SelectParams& p, hipStream_t stream) {
  const unsigned grid = (unsigned)((p.n_rows + kSelWaves - 1) / kSelWaves);
  if (trace_enabled())
    trace_launch("select_count/scan/fill", grid, 64 * kSelWaves, 0,
                 "kind=%d rows=%d n_blocks=%d entries_per_lane=%d eta=%.17g n_steps=%g cap=%d n_mass=%d", p.kind,
                 p.n_rows, p.nblk, EPL, p.eta, p.n_steps, p.max_blocks, p.n_mass);
  if (grid > 0) hipLaunchKernelGGL(select_count_kernel<EPL>, dim3(grid), dim3(64 * kSelWaves), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(scan_rows_kernel, dim3(1), dim3(kScanThreads), 0, stream, p.row_ptr, p.n_rows, p.nnz);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  // No rows: the scan alone writes row_ptr[0] = 0.
  if (grid > 0) hipLaunchKernelGGL(select_fill_kernel<EPL>, dim3(grid), dim3(64 * kSelWaves), 0, stream, p);
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
