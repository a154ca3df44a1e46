// C ABI of libwise (declared in include/wise.h): host-side validation and
// dispatch to the HIP kernels.  Validation is pure host code and touches no
// device state, so invalid calls return before anything is launched.
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/wise.h"
#include "wise_internal.h"

namespace wise {

size_t attn_lds_bytes_d64(int block, int mode, int nblk);
size_t attn_lds_bytes_d96(int block, int mode, int nblk);
size_t attn_lds_bytes_d128(int block, int mode, int nblk);

size_t attn_lds_bytes(int head_dim, int block, int mode, int nblk) {
  switch (head_dim) {
    case 64: return attn_lds_bytes_d64(block, mode, nblk);
    case 96: return attn_lds_bytes_d96(block, mode, nblk);
    case 128: return attn_lds_bytes_d128(block, mode, nblk);
  }
  return 0;
}

hipError_t launch_attn(const AttnLaunch& cfg, const AttnParams& p, hipStream_t stream) {
  switch (cfg.head_dim) {
    case 64: return launch_attn_d64(cfg.block, cfg.mode, p, stream);
    case 96: return launch_attn_d96(cfg.block, cfg.mode, p, stream);
    case 128: return launch_attn_d128(cfg.block, cfg.mode, p, stream);
  }
  return hipErrorInvalidValue;
}

bool trace_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("WISE_TRACE");
    return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
  }();
  return on;
}

void trace_launch(const char* kernel, unsigned grid, unsigned threads, size_t lds, const char* fmt, ...) {
  char detail[192];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(detail, sizeof(detail), fmt, ap);
  va_end(ap);
  std::fprintf(stderr, "[wise] %s grid=%u threads=%u lds=%zu %s\n", kernel, grid, threads, lds, detail);
}

namespace {

thread_local char g_last_error[256] = "";

wise_status_t fail(wise_status_t st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
wise_status_t fail(wise_status_t st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return st;
}

wise_status_t ok() {
  g_last_error[0] = '\0';
  return WISE_OK;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// Shape checks common to every call.  Fills nblk / n_rows on success.
wise_status_t check_desc(const wise_attn_desc_t* d, int32_t* nblk, int64_t* n_rows) {
  if (d == nullptr) return fail(WISE_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 0 || d->heads < 0)
    return fail(WISE_ERR_INVALID_ARG, "batch (%d) and heads (%d) must be >= 0", d->batch, d->heads);
  if (d->block_size != 16 && d->block_size != 32 && d->block_size != 64 && d->block_size != 128)
    return fail(WISE_ERR_UNSUPPORTED, "block_size %d not built (16, 32, 64, 128)", d->block_size);
  if (d->head_dim != 64 && d->head_dim != 96 && d->head_dim != 128)
    return fail(WISE_ERR_UNSUPPORTED, "head_dim %d not built (64, 96, 128)", d->head_dim);
  if (d->seq_len < 0) return fail(WISE_ERR_INVALID_ARG, "seq_len %d must be >= 0", d->seq_len);
  if (d->seq_len > 65536)
    return fail(WISE_ERR_UNSUPPORTED, "seq_len %d above 65536", d->seq_len);
  if (!std::isfinite(d->softmax_scale))
    return fail(WISE_ERR_INVALID_ARG, "softmax_scale is not finite");
  if (d->kv_heads < 0 || (d->kv_heads > 0 && d->heads % d->kv_heads != 0))
    return fail(WISE_ERR_INVALID_ARG, "kv_heads %d must be 0 or divide heads %d", d->kv_heads, d->heads);
  // The last block is short when seq_len is not a multiple of block_size.
  const int32_t nb = (d->seq_len + d->block_size - 1) / d->block_size;
  const int64_t heads_total = (int64_t)d->batch * d->heads;
  const int64_t rows = heads_total * nb;
  if (rows >= (int64_t)INT32_MAX)
    return fail(WISE_ERR_UNSUPPORTED, "batch*heads*n_blocks = %lld too large", (long long)rows);
  *nblk = nb;
  *n_rows = rows;
  return WISE_OK;
}

wise_status_t check_tensor(const void* ptr, const char* name) {
  if (ptr == nullptr) return fail(WISE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(ptr)) return fail(WISE_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return WISE_OK;
}

float scale_log2(const wise_attn_desc_t* d) {
  const double s = d->softmax_scale > 0.f ? (double)d->softmax_scale : 1.0 / std::sqrt((double)d->head_dim);
  return (float)(s * 1.4426950408889634);  // log2(e)
}

wise_status_t run_attn(const wise_attn_desc_t* d, int mode, const void* q, const void* k, const void* v,
                       void* o, float* lse, float* mass, const int32_t* row_ptr, const int32_t* col_idx,
                       void* stream, float* work = nullptr) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(d, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  if (n_rows == 0) return ok();   // nothing to compute; the pointers are not used
  if ((st = check_tensor(q, "q")) != WISE_OK) return st;
  if ((st = check_tensor(k, "k")) != WISE_OK) return st;
  if ((st = check_tensor(v, "v")) != WISE_OK) return st;
  if ((st = check_tensor(o, "o")) != WISE_OK) return st;
  if (o == q || o == k || o == v) return fail(WISE_ERR_INVALID_ARG, "o aliases an input");
  if ((mode == kDenseMass || mode == kDenseMassWs) && mass == nullptr)
    return fail(WISE_ERR_INVALID_ARG, "mass is NULL");
  if (mode == kSparse && (row_ptr == nullptr || col_idx == nullptr))
    return fail(WISE_ERR_INVALID_ARG, "row_ptr / col_idx is NULL");
  if (lse != nullptr && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(WISE_ERR_INVALID_ARG, "lse is not 4-byte aligned");
  if (mass != nullptr && (reinterpret_cast<uintptr_t>(mass) & 3u))
    return fail(WISE_ERR_INVALID_ARG, "mass is not 4-byte aligned");
  if (d->block_size == 16 && d->seq_len % 32 != 0)
    return fail(WISE_ERR_UNSUPPORTED, "block_size 16 attention needs seq_len %d to be a multiple of 32",
                d->seq_len);
  const size_t lds = attn_lds_bytes(d->head_dim, d->block_size, mode, nblk);
  if (lds == 0 || lds > kMaxLds)
    return fail(WISE_ERR_UNSUPPORTED, "seq_len %d needs %zu B of LDS for this call", d->seq_len, lds);

  AttnParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.mass = mass;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.heads_total = d->batch * d->heads;
  p.heads = d->heads;
  p.kv_group = d->kv_heads > 0 ? d->heads / d->kv_heads : 1;
  p.seq = d->seq_len;
  p.nblk = nblk;
  p.scale_log2 = scale_log2(d);
  p.work = work;
  AttnLaunch cfg{d->head_dim, d->block_size, mode};
  const hipError_t e = launch_attn(cfg, p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WISE_ERR_HIP, "attention launch failed: %s", hipGetErrorString(e));
  return ok();
}

// Workspace of the mass launch: one fp32 partial per (row, key block, query
// of the row), for blocks 32, 64 and 128; block 16 needs none.
int64_t accum_workspace_bytes(const wise_attn_desc_t* d, int32_t nblk, int64_t n_rows) {
  if (d->block_size < 32) return 0;
  return n_rows * (int64_t)nblk * d->block_size * 4;
}

int64_t max_nnz(int32_t nblk, int64_t heads_total, int32_t max_blocks) {
  int64_t per_head = 0;
  for (int32_t q = 0; q < nblk; ++q) {
    int64_t n = q + 1;
    if (max_blocks > 0 && n > (int64_t)max_blocks + 2) n = (int64_t)max_blocks + 2;
    per_head += n;
  }
  return per_head * heads_total;
}

// Fixed device buffer of wise_full_attn_accum_noalloc: the block-mass
// partials of the workspace launch for callers that cannot allocate.  Every
// GPU the library runs on holds one copy for the life of the process.  In
// host code `scratch` names a host-side stand-in, not device memory: the
// kernels only ever receive the device address that hipGetSymbolAddress
// reports for the current device, kept per device below.
constexpr int64_t kScratchBytes = 64ll << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kScratchDevices = 64;
std::atomic<void*> g_scratch_ptr[kScratchDevices];   // per device; null until first looked up

// Device address of `scratch` on the current device (looked up once per
// device; concurrent first calls may both look it up and store the same
// value).  Returns nullptr and sets the error text on failure.
void* scratch_ptr() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kScratchDevices) {
    fail(WISE_ERR_HIP, "no usable current device for the scratch buffer");
    return nullptr;
  }
  void* ptr = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (ptr == nullptr) {
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      fail(WISE_ERR_HIP, "hipGetSymbolAddress(scratch) failed on device %d: %s", dev, hipGetErrorString(e));
      return nullptr;
    }
    g_scratch_ptr[dev].store(ptr, std::memory_order_release);
  }
  return ptr;
}

}  // namespace
}  // namespace wise

using namespace wise;

extern "C" {

wise_status_t wise_full_attn(const wise_attn_desc_t* desc, const void* q, const void* k, const void* v,
                             void* o, float* lse, void* stream) {
  return run_attn(desc, kDense, q, k, v, o, lse, nullptr, nullptr, nullptr, stream);
}

wise_status_t wise_full_attn_accum(const wise_attn_desc_t* desc, const void* q, const void* k,
                                   const void* v, void* o, float* mass, void* stream) {
  return run_attn(desc, kDenseMass, q, k, v, o, nullptr, mass, nullptr, nullptr, stream);
}

int64_t wise_full_attn_accum_workspace_bytes(const wise_attn_desc_t* desc) {
  int32_t nblk;
  int64_t n_rows;
  if (check_desc(desc, &nblk, &n_rows) != WISE_OK) return -1;
  return accum_workspace_bytes(desc, nblk, n_rows);
}

wise_status_t wise_full_attn_accum_ws(const wise_attn_desc_t* desc, const void* q, const void* k,
                                      const void* v, void* o, float* mass, void* workspace,
                                      int64_t workspace_bytes, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  const int64_t need = accum_workspace_bytes(desc, nblk, n_rows);
  if (need == 0) return run_attn(desc, kDenseMass, q, k, v, o, nullptr, mass, nullptr, nullptr, stream);
  if (workspace == nullptr) return fail(WISE_ERR_INVALID_ARG, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(workspace) & 15u)
    return fail(WISE_ERR_INVALID_ARG, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(WISE_ERR_CAPACITY, "workspace_bytes %lld below the %lld this call needs",
                (long long)workspace_bytes, (long long)need);
  if (workspace == q || workspace == k || workspace == v || workspace == o || workspace == mass)
    return fail(WISE_ERR_INVALID_ARG, "workspace aliases an input or output");
  return run_attn(desc, kDenseMassWs, q, k, v, o, nullptr, mass, nullptr, nullptr, stream,
                  static_cast<float*>(workspace));
}

wise_status_t wise_full_attn_accum_noalloc(const wise_attn_desc_t* desc, const void* q, const void* k,
                                           const void* v, void* o, float* mass, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  const int64_t need = accum_workspace_bytes(desc, nblk, n_rows);
  if (need == 0) return run_attn(desc, kDenseMass, q, k, v, o, nullptr, mass, nullptr, nullptr, stream);
  if (need > kScratchBytes)
    return fail(WISE_ERR_CAPACITY, "this call needs %lld bytes of block-mass partials; the fixed buffer "
                "holds %lld (batch * heads * n_blocks^2 * block_size * 4 must not exceed it)",
                (long long)need, (long long)kScratchBytes);
  // Validate the caller's arguments before the first device call.
  if ((st = check_tensor(q, "q")) != WISE_OK) return st;
  if ((st = check_tensor(k, "k")) != WISE_OK) return st;
  if ((st = check_tensor(v, "v")) != WISE_OK) return st;
  if ((st = check_tensor(o, "o")) != WISE_OK) return st;
  if (mass == nullptr) return fail(WISE_ERR_INVALID_ARG, "mass is NULL");
  void* ws = scratch_ptr();
  if (ws == nullptr) return WISE_ERR_HIP;
  return run_attn(desc, kDenseMassWs, q, k, v, o, nullptr, mass, nullptr, nullptr, stream,
                  static_cast<float*>(ws));
}

int64_t wise_full_attn_accum_noalloc_max_bytes(void) { return kScratchBytes; }

wise_status_t wise_sparse_attn(const wise_attn_desc_t* desc, const void* q, const void* k, const void* v,
                               const int32_t* row_ptr, const int32_t* col_idx, void* o, void* stream) {
  return run_attn(desc, kSparse, q, k, v, o, nullptr, nullptr, row_ptr, col_idx, stream);
}

int64_t wise_select_max_nnz(const wise_attn_desc_t* desc, int32_t max_blocks) {
  int32_t nblk;
  int64_t n_rows;
  if (check_desc(desc, &nblk, &n_rows) != WISE_OK || max_blocks < 0) return -1;
  return max_nnz(nblk, (int64_t)desc->batch * desc->heads, max_blocks);
}

wise_status_t wise_select_support(const wise_attn_desc_t* desc, const float* mass, int32_t n_steps,
                                  double eta, int32_t max_blocks, int32_t* row_ptr, int32_t* col_idx,
                                  int64_t col_capacity, int64_t* nnz, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  if (row_ptr == nullptr || (n_rows > 0 && (mass == nullptr || col_idx == nullptr)))
    return fail(WISE_ERR_INVALID_ARG, "mass / row_ptr / col_idx is NULL");
  if ((reinterpret_cast<uintptr_t>(mass) | reinterpret_cast<uintptr_t>(row_ptr) |
       reinterpret_cast<uintptr_t>(col_idx)) & 3u)
    return fail(WISE_ERR_INVALID_ARG, "mass / row_ptr / col_idx not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(nnz) & 7u) return fail(WISE_ERR_INVALID_ARG, "nnz not 8-byte aligned");
  if (n_steps < 1) return fail(WISE_ERR_INVALID_ARG, "n_steps %d must be >= 1", n_steps);
  if (!(eta > 0.0 && eta <= 1.0)) return fail(WISE_ERR_INVALID_ARG, "eta %g outside (0, 1]", eta);
  if (max_blocks < 0) return fail(WISE_ERR_INVALID_ARG, "max_blocks %d < 0", max_blocks);
  if (nblk > 64 * 32) return fail(WISE_ERR_UNSUPPORTED, "n_blocks %d above 2048", nblk);
  const int64_t need = max_nnz(nblk, (int64_t)desc->batch * desc->heads, max_blocks);
  if (need >= (int64_t)INT32_MAX)
    return fail(WISE_ERR_UNSUPPORTED, "worst-case nnz %lld does not fit int32", (long long)need);
  if (col_capacity < need)
    return fail(WISE_ERR_CAPACITY, "col_capacity %lld below worst-case nnz %lld", (long long)col_capacity,
                (long long)need);
  SelectParams p{};
  p.mass = mass;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.n_rows = (int32_t)n_rows;
  p.nblk = nblk;
  p.max_blocks = max_blocks;
  p.n_steps = (double)n_steps;
  p.eta = eta;
  p.nnz = nnz;
  const hipError_t e = launch_select(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WISE_ERR_HIP, "selection launch failed: %s", hipGetErrorString(e));
  return ok();
}

wise_status_t wise_select_variant(const wise_attn_desc_t* desc, int32_t kind, const float* step_mass,
                                  int32_t n_mass, double eta, int32_t* row_ptr, int32_t* col_idx,
                                  int64_t col_capacity, int64_t* nnz, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  if (row_ptr == nullptr || (n_rows > 0 && (step_mass == nullptr || col_idx == nullptr)))
    return fail(WISE_ERR_INVALID_ARG, "step_mass / row_ptr / col_idx is NULL");
  if ((reinterpret_cast<uintptr_t>(step_mass) | reinterpret_cast<uintptr_t>(row_ptr) |
       reinterpret_cast<uintptr_t>(col_idx)) & 3u)
    return fail(WISE_ERR_INVALID_ARG, "step_mass / row_ptr / col_idx not 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(nnz) & 7u) return fail(WISE_ERR_INVALID_ARG, "nnz not 8-byte aligned");
  if (kind < WISE_SELECT_UNION || kind > WISE_SELECT_SIZE_MATCHED)
    return fail(WISE_ERR_INVALID_ARG, "unknown selection kind %d", kind);
  const int32_t min_mass = (kind == WISE_SELECT_UNION || kind == WISE_SELECT_STATIC) ? 1 : 2;
  if (n_mass < min_mass || (kind == WISE_SELECT_STATIC && n_mass != 1))
    return fail(WISE_ERR_INVALID_ARG, "n_mass %d invalid for selection kind %d", n_mass, kind);
  if (!(eta > 0.0 && eta <= 1.0)) return fail(WISE_ERR_INVALID_ARG, "eta %g outside (0, 1]", eta);
  if (nblk > 64 * 32) return fail(WISE_ERR_UNSUPPORTED, "n_blocks %d above 2048", nblk);
  const int64_t need = max_nnz(nblk, (int64_t)desc->batch * desc->heads, 0);
  if (need >= (int64_t)INT32_MAX)
    return fail(WISE_ERR_UNSUPPORTED, "worst-case nnz %lld does not fit int32", (long long)need);
  if (col_capacity < need)
    return fail(WISE_ERR_CAPACITY, "col_capacity %lld below worst-case nnz %lld", (long long)col_capacity,
                (long long)need);
  SelectParams p{};
  p.mass = step_mass;
  p.row_ptr = row_ptr;
  p.col_idx = col_idx;
  p.n_rows = (int32_t)n_rows;
  p.nblk = nblk;
  p.max_blocks = 0;
  p.n_steps = 1.0;
  p.eta = eta;
  p.kind = kind;
  p.n_mass = n_mass;
  p.mass_stride = n_rows * nblk;
  p.nnz = nnz;
  const hipError_t e = launch_select(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WISE_ERR_HIP, "selection launch failed: %s", hipGetErrorString(e));
  return ok();
}

wise_status_t wise_support_mass(const wise_attn_desc_t* desc, const float* mass, const int32_t* row_ptr,
                                const int32_t* col_idx, float* retained, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  if (n_rows == 0) return ok();
  if (mass == nullptr || row_ptr == nullptr || col_idx == nullptr || retained == nullptr)
    return fail(WISE_ERR_INVALID_ARG, "mass / row_ptr / col_idx / retained is NULL");
  if ((reinterpret_cast<uintptr_t>(mass) | reinterpret_cast<uintptr_t>(row_ptr) |
       reinterpret_cast<uintptr_t>(col_idx) | reinterpret_cast<uintptr_t>(retained)) & 3u)
    return fail(WISE_ERR_INVALID_ARG, "mass / row_ptr / col_idx / retained not 4-byte aligned");
  if (nblk > 64 * 32) return fail(WISE_ERR_UNSUPPORTED, "n_blocks %d above 2048", nblk);
  const hipError_t e = launch_support_mass(mass, row_ptr, col_idx, retained, (int)n_rows, nblk,
                                           static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WISE_ERR_HIP, "support-mass launch failed: %s", hipGetErrorString(e));
  return ok();
}

wise_status_t wise_support_overlap(const wise_attn_desc_t* desc, const int32_t* row_ptr_a,
                                   const int32_t* col_idx_a, const int32_t* row_ptr_b, const int32_t* col_idx_b,
                                   int32_t* n_inter, int32_t* n_union, void* stream) {
  int32_t nblk;
  int64_t n_rows;
  wise_status_t st = check_desc(desc, &nblk, &n_rows);
  if (st != WISE_OK) return st;
  if (n_rows == 0) return ok();
  if (row_ptr_a == nullptr || col_idx_a == nullptr || row_ptr_b == nullptr || col_idx_b == nullptr ||
      n_inter == nullptr || n_union == nullptr)
    return fail(WISE_ERR_INVALID_ARG, "a CSR array or an output is NULL");
  if ((reinterpret_cast<uintptr_t>(row_ptr_a) | reinterpret_cast<uintptr_t>(col_idx_a) |
       reinterpret_cast<uintptr_t>(row_ptr_b) | reinterpret_cast<uintptr_t>(col_idx_b) |
       reinterpret_cast<uintptr_t>(n_inter) | reinterpret_cast<uintptr_t>(n_union)) & 3u)
    return fail(WISE_ERR_INVALID_ARG, "CSR arrays / outputs not 4-byte aligned");
  if (nblk > 64 * 32) return fail(WISE_ERR_UNSUPPORTED, "n_blocks %d above 2048", nblk);
  const hipError_t e = launch_support_overlap(row_ptr_a, col_idx_a, row_ptr_b, col_idx_b, n_inter, n_union,
                                              (int)n_rows, nblk, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(WISE_ERR_HIP, "support-overlap launch failed: %s", hipGetErrorString(e));
  return ok();
}

const char* wise_status_string(wise_status_t status) {
  switch (status) {
    case WISE_OK: return "WISE_OK";
    case WISE_ERR_INVALID_ARG: return "WISE_ERR_INVALID_ARG";
    case WISE_ERR_UNSUPPORTED: return "WISE_ERR_UNSUPPORTED";
    case WISE_ERR_CAPACITY: return "WISE_ERR_CAPACITY";
    case WISE_ERR_HIP: return "WISE_ERR_HIP";
    case WISE_ERR_OVERFLOW: return "WISE_ERR_OVERFLOW";
  }
  return "WISE_ERR_UNKNOWN";
}

const char* wise_last_error(void) { return g_last_error; }

int32_t wise_abi_version(void) { return WISE_ABI_VERSION; }

}  // extern "C"
