// Internal declarations shared by the HIP translation units of libwise.
// Not part of the public interface (that is include/wise.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wise {

// Kinds of attention launch: the same kernel body serves all of them.
enum AttnMode : int {
  kDense = 0,       // Eq. (2) over every admissible key block
  kDenseMass = 1,   // Eq. (2) plus the block mass of Eq. (5), added into `mass`
  kSparse = 2,      // Eq. (8): only the key blocks listed in the CSR row
  kMassTwoPass = 3, // kDenseMass in two passes over the keys (launcher's choice
                    // for long rows): row max and sum first, then P, O and mass
  kDenseMassWs = 4  // kDenseMass with the per-(query, key block) partials in a
                    // caller's workspace in HBM instead of LDS (blocks 64, 128)
};

struct AttnParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;              // optional, kDense only
  float* mass;             // kDenseMass only
  const int32_t* row_ptr;  // kSparse only
  const int32_t* col_idx;  // kSparse only
  int32_t heads_total;     // batch * heads
  int32_t heads;           // query heads per batch entry
  int32_t kv_group;        // query heads per K/V head (1: one K/V head each)
  int32_t seq;
  int32_t nblk;            // seq / block
  float scale_log2;        // softmax scale * log2(e)
  int32_t head_chunk;      // workgroup order (set by the launcher): 0, or heads per chunk within an XCD
  float* work;             // kDenseMassWs: partials [row][key block][query of the row]
};

struct AttnLaunch {
  int head_dim;
  int block;
  int mode;
};

// Bytes of dynamic LDS a launch needs (0 if the shape is not built).
size_t attn_lds_bytes(int head_dim, int block, int mode, int nblk);

// Launch one attention pass over all rows; returns hipSuccess or the error.
hipError_t launch_attn(const AttnLaunch& cfg, const AttnParams& p, hipStream_t stream);

// Per-D launchers (one translation unit each).
hipError_t launch_attn_d64(int block, int mode, const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_d96(int block, int mode, const AttnParams& p, hipStream_t stream);
hipError_t launch_attn_d128(int block, int mode, const AttnParams& p, hipStream_t stream);

// Selection kinds (values match wise_select_kind_t, 0 = the main selection).
enum SelectKind : int {
  kSelMean = 0,         // Eq. (6) on the mean of the accumulated discovery masses
  kSelUnion = 1,        // Eq. (6) left / Eq. (18): union of per-step supports
  kSelStatic = 2,       // Eq. (19): first step's support
  kSelMassMatched = 3,  // Eq. (20)-(21)
  kSelSizeMatched = 4   // Eq. (22)
};

struct SelectParams {
  const float* mass;   // kSelMean: accumulated sum; else [n_mass] single-step masses
  int32_t* row_ptr;
  int32_t* col_idx;
  int32_t n_rows;
  int32_t nblk;
  int32_t max_blocks;  // 0 = no cap (kSelMean only)
  double n_steps;      // discovery steps summed into mass (kSelMean)
  double eta;
  int32_t kind;        // SelectKind
  int32_t n_mass;      // step masses given (variants)
  int64_t mass_stride; // elements between consecutive step masses
  int64_t* nnz;        // optional: total entries, written after the scan
};

hipError_t launch_select(const SelectParams& p, hipStream_t stream);

// Diagnostics: retained mass of a support, and per-row overlap of two supports.
hipError_t launch_support_mass(const float* mass, const int32_t* row_ptr, const int32_t* col_idx, float* out,
                               int n_rows, int nblk, hipStream_t stream);
hipError_t launch_support_overlap(const int32_t* rp_a, const int32_t* ci_a, const int32_t* rp_b,
                                  const int32_t* ci_b, int32_t* inter, int32_t* uni, int n_rows, int nblk,
                                  hipStream_t stream);

// LDS budget of one workgroup on gfx950.
constexpr size_t kMaxLds = 160 * 1024;

// Per-launch trace on stderr when the environment sets WISE_TRACE to a
// non-empty value other than "0" (read once per process): kernel, grid,
// workgroup size, dynamic LDS and launch parameters, one line per launch.
bool trace_enabled();
void trace_launch(const char* kernel, unsigned grid, unsigned threads, size_t lds, const char* fmt, ...)
    __attribute__((format(printf, 5, 6)));

}  // namespace wise
