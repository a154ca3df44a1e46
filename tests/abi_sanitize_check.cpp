// Host-side validation of the C ABI (include/wise.h), built with the host
// address and undefined-behaviour sanitizers.  Every call below is refused
// (or is an empty no-op) before any device work, so this runs without a GPU;
// the sanitizers check the validation code's own memory accesses and
// arithmetic.  Exits 0 when every status is the expected one.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../include/wise.h"

namespace {
int g_fail = 0;
void expect(const char* what, int got, int want) {
  if (got != want) {
    std::fprintf(stderr, "FAIL %s: status %d, want %d (%s)\n", what, got, want, wise_last_error());
    ++g_fail;
  }
}
wise_attn_desc_t desc(int b, int h, int s, int d, int blk, float scale = 0.f, int kv = 0) {
  wise_attn_desc_t x;
  x.batch = b; x.heads = h; x.seq_len = s; x.head_dim = d; x.block_size = blk;
  x.softmax_scale = scale; x.kv_heads = kv;
  return x;
}
}  // namespace

int main() {
  void* fake = reinterpret_cast<void*>(uintptr_t{0x10000});   // aligned, never dereferenced
  auto* ffake = static_cast<float*>(fake);
  auto* ifake = static_cast<int32_t*>(fake);
  char* cfake = static_cast<char*>(fake);

  expect("abi version", wise_abi_version(), WISE_ABI_VERSION);
  expect("status string", std::strcmp(wise_status_string(WISE_ERR_CAPACITY), "WISE_ERR_CAPACITY"), 0);

  // descriptors
  wise_attn_desc_t d = desc(1, 2, 256, 64, 32);
  expect("null desc", wise_full_attn(nullptr, fake, fake, fake, fake, nullptr, nullptr), WISE_ERR_INVALID_ARG);
  wise_attn_desc_t bad = desc(1, 2, 256, 80, 32);
  expect("head_dim 80", wise_full_attn(&bad, fake, fake, fake, fake, nullptr, nullptr), WISE_ERR_UNSUPPORTED);
  bad = desc(1, 2, 256, 64, 48);
  expect("block 48", wise_sparse_attn(&bad, fake, fake, fake, ifake, ifake, fake, nullptr), WISE_ERR_UNSUPPORTED);
  bad = desc(-1, 2, 256, 64, 32);
  expect("negative batch", wise_full_attn_accum(&bad, fake, fake, fake, fake, ffake, nullptr), WISE_ERR_INVALID_ARG);
  bad = desc(1, 2, 70000, 64, 64);
  expect("seq above 65536", wise_full_attn(&bad, fake, fake, fake, fake, nullptr, nullptr), WISE_ERR_UNSUPPORTED);
  bad = desc(1, 4, 256, 64, 32, 0.f, 3);
  expect("kv_heads 3 of 4", wise_full_attn(&bad, fake, fake, fake, fake, nullptr, nullptr), WISE_ERR_INVALID_ARG);
  bad = desc(1 << 20, 1 << 10, 65536, 64, 16);
  expect("rows overflow", wise_full_attn(&bad, fake, fake, fake, fake, nullptr, nullptr), WISE_ERR_UNSUPPORTED);
  expect("max_nnz of bad desc", (int)wise_select_max_nnz(&bad, 0), -1);

  // pointers and alignment
  expect("q null", wise_full_attn(&d, nullptr, fake, fake, fake, nullptr, nullptr), WISE_ERR_INVALID_ARG);
  expect("k misaligned", wise_full_attn(&d, fake, cfake + 8, fake, cfake + 4096, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("o aliases q", wise_full_attn(&d, fake, cfake + 4096, cfake + 8192, fake, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("mass null", wise_full_attn_accum(&d, fake, fake, fake, cfake + 4096, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("csr null", wise_sparse_attn(&d, fake, fake, fake, nullptr, ifake, cfake + 4096, nullptr),
         WISE_ERR_INVALID_ARG);

  // workspace
  wise_attn_desc_t d64 = desc(1, 2, 256, 64, 64);
  const int64_t need = wise_full_attn_accum_workspace_bytes(&d64);
  expect("workspace bytes", need == 2LL * 4 * 4 * 64 * 4, 1);
  expect("workspace small", wise_full_attn_accum_ws(&d64, fake, fake, fake, cfake + 4096, ffake, cfake + 65536,
                                                    need - 1, nullptr), WISE_ERR_CAPACITY);
  expect("workspace null", wise_full_attn_accum_ws(&d64, fake, fake, fake, cfake + 4096, ffake, nullptr, need,
                                                   nullptr), WISE_ERR_INVALID_ARG);
  wise_attn_desc_t big = desc(1, 65, 4096, 128, 64);
  expect("noalloc above its buffer", wise_full_attn_accum_noalloc(&big, fake, fake, fake, cfake + 4096, ffake,
                                                                  nullptr), WISE_ERR_CAPACITY);

  // selection
  const int64_t cap = wise_select_max_nnz(&d, 0);
  expect("max nnz", cap == 2 * 36, 1);
  expect("eta 0", wise_select_support(&d, ffake, 2, 0.0, 0, ifake, ifake, cap, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("eta above 1", wise_select_support(&d, ffake, 2, 1.5, 0, ifake, ifake, cap, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("n_steps 0", wise_select_support(&d, ffake, 0, 0.9, 0, ifake, ifake, cap, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("capacity", wise_select_support(&d, ffake, 2, 0.9, 0, ifake, ifake, cap - 1, nullptr, nullptr),
         WISE_ERR_CAPACITY);
  expect("nnz misaligned", wise_select_support(&d, ffake, 2, 0.9, 0, ifake, ifake, cap,
                                               reinterpret_cast<int64_t*>(cfake + 4), nullptr), WISE_ERR_INVALID_ARG);
  expect("variant kind", wise_select_variant(&d, 9, ffake, 2, 0.9, ifake, ifake, cap, nullptr, nullptr),
         WISE_ERR_INVALID_ARG);
  expect("static needs one step", wise_select_variant(&d, WISE_SELECT_STATIC, ffake, 2, 0.9, ifake, ifake, cap,
                                                      nullptr, nullptr), WISE_ERR_INVALID_ARG);

  // empty problems: no launch, success
  wise_attn_desc_t empty = desc(0, 4, 256, 64, 64);
  expect("empty dense", wise_full_attn(&empty, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr), WISE_OK);
  expect("empty sparse", wise_sparse_attn(&empty, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr),
         WISE_OK);
  expect("empty diag", wise_support_mass(&empty, nullptr, nullptr, nullptr, nullptr, nullptr), WISE_OK);

  if (g_fail == 0) std::printf("abi validation: all checks passed\n");
  return g_fail == 0 ? 0 : 1;
}
