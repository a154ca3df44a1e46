// Flash-style causal attention kernel for gfx950 (CDNA4), bf16 MFMA.
//
// One workgroup owns one row = (batch*head, query block q) of B = BLK
// queries; wave w of the workgroup owns queries [q*B + 32w, q*B + 32w + 32).
// The workgroup walks a list of key blocks (all of 0..q for the dense modes,
// the CSR row for the sparse mode), KT keys at a time:
//
//   global --(16-byte loads, prefetched one tile ahead into VGPRs)--> LDS
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K tile from LDS, Q in VGPRs
//   P   = exp2(S^T * scale*log2e - m)   (fp32, lazily rescaled running max)
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, V^T tile from LDS, P in VGPRs
//
// Computing the transposed score tile makes the MFMA accumulator layout of
// S^T (lane = query, 16 keys per lane) coincide with the B-operand layout
// the PV product needs, so P never leaves registers.  V is transposed on its
// way into LDS (4 keys x 8 dims per thread, packed 8-byte LDS stores).
//
// Softmax: the reference max m of a query is only raised when a new score
// exceeds it by more than 2^kTau (in log2 units); otherwise P may grow up to
// 2^kTau, which fp32 accumulators and bf16 P operands absorb without loss
// of relative precision.  This keeps the per-tile cross-lane max reduction
// off the common path.  The block mass of Eq. (5) reuses the same fp32 P:
// each (query, key block) partial sum is stored in LDS relative to m and
// normalised by the query's final row sum in the epilogue.
#pragma once

#include "wise_internal.h"

namespace wise {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kTau = 8.0f;  // lazy-rescale slack, log2 units

// (a.lo16, b.lo16) and (a.hi16, b.hi16) as packed 32-bit words (one v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

template <int D, int BLK, int KT>
struct AttnShape {
  static constexpr int kWaves = BLK / 32;
  static constexpr int kThreads = 64 * kWaves;
  // LDS row strides (u16 elements).  K rows: D/8 + 1 chunks of 16 bytes (odd,
  // so the 16 rows read per pass by the QK operand land on distinct banks).
  // V rows: (stride in chunks) % 16 in {4, 12}, so the transposing reads of
  // 4 rows x 4 chunks per pass and the 16-chunk row stores are conflict free.
  static constexpr int kKsStride = D + 8;
  static constexpr int kVChunks = (D / 8) % 16 == 4 || (D / 8) % 16 == 12 ? D / 8 : D / 8 + 4;
  static constexpr int kVStride = kVChunks * 8;
  static constexpr int kSub = BLK / KT;      // key tiles per key block
  static constexpr int kChunks = D / 16;     // K-steps of the QK^T product
  static constexpr int kDTiles = D / 32;     // 32-wide output column tiles
  static constexpr int kM = KT / 32;         // 32-key sub-tiles per key tile
  static constexpr int kUnits = KT * D / 8;  // 16-byte chunks of a K or V tile
  static constexpr int kPer = (kUnits + kThreads - 1) / kThreads;
  static constexpr size_t kTileLds = (size_t)KT * kKsStride * 2 + (size_t)KT * kVStride * 2;
  static_assert(D % 32 == 0 && BLK % KT == 0 && KT % 32 == 0, "tile shape");
  static_assert(kVChunks % 16 == 4 || kVChunks % 16 == 12, "V stride");
};

template <int D, int BLK, int KT>
__host__ __device__ constexpr size_t attn_lds_need(int mode, int nblk) {
  return AttnShape<D, BLK, KT>::kTileLds +
         (mode == kDenseMass ? ((size_t)nblk * (BLK + 1) + BLK) * 4 : 0) +
         (mode == kSparse ? ((size_t)nblk + 1) * 4 : 0);
}

// Global -> VGPR prefetch of one key tile, through buffer resources that
// span one head of K and V (hardware-checked bounds, scalar tile offset,
// lane offsets fixed for the whole kernel).  A tile is a contiguous run of
// KT rows of K (and of V), read as 16-byte chunks.
template <int D, int BLK, int KT>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                          int key0, int tid,
                                          u32x4_t (&kreg)[AttnShape<D, BLK, KT>::kPer],
                                          u32x4_t (&vreg)[AttnShape<D, BLK, KT>::kPer]) {
  using Sh = AttnShape<D, BLK, KT>;
  constexpr int NT = Sh::kThreads;
  const int tile_off = key0 * D * 2;
#pragma unroll
  for (int i = 0; i < Sh::kPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kUnits % NT == 0 || u < Sh::kUnits) {
      kreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, u * 16, tile_off, 0));
      vreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, u * 16, tile_off, 0));
    }
  }
}

// VGPR -> LDS: K and V both row-major with padded rows.
template <int D, int BLK, int KT>
__device__ __forceinline__ void store_tile(uint16_t* Ks, uint16_t* Vs, int tid,
                                           const u32x4_t (&kreg)[AttnShape<D, BLK, KT>::kPer],
                                           const u32x4_t (&vreg)[AttnShape<D, BLK, KT>::kPer]) {
  using Sh = AttnShape<D, BLK, KT>;
  constexpr int NT = Sh::kThreads;
#pragma unroll
  for (int i = 0; i < Sh::kPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kUnits % NT == 0 || u < Sh::kUnits) {
      const int r = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<u32x4_t*>(Ks + r * Sh::kKsStride + c8 * 8) = kreg[i];
      *reinterpret_cast<u32x4_t*>(Vs + r * Sh::kVStride + c8 * 8) = vreg[i];
    }
  }
}

// Scores of one key tile: causal mask (MASKED: diagonal block only), the
// lazy-rescale check, and the rare rescale of everything accumulated so far.
template <int D, int BLK, int KT, int MODE, bool MASKED>
__device__ __forceinline__ void softmax_prep(float* part, float scale_log2, int rel, int g, int n,
                                             int wave, int kb, float& m_ref, float& l_part,
                                             float& blk_part,
                                             f32x16_t (&s)[AttnShape<D, BLK, KT>::kM],
                                             f32x16_t (&oacc)[AttnShape<D, BLK, KT>::kDTiles]) {
  using Sh = AttnShape<D, BLK, KT>;
  if constexpr (MASKED) {
    // key offset within the tile > query offset within the tile -> -inf
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int koff = m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
        s[m][i] = (koff > rel) ? -INFINITY : s[m][i];
      }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
    for (int i = 0; i < 16; ++i) tmax = fmaxf(tmax, s[m][i]);
  const float tmax2 = tmax * scale_log2;  // scale > 0: max commutes with scaling

  if (__any(tmax2 > m_ref + kTau)) {
    // Rare path: raise the reference max of the queries that need it and
    // rescale everything accumulated relative to the old one.
    const float rmax = fmaxf(tmax2, __shfl_xor(tmax2, 32));
    const float m_new = (rmax > m_ref + kTau) ? rmax : m_ref;
    const float f = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
    for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) oacc[t][i] *= f;
    l_part *= f;
    if constexpr (MODE == kDenseMass) {
      blk_part *= f;
      if (g == 0 && f != 1.f)
        for (int b = 0; b < kb; ++b) part[b * (BLK + 1) + wave * 32 + n] *= f;
    }
    m_ref = m_new;
  }
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <int D, int BLK, int KT, int MODE>
__global__ void __launch_bounds__(64 * (BLK / 32), 2) wise_attn_kernel(AttnParams p) {
  using Sh = AttnShape<D, BLK, KT>;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vs = Ks + KT * Sh::kKsStride;
  int32_t* blist = reinterpret_cast<int32_t*>(Vs + KT * Sh::kVStride);   // kSparse: [nblk + 1]
  float* part = reinterpret_cast<float*>(Vs + KT * Sh::kVStride);       // kDenseMass: [nblk][BLK+1]
  float* invl = part + (size_t)p.nblk * (BLK + 1);                      // kDenseMass: [BLK]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;  // query within the wave; also key row within a 32-key MFMA tile
  const int g = lane >> 5;  // lane half

  // Longest rows first: blockIdx.x runs over query blocks from the last one.
  const int L = blockIdx.x;
  const int qb = p.nblk - 1 - L / p.heads_total;
  const int bh = L % p.heads_total;
  const int row = bh * p.nblk + qb;

  const size_t head_off = (size_t)bh * p.seq * D;
  const uint16_t* Qh = p.q + head_off;
  const uint16_t* Kh = p.k + head_off;
  const uint16_t* Vh = p.v + head_off;
  const int qrow = qb * BLK + wave * 32 + n;

  bf16x8_t qf[Sh::kChunks];
#pragma unroll
  for (int c = 0; c < Sh::kChunks; ++c)
    qf[c] = *reinterpret_cast<const bf16x8_t*>(Qh + (size_t)qrow * D + c * 16 + 8 * g);

  // Key blocks of this row.  Dense: 0..qb.  Sparse: the CSR row, compacted
  // into LDS by wave 0; entries out of [0, qb], repeated or not ascending
  // are dropped, so every listed block is read once and the diagonal block,
  // if listed, is last.
  int n_blk = qb + 1;
  bool has_diag = true;
  if constexpr (MODE == kSparse) {
    if (wave == 0) {
      int e_begin = p.row_ptr[row];
      int e_end = p.row_ptr[row + 1];
      if (e_end < e_begin) e_end = e_begin;
      int carry = -1, count = 0;
      for (int base = e_begin; base < e_end; base += 64) {
        const int idx = base + lane;
        const int c = idx < e_end ? p.col_idx[idx] : -1;
        const bool inr = idx < e_end && c >= 0 && c <= qb;
        int incl = inr ? c : -1;  // inclusive prefix max over lanes
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int y = __shfl_up(incl, off);
          if (lane >= off) incl = max(incl, y);
        }
        int excl = __shfl_up(incl, 1);
        if (lane == 0) excl = -1;
        excl = max(excl, carry);
        const bool acc = inr && c > excl;
        const uint64_t bal = __ballot(acc);
        if (acc) blist[1 + count + __popcll(bal & ((1ull << lane) - 1ull))] = c;
        count += __popcll(bal);
        carry = max(carry, __shfl(incl, 63));
      }
      if (lane == 0) blist[0] = count;
    }
    __syncthreads();
    n_blk = __builtin_amdgcn_readfirstlane(blist[0]);
    has_diag = n_blk > 0 && __builtin_amdgcn_readfirstlane(blist[n_blk]) == qb;
  }
  auto block_of = [&](int e) -> int {
    if constexpr (MODE == kSparse) return __builtin_amdgcn_readfirstlane(blist[1 + e]);
    else return e;
  };
  const int n_tiles = n_blk * Sh::kSub;
  const int n_main = (n_blk - (has_diag ? 1 : 0)) * Sh::kSub;  // tiles without masking

  f32x16_t oacc[Sh::kDTiles];
#pragma unroll
  for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  float m_ref = -INFINITY;  // identical in both lanes of a query
  float l_part = 0.f;       // this lane's share of the row sum
  float blk_part = 0.f;     // this lane's share of the current key block's mass

  u32x4_t kreg[Sh::kPer];
  u32x4_t vreg[Sh::kPer];

  // Lane address of the PV operand (V^T, 32 dims x 16 keys) read with
  // ds_read_b64_tr_b16: within each 16-lane group G = lane/16, source lane
  // s = lane%16 points at row 4g + s/4 (+ 32m + 16kk + 8j) and dims
  // 16(G%2) + 4(s%4) (+ 32dt); lane i of the group then receives 4
  // consecutive keys at dim 16(G%2) + i, which is the A-operand layout.
  const int v_lane_off = (4 * g + ((lane & 15) >> 2)) * Sh::kVStride + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  // Buffer resources over this head's K and V (word 3: raw 32-bit data format).
  const int head_bytes = p.seq * D * 2;
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kh), 0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vh), 0, head_bytes, 0x00020000);

  if (n_tiles > 0) load_tile<D, BLK, KT>(krs, vrs, block_of(0) * BLK, tid, kreg, vreg);

  // One pipeline step: publish the prefetched tile, prefetch the next one,
  // then compute on the published tile.
  auto step = [&]<bool MASKED>(int it) __attribute__((always_inline)) {
    const int sub = it % Sh::kSub;
    const int kb = block_of(it / Sh::kSub);
    const int key0 = kb * BLK + sub * KT;

    __syncthreads();  // previous tile fully consumed
    store_tile<D, BLK, KT>(Ks, Vs, tid, kreg, vreg);
    __syncthreads();
    if (it + 1 < n_tiles)
      load_tile<D, BLK, KT>(krs, vrs, block_of((it + 1) / Sh::kSub) * BLK + ((it + 1) % Sh::kSub) * KT,
                            tid, kreg, vreg);

    // S^T = K Q^T
    f32x16_t s[Sh::kM];
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m) {
#pragma unroll
      for (int i = 0; i < 16; ++i) s[m][i] = 0.f;
#pragma unroll
      for (int c = 0; c < Sh::kChunks; ++c) {
        const bf16x8_t a =
            *reinterpret_cast<const bf16x8_t*>(Ks + (m * 32 + n) * Sh::kKsStride + c * 16 + 8 * g);
        s[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], s[m], 0, 0, 0);
      }
    }

    softmax_prep<D, BLK, KT, MODE, MASKED>(part, p.scale_log2, qrow - key0, g, n, wave, kb, m_ref,
                                           l_part, blk_part, s, oacc);

    // P = exp2(s * scale*log2e - m) per 32-key sub-tile, then that
    // sub-tile's O^T += V^T P^T; the exponentials of sub-tile m+1 are
    // independent of the MFMAs of sub-tile m.  Masked scores are -inf -> 0.
    const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
    float tsum = 0.f;
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m) {
      bf16x8_t pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[m][kk * 8 + e], p.scale_log2, neg_m));
          if constexpr (MODE == kDenseMass) tsum += pv;   // block mass needs the fp32 values
          pf[kk][e] = (__bf16)pv;
        }
      if constexpr (MODE != kDenseMass) {
        // Row sum of the bf16 operands themselves (the same values the PV
        // product uses), two per packed dot product.
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const bf16x2_t pair = {pf[kk][2 * w], pf[kk][2 * w + 1]};
            tsum = __builtin_amdgcn_fdot2_f32_bf16(pair, one, tsum, false);
          }
      }
#pragma unroll
      for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint16_t* vp = Vs + v_lane_off + (32 * m + 16 * kk) * Sh::kVStride + 32 * t;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp + 8 * Sh::kVStride));
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[t], 0, 0, 0);
        }
    }
    l_part += tsum;
    if constexpr (MODE == kDenseMass) blk_part += tsum;

    if constexpr (MODE == kDenseMass) {
      if (sub == Sh::kSub - 1) {
        const float bp = blk_part + __shfl_xor(blk_part, 32);
        if (g == 0) part[kb * (BLK + 1) + wave * 32 + n] = bp;
        blk_part = 0.f;
      }
    }
  };

  int it = 0;
  for (; it < n_main; ++it) step.template operator()<false>(it);
  for (; it < n_tiles; ++it) step.template operator()<true>(it);

  // ---- epilogue -----------------------------------------------------------
  const float lt = l_part + __shfl_xor(l_part, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* Oh = p.o + head_off + (size_t)qrow * D;
#pragma unroll
  for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      __bf16 b0 = (__bf16)(oacc[t][4 * j + 0] * inv);
      __bf16 b1 = (__bf16)(oacc[t][4 * j + 1] * inv);
      __bf16 b2 = (__bf16)(oacc[t][4 * j + 2] * inv);
      __bf16 b3 = (__bf16)(oacc[t][4 * j + 3] * inv);
      u32x2_t w;
      w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
      w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      *reinterpret_cast<u32x2_t*>(Oh + t * 32 + 8 * j + 4 * g) = w;
    }

  if (MODE == kDense && p.lse != nullptr && g == 0) {
    const float lse = (lt > 0.f) ? (m_ref + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
    p.lse[(size_t)bh * p.seq + qrow] = lse;
  }

  if constexpr (MODE == kDenseMass) {
    if (g == 0) invl[wave * 32 + n] = inv;
    __syncthreads();
    float* mrow = p.mass + (size_t)row * p.nblk;
    for (int b = tid; b <= qb; b += Sh::kThreads) {
      const float* pr = part + b * (BLK + 1);
      float acc = 0.f;
      for (int i = 0; i < BLK; ++i) acc = fmaf(pr[i], invl[i], acc);
      mrow[b] += acc * (1.0f / BLK);
    }
  }
}

template <int D, int BLK, int KT, int MODE>
hipError_t launch_attn_t(const AttnParams& p, hipStream_t stream) {
  using Sh = AttnShape<D, BLK, KT>;
  const size_t lds = attn_lds_need<D, BLK, KT>(MODE, p.nblk);
  auto kern = wise_attn_kernel<D, BLK, KT, MODE>;
  static bool attr_set = false;  // benign race: idempotent attribute
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const unsigned grid = (unsigned)p.heads_total * (unsigned)p.nblk;
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Sh::kThreads), lds, stream, p);
  return hipGetLastError();
}

// Key tile: 64 keys when it fits; the mass mode at long contexts drops to
// 32 keys so that the per-(query, block) partials still fit in LDS.
template <int D, int BLK>
int choose_kt(int mode, int nblk) {
  if constexpr (BLK == 32) {
    return attn_lds_need<D, 32, 32>(mode, nblk) <= kMaxLds ? 32 : 0;
  } else if constexpr (BLK == 64 && D == 128) {
    // The mass mode's extra live state does not fit 64-key tiles in 256 VGPRs.
    if (mode != kDenseMass && attn_lds_need<D, BLK, 64>(mode, nblk) <= kMaxLds) return 64;
    if (attn_lds_need<D, BLK, 32>(mode, nblk) <= kMaxLds) return 32;
    return 0;
  } else {
    if (attn_lds_need<D, BLK, 64>(mode, nblk) <= kMaxLds) return 64;
    if (attn_lds_need<D, BLK, 32>(mode, nblk) <= kMaxLds) return 32;
    return 0;
  }
}

template <int D, int BLK>
hipError_t launch_attn_blk(int mode, const AttnParams& p, hipStream_t stream) {
  const int kt = choose_kt<D, BLK>(mode, p.nblk);
  if (kt == 0) return hipErrorInvalidValue;
  if constexpr (BLK == 32) {
    switch (mode) {
      case kDense: return launch_attn_t<D, BLK, 32, kDense>(p, stream);
      case kDenseMass: return launch_attn_t<D, BLK, 32, kDenseMass>(p, stream);
      default: return launch_attn_t<D, BLK, 32, kSparse>(p, stream);
    }
  } else {
    if (mode == kDense) return launch_attn_t<D, BLK, 64, kDense>(p, stream);
    if (mode == kSparse) return launch_attn_t<D, BLK, 64, kSparse>(p, stream);
    if (kt == 64) return launch_attn_t<D, BLK, 64, kDenseMass>(p, stream);
    return launch_attn_t<D, BLK, 32, kDenseMass>(p, stream);
  }
}

template <int D>
size_t attn_lds_bytes_d(int block, int mode, int nblk) {
  switch (block) {
    case 32: return choose_kt<D, 32>(mode, nblk) ? attn_lds_need<D, 32, 32>(mode, nblk) : 0;
    case 64: {
      int kt = choose_kt<D, 64>(mode, nblk);
      return kt == 64 ? attn_lds_need<D, 64, 64>(mode, nblk)
                      : (kt == 32 ? attn_lds_need<D, 64, 32>(mode, nblk) : 0);
    }
    case 128: {
      int kt = choose_kt<D, 128>(mode, nblk);
      return kt == 64 ? attn_lds_need<D, 128, 64>(mode, nblk)
                      : (kt == 32 ? attn_lds_need<D, 128, 32>(mode, nblk) : 0);
    }
  }
  return 0;
}

template <int D>
hipError_t launch_attn_d(int block, int mode, const AttnParams& p, hipStream_t stream) {
  switch (block) {
    case 32: return launch_attn_blk<D, 32>(mode, p, stream);
    case 64: return launch_attn_blk<D, 64>(mode, p, stream);
    case 128: return launch_attn_blk<D, 128>(mode, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace wise
