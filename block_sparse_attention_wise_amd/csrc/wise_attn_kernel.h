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
  static constexpr int kKsStride = D + 8;    // u16 per K row in LDS (16 B pad)
  static constexpr int kVtStride = KT + 8;   // u16 per V^T row in LDS (16 B pad)
  static constexpr int kSub = BLK / KT;      // key tiles per key block
  static constexpr int kChunks = D / 16;     // K-steps of the QK^T product
  static constexpr int kDTiles = D / 32;     // 32-wide output column tiles
  static constexpr int kM = KT / 32;         // 32-key sub-tiles per key tile
  static constexpr int kKUnits = KT * D / 8;         // 16-byte chunks of a K tile
  static constexpr int kVUnits = (KT / 4) * (D / 8); // 4-key x 8-dim pieces of V
  static constexpr int kKPer = (kKUnits + kThreads - 1) / kThreads;
  static constexpr int kVPer = (kVUnits + kThreads - 1) / kThreads;
  static constexpr size_t kTileLds = (size_t)KT * kKsStride * 2 + (size_t)D * kVtStride * 2;
  static_assert(D % 32 == 0 && BLK % KT == 0 && KT % 32 == 0, "tile shape");
};

template <int D, int BLK, int KT>
__host__ __device__ constexpr size_t attn_lds_need(int mode, int nblk) {
  return AttnShape<D, BLK, KT>::kTileLds +
         (mode == kDenseMass ? ((size_t)nblk * (BLK + 1) + BLK) * 4 : 0) +
         (mode == kSparse ? ((size_t)nblk + 1) * 4 : 0);
}

// Stored position of key kappa (0..KT-1) inside a V^T row: within each
// group of 16 keys the key quads are stored in the order 0, 2, 1, 3, so the
// 8 keys an MFMA lane group needs ({4g..4g+3} and {8+4g..8+4g+3}) are
// contiguous.
__device__ __forceinline__ int vt_pos(int kappa) {
  int quad = (kappa >> 2) & 3;
  int sq = (quad == 1) ? 2 : (quad == 2 ? 1 : quad);
  return (kappa & ~15) | (sq << 2) | (kappa & 3);
}

// Global -> VGPR prefetch of one key tile, through buffer resources that
// span one head of K and V (hardware-checked bounds, scalar tile offset,
// lane offsets fixed for the whole kernel).  K is a contiguous run of KT
// rows, read as 16-byte chunks; V is read as 4-key x 8-dim pieces so they
// can be transposed on the way into LDS.
template <int D, int BLK, int KT>
__device__ __forceinline__ void load_tile(__amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                                          int key0, int tid,
                                          u32x4_t (&kreg)[AttnShape<D, BLK, KT>::kKPer],
                                          u32x4_t (&vreg)[AttnShape<D, BLK, KT>::kVPer][4]) {
  using Sh = AttnShape<D, BLK, KT>;
  constexpr int NT = Sh::kThreads;
  const int tile_off = key0 * D * 2;
#pragma unroll
  for (int i = 0; i < Sh::kKPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kKUnits % NT == 0 || u < Sh::kKUnits)
      kreg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(krs, u * 16, tile_off, 0));
  }
#pragma unroll
  for (int i = 0; i < Sh::kVPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kVUnits % NT == 0 || u < Sh::kVUnits) {
      const int a = u % (KT / 4), dc = u / (KT / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        vreg[i][j] = __builtin_bit_cast(
            u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(vrs, (4 * a + j) * D * 2 + dc * 16, tile_off, 0));
    }
  }
}

// VGPR -> LDS: K row-major (padded rows), V transposed to [dim][key] with
// the key order of vt_pos.
template <int D, int BLK, int KT>
__device__ __forceinline__ void store_tile(uint16_t* Ks, uint16_t* Vt, int tid,
                                           const u32x4_t (&kreg)[AttnShape<D, BLK, KT>::kKPer],
                                           const u32x4_t (&vreg)[AttnShape<D, BLK, KT>::kVPer][4]) {
  using Sh = AttnShape<D, BLK, KT>;
  constexpr int NT = Sh::kThreads;
#pragma unroll
  for (int i = 0; i < Sh::kKPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kKUnits % NT == 0 || u < Sh::kKUnits) {
      const int r = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<u32x4_t*>(Ks + r * Sh::kKsStride + c8 * 8) = kreg[i];
    }
  }
#pragma unroll
  for (int i = 0; i < Sh::kVPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kVUnits % NT == 0 || u < Sh::kVUnits) {
      const int a = u % (KT / 4), dc = u / (KT / 4);
      uint16_t* dst = Vt + (dc * 8) * Sh::kVtStride + vt_pos(4 * a);
      const u32x4_t k0 = vreg[i][0], k1 = vreg[i][1], k2 = vreg[i][2], k3 = vreg[i][3];
      const uint32_t w0[4] = {k0.x, k0.y, k0.z, k0.w};
      const uint32_t w1[4] = {k1.x, k1.y, k1.z, k1.w};
      const uint32_t w2[4] = {k2.x, k2.y, k2.z, k2.w};
      const uint32_t w3[4] = {k3.x, k3.y, k3.z, k3.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        // dims 2h and 2h+1 of the 4 keys
        u32x2_t even, odd;
        even.x = pack_lo(w0[h], w1[h]);
        even.y = pack_lo(w2[h], w3[h]);
        odd.x = pack_hi(w0[h], w1[h]);
        odd.y = pack_hi(w2[h], w3[h]);
        *reinterpret_cast<u32x2_t*>(dst + (2 * h) * Sh::kVtStride) = even;
        *reinterpret_cast<u32x2_t*>(dst + (2 * h + 1) * Sh::kVtStride) = odd;
      }
    }
  }
}

// Scores of one key tile -> P (bf16 operands) and running statistics.
// MASKED applies the causal mask key > query (diagonal block only).
template <int D, int BLK, int KT, int MODE, bool MASKED>
__device__ __forceinline__ void softmax_tile(float* part, float scale_log2, int rel, int g, int n,
                                             int wave, int kb, float& m_ref, float& l_part,
                                             float& blk_part,
                                             f32x16_t (&s)[AttnShape<D, BLK, KT>::kM],
                                             bf16x8_t (&pf)[AttnShape<D, BLK, KT>::kM][2],
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

  // P = exp2(s * scale*log2e - m); masked scores are -inf and give 0.
  const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
  float tsum = 0.f;
#pragma unroll
  for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
    for (int kk = 0; kk < 2; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[m][kk * 8 + e], scale_log2, neg_m));
        tsum += pv;
        pf[m][kk][e] = (__bf16)pv;
      }
  l_part += tsum;
  if constexpr (MODE == kDenseMass) blk_part += tsum;
}

template <int D, int BLK, int KT, int MODE>
__global__ void __launch_bounds__(64 * (BLK / 32), 2) wise_attn_kernel(AttnParams p) {
  using Sh = AttnShape<D, BLK, KT>;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vt = Ks + KT * Sh::kKsStride;
  int32_t* blist = reinterpret_cast<int32_t*>(Vt + D * Sh::kVtStride);   // kSparse: [nblk + 1]
  float* part = reinterpret_cast<float*>(Vt + D * Sh::kVtStride);       // kDenseMass: [nblk][BLK+1]
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

  u32x4_t kreg[Sh::kKPer];
  u32x4_t vreg[Sh::kVPer][4];

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
    store_tile<D, BLK, KT>(Ks, Vt, tid, kreg, vreg);
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

    bf16x8_t pf[Sh::kM][2];
    softmax_tile<D, BLK, KT, MODE, MASKED>(part, p.scale_log2, qrow - key0, g, n, wave, kb, m_ref,
                                           l_part, blk_part, s, pf, oacc);

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
      for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(
              Vt + (t * 32 + n) * Sh::kVtStride + (2 * m + kk) * 16 + 8 * g);
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[m][kk], oacc[t], 0, 0, 0);
        }

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
