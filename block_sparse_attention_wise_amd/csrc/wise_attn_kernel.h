// Flash-style causal attention kernel for gfx950 (CDNA4), bf16 MFMA, for
// the three attention steps of "Attention Routing Stabilizes Early:
// Working-Set Inference for Recurrent Language Models" (WISE): dense causal
// attention (Section 3, Eq. 2), the same with the block mass of Section 5.1,
// Eq. (5), and attention inside the working set (Section 5.2, Eq. 7-8).
//
// A workgroup owns RPW adjacent rows = (batch*head, query block q) of
// B = BLK queries each; the waves of a row own 32 queries apiece.  The
// workgroup walks a list of key blocks, KT keys at a time: all of 0..q for
// the dense modes, the union of its rows' CSR lists for the sparse mode
// (each wave computes only on blocks its own row lists):
//
//   global --(buffer_load_dwordx4 ... lds, two stages)--> LDS
//             (mass mode: 16-byte loads into VGPRs, then LDS stores)
//   S^T = K Q^T      v_mfma_f32_32x32x16_bf16, K rows from LDS, Q in VGPRs
//   P   = exp2(S^T * scale*log2e - m)   (fp32, lazily rescaled running max)
//   O^T += V^T P^T   v_mfma_f32_32x32x16_bf16, V^T read from row-major V
//                    with ds_read_b64_tr_b16, P in VGPRs
//
// Computing the transposed score tile makes the MFMA accumulator layout of
// S^T (lane = query, 16 keys per lane) coincide with the B-operand layout
// the PV product needs, so P never leaves registers.
//
// Softmax: the reference max m of a query is only raised when a new scaled
// score exceeds it by more than kTau (log2 units); otherwise P may grow up
// to 2^kTau.  bf16 P operands share fp32's exponent range and the O, l and
// mass accumulators are fp32, so even 2^64 loses no relative precision and
// leaves O far from overflow (2^64 x 2^16 keys x |v|).  A wide slack keeps
// the rescale of O (a multiply per accumulator) and the cross-lane max
// reduction off the common path: with attention logits that keep growing
// along the key walk, a slack of 8 rescaled on 43% of 64-key wave tiles,
// 64 only on each wave's first tile.  The block mass of Eq. (5) reuses the same fp32 P:
// each (query, key block) partial sum is stored relative to m (in LDS, or
// in a caller's workspace in device memory) and normalised by the query's
// final row sum in the epilogue.
#pragma once

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "wise_internal.h"

namespace wise {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kTau = 64.0f;  // lazy-rescale slack, log2 units

// (a.lo16, b.lo16) and (a.hi16, b.hi16) as packed 32-bit words (one v_perm_b32).
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Workgroup barrier that orders LDS accesses only: unlike __syncthreads it
// does not wait for outstanding global->LDS loads, which the caller waits
// for explicitly (s_waitcnt vmcnt) when it needs them.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// s_waitcnt immediate: vmcnt <= 0, expcnt and lgkmcnt not waited for.
constexpr int kWaitVm0 = 0x0F70;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over `bytes` bytes at `base` (word 3: 32-bit raw
// data format, no swizzle).
__device__ __forceinline__ i32x4_t buffer_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4_t d;
  d.x = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
  d.y = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xFFFF);
  d.z = (int)bytes;
  d.w = 0x00020000;
  return d;
}

// 16 bytes per lane from buffer offset voff + soff straight into LDS at
// lds_base + 16 * lane (buffer_load_dwordx4 ... lds; M0 holds the LDS base).
// Written as inline assembly so that the compiler does not track these
// LDS writes: completion is waited for explicitly (s_waitcnt vmcnt before
// the barrier that publishes a stage), and LDS reads of the other stage
// need not wait for them.
// (The compiler warns that M0 is a reserved register; these two helpers are
// the only code that writes it, and declaring the clobber is what keeps the
// compiler from relying on an old M0 value afterwards.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(i32x4_t desc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(desc), "s"(soff)
               : "memory", "m0");
}

// The same load without a compiler memory clobber, for loads into the stage
// that no LDS access of the current step touches: LDS reads of the current
// stage may then be scheduled across it.  It stays ordered with the
// barriers (both are volatile side effects), and completion is waited for
// explicitly as for dma16.
__device__ __forceinline__ void dma16_free(i32x4_t desc, uint32_t lds_base, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(lds_base), "v"(voff), "s"(desc), "s"(soff)
               : "m0");
}
#pragma clang diagnostic pop

template <int D, int BLK, int KT, int RPW = 1>
struct AttnShape {
  static constexpr int kWaves = BLK / 32 * RPW;   // RPW rows of BLK queries per workgroup
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

// K/V tiles written straight from global memory into LDS
// (buffer_load_dwordx4 ... lds): one wave instruction fills 1 KiB of LDS
// contiguously (lane l at +16 l), so rows are unpadded (2D bytes) and bank
// conflicts are avoided by permuting the 16-byte chunks of each row with an
// XOR of row-index bits instead; the permutation is undone on the global
// side of the load, so every lane still reads 16 contiguous bytes.  Two
// stages: the tile after the current one lands while the current one is
// used.
//   K (read as the A operand, 16 rows x one chunk per pass):
//     D=128: chunk ^ (r & 15); D=96: chunk ^ ((r >> 2) & 3); D=64: chunk ^ ((r >> 1) & 7)
//   V (read transposed, 4 rows x 4 chunks per pass):
//     D=128: chunk ^ 4(r & 3);  D=96: identity;            D=64: chunk ^ 4((r >> 1) & 1)
// Both depend on r mod 32 only for K and r mod 8 only for V, so the row
// offsets of the MFMA sub-tiles stay compile-time immediates.
template <int D, int KT, int NT>
struct DmaTile {
  static constexpr int kCpr = D / 8;                          // 16-byte chunks per row
  static constexpr int kTileBytes = KT * D * 2;               // one of K or V
  static constexpr int kStageBytes = 2 * kTileBytes;
  static constexpr int kStages = 2;
  static constexpr int kWaves = NT / 64;
  static constexpr int kInstr = KT * kCpr / 64 / kWaves;      // per wave and tensor
  static constexpr bool kSplits = (KT * kCpr) % (64 * kWaves) == 0;  // whole wave loads
  static __device__ __forceinline__ int kx(int r) {
    return D == 128 ? (r & 15) : D == 96 ? ((r >> 2) & 3) : ((r >> 1) & 7);
  }
  static __device__ __forceinline__ int vx(int r) {
    return D == 128 ? 4 * (r & 3) : D == 96 ? 0 : 4 * ((r >> 1) & 1);
  }
};

template <int MODE>
__host__ __device__ constexpr bool uses_dma() { return MODE != kDenseMass; }

// Rows (query blocks) per workgroup: two adjacent rows for block 64, so
// that four waves share every staged K/V tile (the two rows' key-block
// lists overlap heavily), several one-wave rows for block 32 (rpw32), one
// row for block 128.  The mass mode keeps one row when the per-(query, key
// block) partials of two rows would not fit.
// nblk: physical blocks of BLK keys; LPR logical blocks of BLK/LPR keys per
// physical block (LPR = 2 runs block 16 on 32 x 32 tiles).
template <int D, int BLK, int KT, int RPW, int LPR = 1>
__host__ __device__ constexpr size_t attn_lds_need(int mode, int nblk) {
  return (mode != kDenseMass ? (size_t)DmaTile<D, KT, AttnShape<D, BLK, KT, RPW>::kThreads>::kStages *
                                   DmaTile<D, KT, AttnShape<D, BLK, KT, RPW>::kThreads>::kStageBytes
                             : AttnShape<D, BLK, KT, RPW>::kTileLds) +
         (mode == kDenseMass ? (size_t)RPW * ((size_t)nblk * LPR * (BLK + 1) + BLK) * 4 : 0) +
         (mode == kDenseMassWs ? (size_t)RPW * BLK * 4 : 0) +
         (mode == kMassTwoPass ? (size_t)RPW * LPR * nblk * LPR * (BLK / 32) * 4 : 0) +
         (mode == kSparse ? (size_t)RPW * LPR * ((nblk * LPR + 31) / 32) * 4 + ((size_t)nblk + 1) * 4 : 0);
}

template <int D, int BLK, int KT, int RPW>
__device__ __forceinline__ void load_rows(__amdgpu_buffer_rsrc_t rs, int key0, int tid,
                                          u32x4_t (&reg)[AttnShape<D, BLK, KT, RPW>::kPer]) {
  using Sh = AttnShape<D, BLK, KT, RPW>;
  constexpr int NT = Sh::kThreads;
  const int tile_off = key0 * D * 2;
#pragma unroll
  for (int i = 0; i < Sh::kPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kUnits % NT == 0 || u < Sh::kUnits)
      reg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, u * 16, tile_off, 0));
  }
}

// load_rows for a tile that reaches past the end of the sequence: `rs`
// starts at the tile's first in-range row and every lane's offset is
// clamped to `lim`, the last in-range 16 bytes, so no lane reads outside
// the tensor (the rows past the end receive copies of in-range data).
template <int D, int BLK, int KT, int RPW>
__device__ __forceinline__ void load_rows_clamped(__amdgpu_buffer_rsrc_t rs, int lim, int tid,
                                                  u32x4_t (&reg)[AttnShape<D, BLK, KT, RPW>::kPer]) {
  using Sh = AttnShape<D, BLK, KT, RPW>;
  constexpr int NT = Sh::kThreads;
#pragma unroll
  for (int i = 0; i < Sh::kPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kUnits % NT == 0 || u < Sh::kUnits)
      reg[i] = __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(rs, min(u * 16, lim), 0, 0));
  }
}

// VGPR -> LDS, row-major with padded rows of STRIDE u16.
template <int D, int BLK, int KT, int RPW, int STRIDE>
__device__ __forceinline__ void store_rows(uint16_t* dst, int tid,
                                           const u32x4_t (&reg)[AttnShape<D, BLK, KT, RPW>::kPer]) {
  using Sh = AttnShape<D, BLK, KT, RPW>;
  constexpr int NT = Sh::kThreads;
#pragma unroll
  for (int i = 0; i < Sh::kPer; ++i) {
    const int u = tid + i * NT;
    if (Sh::kUnits % NT == 0 || u < Sh::kUnits) {
      const int r = u / (D / 8), c8 = u % (D / 8);
      *reinterpret_cast<u32x4_t*>(dst + r * STRIDE + c8 * 8) = reg[i];
    }
  }
}

// Scores of one key tile: causal mask (MASKED: diagonal block only), the
// lazy-rescale check, and the rare rescale of everything accumulated so far.
// Returns the larger of run_max and this lane's largest (masked) raw score
// of the tile.  Passing the lane's running raw maximum as run_max cannot
// trigger a rescale by itself: that maximum, scaled, never exceeds the
// reference by more than the threshold.
template <int D, int BLK, int KT, int MODE, bool MASKED>
__device__ __forceinline__ float softmax_prep(float* part, float scale_log2, int rel, int g, int n,
                                             int wave, int kb, float& m_ref, float& l_part,
                                             float& blk_part, float run_max, int pstride,
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
  float tmax = run_max;
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
    // While a query's reference is still -inf nothing has been accumulated
    // for it, so a wave whose queries all start here has nothing to rescale.
    if (!__all(m_ref == -INFINITY)) {
      const float f = (m_new == m_ref) ? 1.f : __builtin_amdgcn_exp2f(m_ref - m_new);
#pragma unroll
      for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[t][i] *= f;
      l_part *= f;
      if constexpr (MODE == kDenseMass || MODE == kDenseMassWs) {
        blk_part *= f;
        if (g == 0 && f != 1.f)
          for (int b = 0; b < kb; ++b) part[(size_t)b * pstride + wave * 32 + n] *= f;
      }
    }
    m_ref = m_new;
  }
  return tmax;
}

typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// LPR = 2: block 16 run on 32-query x 32-key physical tiles.  Each physical
// row holds logical query blocks 2q and 2q+1 (queries 0-15 and 16-31 of the
// wave), each physical key tile logical key blocks 2kb and 2kb+1 (a lane's
// score values 0-7 and 8-15); CSR rows, masses and the sparse masks are per
// logical block.
template <int D, int BLK, int KT, int MODE, int RPW, int LPR = 1>
__global__ void __launch_bounds__(64 * (BLK / 32) * RPW, 2) wise_attn_kernel(AttnParams p) {
  using Sh = AttnShape<D, BLK, KT, RPW>;
  constexpr int WR = BLK / 32;                 // waves per row
  constexpr int kLB = BLK / LPR;               // logical block size
  static_assert(LPR == 1 || (LPR == 2 && BLK == 32 && KT == 32 && RPW <= 2 && MODE != kDense),
                "logical sub-blocks: block 16 on 32 x 32 tiles, at most two rows per workgroup");
  static_assert(RPW * LPR * LPR <= 8, "list-entry tag bits");
  static_assert(MODE != kDenseMassWs || (LPR == 1 && BLK >= 32), "workspace mass mode: blocks 32, 64 and 128");
  constexpr bool kMass1 = (MODE == kDenseMass || MODE == kDenseMassWs);   // one-pass block mass

  using Dm = DmaTile<D, KT, Sh::kThreads>;
  constexpr bool kDma = uses_dma<MODE>();
  static_assert(!kDma || Dm::kSplits, "K/V tile must split into whole wave loads");

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* Ks = reinterpret_cast<uint16_t*>(smem);
  uint16_t* Vs = Ks + KT * Sh::kKsStride;
  unsigned char* extra = smem + (kDma ? (size_t)Dm::kStages * Dm::kStageBytes : Sh::kTileLds);
  const int lnb = p.nblk * LPR;                 // logical blocks per head
  const int nwords = (lnb + 31) / 32;
  uint32_t* bits = reinterpret_cast<uint32_t*>(extra);                  // kSparse: [RPW*LPR][nwords]
  int32_t* ulist = reinterpret_cast<int32_t*>(bits + RPW * LPR * nwords);   // kSparse: [nblk + 1]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int n = lane & 31;  // query within the wave; also key row within a 32-key MFMA tile
  const int g = lane >> 5;  // lane half
  const int slot = wave / WR;   // which of the workgroup's rows this wave serves
  const int wr = wave % WR;

  // Workgroup -> (head, row group).  Workgroups are dealt round-robin to the
  // eight XCDs, each with its own L2.  With head_chunk > 0 (heads_total a
  // multiple of 8), the workgroups with blockIdx % 8 == x serve heads
  // [x*hpx, (x+1)*hpx) only, taken in chunks of head_chunk heads; inside a
  // chunk, longest row groups first with the chunk's heads interleaved.  A
  // chunk of all hpx heads is plain longest-first order; smaller chunks keep
  // fewer heads' K/V in flight per L2.  head_chunk == 0: longest first over
  // all heads.
  const int n_groups = (p.nblk + RPW - 1) / RPW;
  int grp, bh;
  if (p.head_chunk > 0) {
    const int x = blockIdx.x & 7;
    const int j = blockIdx.x >> 3;
    const int hpx = p.heads_total >> 3;
    const int per_chunk = p.head_chunk * n_groups;
    const int c = j / per_chunk;
    const int r = j - c * per_chunk;
    const int hc = min(p.head_chunk, hpx - c * p.head_chunk);
    grp = n_groups - 1 - r / hc;
    bh = x * hpx + c * p.head_chunk + r % hc;
  } else {
    grp = n_groups - 1 - (int)blockIdx.x / p.heads_total;
    bh = (int)blockIdx.x % p.heads_total;
  }
  const int q_lo = grp * RPW;
  const int q_hi = min(q_lo + RPW - 1, p.nblk - 1);
  const int qb = q_lo + slot;           // this wave's query block
  const bool row_ok = qb < p.nblk;
  const int row = bh * p.nblk + qb;

  // One-pass block mass: this wave's row of (query, key block) partials,
  // [key block][query of the row] with stride pstride, and the queries'
  // 1/l.  In LDS for kDenseMass (rows padded by one against bank
  // conflicts); in the caller's workspace for kDenseMassWs, 1/l in LDS.
  float* part = reinterpret_cast<float*>(extra) + (size_t)slot * ((size_t)lnb * (BLK + 1) + BLK);
  float* invl = part + (size_t)lnb * (BLK + 1);                           // kDenseMass
  int pstride = BLK + 1;
  if constexpr (MODE == kDenseMassWs) {
    part = p.work + (size_t)row * lnb * BLK;
    invl = reinterpret_cast<float*>(extra) + (size_t)slot * BLK;
    pstride = BLK;
  }
  float* slots = reinterpret_cast<float*>(extra);   // kMassTwoPass: [RPW*LPR][lnb][BLK/32]

  const size_t head_off = (size_t)bh * p.seq * D;
  // grouped-query attention: query head h of batch entry b reads K/V head h / kv_group
  const int kv_bh = (bh / p.heads) * (p.heads / p.kv_group) + (bh % p.heads) / p.kv_group;
  const size_t kv_off = (size_t)kv_bh * p.seq * D;
  const uint16_t* Qh = p.q + head_off;
  const uint16_t* Kh = p.k + kv_off;
  const uint16_t* Vh = p.v + kv_off;
  const int qrow = qb * BLK + wr * 32 + n;
  // When seq_len is not a multiple of the block size the last query block
  // is short: its queries past the end are computed on zero Q, and neither
  // stored nor counted in the block mass.
  const bool q_ok = row_ok && qrow < p.seq;

  bf16x8_t qf[Sh::kChunks];
#pragma unroll
  for (int c = 0; c < Sh::kChunks; ++c)
    qf[c] = q_ok ? *reinterpret_cast<const bf16x8_t*>(Qh + (size_t)qrow * D + c * 16 + 8 * g)
                 : bf16x8_t{};

  const int head_bytes = p.seq * D * 2;
  // Direct-to-LDS staging (dense and sparse): per-lane read offsets into a
  // stage (u16 elements) and per-lane global byte offsets of each wave
  // load, both through the row-chunk permutations of DmaTile.
  int koff[Sh::kChunks];
  int voffs[Sh::kDTiles];
  uint32_t dk[Dm::kInstr];
  uint32_t dv[Dm::kInstr];
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  if constexpr (kDma) {
#pragma unroll
    for (int c = 0; c < Sh::kChunks; ++c) koff[c] = n * D + (((2 * c + g) ^ Dm::kx(n)) * 8);
    const int vrow = 4 * g + ((lane & 15) >> 2);
    const int lc0 = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
#pragma unroll
    for (int t = 0; t < Sh::kDTiles; ++t)
      voffs[t] = vrow * D + (((lc0 + 4 * t) ^ Dm::vx(vrow)) * 8) + 4 * (lane & 1);
#pragma unroll
    for (int i = 0; i < Dm::kInstr; ++i) {
      const int ci = (i * Dm::kWaves + wave) * 64 + lane;
      const int r = ci / Dm::kCpr, pc = ci % Dm::kCpr;
      dk[i] = (uint32_t)(r * D * 2 + ((pc ^ Dm::kx(r)) * 16));
      dv[i] = (uint32_t)(r * D * 2 + ((pc ^ Dm::vx(r)) * 16));
    }
  }

  // Issue this wave's share of one K/V tile into LDS stage `stage`.
  const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) unsigned char*)smem;
  const i32x4_t kdesc = buffer_desc(Kh, (uint32_t)head_bytes);
  const i32x4_t vdesc = buffer_desc(Vh, (uint32_t)head_bytes);
  // A tile that reaches past the end of the sequence (only in the last key
  // block, when seq_len is not a multiple of the block size) is read
  // through a resource that starts at its first in-range row (row seq-1 for
  // a tile wholly past the end), with every lane's offset clamped to the
  // last in-range 16 bytes: no lane reads outside the tensor, and the rows
  // past the end receive copies of in-range data.  Their keys come after
  // every real query of the only row that lists the block, its diagonal
  // one, so the causal mask removes them.
  auto dma_part = [&](int stage, int key0, bool with_v) __attribute__((always_inline)) {
    const int r0 = min(key0, p.seq - 1);
    const uint32_t bytes = (uint32_t)(p.seq - r0) * D * 2;
    const uint32_t lim = bytes - 16;
    const i32x4_t kd = buffer_desc(Kh + (size_t)r0 * D, bytes);
    const i32x4_t vd = buffer_desc(Vh + (size_t)r0 * D, bytes);
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds0 + stage * Dm::kStageBytes + wave_u * 1024);
#pragma unroll
    for (int i = 0; i < Dm::kInstr; ++i) {
      dma16(kd, kbase + i * Dm::kWaves * 1024, min(dk[i], lim), 0);
      if (with_v) dma16(vd, kbase + i * Dm::kWaves * 1024 + Dm::kTileBytes, min(dv[i], lim), 0);
    }
  };
  auto dma_tile = [&](int stage, int key0) __attribute__((always_inline)) {
    if (key0 + KT > p.seq) {
      dma_part(stage, key0, true);
      return;
    }
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)key0 * D * 2);
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds0 + stage * Dm::kStageBytes + wave_u * 1024);
#pragma unroll
    for (int i = 0; i < Dm::kInstr; ++i) {
      dma16(kdesc, kbase + i * Dm::kWaves * 1024, dk[i], soff);
      dma16(vdesc, kbase + i * Dm::kWaves * 1024 + Dm::kTileBytes, dv[i], soff);
    }
  };
  // K half only (first pass of the two-pass mass mode).
  auto dma_k = [&](int stage, int key0) __attribute__((always_inline)) {
    if (key0 + KT > p.seq) {
      dma_part(stage, key0, false);
      return;
    }
    const uint32_t soff = __builtin_amdgcn_readfirstlane((uint32_t)key0 * D * 2);
    const uint32_t kbase = __builtin_amdgcn_readfirstlane(lds0 + stage * Dm::kStageBytes + wave_u * 1024);
#pragma unroll
    for (int i = 0; i < Dm::kInstr; ++i) dma16(kdesc, kbase + i * Dm::kWaves * 1024, dk[i], soff);
  };

  // The first tile of every dense row and of every row the selection
  // writes is key block 0 (the sink), so its load is issued now, before the
  // list is known; the sparse prologue below re-issues it if the list
  // starts elsewhere.
  if constexpr (MODE == kMassTwoPass) {
    dma_k(0, 0);
    for (int i = tid; i < RPW * LPR * lnb * WR; i += Sh::kThreads) slots[i] = 0.f;
  } else if constexpr (kDma) {
    dma_tile(0, 0);
  }

  // Key blocks walked by the workgroup: the union of its rows' lists, in
  // ascending order, each entry tagged with the rows that list it.  Dense:
  // 0..q_hi, row `slot` lists kb <= its query block.  Sparse: each row's CSR
  // entries within [0, q] are ORed into an LDS bitmap (repeats count once,
  // order does not matter), then wave 0 compacts the union with ballots.
  int n_ent = q_hi + 1;
  if constexpr (MODE == kSparse) {
    for (int i = tid; i < RPW * LPR * nwords; i += Sh::kThreads) bits[i] = 0u;
    lds_barrier();
    if (wr == 0 && row_ok) {
#pragma unroll
      for (int lr = 0; lr < LPR; ++lr) {
        const int lrow = row * LPR + lr, lq = qb * LPR + lr;   // logical row and query block
        int e_begin = p.row_ptr[lrow];
        int e_end = p.row_ptr[lrow + 1];
        if (e_begin < 0) e_begin = 0;         // malformed pointers: read nothing before col_idx
        if (e_end < e_begin) e_end = e_begin; // and a decreasing pair as an empty row
        uint32_t* rb = bits + (slot * LPR + lr) * nwords;
        for (int idx = e_begin + lane; idx < e_end; idx += 64) {
          const int c = p.col_idx[idx];
          if (c >= 0 && c <= lq) atomicOr(&rb[c >> 5], 1u << (c & 31));
        }
      }
    }
    lds_barrier();
    if (wave == 0) {
      // tag bit 24 + (row slot * LPR + logical row) * LPR + logical key half
      int count = 0;
      for (int base = 0; base <= q_hi; base += 64) {
        const int c = base + lane;
        uint32_t tag = 0;
        if (c <= q_hi) {
#pragma unroll
          for (int r = 0; r < RPW * LPR; ++r)
#pragma unroll
            for (int kh = 0; kh < LPR; ++kh) {
              const int lc = c * LPR + kh;
              tag |= ((bits[r * nwords + (lc >> 5)] >> (lc & 31)) & 1u) << (24 + r * LPR + kh);
            }
        }
        const uint64_t bal = __ballot(tag != 0);
        if (tag != 0) ulist[1 + count + __popcll(bal & ((1ull << lane) - 1ull))] = (int)(tag | (uint32_t)c);
        count += __popcll(bal);
      }
      if (lane == 0) ulist[0] = count;
    }
    lds_barrier();
    n_ent = __builtin_amdgcn_readfirstlane(ulist[0]);
  }
  // Entry e -> (key block, does this wave's row list it, and for LPR = 2
  // which (logical query block, logical key block) pairs it lists: bit
  // 2*lr + kh).
  auto entry3 = [&](int e, int& kb, bool& mine, uint32_t& pairs) {
    if constexpr (MODE == kSparse) {
      const uint32_t code = (uint32_t)__builtin_amdgcn_readfirstlane(ulist[1 + e]);
      kb = (int)(code & 0x00FFFFFFu);
      pairs = (code >> (24 + slot * LPR * LPR)) & ((1u << (LPR * LPR)) - 1u);
      mine = row_ok && pairs != 0;
    } else {
      kb = e;
      mine = row_ok && e <= qb;
      pairs = (1u << (LPR * LPR)) - 1u;
    }
  };
  auto entry = [&](int e, int& kb, bool& mine) {
    uint32_t pairs;
    entry3(e, kb, mine, pairs);
  };
  const int n_tiles = n_ent * Sh::kSub;

  f32x16_t oacc[Sh::kDTiles];
#pragma unroll
  for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
    for (int i = 0; i < 16; ++i) oacc[t][i] = 0.f;
  float m_ref = -INFINITY;  // identical in both lanes of a query
  float l_part = 0.f;       // this lane's share of the row sum
  float m_hi = -INFINITY;   // mass modes: this lane's largest raw score so far
  float l_two = 0.f;        // two-pass: row sum relative to the exact max
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
  const __amdgpu_buffer_rsrc_t krs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kh), 0, head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t vrs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vh), 0, head_bytes, 0x00020000);

  auto tile_key0 = [&](int it) {
    int kb;
    bool mine;
    entry(it / Sh::kSub, kb, mine);
    return kb * BLK + (it % Sh::kSub) * KT;
  };
  if constexpr (MODE == kSparse) {
    // The speculative first load was wrong (or is not needed): let it land,
    // then load the list's first tile.  Nothing may still be writing this
    // workgroup's LDS when it exits.
    if (n_tiles == 0 || tile_key0(0) != 0) {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      if (n_tiles > 0) dma_tile(0, tile_key0(0));
    }
  }

  // S^T = K Q^T for one key tile (Kt: the LDS slot holding its K rows).
  // With LOAD (direct-to-LDS staging), this wave's loads of the next tile
  // (keys from nkey0, into stage nstage) are spread over the QK^T MFMAs, one
  // load per few MFMAs, instead of leaving every wave of the workgroup to
  // issue all of them at once after the barrier.  LOAD: 0 no loads, 1 the
  // next tile's K and V, 2 its K only.
  auto scores_l = [&]<int LOAD>(f32x16_t (&sc)[Sh::kM], const uint16_t* Kt, int nstage, int nkey0)
                      __attribute__((always_inline)) {
    constexpr int nQK = Sh::kM * Sh::kChunks;
    constexpr int nLoad = (LOAD == 2 ? 1 : 2) * Dm::kInstr;
    uint32_t soff = 0, kbase = 0;
    if (kDma && LOAD) {
      soff = __builtin_amdgcn_readfirstlane((uint32_t)nkey0 * D * 2);
      kbase = __builtin_amdgcn_readfirstlane(lds0 + nstage * Dm::kStageBytes + wave_u * 1024);
    }
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sc[m][i] = 0.f;
#pragma unroll
      for (int c = 0; c < Sh::kChunks; ++c) {
        const uint16_t* kp = kDma ? Kt + koff[c] + m * 32 * D
                                  : Ks + (m * 32 + n) * Sh::kKsStride + c * 16 + 8 * g;
        const bf16x8_t a = *reinterpret_cast<const bf16x8_t*>(kp);
        sc[m] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[c], sc[m], 0, 0, 0);
        if constexpr (kDma && LOAD) {
          const int i = m * Sh::kChunks + c;
#pragma unroll
          for (int j = i * nLoad / nQK; j < (i + 1) * nLoad / nQK; ++j) {
            if (j < Dm::kInstr) dma16_free(kdesc, kbase + j * Dm::kWaves * 1024, dk[j], soff);
            else dma16_free(vdesc, kbase + (j - Dm::kInstr) * Dm::kWaves * 1024 + Dm::kTileBytes,
                            dv[j - Dm::kInstr], soff);
          }
        }
      }
    }
  };

  // Causal mask (diagonal block only), lazy-rescale check and rare rescale.
  auto prep = [&]<bool MASKED>(int kb, int sub, f32x16_t (&sc)[Sh::kM]) __attribute__((always_inline)) {
    constexpr bool kTrack = (kMass1 || MODE == kMassTwoPass);
    return softmax_prep<D, BLK, KT, MODE, MASKED>(part, p.scale_log2, qrow - (kb * BLK + sub * KT), g, n, wr,
                                                  kb * LPR, m_ref, l_part, blk_part,
                                                  kTrack ? m_hi : -INFINITY, pstride, sc, oacc);
  };

  // P = exp2(s * scale*log2e - m) per 32-key sub-tile, then that
  // sub-tile's O^T += V^T P^T (Vt: the LDS slot holding the tile's V rows);
  // the exponentials of sub-tile m+1 are independent of the MFMAs of
  // sub-tile m.  Masked scores are -inf -> 0.
  auto expv = [&](int kb, int sub, f32x16_t (&sc)[Sh::kM], const uint16_t* Vt) __attribute__((always_inline)) {
    const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
    float tsum = 0.f;
    float hsum[2] = {0.f, 0.f};   // LPR = 2 mass: per logical key half
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m) {
      bf16x8_t pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[m][kk * 8 + e], p.scale_log2, neg_m));
          if constexpr (kMass1) tsum += pv;   // block mass needs the fp32 values
          if constexpr (MODE == kDenseMass && LPR == 2) hsum[kk] += pv;
          pf[kk][e] = (__bf16)pv;
        }
      if constexpr (!kMass1) {
        // Row sum of the bf16 operands themselves (the same values the PV
        // product uses), two per packed dot product.  O is divided by this
        // sum: the weights then add up to one however P was rounded, so the
        // rounding error of a dominant weight is damped by one minus that
        // weight.  (The mass mode needs the fp32 sum for the block mass; its
        // divisor is fixed up in the epilogue instead.)
        const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const bf16x2_t pair = {pf[kk][2 * w], pf[kk][2 * w + 1]};
            tsum = __builtin_amdgcn_fdot2_f32_bf16(pair, one, tsum, false);
          }
      }
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          constexpr int kVRow = kDma ? D : Sh::kVStride;
          const uint16_t* vp = kDma ? Vt + voffs[t] + (32 * m + 16 * kk) * D
                                    : Vs + v_lane_off + (32 * m + 16 * kk) * Sh::kVStride + 32 * t;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp + 8 * kVRow));
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[t], 0, 0, 0);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    l_part += tsum;
    if constexpr (MODE == kDenseMass && LPR == 2) {
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const float bp = hsum[kh] + __shfl_xor(hsum[kh], 32);
        if (g == 0) part[(kb * 2 + kh) * (BLK + 1) + n] = bp;
      }
    } else if constexpr (kMass1) {
      blk_part += tsum;
      if (sub == Sh::kSub - 1) {
        const float bp = blk_part + __shfl_xor(blk_part, 32);
        if (g == 0) part[(size_t)kb * pstride + wr * 32 + n] = bp;
        blk_part = 0.f;
      }
    }
  };

  // One whole tile for this wave's row.
  // The MFMA stretches run at raised wave priority: when both waves of a
  // SIMD are ready, the one feeding the matrix core issues first and the
  // other's softmax work fills the MFMA shadow.
  auto compute_tile = [&]<bool MASKED, bool LOAD = false>(int kb, int sub, const uint16_t* Kt, const uint16_t* Vt,
                                                           uint32_t pairs, int nstage = 0, int nkey0 = 0)
                          __attribute__((always_inline)) {
    f32x16_t sc[Sh::kM];
    __builtin_amdgcn_s_setprio(1);
    scores_l.template operator()<LOAD ? 1 : 0>(sc, Kt, nstage, nkey0);
    __builtin_amdgcn_s_setprio(0);
    if constexpr (LPR == 2 && MODE == kSparse) {
      // logical pairs this tile does not list: query half n/16, key half i/8
      if (pairs != 0xFu) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (!((pairs >> (2 * (n >> 4) + (i >> 3))) & 1u)) sc[0][i] = -INFINITY;
      }
    }
    const float run_max = prep.template operator()<MASKED>(kb, sub, sc);
    if constexpr (kMass1) m_hi = run_max;
    expv(kb, sub, sc, Vt);
  };

  // Two-pass mass mode, first pass: running max, fp32 row sum and the
  // exact largest score.
  auto sum_tile = [&]<bool MASKED, bool LOAD = false>(int kb, int sub, const uint16_t* Kt, int nstage = 0,
                                                       int nkey0 = 0) __attribute__((always_inline)) {
    f32x16_t sc[Sh::kM];
    scores_l.template operator()<LOAD ? 2 : 0>(sc, Kt, nstage, nkey0);
    m_hi = prep.template operator()<MASKED>(kb, sub, sc);
    const float neg_m = (m_ref == -INFINITY) ? 0.f : -m_ref;
    float tsum = 0.f;
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) tsum += __builtin_amdgcn_exp2f(fmaf(sc[m][i], p.scale_log2, neg_m));
    l_part += tsum;
  };

  // Two-pass mass mode, second pass: p = exp2(s*scale*log2e - m) with m the
  // row's exact largest scaled score, so the largest p is exactly 1 in bf16.
  // The block mass is the fp32 sum of p times 1/l (l: the first pass's fp32
  // row sum, brought to m), added to this wave's slot of the key block.
  // O^T += V^T P^T takes p rounded to bf16; O is divided by l at the end.
  // (Feeding p/l instead saves that division but rounds the dominant
  // weight itself, whose error then reaches O undamped.)
  auto mass_tile = [&]<bool MASKED, bool LOAD = false>(int kb, int sub, const uint16_t* Kt, const uint16_t* Vt,
                                                        float neg_m, float inv_l, int nstage = 0, int nkey0 = 0)
                       __attribute__((always_inline)) {
    f32x16_t sc[Sh::kM];
    scores_l.template operator()<LOAD ? 1 : 0>(sc, Kt, nstage, nkey0);
    if constexpr (MASKED) {
      const int rel = qrow - (kb * BLK + sub * KT);
#pragma unroll
      for (int m = 0; m < Sh::kM; ++m)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int koff = m * 32 + 8 * (i >> 2) + 4 * g + (i & 3);
          sc[m][i] = (koff > rel) ? -INFINITY : sc[m][i];
        }
    }
    float tsum = 0.f;
    float hs[2] = {0.f, 0.f};     // LPR = 2: per logical key half
#pragma unroll
    for (int m = 0; m < Sh::kM; ++m) {
      bf16x8_t pf[2];
#pragma unroll
      for (int kk = 0; kk < 2; ++kk)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = __builtin_amdgcn_exp2f(fmaf(sc[m][kk * 8 + e], p.scale_log2, neg_m));
          tsum += pv;
          if constexpr (LPR == 2) hs[kk] += pv;
          pf[kk][e] = (__bf16)pv;
        }
#pragma unroll
      for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint16_t* vp = Vt + voffs[t] + (32 * m + 16 * kk) * D;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (__attribute__((address_space(3))) i16x4_t*)(vp + 8 * D));
          const bf16x8_t a =
              __builtin_bit_cast(bf16x8_t, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf[kk], oacc[t], 0, 0, 0);
        }
    }
    if constexpr (LPR == 1) {
      // sum over the wave's 32 queries x 2 lane halves, fixed butterfly order
      tsum *= inv_l;
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) tsum += __shfl_xor(tsum, off);
      if (lane == 0) slots[(slot * lnb + kb) * WR + wr] += tsum;
    } else {
      // per (logical query block = query half, logical key block = key half)
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        float v = hs[kh] * inv_l;
        v += __shfl_xor(v, 32);
#pragma unroll
        for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off);
        if ((lane & 47) == 0)   // lanes 0 and 16
          slots[((slot * LPR + (lane >> 4)) * lnb + kb * 2 + kh) * WR + wr] += v;
      }
    }
  };

  // Publish the prefetched tile, prefetch the next one, then every wave whose
  // row lists the block computes on it (the causal mask only in the row's
  // own diagonal block; the branches are wave-uniform).
  if constexpr (MODE == kMassTwoPass) {
    // First pass: K tiles only; running max and row sum of every query.
    for (int it = 0; it < n_tiles; ++it) {
      int kb;
      bool mine;
      entry(it / Sh::kSub, kb, mine);
      const int sub = it % Sh::kSub;
      const int st = it & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      lds_barrier();
      const uint16_t* Kt = reinterpret_cast<const uint16_t*>(smem + st * Dm::kStageBytes);
      const int nkey0 = it + 1 < n_tiles ? tile_key0(it + 1) : -1;
      if (mine && nkey0 >= 0 && nkey0 + KT <= p.seq) {
        if (kb == qb) sum_tile.template operator()<true, true>(kb, sub, Kt, st ^ 1, nkey0);
        else sum_tile.template operator()<false, true>(kb, sub, Kt, st ^ 1, nkey0);
      } else {
        if (nkey0 >= 0) dma_k(st ^ 1, nkey0);
        if (mine) {
          if (kb == qb) sum_tile.template operator()<true>(kb, sub, Kt);
          else sum_tile.template operator()<false>(kb, sub, Kt);
        }
      }
    }
    // Bring the row sum from the lazy reference to the exact max.
    const float mh = fmaxf(m_hi, __shfl_xor(m_hi, 32));
    const float m_ex = mh * p.scale_log2;
    l_two = (mh == -INFINITY) ? 0.f
                              : (l_part + __shfl_xor(l_part, 32)) * __builtin_amdgcn_exp2f(m_ref - m_ex);
    const float inv_l = (l_two > 0.f && q_ok) ? 1.f / l_two : 0.f;   // padded queries add no mass
    const float neg_m = (mh == -INFINITY) ? 0.f : -m_ex;
    // Second pass over the same tiles with K and V.
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    lds_barrier();
    dma_tile(0, tile_key0(0));
    for (int it = 0; it < n_tiles; ++it) {
      int kb;
      bool mine;
      entry(it / Sh::kSub, kb, mine);
      const int sub = it % Sh::kSub;
      const int st = it & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      lds_barrier();
      const uint16_t* Kt = reinterpret_cast<const uint16_t*>(smem + st * Dm::kStageBytes);
      const uint16_t* Vt = Kt + KT * D;
      const int nkey0 = it + 1 < n_tiles ? tile_key0(it + 1) : -1;
      if (mine && nkey0 >= 0 && nkey0 + KT <= p.seq) {
        if (kb == qb) mass_tile.template operator()<true, true>(kb, sub, Kt, Vt, neg_m, inv_l, st ^ 1, nkey0);
        else mass_tile.template operator()<false, true>(kb, sub, Kt, Vt, neg_m, inv_l, st ^ 1, nkey0);
      } else {
        if (nkey0 >= 0) dma_tile(st ^ 1, nkey0);
        if (mine) {
          if (kb == qb) mass_tile.template operator()<true>(kb, sub, Kt, Vt, neg_m, inv_l);
          else mass_tile.template operator()<false>(kb, sub, Kt, Vt, neg_m, inv_l);
        }
      }
    }
  } else if constexpr (kDma) {
    // Wait for this wave's loads of tile `it`, then one barrier: every
    // wave's share has landed and every wave is done with the other stage,
    // which then receives tile it+1 while tile it is used (tile 0 is
    // already on its way).
    for (int it = 0; it < n_tiles; ++it) {
      int kb;
      bool mine;
      uint32_t pairs;
      entry3(it / Sh::kSub, kb, mine, pairs);
      const int sub = it % Sh::kSub;
      const int st = it & 1;
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
      lds_barrier();
      const uint16_t* Kt = reinterpret_cast<const uint16_t*>(smem + st * Dm::kStageBytes);
      const uint16_t* Vt = Kt + KT * D;
      // The next tile's loads ride along with this tile's QK^T MFMAs when
      // this wave computes; a wave with nothing to compute issues them at
      // once, and so does every wave for a tile past the sequence end.
      const int nkey0 = it + 1 < n_tiles ? tile_key0(it + 1) : -1;
      if (mine && nkey0 >= 0 && nkey0 + KT <= p.seq) {
        if (kb == qb) compute_tile.template operator()<true, true>(kb, sub, Kt, Vt, pairs, st ^ 1, nkey0);
        else compute_tile.template operator()<false, true>(kb, sub, Kt, Vt, pairs, st ^ 1, nkey0);
      } else {
        if (nkey0 >= 0) dma_tile(st ^ 1, nkey0);
        if (mine) {
          if (kb == qb) compute_tile.template operator()<true>(kb, sub, Kt, Vt, pairs);
          else compute_tile.template operator()<false>(kb, sub, Kt, Vt, pairs);
        }
      }
    }
  } else {
  // K/V of one tile into registers (clamped past the sequence end, as for
  // the direct-to-LDS loads).
  auto load_kv = [&](int key0) __attribute__((always_inline)) {
    if (key0 + KT <= p.seq) {
      load_rows<D, BLK, KT, RPW>(krs, key0, tid, kreg);
      load_rows<D, BLK, KT, RPW>(vrs, key0, tid, vreg);
    } else {
      const int r0 = min(key0, p.seq - 1);
      const int bytes = (p.seq - r0) * D * 2;
      load_rows_clamped<D, BLK, KT, RPW>(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Kh + (size_t)r0 * D), 0, bytes, 0x00020000),
          bytes - 16, tid, kreg);
      load_rows_clamped<D, BLK, KT, RPW>(
          __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(Vh + (size_t)r0 * D), 0, bytes, 0x00020000),
          bytes - 16, tid, vreg);
    }
  };
  if (n_tiles > 0) load_kv(tile_key0(0));
  for (int it = 0; it < n_tiles; ++it) {
    int kb;
    bool mine;
    entry(it / Sh::kSub, kb, mine);
    const int sub = it % Sh::kSub;
    __syncthreads();  // previous tile fully consumed
    store_rows<D, BLK, KT, RPW, Sh::kKsStride>(Ks, tid, kreg);
    store_rows<D, BLK, KT, RPW, Sh::kVStride>(Vs, tid, vreg);
    __syncthreads();
    if (it + 1 < n_tiles) load_kv(tile_key0(it + 1));
    if (mine) {
      if (kb == qb) compute_tile.template operator()<true>(kb, sub, Ks, Vs, 0xFu);
      else compute_tile.template operator()<false>(kb, sub, Ks, Vs, 0xFu);
    }
  }
  }

  // ---- epilogue -----------------------------------------------------------
  const float lt = (MODE == kMassTwoPass) ? l_two : l_part + __shfl_xor(l_part, 32);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  // O's divisor.  The one-pass mass mode sums fp32 p for the block mass; O
  // is divided by that sum with the row's largest term counted at its bf16
  // value, the one the PV product used, so that the dominant weight's
  // rounding error is damped as in the other modes.  That term was taken
  // against the final reference max: a later tile can raise the reference
  // only with a score above this one.  (Lanes of a query that hold an equal
  // largest score each count theirs.)
  float lo = lt;
  if constexpr (kMass1) {
    const float mh = fmaxf(m_hi, __shfl_xor(m_hi, 32));
    float d = 0.f;
    if (mh != -INFINITY && m_hi == mh) {
      const float pm = __builtin_amdgcn_exp2f(fmaf(m_hi, p.scale_log2, -m_ref));
      d = (float)(__bf16)pm - pm;
    }
    lo = lt + (d + __shfl_xor(d, 32));
  }
  const float inv_o = lo > 0.f ? 1.f / lo : 0.f;
  if (q_ok) {
    uint16_t* Oh = p.o + head_off + (size_t)qrow * D;
#pragma unroll
    for (int t = 0; t < Sh::kDTiles; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        __bf16 b0 = (__bf16)(oacc[t][4 * j + 0] * inv_o);
        __bf16 b1 = (__bf16)(oacc[t][4 * j + 1] * inv_o);
        __bf16 b2 = (__bf16)(oacc[t][4 * j + 2] * inv_o);
        __bf16 b3 = (__bf16)(oacc[t][4 * j + 3] * inv_o);
        u32x2_t w;
        w.x = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        w.y = (uint32_t)__builtin_bit_cast(uint16_t, b2) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
        *reinterpret_cast<u32x2_t*>(Oh + t * 32 + 8 * j + 4 * g) = w;
      }
    if (MODE == kDense && p.lse != nullptr && g == 0) {
      const float lse = (lt > 0.f) ? (m_ref + __log2f(lt)) * 0.69314718055994531f : -INFINITY;
      p.lse[(size_t)bh * p.seq + qrow] = lse;
    }
  }

  // |I_q| of Eq. (5): the block's query count, short for the last block
  // when seq_len is not a multiple of the block size.
  auto mass_div = [&](float acc, int lq) __attribute__((always_inline)) {
    const int cnt = min(kLB, p.seq - lq * kLB);
    return cnt == kLB ? acc * (1.0f / kLB) : acc / (float)cnt;
  };
  if constexpr (MODE == kMassTwoPass) {
    lds_barrier();
    // r_qb = (1/|I_q|) * (sum of the logical row's wave slots, in wave order).
    for (int w = tid; w < RPW * LPR * lnb; w += Sh::kThreads) {
      const int rl = w / lnb, b = w % lnb;
      const int qphys = q_lo + rl / LPR;
      if (qphys >= p.nblk) continue;
      const int lq = qphys * LPR + rl % LPR;
      if (b > lq) continue;
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < WR; ++i) acc += slots[(rl * lnb + b) * WR + i];
      p.mass[((size_t)bh * lnb + lq) * lnb + b] += mass_div(acc, lq);
    }
  }
  if constexpr (MODE == kDenseMass) {
    if (row_ok && g == 0) invl[wr * 32 + n] = q_ok ? inv : 0.f;   // padded queries add no mass
    __syncthreads();
    // Row slot r's masses: r_qb = (1/|I_q|) sum_i partial_ib / l_i, one
    // sequential sum per key block (deterministic).
    for (int w = tid; w < RPW * LPR * lnb; w += Sh::kThreads) {
      const int rl = w / lnb, b = w % lnb;
      const int r = rl / LPR, lr = rl % LPR;
      const int qr = q_lo + r;
      if (qr >= p.nblk) continue;
      const int lq = qr * LPR + lr;
      if (b > lq) continue;
      const float* pr = reinterpret_cast<float*>(extra) + (size_t)r * ((size_t)lnb * (BLK + 1) + BLK);
      const float* il = pr + (size_t)lnb * (BLK + 1);
      pr += b * (BLK + 1);
      float acc = 0.f;
      for (int i = lr * kLB; i < (lr + 1) * kLB; ++i) acc = fmaf(pr[i], il[i], acc);
      p.mass[((size_t)bh * lnb + lq) * lnb + b] += mass_div(acc, lq);
    }
  }
  if constexpr (MODE == kDenseMassWs) {
    if (row_ok && g == 0) invl[wr * 32 + n] = q_ok ? inv : 0.f;
    // The barrier (with its workgroup-scope fences) also makes every wave's
    // partial stores to the workspace visible to the whole workgroup.
    __syncthreads();
    // Row slot r's masses: r_qb = (1/|I_q|) sum_i partial_ib / l_i, one
    // sequential sum per key block (deterministic), the B partials of a
    // block contiguous in the workspace.
    for (int w = tid; w < RPW * lnb; w += Sh::kThreads) {
      const int r = w / lnb, b = w % lnb;
      const int qr = q_lo + r;
      if (qr >= p.nblk || b > qr) continue;
      const float* pr = p.work + ((size_t)(bh * p.nblk + qr) * lnb + b) * BLK;
      const float* il = reinterpret_cast<const float*>(extra) + (size_t)r * BLK;
      float acc = 0.f;
      for (int i = 0; i < BLK; ++i) acc = fmaf(pr[i], il[i], acc);
      p.mass[((size_t)bh * lnb + qr) * lnb + b] += mass_div(acc, qr);
    }
  }
}

// Heads per chunk for the workgroup order (see the kernel prologue).  When
// one XCD's workgroups are at most four times its resident slots, plain
// longest-first order over its heads keeps the tail short; above that,
// chunks of about two slot-fills keep few heads' K/V per L2.  Needs
// heads_total % 8 == 0 (each head then stays on one XCD).
constexpr int kMaxDevices = 64;

// Compute units of device `dev`, cached per device (0 if unknown).
inline int device_cus(int dev) {
  static std::atomic<int> cache[kMaxDevices];   // zero: not read yet
  if (dev < 0 || dev >= kMaxDevices) return 0;
  int c = cache[dev].load(std::memory_order_relaxed);
  if (c == 0) {
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c < 1) return 0;
    cache[dev].store(c, std::memory_order_relaxed);
  }
  return c;
}

inline int choose_head_chunk(int dev, int heads_total, int n_groups, int wgs_per_cu) {
  if (heads_total % 8 != 0) return 0;
  const int cus = device_cus(dev);
  if (cus < 8) return 0;
  const int hpx = heads_total / 8;
  const long slots = (long)wgs_per_cu * (cus / 8);
  if ((long)hpx * n_groups <= 4 * slots) return hpx;
  const long hc = (2 * slots + n_groups - 1) / n_groups;
  return (int)std::max(1L, std::min<long>(hc, hpx));
}

template <int D, int BLK, int KT, int MODE, int RPW, int LPR = 1>
hipError_t launch_attn_t(const AttnParams& p_in, hipStream_t stream) {
  using Sh = AttnShape<D, BLK, KT, RPW>;
  const size_t lds = attn_lds_need<D, BLK, KT, RPW, LPR>(MODE, p_in.nblk);
  auto kern = wise_attn_kernel<D, BLK, KT, MODE, RPW, LPR>;
  // Once per device: allow the full LDS budget and read how many
  // workgroups fit one CU by registers alone.  Concurrent first calls may
  // both do it; the attribute is idempotent and the value the same.
  static std::atomic<int> ready[kMaxDevices];   // 0: not yet; else 1 + workgroups per CU
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int rw = ready[dev].load(std::memory_order_acquire);
  if (rw == 0) {
    if (hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)kMaxLds) != hipSuccess)
      return hipErrorInvalidDeviceFunction;
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kern, Sh::kThreads, 0) != hipSuccess)
      return hipErrorInvalidDeviceFunction;
    rw = 1 + n;
    ready[dev].store(rw, std::memory_order_release);
  }
  const int regs_wgs = rw - 1;
  AttnParams p = p_in;
  const int n_groups = (p.nblk + RPW - 1) / RPW;
  p.head_chunk = choose_head_chunk(dev, p.heads_total, n_groups,
                                   std::max(1, std::min(regs_wgs, (int)(kMaxLds / std::max<size_t>(lds, 1)))));
  const unsigned grid = (unsigned)p.heads_total * (unsigned)n_groups;
  if (trace_enabled()) {
    static const char* const kModeName[] = {"dense", "dense+mass", "sparse", "mass two-pass", "dense+mass ws"};
    trace_launch("wise_attn_kernel", grid, Sh::kThreads, lds,
                 "mode=%s head_dim=%d block=%d keys_per_tile=%d rows_per_wg=%d logical_per_row=%d seq=%d "
                 "n_blocks=%d heads=%d kv_group=%d head_chunk=%d wgs_per_cu_by_registers=%d",
                 kModeName[MODE], D, BLK / LPR, KT, RPW, LPR, p.seq, p.nblk * LPR, p.heads_total, p.kv_group,
                 p.head_chunk, regs_wgs);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(Sh::kThreads), lds, stream, p);
  return hipGetLastError();
}

// Launch shape: keys per tile and rows per workgroup.
struct AttnCfg {
  int kt;
  int rpw;
};

template <int D, int BLK>
size_t cfg_lds(int kt, int rpw, int mode, int nblk) {
  if constexpr (BLK >= 64) {
    if (kt == 64 && rpw == 1) return attn_lds_need<D, BLK, 64, 1>(mode, nblk);
    if (kt == 64 && rpw == 2) return attn_lds_need<D, BLK, 64, 2>(mode, nblk);
  }
  if (kt == 32 && rpw == 1) return attn_lds_need<D, BLK, 32, 1>(mode, nblk);
  if (kt == 32 && rpw == 2) return attn_lds_need<D, BLK, 32, 2>(mode, nblk);
  if (kt == 32 && rpw == 4) return attn_lds_need<D, BLK, 32, 4>(mode, nblk);
  return 0;
}

#ifndef WISE_SPARSE_RPW64
#define WISE_SPARSE_RPW64 2
#endif

// Rows per workgroup of the block-32 dense, sparse and two-pass launches:
// one-wave rows, so several share every staged tile (four for the dense
// walks, two for the sparse union walk; two at head_dim 96, whose 32-key
// tile does not split into four waves' loads).
template <int D, int MODE>
constexpr int rpw32() { return (MODE == kSparse || D == 96) ? 2 : 4; }

// Dense and sparse launches: 64-key tiles (32 for block 32), two rows per
// workgroup for block 64, rpw32() rows for block 32.  Mass launches: the candidate with the most
// resident waves per CU under the LDS budget (two 2-wave rows, or one row;
// 64- or 32-key tiles), preferring two rows and larger tiles on ties.
template <int D, int BLK>
AttnCfg choose_cfg(int mode, int nblk) {
  constexpr int kWavesPerRow = BLK / 32;
  if (mode != kDenseMass) {
    const int r32 = mode == kSparse ? rpw32<D, kSparse>() : rpw32<D, kDense>();
    const AttnCfg c{BLK >= 64 ? 64 : 32, BLK == 64 ? (mode == kSparse ? WISE_SPARSE_RPW64 : 2)
                                                   : (BLK == 32 ? r32 : 1)};
    return cfg_lds<D, BLK>(c.kt, c.rpw, mode, nblk) <= kMaxLds ? c : AttnCfg{0, 0};
  }
  // (head_dim 128 at block 64 with 64-key tiles spills registers in this mode)
  AttnCfg cands[4];
  int nc = 0;
  if (BLK == 64 && D != 128) cands[nc++] = {64, 2};
  if (BLK == 64) cands[nc++] = {32, 2};
  if (BLK >= 64 && !(BLK == 64 && D == 128)) cands[nc++] = {64, 1};
  cands[nc++] = {32, 1};
  AttnCfg best{0, 0};
  int best_waves = 0;
  for (int i = 0; i < nc; ++i) {
    const size_t lds = cfg_lds<D, BLK>(cands[i].kt, cands[i].rpw, mode, nblk);
    if (lds == 0 || lds > kMaxLds) continue;
    const int waves = std::min((int)(kMaxLds / lds) * kWavesPerRow * cands[i].rpw, 8);
    if (waves > best_waves) { best = cands[i]; best_waves = waves; }
  }
  return best;
}

#ifndef WISE_TWO_PASS_BELOW_WAVES
#define WISE_TWO_PASS_BELOW_WAVES 4
#endif

// Resident waves per CU of the best single-pass mass configuration (0 if
// none fits the LDS budget).
template <int D, int BLK>
int fused_mass_waves(int nblk) {
  const AttnCfg c = choose_cfg<D, BLK>(kDenseMass, nblk);
  if (c.kt == 0) return 0;
  const size_t lds = cfg_lds<D, BLK>(c.kt, c.rpw, kDenseMass, nblk);
  return std::min((int)(kMaxLds / lds) * (BLK / 32) * c.rpw, 8);
}

// The mass launch runs in one pass (O and the block mass from the same P,
// with nB x (B+1) fp32 partials per row in LDS) unless those partials leave
// fewer than WISE_TWO_PASS_BELOW_WAVES resident waves per CU; then it runs
// in two passes over the keys (row max and sum, then P, O and the mass), which
// needs only one fp32 per (row, key block, wave) of LDS.
// The one-pass mass kernel with one 32-query wave per workgroup stages a
// whole 32-key tile per lane in VGPRs; at head_dim 128 that spills.
template <int D, int BLK>
constexpr bool fused_mass_spills() { return D == 128 && BLK == 32; }

// Block 32 mass launches always take the two-pass form: it runs rpw32()
// one-wave rows per workgroup sharing every staged tile, the one-pass form
// only one.
template <int D, int BLK>
constexpr bool two_pass_only() { return BLK == 32; }

template <int D, int BLK>
int effective_mode(int mode, int nblk) {
  if (mode != kDenseMass) return mode;
  if constexpr (two_pass_only<D, BLK>()) return kMassTwoPass;
  if (fused_mass_waves<D, BLK>(nblk) >= WISE_TWO_PASS_BELOW_WAVES) return kDenseMass;
  const AttnCfg c = choose_cfg<D, BLK>(kMassTwoPass, nblk);
  return c.kt != 0 ? kMassTwoPass : kDenseMass;
}

template <int D, int BLK, int MODE>
hipError_t launch_cfg(AttnCfg c, const AttnParams& p, hipStream_t stream) {
  if constexpr (MODE != kDenseMass) {
    if constexpr (BLK == 64) return launch_attn_t<D, 64, 64, MODE, MODE == kSparse ? WISE_SPARSE_RPW64 : 2>(p, stream);
    else if constexpr (BLK == 128) return launch_attn_t<D, 128, 64, MODE, 1>(p, stream);
    else return launch_attn_t<D, 32, 32, MODE, rpw32<D, MODE>()>(p, stream);
  } else {
    if constexpr (BLK == 64) {
      if constexpr (D != 128) {
        if (c.kt == 64 && c.rpw == 2) return launch_attn_t<D, 64, 64, MODE, 2>(p, stream);
        if (c.kt == 64 && c.rpw == 1) return launch_attn_t<D, 64, 64, MODE, 1>(p, stream);
      }
      if (c.kt == 32 && c.rpw == 2) return launch_attn_t<D, 64, 32, MODE, 2>(p, stream);
      if (c.kt == 32 && c.rpw == 1) return launch_attn_t<D, 64, 32, MODE, 1>(p, stream);
      return hipErrorInvalidValue;
    } else if constexpr (BLK == 128) {
      if (c.kt == 64) return launch_attn_t<D, 128, 64, MODE, 1>(p, stream);
      return launch_attn_t<D, 128, 32, MODE, 1>(p, stream);
    } else {
      return hipErrorInvalidValue;   // block 32 mass launches are two-pass (effective_mode)
    }
  }
}

template <int D, int BLK>
hipError_t launch_attn_blk(int mode_in, const AttnParams& p, hipStream_t stream) {
  const int mode = effective_mode<D, BLK>(mode_in, p.nblk);
  const AttnCfg c = choose_cfg<D, BLK>(mode, p.nblk);
  if (c.kt == 0) return hipErrorInvalidValue;
  switch (mode) {
    case kDense: return launch_cfg<D, BLK, kDense>(c, p, stream);
    case kSparse: return launch_cfg<D, BLK, kSparse>(c, p, stream);
    case kMassTwoPass: return launch_cfg<D, BLK, kMassTwoPass>(c, p, stream);
    case kDenseMassWs:
      if constexpr (BLK >= 32) return launch_cfg<D, BLK, kDenseMassWs>(c, p, stream);
      else return hipErrorInvalidValue;
    default: return launch_cfg<D, BLK, kDenseMass>(c, p, stream);
  }
}

// Block 16: 32 x 32 physical tiles, two logical blocks per physical block
// (nblk16 logical blocks, even).  The dense baseline does not depend on the
// block size and runs the block-32 launch; the mass mode runs one pass when
// its partials leave at least 4 resident waves per CU, else two passes.
template <int D>
int b16_mode(int mode, int nblk16) {
  if (mode != kDenseMass) return mode;
  if constexpr (fused_mass_spills<D, 32>()) return kMassTwoPass;
  const size_t lds = attn_lds_need<D, 32, 32, 1, 2>(kDenseMass, nblk16 / 2);
  const int waves = lds <= kMaxLds ? std::min((int)(kMaxLds / lds), 8) : 0;
  return waves >= WISE_TWO_PASS_BELOW_WAVES ? kDenseMass : kMassTwoPass;
}

template <int D>
size_t attn_lds_bytes_b16(int mode, int nblk16) {
  if (nblk16 % 2 != 0) return 0;
  if (mode == kDense) return attn_lds_need<D, 32, 32, rpw32<D, kDense>()>(kDense, nblk16 / 2);
  const int m = b16_mode<D>(mode, nblk16);
  return m == kDenseMass ? attn_lds_need<D, 32, 32, 1, 2>(m, nblk16 / 2)
                         : attn_lds_need<D, 32, 32, 2, 2>(m, nblk16 / 2);
}

template <int D>
hipError_t launch_attn_b16(int mode, const AttnParams& p16, hipStream_t stream) {
  if (p16.nblk % 2 != 0) return hipErrorInvalidValue;
  AttnParams p = p16;
  p.nblk = p16.nblk / 2;     // physical 32-key blocks
  switch (mode == kDense ? kDense : b16_mode<D>(mode, p16.nblk)) {
    case kDense: return launch_attn_t<D, 32, 32, kDense, rpw32<D, kDense>()>(p, stream);
    case kSparse: return launch_attn_t<D, 32, 32, kSparse, 2, 2>(p, stream);
    case kMassTwoPass: return launch_attn_t<D, 32, 32, kMassTwoPass, 2, 2>(p, stream);
    default:
      if constexpr (fused_mass_spills<D, 32>()) return hipErrorInvalidValue;
      else return launch_attn_t<D, 32, 32, kDenseMass, 1, 2>(p, stream);
  }
}

template <int D, int BLK>
size_t attn_lds_bytes_blk(int mode_in, int nblk) {
  const int mode = effective_mode<D, BLK>(mode_in, nblk);
  const AttnCfg c = choose_cfg<D, BLK>(mode, nblk);
  return c.kt ? cfg_lds<D, BLK>(c.kt, c.rpw, mode, nblk) : 0;
}

// The workspace mass mode exists for blocks 32, 64 and 128; block 16 runs
// the LDS mass launches (two logical blocks per tile, small partials).
inline int mode_for_block(int block, int mode) {
  return (mode == kDenseMassWs && block < 32) ? kDenseMass : mode;
}

template <int D>
size_t attn_lds_bytes_d(int block, int mode_in, int nblk) {
  const int mode = mode_for_block(block, mode_in);
  switch (block) {
    case 16: return attn_lds_bytes_b16<D>(mode, nblk);
    case 32: return attn_lds_bytes_blk<D, 32>(mode, nblk);
    case 64: return attn_lds_bytes_blk<D, 64>(mode, nblk);
    case 128: return attn_lds_bytes_blk<D, 128>(mode, nblk);
  }
  return 0;
}

template <int D>
hipError_t launch_attn_d(int block, int mode_in, const AttnParams& p, hipStream_t stream) {
  const int mode = mode_for_block(block, mode_in);
  switch (block) {
    case 16: return launch_attn_b16<D>(mode, p, stream);
    case 32: return launch_attn_blk<D, 32>(mode, p, stream);
    case 64: return launch_attn_blk<D, 64>(mode, p, stream);
    case 128: return launch_attn_blk<D, 128>(mode, p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace wise
