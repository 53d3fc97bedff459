// Sparse attention in the MQA mode of MLA over the selected latents (gfx950).
//
// For every query row and head: softmax over the selected tokens of
// scale * <q_h, kv_s> using all D_v + D_r latent columns, then the
// probability-weighted sum of the first D_v columns.  One latent row per token
// is shared by every query head and the selection is made once per query
// position ("DeepSeek V3.2 and the lightning indexer", section "How the
// lightning indexer works"; DeepSeek-V3.2 spec sheet, "Inference efficiency",
// KV-cache design).  Sharing the selected rows across heads is what keeps the
// non-contiguous gather affordable (inference-research record on DSA: sparse
// attention loses to dense unless selection is group-shared).
//
// Mapping (one block of NW waves per query row):
//  * Gather: the selected latent rows are copied 32 at a time straight into
//    LDS with global_load_lds (no register staging), three chunks in flight.
//    Rows are stored with their 16-byte pieces XOR-swizzled by (row & 7) so the
//    operand reads below are free of LDS bank conflicts.
//  * Scores: wave w owns 16*HTQ heads.  S^T[key, head] = K . Q^T on bf16 MFMA
//    16x16x32 with Q^T resident in registers.
//  * Softmax: fp32 in the exp2 domain with a lazily moved running maximum (the
//    accumulators are only rescaled when a head's maximum grows by more than
//    2^8, so probabilities stay <= 256).  P is rounded to bf16 and exchanged
//    through LDS together with the per-head rescale factors.
//  * Values: wave w owns output columns [DV/NW * w, DV/NW * (w+1)) for all 128
//    heads: O^T[d, head] += V^T . P^T on bf16 MFMA 16x16x32.  V^T comes from the
//    row-major latent chunk through the transposing ds_read_b64_tr_b16 and is
//    reused by all eight 16-head tiles, so the slower transposing reads are
//    issued once per wave and d-tile, not once per head tile.
// Per SIMD, Q (128 heads) and the fp32 output accumulators (128 x 512) take
// about 400 of the 512 registers whatever the split; NW = 8 runs two waves per
// SIMD so one wave's softmax overlaps the other's matrix work.
// The MFMA result layout of S^T leaves a lane with one head and the 8 keys
// {4g..4g+3, 16+4g..16+4g+3} (g = lane/16); those 8 values are written as one
// 16-byte row segment of P, and the V^T operand of lane group g reads exactly
// those 8 latent rows, so both operands agree on the key order.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kChunk = 32;     // keys per chunk
constexpr int kStages = 3;     // latent chunks in flight
constexpr int kHeadTiles = 8;  // 128 heads / 16
constexpr int kPRow = 64;      // bytes of one head's P values (32 bf16)
constexpr float kLazyMax = 8.0f;

template <int DQK, int DV, int NW>
struct AttnShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;
  static constexpr int HTQ = 128 / 16 / NW;         // 16-head score tiles per wave
  static constexpr int DTW = DV / 16 / NW;          // value d-tiles per wave
  static constexpr int RS = DQKP * 2;               // LDS bytes per latent row
  static constexpr int PPR = RS / 16;               // 16-byte pieces per LDS row
  static constexpr int RPR = DQK * 2 / 16;          // pieces present in the cache row
  static constexpr int CHUNK_BYTES = kChunk * RS;
  static constexpr int DMA_BLOCKS = CHUNK_BYTES / 1024;  // 64 lanes x 16 bytes
  static constexpr bool SWZ = PPR % 8 == 0;
  static constexpr int P_BYTES = 128 * kPRow;
  static_assert(CHUNK_BYTES % 1024 == 0, "chunk must be whole 1 KiB DMA blocks");
  static_assert(HTQ >= 1 && HTQ * 16 * NW == 128, "score heads must tile 128");
  static_assert(DQK % 8 == 0 && DTW >= 1 && DTW * 16 * NW == DV && DV <= DQK, "unsupported latent shape");
};

// q / d for 0 <= q < n as (q * ceil(2^19 / d)) >> 19: exact when every q in
// range passes and q * multiplier fits 24 bits (both checked at compile time),
// a full-rate 24-bit multiply where a division by a constant costs
// quarter-rate multiply-highs.
constexpr int kDivShift = 19;
constexpr uint32_t div_mul(int d) { return ((1u << kDivShift) + (uint32_t)d - 1u) / (uint32_t)d; }
constexpr bool div_mul_exact(int d, int n) {
  for (int q = 0; q < n; ++q)
    if ((int)(((uint32_t)q * div_mul(d)) >> kDivShift) != q / d) return false;
  return (uint64_t)(n - 1) * div_mul(d) < (1u << 24);
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// N 1 KiB global -> LDS copies: copy n moves 16 bytes per lane i from
// (base + off[n]_i + o_n) to (lds_mid + o_n + 16 i) with o_n = 1024 * (n - 2).
// The instruction's immediate offset moves the LDS destination as well as the
// global source, so one M0 write serves the whole run; rewriting M0 stalls the
// wave while its earlier LDS operations drain, which made a write per copy the
// largest cost of the gather.  Issued through inline assembly so that the
// compiler does not insert a conservative wait for the copies before every
// later LDS read; completion is tracked with explicit vmcnt waits.  `base` is
// wave-uniform (SGPR pair).
#define DSA_DMA(i, o) "global_load_lds_dwordx4 %" #i ", %5 offset:" #o "\n\t"
template <int N>
__device__ __forceinline__ void dma_run(uint32_t lds_mid, const void* base, const uint32_t (&off)[5]) {
  static_assert(N >= 1 && N <= 5, "1 to 5 copies per run");
  if constexpr (N == 5)
    asm volatile("s_mov_b32 m0, %6\n\ts_nop 0\n\t" DSA_DMA(0, -2048) DSA_DMA(1, -1024) DSA_DMA(2, 0)
                 DSA_DMA(3, 1024) DSA_DMA(4, 2048)
                 :: "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds_mid)
                 : "memory", "m0");
  else if constexpr (N == 4)
    asm volatile("s_mov_b32 m0, %6\n\ts_nop 0\n\t" DSA_DMA(0, -2048) DSA_DMA(1, -1024) DSA_DMA(2, 0)
                 DSA_DMA(3, 1024)
                 :: "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds_mid)
                 : "memory", "m0");
  else if constexpr (N == 3)
    asm volatile("s_mov_b32 m0, %6\n\ts_nop 0\n\t" DSA_DMA(0, -2048) DSA_DMA(1, -1024) DSA_DMA(2, 0)
                 :: "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds_mid)
                 : "memory", "m0");
  else if constexpr (N == 2)
    asm volatile("s_mov_b32 m0, %6\n\ts_nop 0\n\t" DSA_DMA(0, -2048) DSA_DMA(1, -1024)
                 :: "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds_mid)
                 : "memory", "m0");
  else
    asm volatile("s_mov_b32 m0, %6\n\ts_nop 0\n\t" DSA_DMA(0, -2048)
                 :: "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "v"(off[4]), "s"(base), "s"(lds_mid)
                 : "memory", "m0");
}
#undef DSA_DMA

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

// MASKED: the masked mode for short prefill.  The row's whole causal range
// [0, pos(t)] is streamed in contiguous chunks and the entries outside the
// selection are masked in the softmax, instead of gathering the selected rows.
template <int DQK, int DV, int NW, bool MASKED>
__global__ __launch_bounds__(64 * NW) void sparse_mla_kernel(AttnArgs a) {
  using S = AttnShape<DQK, DV, NW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* kvb = smem;                                        // [kStages][CHUNK_BYTES]
  uint8_t* pbuf = smem + kStages * S::CHUNK_BYTES;            // [2][8 tiles][4 g][16 heads][16 B]
  float* alpha_s = (float*)(pbuf + 2 * S::P_BYTES);           // [2][16 lanes][8 head tiles]
  float* lsum_s = alpha_s + 2 * 128;                          // [128]
  int32_t* sidx = (int32_t*)(lsum_s + 128);                   // [nch * kChunk]
  uint32_t* selm = (uint32_t*)sidx;  // masked mode: [nch] selection bit per key of a chunk

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  __builtin_assume(wave >= 0 && wave < NW);
  const int g = lane >> 4;
  const int li = lane & 15;
  // Workgroups are dealt to the 8 XCDs in turn (block b to XCD b % 8), each
  // with its own L2.  Neighbouring query rows select largely the same latent
  // rows, so (row, part) items go to the XCDs in runs of kXcdRun consecutive
  // ones instead of one at a time, and their gathers meet in the same L2;
  // runs rather than one range per XCD keep the causal rows' uneven work
  // spread over all XCDs.  Blocks past the last whole round keep their index.
  constexpr int kXcdRun = 32;  // swept 8..128 at L=32K and L=4K: 32 best
  const int nb = gridDim.x;
  const int full = nb / (8 * kXcdRun) * (8 * kXcdRun);
  const int xi = blockIdx.x >> 3;
  const int vb = (int)blockIdx.x < full
                     ? ((xi / kXcdRun) * 8 + (int)(blockIdx.x & 7)) * kXcdRun + xi % kXcdRun
                     : (int)blockIdx.x;
  const int row = vb / a.nsplit;
  const int part = vb % a.nsplit;
  const int b = row / a.Lq;
  // masked mode: the row's causal range [0, n_keys) in chunks of kChunk keys
  const int n_keys = MASKED ? min(a.q_start + row % a.Lq + 1, a.Lk) : 0;
  const int nch = ((MASKED ? n_keys : a.k) + kChunk - 1) / kChunk;
  // chunks [c_lo, c_hi) of the row belong to this block
  const int c_lo = part * nch / a.nsplit, c_hi = (part + 1) * nch / a.nsplit;
  float* out_base = a.nsplit > 1 ? a.part_out + (size_t)vb * a.H * DV
                                 : a.out + (size_t)row * a.H * DV;
  float* lse_base = a.nsplit > 1 ? a.part_lse + (size_t)vb * a.H
                                 : (a.lse ? a.lse + (size_t)row * a.H : nullptr);

  uint64_t chunk_mask = 0, full_mask = 0;  // sparse: chunks with some / with only valid entries
  const int32_t* idx_row = a.indices + (size_t)row * a.k;
  if constexpr (MASKED) {
    // ---- selection bitmap of this block's chunks (entries outside its key
    // range, past pos(t) included, are not set; a repeated entry counts once)
    for (int i = c_lo + threadIdx.x; i < c_hi; i += blockDim.x) selm[i] = 0u;
    __syncthreads();
    const int s_lo = kChunk * c_lo, s_hi = min(kChunk * c_hi, n_keys);
    for (int i = threadIdx.x; i < a.k; i += blockDim.x) {
      const int v = idx_row[i];
      if (v >= s_lo && v < s_hi) atomicOr(&selm[v / kChunk], 1u << (v % kChunk));
    }
    __syncthreads();
  } else {
    // ---- selected indices -> LDS (entries outside [0, Lk) become -1)
    for (int i = c_lo * kChunk + threadIdx.x; i < c_hi * kChunk; i += blockDim.x) {
      const int v = i < a.k ? idx_row[i] : -1;
      sidx[i] = (v >= 0 && v < a.Lk) ? v : -1;
    }
    __syncthreads();
    const bool mine = lane >= c_lo && lane < c_hi;
    bool any = false, all = mine;
    if (mine)
      for (int j = 0; j < kChunk; ++j) {
        const bool v = sidx[lane * kChunk + j] >= 0;
        any |= v;
        all &= v;
      }
    chunk_mask = __ballot(any);
    full_mask = __ballot(all);
  }

  // ---- Q^T fragments of this wave's score heads (B operand)
  v8bf qf[S::HTQ][S::KST];
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    const int head = 16 * (S::HTQ * wave + ht) + li;
    const bool ok = head < a.H;
    const uint16_t* qrow = a.q + ((size_t)row * a.H + (ok ? head : 0)) * DQK;
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      v4i v = {0, 0, 0, 0};
      if (d0 + 8 <= DQK) v = *(const v4i*)(qrow + (d0 + 8 <= DQK ? d0 : 0));  // compile-time for DQK % 32 == 0
      if (!ok) v = (v4i){0, 0, 0, 0};
      qf[ht][ks] = __builtin_bit_cast(v8bf, v);
    }
  }

  // ---- gather of one chunk: this wave copies the 1 KiB blocks [j_lo, j_lo + n_j)
  // of the chunk (4 or 5 for the 576-wide rows), so one M0 value (the LDS
  // address of block j_lo + 2) and immediate offsets -2048..2048 reach them all.
  // The global base sits 4 KiB below the sequence's cache so that the per-lane
  // offsets, which absorb the immediate, stay non-negative.
  const uint8_t* kv_bias = (const uint8_t*)(a.kv + (size_t)b * a.Lk * DQK) - 4096;
  constexpr int NJ = (S::DMA_BLOCKS + NW - 1) / NW;
  static_assert(NJ <= 5 && S::DMA_BLOCKS / NW >= 1, "1 to 5 copies per wave and chunk");
  static_assert(div_mul_exact(S::PPR, 64 * S::DMA_BLOCKS), "piece -> row split by multiply-shift");
  const int j_lo = wave * S::DMA_BLOCKS / NW;
  const bool long_run = (wave + 1) * S::DMA_BLOCKS / NW - j_lo == NJ;
  auto issue = [&](int c, int buf) {
    // All row indices are read before the copies are issued: the copies are
    // one asm statement with a memory clobber, so no look-up can move past it.
    // The lane offsets are recomputed per call (hoisting them out of the chunk
    // loop would hold ~10 registers), and any spill reload here would make the
    // compiler wait for every gather in flight.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    uint32_t off[5] = {0, 0, 0, 0, 0};
#pragma unroll
    for (int j0 = 0; j0 < NJ; ++j0) {
      const int j = min(j_lo + j0, S::DMA_BLOCKS - 1);
      const uint32_t p = 64u * (uint32_t)j + (uint32_t)ln;
      const uint32_t r = __umul24(p, div_mul(S::PPR)) >> kDivShift;
      const uint32_t pp = p - r * (uint32_t)S::PPR;
      const uint32_t lp = S::SWZ ? (pp ^ (r & 7u)) : pp;
      // Pad pieces (score width rounded up to 32) re-read real ones; they
      // meet zero q.  The swizzle keeps a piece inside its aligned group of
      // 8, so without padding every piece is a real one.
      uint32_t src_col = lp;
      if constexpr (S::PPR != S::RPR) src_col = lp < (uint32_t)S::RPR ? lp : lp - S::RPR;
      const int idx = MASKED ? min(kChunk * c + (int)r, n_keys - 1) : max(sidx[c * kChunk + r], 0);
      // row indices are < 2^24 and the cache is < 4 GiB - 8 KiB (checked by the host)
      off[j0] = __umul24((uint32_t)idx, DQK * 2) + 16 * src_col + 4096 - 1024 * (j0 - 2);
    }
    const uint32_t mid =
        __builtin_amdgcn_readfirstlane(lds_offset(kvb + buf * S::CHUNK_BYTES + 1024 * (j_lo + 2)));
    if (long_run) dma_run<NJ>(mid, kv_bias, off);
    else dma_run<NJ - 1>(mid, kv_bias, off);
  };

  // physical byte offset of logical 16-byte piece `lp` in LDS row `r`
  auto piece = [](int r, int lp) { return 16 * (S::SWZ ? (lp ^ (r & 7)) : lp); };

  v4f acc[kHeadTiles][S::DTW];
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht)
#pragma unroll
    for (int dt = 0; dt < S::DTW; ++dt) acc[ht][dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  float m_use[S::HTQ], l_part[S::HTQ];
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    m_use[ht] = -INFINITY;
    l_part[ht] = 0.0f;
  }

  // The chunks this block computes, in order: the set bits of chunk_mask, or
  // in masked mode every chunk c_lo .. c_hi - 1.
  uint64_t to_issue = chunk_mask, to_compute = chunk_mask;
  int next_issue = c_lo;
  const int total = MASKED ? c_hi - c_lo : __builtin_popcountll(chunk_mask);
  auto issue_next = [&](int slot) {
    if constexpr (MASKED) {
      if (next_issue < c_hi) issue(next_issue++, slot);
    } else if (to_issue) {
      issue(__builtin_ctzll(to_issue), slot);
      to_issue &= to_issue - 1;
    }
  };
#pragma unroll
  for (int s = 0; s < kStages - 1; ++s) issue_next(s);

  // Per-lane LDS byte offsets of the operand reads.  With the swizzle, logical
  // piece lp of row r sits at piece lp ^ (r & 7): 8*(lp>>3) + ((lp&7) ^ (r&7)).
  //  K rows 16kt + li (row & 7 == li & 7); logical piece 4ks + g, so piece
  //  8*(ks>>1) + ((4*(ks&1) + g) ^ (li&7)): a per-lane base per ks parity plus
  //  a compile-time 128-byte step.
  int k_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) k_off[par] = li * S::RS + piece(li, 4 * par + g);
  //  V^T rows 4g + li/4 (k-slots 8g..8g+3) and 16 + 4g + li/4 (8g+4..8g+7),
  //  both with row & 7 == (4g + li/4) & 7; logical piece 2*dtg + (li&3)/2 of
  //  d-tile dtg, plus 8*(li&1) bytes inside the piece.
  const int r_v0 = 4 * g + (li >> 2);
  const int v_base = r_v0 * S::RS + 8 * (li & 1);
  const int v_sel = (li & 3) >> 1;
  //  P is stored piece-major: the 16-byte piece g of head 16ht + li sits at
  //  1024 ht + 256 g + 16 li, so both its writes and its reads are linear in
  //  the lane index.  (A head-major layout with an XOR swizzle, balanced over
  //  the 64 banks on paper, measured at half the LDS read rate.)
  const int p_off = 256 * g + 16 * li;

  for (int it = 0; it < total; ++it) {
    int c;
    if constexpr (MASKED) {
      c = c_lo + it;
    } else {
      c = __builtin_ctzll(to_compute);
      to_compute &= to_compute - 1;
    }
    const int buf = it % kStages;
    const uint8_t* kb = kvb + buf * S::CHUNK_BYTES;
    const int pslot = it & 1;

    // wait for this chunk's gather: at most one later chunk is in flight here
    if (it + 1 < total) {
      if (long_run) wait_vmcnt<NJ>();
      else wait_vmcnt<NJ - 1>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();

    // ---- S^T = K_chunk . Q^T for 2 key tiles x HTQ head tiles
    v4f s[S::HTQ][2];
#pragma unroll
    for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[ht][kt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    // K fragments are prefetched two K-steps ahead; the scheduling fences keep
    // the compiler from hoisting the whole chunk's loads (register pressure).
    constexpr int kPre = 2;
    v8bf kf[kPre + 1][2];
    auto load_k = [&](int ks, v8bf* dst) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        dst[kt] = __builtin_bit_cast(
            v8bf, *(const v4i*)(kb + k_off[ks & 1] + 16 * kt * S::RS + 128 * (ks >> 1)));
    };
#pragma unroll
    for (int ks = 0; ks < kPre && ks < S::KST; ++ks) load_k(ks, kf[ks]);
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      if (ks + kPre < S::KST) load_k(ks + kPre, kf[(ks + kPre) % (kPre + 1)]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < S::HTQ; ++ht)
          s[ht][kt] = mfma_bf16_16x16x32(kf[ks % (kPre + 1)][kt], qf[ht][ks], s[ht][kt]);
      __builtin_amdgcn_sched_barrier(0);
    }

    // ---- softmax for this lane's heads over its 8 keys; P and alpha -> LDS
    // Raw scores; the scale (> 0, so it keeps the order) is applied to the
    // maximum and folded into the exponent's FMA.  Only chunks holding
    // invalid entries (-1 padding) are masked: a wave-uniform branch.  In
    // masked mode chunks not wholly selected are masked by their bits; a head's
    // maximum stays -inf until a selected entry is seen, and while it does
    // every score is -inf and is taken against 0 (giving p = 0, not NaN).
    uint32_t bits = 0;
    if constexpr (MASKED) bits = __builtin_amdgcn_readfirstlane(selm[c]);
    const bool full = MASKED ? bits == 0xFFFFFFFFu : (full_mask >> c) & 1;
#pragma unroll
    for (int ht = 0; ht < S::HTQ; ++ht) {
      float z[8];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        z[r] = s[ht][0][r];
        z[4 + r] = s[ht][1][r];
      }
      if (MASKED && !full) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[r] = (bits >> (4 * g + r)) & 1u ? z[r] : -INFINITY;
          z[4 + r] = (bits >> (16 + 4 * g + r)) & 1u ? z[4 + r] : -INFINITY;
        }
      } else if (!MASKED && !full) {
        const v4i id0 = *(const v4i*)(sidx + c * kChunk + 4 * g);
        const v4i id1 = *(const v4i*)(sidx + c * kChunk + 16 + 4 * g);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          z[r] = id0[r] >= 0 ? z[r] : -INFINITY;
          z[4 + r] = id1[r] >= 0 ? z[4 + r] : -INFINITY;
        }
      }
      float mloc = fmaxf(fmaxf(fmaxf(z[0], z[1]), fmaxf(z[2], z[3])),
                         fmaxf(fmaxf(z[4], z[5]), fmaxf(z[6], z[7])));
      mloc = max_xor32(max_xor16(mloc)) * a.scale_log2;
      float al = 1.0f;
      if (mloc > m_use[ht] + kLazyMax) {
        al = fast_exp2(m_use[ht] - mloc);
        m_use[ht] = mloc;
      }
      uint32_t pk[4];
      float psum = 0.0f;
      float m_sub = m_use[ht];
      if constexpr (MASKED) m_sub = m_sub == -INFINITY ? 0.0f : m_sub;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p0 = fast_exp2(fmaf(z[2 * i], a.scale_log2, -m_sub));
        const float p1 = fast_exp2(fmaf(z[2 * i + 1], a.scale_log2, -m_sub));
        psum += p0 + p1;
        pk[i] = pack_bf16x2(p0, p1);
      }
      l_part[ht] = l_part[ht] * al + psum;
      const int head = 16 * (S::HTQ * wave + ht) + li;
      *(v4i*)(pbuf + pslot * S::P_BYTES + 1024 * (head >> 4) + p_off) =
          (v4i){(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]};
      if (g == 0) alpha_s[pslot * 128 + li * kHeadTiles + (head >> 4)] = al;
    }
    __syncthreads();

    // the chunk before this one is done everywhere: reuse its buffer for the next gather
    issue_next((it + kStages - 1) % kStages);

    // ---- O^T = alpha * O^T + V^T . P^T for this wave's d-range, all 128 heads
    float al8[kHeadTiles];
    {
      const v4f a0 = *(const v4f*)(alpha_s + pslot * 128 + li * kHeadTiles);
      const v4f a1 = *(const v4f*)(alpha_s + pslot * 128 + li * kHeadTiles + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        al8[i] = a0[i];
        al8[4 + i] = a1[i];
      }
    }
    bool rescale = false;
#pragma unroll
    for (int ht = 0; ht < kHeadTiles; ++ht) rescale |= al8[ht] != 1.0f;
    if (__ballot(rescale)) {
#pragma unroll
      for (int ht = 0; ht < kHeadTiles; ++ht)
#pragma unroll
        for (int dt = 0; dt < S::DTW; ++dt) acc[ht][dt] *= al8[ht];
    }
    // V^T fragments of this wave's d-tiles, then one P fragment per head tile
    v8bf va[S::DTW];
#pragma unroll
    for (int dt = 0; dt < S::DTW; ++dt) {
      const int voff = v_base + piece(r_v0, 2 * (wave * S::DTW + dt) + v_sel);
      const v4s lo = lds_read_tr16(kb + voff);
      const v4s hi = lds_read_tr16(kb + voff + 16 * S::RS);
      va[dt] = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
    const uint8_t* pb = pbuf + pslot * S::P_BYTES + p_off;
    auto load_p = [&](int ht) { return __builtin_bit_cast(v8bf, *(const v4i*)(pb + 16 * kPRow * ht)); };
    v8bf pf[2];
    pf[0] = load_p(0);
#pragma unroll
    for (int ht = 0; ht < kHeadTiles; ++ht) {
      if (ht + 1 < kHeadTiles) pf[(ht + 1) & 1] = load_p(ht + 1);
#pragma unroll
      for (int dt = 0; dt < S::DTW; ++dt) acc[ht][dt] = mfma_bf16_16x16x32(va[dt], pf[ht & 1], acc[ht][dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // ---- row sums of the score heads -> LDS; lse
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    float l = l_part[ht] + __shfl_xor(l_part[ht], 16);
    l += __shfl_xor(l, 32);
    const int head = 16 * (S::HTQ * wave + ht) + li;
    if (g == 0) {
      lsum_s[head] = l;
      if (lse_base && head < a.H)
        lse_base[head] = l > 0.0f ? (m_use[ht] + fast_log2(l)) * 0.69314718055994530942f : -INFINITY;
    }
  }
  __syncthreads();

  // ---- normalise and store this wave's columns of every head
#pragma unroll
  for (int ht = 0; ht < kHeadTiles; ++ht) {
    const int head = 16 * ht + li;
    if (head < a.H) {
      const float l = lsum_s[head];
      const float inv = l > 0.0f ? 1.0f / l : 0.0f;
      float* orow = out_base + (size_t)head * DV;
#pragma unroll
      for (int dt = 0; dt < S::DTW; ++dt) {
        const int d0 = 16 * (wave * S::DTW + dt) + 4 * g;
        *(v4f*)(orow + d0) = acc[ht][dt] * inv;
      }
    }
  }
}

// Merge of the parts of split rows: lse = log(sum_p exp(lse_p)) and
// out = sum_p exp(lse_p - lse) * out_p (each part is normalised by its own
// softmax sum); a row without any valid entry keeps out = 0, lse = -inf.
// One block per (row, head), one 4-column group per thread.
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int rh = blockIdx.x;  // row * H + head
  const int row = rh / a.H, head = rh % a.H;
  const float* lp = a.part_lse + (size_t)row * a.nsplit * a.H + head;
  float m = -INFINITY;
  for (int p = 0; p < a.nsplit; ++p) m = fmaxf(m, lp[(size_t)p * a.H]);
  float sum = 0.0f;
  for (int p = 0; p < a.nsplit; ++p) sum += m == -INFINITY ? 0.0f : __expf(lp[(size_t)p * a.H] - m);
  const float lse = sum > 0.0f ? m + __logf(sum) : -INFINITY;
  if (threadIdx.x == 0 && a.lse) a.lse[rh] = lse;
  for (int d4 = threadIdx.x; d4 < a.Dv / 4; d4 += blockDim.x) {
    v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int p = 0; p < a.nsplit; ++p) {
      const float lpp = lp[(size_t)p * a.H];
      if (lpp == -INFINITY) continue;
      const float wgt = __expf(lpp - lse);
      o += wgt * *(const v4f*)(a.part_out + (((size_t)row * a.nsplit + p) * a.H + head) * a.Dv + 4 * d4);
    }
    *(v4f*)(a.out + (size_t)rh * a.Dv + 4 * d4) = o;
  }
}

template <int DQK, int DV, int NW, bool MASKED>
hipError_t launch_shape(const AttnArgs& a, hipStream_t stream) {
  using S = AttnShape<DQK, DV, NW>;
  // sparse: the staged indices; masked: one selection word per chunk of the row
  const size_t tail = MASKED ? (size_t)((a.Lk + kChunk - 1) / kChunk) * sizeof(uint32_t)
                             : (size_t)((a.k + kChunk - 1) / kChunk) * kChunk * sizeof(int32_t);
  const size_t smem = (size_t)kStages * S::CHUNK_BYTES + 2 * (size_t)S::P_BYTES +
                      3 * 128 * sizeof(float) + tail;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)sparse_mla_kernel<DQK, DV, NW, MASKED>, hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  const long long rows = (long long)a.B * a.Lq;
  const hipError_t e = launch_kernel((const void*)sparse_mla_kernel<DQK, DV, NW, MASKED>,
                                     dim3((unsigned)(rows * a.nsplit)), dim3(64 * NW), smem, stream, a);
  if (e != hipSuccess || a.nsplit == 1) return e;
  return launch_kernel((const void*)attn_combine_kernel, dim3((unsigned)(rows * a.H)), dim3(128), 0,
                       stream, a);
}

}  // namespace

int attn_splits(int rows, int k) {
  // one block per CU at a time (the chunk ring fills most of the LDS): split
  // the chunks of a row when there are fewer rows than CUs
  constexpr int kCUs = 256;
  const int nch = (k + kChunk - 1) / kChunk;
  if (rows >= kCUs || nch < 4) return 1;
  int ns = kCUs / rows;
  if (ns > 8) ns = 8;
  if (ns > nch / 2) ns = nch / 2;
  return ns < 1 ? 1 : ns;
}

size_t attn_workspace_bytes(int rows, int k, int H, int Dv) {
  const int ns = attn_splits(rows, k);
  return ns > 1 ? (size_t)rows * ns * H * (Dv + 1) * sizeof(float) : 0;
}

hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.Dv == 512 && a.Dr == 64) return launch_shape<576, 512, 8, false>(a, stream);
  if (a.Dv == 64 && a.Dr == 16) return launch_shape<80, 64, 4, false>(a, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_masked_mha_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.nsplit != 1) return hipErrorInvalidValue;
  if (a.Dv == 512 && a.Dr == 64) return launch_shape<576, 512, 8, true>(a, stream);
  if (a.Dv == 64 && a.Dr == 16) return launch_shape<80, 64, 4, true>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
