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
//    LDS with global_load_lds (no register staging), up to three chunks in
//    flight ahead of the one computed, by the older wave of each SIMD at the
//    end of its chunk (see the gather below).  Rows are stored with their
//    16-byte pieces XOR-swizzled by (row & 7) so the operand reads below are
//    free of LDS bank conflicts.
//  * Each wave owns 16*HTQ heads from scores to output, so the waves share
//    nothing but the latent chunks and meet at one barrier per chunk.
//  * Scores: S^T[key, head] = K . Q^T on bf16 MFMA 16x16x32 with Q^T resident
//    in registers.
//  * Softmax: fp32 in the exp2 domain with a lazily moved running maximum (the
//    accumulators are only rescaled when a head's maximum grows by more than
//    2^8, so probabilities stay <= 256).  P is rounded to bf16 and stays in
//    registers: the MFMA result layout of S^T leaves a lane with one head and
//    the 8 keys {4g..4g+3, 16+4g..16+4g+3} (g = lane/16), which is exactly
//    the B operand of the value product whose V^T operand (lane group g)
//    reads those 8 latent rows.
//  * Values: O^T[d, head] += V^T . P^T on bf16 MFMA 16x16x32 over all D_v
//    columns of the wave's heads; V^T comes from the row-major latent chunk
//    through the transposing ds_read_b64_tr_b16.
// Per wave, Q^T (16 heads x 576) takes 72 registers and the fp32 output
// accumulators (16 heads x 512) 128; NW = 8 runs two waves per SIMD, and with
// no barrier between a wave's softmax and its value products one wave's
// softmax overlaps the other's matrix work.  Every wave reads the whole chunk
// (K for its scores, V for its values): 8 x 68 KiB of LDS reads per 32-key
// chunk, against 8 x 68 matrix products of 16 x 16 x 32.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kChunk = 32;     // keys per chunk
constexpr float kLazyMax = 8.0f;

template <int DQK, int DV, int NW>
struct AttnShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;
  static constexpr int HTQ = 128 / 16 / NW;         // 16-head tiles per wave
  static constexpr int DT = DV / 16;                // value d-tiles (all of them, per wave)
  static constexpr int RS = DQKP * 2;               // LDS bytes per latent row
  static constexpr int PPR = RS / 16;               // 16-byte pieces per LDS row
  static constexpr int RPR = DQK * 2 / 16;          // pieces present in the cache row
  static constexpr int CHUNK_BYTES = kChunk * RS;
  static constexpr int DMA_BLOCKS = CHUNK_BYTES / 1024;  // 64 lanes x 16 bytes
  static constexpr bool SWZ = PPR % 8 == 0;
  static_assert(CHUNK_BYTES % 1024 == 0, "chunk must be whole 1 KiB DMA blocks");
  static_assert(HTQ >= 1 && HTQ * 16 * NW == 128, "score heads must tile 128");
  static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "unsupported latent shape");
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
// STAGES: latent chunks in the LDS ring (STAGES - 1 gathers in flight).
template <int DQK, int DV, int NW, bool MASKED, int STAGES>
__global__ __launch_bounds__(64 * NW) void sparse_mla_kernel(AttnArgs a) {
  using S = AttnShape<DQK, DV, NW>;
  static_assert(STAGES >= 2 && STAGES <= 4, "2 to 4 chunk buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* kvb = smem;                                        // [STAGES][CHUNK_BYTES]
  int32_t* sidx = (int32_t*)(smem + STAGES * S::CHUNK_BYTES);  // [nch * kChunk]
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

  // sparse mode: the row's selected indices, loaded ahead of Q (k <= 64 chunks)
  const int32_t* idx_row0 = a.indices + (size_t)row * a.k;
  constexpr int kIdxPer = (64 * kChunk + 64 * NW - 1) / (64 * NW);
  int iv[kIdxPer];
#pragma unroll
  for (int j = 0; j < kIdxPer; ++j) {
    const int i = c_lo * kChunk + (int)threadIdx.x + j * (int)blockDim.x;
    iv[j] = (!MASKED && i < c_hi * kChunk) ? (i < a.k ? idx_row0[i] : -1) : 0;
  }

  // ---- Q^T fragments of this wave's heads (B operand of the score products),
  // loaded first so that their latency overlaps the index staging below
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
    // ---- selected indices -> LDS (entries outside [0, Lk) become -1); their
    // loads were issued before Q's, so only they are waited for here
    // A chunk's 32 entries belong to one half of one wave, so two ballots
    // give the chunk's "some valid" / "all valid" flags; they meet in a byte
    // per chunk in the last chunk buffer (the first gathers go elsewhere).
    uint8_t* cflag = kvb + (STAGES - 1) * S::CHUNK_BYTES;
#pragma unroll
    for (int j = 0; j < kIdxPer; ++j) {
      const int i = c_lo * kChunk + (int)threadIdx.x + j * (int)blockDim.x;
      const bool in = i < c_hi * kChunk;
      const bool valid = in && iv[j] >= 0 && iv[j] < a.Lk;
      if (in) sidx[i] = valid ? iv[j] : -1;
      const uint64_t vb64 = __ballot(valid);
      const uint32_t half = (uint32_t)(vb64 >> (lane & 32));
      if ((lane & 31) == 0 && in)
        cflag[i / kChunk] = (uint8_t)((half != 0u ? 1 : 0) | (half == 0xFFFFFFFFu ? 2 : 0));
    }
    __syncthreads();
    const bool mine = lane >= c_lo && lane < c_hi;
    const int fl = mine ? cflag[lane] : 0;
    chunk_mask = __ballot(fl & 1);
    full_mask = __ballot(fl & 2);
  }

  // ---- gather of one chunk by the first GW waves, BPW 1 KiB blocks each
  // (blocks [BPW*w, BPW*w + BPW)), in runs of up to 5 blocks: one M0 value
  // per run (the LDS address of the run's third block) and immediate offsets
  // -2048..2048 reach a run's blocks.  Waves w and w + NW/2 share a SIMD and
  // the older one (w < NW/2) is issued first, so it reaches the end of a
  // chunk first; it takes the whole copy while the younger wave catches up.
  // The global base sits 4 KiB below the sequence's cache so that the
  // per-lane offsets, which absorb the immediate, stay non-negative.
  const uint8_t* kv_bias = (const uint8_t*)(a.kv + (size_t)b * a.Lk * DQK) - 4096;
  constexpr int GW = NW / 2;
  constexpr int BPW = S::DMA_BLOCKS / GW;
  constexpr int R1 = BPW < 5 ? BPW : 5;  // blocks of the first run
  constexpr int R2 = BPW - R1;            // and of the second
  static_assert(S::DMA_BLOCKS % GW == 0 && R2 <= 5, "whole runs of 1 to 5 blocks per gathering wave");
  static_assert(div_mul_exact(S::PPR, 64 * S::DMA_BLOCKS), "piece -> row split by multiply-shift");
  const bool gathers = wave < GW;
  const int j_lo = wave * BPW;
  auto issue = [&](int c, int buf) {
    if (!gathers) return;
    // All row indices are read before the copies are issued: the copies are
    // asm statements with a memory clobber, so no look-up can move past them.
    // The lane offsets are recomputed per call (hoisting them out of the chunk
    // loop would hold BPW registers), and any spill reload here would make the
    // compiler wait for every gather in flight.
    int ln;
    asm volatile("v_mov_b32 %0, %1" : "=v"(ln) : "v"(lane));
    uint32_t off[2][5] = {{0, 0, 0, 0, 0}, {0, 0, 0, 0, 0}};
    // When the wave's blocks cover exactly the latent rows 8w .. 8w + 7 of
    // the chunk (576-column rows: 9 blocks of 64 pieces = 8 rows of 72), block
    // j1 spans at most rows t0 and t0 + 1 of them, split at lane `cut`, and
    // the row's low 3 bits are its place among the eight; the eight indices
    // come from two broadcast LDS reads instead of one look-up per block.
    constexpr bool kEightRows = !MASKED && S::SWZ && BPW * 64 == 8 * S::PPR;
    int rid[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if constexpr (kEightRows) {
      const v4i ia = *(const v4i*)(sidx + c * kChunk + 8 * wave);
      const v4i ib = *(const v4i*)(sidx + c * kChunk + 8 * wave + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rid[e] = ia[e];
        rid[4 + e] = ib[e];
      }
    }
#pragma unroll
    for (int j1 = 0; j1 < BPW; ++j1) {
      const int run = j1 < R1 ? 0 : 1, j0 = j1 < R1 ? j1 : j1 - R1;
      uint32_t lp;  // logical piece of this lane's 16 bytes in its row
      int idx;      // latent row index of that row
      if constexpr (kEightRows) {
        const int t0 = 64 * j1 / S::PPR;
        const int cut = S::PPR * (t0 + 1) - 64 * j1;
        const bool first = cut >= 64 || ln < cut;
        const uint32_t t = first ? (uint32_t)t0 : (uint32_t)t0 + 1;
        lp = (64u * (uint32_t)j1 + (uint32_t)ln - t * (uint32_t)S::PPR) ^ t;
        idx = max(first ? rid[t0] : rid[t0 < 7 ? t0 + 1 : 7], 0);
      } else {
        const uint32_t p = 64u * (uint32_t)(j_lo + j1) + (uint32_t)ln;
        const uint32_t r = __umul24(p, div_mul(S::PPR)) >> kDivShift;
        const uint32_t pp = p - r * (uint32_t)S::PPR;
        lp = S::SWZ ? (pp ^ (r & 7u)) : pp;
        idx = MASKED ? min(kChunk * c + (int)r, n_keys - 1) : max(sidx[c * kChunk + r], 0);
      }
      // Pad pieces (score width rounded up to 32) re-read real ones; they
      // meet zero q.  The swizzle keeps a piece inside its aligned group of
      // 8, so without padding every piece is a real one.
      uint32_t src_col = lp;
      if constexpr (S::PPR != S::RPR) src_col = lp < (uint32_t)S::RPR ? lp : lp - S::RPR;
      // row indices are < 2^24 and the cache is < 4 GiB - 8 KiB (checked by the host)
      off[run][j0] = __umul24((uint32_t)idx, DQK * 2) + 16 * src_col + 4096 - 1024 * (j0 - 2);
    }
    const uint8_t* dst = kvb + buf * S::CHUNK_BYTES + 1024 * j_lo;
    dma_run<R1>(__builtin_amdgcn_readfirstlane(lds_offset(dst + 1024 * 2)), kv_bias, off[0]);
    if constexpr (R2 > 0)
      dma_run<R2>(__builtin_amdgcn_readfirstlane(lds_offset(dst + 1024 * (R1 + 2))), kv_bias, off[1]);
  };
  // wait until this wave's copies of all but the `later` (0 .. STAGES - 2)
  // most recently issued chunks have landed
  auto wait_gather = [&](int later) {
    if (!gathers) return;
    if (later <= 0) wait_vmcnt<0>();
    else if (later == 1 || STAGES < 4) wait_vmcnt<BPW>();
    else wait_vmcnt<2 * BPW>();
  };

  // physical byte offset of logical 16-byte piece `lp` in LDS row `r`
  auto piece = [](int r, int lp) { return 16 * (S::SWZ ? (lp ^ (r & 7)) : lp); };

  v4f acc[S::HTQ][S::DT];
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) acc[ht][dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
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
  for (int s = 0; s < STAGES - 1; ++s) issue_next(s);

  // Per-lane LDS byte offsets of the operand reads.  With the swizzle, logical
  // piece lp of row r sits at piece lp ^ (r & 7): 8*(lp>>3) + ((lp&7) ^ (r&7)).
  //  K rows 16kt + li (row & 7 == li & 7); logical piece 4ks + g, so piece
  //  8*(ks>>1) + ((4*(ks&1) + g) ^ (li&7)): a per-lane base per ks parity plus
  //  a compile-time 128-byte step.
  int k_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) k_off[par] = li * S::RS + piece(li, 4 * par + g);
  //  V^T rows 4g + li/4 (k-slots 8g..8g+3) and 16 + 4g + li/4 (8g+4..8g+7),
  //  both with row & 7 == (4g + li/4) & 7; logical piece 2*dt + (li&3)/2 of
  //  d-tile dt, plus 8*(li&1) bytes inside the piece.
  //  Pieces 2dt + sel and 2(dt + 4) + sel differ by 8, outside the swizzle's
  //  low 3 bits, so four per-lane bases (dt & 3) plus a compile-time 128-byte
  //  step per 4 d-tiles reach every d-tile.
  const int r_v0 = 4 * g + (li >> 2);
  int v_off[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) v_off[q] = r_v0 * S::RS + 8 * (li & 1) + piece(r_v0, 2 * q + ((li & 3) >> 1));

  int buf = 0;  // it % STAGES
  for (int it = 0; it < total; ++it, buf = buf + 1 == STAGES ? 0 : buf + 1) {
    int c;
    if constexpr (MASKED) {
      c = c_lo + it;
    } else {
      c = __builtin_ctzll(to_compute);
      to_compute &= to_compute - 1;
    }
    const uint8_t* kb = kvb + buf * S::CHUNK_BYTES;

    // This chunk's rows have landed (for this wave's copies; the barrier then
    // covers every wave's), and every wave is done with the previous chunk,
    // whose buffer takes the next gather.
    wait_gather(min(total - 1 - it, STAGES - 2));
    __syncthreads();

    // ---- S^T = K_chunk . Q^T for 2 key tiles x HTQ head tiles
    v4f s[S::HTQ][2];
#pragma unroll
    for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) s[ht][kt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    {
      // K fragments are prefetched two K-steps ahead; the scheduling fences
      // keep the compiler from hoisting the whole chunk's loads (registers).
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
    }

    // ---- softmax for this lane's heads over its 8 keys, in registers
    // Raw scores; the scale (> 0, so it keeps the order) is applied to the
    // maximum and folded into the exponent's FMA.  Only chunks holding
    // invalid entries (-1 padding) are masked: a wave-uniform branch.  In
    // masked mode chunks not wholly selected are masked by their bits; a head's
    // maximum stays -inf until a selected entry is seen, and while it does
    // every score is -inf and is taken against 0 (giving p = 0, not NaN).
    // P leaves as bf16 in exactly the B-operand layout of the value products:
    // the lane holds head li and keys {4g..4g+3, 16+4g..16+4g+3}, the k-slots
    // 8g..8g+7 of the transposed latent rows read below.
    uint32_t bits = 0;
    if constexpr (MASKED) bits = __builtin_amdgcn_readfirstlane(selm[c]);
    const bool full = MASKED ? bits == 0xFFFFFFFFu : (full_mask >> c) & 1;
    v8bf pf[S::HTQ];
    float al[S::HTQ];
    bool rescale = false;
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
      al[ht] = 1.0f;
      if (mloc > m_use[ht] + kLazyMax) {
        al[ht] = fast_exp2(m_use[ht] - mloc);
        m_use[ht] = mloc;
        rescale = true;
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
      l_part[ht] = l_part[ht] * al[ht] + psum;
      pf[ht] = __builtin_bit_cast(v8bf, (v4i){(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});
    }
    if (__ballot(rescale)) {
#pragma unroll
      for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
        for (int dt = 0; dt < S::DT; ++dt) acc[ht][dt] *= al[ht];
    }

    // ---- O^T = O^T + V^T . P^T for every d-tile of this wave's heads; V^T
    // through the transposing reads, kVPre d-tiles ahead
    constexpr int kVPre = S::DT < 2 ? S::DT : 2;
    __builtin_amdgcn_sched_barrier(0);
    v8bf va[kVPre];
    auto load_v = [&](int dt) {
      const int voff = v_off[dt & 3] + 128 * (dt >> 2);
      const v4s lo = lds_read_tr16(kb + voff);
      const v4s hi = lds_read_tr16(kb + voff + 16 * S::RS);
      return __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    };
#pragma unroll
    for (int dt = 0; dt < kVPre; ++dt) va[dt] = load_v(dt);
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      const v8bf v = va[dt % kVPre];
      if (dt + kVPre < S::DT) va[dt % kVPre] = load_v(dt + kVPre);
#pragma unroll
      for (int ht = 0; ht < S::HTQ; ++ht) acc[ht][dt] = mfma_bf16_16x16x32(v, pf[ht], acc[ht][dt]);
      __builtin_amdgcn_sched_barrier(0);
    }
    // the next gather, into the buffer every wave released at this chunk's
    // barrier; issued last so that the copies queue while waves wait there
    issue_next(buf == 0 ? STAGES - 1 : buf - 1);
  }

  // ---- row sums, lse, and this wave's heads normalised and stored
  float* out_base = a.nsplit > 1 ? a.part_out + (size_t)vb * a.H * DV
                                 : a.out + (size_t)row * a.H * DV;
  float* lse_base = a.nsplit > 1 ? a.part_lse + (size_t)vb * a.H
                                 : (a.lse ? a.lse + (size_t)row * a.H : nullptr);
  // The output rows go out through LDS so that a store instruction writes two
  // heads x 512 contiguous bytes instead of 16 heads x 64 (the MFMA result
  // layout).  Each wave stages 8 d-tiles (16 heads x 128 columns, 8 KiB) at a
  // time in one of the chunk buffers that the last chunk did not use: every
  // wave passed the last chunk's barrier, so no wave reads them any more and
  // no gather into them is in flight.  16-byte unit u of head h sits at unit
  // u ^ h (low 4 bits), so both the writes and the reads are conflict-free.
  constexpr int kPieceDt = 8;
  constexpr bool kStaged = S::HTQ == 1 && S::DT % kPieceDt == 0 && STAGES >= 3 &&
                           (NW / 2) * 16 * kPieceDt * 64 <= S::CHUNK_BYTES;
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    float l = l_part[ht] + __shfl_xor(l_part[ht], 16);
    l += __shfl_xor(l, 32);
    const int head = 16 * (S::HTQ * wave + ht) + li;
    if (g == 0 && lse_base && head < a.H)
      lse_base[head] = l > 0.0f ? (m_use[ht] + fast_log2(l)) * 0.69314718055994530942f : -INFINITY;
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if constexpr (kStaged) {
      const int last = buf == 0 ? STAGES - 1 : buf - 1;  // buffer of the last chunk
      int sb = last + 1 + wave / (NW / 2);
      sb = sb >= STAGES ? sb - STAGES : sb;
      sb = sb >= STAGES ? sb - STAGES : sb;
      uint8_t* slot = kvb + sb * S::CHUNK_BYTES + (wave % (NW / 2)) * (16 * kPieceDt * 64);
      const int hh = lane >> 5, u = lane & 31;
#pragma unroll
      for (int pc = 0; pc < S::DT / kPieceDt; ++pc) {
#pragma unroll
        for (int j = 0; j < kPieceDt; ++j)
          *(v4f*)(slot + li * (kPieceDt * 64) + 16 * ((4 * j + g) ^ li)) = acc[ht][kPieceDt * pc + j] * inv;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int h2 = 2 * j + hh;
          const v4f v = *(const v4f*)(slot + h2 * (kPieceDt * 64) + 16 * (u ^ h2));
          const int hd = 16 * (S::HTQ * wave + ht) + h2;
          if (hd < a.H) *(v4f*)(out_base + (size_t)hd * DV + 16 * kPieceDt * pc + 4 * u) = v;
        }
      }
    } else if (head < a.H) {
      float* orow = out_base + (size_t)head * DV;
#pragma unroll
      for (int dt = 0; dt < S::DT; ++dt) *(v4f*)(orow + 16 * dt + 4 * g) = acc[ht][dt] * inv;
    }
  }
}

// Merge of the parts of split rows: lse = log(sum_p exp(lse_p)) and
// out = sum_p exp(lse_p - lse) * out_p (each part is normalised by its own
// softmax sum); a row without any valid entry keeps out = 0, lse = -inf.
// One block per (row, head), one 4-column group per thread.  Every part's
// lse and columns are loaded before any is used, so a thread waits for one
// memory latency instead of two (the lse, then the columns it weighs).
constexpr int kMaxParts = 8;  // attn_splits never splits a row further
__global__ __launch_bounds__(128) void attn_combine_kernel(AttnArgs a) {
  const int rh = blockIdx.x;  // row * H + head
  const int row = rh / a.H, head = rh % a.H;
  const int np = a.nsplit;
  const float* lp = a.part_lse + (size_t)row * np * a.H + head;
  const float* op = a.part_out + ((size_t)row * np * a.H + head) * a.Dv;
  for (int d4 = threadIdx.x; d4 < a.Dv / 4; d4 += blockDim.x) {
    float lv[kMaxParts];
    v4f ov[kMaxParts];
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) {
      lv[p] = p < np ? lp[(size_t)p * a.H] : -INFINITY;
      ov[p] = p < np ? *(const v4f*)(op + (size_t)p * a.H * a.Dv + 4 * d4) : (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    }
    float m = -INFINITY;
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) m = fmaxf(m, lv[p]);
    float sum = 0.0f;
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p) sum += (p < np && m != -INFINITY) ? __expf(lv[p] - m) : 0.0f;
    const float lse = sum > 0.0f ? m + __logf(sum) : -INFINITY;
    if (d4 == 0 && a.lse) a.lse[rh] = lse;
    v4f o = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int p = 0; p < kMaxParts; ++p)
      if (p < np && lv[p] != -INFINITY) o += __expf(lv[p] - lse) * ov[p];
    *(v4f*)(a.out + (size_t)rh * a.Dv + 4 * d4) = o;
  }
}

template <int DQK, int DV, int NW, bool MASKED, int STAGES>
hipError_t launch_stages(const AttnArgs& a, size_t smem, hipStream_t stream) {
  const void* kern = (const void*)sparse_mla_kernel<DQK, DV, NW, MASKED, STAGES>;
  static const hipError_t attr = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr != hipSuccess) return attr;
  const long long rows = (long long)a.B * a.Lq;
  return launch_kernel(kern, dim3((unsigned)(rows * a.nsplit)), dim3(64 * NW), smem, stream, a);
}

template <int DQK, int DV, int NW, bool MASKED>
hipError_t launch_shape(const AttnArgs& a, hipStream_t stream) {
  using S = AttnShape<DQK, DV, NW>;
  if (a.nsplit < 1 || a.nsplit > kMaxParts) return hipErrorInvalidValue;  // the merge holds 8 parts
  // sparse: the staged indices; masked: one selection word per chunk of the row
  const size_t tail = MASKED ? (size_t)((a.Lk + kChunk - 1) / kChunk) * sizeof(uint32_t)
                             : (size_t)((a.k + kChunk - 1) / kChunk) * kChunk * sizeof(int32_t);
  // four chunk buffers where the LDS holds them, else three
  constexpr size_t kLds = 160 * 1024;
  hipError_t e;
  if (4 * (size_t)S::CHUNK_BYTES + tail <= kLds)
    e = launch_stages<DQK, DV, NW, MASKED, 4>(a, 4 * (size_t)S::CHUNK_BYTES + tail, stream);
  else if (3 * (size_t)S::CHUNK_BYTES + tail <= kLds)
    e = launch_stages<DQK, DV, NW, MASKED, 3>(a, 3 * (size_t)S::CHUNK_BYTES + tail, stream);
  else
    return hipErrorInvalidValue;
  if (e != hipSuccess || a.nsplit == 1) return e;
  const long long rows = (long long)a.B * a.Lq;
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
