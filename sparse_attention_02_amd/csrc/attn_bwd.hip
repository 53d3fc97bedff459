// Backward of the sparse attention in the MQA mode of MLA over fixed indices
// (gfx950): the step on the other side of the path in the sparse training
// stage, where every parameter is trained with the selection on
// (DeepSeek-V3.2 spec sheet, design overview; lightning-indexer post,
// training section).  The indices are fixed: no gradient flows into them.
//
// Per (row t, head h) over the listed entries i (token s_i), with the
// forward's z_i = scale * q . kv_i, p = softmax(z) = exp(z - lse) and
// o = sum_i p_i v_i (v_i = the first D_v columns of kv_i), for an upstream
// gradient dout of o:
//   D = dout . o,  dp_i = dout . v_i,  dz_i = p_i (dp_i - D),
//   dq = scale * sum_i dz_i kv_i,
//   dkv[s_i] += scale * dz_i q  (+ p_i dout on the value columns).
//
// dq contracts over the keys and dkv over the heads, hence separate kernels:
//  1. scores and dq (one wave per 16 heads, 64 heads per block): the
//     selected latent rows are gathered into LDS in chunks of 32; S^T = K.Q^T
//     and dP^T = V.dO^T run on bf16 MFMA sharing each K fragment read; P comes
//     straight from the forward's lse, dZ = P (dP - D); then dQ^T += K^T.dZ^T
//     from the same chunk with the transposing reads of the forward's value
//     product, into accumulators held for the whole row.  P and dZ go to the
//     workspace in bf16, key-major (dZ times scale), for kernel 2.
//  2. dkv: per row, the partial product scale * dZ.Q + P.dO of every slot
//     over the 128 heads on bf16 MFMA (one block per row, Q and dO held in
//     registers), stored in bf16; per key, the sum over the (row, slot) pairs
//     that list it (inverted lists built by count / scan / fill kernels), added
//     into dkv by one wave per key.
#include <algorithm>

#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBChunk = 32;   // keys per chunk
constexpr int kBTiles = 8;    // 128 heads / 16 (absent heads are zero)
constexpr int kBHeads = 128;  // padded head count of the key-major buffers
// per head tile and chunk, the scores kernel holds P and dZ of 8 keys per lane
// and stores the tile's P and dZ (32 keys x 16 heads each) with one 16-byte
// store apiece, after a transpose through LDS
constexpr int kScoreStoreKeys = 8;
constexpr int kScoreStores = 2;
constexpr int kStageBytes = 2 * kBChunk * 16 * 2;  // per wave: [P, dZ][32 keys][16 heads] bf16

template <int DQK, int DV, int NW>
struct BwdShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;              // k-steps of the score product
  static constexpr int KSTV = DV / 32;               // k-steps of the dout . v product
  static constexpr int HTQ = kBTiles / NW;           // 16-head tiles per wave
  static constexpr int NDT = DQKP / 16;              // 16-column d-tiles of dq
  static constexpr int RS = DQKP * 2;                // LDS bytes per latent row
  static constexpr int PPR = RS / 16;                // 16-byte pieces per LDS row
  static constexpr int RPR = DQK * 2 / 16;           // pieces present in the cache row
  static constexpr bool SWZ = PPR % 8 == 0;
  static constexpr int CHUNK_BYTES = kBChunk * RS;
  static constexpr int NT = 64 * NW;
  static constexpr int PIECES = kBChunk * PPR;
  static constexpr int PER = (PIECES + NT - 1) / NT;  // pieces per thread in a chunk load
  static_assert(DV % 32 == 0 && DQK % 8 == 0 && HTQ * NW == kBTiles, "unsupported latent shape");
};

// physical byte offset of logical 16-byte piece lp in LDS row r (the forward's
// swizzle: the K-fragment and transposing V reads are free of bank conflicts)
template <typename S>
__device__ __forceinline__ int bwd_piece(int r, int lp) {
  return 16 * (S::SWZ ? (lp ^ (r & 7)) : lp);
}

// A chunk of 32 selected latent rows: loaded into registers (the next chunk
// while the current one is used), then stored to LDS.  Entries outside
// [0, Lk) load row 0 (in bounds; their probabilities are zero).
// The thread index goes through an opaque move in each call so that the
// per-piece row/column split is recomputed rather than hoisted out of the
// chunk loop, where it would hold registers for the whole kernel.
__device__ __forceinline__ int opaque_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"((int)threadIdx.x));
  return t;
}

// Global stores issued through inline assembly, one instruction each, in
// the loops whose vmcnt waits count them: the number of vector memory
// operations between a chunk's copies and the wait is then fixed by the
// source, not by how the compiler might split or merge the stores.  The
// s_nop keeps the store data registers untouched for the wait states a
// VALU write after a store needs (the hazard check does not see into asm).
__device__ __forceinline__ void store_b128(void* p, v4i v) {
  asm volatile("global_store_dwordx4 %0, %1, off\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}
__device__ __forceinline__ void store_b64(void* p, v2i v) {
  asm volatile("global_store_dwordx2 %0, %1, off\n\ts_nop 1" :: "v"(p), "v"(v) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Gather of a chunk's 32 latent rows straight into LDS: each copy moves 16
// bytes per lane from (base + off_i) to LDS (m0 + 16 i), so lane i fetches
// the logical piece that the swizzle puts at physical slot i of the row.
// Issued through inline assembly (the compiler does not track these LDS
// writes); the caller waits for them with s_waitcnt vmcnt(0) and a barrier
// before the chunk is read.  `base` is wave-uniform.
template <typename S, int NW>
__device__ __forceinline__ void dma_chunk(uint8_t* dst, const uint8_t* base, const int32_t* sidx_c, int wave) {
  constexpr int BLOCKS = S::CHUNK_BYTES / 1024;
  const int ln = opaque_tid() & 63;
#pragma unroll
  for (int j = 0; j < (BLOCKS + NW - 1) / NW; ++j) {
    const int blk = wave + NW * j;
    if (blk < BLOCKS) {
      const int p = 64 * blk + ln;
      const int r = p / S::PPR, pp = p % S::PPR;
      const int lp = S::SWZ ? (pp ^ (r & 7)) : pp;
      const int col = lp < S::RPR ? lp : lp - S::RPR;  // pad pieces re-read real ones (they meet zero q)
      const uint32_t off = (uint32_t)max(sidx_c[r], 0) * (uint32_t)(S::RPR * 16) + 16u * (uint32_t)col;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * blk));
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                   :: "v"(off), "s"(m0), "s"(base) : "memory", "m0");
    }
  }
}

template <typename S>
struct ChunkRegs {
  v4i pf[S::PER];
  __device__ __forceinline__ void load(const uint8_t* seq, const int32_t* sidx_c) {
    const int tid = opaque_tid();
#pragma unroll
    for (int j = 0; j < S::PER; ++j) {
      const int p = tid + j * S::NT;
      if (p < S::PIECES) {
        const int r = p / S::PPR, lp = p % S::PPR;
        const int idx = max(sidx_c[r], 0);
        pf[j] = lp < S::RPR ? *(const v4i*)(seq + (size_t)idx * (S::RPR * 16) + 16 * lp) : (v4i){0, 0, 0, 0};
      }
    }
  }
  __device__ __forceinline__ void store(uint8_t* dst) const {
    const int tid = opaque_tid();
#pragma unroll
    for (int j = 0; j < S::PER; ++j) {
      const int p = tid + j * S::NT;
      if (p < S::PIECES) {
        const int r = p / S::PPR, lp = p % S::PPR;
        *(v4i*)(dst + r * S::RS + bwd_piece<S>(r, lp)) = pf[j];
      }
    }
  }
};

// Selected indices of a row -> LDS (entries outside [0, Lk) become -1, slots
// past k too).  Ends with a barrier.
__device__ __forceinline__ void stage_indices(const AttnBwdArgs& a, int row, int nch, int32_t* sidx) {
  const int32_t* idx_row = a.indices + (size_t)row * a.k;
  for (int i = threadIdx.x; i < nch * kBChunk; i += blockDim.x) {
    const int v = i < a.k ? idx_row[i] : -1;
    sidx[i] = (v >= 0 && v < a.Lk) ? v : -1;
  }
  __syncthreads();
}

// ---- 1. scores and dq: P and dZ of every (row, entry, head) -> workspace,
//         dq = scale * sum_i dZ_i kv_i -> dq
// Q^T and dO^T of its heads stay in the wave's registers for the whole row
// (72 + 64 per 16 heads at the 576/512 shape) and so do the fp32 dq
// accumulators (144, matrix accumulator registers), more than two waves per
// SIMD leave room for, so the kernel runs one wave per SIMD; the 8 head tiles
// are split over SPLIT blocks of NW waves with HTQ tiles each.  The chunks are
// copied straight into LDS, so no register holds the next chunk.  The dq
// products of a chunk read its K^T tiles four ahead: with one wave per SIMD
// nothing else hides the read latency (without the prefetch the fused kernel
// gained 3 % over a separate dq kernel, with it 12 %).
template <int DQK, int DV, int NW, int SPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_scores_kernel(AttnBwdArgs a) {
  using S = BwdShape<DQK, DV, NW * SPLIT>;  // HTQ = 8 / (NW * SPLIT) head tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* kvb = smem;                                   // [2][CHUNK_BYTES]
  int32_t* sidx = (int32_t*)(smem + 2 * S::CHUNK_BYTES);  // [nch * 32]
  // per wave: P and dZ of a head tile, key-major, for the 16-byte stores
  uint16_t* stg = (uint16_t*)(smem + 2 * S::CHUNK_BYTES + (size_t)((a.k + kBChunk - 1) / kBChunk) * kBChunk * 4 +
                              kStageBytes * (threadIdx.x >> 6));

  const int lane = threadIdx.x & 63;
  const int wave_b = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave in the block
  const int g = lane >> 4, li = lane & 15;
  const int row = blockIdx.x / SPLIT;
  const int wave = (int)(blockIdx.x % SPLIT) * NW + wave_b;  // wave among the row's NW * SPLIT
  const int b = row / a.Lq;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  stage_indices(a, row, nch, sidx);

  // ---- per-wave operands: Q^T and dO^T of its heads (B operands), D, lse
  v8bf qf[S::HTQ][S::KST], dof[S::HTQ][S::KSTV];
  float Dh[S::HTQ], lse2[S::HTQ];
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    const int head = 16 * (S::HTQ * wave + ht) + li;
    const bool ok = head < a.H;
    const uint16_t* qrow = a.q + ((size_t)row * a.H + (ok ? head : 0)) * DQK;
    const float* grow = a.dout + ((size_t)row * a.H + (ok ? head : 0)) * DV;
    const float* orow = a.out + ((size_t)row * a.H + (ok ? head : 0)) * DV;
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      v4i v = {0, 0, 0, 0};
      if (ok && d0 + 8 <= DQK) v = *(const v4i*)(qrow + d0);
      qf[ht][ks] = __builtin_bit_cast(v8bf, v);
    }
    float dpart = 0.0f;
#pragma unroll
    for (int ks = 0; ks < S::KSTV; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      v4f g0 = {0, 0, 0, 0}, g1 = g0, o0 = g0, o1 = g0;
      if (ok) {
        g0 = *(const v4f*)(grow + d0);
        g1 = *(const v4f*)(grow + d0 + 4);
        o0 = *(const v4f*)(orow + d0);
        o1 = *(const v4f*)(orow + d0 + 4);
      }
      const v4i pk = {(int)pack_bf16x2(g0[0], g0[1]), (int)pack_bf16x2(g0[2], g0[3]),
                      (int)pack_bf16x2(g1[0], g1[1]), (int)pack_bf16x2(g1[2], g1[3])};
      dof[ht][ks] = __builtin_bit_cast(v8bf, pk);
      // D = dout . o from the same bf16-rounded dout as dP = dout . v, so that
      // sum_i p_i (dP_i - D) = 0 holds as in exact arithmetic (with fp32 dout
      // here a one-token row would get dZ ~ rounding of dout instead of 0)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t x = (uint32_t)pk[w];
        const float ov0 = w < 2 ? o0[2 * w] : o1[2 * w - 4], ov1 = w < 2 ? o0[2 * w + 1] : o1[2 * w - 3];
        dpart += __uint_as_float(x << 16) * ov0 + __uint_as_float(x & 0xFFFF0000u) * ov1;
      }
      // consumed step by step: issuing every step's loads at once would take
      // 256 registers and push the operands above into scratch
      __builtin_amdgcn_sched_barrier(0);
    }
    // the four lane groups hold the head's columns 8g..8g+7 of every k-step
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(dpart), __float_as_uint(dpart), false, false);
    dpart = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(dpart), __float_as_uint(dpart), false, false);
    Dh[ht] = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    lse2[ht] = ok ? a.lse[(size_t)row * a.H + head] * 1.44269504088896340736f : -INFINITY;
  }

  int k_off[2];
#pragma unroll
  for (int par = 0; par < 2; ++par) k_off[par] = li * S::RS + bwd_piece<S>(li, 4 * par + g);
  // dQ^T = K^T . dZ^T from the chunk in LDS: the A operand of d-tile t through
  // the transposing reads of rows 4g + li/4 and 16 + 4g + li/4 (k-slots
  // 8g..8g+7, the key order of the dZ fragment); four per-lane bases (t & 3)
  // and a 128-byte step per four tiles reach every tile.
  const int r_v0 = 4 * g + (li >> 2);
  int v_off[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4)
    v_off[q4] = r_v0 * S::RS + 8 * (li & 1) + bwd_piece<S>(r_v0, 2 * q4 + ((li & 3) >> 1));
  v4f dacc[S::HTQ][S::NDT];
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
    for (int t = 0; t < S::NDT; ++t) dacc[ht][t] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  const uint8_t* seq = (const uint8_t*)(a.kv + (size_t)b * a.Lk * DQK);
  dma_chunk<S, NW>(kvb, seq, sidx, wave_b);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  const size_t kpad = (size_t)nch * kBChunk;
  for (int c = 0; c < nch; ++c) {
    const uint8_t* kb = kvb + (c & 1) * S::CHUNK_BYTES;
    // the next chunk lands in the other buffer while this one is used
    if (c + 1 < nch)
      dma_chunk<S, NW>(kvb + ((c + 1) & 1) * S::CHUNK_BYTES, seq, sidx + (c + 1) * kBChunk, wave_b);

    v4f sacc[S::HTQ][2], pacc[S::HTQ][2];
#pragma unroll
    for (int ht = 0; ht < S::HTQ; ++ht)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) sacc[ht][kt] = pacc[ht][kt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    // K fragments two k-steps ahead; the scheduling fences keep the compiler
    // from hoisting the whole chunk's loads (register pressure)
    constexpr int kPre = 2;
    v8bf kf[kPre + 1][2];
    auto load_k = [&](int ks, v8bf* dst) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
        dst[kt] = __builtin_bit_cast(v8bf, *(const v4i*)(kb + k_off[ks & 1] + 16 * kt * S::RS + 128 * (ks >> 1)));
    };
#pragma unroll
    for (int ks = 0; ks < kPre && ks < S::KST; ++ks) load_k(ks, kf[ks]);
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      if (ks + kPre < S::KST) load_k(ks + kPre, kf[(ks + kPre) % (kPre + 1)]);
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < S::HTQ; ++ht) {
          sacc[ht][kt] = mfma_bf16_16x16x32(kf[ks % (kPre + 1)][kt], qf[ht][ks], sacc[ht][kt]);
          if (ks < S::KSTV)
            pacc[ht][kt] = mfma_bf16_16x16x32(kf[ks % (kPre + 1)][kt], dof[ht][ks], pacc[ht][kt]);
        }
      __builtin_amdgcn_sched_barrier(0);
    }

    // lane: head 16*tile + li, keys 4g + r (tile kt = 0) and 16 + 4g + r (kt = 1)
#pragma unroll
    for (int ht = 0; ht < S::HTQ; ++ht) {
      const int tile = S::HTQ * wave + ht;
      const int head = 16 * tile + li;
      float pv[kScoreStoreKeys], zv[kScoreStoreKeys];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = 16 * kt + 4 * g + r;
          const bool valid = sidx[c * kBChunk + key] >= 0 && head < a.H;
          const float p = valid ? fast_exp2(fmaf(sacc[ht][kt][r], a.scale_log2, -lse2[ht])) : 0.0f;
          pv[4 * kt + r] = p;
          zv[4 * kt + r] = p * (pacc[ht][kt][r] - Dh[ht]);
        }
      // dZ in bf16 as the B operand of dQ^T += K^T . dZ^T (k-slots 8g..8g+7)
      const v4i zf = {(int)pack_bf16x2(zv[0], zv[1]), (int)pack_bf16x2(zv[2], zv[3]),
                      (int)pack_bf16x2(zv[4], zv[5]), (int)pack_bf16x2(zv[6], zv[7])};
      const v8bf zb = __builtin_bit_cast(v8bf, zf);
      auto load_kt = [&](int t) {
        const int voff = v_off[t & 3] + 128 * (t >> 2);
        const v4s lo = lds_read_tr16(kb + voff);
        const v4s hi = lds_read_tr16(kb + voff + 16 * S::RS);
        return __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      };
      constexpr int kTPre = 4;  // K^T tiles read ahead
      v8bf ktp[kTPre + 1];
#pragma unroll
      for (int t = 0; t < kTPre && t < S::NDT; ++t) ktp[t] = load_kt(t);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < S::NDT; ++t) {
        if (t + kTPre < S::NDT) ktp[(t + kTPre) % (kTPre + 1)] = load_kt(t + kTPre);
        dacc[ht][t] = mfma_bf16_16x16x32(ktp[t % (kTPre + 1)], zb, dacc[ht][t]);
        __builtin_amdgcn_sched_barrier(0);
      }
      // P and scale * dZ key-major [row][slot][128 heads] for the dkv
      // products: the tile goes through the wave's LDS stage ([32 keys][16
      // heads] each), then lane 2k + u stores heads 8u .. 8u + 7 of key k
      // (LDS operations of one wave complete in order, so no barrier)
#pragma unroll
      for (int e = 0; e < kScoreStoreKeys; ++e) {
        const int key = 16 * (e >> 2) + 4 * g + (e & 3);
        stg[key * 16 + li] = (uint16_t)(pack_bf16x2(pv[e], 0.0f) & 0xFFFFu);
        stg[kBChunk * 16 + key * 16 + li] = (uint16_t)(pack_bf16x2(zv[e] * a.scale, 0.0f) & 0xFFFFu);
      }
      const int ln = opaque_tid() & 63;
      const v4i pst = *(const v4i*)(stg + 8 * ln);
      const v4i zst = *(const v4i*)(stg + kBChunk * 16 + 8 * ln);
      const size_t o = ((size_t)row * kpad + (size_t)c * kBChunk + (ln >> 1)) * kBHeads + 16 * tile + 8 * (ln & 1);
      store_b128(a.ws_pk + o, pst);
      store_b128(a.ws_dzk + o, zst);
    }
    // the next chunk's copies are complete and every wave is done with this
    // one.  Vector memory operations retire in issue order, so waiting until
    // only this chunk's stores (kScoreStores per head tile, all issued after
    // the copies) may be outstanding is enough: the stores drain behind the
    // next chunk.
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(kScoreStores * S::HTQ) : "memory");
    __syncthreads();
  }

  // dq of this wave's heads: lane holds d = 16t + 4g + r of head 16*tile + li
#pragma unroll
  for (int ht = 0; ht < S::HTQ; ++ht) {
    const int head = 16 * (S::HTQ * wave + ht) + li;
    if (head >= a.H) continue;
#pragma unroll
    for (int t = 0; t < S::NDT; ++t) {
      const int d0 = 16 * t + 4 * g;
      if (d0 < DQK) *(v4f*)(a.dq + ((size_t)row * a.H + head) * DQK + d0) = dacc[ht][t] * a.scale;
    }
  }
}

// ---- 2. dkv[s] += sum over the (row, slot) pairs listing s of
//         scale * dZ[slot,:] . Q + P[slot,:] . dO        (contracted over heads)
// Fp32 atomics into dkv run at about one element per L2 channel and clock,
// far below the rate the partial products are made at, so the reduction goes
// through memory instead: every (row, slot) product is stored once in bf16,
// the pairs are listed per key (count, scan, fill), and one wave per key sums
// its list in fp32 and adds the total into dkv.  Each key is written by one
// wave only; the order of a list depends on the fill's atomics, so the last
// bits of dkv may vary from run to run.

constexpr int kScanThreads = 256;
constexpr int kScanPer = 16;
constexpr int kScanBlock = kScanThreads * kScanPer;  // keys per block of the scan

__global__ __launch_bounds__(256) void bwd_zero_kernel(int32_t* p, long long n) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < n; i += (long long)gridDim.x * 256) p[i] = 0;
}

// number of valid entries per key (b, s)
__global__ __launch_bounds__(256) void bwd_count_kernel(AttnBwdArgs a) {
  const long long total = (long long)a.B * a.Lq * a.k;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int s = a.indices[i];
  if (s < 0 || s >= a.Lk) return;
  const int b = (int)(i / ((long long)a.Lq * a.k));
  atomicAdd(a.ws_cnt + (size_t)b * a.Lk + s, 1);
}

// exclusive scan of NT values over the block; `total` gets the block sum
template <int NT>
__device__ __forceinline__ int block_exclusive_scan(int v, int* lds, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int before = 0, sum = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
    const int t = lds[w];
    before += w < wave ? t : 0;
    sum += t;
  }
  __syncthreads();
  total = sum;
  return before + x - v;
}

// per block of kScanBlock keys: the sum of its counts
__global__ __launch_bounds__(kScanThreads) void bwd_scan_sums_kernel(const int32_t* cnt, int32_t* bsum, long long n) {
  __shared__ int lds[kScanThreads / 64];
  const long long base = (long long)blockIdx.x * kScanBlock + (long long)threadIdx.x * kScanPer;
  int v = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) v += base + j < n ? cnt[base + j] : 0;
  int total;
  block_exclusive_scan<kScanThreads>(v, lds, total);
  if (threadIdx.x == 0) bsum[blockIdx.x] = total;
}

// exclusive scan of the block sums in place (one block)
__global__ __launch_bounds__(1024) void bwd_scan_top_kernel(int32_t* bsum, int nb) {
  __shared__ int lds[16];
  int carry = 0;
  for (int base = 0; base < nb; base += 1024) {
    const int i = base + (int)threadIdx.x;
    const int v = i < nb ? bsum[i] : 0;
    int total;
    const int ex = block_exclusive_scan<1024>(v, lds, total);
    if (i < nb) bsum[i] = carry + ex;
    carry += total;
  }
}

// list offsets of the keys: off = cur = exclusive scan of the counts
__global__ __launch_bounds__(kScanThreads) void bwd_scan_apply_kernel(AttnBwdArgs a, long long n) {
  __shared__ int lds[kScanThreads / 64];
  const long long base = (long long)blockIdx.x * kScanBlock + (long long)threadIdx.x * kScanPer;
  int c[kScanPer];
  int v = 0;
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    c[j] = base + j < n ? a.ws_cnt[base + j] : 0;
    v += c[j];
  }
  int total;
  int run = block_exclusive_scan<kScanThreads>(v, lds, total) + a.ws_bsum[blockIdx.x];
#pragma unroll
  for (int j = 0; j < kScanPer; ++j) {
    if (base + j < n) {
      a.ws_off[base + j] = run;
      a.ws_cur[base + j] = run;
    }
    run += c[j];
  }
}

// place every valid (row, slot) in its key's list as row * kpad + slot
__global__ __launch_bounds__(256) void bwd_fill_kernel(AttnBwdArgs a) {
  const long long total = (long long)a.B * a.Lq * a.k;
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int s = a.indices[i];
  if (s < 0 || s >= a.Lk) return;
  const long long row = i / a.k;
  const int slot = (int)(i - row * a.k);
  const int b = (int)(row / a.Lq);
  const int kpad = (a.k + kBChunk - 1) / kBChunk * kBChunk;
  const int p = atomicAdd(a.ws_cur + (size_t)b * a.Lk + s, 1);
  a.ws_list[p] = (int)(row * kpad + slot);
}

// 1 KB of a chunk copied straight into LDS: lane i fills bytes 16i..16i+15
// of the destination from base + off.  Waited for by the caller (vmcnt(0) and a
// barrier).  `base` is wave-uniform.
__device__ __forceinline__ void dma_1k(uint8_t* dst, const uint8_t* base, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst));
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
               :: "v"(off), "s"(m0), "s"(base) : "memory", "m0");
}

// Partial products of one row: part[row*kpad + slot, :] (bf16) =
//   (scale dZ)[slot, :] . Q  (+ P[slot, :] . dO on the value columns),
// contracted over the 128 (padded) heads on bf16 MFMA in transposed form,
// part^T = Q^T . (scale dZ)^T + dO^T . P^T: wave w holds Q^T and dO^T of the
// 16-column tiles w, w + NW, ... (NW * TPW tiles cover the row exactly) as A
// operands for the whole row, and the
// key-major dZ / P chunks of 32 slots come through LDS as B operands shared by
// all waves.  Each lane then holds 4 consecutive columns of one slot.
// LDS rows (one slot, 128 heads = 256 bytes) store 16-byte piece lp at
// physical piece lp ^ (slot & 15), so the 16 slots of a B fragment read hit 16
// different bank groups.
template <int DQK, int DV, int NW, int TPW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dkv_part_kernel(AttnBwdArgs a) {
  constexpr int NDT = DQK / 16;
  constexpr int CH = kBChunk * kBHeads * 2;  // bytes of one chunk of dZ (or P)
  static_assert(DQK % 16 == 0 && DV % 16 == 0 && NW * TPW == NDT, "column tiles must split evenly over the waves");
  __shared__ __attribute__((aligned(16))) uint8_t buf[2][2][CH];  // [stage][dZ, P][slot][heads]
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int row = blockIdx.x;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  const size_t kpad = (size_t)nch * kBChunk;

  // A operands: column 16t + li, heads 32 ks + 8g .. +7.  Absent heads, and
  // dO on the rope columns, are zero (loads use clamped in-bounds addresses,
  // then select), so every wave runs the same branch-free loop.
  v8bf qa[TPW][4], ga[TPW][4];
#pragma unroll
  for (int j = 0; j < TPW; ++j) {
    const int t = wave + NW * j;
    const bool has_v = 16 * t < DV;  // wave-uniform
    const int col = 16 * t + li;
    const uint16_t* qrow = a.q + (size_t)row * a.H * DQK + col;
    const float* grow = a.dout + (size_t)row * a.H * DV + (has_v ? col : 0);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      // an opaque copy of the lane's first head keeps the compiler from
      // holding every head's address across tiles (it recomputes them)
      const int h0 = 32 * ks + 8 * (opaque_tid() >> 4 & 3);
      uint32_t qw[4], gw[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float qv[2], gv[2];
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          const int head = h0 + 2 * e + u;
          const int hc = min(head, a.H - 1);
          const bool ok = head < a.H;
          const float x = bf16_bits_to_float(qrow[(size_t)hc * DQK]);
          const float y = grow[(size_t)hc * DV];  // in bounds for rope tiles too
          qv[u] = ok ? x : 0.0f;
          gv[u] = ok && has_v ? y : 0.0f;
        }
        qw[e] = pack_bf16x2(qv[0], qv[1]);
        gw[e] = pack_bf16x2(gv[0], gv[1]);
      }
      // packed here: the empty asm keeps the compiler from sinking the
      // conversion into the chunk loop (it would keep the unpacked values)
      v4i qp = {(int)qw[0], (int)qw[1], (int)qw[2], (int)qw[3]};
      v4i gp = {(int)gw[0], (int)gw[1], (int)gw[2], (int)gw[3]};
      asm volatile("" : "+v"(qp), "+v"(gp));
      qa[j][ks] = __builtin_bit_cast(v8bf, qp);
      ga[j][ks] = __builtin_bit_cast(v8bf, gp);
    }
  }

  // chunk c of dZ and P (contiguous CH bytes each) -> buf[st]; 1 KB per copy
  const uint8_t* zsrc = (const uint8_t*)(a.ws_dzk + (size_t)row * kpad * kBHeads);
  const uint8_t* psrc = (const uint8_t*)(a.ws_pk + (size_t)row * kpad * kBHeads);
  auto issue = [&](int c, int st) {
    constexpr int BLOCKS = 2 * CH / 1024;
#pragma unroll
    for (int j = 0; j < (BLOCKS + NW - 1) / NW; ++j) {
      const int blk = wave + NW * j;
      if (blk < BLOCKS) {
        const int arr = blk / (CH / 1024), sub = blk % (CH / 1024);
        const int slot = 4 * sub + (lane >> 4);
        const int lp = (lane & 15) ^ (slot & 15);
        const uint8_t* base = (arr ? psrc : zsrc) + (size_t)c * CH;
        dma_1k(&buf[st][arr][1024 * sub], base, (uint32_t)(slot * 256 + 16 * lp));
      }
    }
  };

  issue(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int st = c & 1;
    if (c + 1 < nch) issue(c + 1, st ^ 1);
    v4f acc[TPW][2];
#pragma unroll
    for (int j = 0; j < TPW; ++j) acc[j][0] = acc[j][1] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int slot = 16 * kt + li;
        const int off = slot * 256 + 16 * ((4 * ks + g) ^ (slot & 15));
        const v8bf zb = __builtin_bit_cast(v8bf, *(const v4i*)&buf[st][0][off]);
        const v8bf pb = __builtin_bit_cast(v8bf, *(const v4i*)&buf[st][1][off]);
#pragma unroll
        for (int j = 0; j < TPW; ++j) {
          acc[j][kt] = mfma_bf16_16x16x32(qa[j][ks], zb, acc[j][kt]);
          acc[j][kt] = mfma_bf16_16x16x32(ga[j][ks], pb, acc[j][kt]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane: columns 16t + 4g .. +3 of slot 32c + 16kt + li
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      uint16_t* prow = a.ws_part + ((size_t)row * kpad + (size_t)c * kBChunk + 16 * kt + li) * DQK;
#pragma unroll
      for (int j = 0; j < TPW; ++j)
        store_b64(prow + 16 * (wave + NW * j) + 4 * g, (v2i){(int)pack_bf16x2(acc[j][kt][0], acc[j][kt][1]),
                                                            (int)pack_bf16x2(acc[j][kt][2], acc[j][kt][3])});
    }
    // the next chunk's copies are complete and every wave is done with this
    // one; only this chunk's 2 * TPW partial-row stores (one store_b64 per
    // key tile and column tile, issued after the copies; vector memory
    // operations retire in issue order) may still be outstanding
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(2 * TPW) : "memory");
    __syncthreads();
  }
}

// One wave per key (b, s): dkv[b, s, :] += sum of the partial rows its list
// names, in fp32.  Lane l owns 16-byte pieces l, l + 64, ... of the row; the
// list is read 64 entries at a time and each entry broadcast from its lane.
template <int DQK>
__global__ __launch_bounds__(256) void attn_bwd_dkv_reduce_kernel(AttnBwdArgs a) {
  constexpr int NP = DQK / 8;
  constexpr int PPL = (NP + 63) / 64;
  constexpr int U = 4;  // entries in flight
  const int lane = threadIdx.x & 63;
  const long long key = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (key >= (long long)a.B * a.Lk) return;
  const int n = a.ws_cnt[key];
  if (n == 0) return;
  const int base = a.ws_off[key];
  float acc[PPL][8];
#pragma unroll
  for (int pp = 0; pp < PPL; ++pp)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[pp][e] = 0.0f;
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int m = min(64, n - i0);
    const int mine = lane < m ? a.ws_list[base + i0 + lane] : 0;
    for (int e = 0; e < m; e += U) {
      v4i v[U][PPL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int pos = __builtin_amdgcn_readlane(mine, e + u);  // e + u < 64
        const uint16_t* prow = a.ws_part + (size_t)pos * DQK;
#pragma unroll
        for (int pp = 0; pp < PPL; ++pp) {
          const int piece = lane + 64 * pp;
          v[u][pp] = e + u < m && piece < NP ? *(const v4i*)(prow + 8 * piece) : (v4i){0, 0, 0, 0};
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int pp = 0; pp < PPL; ++pp)
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            const uint32_t x = (uint32_t)v[u][pp][w];
            acc[pp][2 * w] += __uint_as_float(x << 16);
            acc[pp][2 * w + 1] += __uint_as_float(x & 0xFFFF0000u);
          }
    }
  }
  float* drow = a.dkv + (size_t)key * DQK;
#pragma unroll
  for (int pp = 0; pp < PPL; ++pp) {
    const int piece = lane + 64 * pp;
    if (piece < NP) {
      v4f* d = (v4f*)(drow + 8 * piece);
      v4f lo = d[0], hi = d[1];
      lo += (v4f){acc[pp][0], acc[pp][1], acc[pp][2], acc[pp][3]};
      hi += (v4f){acc[pp][4], acc[pp][5], acc[pp][6], acc[pp][7]};
      d[0] = lo;
      d[1] = hi;
    }
  }
}

// Workspace layout (byte offsets, each part 256-byte aligned).
struct BwdLayout {
  size_t pk, dzk, part, list, cnt, off, cur, bsum, total;
};

size_t align256(size_t x) { return (x + 255) / 256 * 256; }

BwdLayout bwd_layout(int B, int Lq, int Lk, int k, int dqk) {
  const size_t rows = (size_t)B * Lq;
  const size_t kpad = (size_t)(k + kBChunk - 1) / kBChunk * kBChunk;
  const size_t keys = (size_t)B * Lk;
  const size_t hm = align256(rows * kpad * kBHeads * sizeof(uint16_t));
  BwdLayout l{};
  l.pk = 0;
  l.dzk = l.pk + hm;
  l.part = l.dzk + hm;
  l.list = l.part + align256(rows * kpad * dqk * sizeof(uint16_t));
  l.cnt = l.list + align256(rows * k * sizeof(int32_t));
  l.off = l.cnt + align256(keys * sizeof(int32_t));
  l.cur = l.off + align256(keys * sizeof(int32_t));
  l.bsum = l.cur + align256(keys * sizeof(int32_t));
  l.total = l.bsum + align256((keys + kScanBlock - 1) / kScanBlock * sizeof(int32_t));
  return l;
}

// Scores (and dq) kernel: SPLIT blocks of NW1 waves per row;
// partial-product kernel: NW3 waves with TPW column tiles each.
template <int DQK, int DV, int NW1, int SPLIT, int NW3, int TPW>
hipError_t launch_bwd_shape(const AttnBwdArgs& a, hipStream_t stream) {
  using S1 = BwdShape<DQK, DV, NW1 * SPLIT>;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  const size_t sidx_bytes = (size_t)nch * kBChunk * sizeof(int32_t);
  const size_t smem1 = 2 * (size_t)S1::CHUNK_BYTES + sidx_bytes + (size_t)NW1 * kStageBytes;
  static const hipError_t attr1 = hipFuncSetAttribute(
      (const void*)attn_bwd_scores_kernel<DQK, DV, NW1, SPLIT>, hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr1 != hipSuccess) return attr1;
  const unsigned rows = (unsigned)((long long)a.B * a.Lq);
  const long long entries = (long long)rows * a.k;
  const long long keys = (long long)a.B * a.Lk;
  const unsigned nb = (unsigned)((keys + kScanBlock - 1) / kScanBlock);
  const unsigned eb = (unsigned)((entries + 255) / 256);

  // key lists of the (row, slot) pairs
  hipError_t e = launch_kernel((const void*)bwd_zero_kernel, dim3((unsigned)std::min<long long>((keys + 255) / 256, 4096)),
                               dim3(256), 0, stream, a.ws_cnt, keys);
  if (e != hipSuccess) return e;
  if ((e = launch_kernel((const void*)bwd_count_kernel, dim3(eb), dim3(256), 0, stream, a)) != hipSuccess) return e;
  if ((e = launch_kernel((const void*)bwd_scan_sums_kernel, dim3(nb), dim3(kScanThreads), 0, stream,
                         (const int32_t*)a.ws_cnt, a.ws_bsum, keys)) != hipSuccess)
    return e;
  if ((e = launch_kernel((const void*)bwd_scan_top_kernel, dim3(1), dim3(1024), 0, stream, a.ws_bsum, (int)nb)) !=
      hipSuccess)
    return e;
  if ((e = launch_kernel((const void*)bwd_scan_apply_kernel, dim3(nb), dim3(kScanThreads), 0, stream, a, keys)) !=
      hipSuccess)
    return e;
  if ((e = launch_kernel((const void*)bwd_fill_kernel, dim3(eb), dim3(256), 0, stream, a)) != hipSuccess) return e;

  if ((e = launch_kernel((const void*)attn_bwd_scores_kernel<DQK, DV, NW1, SPLIT>, dim3(rows * SPLIT), dim3(64 * NW1),
                         smem1, stream, a)) != hipSuccess)
    return e;
  if ((e = launch_kernel((const void*)attn_bwd_dkv_part_kernel<DQK, DV, NW3, TPW>, dim3(rows), dim3(64 * NW3), 0,
                         stream, a)) != hipSuccess)
    return e;
  return launch_kernel((const void*)attn_bwd_dkv_reduce_kernel<DQK>, dim3((unsigned)((keys + 3) / 4)), dim3(256), 0,
                       stream, a);
}

}  // namespace

size_t attn_bwd_workspace_bytes(int B, int Lq, int Lk, int k, int dqk) {
  return bwd_layout(B, Lq, Lk, k, dqk).total;
}

hipError_t launch_sparse_mla_attn_bwd(const AttnBwdArgs& args, void* workspace, hipStream_t stream) {
  AttnBwdArgs a = args;
  const BwdLayout l = bwd_layout(a.B, a.Lq, a.Lk, a.k, a.Dv + a.Dr);
  uint8_t* w = (uint8_t*)workspace;
  a.ws_pk = (uint16_t*)(w + l.pk);
  a.ws_dzk = (uint16_t*)(w + l.dzk);
  a.ws_part = (uint16_t*)(w + l.part);
  a.ws_list = (int32_t*)(w + l.list);
  a.ws_cnt = (int32_t*)(w + l.cnt);
  a.ws_off = (int32_t*)(w + l.off);
  a.ws_cur = (int32_t*)(w + l.cur);
  a.ws_bsum = (int32_t*)(w + l.bsum);
  if (a.Dv == 512 && a.Dr == 64) return launch_bwd_shape<576, 512, 4, 2, 12, 3>(a, stream);
  if (a.Dv == 64 && a.Dr == 16) return launch_bwd_shape<80, 64, 4, 1, 5, 1>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
