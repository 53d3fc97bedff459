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
// Three kernels, because dq contracts over the keys and dkv over the heads:
//  1. scores (one wave per 16 heads, 64 heads per block): the
//     selected latent rows are gathered into LDS in chunks of 32; S^T = K.Q^T
//     and dP^T = V.dO^T run on bf16 MFMA sharing each K fragment read; P comes
//     straight from the forward's lse, dZ = P (dP - D).  P and dZ go to the
//     workspace in bf16, dZ once in the MFMA operand order of kernel 2 and
//     both once key-major for kernel 3.
//  2. dq (one block per row): dQ^T = K^T.dZ^T per chunk with the transposing
//     K reads of the forward's value product; wave w owns d-tiles w, w+NW, ...
//  3. dkv (one block per row and 64 columns): per 32-key chunk,
//     scale * dZ.Q + P.dO over the 128 heads on bf16 MFMA with Q and dO held
//     in registers for the whole row, then one fp32 atomic add per element of
//     the chunk's rows (rows are shared between queries).
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kBChunk = 32;   // keys per chunk
constexpr int kBTiles = 8;    // 128 heads / 16 (absent heads are zero)
constexpr int kBHeads = 128;  // padded head count of the key-major buffers

template <int DQK, int DV, int NW>
struct BwdShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;              // k-steps of the score product
  static constexpr int KSTV = DV / 32;               // k-steps of the dout . v product
  static constexpr int HTQ = kBTiles / NW;           // 16-head tiles per wave
  static constexpr int NDT = DQKP / 16;              // 16-column d-tiles
  static constexpr int DTQ = (NDT + NW - 1) / NW;    // d-tiles per wave in the dq kernel
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

// ---- 1. scores: P and dZ of every (row, entry, head) -> workspace
// Q^T and dO^T of its heads stay in the wave's registers for the whole row
// (72 + 64 per 16 heads at the 576/512 shape, more than two waves per SIMD
// leave room for), so the kernel runs one wave per SIMD; the 8 head tiles
// are split over SPLIT blocks of NW waves with HTQ tiles each.  The chunks are
// copied straight into LDS, so no register holds the next chunk.
template <int DQK, int DV, int NW, int SPLIT>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(1, 1)))
void attn_bwd_scores_kernel(AttnBwdArgs a) {
  using S = BwdShape<DQK, DV, NW * SPLIT>;  // HTQ = 8 / (NW * SPLIT) head tiles per wave
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* kvb = smem;                                   // [2][CHUNK_BYTES]
  int32_t* sidx = (int32_t*)(smem + 2 * S::CHUNK_BYTES);  // [nch * 32]

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
#pragma unroll
      for (int e = 0; e < 4; ++e) dpart += g0[e] * o0[e] + g1[e] * o1[e];
      const v4i pk = {(int)pack_bf16x2(g0[0], g0[1]), (int)pack_bf16x2(g0[2], g0[3]),
                      (int)pack_bf16x2(g1[0], g1[1]), (int)pack_bf16x2(g1[2], g1[3])};
      dof[ht][ks] = __builtin_bit_cast(v8bf, pk);
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
      float pv[8], zv[8];
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
      // dZ in the B-operand order of the dq kernel (k-slots 8g..8g+7)
      const v4i zf = {(int)pack_bf16x2(zv[0], zv[1]), (int)pack_bf16x2(zv[2], zv[3]),
                      (int)pack_bf16x2(zv[4], zv[5]), (int)pack_bf16x2(zv[6], zv[7])};
      *(v4i*)(a.ws_dzf + ((((size_t)row * nch + c) * kBTiles + tile) * 64 + lane) * 8) = zf;
      // P and dZ key-major [row][slot][128 heads] for the dkv kernel
      const int ln = opaque_tid() & 63;
      const size_t kmbase = ((size_t)row * kpad + (size_t)c * kBChunk + 4 * (ln >> 4)) * kBHeads +
                            16 * tile + (ln & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const size_t o = kmbase + (size_t)(16 * (e >> 2) + (e & 3)) * kBHeads;
        a.ws_pk[o] = (uint16_t)(pack_bf16x2(pv[e], 0.0f) & 0xFFFFu);
        a.ws_dzk[o] = (uint16_t)(pack_bf16x2(zv[e], 0.0f) & 0xFFFFu);
      }
    }
    // the next chunk's copies are complete and every wave is done with this one
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
}

// ---- 2. dq = scale * sum_i dZ_i kv_i
template <int DQK, int DV, int NW>
__global__ __launch_bounds__(64 * NW) void attn_bwd_dq_kernel(AttnBwdArgs a) {
  using S = BwdShape<DQK, DV, NW>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* kvb = smem;                                        // [2][CHUNK_BYTES]
  uint8_t* zbuf = smem + 2 * S::CHUNK_BYTES;                  // [2][8 tiles][64 lanes][16 B]
  int32_t* sidx = (int32_t*)(zbuf + 2 * kBTiles * 1024);      // [nch * 32]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int row = blockIdx.x;
  const int b = row / a.Lq;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  stage_indices(a, row, nch, sidx);

  // A operand (K^T of d-tile t) through the transposing reads of the
  // forward's value product: rows 4g + li/4 and 16 + 4g + li/4 of the chunk
  // give the k-slots 8g..8g+7 in the key order the dZ fragments use.
  const int r_v0 = 4 * g + (li >> 2);
  const int v_base = r_v0 * S::RS + 8 * (li & 1);
  const int v_sel = (li & 3) >> 1;

  const uint8_t* seq = (const uint8_t*)(a.kv + (size_t)b * a.Lk * DQK);
  const v4i* zsrc = (const v4i*)(a.ws_dzf + (size_t)row * nch * kBTiles * 64 * 8);
  constexpr int ZPER = (kBTiles * 64 + S::NT - 1) / S::NT;  // dZ pieces per thread
  ChunkRegs<S> cr;
  v4i zr[ZPER];
  auto load_z = [&](int c) {
#pragma unroll
    for (int j = 0; j < ZPER; ++j) {
      const int p = threadIdx.x + j * S::NT;
      if (p < kBTiles * 64) zr[j] = zsrc[(size_t)c * kBTiles * 64 + p];
    }
  };
  auto store_z = [&](int buf) {
#pragma unroll
    for (int j = 0; j < ZPER; ++j) {
      const int p = threadIdx.x + j * S::NT;
      if (p < kBTiles * 64) *(v4i*)(zbuf + buf * kBTiles * 1024 + 16 * p) = zr[j];
    }
  };
  cr.load(seq, sidx);
  load_z(0);
  cr.store(kvb);
  store_z(0);
  __syncthreads();

  v4f acc[S::DTQ][kBTiles];
#pragma unroll
  for (int j = 0; j < S::DTQ; ++j)
#pragma unroll
    for (int ht = 0; ht < kBTiles; ++ht) acc[j][ht] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const uint8_t* kb = kvb + buf * S::CHUNK_BYTES;
    if (c + 1 < nch) {
      cr.load(seq, sidx + (c + 1) * kBChunk);
      load_z(c + 1);
    }
    v8bf kt_[S::DTQ];
#pragma unroll
    for (int j = 0; j < S::DTQ; ++j) {
      const int t = wave + NW * j;
      const int tt = t < S::NDT ? t : 0;  // tiles past the width are not stored
      const int voff = v_base + bwd_piece<S>(r_v0, 2 * tt + v_sel);
      const v4s lo = lds_read_tr16(kb + voff);
      const v4s hi = lds_read_tr16(kb + voff + 16 * S::RS);
      kt_[j] = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
    }
#pragma unroll
    for (int ht = 0; ht < kBTiles; ++ht) {
      const v8bf zf = __builtin_bit_cast(v8bf, *(const v4i*)(zbuf + buf * kBTiles * 1024 + ht * 1024 + 16 * lane));
#pragma unroll
      for (int j = 0; j < S::DTQ; ++j) acc[j][ht] = mfma_bf16_16x16x32(kt_[j], zf, acc[j][ht]);
    }
    __syncthreads();
    if (c + 1 < nch) {
      cr.store(kvb + ((c + 1) & 1) * S::CHUNK_BYTES);
      store_z((c + 1) & 1);
      __syncthreads();
    }
  }

  // lane: d = 16t + 4g + r, head 16ht + li
#pragma unroll
  for (int j = 0; j < S::DTQ; ++j) {
    const int t = wave + NW * j;
    const int d0 = 16 * t + 4 * g;
    if (t >= S::NDT || d0 >= DQK) continue;
#pragma unroll
    for (int ht = 0; ht < kBTiles; ++ht) {
      const int head = 16 * ht + li;
      if (head < a.H) *(v4f*)(a.dq + ((size_t)row * a.H + head) * DQK + d0) = acc[j][ht] * a.scale;
    }
  }
}

// ---- 3. dkv[s] += scale * sum_h dZ[s,h] q[h] + sum_h P[s,h] dout[h]
// Block (row, slice of 64 columns); wave w owns d-tile 4 * slice + w.
template <int DQK, int DV>
__global__ __launch_bounds__(256) void attn_bwd_dkv_kernel(AttnBwdArgs a) {
  constexpr int DQKP = (DQK + 31) / 32 * 32;
  constexpr int NDT = DQKP / 16;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int nsl = (NDT + 3) / 4;
  const int row = blockIdx.x / nsl;
  const int t = 4 * (blockIdx.x % nsl) + wave;
  if (t >= NDT) return;  // wave-uniform; no barrier follows
  const int b = row / a.Lq;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  const size_t kpad = (size_t)nch * kBChunk;
  const int d = 16 * t + li;             // this lane's column (B operand and output)
  const bool d_ok = d < DQK, v_ok = d < DV;
  const bool any_v = 16 * t < DV;         // wave-uniform: the tile has value columns

  // B operands [heads 32 hs + 8g .. +7] x [column d], held for the whole row
  v8bf qb[4], gb[4];
#pragma unroll
  for (int hs = 0; hs < 4; ++hs) {
    uint32_t qw[4], gw[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float qv[2], gv[2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int head = 32 * hs + 8 * g + 2 * e + u;
        const bool ok = head < a.H;
        qv[u] = ok && d_ok ? bf16_bits_to_float(a.q[((size_t)row * a.H + head) * DQK + d]) : 0.0f;
        gv[u] = ok && v_ok ? a.dout[((size_t)row * a.H + head) * DV + d] : 0.0f;
      }
      qw[e] = pack_bf16x2(qv[0], qv[1]);
      gw[e] = pack_bf16x2(gv[0], gv[1]);
    }
    qb[hs] = __builtin_bit_cast(v8bf, (v4i){(int)qw[0], (int)qw[1], (int)qw[2], (int)qw[3]});
    gb[hs] = __builtin_bit_cast(v8bf, (v4i){(int)gw[0], (int)gw[1], (int)gw[2], (int)gw[3]});
  }

  const int32_t* idx_row = a.indices + (size_t)row * a.k;
  float* dkv_seq = a.dkv + (size_t)b * a.Lk * DQK;
  for (int c = 0; c < nch; ++c) {
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      // A operands: key 32c + 16kt + li, heads 32 hs + 8g .. +7
      const size_t abase = ((size_t)row * kpad + (size_t)c * kBChunk + 16 * kt + li) * kBHeads + 8 * g;
      v4f accz = {0.0f, 0.0f, 0.0f, 0.0f}, accp = accz;
#pragma unroll
      for (int hs = 0; hs < 4; ++hs) {
        const v8bf za = __builtin_bit_cast(v8bf, *(const v4i*)(a.ws_dzk + abase + 32 * hs));
        accz = mfma_bf16_16x16x32(za, qb[hs], accz);
        if (any_v) {
          const v8bf pa = __builtin_bit_cast(v8bf, *(const v4i*)(a.ws_pk + abase + 32 * hs));
          accp = mfma_bf16_16x16x32(pa, gb[hs], accp);
        }
      }
      // lane: keys 16kt + 4g + r, column d
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int slot = c * kBChunk + 16 * kt + 4 * g + r;
        const int s = slot < a.k ? idx_row[slot] : -1;
        if (d_ok && s >= 0 && s < a.Lk)
          unsafeAtomicAdd(dkv_seq + (size_t)s * DQK + d, a.scale * accz[r] + accp[r]);
      }
    }
  }
}

// Scores kernel: SPLIT blocks of NW1 waves per row; dq kernel: NW2 waves.
template <int DQK, int DV, int NW1, int SPLIT, int NW2>
hipError_t launch_bwd_shape(const AttnBwdArgs& a, hipStream_t stream) {
  using S1 = BwdShape<DQK, DV, NW1 * SPLIT>;
  using S2 = BwdShape<DQK, DV, NW2>;
  const int nch = (a.k + kBChunk - 1) / kBChunk;
  const size_t sidx_bytes = (size_t)nch * kBChunk * sizeof(int32_t);
  const size_t smem1 = 2 * (size_t)S1::CHUNK_BYTES + sidx_bytes;
  const size_t smem2 = 2 * (size_t)S2::CHUNK_BYTES + 2 * kBTiles * 1024 + sidx_bytes;
  static const hipError_t attr1 = hipFuncSetAttribute(
      (const void*)attn_bwd_scores_kernel<DQK, DV, NW1, SPLIT>, hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  static const hipError_t attr2 = hipFuncSetAttribute(
      (const void*)attn_bwd_dq_kernel<DQK, DV, NW2>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  if (attr1 != hipSuccess) return attr1;
  if (attr2 != hipSuccess) return attr2;
  const unsigned rows = (unsigned)((long long)a.B * a.Lq);
  hipError_t e = launch_kernel((const void*)attn_bwd_scores_kernel<DQK, DV, NW1, SPLIT>, dim3(rows * SPLIT),
                               dim3(64 * NW1), smem1, stream, a);
  if (e != hipSuccess) return e;
  e = launch_kernel((const void*)attn_bwd_dq_kernel<DQK, DV, NW2>, dim3(rows), dim3(64 * NW2), smem2, stream, a);
  if (e != hipSuccess) return e;
  const unsigned nsl = (unsigned)((S2::NDT + 3) / 4);
  return launch_kernel((const void*)attn_bwd_dkv_kernel<DQK, DV>, dim3(rows * nsl), dim3(256), 0, stream, a);
}

}  // namespace

size_t attn_bwd_workspace_bytes(int rows, int k) {
  const size_t kpad = (size_t)(k + kBChunk - 1) / kBChunk * kBChunk;
  // dZ in operand order + P and dZ key-major, bf16, 128 padded heads each
  return 3 * (size_t)rows * kpad * kBHeads * sizeof(uint16_t);
}

hipError_t launch_sparse_mla_attn_bwd(const AttnBwdArgs& a, hipStream_t stream) {
  if (a.Dv == 512 && a.Dr == 64) return launch_bwd_shape<576, 512, 4, 2, 8>(a, stream);
  if (a.Dv == 64 && a.Dr == 16) return launch_bwd_shape<80, 64, 4, 1, 4>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
