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
// Mapping.  One block per query row; wave w owns heads [16w, 16w+16).  The
// selected latent rows are gathered 32 at a time straight into LDS with
// global_load_lds (no register staging), double-buffered so the next chunk's
// gather overlaps this chunk's math.  Every wave reads the same chunk:
//   S^T[key, head] = K_chunk . Q^T   bf16 MFMA 16x16x32, Q^T held in registers
//   online softmax in fp32 (exp2 domain), P rounded to bf16
//   O^T[d, head]  += V^T . P^T       bf16 MFMA 16x16x32
// The MFMA result layout of S^T leaves each lane with one head and 8 keys,
// which is exactly a B operand of the value product once the 32 keys of the
// chunk are taken in the order (4g..4g+3, 16+4g..16+4g+3) for lane group g;
// the matching V^T operand comes from row-major LDS through the transposing
// ds_read_b64_tr_b16.  So P never leaves registers and the latent chunk is
// stored once, row-major, for both products.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kChunk = 32;

template <int DQK, int DV>
struct AttnShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;
  static constexpr int DT = DV / 16;
  static constexpr int RS = DQKP * 2;               // LDS bytes per latent row
  static constexpr int PPR = RS / 16;               // 16-byte pieces per LDS row
  static constexpr int RPR = DQK * 2 / 16;          // pieces present in the cache row
  static constexpr int CHUNK_BYTES = kChunk * RS;
  static constexpr int DMA_BLOCKS = CHUNK_BYTES / 1024;  // 64 lanes x 16 bytes
  static_assert(CHUNK_BYTES % 1024 == 0, "chunk must be whole 1 KiB DMA blocks");
  static_assert(DQK % 8 == 0 && DV % 16 == 0 && DV <= DQK, "unsupported latent shape");
};

template <int DQK, int DV>
__global__ __launch_bounds__(512) void sparse_mla_kernel(AttnArgs a) {
  using S = AttnShape<DQK, DV>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint8_t* bufs = smem;                                           // [2][CHUNK_BYTES]
  int32_t* sidx = (int32_t*)(smem + 2 * S::CHUNK_BYTES);          // [nch * kChunk]

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nwaves = blockDim.x >> 6;
  const int g = lane >> 4;
  const int li = lane & 15;
  const int row = blockIdx.x;
  const int b = row / a.Lq;
  const int nch = (a.k + kChunk - 1) / kChunk;

  // ---- selected indices -> LDS; chunk validity mask (k <= 2048 -> nch <= 64)
  const int32_t* idx_row = a.indices + (size_t)row * a.k;
  for (int i = threadIdx.x; i < nch * kChunk; i += blockDim.x) {
    int v = i < a.k ? idx_row[i] : -1;
    sidx[i] = (v >= 0 && v < a.Lk) ? v : -1;
  }
  __syncthreads();
  uint64_t chunk_mask = 0;
  {
    bool any = false;
    if (lane < nch) {
      for (int j = 0; j < kChunk; ++j) any |= sidx[lane * kChunk + j] >= 0;
    }
    chunk_mask = __ballot(any);
  }

  // ---- Q^T fragments of this wave's 16 heads (B operand of the score product)
  const int head = 16 * wave + li;
  const bool head_ok = head < a.H;
  v8bf qf[S::KST];
  {
    const uint16_t* qrow = a.q + ((size_t)row * a.H + (head_ok ? head : 0)) * DQK;
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      v4i v = {0, 0, 0, 0};
      if (head_ok && d0 + 8 <= DQK) v = *(const v4i*)(qrow + d0);
      qf[ks] = __builtin_bit_cast(v8bf, v);
    }
  }

  const uint8_t* kv_seq = (const uint8_t*)(a.kv + (size_t)b * a.Lk * DQK);
  auto gather = [&](int c, int buf) {
    uint8_t* dst = bufs + buf * S::CHUNK_BYTES;
    for (int j = wave; j < S::DMA_BLOCKS; j += nwaves) {
      const int p = 64 * j + lane;
      const int r = p / S::PPR, col = p % S::PPR;
      const int idx = sidx[c * kChunk + r];
      const int src_row = idx >= 0 ? idx : 0;
      const int src_col = col < S::RPR ? col : col - S::RPR;  // pad pieces meet zero q
      const uint8_t* src = kv_seq + (size_t)src_row * (DQK * 2) + 16 * src_col;
      __builtin_amdgcn_global_load_lds((const void*)src,
                                       (__attribute__((address_space(3))) void*)(dst + 1024 * j),
                                       16, 0, 0);
    }
  };

  v4f acc[S::DT];
#pragma unroll
  for (int dt = 0; dt < S::DT; ++dt) acc[dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY;
  float l_part = 0.0f;

  uint64_t pending = chunk_mask;
  int cur = pending ? __builtin_ctzll(pending) : -1;
  if (cur >= 0) {
    pending &= pending - 1;
    gather(cur, 0);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  int buf = 0;
  while (cur >= 0) {
    const int nxt = pending ? __builtin_ctzll(pending) : -1;
    if (nxt >= 0) {
      pending &= pending - 1;
      gather(nxt, buf ^ 1);
    }
    const uint8_t* kb = bufs + buf * S::CHUNK_BYTES;

    // ---- S^T = K_chunk . Q^T  (two 16-key tiles)
    v4f s[2] = {{0.0f, 0.0f, 0.0f, 0.0f}, {0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const v4i raw = *(const v4i*)(kb + (16 * kt + li) * S::RS + (32 * ks + 8 * g) * 2);
        s[kt] = mfma_bf16_16x16x32(__builtin_bit_cast(v8bf, raw), qf[ks], s[kt]);
      }
    }

    // ---- online softmax for this lane's head over its 8 keys
    const v4i id0 = *(const v4i*)(sidx + cur * kChunk + 4 * g);
    const v4i id1 = *(const v4i*)(sidx + cur * kChunk + 16 + 4 * g);
    float z[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      z[r] = id0[r] >= 0 ? s[0][r] * a.scale_log2 : -INFINITY;
      z[4 + r] = id1[r] >= 0 ? s[1][r] * a.scale_log2 : -INFINITY;
    }
    float mloc = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mloc = fmaxf(mloc, z[i]);
    mloc = fmaxf(mloc, __shfl_xor(mloc, 16));
    mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
    const float m_new = fmaxf(m_run, mloc);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    uint32_t pk[4];
    float psum = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t lo = float_to_bf16_bits(fast_exp2(z[2 * i] - m_new));
      const uint32_t hi = float_to_bf16_bits(fast_exp2(z[2 * i + 1] - m_new));
      psum += bf16_bits_to_float(lo) + bf16_bits_to_float(hi);
      pk[i] = lo | (hi << 16);
    }
    l_part = l_part * alpha + psum;
    const v8bf pb = __builtin_bit_cast(v8bf, (v4i){(int)pk[0], (int)pk[1], (int)pk[2], (int)pk[3]});

    // ---- O^T = alpha * O^T + V^T . P^T
    const uint8_t* vrow0 = kb + (4 * g + (li >> 2)) * S::RS + 4 * (li & 3) * 2;
    const uint8_t* vrow1 = vrow0 + 16 * S::RS;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      const v4s lo = lds_read_tr16(vrow0 + 32 * dt);
      const v4s hi = lds_read_tr16(vrow1 + 32 * dt);
      const v8bf va = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
      acc[dt] = mfma_bf16_16x16x32(va, pb, acc[dt] * alpha);
    }

    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    cur = nxt;
    buf ^= 1;
  }

  // ---- normalise and store
  float l_tot = l_part + __shfl_xor(l_part, 16);
  l_tot += __shfl_xor(l_tot, 32);
  if (head_ok) {
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
    float* orow = a.out + ((size_t)row * a.H + head) * DV;
#pragma unroll
    for (int dt = 0; dt < S::DT; ++dt) {
      const v4f o = acc[dt] * inv;
      *(v4f*)(orow + 16 * dt + 4 * g) = o;
    }
    if (a.lse && g == 0)
      a.lse[(size_t)row * a.H + head] =
          l_tot > 0.0f ? (m_run + fast_log2(l_tot)) * 0.69314718055994530942f : -INFINITY;
  }
}

template <int DQK, int DV>
hipError_t launch_shape(const AttnArgs& a, hipStream_t stream) {
  using S = AttnShape<DQK, DV>;
  const int nch = (a.k + kChunk - 1) / kChunk;
  const size_t smem = 2 * (size_t)S::CHUNK_BYTES + (size_t)nch * kChunk * sizeof(int32_t);
  const int nwaves = (a.H + 15) / 16;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)sparse_mla_kernel<DQK, DV>, hipFuncAttributeMaxDynamicSharedMemorySize,
      160 * 1024);
  if (attr != hipSuccess) return attr;
  return launch_kernel((const void*)sparse_mla_kernel<DQK, DV>,
                       dim3((unsigned)((long long)a.B * a.Lq)), dim3(64 * nwaves), smem, stream, a);
}

}  // namespace

hipError_t launch_sparse_mla_attn(const AttnArgs& a, hipStream_t stream) {
  if (a.Dv == 512 && a.Dr == 64) return launch_shape<576, 512>(a, stream);
  if (a.Dv == 64 && a.Dr == 16) return launch_shape<80, 64>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace dsa
