// Dense warm-up objective of the indexer (gfx950): only the indexer is
// trained, so that its softmax over a query's scores matches the main
// attention's distribution summed over the heads, under a KL loss
// (DeepSeek-V3.2 spec sheet, design overview and the curriculum row of its
// training table; lightning-indexer post, training section).
//
// Readings: the main attention is dense over s <= pos(t); the summed
// distribution is divided by the head count, p[t,s] = (1/H) sum_h
// softmax_s(z[t,h,s]) with z = scale * q . kv; a row's loss is
// KL(p_t || softmax(I_t)) and its gradient with respect to the scores is
// softmax(I_t) - p_t.
//
// Kernels:
//  1. target (one block of 8 waves per two adjacent rows, 32 heads per
//     wave): the rows' causal keys stream through LDS in chunks of 32
//     contiguous latent rows; S = Q.K^T runs on bf16 MFMA with Q in
//     registers, so a lane holds 4 heads of one key.  A caller that has each
//     head's lse (the dense forward computes it) can pass it and skip pass 1.  Pass 1 keeps a running max and sum per lane and head
//     and merges them over the 16 key lanes into the head's lse; pass 2
//     recomputes S and sums exp(z - lse) over the heads (in lane, across the
//     4 lane rows, then across the waves through LDS) into the target row.
//  2. KL (one block per row, HBM-bound): online max / sum of the scores for
//     log Z, then the loss and dI = exp(I - log Z) - p in one more read.
#include <algorithm>

#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kWChunk = 32;  // keys per chunk
constexpr int kWWaves = 8;   // 2 rows x 4 waves x 32 heads

template <int DQK>
struct WShape {
  static constexpr int DQKP = (DQK + 31) / 32 * 32;  // score width padded to K=32 steps
  static constexpr int KST = DQKP / 32;
  static constexpr int RS = DQKP * 2;                // LDS bytes per key row
  static constexpr int PPR = RS / 16;                // 16-byte pieces per LDS row
  static constexpr int RPR = DQK * 2 / 16;           // pieces present in the cache row
  static constexpr bool SWZ = PPR % 8 == 0;
  static constexpr int CHUNK_BYTES = kWChunk * RS;
  static constexpr int BLOCKS = CHUNK_BYTES / 1024;  // 1 KB copies per chunk
  static_assert(CHUNK_BYTES % 1024 == 0 && DQK % 8 == 0, "unsupported latent shape");
};

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Keys s0 .. s0+31 (clamped to n - 1) of one sequence's cache -> LDS row r
// at `dst`; piece lp of row r sits at physical piece lp ^ (r & 7) when the
// row has a multiple of 8 pieces (conflict-free fragment reads).  Pad pieces
// past the cache row re-read real ones (they meet zero q).  Each copy moves
// 1 KB (lane i: bytes 16i..16i+15 of the block); waited for by the caller.
template <typename S>
__device__ __forceinline__ void load_chunk(uint8_t* dst, const uint8_t* seq, int s0, int n, int wave, int lane) {
#pragma unroll
  for (int j = 0; j < (S::BLOCKS + kWWaves - 1) / kWWaves; ++j) {
    const int blk = wave + kWWaves * j;
    if (blk < S::BLOCKS) {
      const int p = 64 * blk + lane;
      const int r = p / S::PPR, pp = p % S::PPR;
      const int lp = S::SWZ ? (pp ^ (r & 7)) : pp;
      const int col = lp < S::RPR ? lp : lp - S::RPR;
      const int key = min(s0 + r, n - 1);
      const uint32_t off = (uint32_t)key * (uint32_t)(S::RPR * 16) + 16u * (uint32_t)col;
      const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_addr(dst + 1024 * blk));
      asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %2"
                   :: "v"(off), "s"(m0), "s"(seq) : "memory", "m0");
    }
  }
}

// 16-lane (one MFMA lane row) exchanges
__device__ __forceinline__ float xor_lanes(float v, int m) { return __shfl_xor(v, m, 64); }

// Two adjacent query rows per block (their causal ranges differ by one key):
// waves 0-3 take row t0, waves 4-7 row t0 + 1, each wave 32 heads (2 tiles),
// so every K fragment read from LDS feeds two MFMAs.
constexpr int kWRows = 2;
constexpr int kWHt = 2;  // 16-head tiles per wave

template <int DQK>
__global__ __launch_bounds__(64 * kWWaves) void warmup_target_kernel(WarmupArgs a) {
  using S = WShape<DQK>;
  constexpr int WPR = kWWaves / kWRows;  // waves per row
  __shared__ __attribute__((aligned(16))) uint8_t kbuf[2][S::CHUNK_BYTES];
  __shared__ float red[2][kWWaves][kWChunk];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int rr = wave / WPR, hg = wave % WPR;

  // longest row pairs first (their blocks start earliest); pairs go to the
  // XCDs in runs of 32 consecutive pairs, which stream the same keys
  const int pairs = (a.Lq + kWRows - 1) / kWRows;
  const int nb = (int)gridDim.x;
  constexpr int kRun = 32;
  const int full = nb / (8 * kRun) * (8 * kRun);
  const int xi = (int)blockIdx.x >> 3;
  const int lin = (int)blockIdx.x < full ? ((xi / kRun) * 8 + (int)(blockIdx.x & 7)) * kRun + xi % kRun
                                         : (int)blockIdx.x;
  const int bq = lin % a.B, t0 = kWRows * (pairs - 1 - lin / a.B);  // batches interleaved, late pairs first
  const int t = t0 + rr;
  const bool row_ok = t < a.Lq;  // wave-uniform
  const size_t row = (size_t)bq * a.Lq + (row_ok ? t : t0);
  const int n = min(a.q_start + t + 1, a.Lk);                          // this wave's keys 0 .. n-1
  const int n_max = min(a.q_start + min(t0 + kWRows, a.Lq), a.Lk);     // the block's longest row
  const int nch = (n_max + kWChunk - 1) / kWChunk;
  const uint8_t* seq = (const uint8_t*)(a.kv + (size_t)bq * a.Lk * DQK);

  // B operands: head 32 hg + 16 ht + li, dims 32 ks + 8g .. +7 (zero past DQK or H)
  v8bf qf[kWHt][S::KST];
  bool hv[kWHt][4];  // this lane's heads 32 hg + 16 ht + 4g + r present
#pragma unroll
  for (int ht = 0; ht < kWHt; ++ht) {
    const int head = 32 * hg + 16 * ht + li;
    const bool ok = row_ok && head < a.H;
    const uint16_t* qrow = a.q + (row * a.H + min(head, a.H - 1)) * DQK;
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      const int d0 = 32 * ks + 8 * g;
      v4i v = {0, 0, 0, 0};
      if (d0 < DQK && ok) v = *(const v4i*)(qrow + d0);
      qf[ht][ks] = __builtin_bit_cast(v8bf, v);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) hv[ht][r] = row_ok && 32 * hg + 16 * ht + 4 * g + r < a.H;
  }

  // S tiles of chunk c: acc[ht][kt][r] = q[head 16ht + 4g + r] . kv[key 32c + 16kt + li]
  auto scores = [&](int st, v4f (&acc)[kWHt][2]) {
#pragma unroll
    for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) acc[ht][kt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    // k-steps outermost: the four accumulators take turns, so a product
    // never waits on the one just issued
#pragma unroll
    for (int ks = 0; ks < S::KST; ++ks) {
      const int lp = 4 * ks + g;
      v8bf kf[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int kr = 16 * kt + li;
        kf[kt] = __builtin_bit_cast(v8bf, *(const v4i*)(&kbuf[st][kr * S::RS] + 16 * (S::SWZ ? (lp ^ (kr & 7)) : lp)));
      }
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int ht = 0; ht < kWHt; ++ht) acc[ht][kt] = mfma_bf16_16x16x32(qf[ht][ks], kf[kt], acc[ht][kt]);
    }
  };

  float lse2[kWHt][4];
  if (a.lse_in) {  // block-uniform: the caller has each head's lse (natural log)
#pragma unroll
    for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int head = 32 * hg + 16 * ht + 4 * g + r;
        lse2[ht][r] = hv[ht][r] ? a.lse_in[row * a.H + head] * 1.44269504088896340736f : 0.0f;
      }
  } else {
  // ---- pass 1: lse of every head over keys 0 .. n-1 (base 2)
  float m[kWHt][4], l[kWHt][4];
#pragma unroll
  for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) m[ht][r] = -INFINITY, l[ht][r] = 0.0f;
  load_chunk<S>(kbuf[0], seq, 0, n_max, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int st = c & 1;
    if (c + 1 < nch) load_chunk<S>(kbuf[st ^ 1], seq, kWChunk * (c + 1), n_max, wave, lane);
    v4f acc[kWHt][2];
    scores(st, acc);
    const bool ok0 = kWChunk * c + li < n, ok1 = kWChunk * c + 16 + li < n;
#pragma unroll
    for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float x0 = ok0 ? acc[ht][0][r] * a.scale_log2 : -INFINITY;
        const float x1 = ok1 ? acc[ht][1][r] * a.scale_log2 : -INFINITY;
        const float mn = fmaxf(m[ht][r], fmaxf(x0, x1));
        const float ms = mn == -INFINITY ? 0.0f : mn;  // nothing seen yet: every term is 0
        l[ht][r] = l[ht][r] * fast_exp2(m[ht][r] - ms) + fast_exp2(x0 - ms) + fast_exp2(x1 - ms);
        m[ht][r] = mn;
      }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  }
#pragma unroll
  for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float mm = m[ht][r], ll = l[ht][r];
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) {
        const float mo = xor_lanes(mm, o), lo = xor_lanes(ll, o);
        const float mn = fmaxf(mm, mo);
        const float ms = mn == -INFINITY ? 0.0f : mn;
        ll = ll * fast_exp2(mm - ms) + lo * fast_exp2(mo - ms);
        mm = mn;
      }
      lse2[ht][r] = mm + fast_log2(ll);  // key 0 is always present: finite for every present head
      if (a.lse_out && li == 0 && hv[ht][r])
        a.lse_out[row * a.H + 32 * hg + 16 * ht + 4 * g + r] = lse2[ht][r] * 0.69314718055994530942f;
    }
  }

  // ---- pass 2: target[row, s] = (1/H) sum_h exp2(z * log2e - lse2[h])
  load_chunk<S>(kbuf[0], seq, 0, n_max, wave, lane);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    const int st = c & 1;
    if (c + 1 < nch) load_chunk<S>(kbuf[st ^ 1], seq, kWChunk * (c + 1), n_max, wave, lane);
    v4f acc[kWHt][2];
    scores(st, acc);
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      float s = 0.0f;
#pragma unroll
      for (int ht = 0; ht < kWHt; ++ht)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          s += hv[ht][r] ? fast_exp2(fmaf(acc[ht][kt][r], a.scale_log2, -lse2[ht][r])) : 0.0f;
      s += xor_lanes(s, 16);
      s += xor_lanes(s, 32);
      if (g == 0) red[st][wave][16 * kt + li] = s;
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x < kWRows * kWChunk) {
      const int r2 = threadIdx.x / kWChunk, kk = threadIdx.x % kWChunk;
      const int tt = t0 + r2;
      const int key = kWChunk * c + kk;
      if (tt < a.Lq && key < min(a.q_start + tt + 1, a.Lk)) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < WPR; ++w) v += red[st][r2 * WPR + w][kk];
        a.target[((size_t)bq * a.Lq + tt) * a.Lk + key] = v * a.inv_heads;
      }
    }
  }
}

// ---- KL of a row and its score gradient
template <int NT>
__device__ __forceinline__ void block_max_sum(float& m, float& l, float* sm, float* sl) {
  // merge (max, sum of exp(x - max)) pairs over the block (natural exp)
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const float mo = __shfl_xor(m, o, 64), lo = __shfl_xor(l, o, 64);
    const float mn = fmaxf(m, mo);
    const float ms = mn == -INFINITY ? 0.0f : mn;
    l = l * __expf(m - ms) + lo * __expf(mo - ms);
    m = mn;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) sm[wave] = m, sl[wave] = l;
  __syncthreads();
  m = -INFINITY;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) m = fmaxf(m, sm[w]);
  const float ms = m == -INFINITY ? 0.0f : m;
  l = 0.0f;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) l += sl[w] * __expf(sm[w] - ms);
  __syncthreads();
}

constexpr int kKlThreads = 256;

__global__ __launch_bounds__(kKlThreads) void warmup_kl_kernel(WarmupArgs a) {
  __shared__ float sm[kKlThreads / 64], sl[kKlThreads / 64];
  __shared__ double sd[kKlThreads / 64];
  const int row = blockIdx.x;
  const int t = row % a.Lq;
  const int n = min(a.q_start + t + 1, a.Lk);
  const float* I = a.scores + (size_t)row * a.Lk;
  const float* P = a.target + (size_t)row * a.Lk;
  float* D = a.dscores + (size_t)row * a.Lk;
  // online max / sum over the row (4 entries per thread per step where aligned)
  float m = -INFINITY, l = 0.0f;
  for (int s = threadIdx.x; s < n; s += kKlThreads) {
    const float x = I[s];
    const float mn = fmaxf(m, x);
    l = l * __expf(m - mn) + __expf(x - mn);
    m = mn;
  }
  block_max_sum<kKlThreads>(m, l, sm, sl);
  const float logz = m + __logf(l);
  double loss = 0.0;
  for (int s = threadIdx.x; s < n; s += kKlThreads) {
    const float lp = I[s] - logz;  // log softmax
    const float p = P[s];
    if (p > 0.0f) loss += (double)p * ((double)__logf(p) - (double)lp);
    D[s] = __expf(lp) - p;  // the same thread read I[s] above: in place is safe
  }
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) loss += __shfl_xor(loss, o, 64);
  if ((threadIdx.x & 63) == 0) sd[threadIdx.x >> 6] = loss;
  __syncthreads();
  if (threadIdx.x == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < kKlThreads / 64; ++w) tot += sd[w];
    a.loss[row] = (float)tot;
  }
}

}  // namespace

hipError_t launch_warmup_target(const WarmupArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)a.B * ((a.Lq + kWRows - 1) / kWRows))), block(64 * kWWaves);
  if (a.Dv == 512 && a.Dr == 64) return launch_kernel((const void*)warmup_target_kernel<576>, grid, block, 0, stream, a);
  if (a.Dv == 64 && a.Dr == 16) return launch_kernel((const void*)warmup_target_kernel<80>, grid, block, 0, stream, a);
  return hipErrorInvalidValue;
}

hipError_t launch_warmup_kl(const WarmupArgs& a, hipStream_t stream) {
  return launch_kernel((const void*)warmup_kl_kernel, dim3((unsigned)((long long)a.B * a.Lq)), dim3(kKlThreads), 0,
                       stream, a);
}

}  // namespace dsa
