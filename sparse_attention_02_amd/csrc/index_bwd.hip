// Gradients of the lightning indexer's scores with respect to its inputs
// (gfx950), for the indexer's training in the dense warm-up (DeepSeek-V3.2
// spec sheet, design overview and the curriculum row of its training table;
// lightning-indexer post, training section).  With I[t,s] = sum_j w[t,j]
// ReLU(u[t,j,s]), u = q_I[t,j] . k_I[s], and a gradient dI of the scores
// (entries s <= pos(t)), the ReLU's derivative taken as 0 at 0:
//   c[t,j,s] = dI[t,s] w[t,j] [u > 0]
//   dw[t,j]  = sum_s dI[t,s] ReLU(u[t,j,s])
//   dq_I[t,j] = sum_s c[t,j,s] k_I[s],   dk_I[s] = sum_(t,j) c[t,j,s] q_I[t,j].
//
// Every e4m3 value is exact in bf16, so u is recomputed on bf16 MFMA with
// fp32 accumulation (exact whenever the fp32 sum is, as on the input grids);
// c is rounded to bf16 for the two products.  Two kernels:
//  1. query-stationary (block = 4 query rows x 64 heads, 8 waves of one row
//     and 32 heads): key tiles of 32 are staged in LDS as bf16, key-major;
//     u^T = K.Q^T reads them directly and dq^T = K^T.c^T through the
//     transposing LDS reads; a lane's 8 keys of a c^T fragment are the 8 keys
//     the u^T tile left in it, so the transposing reads take the same order.
//  2. key-stationary (block = 256 keys in registers, 32 per wave, x a range of
//     query rows): each row's q_I is staged as bf16 head-major, read directly
//     for u = Q.K^T and through the transposing reads for dk^T = Q^T.c, and
//     the block's partial dk_I goes to memory with one fp32 atomic add per
//     element at the end.
// (A second, d-major copy of each staged tile written with 2-byte stores
// took the transposed operands before: 69 ms at the 32K prefill against 54.)
#include <algorithm>

#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

// 8 e4m3fn bytes (two words) -> 8 bf16 as 4 packed words, exactly: the
// hardware converts two bytes at a time to fp32 (gfx950's FP8 conversions
// use the OCP e4m3fn format), and every e4m3 value has at most 4 significant
// bits, so its bf16 is the upper half of that fp32.
__device__ __forceinline__ v4i e4m3x8_to_bf16(uint32_t lo, uint32_t hi) {
  v4i r;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const uint32_t x = i ? hi : lo;
    const v2f f0 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, false);  // bytes 0, 1
    const v2f f1 = __builtin_amdgcn_cvt_pk_f32_fp8((int)x, true);   // bytes 2, 3
    r[2 * i] = (int)((__float_as_uint(f0.x) >> 16) | (__float_as_uint(f0.y) & 0xFFFF0000u));
    r[2 * i + 1] = (int)((__float_as_uint(f1.x) >> 16) | (__float_as_uint(f1.y) & 0xFFFF0000u));
  }
  return r;
}

constexpr int kQRows = 4;     // query rows per block of kernel 1
constexpr int kKeysPerBlock = 256;

// piece p (8 dims) of row k of a key-major / head-major bf16 tile with NP
// pieces per row: XOR-swizzled when NP is a power of two
template <int NP>
__device__ __forceinline__ int swz(int p, int k) {
  return (NP & (NP - 1)) == 0 ? (p ^ (k & (NP - 1))) : p;
}

// ---- 1. dq_I and dw
template <int DI>
__global__ __launch_bounds__(512) void index_bwd_q_kernel(IndexBwdArgs a) {
  constexpr int KST = DI / 32, NDT = DI / 16, NP = DI / 8;
  __shared__ __attribute__((aligned(16))) uint16_t kb[2][32 * DI];      // [key][d] (swizzled pieces)
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int qb = (a.Lq + kQRows - 1) / kQRows;
  const int b = blockIdx.x / qb, t0 = kQRows * (blockIdx.x % qb);
  const int rr = wave >> 1, hh = wave & 1;
  const int t = t0 + rr;
  const bool row_ok = t < a.Lq;  // wave-uniform
  const size_t row = (size_t)b * a.Lq + (row_ok ? t : 0);
  const int n_r = min(a.q_start + t + 1, a.Lk);
  const int n_max = min(a.q_start + min(t0 + kQRows, a.Lq), a.Lk);  // keys of the block's last row
  const int ntile = (n_max + 31) / 32;
  const uint8_t* kseq = a.k_idx + (size_t)b * a.Lk * DI;

  // B operands Q^T: head 32hh + 16ht + li, dims 32ks + 8g .. +7
  v8bf qf[2][KST];
  float wh[2];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = 32 * hh + 16 * ht + li;
    const bool ok = row_ok && head < a.H;
    const uint8_t* qp = a.q_idx + (row * a.H + (ok ? head : 0)) * DI;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const uint2 raw = ok ? *(const uint2*)(qp + 32 * ks + 8 * g) : make_uint2(0u, 0u);
      qf[ht][ks] = __builtin_bit_cast(v8bf, e4m3x8_to_bf16(raw.x, raw.y));
    }
    wh[ht] = ok ? a.w[row * a.H + head] : 0.0f;
  }

  // staging: thread -> key k, piece p (8 dims) of the 32 x DI byte tile
  const bool stager = tid < 4 * DI;
  const int sk = tid / NP, sp = tid % NP;
  auto fetch = [&](int c) -> uint2 {
    const int key = min(32 * c + sk, n_max - 1);
    return stager ? *(const uint2*)(kseq + (size_t)key * DI + 8 * sp) : make_uint2(0u, 0u);
  };
  auto stage = [&](int st, uint2 raw) {
    if (!stager) return;
    const v4i v = e4m3x8_to_bf16(raw.x, raw.y);
    *(v4i*)&kb[st][sk * DI + 8 * swz<NP>(sp, sk)] = v;
  };
  // K^T fragments through the transposing reads: group g's lanes address key
  // rows 4g + li/4 (and 16 + 4g + li/4), 4 dims each at d = 16dt + 4(li&3),
  // so lane li receives d = 16dt + li for the keys 4g..4g+3 (16 + ..): the
  // k-slots 8g..8g+7 in the key order of the c^T fragment
  const int tr_key = 4 * g + (li >> 2);
  const int tr_sel = (li & 3) >> 1, tr_half = 8 * (li & 1);

  v4f acc[2][NDT];
#pragma unroll
  for (int ht = 0; ht < 2; ++ht)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[ht][dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  float dwa[2] = {0.0f, 0.0f};
  const float* drow = a.dscores + row * a.Lk;

  stage(0, fetch(0));
  __syncthreads();
  for (int c = 0; c < ntile; ++c) {
    const int st = c & 1;
    uint2 nxt = make_uint2(0u, 0u);
    if (c + 1 < ntile) nxt = fetch(c + 1);
    if (row_ok && 32 * c < n_r) {
      // u^T tiles: lane holds key 16kt + 4g + r, head 16ht + li
      v4f u[2][2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int k = 16 * kt + li;
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) u[kt][ht] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int ks = 0; ks < KST; ++ks) {
          const v8bf kf = __builtin_bit_cast(v8bf, *(const v4i*)&kb[st][k * DI + 8 * swz<NP>(4 * ks + g, k)]);
#pragma unroll
          for (int ht = 0; ht < 2; ++ht) u[kt][ht] = mfma_bf16_16x16x32(kf, qf[ht][ks], u[kt][ht]);
        }
      }
      float dv[2][4];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int s = 32 * c + 16 * kt + 4 * g + r;
          dv[kt][r] = s < n_r ? drow[s] : 0.0f;
        }
      // c^T as the B operand: k-slots 8g..8g+7 <-> keys 4g..4g+3, 16+4g..16+4g+3
      v8bf cb[2];
#pragma unroll
      for (int ht = 0; ht < 2; ++ht) {
        float cv[8];
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float x = u[kt][ht][r];
            cv[4 * kt + r] = x > 0.0f ? dv[kt][r] * wh[ht] : 0.0f;
            dwa[ht] = fmaf(dv[kt][r], fmaxf(x, 0.0f), dwa[ht]);
          }
        cb[ht] = __builtin_bit_cast(v8bf, (v4i){(int)pack_bf16x2(cv[0], cv[1]), (int)pack_bf16x2(cv[2], cv[3]),
                                                 (int)pack_bf16x2(cv[4], cv[5]), (int)pack_bf16x2(cv[6], cv[7])});
      }
      // dq^T += K^T . c^T: A lane (d = 16dt + li) holds the same 8 keys
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int pc = swz<NP>(2 * dt + tr_sel, tr_key);  // same for rows tr_key and tr_key + 16
        const uint8_t* kr = (const uint8_t*)&kb[st][tr_key * DI] + 16 * pc + tr_half;
        const v4s lo = lds_read_tr16(kr);
        const v4s hi = lds_read_tr16(kr + 16 * DI * 2);
        const v8bf ka = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
        for (int ht = 0; ht < 2; ++ht) acc[ht][dt] = mfma_bf16_16x16x32(ka, cb[ht], acc[ht][dt]);
      }
    }
    if (c + 1 < ntile) stage(st ^ 1, nxt);
    __syncthreads();
  }

  if (!row_ok) return;
#pragma unroll
  for (int ht = 0; ht < 2; ++ht) {
    const int head = 32 * hh + 16 * ht + li;
    float s = dwa[ht];
    s += __shfl_xor(s, 16, 64);
    s += __shfl_xor(s, 32, 64);
    if (head < a.H) {
      if (g == 0) a.dw[row * a.H + head] = s;
      float* dq = a.dq_idx + (row * a.H + head) * DI;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) *(v4f*)(dq + 16 * dt + 4 * g) = acc[ht][dt];
    }
  }
}

// ---- 2. dk_I (accumulated)
template <int DI>
__global__ __launch_bounds__(512) void index_bwd_k_kernel(IndexBwdArgs a, int rows_per_block) {
  constexpr int KST = DI / 32, NDT = DI / 16, NP = DI / 8, NP16 = DI / 16;
  __shared__ __attribute__((aligned(16))) uint16_t qa[2][64 * DI];     // [head][d] (swizzled pieces)
  __shared__ float ws[2][64];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 4, li = lane & 15;
  const int nkb = (a.Lk + kKeysPerBlock - 1) / kKeysPerBlock;
  const int nsp = (a.Lq + rows_per_block - 1) / rows_per_block;
  const int per_b = nkb * nsp;
  const int b = blockIdx.x / per_b;
  const int kbi = (blockIdx.x % per_b) / nsp, spi = blockIdx.x % nsp;
  const int s_base = kKeysPerBlock * kbi;
  // rows whose causal range reaches this block's first key
  const int t_lo = max(spi * rows_per_block, s_base - a.q_start);
  const int t_hi = min((spi + 1) * rows_per_block, a.Lq);
  if (t_lo >= t_hi) return;  // block-uniform, before any barrier

  // B operands K^T: key s_base + 32 wave + 16kt + li, dims 32ks + 8g .. +7
  v8bf kf[2][KST];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = s_base + 32 * wave + 16 * kt + li;
    const bool ok = key < a.Lk;
    const uint8_t* kp = a.k_idx + ((size_t)b * a.Lk + (ok ? key : 0)) * DI;
#pragma unroll
    for (int ks = 0; ks < KST; ++ks) {
      const uint2 raw = ok ? *(const uint2*)(kp + 32 * ks + 8 * g) : make_uint2(0u, 0u);
      kf[kt][ks] = __builtin_bit_cast(v8bf, e4m3x8_to_bf16(raw.x, raw.y));
    }
  }

  // staging of row t: thread -> head h, 16-dim piece p of the 64 x DI tile
  const bool stager = tid < 4 * DI;
  const int sh = tid / NP16, sq = tid % NP16;
  auto fetch = [&](int t) -> uint4 {
    const size_t row = (size_t)b * a.Lq + t;
    return stager && sh < a.H ? *(const uint4*)(a.q_idx + (row * a.H + sh) * DI + 16 * sq) : make_uint4(0u, 0u, 0u, 0u);
  };
  auto fetch_w = [&](int t) -> float {
    const size_t row = (size_t)b * a.Lq + t;
    return tid < 64 && tid < a.H ? a.w[row * a.H + tid] : 0.0f;
  };
  auto stage = [&](int st, uint4 raw, float wv) {
    if (tid < 64) ws[st][tid] = wv;
    if (!stager) return;
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      const v4i v = e4m3x8_to_bf16(hf ? raw.z : raw.x, hf ? raw.w : raw.y);
      const int p = 2 * sq + hf;
      *(v4i*)&qa[st][sh * DI + 8 * swz<NP>(p, sh)] = v;
    }
  };
  // Q^T fragments through the transposing reads: group g's lanes address head
  // rows 32hs + 4g + li/4 (and + 16), 4 dims each at d = 16dt + 4(li&3), so
  // lane li receives d = 16dt + li for the k-slots 8g..8g+7 of the c fragment
  const int tr_head = 4 * g + (li >> 2);
  const int tr_sel = (li & 3) >> 1, tr_half = 8 * (li & 1);

  v4f acc[2][NDT];
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) acc[kt][dt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
  const int key0 = s_base + 32 * wave + li;

  stage(0, fetch(t_lo), fetch_w(t_lo));
  __syncthreads();
  for (int t = t_lo; t < t_hi; ++t) {
    const int st = (t - t_lo) & 1;
    uint4 nxt = make_uint4(0u, 0u, 0u, 0u);
    float nw = 0.0f;
    if (t + 1 < t_hi) nxt = fetch(t + 1), nw = fetch_w(t + 1);
    const int pos = a.q_start + t;
    if (s_base + 32 * wave <= pos) {  // wave-uniform: some key of the wave is in range
      const float* drow = a.dscores + ((size_t)b * a.Lq + t) * a.Lk;
      float dv[2];
#pragma unroll
      for (int kt = 0; kt < 2; ++kt) {
        const int key = key0 + 16 * kt;
        dv[kt] = key <= pos && key < a.Lk ? drow[key] : 0.0f;
      }
      // u tiles: lane holds head 16ht + 4g + r, key 16kt + li
      v8bf cb[2][2];  // [head half hs][kt]: k-slots 8g.. <-> heads 32hs + 4g + r, 32hs + 16 + 4g + r
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        float cv[2][8];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int ht = 2 * hs + h2;
          const int hr = 16 * ht + li;
          v4f u[2] = {(v4f){0.0f, 0.0f, 0.0f, 0.0f}, (v4f){0.0f, 0.0f, 0.0f, 0.0f}};
#pragma unroll
          for (int ks = 0; ks < KST; ++ks) {
            const v8bf qf = __builtin_bit_cast(v8bf, *(const v4i*)&qa[st][hr * DI + 8 * swz<NP>(4 * ks + g, hr)]);
#pragma unroll
            for (int kt = 0; kt < 2; ++kt) u[kt] = mfma_bf16_16x16x32(qf, kf[kt][ks], u[kt]);
          }
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r)
              cv[kt][4 * h2 + r] = u[kt][r] > 0.0f ? dv[kt] * ws[st][16 * ht + 4 * g + r] : 0.0f;
        }
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          cb[hs][kt] = __builtin_bit_cast(
              v8bf, (v4i){(int)pack_bf16x2(cv[kt][0], cv[kt][1]), (int)pack_bf16x2(cv[kt][2], cv[kt][3]),
                          (int)pack_bf16x2(cv[kt][4], cv[kt][5]), (int)pack_bf16x2(cv[kt][6], cv[kt][7])});
      }
      // dk^T += Q^T . c: A lane (d = 16dt + li) holds the same 8 heads
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const int pc = swz<NP>(2 * dt + tr_sel, tr_head);  // same for every head row the lane reads
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const uint8_t* qr = (const uint8_t*)&qa[st][(32 * hs + tr_head) * DI] + 16 * pc + tr_half;
          const v4s lo = lds_read_tr16(qr);
          const v4s hi = lds_read_tr16(qr + 16 * DI * 2);
          const v8bf qa8 = __builtin_bit_cast(v8bf, (v8s_t){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]});
#pragma unroll
          for (int kt = 0; kt < 2; ++kt) acc[kt][dt] = mfma_bf16_16x16x32(qa8, cb[hs][kt], acc[kt][dt]);
        }
      }
    }
    if (t + 1 < t_hi) stage(st ^ 1, nxt, nw);
    __syncthreads();
  }

#pragma unroll
  for (int kt = 0; kt < 2; ++kt) {
    const int key = key0 + 16 * kt;
    if (key < a.Lk) {
      float* dk = a.dk_idx + ((size_t)b * a.Lk + key) * DI;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
#pragma unroll
        for (int r = 0; r < 4; ++r) unsafeAtomicAdd(dk + 16 * dt + 4 * g + r, acc[kt][dt][r]);
    }
  }
}

template <int DI>
hipError_t launch_di(const IndexBwdArgs& a, hipStream_t stream) {
  const long long qblocks = (long long)a.B * ((a.Lq + kQRows - 1) / kQRows);
  hipError_t e = launch_kernel((const void*)index_bwd_q_kernel<DI>, dim3((unsigned)qblocks), dim3(512), 0, stream, a);
  if (e != hipSuccess) return e;
  // rows per key block: 128 (a sweep at 32K: 32 / 64 / 128 / 256 / 512 rows
  // -> 70.4 / 68.2 / 68.8 / 72.2 / 79.9 ms for the indexer backward; fewer
  // rows balance the causal triangle better, more rows add fewer atomics),
  // halved while the grid would not fill the chip several times over
  const long long nkb = (a.Lk + kKeysPerBlock - 1) / kKeysPerBlock;
  int rows = 128;
  while (rows > 32 && (long long)a.B * nkb * ((a.Lq + rows - 1) / rows) < 4 * 256) rows /= 2;
  const long long kblocks = (long long)a.B * nkb * ((a.Lq + rows - 1) / rows);
  return launch_kernel((const void*)index_bwd_k_kernel<DI>, dim3((unsigned)kblocks), dim3(512), 0, stream, a, rows);
}

}  // namespace

hipError_t launch_index_scores_bwd(const IndexBwdArgs& a, hipStream_t stream) {
  switch (a.DI) {
    case 32: return launch_di<32>(a, stream);
    case 64: return launch_di<64>(a, stream);
    case 96: return launch_di<96>(a, stream);
    case 128: return launch_di<128>(a, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace dsa
