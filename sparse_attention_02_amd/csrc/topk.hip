// Per-row top-k selection as a radix select over fp32 scores (no matrix cores).
//
// Each query row keeps the min(k, pos(t)+1) tokens s <= pos(t) that come first
// under (score descending, index ascending) — fine-grained token selection of
// the lightning indexer's scores ("DeepSeek V3.2 and the lightning indexer",
// section "How the lightning indexer works"; DeepSeek-V3.2 spec sheet, section
// 2.1).  Ties at the threshold go to the lower index; output is ascending.
//
// Scores are mapped to order-preserving 32-bit keys (-0 folded onto +0).  Up to
// three digit passes (11, 11 and 10 bits) build LDS histograms of the keys that
// still match the chosen prefix and pick the digit holding the k-th largest
// key.  A pass stops early when every key of the chosen bin is selected.  The
// ordered compaction then keeps, in index order, the keys above the threshold
// and the first (needed) keys equal to it.
//  * Rows of up to 32768 candidates: one block, keys held in registers.
//  * Longer rows: two stages through a workspace (per-segment top k, then the
//    top k of the segments' candidates), which also spreads a few long rows
//    (decode) over many blocks.
//  * Rows beyond that: one block re-reading the row from L2 on each pass.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

__device__ __forceinline__ uint32_t order_key(float f) {
  uint32_t u = __float_as_uint(f);
  if (u == 0x80000000u) u = 0u;  // -0 ties with +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inclusive block scan of v over kThreads threads; `sh` holds kWaves+1 words.
__device__ __forceinline__ uint32_t block_inclusive_scan(uint32_t v, uint32_t* sh, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < kWaves ? sh[lane] : 0u;
#pragma unroll
    for (int o = 1; o < kWaves; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane < kWaves) sh[lane] = x;
  }
  __syncthreads();
  const uint32_t add = wave > 0 ? sh[wave - 1] : 0u;
  total = sh[kWaves - 1];
  __syncthreads();
  return v + add;
}

template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan_n(uint32_t v, uint32_t* sh, uint32_t& total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(v, o);
    if (lane >= o) v += y;
  }
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  if (wave == 0) {
    uint32_t x = lane < NWV ? sh[lane] : 0u;
#pragma unroll
    for (int o = 1; o < NWV; o <<= 1) {
      const uint32_t y = __shfl_up(x, o);
      if (lane >= o) x += y;
    }
    if (lane < NWV) sh[lane] = x;
  }
  __syncthreads();
  const uint32_t add = wave > 0 ? sh[wave - 1] : 0u;
  total = sh[NWV - 1];
  __syncthreads();
  return v + add;
}

// Fallback for rows too long for the two-stage path: the row is re-read from
// global memory (L2) on each digit pass.
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                   // kBins
  uint32_t* scan_sh = smem + kBins;        // kWaves + 1
  uint32_t* ctrl = scan_sh + kWaves + 1;   // [0] digit, [1] count above

  const int row = blockIdx.x;
  const int t = row % a.Lq;
  const int pos = a.q_start + t;
  const int n = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;

  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = a.scores + (size_t)row * a.Lk;

  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)a.k;  // keys still to take among those matching prefix
  bool all_ge = false;

#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = order_key(srow[i]);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // Thread i owns bins (2047-2i, 2046-2i); an inclusive scan in descending bin
    // order gives suffix counts.  The chosen digit d satisfies
    // count(>= d) >= need > count(> d).
    const int b0 = kBins - 1 - 2 * (int)threadIdx.x, b1 = b0 - 1;
    const uint32_t h0 = hist[b0], h1 = hist[b1];
    uint32_t total;
    const uint32_t incl = block_inclusive_scan(h0 + h1, scan_sh, total);
    const uint32_t excl = incl - h0 - h1;
    if (excl < need && need <= excl + h0) { ctrl[0] = (uint32_t)b0; ctrl[1] = excl; }
    if (excl + h0 < need && need <= incl) { ctrl[0] = (uint32_t)b1; ctrl[1] = excl + h0; }
    __syncthreads();
    const uint32_t d = ctrl[0];
    need -= ctrl[1];
    prefix |= d << shift;
    mask |= dmask << shift;
    const uint32_t bin_count = hist[d];
    __syncthreads();
    if (bin_count == need) { all_ge = true; break; }
  }

  // ---- ordered compaction
  const uint32_t T = prefix;
  uint32_t gt_base = 0, eq_base = 0;
  for (int base = 0; base < n; base += 4 * kThreads) {
    const int i0 = base + 4 * threadIdx.x;
    uint32_t keys[4];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j;
      keys[j] = i < n ? order_key(srow[i]) : 0u;
      const bool in = i < n;
      const bool is_gt = in && (all_ge ? keys[j] >= T : keys[j] > T);
      const bool is_eq = in && !all_ge && keys[j] == T;
      gt += is_gt; eq += is_eq;
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan(gt | (eq << 16), scan_sh, total);
    const uint32_t excl = incl - (gt | (eq << 16));
    uint32_t gt_before = gt_base + (excl & 0xFFFFu);
    uint32_t eq_before = eq_base + (excl >> 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j;
      if (i >= n) break;
      const bool is_gt = all_ge ? keys[j] >= T : keys[j] > T;
      const bool is_eq = !all_ge && keys[j] == T;
      if (is_gt) {
        const uint32_t o = gt_before + min(eq_before, need);
        if (o < (uint32_t)a.k) out[o] = i;
        ++gt_before;
      } else if (is_eq) {
        if (eq_before < need && gt_before + eq_before < (uint32_t)a.k) out[gt_before + eq_before] = i;
        ++eq_before;
      }
    }
    gt_base += total & 0xFFFFu;
    eq_base += total >> 16;
  }
}

// Register-resident selection among n <= EPT * NT candidates c = 0..n-1:
// thread t holds the keys of the contiguous candidates [EPT*t, EPT*t + EPT), so
// the digit passes touch LDS only for the histogram and the ordered compaction
// needs a single block-wide scan.  Key 0 marks an absent candidate (real keys
// are >= 1 where absent ones can occur).  emit(o, c, key) is called for the k
// selected candidates, o = their rank in ascending c.
template <int EPT, int NT>
struct RegSelect {
  static constexpr int BPT = kBins / NT;  // histogram bins per thread in the digit scan
  uint32_t* hist;
  uint32_t* scan_sh;
  uint32_t* ctrl;

  template <typename Emit>
  __device__ __forceinline__ void run(const uint32_t (&key)[EPT], int cnt, int base, uint32_t k,
                                      Emit&& emit) {
    uint32_t prefix = 0, mask = 0;
    uint32_t need = k;
    bool all_ge = false;
#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
      for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int j = 0; j < EPT; ++j)
        if (j < cnt && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & dmask], 1u);
      __syncthreads();
      // thread i owns bins kBins-1-BPT*i down to kBins-BPT*(i+1); a scan in
      // descending bin order gives suffix counts
      uint32_t h[BPT], hs = 0;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        h[e] = hist[kBins - 1 - BPT * (int)threadIdx.x - e];
        hs += h[e];
      }
      uint32_t total;
      const uint32_t incl = block_inclusive_scan_n<NT>(hs, scan_sh, total);
      uint32_t above = incl - hs;
#pragma unroll
      for (int e = 0; e < BPT; ++e) {
        if (above < need && need <= above + h[e]) {
          ctrl[0] = (uint32_t)(kBins - 1 - BPT * (int)threadIdx.x - e);
          ctrl[1] = above;
        }
        above += h[e];
      }
      __syncthreads();
      const uint32_t d = ctrl[0];
      need -= ctrl[1];
      prefix |= d << shift;
      mask |= dmask << shift;
      const uint32_t bin_count = hist[d];
      __syncthreads();
      if (bin_count == need) { all_ge = true; break; }
    }

    // ---- ordered compaction: one scan of per-thread (greater, equal) counts
    const uint32_t T = prefix;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j < cnt) {
        gt += all_ge ? key[j] >= T : key[j] > T;
        eq += !all_ge && key[j] == T;
      }
    }
    uint32_t total;
    const uint32_t packed = gt | (eq << 16);
    const uint32_t excl = block_inclusive_scan_n<NT>(packed, scan_sh, total) - packed;
    uint32_t gt_before = excl & 0xFFFFu, eq_before = excl >> 16;
#pragma unroll
    for (int j = 0; j < EPT; ++j) {
      if (j < cnt) {
        const bool is_gt = all_ge ? key[j] >= T : key[j] > T;
        const bool is_eq = !all_ge && key[j] == T;
        if (is_gt) {
          const uint32_t o = gt_before + min(eq_before, need);
          if (o < k) emit(o, base + j, key[j]);
          ++gt_before;
        } else if (is_eq) {
          if (eq_before < need && gt_before + eq_before < k) emit(gt_before + eq_before, base + j, key[j]);
          ++eq_before;
        }
      }
    }
  }
};

// Keys of the scores [base, base + cnt) of one row; VEC: 16-byte loads.
template <int EPT, bool VEC>
__device__ __forceinline__ void load_keys(const float* src, int base, int cnt, uint32_t (&key)[EPT]) {
  if (VEC && cnt == EPT) {
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
      const v4f v = *(const v4f*)(src + base + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j + e] = order_key(v[e]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = j < cnt ? order_key(src[base + j]) : 0u;
  }
}

// One block per row of at most EPT * NT candidates.
template <int EPT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void topk_reg_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[NT / 64 + 1];
  __shared__ uint32_t ctrl[4];
  const int row = blockIdx.x;
  const int pos = a.q_start + row % a.Lq;
  const int n = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const int base = EPT * threadIdx.x;
  const int cnt = max(0, min(EPT, n - base));
  uint32_t key[EPT];
  load_keys<EPT, VEC>(a.scores + (size_t)row * a.Lk, base, cnt, key);
  RegSelect<EPT, NT>{hist, scan_sh, ctrl}.run(key, cnt, base, (uint32_t)a.k,
                                              [&](uint32_t o, int c, uint32_t) { out[o] = c; });
}

// Rows longer than one block holds are selected in two stages.  The top k of
// a row are among the union of the top k of its segments (an element beaten
// by k others inside its segment is beaten by them in the row), and the order
// (score descending, index ascending) is the same in both stages because the
// candidates of a row are kept in ascending index order.
//
// Stage 1: one block per (row, segment of kSeg keys) writes its segment's top
// min(k, length) candidates as (key, index) into slots [row][segment][0..k),
// in ascending index order; unused slots hold key 0 and index -1.  Real keys
// are made >= 1 so that a padding slot never ties with a candidate.
constexpr int kSeg = 8192;
constexpr int kSegNT = 256;
constexpr int kCandMax = 64 * 512;  // candidates per row that stage 2 can hold

template <bool VEC>
__global__ __launch_bounds__(kSegNT) void topk_seg_kernel(TopkArgs a) {
  constexpr int EPT = kSeg / kSegNT;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[kSegNT / 64 + 1];
  __shared__ uint32_t ctrl[4];
  const int row = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  const int pos = a.q_start + row % a.Lq;
  const int n_row = min(pos + 1, a.Lk);
  if (n_row <= a.k) return;  // stage 2 writes short rows directly
  const int s0 = seg * kSeg;
  const int n = max(0, min(kSeg, n_row - s0));
  uint32_t* ck = a.cand_key + ((size_t)row * a.nseg + seg) * a.k;
  int32_t* ci = a.cand_idx + ((size_t)row * a.nseg + seg) * a.k;
  const float* src = a.scores + (size_t)row * a.Lk + s0;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kSegNT) {
      ck[i] = i < n ? max(order_key(src[i]), 1u) : 0u;
      ci[i] = i < n ? s0 + i : -1;
    }
    return;
  }
  const int base = EPT * threadIdx.x;
  const int cnt = max(0, min(EPT, n - base));
  uint32_t key[EPT];
  load_keys<EPT, VEC>(src, base, cnt, key);
  RegSelect<EPT, kSegNT>{hist, scan_sh, ctrl}.run(key, cnt, base, (uint32_t)a.k,
                                                  [&](uint32_t o, int c, uint32_t kv) {
                                                    ck[o] = max(kv, 1u);
                                                    ci[o] = s0 + c;
                                                  });
}

// Stage 2: one block per row selects among its nseg * k candidate slots.
__global__ __launch_bounds__(512) void topk_cand_kernel(TopkArgs a) {
  constexpr int NT = 512, EPT = kCandMax / NT;
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[NT / 64 + 1];
  __shared__ uint32_t ctrl[4];
  const int row = blockIdx.x;
  const int pos = a.q_start + row % a.Lq;
  const int n_row = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;
  if (n_row <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n_row ? i : -1;
    return;
  }
  const int n = a.nseg * a.k;
  const uint32_t* ck = a.cand_key + (size_t)row * n;
  const int32_t* ci = a.cand_idx + (size_t)row * n;
  const int base = EPT * threadIdx.x;
  const int cnt = max(0, min(EPT, n - base));
  uint32_t key[EPT];
  if (cnt == EPT) {
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
      const v4i v = *(const v4i*)(ck + base + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j + e] = (uint32_t)v[e];
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = j < cnt ? ck[base + j] : 0u;
  }
  RegSelect<EPT, NT>{hist, scan_sh, ctrl}.run(key, cnt, base, (uint32_t)a.k,
                                              [&](uint32_t o, int c, uint32_t) { out[o] = ci[c]; });
}

// Segments per row for the two-stage path (0: the row fits one block or the
// candidates of its segments would not fit stage 2).
int topk_segments(int Lq, int q_start, int Lk, int k) {
  const int max_n = min(q_start + Lq, Lk);
  if (max_n <= kCandMax) return 0;
  const int nseg = (max_n + kSeg - 1) / kSeg;
  if ((long long)nseg * k > kCandMax || k % 4 != 0) return 0;
  return nseg;
}

}  // namespace

size_t topk_workspace_bytes(int B, int Lq, int q_start, int Lk, int k) {
  const int nseg = topk_segments(Lq, q_start, Lk, k);
  return (size_t)B * Lq * nseg * k * (sizeof(uint32_t) + sizeof(int32_t));
}

hipError_t launch_topk(const TopkArgs& args, hipStream_t stream) {
  TopkArgs a = args;
  const long long rows = (long long)a.B * a.Lq;
  const dim3 grid((unsigned)rows);
  const int max_n = min(a.q_start + a.Lq, a.Lk);
  if (max_n <= kCandMax) {
    if (a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0)
      return launch_kernel((const void*)topk_reg_kernel<64, true, 512>, grid, dim3(512), 0, stream, a);
    return launch_kernel((const void*)topk_reg_kernel<64, false, 512>, grid, dim3(512), 0, stream, a);
  }
  a.nseg = topk_segments(a.Lq, a.q_start, a.Lk, a.k);
  if (a.nseg > 0 && a.workspace) {
    a.cand_key = (uint32_t*)a.workspace;
    a.cand_idx = (int32_t*)(a.cand_key + (size_t)rows * a.nseg * a.k);
    const bool vec = a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0;
    hipError_t e = launch_kernel(vec ? (const void*)topk_seg_kernel<true> : (const void*)topk_seg_kernel<false>,
                                 dim3((unsigned)(rows * a.nseg)), dim3(kSegNT), 0, stream, a);
    if (e != hipSuccess) return e;
    return launch_kernel((const void*)topk_cand_kernel, grid, dim3(512), 0, stream, a);
  }
  const size_t base = (size_t)(kBins + kWaves + 1 + 4) * sizeof(uint32_t);
  return launch_kernel((const void*)topk_kernel, grid, dim3(kThreads), base, stream, a);
}

}  // namespace dsa
