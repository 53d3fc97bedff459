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
// final compaction walks the row in index order with one block-wide scan per
// 4096-element tile: an element is kept when its key is above the threshold,
// or equal to it and among the first (needed) equal keys.  Rows up to 32768
// candidates are cached in LDS as keys after the first pass; longer rows are
// re-read from global memory (L2) on each pass.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;
constexpr int kCacheMax = 32768;

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

template <bool CACHED>
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                   // kBins
  uint32_t* scan_sh = smem + kBins;        // kWaves + 1
  uint32_t* ctrl = scan_sh + kWaves + 1;   // [0] digit, [1] count above
  uint32_t* cache = ctrl + 4;              // kCacheMax keys (CACHED only)

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
      uint32_t key;
      if (!CACHED || pass == 0) {
        key = order_key(srow[i]);
        if (CACHED) cache[i] = key;
      } else {
        key = cache[i];
      }
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
      keys[j] = i < n ? (CACHED ? cache[i] : order_key(srow[i])) : 0u;
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

// Register-resident variant for rows of at most EPT * kThreads candidates:
// thread t holds the keys of the contiguous candidates [EPT*t, EPT*t + EPT), so
// the digit passes touch LDS only for the histogram and the ordered compaction
// needs a single block-wide scan.  LDS use is ~8 KiB, so several rows run per
// CU.  VEC loads the segment with 16-byte loads (row stride a multiple of 4).
template <int EPT, bool VEC, int NT>
__global__ __launch_bounds__(NT) void topk_reg_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kBins];
  __shared__ uint32_t scan_sh[NT / 64 + 1];
  __shared__ uint32_t ctrl[4];

  const int row = blockIdx.x;
  const int t = row % a.Lq;
  const int pos = a.q_start + t;
  const int n = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = a.scores + (size_t)row * a.Lk;
  const int base = EPT * threadIdx.x;
  const int cnt = max(0, min(EPT, n - base));  // valid candidates of this thread

  uint32_t key[EPT];
  if (VEC && cnt == EPT) {
#pragma unroll
    for (int j = 0; j < EPT; j += 4) {
      const v4f v = *(const v4f*)(srow + base + j);
#pragma unroll
      for (int e = 0; e < 4; ++e) key[j + e] = order_key(v[e]);
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; ++j) key[j] = j < cnt ? order_key(srow[base + j]) : 0u;
  }

  uint32_t prefix = 0, mask = 0;
  uint32_t need = (uint32_t)a.k;
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
    constexpr int BPT = kBins / NT;
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
        if (o < (uint32_t)a.k) out[o] = base + j;
        ++gt_before;
      } else if (is_eq) {
        if (eq_before < need && gt_before + eq_before < (uint32_t)a.k) out[gt_before + eq_before] = base + j;
        ++eq_before;
      }
    }
  }
}

}  // namespace

size_t topk_workspace_bytes(int, int, int, int) { return 0; }

hipError_t launch_topk(const TopkArgs& a, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)a.B * a.Lq));
  const int max_n = min(a.q_start + a.Lq, a.Lk);
  const size_t base = (size_t)(kBins + kWaves + 1 + 4) * sizeof(uint32_t);
  if (max_n <= 64 * 512) {
    if (a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0)
      return launch_kernel((const void*)topk_reg_kernel<64, true, 512>, grid, dim3(512), 0, stream, a);
    return launch_kernel((const void*)topk_reg_kernel<64, false, 512>, grid, dim3(512), 0, stream, a);
  }
  if (max_n <= kCacheMax) {
    static const hipError_t attr = hipFuncSetAttribute(
        (const void*)topk_kernel<true>, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
    const size_t smem = base + (size_t)max_n * sizeof(uint32_t);
    return launch_kernel((const void*)topk_kernel<true>, grid, dim3(kThreads), smem, stream, a);
  }
  return launch_kernel((const void*)topk_kernel<false>, grid, dim3(kThreads), base, stream, a);
}

}  // namespace dsa
