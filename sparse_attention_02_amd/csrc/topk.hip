// Per-row top-k selection as a radix select over fp32 scores (no matrix cores).
//
// Each query row keeps the min(k, pos(t)+1) tokens s <= pos(t) that come first
// under (score descending, index ascending) — fine-grained token selection of
// the lightning indexer's scores ("DeepSeek V3.2 and the lightning indexer",
// section "How the lightning indexer works"; DeepSeek-V3.2 spec sheet, section
// 2.1).  Ties at the threshold go to the lower index; output is ascending.
//
// Scores are mapped to order-preserving 32-bit keys (-0 folded onto +0).  Digit
// passes build LDS histograms of the keys that still match the chosen prefix
// and pick the digit holding the k-th largest key; a pass stops early when
// every key of the chosen bin is selected.  The ordered compaction then keeps,
// in index order, the keys above the threshold and the first (needed) keys
// equal to it.  Rows held in registers are first cut down to a few thousand
// candidates with a threshold taken from a sample (see select_top).
//  * Rows of up to 32768 candidates: one block, keys held in registers (as
//    16-bit prefixes, two per register, where every row fits the candidate
//    slots and is 16-byte aligned).
//  * Longer rows, at most 256 of them (decode): a cut taken on a sample of
//    each row, a filter that keeps the keys at or above it in index order,
//    and one exact select (topk_sample_cut_kernel, topk_filter_kernel,
//    topk_cand_kernel).
//  * Longer rows, more of them: two stages through a workspace (per-segment
//    top k, then the top k of the segments' candidates).
//  * Rows beyond that: one block re-reading the row from L2 on each pass.
#include "dsa_common.h"
#include "launch.h"

namespace dsa {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / 64;
constexpr int kBins = 2048;

// Wave-wide inclusive scans through DPP row shifts and row broadcasts (VALU
// only; a shuffle would be an LDS-crossbar round trip per step).  `id` is the
// identity of `op`; lane 63 ends up with the wave total.
template <typename Op>
__device__ __forceinline__ uint32_t wave_scan(uint32_t x, uint32_t id, Op op) {
  auto dpp = [&](uint32_t v, auto ctrl, auto rows) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, decltype(ctrl)::value,
                                                 decltype(rows)::value, 0xf, false);
  };
  x = op(x, dpp(x, std::integral_constant<int, 0x111>(), std::integral_constant<int, 0xf>()));  // row_shr:1
  x = op(x, dpp(x, std::integral_constant<int, 0x112>(), std::integral_constant<int, 0xf>()));  // row_shr:2
  x = op(x, dpp(x, std::integral_constant<int, 0x114>(), std::integral_constant<int, 0xf>()));  // row_shr:4
  x = op(x, dpp(x, std::integral_constant<int, 0x118>(), std::integral_constant<int, 0xf>()));  // row_shr:8
  x = op(x, dpp(x, std::integral_constant<int, 0x142>(), std::integral_constant<int, 0xa>()));  // row_bcast:15
  x = op(x, dpp(x, std::integral_constant<int, 0x143>(), std::integral_constant<int, 0xc>()));  // row_bcast:31
  return x;
}
__device__ __forceinline__ uint32_t wave_scan_add(uint32_t x) {
  return wave_scan(x, 0u, [](uint32_t a, uint32_t b) { return a + b; });
}

// Inclusive block scan of v over NT threads; `sh` holds NT/64 words.
template <int NT>
__device__ __forceinline__ uint32_t block_inclusive_scan_n(uint32_t v, uint32_t* sh, uint32_t& total) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  v = wave_scan_add(v);
  if (lane == 63) sh[wave] = v;
  __syncthreads();
  uint32_t add = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    const uint32_t s = sh[w];
    add += w < wave ? s : 0u;
    tot += s;
  }
  total = tot;
  __syncthreads();
  return v + add;
}

// Block-wide min of lo and max of hi over NT threads (results in every
// thread); `sh` holds at least 2 * NT / 64 words.
template <int NT>
__device__ __forceinline__ void block_minmax(uint32_t& lo, uint32_t& hi, uint32_t* sh) {
  constexpr int NWV = NT / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  lo = wave_scan(lo, 0xFFFFFFFFu, [](uint32_t a, uint32_t b) { return min(a, b); });
  hi = wave_scan(hi, 0u, [](uint32_t a, uint32_t b) { return max(a, b); });
  if (lane == 63) {
    sh[wave] = lo;
    sh[NWV + wave] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NWV; ++w) {
    lo = min(lo, sh[w]);
    hi = max(hi, sh[NWV + w]);
  }
  __syncthreads();
}

// Selection among n candidates whose keys are re-read through key_at(i) on
// every pass (global memory, mostly L2): fixed digits of 11, 11 and 10 bits
// from the top of the key, no register array.  emit(o, c, key) as below.
template <int NT, typename KeyAt, typename Emit>
__device__ __forceinline__ void select_streamed(uint32_t* hist, uint32_t* scan_sh, uint32_t* ctrl,
                                                KeyAt&& key_at, int n, uint32_t k, Emit&& emit) {
  constexpr int BPT = kBins / NT;
  uint32_t prefix = 0, mask = 0;
  uint32_t need = k;  // keys still to take among those matching prefix
  bool all_ge = false;
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
    const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
    for (int i = threadIdx.x; i < kBins; i += NT) hist[i] = 0u;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      const uint32_t key = key_at(i);
      if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread i owns bins kBins-1-BPT*i down to kBins-BPT*(i+1); an inclusive
    // scan in descending bin order gives suffix counts.  The chosen digit d
    // satisfies count(>= d) >= need > count(> d).
    uint32_t h[BPT], hs = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      h[e] = hist[kBins - 1 - BPT * (int)threadIdx.x - e];
      hs += h[e];
    }
    uint32_t total;
    uint32_t above = block_inclusive_scan_n<NT>(hs, scan_sh, total) - hs;
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

  // ---- ordered compaction, 4 * NT candidates at a time
  const uint32_t T = prefix;
  uint32_t gt_base = 0, eq_base = 0;
  for (int base = 0; base < n; base += 4 * NT) {
    const int i0 = base + 4 * threadIdx.x;
    uint32_t keys[4];
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int i = i0 + j;
      const bool in = i < n;
      keys[j] = in ? key_at(i) : 0u;
      gt += in && (all_ge ? keys[j] >= T : keys[j] > T);
      eq += in && !all_ge && keys[j] == T;
    }
    uint32_t total;
    const uint32_t packed = gt | (eq << 16);
    const uint32_t excl = block_inclusive_scan_n<NT>(packed, scan_sh, total) - packed;
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
        if (o < k) emit(o, i, keys[j]);
        ++gt_before;
      } else if (is_eq) {
        if (eq_before < need && gt_before + eq_before < k) emit(gt_before + eq_before, i, keys[j]);
        ++eq_before;
      }
    }
    gt_base += total & 0xFFFFu;
    eq_base += total >> 16;
  }
}

// Fallback for rows too long for the two-stage path: the row is re-read from
// global memory (L2) on each digit pass.
__global__ __launch_bounds__(kThreads) void topk_kernel(TopkArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint32_t smem[];
  uint32_t* hist = smem;                   // kBins
  uint32_t* scan_sh = smem + kBins;        // kWaves + 1
  uint32_t* ctrl = scan_sh + kWaves + 1;   // [0] digit, [1] count above

  const int row = blockIdx.x;
  if (a.only_rows && !a.only_rows[row]) return;
  const int t = row % a.Lq;
  const int pos = a.q_start + t;
  const int n = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;

  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += kThreads) out[i] = i < n ? i : -1;
    return;
  }
  const float* srow = a.scores + (size_t)row * a.Lk;
  select_streamed<kThreads>(hist, scan_sh, ctrl, [&](int i) { return order_key(srow[i]); }, n,
                            (uint32_t)a.k, [&](uint32_t o, int c, uint32_t) { out[o] = c; });
}

// Block-wide selection among n candidates c = 0..n-1 held in registers:
// thread t holds the keys of the contiguous candidates [EPT*t, EPT*t + EPT).
// Key 0 marks an absent candidate (real keys are >= 1 where absent ones can
// occur).  emit(o, c, key) is called for the k selected candidates, o = their
// rank in ascending c.
//
// Radix passes over all n keys cost one LDS atomic per key and pass, random
// histogram updates conflict in the LDS banks, and every pass is a chain of
// barriers, so long rows are first cut down: one histogram pass over a
// stride-16 sample gives a bin edge t with about r sampled keys above it (r a
// few standard deviations above the expected sampled rank of the k-th key),
// the keys >= t are counted, and when there are between k and kCap of them
// they are compacted, in index order, into LDS, where the exact selection
// runs.  This is exact: at least k keys >= t means the k-th largest key is
// >= t, so every key that can be selected, ties included, is a candidate, and
// the candidates keep their index order.  Otherwise the passes run on all keys.
constexpr int kCap = 4096;     // LDS candidate slots
constexpr int kDigit = 12;     // bits per radix digit
constexpr int kHist = 1 << kDigit;

template <int NT>
struct BlockSelect {
  static constexpr int BPT = kHist / NT;  // histogram bins per thread in the digit scan
  uint32_t* hist;
  uint32_t* scan_sh;
  uint32_t* ctrl;

  // One digit pass: histogram of the digit (r >> shift) & dmask of the keys
  // key[j < cnt] with r >> cur == pref (r = key - kmin; every key when cur is
  // 32), then the digit holding the need-th largest of them.  Returns the
  // digit; `above` = the matching keys in higher digits, `in_bin` = in it.
  template <int E>
  __device__ __forceinline__ uint32_t digit_pass(const uint32_t (&key)[E], int cnt, uint32_t kmin, int cur,
                                                 uint32_t pref, int shift, uint32_t dmask, uint32_t need,
                                                 uint32_t& above_out, uint32_t& in_bin) {
    for (int i = threadIdx.x; i < kHist; i += NT) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int j = 0; j < E; ++j) {
      const uint32_t r = key[j] - kmin;
      const bool match = cur >= 32 || (r >> cur) == pref;
      if (j < cnt && match) atomicAdd(&hist[(r >> shift) & dmask], 1u);
    }
    __syncthreads();
    // thread i owns bins kHist-1-BPT*i down to kHist-BPT*(i+1); a scan in
    // descending bin order gives suffix counts
    uint32_t h[BPT], hs = 0;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      h[e] = hist[kHist - 1 - BPT * (int)threadIdx.x - e];
      hs += h[e];
    }
    uint32_t total;
    const uint32_t incl = block_inclusive_scan_n<NT>(hs, scan_sh, total);
    uint32_t above = incl - hs;
#pragma unroll
    for (int e = 0; e < BPT; ++e) {
      if (above < need && need <= above + h[e]) {
        ctrl[0] = (uint32_t)(kHist - 1 - BPT * (int)threadIdx.x - e);
        ctrl[1] = above;
        ctrl[2] = h[e];
      }
      above += h[e];
    }
    __syncthreads();
    const uint32_t dg = ctrl[0];
    above_out = ctrl[1];
    in_bin = ctrl[2];
    __syncthreads();
    return dg;
  }

  // min and max of the keys key[j < cnt] of the block
  template <int E>
  __device__ __forceinline__ void range(const uint32_t (&key)[E], int cnt, uint32_t& lo, uint32_t& hi) {
    lo = 0xFFFFFFFFu;
    hi = 0u;
#pragma unroll
    for (int j = 0; j < E; ++j)
      if (j < cnt) {
        lo = min(lo, key[j]);
        hi = max(hi, key[j]);
      }
    block_minmax<NT>(lo, hi, scan_sh);
  }

  // A key value t such that at least k (1 <= k <= their number) of the keys
  // are >= t: the lower edge of the top digit bin that reaches k.
  template <int E>
  __device__ __forceinline__ uint32_t coarse_threshold(const uint32_t (&key)[E], int cnt, uint32_t k) {
    uint32_t lo, hi;
    range(key, cnt, lo, hi);
    const int cur = hi > lo ? 32 - __builtin_clz(hi - lo) : 0;
    if (cur == 0) return lo;
    const int d = min(kDigit, cur);
    uint32_t above, in_bin;
    const uint32_t dg = digit_pass(key, cnt, lo, 32, 0u, cur - d, (1u << d) - 1u, k, above, in_bin);
    return lo + (dg << (cur - d));
  }

  // Threshold of the k-th largest of the keys key[j < cnt] of the block
  // (1 <= k <= their number): the selected keys are those > T plus the first
  // `need` (in candidate order) equal to T, or all keys >= T when all_ge.
  // The keys are left rebased by kmin (and T is too): restoring them would
  // make the compiler keep the original keys alive as a second copy.
  // The digits are taken from r = key - kmin, starting at the top bit of
  // kmax - kmin: the keys of one row span a few binades, so digits cut from the
  // top of the raw key would crowd them into a handful of bins.
  template <int E>
  __device__ __forceinline__ void threshold(uint32_t (&key)[E], int cnt, uint32_t k, uint32_t& T,
                                            uint32_t& need, bool& all_ge, uint32_t& kmin) {
    uint32_t lo, hi;
    range(key, cnt, lo, hi);
    kmin = lo;
    // Rebased in place, through asm so that each key keeps its register: key -
    // lo recomputed in every pass is hoisted out of the pass loop, and a plain
    // subtraction is given fresh registers while the originals are still live
    // (either way a second copy of the keys).
    const uint32_t lo_s = __builtin_amdgcn_readfirstlane(lo);
#pragma unroll
    for (int j = 0; j < E; ++j) asm volatile("v_subrev_u32 %0, %1, %0" : "+v"(key[j]) : "s"(lo_s));
    int cur = hi > lo ? 32 - __builtin_clz(hi - lo) : 0;  // bits of r still undecided
    uint32_t pref = 0;                                     // r >> cur of the chosen keys
    need = k;
    all_ge = false;
#pragma unroll 1
    while (cur > 0) {
      const int d = min(kDigit, cur);
      const int shift = cur - d;
      uint32_t above, in_bin;
      const uint32_t dg = digit_pass(key, cnt, 0u, cur, pref, shift, (1u << d) - 1u, need, above, in_bin);
      need -= above;
      pref = (pref << d) | dg;
      cur = shift;
      if (in_bin == need) { all_ge = true; break; }
    }
    T = pref << cur;  // cur < 32 here: a range of 32 bits takes a pass
  }

  // Ordered emission of the keys chosen by threshold() (keys and T rebased
  // by kmin): one scan of the per-thread (greater, equal) counts gives every
  // key its output rank.
  template <int E, typename Emit>
  __device__ __forceinline__ void emit_top(const uint32_t (&key)[E], int cnt, int base, uint32_t k,
                                           uint32_t T, uint32_t need, bool all_ge, uint32_t kmin,
                                           Emit&& emit) {
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < E; ++j) {
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
    for (int j = 0; j < E; ++j) {
      if (j < cnt) {
        const bool is_gt = all_ge ? key[j] >= T : key[j] > T;
        const bool is_eq = !all_ge && key[j] == T;
        if (is_gt) {
          const uint32_t o = gt_before + min(eq_before, need);
          if (o < k) emit(o, base + j, key[j] + kmin);
          ++gt_before;
        } else if (is_eq) {
          if (eq_before < need && gt_before + eq_before < k)
            emit(gt_before + eq_before, base + j, key[j] + kmin);
          ++eq_before;
        }
      }
    }
  }
};

// The k largest of the n (> k) candidates held as described above; `ck` and
// `ci` are kCap-slot LDS arrays.
template <int EPT, int NT, typename KeyAt, typename Emit>
__device__ __forceinline__ void select_top(BlockSelect<NT> sel, uint32_t (&key)[EPT], int cnt, int n,
                                           uint32_t k, uint32_t* ck, int32_t* ci, KeyAt&& key_at,
                                           Emit&& emit, int n_real = -1) {
  static_assert(EPT % 16 == 0 && kCap % NT == 0, "sample stride and candidate slots");
  constexpr int S = EPT / 16;     // samples per thread: candidates 16s of its range
  constexpr int E2 = kCap / NT;   // candidates per thread in the exact selection
  const int base = EPT * (int)threadIdx.x;
  // n_real >= 0: the n slots hold n_real real keys (>= 1) among padding
  // keys 0; the cut then never lets the padding through, and the sample's
  // size and rank are taken over the real keys it holds
  const bool padded = n_real >= 0;
  const int nr = padded ? n_real : n;
  uint32_t t = padded ? 1u : 0u;  // every (real) key is >= t
  if (nr > kCap) {
    uint32_t smp[S];
#pragma unroll
    for (int e = 0; e < S; ++e) smp[e] = key[16 * e];
    const int scnt = min(S, (cnt + 15) / 16);
    uint32_t m = (uint32_t)(n + 15) / 16;  // sampled candidates: 0, 16, 32, ... < n
    if (padded) {
      // padding samples take the smallest real sample's value, so that the
      // cut's digits span the real keys only (from 0 they would crowd them
      // into a few coarse bins); they still rank below every real sample
      uint32_t real = 0, lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
      for (int e = 0; e < S; ++e)
        if (e < scnt && smp[e] != 0u) {
          lo = min(lo, smp[e]);
          ++real;
        }
      block_minmax<NT>(lo, hi, sel.scan_sh);
#pragma unroll
      for (int e = 0; e < S; ++e) smp[e] = smp[e] != 0u ? smp[e] : lo;
      block_inclusive_scan_n<NT>(real, sel.scan_sh, m);
      m = max(m, 1u);
    }
    const float qm = (float)k * (float)m / (float)nr;
    const uint32_t r = min(m, (uint32_t)(qm + 4.0f * sqrtf(qm) + 8.0f));
    t = sel.coarse_threshold(smp, scnt, r);
    if (padded) t = max(t, 1u);
  }
  // One scan of the per-thread counts of keys >= t gives both the total (is
  // the cut usable: at least k and at most kCap candidates) and each
  // thread's place in the compaction.
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) mine += j < cnt && key[j] >= t;
  uint32_t total;
  uint32_t o = block_inclusive_scan_n<NT>(mine, sel.scan_sh, total) - mine;
  const bool filtered = total >= k && total <= (uint32_t)kCap;  // block-uniform
  if (filtered) {
    // the predicates are recomputed rather than kept from the count: 64 live
    // ones would cost as many registers as the keys
    asm volatile("" : "+v"(t));
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (j < cnt && key[j] >= t) {
        ck[o] = key[j];
        ci[o] = base + j;
        ++o;
      }
    __syncthreads();
    const int b2 = E2 * (int)threadIdx.x;
    const int cnt2 = max(0, min(E2, (int)total - b2));
    uint32_t k2[E2];
#pragma unroll
    for (int e = 0; e < E2; ++e) k2[e] = e < cnt2 ? ck[b2 + e] : 0u;
    uint32_t T, need, kmin;
    bool all_ge;
    sel.threshold(k2, cnt2, k, T, need, all_ge, kmin);
    sel.emit_top(k2, cnt2, b2, k, T, need, all_ge, kmin,
                 [&](uint32_t o2, int c2, uint32_t kv) { emit(o2, ci[c2], kv); });
  } else {
    // the registers are not used here: a second register-array selection
    // would double the kernel's register count for a rare case
    select_streamed<NT>(sel.hist, sel.scan_sh, sel.ctrl, key_at, n, k, emit);
  }
}

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
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  __shared__ uint32_t cand_k[kCap];
  __shared__ int32_t cand_i[kCap];
  const int row = blockIdx.x;
  if (a.only_rows && !a.only_rows[row]) return;
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
  const float* srow = a.scores + (size_t)row * a.Lk;
  select_top<EPT, NT>(BlockSelect<NT>{hist, scan_sh, ctrl}, key, cnt, n, (uint32_t)a.k, cand_k, cand_i,
                      [&](int i) { return order_key(srow[i]); },
                      [&](uint32_t o, int c, uint32_t) { out[o] = c; });
}

// Rows of up to EPT * NT candidates with the keys held as 16-bit prefixes
// (the top half of the order key), two per register: half the registers of
// the full keys, so three 512-thread blocks fit a CU instead of two.  A cut
// at a prefix boundary, t << 16, keeps the selection exact (a key is >= t << 16
// exactly when its prefix is >= t); the exact stage takes the full keys of
// its at most kCap candidates from the row again (key_at).
template <int EPT, bool VEC>
__device__ __forceinline__ void load_prefixes(const float* src, int base, int cnt, uint32_t (&pk)[EPT / 2]) {
  if (VEC && cnt == EPT) {
    // every load is issued before any is packed: the row's loads then share
    // one memory latency (64 registers in flight, then half of them kept)
    v4f raw[EPT / 4];
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) raw[j] = *(const v4f*)(src + base + 4 * j);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < EPT / 4; ++j) {
      pk[2 * j] = (order_key(raw[j][0]) >> 16) | (order_key(raw[j][1]) & 0xFFFF0000u);
      pk[2 * j + 1] = (order_key(raw[j][2]) >> 16) | (order_key(raw[j][3]) & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int j = 0; j < EPT; j += 2) {
      const uint32_t a0 = j < cnt ? order_key(src[base + j]) : 0u;
      const uint32_t a1 = j + 1 < cnt ? order_key(src[base + j + 1]) : 0u;
      pk[j / 2] = (a0 >> 16) | (a1 & 0xFFFF0000u);
    }
  }
}

template <int EPT>
__device__ __forceinline__ uint32_t prefix_at(const uint32_t (&pk)[EPT / 2], int j) {
  return (j & 1) ? pk[j / 2] >> 16 : pk[j / 2] & 0xFFFFu;
}

template <int EPT, int NT, typename KeyAt, typename Emit>
__device__ __forceinline__ void select_top_prefix(BlockSelect<NT> sel, uint32_t (&pk)[EPT / 2], int cnt,
                                                  int n, uint32_t k, int32_t* ci, KeyAt&& key_at, Emit&& emit) {
  static_assert(EPT % 16 == 0 && kCap % NT == 0, "sample stride and candidate slots");
  constexpr int S = EPT / 16;
  constexpr int E2 = kCap / NT;
  const int base = EPT * (int)threadIdx.x;
  uint32_t t = 0;  // a prefix
  if (n > kCap) {
    uint32_t smp[S];
#pragma unroll
    for (int e = 0; e < S; ++e) smp[e] = prefix_at<EPT>(pk, 16 * e);
    const int scnt = min(S, (cnt + 15) / 16);
    const uint32_t m = (uint32_t)(n + 15) / 16;
    const float qm = (float)k * (float)m / (float)n;
    const uint32_t r = min(m, (uint32_t)(qm + 4.0f * sqrtf(qm) + 8.0f));
    t = sel.coarse_threshold(smp, scnt, r);
  }
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) mine += j < cnt && prefix_at<EPT>(pk, j) >= t;
  uint32_t total;
  uint32_t o = block_inclusive_scan_n<NT>(mine, sel.scan_sh, total) - mine;
  const bool filtered = total >= k && total <= (uint32_t)kCap;
  if (filtered) {
    // the comparisons are made again rather than kept from the count: 64
    // live lane masks would not fit the scalar registers
    asm volatile("" : "+v"(t));
    int cnt_c = cnt;
    asm volatile("" : "+v"(cnt_c));
#pragma unroll
    for (int i = 0; i < EPT / 2; ++i) asm volatile("" : "+v"(pk[i]));
#pragma unroll
    for (int j = 0; j < EPT; ++j)
      if (j < cnt_c && prefix_at<EPT>(pk, j) >= t) ci[o++] = base + j;
    __syncthreads();
    const int b2 = E2 * (int)threadIdx.x;
    const int cnt2 = max(0, min(E2, (int)total - b2));
    uint32_t k2[E2];
#pragma unroll
    for (int e = 0; e < E2; ++e) k2[e] = e < cnt2 ? key_at(ci[b2 + e]) : 0u;
    uint32_t T, need, kmin;
    bool all_ge;
    sel.threshold(k2, cnt2, k, T, need, all_ge, kmin);
    sel.emit_top(k2, cnt2, b2, k, T, need, all_ge, kmin,
                 [&](uint32_t o2, int c2, uint32_t kv) { emit(o2, ci[c2], kv); });
  } else {
    select_streamed<NT>(sel.hist, sel.scan_sh, sel.ctrl, key_at, n, k, emit);
  }
}

// One block per row of at most EPT * NT candidates, keys as prefixes.
template <int EPT, bool VEC, int NT>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(6))) void topk_prefix_kernel(TopkArgs a) {
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  __shared__ int32_t cand_i[kCap];
  const int row = blockIdx.x;
  if (a.only_rows && !a.only_rows[row]) return;
  const int pos = a.q_start + row % a.Lq;
  const int n = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;
  if (n <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n ? i : -1;
    return;
  }
  const int base = EPT * threadIdx.x;
  const int cnt = max(0, min(EPT, n - base));
  const float* srow = a.scores + (size_t)row * a.Lk;
  uint32_t pk[EPT / 2];
  load_prefixes<EPT, VEC>(srow, base, cnt, pk);
  select_top_prefix<EPT, NT>(BlockSelect<NT>{hist, scan_sh, ctrl}, pk, cnt, n, (uint32_t)a.k, cand_i,
                             [&](int i) { return order_key(srow[i]); },
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
// Segments hold kSeg keys (256 threads x 32) or kSegWide keys (512 threads x
// 64).  Short segments give more blocks, long ones fewer candidates: at
// k = 2048 an 8K segment keeps a quarter of its keys, a 32K segment 1/16, so
// the narrow plan writes and re-reads 4x the candidate bytes.  The narrow
// plan is used only when the wide one would leave the chip short of blocks
// (decode over a few rows) and the 512-thread stage 2 can merge it; rows of
// up to 1M keys at k = 2048 use the wide plan and a 1024-thread stage 2 when
// their candidates exceed what the 512-thread one holds.
constexpr int kSeg = 8192;
constexpr int kSegWide = 32768;
constexpr int kCandMax = 64 * 512;    // candidates per row that stage 2 can hold
constexpr int kCandWide = 64 * 1024;  // ... the wide stage 2
constexpr long long kWideMinBlocks = 2048;  // ~4 rounds of 2 resident blocks per CU

template <int EPT, int NT, bool VEC>
__global__ __launch_bounds__(NT) void topk_seg_kernel(TopkArgs a) {
  constexpr int kSegLen = EPT * NT;
  constexpr int kSegNT = NT;
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (kSegNT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  __shared__ uint32_t cand_k[kCap];
  __shared__ int32_t cand_i[kCap];
  const int row = blockIdx.x / a.nseg;
  const int seg = blockIdx.x % a.nseg;
  if (a.only_rows && !a.only_rows[row]) return;
  const int pos = a.q_start + row % a.Lq;
  const int n_row = min(pos + 1, a.Lk);
  if (n_row <= a.k) return;  // stage 2 writes short rows directly
  const int s0 = seg * kSegLen;
  const int n = max(0, min(kSegLen, n_row - s0));
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
  select_top<EPT, kSegNT>(BlockSelect<kSegNT>{hist, scan_sh, ctrl}, key, cnt, n, (uint32_t)a.k, cand_k,
                          cand_i, [&](int i) { return order_key(src[i]); },
                          [&](uint32_t o, int c, uint32_t kv) {
                            ck[o] = max(kv, 1u);
                            ci[o] = s0 + c;
                          });
}

// Stage 2: one block per row selects among its nseg * seg_cap (<= 64 * NT)
// candidate slots.  Fused selection (row_count non-null): the slots come from
// the filtering indexer, and a row is selected only when every split kept all
// its candidates within its slots and at least k were found; otherwise it is
// flagged (flags[row] = 1) for the plain path.  Every row gets its flag.
template <int NT>
// With counts (row_count): a row whose split overflowed its slots, or that
// kept fewer than k keys, is flagged (flags[row] = 1, when flags is given)
// and left to the caller; with stream_scores (the rows' stored scores) the
// block selects such a row itself, by passes over the row.  Every launch
// passes all four arguments (launches through argument pointers do not
// apply defaults).
__global__ __launch_bounds__(NT) void topk_cand_kernel(TopkArgs a, const int32_t* row_count, int32_t* flags,
                                                       const float* stream_scores) {
  constexpr int EPT = 64;
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  __shared__ uint32_t cand_k[kCap];
  __shared__ int32_t cand_i[kCap];
  const int row = blockIdx.x;
  if (a.only_rows && !a.only_rows[row]) return;
  const int pos = a.q_start + row % a.Lq;
  const int n_row = min(pos + 1, a.Lk);
  int32_t* out = a.indices + (size_t)row * a.k;
  if (n_row <= a.k) {
    for (int i = threadIdx.x; i < a.k; i += NT) out[i] = i < n_row ? i : -1;
    if (flags && threadIdx.x == 0) flags[row] = 0;
    return;
  }
  int n_real = -1;  // with counts: the real candidates among the slots
  if (row_count) {
    if (threadIdx.x < 64) {
      int found = 0, over = 0;
      for (int sgi = threadIdx.x; sgi < a.nseg; sgi += 64) {
        const int c = row_count[(size_t)row * a.nseg + sgi];
        found += c;
        over |= c > a.seg_cap;
      }
      found = (int)wave_scan_add((uint32_t)found);
      over = __ballot(over) != 0;
      if (threadIdx.x == 63) {
        ctrl[3] = (over || found < a.k) ? 1u : 0u;
        ctrl[2] = (uint32_t)found;
      }
    }
    __syncthreads();
    const bool bad = ctrl[3] != 0;
    n_real = (int)ctrl[2];
    __syncthreads();
    if (flags && threadIdx.x == 0) flags[row] = bad ? 1 : 0;
    if (bad) {
      if (stream_scores) {
        const float* srow = stream_scores + (size_t)row * a.Lk;
        select_streamed<NT>(hist, scan_sh, ctrl, [&](int i) { return order_key(srow[i]); }, n_row,
                            (uint32_t)a.k, [&](uint32_t o, int c, uint32_t) { out[o] = c; });
      }
      return;
    }
  }
  const int n = a.nseg * a.seg_cap;
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
  select_top<EPT, NT>(BlockSelect<NT>{hist, scan_sh, ctrl}, key, cnt, n, (uint32_t)a.k, cand_k, cand_i,
                      [&](int i) { return ck[i]; },
                      [&](uint32_t o, int c, uint32_t) { out[o] = ci[c]; }, n_real);
}

// Segment plan of the two-stage path: nseg segments of kSeg keys (wide =
// false) or of kSegWide keys (wide = true); nseg = 0 when the row fits one
// block or no plan holds the candidates.
struct SegPlan {
  int nseg;
  bool wide;
};
// Measured on 8192 rows of 131K keys (k = 2048): narrow 3.92 ms, wide
// 2.04 ms; on 64 such rows: narrow 0.060 ms, wide 0.086 ms.
SegPlan topk_plan(long long rows, int Lq, int q_start, int Lk, int k) {
  const int max_n = min(q_start + Lq, Lk);
  if (max_n <= kCandMax || k % 4 != 0) return {0, false};
  const int narrow = (max_n + kSeg - 1) / kSeg;
  const int wide = (max_n + kSegWide - 1) / kSegWide;
  const bool wide_fits = (long long)wide * k <= kCandWide;
  if ((long long)narrow * k <= kCandMax && !(wide_fits && rows * wide >= kWideMinBlocks))
    return {narrow, false};
  if (wide_fits) return {wide, true};
  return {0, false};
}

// Threshold of the fused selection for one row (one block per row): over
// the row's sampled scores (keys s = stride * s'), an order key t with at
// least r samples >= t, r a few standard deviations above the sampled rank
// of the row's k-th largest key (as in select_top's own sample).  About
// r * stride of the row's keys are then >= t, at least k of them with
// overwhelming probability; the select kernel checks that.
template <int EPT, int NT>
__global__ __launch_bounds__(NT) void fused_threshold_kernel(const float* sample, uint32_t* thresh, int Lq, int Lk,
                                                             int q_start, int k, int stride, int ls) {
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  const int row = blockIdx.x;
  const int pos = q_start + row % Lq;
  const int n = min(pos + 1, Lk);
  if (n <= k) {
    if (threadIdx.x == 0) thresh[row] = 0u;
    return;
  }
  const int m = min(pos / stride + 1, ls);  // sampled keys s' with stride * s' <= pos
  // only counts matter here, so a thread holds the samples j * NT + tid
  // (coalesced loads); those below m are a prefix j < cnt of its slots
  const int tid = threadIdx.x;
  const int cnt = tid < m ? min(EPT, (m - tid + NT - 1) / NT) : 0;
  const float* src = sample + (size_t)row * ls + tid;
  uint32_t key[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) key[j] = j < cnt ? order_key(src[j * NT]) : 0u;
  const float qm = (float)k * (float)m / (float)n;
  const uint32_t r = min((uint32_t)m, (uint32_t)(qm + 4.0f * sqrtf(qm) + 8.0f));
  BlockSelect<NT> sel{hist, scan_sh, ctrl};
  const uint32_t t = sel.coarse_threshold(key, cnt, r);
  if (threadIdx.x == 0) thresh[row] = t;
}

// ---- Few long rows (decode): a sampled cut, a filter, and one exact select.
// The two-stage path spends most of its time in per-segment selections that
// keep a quarter of each segment; with few rows the chip is better used by
// (1) one block per row that takes a cut from a sample of the row, (2) a
// filter over every key that keeps those at or above the cut, in index
// order, into fixed slots per split of the row, and (3) the candidate select
// above (topk_cand_kernel with counts and flags), which checks the row and
// selects exactly.  A row whose split overflowed its slots, or that kept
// fewer than k keys, is flagged and redone by the two-stage path restricted
// to the flagged rows.  Exactness as for the fused selection: when at least
// k keys are >= t and all of them were kept, the k-th largest is >= t, so
// every selectable key (ties included) is a candidate, in index order.
constexpr int kRunLen = 64;       // sample: the first 64 keys of every 1024 (or more:
constexpr int kRunStride = 1024;  // the stride doubles until the sample fits the block)
constexpr int kCutSamples = 16 * 512;
__host__ __device__ inline int run_stride(int n) {
  int rs = kRunStride;
  while ((long long)((n + rs - 1) / rs) * kRunLen > kCutSamples) rs *= 2;
  return rs;
}
constexpr int kFiltSplit = 4096;  // keys per split of the filter (256 threads x 16)
constexpr int kFewRows = 256;

// Cut of one row from its sample (the keys rs j .. rs j + 63 below the row's
// length, read as 256-byte runs, rs = 1024 or the least power-of-two multiple
// that keeps the sample within the block), with the same rank rule as
// select_top's own sample; written as an order key.
template <int EPT, int NT>
__global__ __launch_bounds__(NT) void topk_sample_cut_kernel(TopkArgs a, uint32_t* thresh) {
  static_assert(EPT * NT == kCutSamples, "sample size");
  __shared__ uint32_t hist[kHist];
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  __shared__ uint32_t ctrl[4];
  const int row = blockIdx.x;
  const int pos = a.q_start + row % a.Lq;
  const int n = min(pos + 1, a.Lk);
  if (n <= a.k) {
    if (threadIdx.x == 0) thresh[row] = 0u;
    return;
  }
  const int rs = run_stride(n);
  const int full_runs = n / rs, tail = min(kRunLen, n - full_runs * rs);
  const int m = full_runs * kRunLen + tail;  // sampled keys, <= EPT * NT
  const float* src = a.scores + (size_t)row * a.Lk;
  const int tid = threadIdx.x;
  // sample s = j * NT + tid is key (s / 64) * rs + s % 64; those below m
  // are a prefix of the thread's slots
  const int cnt = tid < m ? min(EPT, (m - tid + NT - 1) / NT) : 0;
  uint32_t key[EPT];
#pragma unroll
  for (int j = 0; j < EPT; ++j) {
    const int sidx = j * NT + tid;
    key[j] = j < cnt ? order_key(src[(sidx / kRunLen) * rs + sidx % kRunLen]) : 0u;
  }
  const float qm = (float)a.k * (float)m / (float)n;
  const uint32_t r = min((uint32_t)m, (uint32_t)(qm + 4.0f * sqrtf(qm) + 8.0f));
  BlockSelect<NT> sel{hist, scan_sh, ctrl};
  const uint32_t t = sel.coarse_threshold(key, cnt, r);
  if (threadIdx.x == 0) thresh[row] = t;
}

// The keys >= the row's cut of one split (kFiltSplit keys, EPT per thread,
// contiguous), as (order key, index) in index order into the split's
// a.seg_cap slots; the rest of the slots are padded (key 0 below every kept
// key, which are stored as >= 1, index -1).  The split's count may exceed
// its slots; the select kernel then flags the row.
template <int EPT, int NT, bool VEC>
__global__ __launch_bounds__(NT) void topk_filter_kernel(TopkArgs a, const uint32_t* thresh, int32_t* row_count) {
  static_assert(EPT * NT == kFiltSplit, "one split per block");
  __shared__ uint32_t scan_sh[2 * (NT / 64) + 1];
  const int row = blockIdx.x / a.nseg, split = blockIdx.x % a.nseg;
  const int pos = a.q_start + row % a.Lq;
  const int n_row = min(pos + 1, a.Lk);
  const size_t slot0 = ((size_t)row * a.nseg + split) * a.seg_cap;
  uint32_t* ck = a.cand_key + slot0;
  int32_t* ci = a.cand_idx + slot0;
  const uint32_t t = thresh[row];
  const int base = split * kFiltSplit + EPT * (int)threadIdx.x;
  const int cnt = max(0, min(EPT, n_row - base));
  uint32_t key[EPT];
  load_keys<EPT, VEC>(a.scores + (size_t)row * a.Lk, base, cnt, key);
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < EPT; ++j) mine += j < cnt && key[j] >= t;
  uint32_t total;
  uint32_t o = block_inclusive_scan_n<NT>(mine, scan_sh, total) - mine;
#pragma unroll
  for (int j = 0; j < EPT; ++j)
    if (j < cnt && key[j] >= t) {
      if (o < (uint32_t)a.seg_cap) {
        ck[o] = max(key[j], 1u);
        ci[o] = base + j;
      }
      ++o;
    }
  for (int i = (int)min(total, (uint32_t)a.seg_cap) + (int)threadIdx.x; i < a.seg_cap; i += NT) {
    ck[i] = 0u;
    ci[i] = -1;
  }
  if (threadIdx.x == 0) row_count[(size_t)row * a.nseg + split] = (int32_t)total;
}

// Plan of the few-rows path (use = false where it does not apply).
struct CutPlan {
  bool use;
  int nsplit;  // filter splits per row
  int cap;     // candidate slots per split
};
CutPlan cut_plan(long long rows, int Lq, int q_start, int Lk, int k) {
  const int max_n = min(q_start + Lq, Lk);
  if (rows > kFewRows || max_n <= kCandMax || k % 4 != 0) return {false, 0, 0};
  // expected keys >= the cut in the longest row: r samples scaled by n / m
  const int rs = run_stride(max_n);
  const int runs = max_n / rs, tail = min(kRunLen, max_n - runs * rs);
  const double m = (double)runs * kRunLen + tail;
  const double qm = (double)k * m / max_n;
  const double expect = (qm + 4.0 * sqrt(qm) + 8.0) * max_n / m;
  const int nsplit = (max_n + kFiltSplit - 1) / kFiltSplit;
  int cap = 64;
  while (cap < 2.0 * expect / nsplit + 64.0) cap *= 2;
  if ((long long)nsplit * cap > kCandMax) return {false, 0, 0};
  return {true, nsplit, cap};
}

}  // namespace

// Few-rows path: the cuts and the split counts (each rounded to 256 bytes),
// then the splits' candidate slots.
static size_t round256(size_t n) { return (n + 255) / 256 * 256; }
static size_t cut_region_bytes(long long rows, const CutPlan& c) {
  return round256((size_t)rows * sizeof(uint32_t)) + round256((size_t)rows * c.nsplit * sizeof(int32_t)) +
         (size_t)rows * c.nsplit * c.cap * (sizeof(uint32_t) + sizeof(int32_t));
}

size_t topk_workspace_bytes(int B, int Lq, int q_start, int Lk, int k) {
  const long long rows = (long long)B * Lq;
  const int nseg = topk_plan(rows, Lq, q_start, Lk, k).nseg;
  const size_t two_stage = (size_t)rows * nseg * k * (sizeof(uint32_t) + sizeof(int32_t));
  const CutPlan c = cut_plan(rows, Lq, q_start, Lk, k);
  if (!c.use || nseg == 0) return two_stage;
  return cut_region_bytes(rows, c);
}

hipError_t launch_topk(const TopkArgs& args, hipStream_t stream) {
  TopkArgs a = args;
  const long long rows = (long long)a.B * a.Lq;
  const dim3 grid((unsigned)rows);
  const int max_n = min(a.q_start + a.Lq, a.Lk);
  if (max_n <= kCandMax) {
    // The prefix form re-reads its candidates' full keys from the row.  With
    // every row inside the candidate slots that row was just loaded and is
    // still in L2; longer rows have ~18 % of their keys as candidates, which
    // touch nearly every cache line of the row after L2 has dropped it (at
    // L = 32K: 4.2 GB read from the memory side against 2.2 GB for the full
    // keys, in the same time), so they keep the full keys in registers.
    const bool vec = a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0;
    if (vec && max_n <= kCap)
      return launch_kernel((const void*)topk_prefix_kernel<64, true, 512>, grid, dim3(512), 0, stream, a);
    return launch_kernel(vec ? (const void*)topk_reg_kernel<64, true, 512> : (const void*)topk_reg_kernel<64, false, 512>,
                         grid, dim3(512), 0, stream, a);
  }
  const SegPlan plan = topk_plan(rows, a.Lq, a.q_start, a.Lk, a.k);
  const CutPlan cut = cut_plan(rows, a.Lq, a.q_start, a.Lk, a.k);
  if (cut.use && plan.nseg > 0 && a.workspace && !a.only_rows) {
    // few long rows: cut, filter, exact select (a row the cut does not
    // settle is selected by the same block from its stored scores)
    uint8_t* region = (uint8_t*)a.workspace;
    uint32_t* thresh = (uint32_t*)region;
    int32_t* count = (int32_t*)(region + round256((size_t)rows * sizeof(uint32_t)));
    TopkArgs c = a;
    c.nseg = cut.nsplit;
    c.seg_cap = cut.cap;
    c.cand_key = (uint32_t*)((uint8_t*)count + round256((size_t)rows * cut.nsplit * sizeof(int32_t)));
    c.cand_idx = (int32_t*)(c.cand_key + (size_t)rows * cut.nsplit * cut.cap);
    const bool vec = a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0;
    hipError_t e = launch_kernel((const void*)topk_sample_cut_kernel<kCutSamples / 512, 512>, grid, dim3(512), 0, stream, c, thresh);
    if (e != hipSuccess) return e;
    e = launch_kernel(vec ? (const void*)topk_filter_kernel<16, 256, true> : (const void*)topk_filter_kernel<16, 256, false>,
                      dim3((unsigned)(rows * cut.nsplit)), dim3(256), 0, stream, c, (const uint32_t*)thresh,
                      count);
    if (e != hipSuccess) return e;
    int32_t* no_flags = nullptr;
    return launch_kernel((const void*)topk_cand_kernel<512>, grid, dim3(512), 0, stream, c, (const int32_t*)count,
                         no_flags, a.scores);
  }
  a.nseg = plan.nseg;
  if (a.nseg > 0 && a.workspace) {
    a.seg_cap = a.k;
    a.cand_key = (uint32_t*)a.workspace;
    a.cand_idx = (int32_t*)(a.cand_key + (size_t)rows * a.nseg * a.k);
    const bool vec = a.Lk % 4 == 0 && (uintptr_t)a.scores % 16 == 0;
    const dim3 sgrid((unsigned)(rows * a.nseg));
    hipError_t e;
    if (plan.wide)
      e = launch_kernel(vec ? (const void*)topk_seg_kernel<64, 512, true> : (const void*)topk_seg_kernel<64, 512, false>,
                        sgrid, dim3(512), 0, stream, a);
    else
      e = launch_kernel(vec ? (const void*)topk_seg_kernel<32, 256, true> : (const void*)topk_seg_kernel<32, 256, false>,
                        sgrid, dim3(256), 0, stream, a);
    if (e != hipSuccess) return e;
    const int32_t* no_count = nullptr;
    int32_t* no_flags = nullptr;
    const float* no_scores = nullptr;
    if ((long long)a.nseg * a.k > kCandMax)
      return launch_kernel((const void*)topk_cand_kernel<1024>, grid, dim3(1024), 0, stream, a, no_count, no_flags,
                           no_scores);
    return launch_kernel((const void*)topk_cand_kernel<512>, grid, dim3(512), 0, stream, a, no_count, no_flags,
                         no_scores);
  }
  const size_t base = (size_t)(kBins + kWaves + 1 + 4) * sizeof(uint32_t);
  return launch_kernel((const void*)topk_kernel, grid, dim3(kThreads), base, stream, a);
}

FusedPlan fused_plan(int B, int Lq, int Lk, int q_start, int HI, int dI, int k) {
  FusedPlan f{};
  const int max_n = min(q_start + Lq, Lk);
  // Only where the plain path would take the two-stage top-k (rows longer
  // than one block's candidate capacity): up to that length the one-pass
  // select reads the written scores faster than the sampling, threshold and
  // filtering passes cost.  The filtering indexer runs the prefill shape.
  if (Lq < 8 || max_n <= kCandMax || max_n <= 2 * k) return f;
  f.stride = 16;
  // at most 16384 sampled keys per row: the sampled pass and the threshold
  // cost little next to the filtering pass (up to 32768 fit one block)
  while ((long long)f.stride * 16384 < max_n) f.stride *= 2;
  f.ls = (max_n + f.stride - 1) / f.stride;  // sampled keys any row reaches (<= 32768)
  IndexArgs a{};
  a.B = B; a.Lq = Lq; a.Lk = Lk; a.q_start = q_start; a.HI = HI; a.dI = dI; a.key_stride = 1;
  f.n_splits = index_splits(a);
  // expected candidates of a long row: r * stride (the threshold kernel's r
  // for the longest row), spread over the splits; twice that per split plus
  // 64, rounded up to a power of two (at least 256).  The margin covers the
  // threshold's coarseness: it is the lower edge of a digit bin, so up to a
  // few times r samples can lie above it.
  const float m = (float)((max_n - 1) / f.stride + 1);
  const float qm = (float)k * m / (float)max_n;
  const float expect = (qm + 4.0f * sqrtf(qm) + 8.0f) * (float)f.stride;
  const float per_split = 2.0f * expect / (float)f.n_splits + 64.0f;
  int cap = 256;
  while (cap < per_split) cap *= 2;
  f.cap_s = cap;
  f.use = (long long)f.n_splits * cap <= kCandWide;
  return f;
}

hipError_t launch_fused_threshold(const float* sample, uint32_t* thresh, int B, int Lq, int Lk, int q_start, int k,
                                  int stride, int ls, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)B * Lq));
  if (ls <= 2048)
    return launch_kernel((const void*)fused_threshold_kernel<16, 128>, grid, dim3(128), 0, stream, sample, thresh,
                         Lq, Lk, q_start, k, stride, ls);
  if (ls <= 8192)
    return launch_kernel((const void*)fused_threshold_kernel<32, 256>, grid, dim3(256), 0, stream, sample, thresh,
                         Lq, Lk, q_start, k, stride, ls);
  if (ls <= 32768)
    return launch_kernel((const void*)fused_threshold_kernel<64, 512>, grid, dim3(512), 0, stream, sample, thresh,
                         Lq, Lk, q_start, k, stride, ls);
  return hipErrorInvalidValue;
}

hipError_t launch_fused_select(const TopkArgs& a, const int32_t* row_count, int32_t* flags, hipStream_t stream) {
  const dim3 grid((unsigned)((long long)a.B * a.Lq));
  const float* no_scores = nullptr;  // flagged rows go back to the caller
  const long long n = (long long)a.nseg * a.seg_cap;
  if (n <= kCandMax)
    return launch_kernel((const void*)topk_cand_kernel<512>, grid, dim3(512), 0, stream, a, row_count, flags,
                         no_scores);
  if (n <= kCandWide)
    return launch_kernel((const void*)topk_cand_kernel<1024>, grid, dim3(1024), 0, stream, a, row_count, flags,
                         no_scores);
  return hipErrorInvalidValue;
}

}  // namespace dsa
