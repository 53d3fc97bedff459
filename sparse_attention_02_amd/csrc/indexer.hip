// Lightning indexer on gfx950 FP8 matrix cores.
//
// I[b,t,s] = sum_j w[b,t,j] * ReLU(q_I[b,t,j,:] . k_I[b,s,:]) for s <= pos(t)
// ("DeepSeek V3.2 and the lightning indexer", section "How the lightning
// indexer works"; DeepSeek-V3.2 spec sheet, section 2.1: a few indexer heads,
// weighted sum of ReLU'd dot products, FP8, one key per preceding token).
//
// Mapping.  The contraction runs as a GEMM whose rows are (query, head) pairs
// and whose columns are keys: one v_mfma_f32_16x16x128_f8f6f4 multiplies 16
// heads of one query by 16 keys over the whole d_I = 128 (shorter d_I is zero
// padded).  The product sums over d, so the d-bytes may be dealt to the lanes
// in any order both operands share.  Decode deals lane group g the bytes
// [32g, 32g+32) and keeps 144-byte padded key rows in LDS; prefill deals it
// [16g, 16g+16) and [64+16g, 64+16g+16) over 128-byte rows whose 16-byte
// pieces are XOR-swizzled by (row & 7), which spreads a wave's key reads
// evenly over the 64 LDS banks (the contiguous order runs them 2-way
// conflicted).  Decode keeps the contiguous order: the swizzled one needs a
// second read address per key tile, and the decode variant has no register
// left for it.  Each lane then owns 4 heads x 1 key of the 16x16 result, applies
// the ReLU and the head weight in registers and keeps a running partial sum;
// partial sums over the four lane groups are combined with two butterfly
// exchanges that also spread the 4 key tiles so that lane l ends with key l of
// the 64-key stage.  The score row is then written with one coalesced 256-byte
// store per query.
//
// Work split.  A block of 4 waves owns a tile of consecutive query rows of one
// sequence and walks the keys 0 .. (last position of the tile) in stages:
//  - prefill (NKL = 1): 4 waves x 1 query; every wave reads the same 64-key
//    stage from LDS, so each key byte fetched from L2 feeds 4 queries.  One
//    query per wave keeps a wave at ~96 registers, so 5 waves share a SIMD
//    and hide each other's MFMA -> epilogue latency (the epilogue's VALU work
//    is as long as the MFMA work, so neither pipe may wait on the other).
//  - decode  (NKL = 4): 4 waves x 2 queries of one query group; the waves take
//    4 different 64-key slices of a 256-key stage (nothing to share between
//    queries).
// Key stages are double-buffered in LDS; the next stage's global loads are in
// flight while the current one is multiplied.  The causal triangle is skipped
// at stage granularity; keys past a row's position are computed but not
// stored.  Blocks are ordered longest-first so the triangle's long rows start
// early, and long key ranges can be split over several blocks.
#include "dsa_common.h"
#include "launch.h"

#include <algorithm>

namespace dsa {

namespace {

constexpr int kPrefillWaves = 4, kPrefillQPW = 1;
constexpr int kDecodeWaves = 4, kDecodeQPW = 2;
constexpr int kKeysPerWave = 64;

// NHG = number of 16-head groups (H_I <= 16 * NHG; absent heads have zero
// queries and weights).  A compile-time count keeps the MFMA sequence free of
// branches, so the 2 * NHG products of a key tile are issued back to back into
// separate accumulators before their epilogues read them.
// FULLD: d_I == 128, every lane group's 32 bytes are present.
// ReLU as a single v_max_f32.  This file is compiled without NaN semantics
// (the scores of NaN inputs are undefined): with them, fmaxf(x, 0) costs two
// VALU operations (a NaN-quieting canonicalisation of x, then the max), and
// the epilogue's VALU work already matches the matrix work.  A zero of either
// sign may come out; it only ever multiplies a head weight into a sum that
// starts at +0.
__device__ __forceinline__ float relu(float x) { return fmaxf(x, 0.0f); }

// MODE 0: every key, scores written at [row, key].  MODE 1 (sampling): the
// keys key_stride * s', scores at [row * out_ld + s'].  MODE 2 (filtering):
// every key, and instead of the scores the candidates at or above the row's
// threshold (IndexArgs, "Filtering").  Modes 1 and 2 run the prefill shape
// (one query per wave); the stride is a compile-time 1 outside mode 1, so the
// plain kernel's address arithmetic stays as simple as it can be.
template <int NKL, int NHG, bool FULLD, int NW, int kQPW, int MODE>
__global__ __launch_bounds__(64 * NW) void index_scores_kernel(IndexArgs a) {
  constexpr bool FILTER = MODE == 2;
  constexpr bool SAMPLED = MODE == 1;
  static_assert(MODE == 0 || (NKL == 1 && kQPW == 1), "sampling and filtering run one query per wave");
  constexpr int kThreads = 64 * NW;
  constexpr int NQG = NW / NKL;         // query groups per block
  constexpr int QT = kQPW * NQG;        // queries per block
  constexpr int KS = kKeysPerWave * NKL;  // keys per stage
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int g = lane >> 4;              // lane group: k-bytes [32g, 32g+32)
  const int qgroup = wave % NQG;
  const int klane = wave / NQG;

  const int bid = blockIdx.x;
  const int split = bid % a.n_splits;
  const int rest = bid / a.n_splits;
  const int b = rest % a.B;
  const int tile = a.n_qtiles - 1 - rest / a.B;

  const int t_first = tile * QT;
  const int t_last = min(t_first + QT, a.Lq) - 1;
  if (a.only_rows) {
    bool any = false;
    for (int t = t_first; t <= t_last; ++t) any |= a.only_rows[(size_t)b * a.Lq + t] != 0;
    if (!any) return;
  }
  // keys are s = stride * s' for s' < ls; a tile needs s' <= (its last position) / stride
  const int stride = SAMPLED ? a.key_stride : 1;
  const int out_ld = SAMPLED ? a.out_ld : a.Lk;
  const int ls = (a.Lk + stride - 1) / stride;
  const int kv_end = min(ls, (a.q_start + t_last) / stride + 1);
  const int nst_total = (kv_end + KS - 1) / KS;
  const int st_begin = (int)((long long)nst_total * split / a.n_splits);
  const int st_end = (int)((long long)nst_total * (split + 1) / a.n_splits);
  if (st_begin >= st_end) {
    if constexpr (FILTER) {  // an empty split still reports: no candidates
      const int t = t_first + qgroup * kQPW;
      if (t < a.Lq) {
        const size_t r = (size_t)b * a.Lq + t;
        for (int j = lane; j < a.cap_s; j += 64) {
          a.cand_key[(r * a.n_splits + split) * a.cap_s + j] = 0u;
          a.cand_idx[(r * a.n_splits + split) * a.cap_s + j] = -1;
        }
        if (lane == 0) a.row_count[r * a.n_splits + split] = 0;
      }
    }
    return;
  }

  const int dI = a.dI;
  constexpr bool SWZ = NKL == 1;        // prefill: swizzled 128-byte rows (see above)
  const int row_bytes = SWZ ? 128 : dI + 16;
  const int stage_bytes = KS * row_bytes;
  // d-bytes of this lane group: [off_lo, off_lo + 16) and [off_hi, off_hi + 16)
  const int off_lo = SWZ ? 16 * g : 32 * g;
  const int off_hi = SWZ ? 64 + 16 * g : 32 * g + 16;
  const bool lo_ok = FULLD || off_lo < dI;
  const bool hi_ok = FULLD || off_hi < dI;

  // ---- A operands (query heads) and head weights, resident for the whole block
  v8i qa[kQPW][NHG];
  float wr[kQPW][NHG][4];
#pragma unroll
  for (int q = 0; q < kQPW; ++q) {
    const int t = t_first + qgroup * kQPW + q;
#pragma unroll
    for (int hg = 0; hg < NHG; ++hg) {
      const int head = 16 * hg + (lane & 15);
      v8i v = {0, 0, 0, 0, 0, 0, 0, 0};
      if (t < a.Lq && head < a.HI) {
        const uint8_t* src = a.q_idx + (((size_t)b * a.Lq + t) * a.HI + head) * dI;
        const v4i zero = {0, 0, 0, 0};
        const v4i lo = lo_ok ? *(const v4i*)(src + off_lo) : zero;
        const v4i hi = hi_ok ? *(const v4i*)(src + off_hi) : zero;
        v = (v8i){lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      }
      qa[q][hg] = v;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int h = 16 * hg + 4 * g + r;
        wr[q][hg][r] = (t < a.Lq && h < a.HI) ? a.w[((size_t)b * a.Lq + t) * a.HI + h] : 0.0f;
      }
    }
  }

  // ---- stage loader: KS keys x dI bytes, 16-byte pieces spread over the block
  const int pieces_per_row = dI >> 4;
  const int stage_pieces = KS * pieces_per_row;
  constexpr int kMaxPieces = (KS * 8 + kThreads - 1) / kThreads;  // dI <= 128
  const uint8_t* kseq = a.k_idx + (size_t)b * a.Lk * dI;
  v4i pf[kMaxPieces];

  auto load_stage = [&](int st) {
    const int kbase = st * KS;
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      const int p = threadIdx.x + j * kThreads;
      if (p < stage_pieces) {
        const int key = min(kbase + p / pieces_per_row, ls - 1);
        pf[j] = *(const v4i*)(kseq + (size_t)key * stride * dI + 16 * (p % pieces_per_row));
      }
    }
  };
  auto store_stage = [&](int buf) {
    uint8_t* dst = smem + buf * stage_bytes;
#pragma unroll
    for (int j = 0; j < kMaxPieces; ++j) {
      const int p = threadIdx.x + j * kThreads;
      if (p < stage_pieces) {
        const int r = p / pieces_per_row, q = p % pieces_per_row;
        *(v4i*)(dst + r * row_bytes + 16 * (SWZ ? q ^ (r & 7) : q)) = pf[j];
      }
    }
  };

  // last (sampled) key of each query row: s' <= lim, or none for absent rows
  int lim[kQPW];
#pragma unroll
  for (int q = 0; q < kQPW; ++q) {
    const int t = t_first + qgroup * kQPW + q;
    lim[q] = t < a.Lq ? min(ls - 1, (a.q_start + t) / stride) : -1;
  }
  // filtering: this wave's threshold (as the score whose order key it is: a
  // score passes iff it is >= that value, -0 and +0 alike) and candidate slots
  int cursor = 0;
  float thr = __builtin_nanf("");
  uint32_t* fck = nullptr;
  int32_t* fci = nullptr;
  const int frow_t = t_first + qgroup * kQPW;
  if constexpr (FILTER) {
    if (frow_t < a.Lq) {
      const size_t r = (size_t)b * a.Lq + frow_t;
      const uint32_t tk = a.thresh[r];
      thr = __uint_as_float((tk & 0x80000000u) ? (tk & 0x7FFFFFFFu) : ~tk);
      fck = a.cand_key + (r * a.n_splits + split) * a.cap_s;
      fci = a.cand_idx + (r * a.n_splits + split) * a.cap_s;
    }
  }

  load_stage(st_begin);
  store_stage(0);
  // The operand loads above sit in branches, so the compiler cannot prove
  // they are complete when the loop starts; without this wait it drains every
  // outstanding load, the next stage's prefetch included, before the first
  // matrix product of each stage (13 % of the decode time).
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  for (int st = st_begin; st < st_end; ++st) {
    const int buf = (st - st_begin) & 1;
    if (st + 1 < st_end) load_stage(st + 1);

    const uint8_t* sb = smem + buf * stage_bytes;
    float part[kQPW][4];
#pragma unroll
    for (int q = 0; q < kQPW; ++q)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) part[q][kt] = 0.0f;

#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const int key_local = kKeysPerWave * klane + 16 * kt + (lane & 15);
      // With d_I < 128, pieces past d_I are read from within the row (stale
      // bytes, or the row's first bytes) and replaced by zeros (stale bytes
      // could be FP8 NaNs, and 0 * NaN is NaN).  Swizzled rows: pieces g and
      // g + 4 of row key_local, whose & 7 is lane & 7.
      const uint8_t* row = sb + key_local * row_bytes;
      v4i lo, hi4;
      if constexpr (SWZ) {
        const int o = 16 * (g ^ (lane & 7));
        lo = *(const v4i*)(row + o);
        hi4 = *(const v4i*)(row + (o ^ 64));
      } else {
        const v4i* s4 = (const v4i*)(row + (lo_ok ? off_lo : 0));
        lo = s4[0];
        hi4 = s4[1];
      }
      if (!lo_ok) lo = (v4i){0, 0, 0, 0};
      if (!hi_ok) hi4 = (v4i){0, 0, 0, 0};
      const v8i kb = (v8i){lo[0], lo[1], lo[2], lo[3], hi4[0], hi4[1], hi4[2], hi4[3]};
      v4f x[kQPW][NHG];
#pragma unroll
      for (int q = 0; q < kQPW; ++q)
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
          x[q][hg] = mfma_f8_16x16x128(qa[q][hg], kb, (v4f){0.0f, 0.0f, 0.0f, 0.0f});
#pragma unroll
      for (int q = 0; q < kQPW; ++q)
#pragma unroll
        for (int hg = 0; hg < NHG; ++hg)
#pragma unroll
          for (int r = 0; r < 4; ++r) part[q][kt] += wr[q][hg][r] * relu(x[q][hg][r]);
    }

    // ---- head-group reduction + key-tile spread, then the store
    const int key = st * KS + kKeysPerWave * klane + lane;
#pragma unroll
    for (int q = 0; q < kQPW; ++q) {
      // v_permlane32_swap(x, y) trades the upper half of x for the lower half
      // of y, so x' + y' is, in lanes 0..31, key tile 0 summed over lane groups
      // g and g^2 and, in lanes 32..63, the same for tile 2 (tiles 1 and 3
      // likewise).  permlane16_swap then adds groups g and g^1 and leaves
      // lane l with key l of the stage.
      const auto a02 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[q][0]),
                                                        __float_as_uint(part[q][2]), false, false);
      const auto a13 = __builtin_amdgcn_permlane32_swap(__float_as_uint(part[q][1]),
                                                        __float_as_uint(part[q][3]), false, false);
      const float k0 = __uint_as_float(a02[0]) + __uint_as_float(a02[1]);
      const float k1 = __uint_as_float(a13[0]) + __uint_as_float(a13[1]);
      const auto b01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(k0), __float_as_uint(k1), false, false);
      const float fin = __uint_as_float(b01[0]) + __uint_as_float(b01[1]);
      const int t = t_first + qgroup * kQPW + q;
      const bool valid = key <= lim[q];
      if constexpr (FILTER) {
        // the row's keys >= its threshold, in ascending index order
        const bool keep = valid && fin >= thr;
        const uint64_t m = __ballot(keep);
        if (m) {
          const int slot = cursor + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                                   __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
          if (keep && slot < a.cap_s) {
            fck[slot] = max(order_key(fin), 1u);
            fci[slot] = key;
          }
          cursor += __builtin_popcountll(m);
        }
      } else if (valid) {
        a.scores[((size_t)b * a.Lq + t) * out_ld + key] = fin;
      }
    }

    if (st + 1 < st_end) store_stage(buf ^ 1);
    __syncthreads();
  }
  if constexpr (FILTER) {
    if (frow_t < a.Lq) {
      for (int j = min(cursor, a.cap_s) + lane; j < a.cap_s; j += 64) {
        fck[j] = 0u;
        fci[j] = -1;
      }
      if (lane == 0) a.row_count[((size_t)b * a.Lq + frow_t) * a.n_splits + split] = cursor;
    }
  }
}

}  // namespace

// Long key ranges are split over several blocks.  The splits write disjoint
// key ranges, but each one pays its own prologue (query operands, head
// weights, a first stage load that nothing hides), so a split is worth it
// only while the chip is under-filled or the grid's last round is.
//  - decode: one round of resident blocks (a 256-key stage pair takes
//    ~74 KB of LDS, so two blocks per CU): more rounds only add prologues.
//  - prefill: first at least two rounds (~5 blocks per CU) while a split
//    keeps >= 16 stages; then, because rows of equal length (chunked
//    prefill) end together and leave the last round part-empty, up to 32768
//    blocks while a split keeps >= 256 stages.  Causal rows from position 0
//    need no such help: their lengths differ and the longest start first.
// Measured on the 64 x 128 indexer: decode over 64 x 128K keys is fastest at
// 8 splits, over 4 x 1M at 128; prefill over 4K at 2, over 32K at 1, 8K new
// tokens of 128K at 4-8, 4K of 1M at 32.  With key sampling the stages are
// counted in sampled keys.
int index_splits(const IndexArgs& a) {
  const bool decode = a.Lq < 8;
  const int QT = decode ? kDecodeQPW * kDecodeWaves / 4 : kPrefillQPW * kPrefillWaves;
  const int KS = decode ? 4 * kKeysPerWave : kKeysPerWave;
  const int stride = a.key_stride;
  const long long n_qtiles = (a.Lq + QT - 1) / QT;
  const long long tiles = (long long)a.B * n_qtiles;
  const int ls = (a.Lk + stride - 1) / stride;
  const int max_st = (ls + KS - 1) / KS;
  // stages of an average tile: a tile's keys end at its last position
  const long long avg_st = (((long long)a.q_start + (a.Lq + 1) / 2) / stride + KS - 1) / KS;
  int splits = 1;
  auto grow = [&](long long blocks, long long min_stages) {
    while (tiles * splits < blocks && splits * 2 <= max_st && avg_st >= 2LL * splits * min_stages)
      splits *= 2;
  };
  if (decode) {
    const long long per_cu = std::max<long long>(1, (160 * 1024) / (2LL * KS * (a.dI + 16)));
    grow(256 * per_cu, 8);
  } else {
    grow(2 * 256 * 5, 16);
    grow(32768, 256);
  }
  return splits;
}

hipError_t launch_index_scores(const IndexArgs& args_in, hipStream_t stream) {
  IndexArgs a = args_in;
  const bool decode = a.Lq < 8;
  const bool filter = a.thresh != nullptr;
  const bool sampled = a.key_stride != 1;
  if ((filter || sampled) && decode) return hipErrorInvalidValue;
  if (filter && sampled) return hipErrorInvalidValue;
  const int QT = decode ? kDecodeQPW * kDecodeWaves / 4 : kPrefillQPW * kPrefillWaves;
  const int KS = decode ? 4 * kKeysPerWave : kKeysPerWave;
  a.n_qtiles = (a.Lq + QT - 1) / QT;
  // a filtering launch uses the split count its candidate slots were sized for
  if (!filter) a.n_splits = index_splits(a);
  const size_t smem = 2 * (size_t)KS * (decode ? a.dI + 16 : 128);  // two stages of key rows
  const dim3 grid((unsigned)((long long)a.B * a.n_qtiles * a.n_splits));
  const int nhg = (a.HI + 15) >> 4;
  const bool full = a.dI == 128;
#define DSA_K1(NKL, NHG, NW, QPW, F)                                    \
  (full ? (const void*)index_scores_kernel<NKL, NHG, true, NW, QPW, F> \
        : (const void*)index_scores_kernel<NKL, NHG, false, NW, QPW, F>)
  const void* kern;
  int threads;
  if (decode) {
    threads = 64 * kDecodeWaves;
    kern = nhg == 1   ? DSA_K1(4, 1, kDecodeWaves, kDecodeQPW, 0)
           : nhg == 2 ? DSA_K1(4, 2, kDecodeWaves, kDecodeQPW, 0)
                      : DSA_K1(4, 4, kDecodeWaves, kDecodeQPW, 0);
  } else if (filter) {
    threads = 64 * kPrefillWaves;
    kern = nhg == 1   ? DSA_K1(1, 1, kPrefillWaves, kPrefillQPW, 2)
           : nhg == 2 ? DSA_K1(1, 2, kPrefillWaves, kPrefillQPW, 2)
                      : DSA_K1(1, 4, kPrefillWaves, kPrefillQPW, 2);
  } else if (sampled) {
    threads = 64 * kPrefillWaves;
    kern = nhg == 1   ? DSA_K1(1, 1, kPrefillWaves, kPrefillQPW, 1)
           : nhg == 2 ? DSA_K1(1, 2, kPrefillWaves, kPrefillQPW, 1)
                      : DSA_K1(1, 4, kPrefillWaves, kPrefillQPW, 1);
  } else {
    threads = 64 * kPrefillWaves;
    kern = nhg == 1   ? DSA_K1(1, 1, kPrefillWaves, kPrefillQPW, 0)
           : nhg == 2 ? DSA_K1(1, 2, kPrefillWaves, kPrefillQPW, 0)
                      : DSA_K1(1, 4, kPrefillWaves, kPrefillQPW, 0);
  }
#undef DSA_K1
  if (smem > 64 * 1024) {
    const hipError_t attr =
        hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (attr != hipSuccess) return attr;
  }
  return launch_kernel(kern, grid, dim3(threads), smem, stream, a);
}

}  // namespace dsa
