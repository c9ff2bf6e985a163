// bq_table.cpp -- host-side preparation of a code table for the quantize kernels.
//
// Validates the table, builds the exact decision thresholds T_k, the zero code z, and the
// bucket LUT that lets the kernels find the nearest code with one LDS read and at most M
// compares per element.  All of it is plain integer / binary32 / binary64 arithmetic, done
// per call (a 256-entry table takes a few microseconds) and handed to the kernels by value.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <vector>

#include "bq_internal.h"

namespace bq {
namespace {

// Smallest binary32 value strictly greater than the binary64 value m.
float next_float_above(double m) {
  float f = (float)m;  // round to nearest
  if ((double)f > m) return f;
  return nextafterf(f, INFINITY);
}

// Number of thresholds T_k <= y (thresholds ascending).
int count_le(const std::vector<float>& thr, float y) {
  return (int)(std::upper_bound(thr.begin(), thr.end(), y) - thr.begin());
}

// LIN bucket of y in [-1, 1] with H buckets of width 2/H: fma(y, H/2, 2^23 + H/2) rounded to
// nearest (correctly rounded, as v_fma_f32) is the integer 2^23 + idx.
uint32_t lin_bucket(float y, int H) {
  const float zz = fmaf(y, 0.5f * (float)H, 8388608.0f + 0.5f * (float)H);
  return f32_bits(zz) - kLinBits;
}

// Bits of binary16(y) rounded toward zero, as v_cvt_pkrtz_f16_f32 (finite |y| < 65520; the
// kernels only convert y in [-1, 1]).  Subnormal binary16 results are kept.
uint32_t f16_rtz_bits(float y) {
  const uint32_t u = f32_bits(y);
  const uint32_t sign = (u >> 16) & 0x8000u;
  const int e = (int)((u >> 23) & 0xff) - 127;  // exponent of a normal binary32 value
  const uint32_t mant = u & 0x7fffffu;
  if (((u >> 23) & 0xff) == 0) return sign;     // zero or binary32 subnormal: below 2^-126
  if (e >= -14) return sign | ((uint32_t)(e + 15) << 10) | (mant >> 13);
  const int sh = -1 - e;                          // subnormal binary16: (2^23 + mant) * 2^(e + 1) / 2^23 * 2^24
  return sign | (sh >= 24 ? 0u : ((0x800000u | mant) >> sh));
}

// F16B bucket of y (see bq_internal.h): the sign moved from bit 15 to bit 14, then >> 4.
int f16b_bucket(float y) {
  const uint32_t h = f16_rtz_bits(y);
  return (int)((((h & 0x3ff0u) | ((h & 0x8000u) >> 1))) >> 4);
}

struct LogParams {
  int sh;
  uint32_t lo, hi;
  int nj;
};

LogParams log_params(int sh, int e) {
  LogParams p;
  p.sh = sh;
  p.lo = (uint32_t)(127 - e) << 23;  // bits of 2^-e
  p.hi = 0x3f800000u + (1u << sh);
  p.nj = (int)((0x3f800000u - p.lo) >> sh) + 2;
  return p;
}

// Monotone rank of the LOG bucket holding y (finite y).
int log_rank(float y, const LogParams& p) {
  uint32_t u = f32_bits(y);
  uint32_t a = u & 0x7fffffffu;
  uint32_t t = std::min(std::max(a, p.lo), p.hi);
  int j = (int)((t - p.lo) >> p.sh);
  return (u >> 31) ? (p.nj - 1 - j) : (p.nj + j);
}

// Per-bucket base and the largest number of thresholds sharing a bucket, from the rank of
// every threshold's bucket.  rank_of_idx maps a LUT index to its rank.
template <typename RankOfIdx>
int fill_lut(const std::vector<int>& thr_rank, int nranks, int nidx, RankOfIdx rank_of_idx,
             int special0, int special1, int z, uint8_t* base) {
  std::vector<int> cnt(nranks + 1, 0);
  for (int r : thr_rank) cnt[r]++;
  std::vector<int> below(nranks + 1, 0);
  for (int r = 1; r <= nranks; ++r) below[r] = below[r - 1] + cnt[r - 1];
  int M = 0;
  for (int idx = 0; idx < nidx; ++idx) {
    if (idx == special0 || idx == special1) {
      base[idx] = (uint8_t)z;
      continue;
    }
    int r = rank_of_idx(idx);
    base[idx] = (uint8_t)below[r];
    M = std::max(M, cnt[r]);
  }
  return M;
}

}  // namespace

bool prepare_table(const float* entries, int size, PreparedTable* out) {
  if (entries == nullptr || (size != 16 && size != 256)) return false;
  float c[256];
  for (int k = 0; k < size; ++k) {
    float v = entries[k];
    if (!isfinite(v) || v < -1.0f || v > 1.0f) return false;
    if (v == 0.0f) v = 0.0f;  // -0.0 reads as +0.0
    if (v != 0.0f && fabsf(v) < 0x1p-20f) return false;
    if (k > 0 && !(v > c[k - 1])) return false;
    c[k] = v;
  }
  memset(out, 0, sizeof(*out));
  out->K = size;
  memcpy(out->c, c, sizeof(float) * size);

  // Thresholds: midpoints are exact in binary64 (entries are multiples of 2^-43, |c| <= 1).
  std::vector<float> thr(size - 1);
  for (int k = 0; k + 1 < size; ++k) thr[k] = next_float_above(((double)c[k] + (double)c[k + 1]) * 0.5);
  QuantArgs& qa = out->qa;
  for (int k = 0; k < 260; ++k) qa.thr[k] = k < size - 1 ? thr[k] : NAN;
  qa.K = size;
  qa.z = count_le(thr, 0.0f);

  // Candidate bucketings; cost ~ VALU instructions per element.
  struct Choice { int mode, M, sh, nidx; LogParams lp; uint8_t base[kLutMax]; };
  Choice best;
  best.mode = SEARCH;
  best.M = 0;
  int best_cost = 4 * (size == 16 ? 4 : 8) + 2;

  // Uniform buckets, the fewest that keep the compares per element lowest (a smaller LUT is
  // cheaper to build in every workgroup).  Thresholds lie in (-1, 1], in buckets 0..H.
  for (int H : {64, 128, 256, 512}) {
    if (H + 1 > kLinLutMax) continue;
    std::vector<int> ranks(size - 1);
    for (int k = 0; k + 1 < size; ++k) ranks[k] = (int)lin_bucket(thr[k], H);
    Choice ch;
    ch.mode = LIN;
    ch.sh = H;
    ch.nidx = H + 1;
    ch.M = fill_lut(ranks, H + 1, H + 1, [](int idx) { return idx; }, -1, -1, qa.z, ch.base);
    int cost = 2 + 2 * ch.M;
    if (ch.M <= 3 && cost < best_cost) { best = ch; best_cost = cost; }
  }
  for (auto se : {std::pair<int, int>{17, 16}, std::pair<int, int>{18, 16}, std::pair<int, int>{18, 24},
                  std::pair<int, int>{17, 12}}) {
    LogParams lp = log_params(se.first, se.second);
    if (2 * lp.nj > kLutMax) continue;
    std::vector<int> ranks(size - 1);
    for (int k = 0; k + 1 < size; ++k) ranks[k] = log_rank(thr[k], lp);
    Choice ch;
    ch.mode = LOG;
    ch.sh = lp.sh;
    ch.lp = lp;
    ch.nidx = 2 * lp.nj;
    int nj = lp.nj;
    ch.M = fill_lut(ranks, 2 * nj, 2 * nj,
                    [nj](int idx) { return idx >= nj ? nj - 1 - (idx - nj) : nj + idx; },
                    nj - 1, 2 * nj - 1, qa.z, ch.base);
    int cost = 6 + 2 * ch.M;
    if (ch.M <= 3 && cost < best_cost) { best = ch; best_cost = cost; }
  }

  // binary16 buckets: one compare per element and a three-operation offset per pair.
  {
    std::vector<int> ranks(size - 1);
    // rank in y order: negative buckets (largest index = most negative) first, then positive
    auto rank_of_idx = [](int idx) { return idx >= kF16NegLo ? kF16Size - 1 - idx : kF16Pos + idx; };
    bool ok = true;
    for (int k = 0; k + 1 < size; ++k) {
      const int idx = f16b_bucket(thr[k]);
      if (!(idx < kF16Pos || (idx >= kF16NegLo && idx < kF16Size))) ok = false;
      ranks[k] = ok ? rank_of_idx(idx) : 0;
    }
    if (ok) {
      std::vector<uint8_t> full(kF16Size, 0);
      const int nr = 2 * kF16Pos;
      std::vector<int> cnt(nr + 1, 0), below(nr + 1, 0);
      for (int r : ranks) cnt[r]++;
      for (int r = 1; r <= nr; ++r) below[r] = below[r - 1] + cnt[r - 1];
      int M = 0;
      for (int r = 0; r < nr; ++r) M = std::max(M, cnt[r]);
      const int cost = 2 + 2 * M;
      if (M == 1 && cost < best_cost) {
        Choice ch;
        ch.mode = F16B;
        ch.M = 1;
        ch.sh = 4;
        ch.nidx = kF16Size;
        memset(ch.base, 0, sizeof(ch.base));
        for (int idx = 0; idx < kF16Pos; ++idx) ch.base[idx] = (uint8_t)below[rank_of_idx(idx)];
        for (int idx = kF16NegLo; idx < kF16Size; ++idx) ch.base[idx - kF16NegBase] = (uint8_t)below[rank_of_idx(idx)];
        best = ch;
        best_cost = cost;
      }
    }
  }

  out->mode = best.mode;
  out->M = best.M;
  if (best.mode == LIN) {
    const int H = best.sh;
    const int e = best.M <= 1 ? 3 : 4;  // log2 of the LUT entry size (uint2 or uint4)
    qa.lin_scale = 0.5f * (float)H;
    qa.lin_bias = 8388608.0f + 0.5f * (float)H;
    qa.lin_off = 0u - (kLinBits << e);
    qa.nbuckets = H + 1;
    qa.special0 = qa.special1 = -1;  // y is always in [-1, 1]: no bucket for non-finite values
    memcpy(qa.base, best.base, (size_t)qa.nbuckets);
  } else if (best.mode == LOG) {
    qa.sh = best.lp.sh;
    qa.lo = best.lp.lo;
    qa.hi = best.lp.hi;
    qa.nj = best.lp.nj;
    const int e = best.M == 1 ? 3 : 4;  // log2 of the LUT entry size (uint2 or uint4)
    qa.jlo = qa.lo >> qa.sh;
    qa.jhi = qa.hi >> qa.sh;
    qa.log_bias = 0u - (qa.jlo << e);
    qa.log_nbias = qa.log_bias + ((uint32_t)qa.nj << e);
    qa.nbuckets = 2 * best.lp.nj;
    qa.special0 = best.lp.nj - 1;
    qa.special1 = 2 * best.lp.nj - 1;
    memcpy(qa.base, best.base, (size_t)qa.nbuckets);
  } else if (best.mode == F16B) {
    qa.nbuckets = kF16Size;
    qa.special0 = qa.special1 = -1;  // y is always in [-1, 1]
    memcpy(qa.base, best.base, (size_t)(2 * kF16Pos));
  } else {
    qa.nbuckets = 0;
    qa.special0 = qa.special1 = -1;
  }
  return true;
}

}  // namespace bq

// ---- host replay of the kernels' search (test hook of include/bq_debug.h) ----------------

#include "bq_debug.h"

namespace {

uint32_t host_nearest(const bq::PreparedTable& t, float y) {
  using namespace bq;
  const QuantArgs& qa = t.qa;
  if (t.mode == SEARCH) {
    if (!(fabsf(y) <= 1.0f)) return (uint32_t)qa.z;
    int q = 0;
    for (int step = qa.K >> 1; step >= 1; step >>= 1) q += (y >= qa.thr[q + step - 1]) ? step : 0;
    return (uint32_t)q;
  }
  if (t.mode == F16B) {
    // The kernels bring a non-finite element to y = 0, whose code is z.
    if (!(fabsf(y) <= 1.0f)) y = 0.0f;
    const uint32_t h = f16_rtz_bits(y);
    const uint32_t idx = (uint32_t)f16b_bucket(y);
    // The kernels' form on a pair word h | 0 << 16: mask, shifted sign inserted into bit 14,
    // byte offset of an 8-byte entry = bits 1..15.
    const uint32_t m = h & 0x3ff03ff0u, t = h >> 1;
    const uint32_t p = (0x40004000u & t) | (~0x40004000u & m);
    if (((p >> 1) & 0x7fffu) != idx << 3) return 0xffffffffu;
    if (!(idx < (uint32_t)kF16Pos || (idx >= (uint32_t)kF16NegLo && idx < (uint32_t)kF16Size))) return 0xffffffffu;
    const uint32_t b = qa.base[idx >= (uint32_t)kF16NegLo ? idx - kF16NegBase : idx];
    return b + ((y >= qa.thr[b]) ? 1u : 0u);
  }
  uint32_t idx;
  if (t.mode == LIN) {
    // The kernels bring a non-finite element to y = 0, whose code is z.
    if (!(fabsf(y) <= 1.0f)) y = 0.0f;
    const float zz = fmaf(y, qa.lin_scale, qa.lin_bias);
    idx = f32_bits(zz) - kLinBits;
    // The kernels' form: the entry's byte offset from bits(zz) in one shift-and-add.
    const int e = t.M <= 1 ? 3 : 4;
    if ((f32_bits(zz) << e) + qa.lin_off != idx << e || idx >= (uint32_t)qa.nbuckets) return 0xffffffffu;
  } else {
    uint32_t u = f32_bits(y);
    uint32_t a = std::min(std::max(u & 0x7fffffffu, qa.lo), qa.hi);
    idx = ((a - qa.lo) >> qa.sh) + ((u >> 31) ? (uint32_t)qa.nj : 0u);
    // The kernels' form of the same bucket: the LUT entry's byte offset.  A mismatch returns an
    // impossible code, so the table tests fail.
    const int e = t.M == 1 ? 3 : 4;
    const uint32_t j = std::min(std::max((u & 0x7fffffffu) >> qa.sh, qa.jlo), qa.jhi);
    if ((j << e) + ((u >> 31) ? qa.log_nbias : qa.log_bias) != idx << e) return 0xffffffffu;
  }
  if ((int)idx == qa.special0 || (int)idx == qa.special1) return (uint32_t)qa.z;
  uint32_t b = qa.base[idx];
  uint32_t q = b;
  for (int m = 0; m < std::max(t.M, 1); ++m) q += (y >= qa.thr[b + m]) ? 1u : 0u;
  return q;
}

}  // namespace

extern "C" bq_status bq_debug_nearest_codes(const bq_code_table* table, const float* y, int64_t count,
                                            int32_t* codes, int32_t* mode, int32_t* compares) {
  if (table == nullptr || table->entries == nullptr || (count > 0 && (y == nullptr || codes == nullptr)))
    return BQ_ERR_NULL;
  static thread_local bq::PreparedTable t;
  if (!bq::prepare_table(table->entries, table->size, &t)) return BQ_ERR_TABLE;
  for (int64_t i = 0; i < count; ++i) codes[i] = (int32_t)host_nearest(t, y[i]);
  if (mode) *mode = t.mode;
  if (compares) *compares = t.mode == bq::SEARCH ? 0 : std::max(t.M, 1);
  return BQ_OK;
}
