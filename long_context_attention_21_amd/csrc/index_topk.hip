// index_topk.hip -- Lightning-Indexer scores fused with exact per-query top-k.
//
// Method: "deepseek V4 技术论文" 1.1 (a low-rank, FP4 Lightning Indexer picks
// the top-k compressed entries for each query token), "DeepSeek-V4: Towards
// Highly Efficient Million-Token Context Intelligence" wiki summary,
// Proposed method item 1 (index scores computed in FP4) and Post-training
// item 3 (MXFP4 on the indexer QK path), aifrontier EP95 (top-k has to look
// at every entry, so the scorer must be light).  Score (DSA form):
//     I[t,s] = sum_h w[t,h] * relu(<qI[t,h], kI[s]>),   h ascending, fp32 fma chain.
// Selection: the min(k, n_vis) largest scores, ties to the lower entry index,
// written in a canonical order (grouped by (entry / 32) % 8, the groups in
// ascending order, ascending within each group) followed by -1 padding.
//
// Design for CDNA4
//  * A work-group of 8 waves serves QT query tokens: 2 tokens for rows of up
//    to 64K entries (two work-groups per CU), 4 tokens for longer rows, 1
//    token for single-token decode.  Scores: one
//    v_mfma_scale_f32_32x32x64_f8f6f4 (MXFP4) or four
//    v_mfma_f32_32x32x16_bf16 per 32 entries.  The 32 A rows are 4 token
//    slots x 8 heads, placed so each lane's accumulator rows are all 8 heads
//    of its token(s): lanes 0..31 hold tokens 0 and 2, lanes 32..63 tokens 1
//    and 3.  The head sum is an in-lane fma chain in ascending head order
//    (MXFP4 dot products are exact, so MXFP4 scores are bit-identical to a
//    sequential evaluation).  Entry rows come through range-checked buffer
//    loads, four tiles in flight per wave.
//  * Selection in one scoring pass:
//      1. a sample of the visible entries (one in S, in runs of 8 consecutive
//         entries; sized so that about kMinAbove samples lie above the cut)
//         is scored; each token's threshold is the sample quantile that
//         leaves about k + 850 entries above it;
//      2. every entry is scored once; scores >= threshold are appended to the
//         wave's private region of the token's LDS candidate buffer (ballot +
//         mbcnt, counts in registers: no atomics);
//      3. the waves serving a token (its "group") load the candidates into
//         registers and find the exact k-th largest (score desc, index asc)
//         with a radix selection over a histogram they share; after the
//         first digit the surviving keys move to short LDS lists.  The kept
//         indices are then written region by region.
//    Any threshold with at least k candidates above it keeps every top-k
//    member, so the result is exact.  If a region overflows or a token ends
//    up with fewer than k candidates, the work-group reruns its tokens with
//    the exact streaming method (buffers shrunk to exactly k whenever they
//    fill).
//  * Tokens whose visible entries all fit in k skip scoring.
//  * Few tokens over long entry lists (decode) split each row over
//    partitions of 16384 entries: each partition keeps its highest scores by
//    a cut of its own (a histogram over its scores held in LDS), and a
//    selection work-group per row checks that the cuts kept every top-k
//    member before it selects (see index_split_cut_kernel).
#include <cmath>

#include "device.h"
#include "kernels.h"

namespace csa {

constexpr int kCap = 4096;             // candidate buffer per token
// Work-group shape for QT tokens: 8 waves.  With 2 tokens the 70 KB of LDS
// lets two work-groups share a CU (4 waves per SIMD), so one's scoring
// overlaps the other's selections, and each token's selection is shared by
// 4 waves.  Each lane scores TPL tokens of a tile (all 64 lanes are busy
// once QT >= 2).
template <int QT>
struct Shape {
  static constexpr int W = 8;  // waves per work-group
  static constexpr int T = 64 * W;          // threads
  static constexpr int Tile = 32 * W;       // entries per round of the work-group
  static constexpr int Reg = kCap / W;      // per-wave candidate region of a token's buffer
  static constexpr int TPL = QT > 2 ? 2 : 1;
};
constexpr int kDepth = 4;              // score tiles in flight per wave
constexpr int kMinAbove = 256;         // sampled entries expected above the threshold
constexpr int kList = 512;             // per-member key list after the first radix digit

// Sort key of the canonical row order (see emit_canonical): the 32-entry
// tile modulo 8, then the entry (entries are below 2^24).
__device__ __forceinline__ uint32_t canon_key(uint32_t e) { return (((e >> 5) & 7u) << 24) | e; }

// Lane mask of a predicate (the compare result itself, no int round trip).
__device__ __forceinline__ uint64_t ballot(bool pred) { return __builtin_amdgcn_ballot_w64(pred); }

__device__ __forceinline__ uint32_t okey(uint32_t fbits) {
  return (fbits & 0x80000000u) ? ~fbits : (fbits | 0x80000000u);
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Row r of the 32-row A operand -> (token j, head h); see the header comment.
__device__ __forceinline__ void row_to_token_head(int r, int& j, int& h) {
  const int half = (r >> 2) & 1;
  const int ic = 4 * (r >> 3) + (r & 3);
  j = half + 2 * (ic >> 3);
  h = ic & 7;
}

// Token j of a work-group is served by the "group" of waves w with
// w % QT == j (W / QT of them); group member h = w / QT.
template <int QT>
struct TopkSmem {
  static constexpr int kWaves = Shape<QT>::W;
  uint2 cand[QT][kCap];       // {fp32 score bits, entry}; samples in phase 1; output bitmap at the end
  uint32_t hist[2][QT][256];  // double-buffered radix histograms, one per token group
  uint32_t xchg[kWaves][2];   // per-wave values read by the other group members
  int gdone[2][QT];           // radix selection finished, per token group (double-buffered)
  int wcnt[kWaves][QT];       // candidates per (wave, token) region
  float thr[QT];
  int cnt[QT];
  int fallback;
  int ties;
  uint32_t vcnt[QT][8];       // kept entries per canonical group (output)
  int staged;                 // split path: kept entries staged for sorting
  int above;                  // split path: candidates at or above the row's bound
  uint32_t sel[4];
};

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xf, 0xf, true);
}
__device__ __forceinline__ uint32_t wave_max_dpp(uint32_t x) {
  x = max(x, dpp<0xB1>(x));   // quad_perm [1,0,3,2]
  x = max(x, dpp<0x4E>(x));   // quad_perm [2,3,0,1]
  x = max(x, dpp<0x124>(x));  // row_ror:4
  x = max(x, dpp<0x128>(x));  // row_ror:8
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = max((uint32_t)p[0], (uint32_t)p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}
__device__ __forceinline__ uint32_t wave_min_dpp(uint32_t x) {
  x = min(x, dpp<0xB1>(x));
  x = min(x, dpp<0x4E>(x));
  x = min(x, dpp<0x124>(x));
  x = min(x, dpp<0x128>(x));
  auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
  x = min((uint32_t)p[0], (uint32_t)p[1]);
  auto q = __builtin_amdgcn_permlane32_swap(x, x, false, false);
  return min((uint32_t)q[0], (uint32_t)q[1]);
}
// inclusive prefix sum over lanes 0..63
__device__ __forceinline__ uint32_t wave_prefix_sum(uint32_t x) {
  const int lane = threadIdx.x & 63;
  x += dpp<0x111>(x);  // row_shr:1 (zero from outside the row)
  x += dpp<0x112>(x);  // row_shr:2
  x += dpp<0x114>(x);  // row_shr:4
  x += dpp<0x118>(x);  // row_shr:8
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane >> 4;
  x += (row >= 1 ? t0 : 0u) + (row >= 2 ? t1 : 0u) + (row >= 3 ? t2 : 0u);
  return x;
}

// ----------------------------------------------------------------------------
// Radix selection of the r-th largest (1-based) key held in registers by a
// token's group (kr[m] of every lane of every member; slot m may hold keys
// only where bit m of smask is set, uniformly).  Zero keys mark empty lanes:
// they sort below every real key (order keys of finite floats and inverted
// entry indices are never 0), so they cannot change the result while r does
// not exceed the number of real keys (n_valid).  Digits of up to 8 bits are
// taken from key - (kmin - 1) (kmin, kmax: extremes of the real keys),
// starting at its top bit over the real range; a histogram shared by the group is filled with
// LDS atomics and scanned by every member alike, so all members reach the
// same decision.  Stops when the chosen bin holds exactly the remaining rank
// (then keep(key) = key >= T selects exactly r) or at most slack keys (then
// it selects r .. r + slack - 1), otherwise resolves all bits (exact: T is
// the r-th key, inbin the number equal to it, above the number greater).  Every wave of the work-group must call it the
// same number of times (it synchronises the work-group); groups with nothing
// to select pass active = false.
struct RadixOut {
  uint32_t T, above, inbin;
  int exact;
};

template <int QT, int NS>
__device__ __forceinline__ RadixOut group_radix(TopkSmem<QT>& sm, const uint32_t (&kr)[NS], uint32_t smask, uint32_t r,
                                                uint32_t n_valid, bool active, uint32_t slack = 0u) {
  constexpr int G = Shape<QT>::W / QT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = wave % QT, h = wave / QT;
  uint32_t kmax = 0u, kmin1 = 0xffffffffu;  // kmin1 = min(key - 1): empty (0) keys wrap to the top
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    kmax = max(kmax, kr[m]);
    kmin1 = min(kmin1, kr[m] - 1u);
  }
  kmax = wave_max_dpp(kmax);
  kmin1 = wave_min_dpp(kmin1);
  if (lane == 0) { sm.xchg[wave][0] = kmax; sm.xchg[wave][1] = kmin1; }
  if (lane < 64 / G) *(u32x4*)&sm.hist[0][j][h * (256 / G) + 4 * lane] = u32x4{0u, 0u, 0u, 0u};
  __syncthreads();
#pragma unroll
  for (int g = 0; g < G; ++g) {
    kmax = max(kmax, sm.xchg[j + QT * g][0]);
    kmin1 = min(kmin1, sm.xchg[j + QT * g][1]);
  }
  const uint32_t kmin = kmin1 + 1u;
  RadixOut o{0u, 0u, 0u, 0};
  bool done = !active;
  if (!done && kmax == kmin) {  // every real key is equal
    o = RadixOut{kmax, 0u, n_valid, 1};
    done = true;
  }
  // digits of v(key) = max(key, base) - base with base = kmin - 1: real keys
  // map to 1 .. kmax - base and empty slots to 0, still below every real
  // key; the first digit splits the real range into up to 256 equal bins
  const uint32_t base = kmin - 1u;
  int top = 0;
  uint32_t prefix = 0u, r_left = r, above = 0u;
  if (!done) top = 31 - __builtin_clz(kmax - base);
  // after the first digit the keys of the chosen bin are usually few: each
  // member then copies its share into a list in the token's (free) buffer,
  // and the remaining digits scan the lists instead of every register slot
  uint32_t* list = (uint32_t*)&sm.cand[j][0] + h * kList;
  int lcnt = 0;
  bool listmode = false;
#pragma unroll 1
  for (int it = 0; it < 4; ++it) {  // at most 4 digits of 8 bits
    uint32_t* hc = sm.hist[it & 1][j];
    const int lo = top >= 7 ? top - 7 : 0;
    const uint32_t dmask = (1u << (top - lo + 1)) - 1u;
    const uint32_t pb = prefix >> lo;
    if (!done) {
      if (!listmode) {
#pragma unroll
        for (int m = 0; m < NS; ++m) {
          if ((smask >> m) & 1u) {
            const uint32_t d = ((max(kr[m], base) - base) >> lo) - pb;  // digit, if the key matches the prefix
            if (d <= dmask) atomicAdd(&hc[d], 1u);
          }
        }
      } else {
        for (int s0 = 0; s0 < lcnt; s0 += 64) {
          const int i = s0 + lane;
          if (i < lcnt) {
            const uint32_t d = ((max(list[i], base) - base) >> lo) - pb;
            if (d <= dmask) atomicAdd(&hc[d], 1u);
          }
        }
      }
    }
    __syncthreads();
    if (!done) {
      // lane l owns bins 252-4l .. 255-4l, so a prefix sum over lanes counts
      // the keys in bins >= the lane's lowest bin
      const u32x4 hv = *(const u32x4*)(hc + 252 - 4 * lane);
      const uint32_t c = hv[0] + hv[1] + hv[2] + hv[3];
      const uint32_t incl = wave_prefix_sum(c);
      const int L = __builtin_ctzll(ballot(incl >= r_left));
      uint32_t acc = incl - c, d = 0u, hd = 0u;
      if (lane == L) {
        d = 252 - 4 * lane;
        if (acc + hv[3] >= r_left) { d += 3; hd = hv[3]; }
        else {
          acc += hv[3];
          if (acc + hv[2] >= r_left) { d += 2; hd = hv[2]; }
          else {
            acc += hv[2];
            if (acc + hv[1] >= r_left) { d += 1; hd = hv[1]; }
            else { acc += hv[1]; hd = hv[0]; }
          }
        }
      }
      d = (uint32_t)__builtin_amdgcn_readlane((int)d, L);
      acc = (uint32_t)__builtin_amdgcn_readlane((int)acc, L);
      hd = (uint32_t)__builtin_amdgcn_readlane((int)hd, L);
      above += acc;
      r_left -= acc;
      prefix |= d << lo;
      if (hd == r_left || lo == 0 || hd <= slack) {
        // lo == 0: exact; otherwise the bin's lower bound (keep = key >= T
        // then selects r .. r + hd - 1 keys, exactly r when hd == r_left)
        o = RadixOut{prefix + base, above, hd, lo == 0 ? 1 : 0};
        done = true;
      } else {
        top = lo - 1;
        if (!listmode && hd <= (uint32_t)kList) {
          // keys of the chosen bin -> this member's list (hd bounds every member's share)
#pragma unroll
          for (int m = 0; m < NS; ++m) {
            if ((smask >> m) & 1u) {
              const bool in = ((max(kr[m], base) - base) >> lo) - pb == d;
              const uint64_t bal = ballot(in);
              const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                              __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
              if (in) list[lcnt + rank] = kr[m];
              lcnt += __builtin_popcountll(bal);
            }
          }
          listmode = true;
        } else if (listmode) {
          // keep only the chosen bin, in place (writes never pass the chunk being read)
          int nc = 0;
          for (int s0 = 0; s0 < lcnt; s0 += 64) {
            const int i = s0 + lane;
            const uint32_t key = i < lcnt ? list[i] : 0u;
            const bool in = i < lcnt && ((max(key, base) - base) >> lo) - pb == d;
            const uint64_t bal = ballot(in);
            const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32),
                                                            __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
            if (in) list[nc + rank] = key;
            nc += __builtin_popcountll(bal);
          }
          lcnt = nc;
        }
      }
    }
    // the other buffer was last read before the previous barrier
    if (lane < 64 / G) *(u32x4*)&sm.hist[(it + 1) & 1][j][h * (256 / G) + 4 * lane] = u32x4{0u, 0u, 0u, 0u};
    if (h == 0 && lane == 0) sm.gdone[it & 1][j] = done ? 1 : 0;
    __syncthreads();
    // leave together once every group is done (the flags of this iteration
    // are not rewritten before the next barrier)
    bool all = true;
#pragma unroll
    for (int g = 0; g < QT; ++g) all &= sm.gdone[it & 1][g] != 0;
    if (all) break;
  }
  return o;
}

// ----------------------------------------------------------------------------
// Linear-bin selection over a token group's keys (kr[NS] per member lane,
// 0 = empty slot).  Bins are (key - lo) >> s over the order keys, 256 of
// them; every member counts its keys into the group's histogram with LDS
// atomics and scans it alike.  Unlike group_radix it needs no per-slot
// register masks and spreads the keys over all members.

// extremes of the group's real keys (kmin = 0 when it has none); every wave
// calls it (one barrier); also clears both histogram buffers of the group
template <int QT, int NS>
__device__ __forceinline__ void group_extremes(TopkSmem<QT>& sm, const uint32_t (&kr)[NS], uint32_t& kmin,
                                               uint32_t& kmax) {
  constexpr int G = Shape<QT>::W / QT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = wave % QT, h = wave / QT;
  uint32_t mx = 0u, mn1 = 0xffffffffu;  // mn1 = min(key - 1): empty (0) slots wrap to the top
#pragma unroll
  for (int m = 0; m < NS; ++m) {
    mx = max(mx, kr[m]);
    mn1 = min(mn1, kr[m] - 1u);
  }
  mx = wave_max_dpp(mx);
  mn1 = wave_min_dpp(mn1);
  if (lane == 0) { sm.xchg[wave][0] = mx; sm.xchg[wave][1] = mn1; }
  if (lane < 64 / G) {
    *(u32x4*)&sm.hist[0][j][h * (256 / G) + 4 * lane] = u32x4{0u, 0u, 0u, 0u};
    *(u32x4*)&sm.hist[1][j][h * (256 / G) + 4 * lane] = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  mx = 0u;
  mn1 = 0xffffffffu;
#pragma unroll
  for (int g = 0; g < G; ++g) {
    mx = max(mx, sm.xchg[j + QT * g][0]);
    mn1 = min(mn1, sm.xchg[j + QT * g][1]);
  }
  kmax = mx;
  kmin = mn1 + 1u;
}

// The bin of the r-th largest key within [lo, lo + (256 << s)) counted from
// `above` keys already known to lie above that range: its index b, its count
// hb and the count above it (including `above`).  Histogram buffer `buf` of
// the group must be zero; every wave calls it (one barrier).
struct BinOut {
  uint32_t b, hb, above;
};

// The bin of the r-th largest key in a 256-bin histogram hc (bin 255 the
// highest), counted from `above` keys known to lie above bin 255; every lane
// of the wave calls it and gets the same result.
__device__ __forceinline__ BinOut find_bin(const uint32_t* hc, uint32_t r, uint32_t above) {
  const int lane = threadIdx.x & 63;
  // lane l owns bins 252-4l .. 255-4l: a prefix sum over lanes counts the
  // keys in bins >= the lane's lowest bin
  const u32x4 hv = *(const u32x4*)(hc + 252 - 4 * lane);
  const uint32_t c = hv[0] + hv[1] + hv[2] + hv[3];
  const uint32_t incl = wave_prefix_sum(c) + above;
  const uint64_t hit = ballot(incl >= r);
  const int L = hit ? __builtin_ctzll(hit) : 63;
  uint32_t acc = incl - c, d = 0u, hd = 0u;
  if (lane == L) {
    d = 252 - 4 * lane;
    if (acc + hv[3] >= r) { d += 3; hd = hv[3]; }
    else {
      acc += hv[3];
      if (acc + hv[2] >= r) { d += 2; hd = hv[2]; }
      else {
        acc += hv[2];
        if (acc + hv[1] >= r) { d += 1; hd = hv[1]; }
        else { acc += hv[1]; hd = hv[0]; }
      }
    }
  }
  BinOut o;
  o.b = (uint32_t)__builtin_amdgcn_readlane((int)d, L);
  o.above = (uint32_t)__builtin_amdgcn_readlane((int)acc, L);
  o.hb = (uint32_t)__builtin_amdgcn_readlane((int)hd, L);
  return o;
}
template <int QT, int NS>
__device__ __forceinline__ BinOut group_bin(TopkSmem<QT>& sm, int buf, const uint32_t (&kr)[NS], uint32_t lo, int s,
                                            uint32_t r, uint32_t above, bool active) {
  const int wave = threadIdx.x >> 6;
  const int j = wave % QT;
  uint32_t* hc = sm.hist[buf][j];
  if (active) {
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      const uint32_t x = kr[m];
      if (x != 0u && x >= lo) {
        const uint32_t d = (x - lo) >> s;
        if (d < 256u) atomicAdd(&hc[d], 1u);
      }
    }
  }
  __syncthreads();
  return active ? find_bin(hc, r, above) : BinOut{0u, 0u, above};
}

// shift that maps [kmin, kmax] onto at most 256 bins
__device__ __forceinline__ int bin_shift(uint32_t kmin, uint32_t kmax) {
  const uint32_t span = kmax - kmin;
  const int top = span ? 31 - __builtin_clz(span) : 0;
  return top > 7 ? top - 7 : 0;
}

// Approximate r-th largest of the group's keys (a cut with at least r keys at
// or above it, and about r): the lower edge of the bin holding the r-th key,
// refined once inside that bin when it holds more than r / 16 keys.  Returns
// the order key of the cut (0 for groups with no keys).  Every wave calls it.
template <int QT, int NS>
__device__ __forceinline__ uint32_t group_cut(TopkSmem<QT>& sm, const uint32_t (&kr)[NS], uint32_t r, bool active) {
  uint32_t kmin, kmax;
  group_extremes<QT, NS>(sm, kr, kmin, kmax);
  active = active && kmax != 0u && r >= 1u;
  const int s = bin_shift(kmin, kmax);
  const BinOut o = group_bin<QT, NS>(sm, 0, kr, kmin, s, r, 0u, active);
  uint32_t lo = kmin + (o.b << s);
  const bool refine = active && s > 0 && o.hb > max(r >> 4, 1u);
  const int s2 = s > 8 ? s - 8 : 0;
  const BinOut o2 = group_bin<QT, NS>(sm, 1, kr, lo, s2, r, o.above, refine);
  if (refine) lo += o2.b << s2;
  return active ? lo : 0u;
}

// ----------------------------------------------------------------------------
// Exact streaming fallback (work-group wide): buffers hold order keys and are
// shrunk to exactly k whenever they fill.

template <int kThreads, class KeyFn, class FiltFn>
__device__ uint32_t wg_radix_select(uint32_t* hist, uint32_t* sel, int cnt, uint32_t r, KeyFn keyfn,
                                    FiltFn filt, uint32_t* above, uint32_t* equal) {
  const int tid = threadIdx.x, lane = tid & 63;
  uint32_t prefix = 0, pmask = 0, r_left = r, gt_total = 0;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int i = tid; i < cnt; i += kThreads) {
      if (!filt(i)) continue;
      const uint32_t k = keyfn(i);
      if ((k & pmask) == prefix) atomicAdd(&hist[(k >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      const uint32_t h0 = hist[4 * lane], h1 = hist[4 * lane + 1], h2 = hist[4 * lane + 2],
                     h3 = hist[4 * lane + 3];
      const uint32_t c = h0 + h1 + h2 + h3;
      uint32_t suf = c;
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = (uint32_t)__shfl_down((int)suf, off);
        if (lane + off < 64) suf += o;
      }
      const uint64_t bal = ballot(suf >= r_left);
      const int L = 63 - __builtin_clzll(bal);
      if (lane == L) {
        uint32_t acc = suf - c;
        const uint32_t hh[4] = {h0, h1, h2, h3};
        int d = 4 * lane;
  #pragma unroll
      for (int i = 3; i >= 0; --i) {
          if (acc + hh[i] >= r_left) { d = 4 * lane + i; break; }
          acc += hh[i];
        }
        sel[0] = (uint32_t)d;
        sel[1] = acc;
        sel[2] = hist[d];
      }
    }
    __syncthreads();
    const uint32_t d = sel[0], acc = sel[1];
    gt_total += acc;
    r_left -= acc;
    prefix |= d << shift;
    pmask |= 255u << shift;
    if (shift == 0) *equal = sel[2];
    __syncthreads();
  }
  *above = gt_total;
  return prefix;
}

template <int QT>
__device__ void wg_shrink_exact(TopkSmem<QT>& sm, int j, int kk) {
  constexpr int kThreads = Shape<QT>::T;
  const int tid = threadIdx.x;
  const int cnt = sm.cnt[j];
  if (cnt <= kk) return;
  uint32_t above, equal;
  uint2* cd = sm.cand[j];
  uint32_t* hist = &sm.hist[0][0][0];
  const uint32_t tau = wg_radix_select<kThreads>(hist, sm.sel, cnt, (uint32_t)kk, [&](int i) { return cd[i].x; },
                                       [](int) { return true; }, &above, &equal);
  const uint32_t need = (uint32_t)kk - above;
  uint32_t tau_inv = 0;
  const bool cut_ties = need < equal;
  if (cut_ties) {
    uint32_t a2, e2;
    tau_inv = wg_radix_select<kThreads>(hist, sm.sel, cnt, need, [&](int i) { return ~cd[i].y; },
                              [&](int i) { return cd[i].x == tau; }, &a2, &e2);
  }
  constexpr int PER = kCap / kThreads;
  uint32_t kv[PER];
  int32_t iv[PER];
  int nk = 0;
#pragma unroll
  for (int q = 0; q < PER; ++q) {
    const int i = tid + q * kThreads;
    kv[q] = 0;
    iv[q] = -1;
    if (i < cnt) {
      const uint32_t k = cd[i].x;
      const int32_t id = (int32_t)cd[i].y;
      const bool keep = (k > tau) || (k == tau && (!cut_ties || ~(uint32_t)id >= tau_inv));
      if (keep) { kv[q] = k; iv[q] = id; ++nk; }
    }
  }
  __syncthreads();
  if (tid == 0) sm.cnt[j] = 0;
  __syncthreads();
  int base = atomicAdd(&sm.cnt[j], nk);
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (iv[q] >= 0) { cd[base] = make_uint2(kv[q], (uint32_t)iv[q]); ++base; }
  if (tid == 0) sm.thr[j] = __uint_as_float(tau + 1u);  // order key, strictly above the k-th
  __syncthreads();
}

template <int QT>
__device__ void wg_bitonic_sort(TopkSmem<QT>& sm, int j, int cnt) {
  constexpr int kThreads = Shape<QT>::T;
  const int tid = threadIdx.x;
  int P = 1;
  while (P < cnt) P <<= 1;
  uint2* s = sm.cand[j];  // sorts the entry field
  for (int i = cnt + tid; i < P; i += kThreads) s[i].y = 0x7fffffffu;  // canon_key: largest
  __syncthreads();
  for (int size = 2; size <= P; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < (P >> 1); i += kThreads) {
        const int lo = 2 * i - (i & (stride - 1));
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const uint32_t a = s[lo].y, bb = s[hi].y;
        if ((canon_key(a) > canon_key(bb)) == asc) { s[lo].y = bb; s[hi].y = a; }
      }
      __syncthreads();
    }
  }
}

// ----------------------------------------------------------------------------
// Canonical row order.  The indices of a row are written grouped by
// (index / 32) % 8 -- the 32-entry tile modulo 8 -- groups in ascending
// order, ascending within each group; -1 padding follows.  The order depends
// on the selected set only, so every path (work-groups of 1, 2 or 4 tokens,
// the split decode path, the exact streaming path) writes the same row, and
// attention, whose sums follow the row's order, sees the same keys in the
// same order.  Wave w of the scoring pass scores the tiles T with
// T % kWaves == w in ascending order, so with 8 waves its region of a
// token's buffer holds exactly group w, in ascending order: the row is
// written straight from the regions.

// Entries 0 .. nv-1 (all kept), in the canonical order: position i.
__device__ __forceinline__ int32_t canon_all(int i, int nv) {
  const int nt = nv >> 5, rem = nv & 31;
  int base = 0;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    const int full = nt > v ? (nt - v + 7) >> 3 : 0;  // full tiles T < nt with T % 8 == v
    const int cnt = 32 * full + ((nt & 7) == v ? rem : 0);
    if (i < base + cnt) {
      const int r = i - base;
      return 32 * (v + 8 * (r >> 5)) + (r & 31);
    }
    base += cnt;
  }
  return -1;
}

// Main path output of a token group's kept entries (ir[sl] where bit sl of
// keep is set; kk of them), then -1 padding up to k.  Every wave of the
// work-group calls it (one barrier); groups of rows past n pass live = false.
template <int QT, int NS>
__device__ __forceinline__ void emit_canonical(TopkSmem<QT>& sm, bool live, const uint32_t (&ir)[NS], uint32_t keep,
                                               int kk, int k, int32_t* o) {
  constexpr int W = Shape<QT>::W, G = W / QT, VPW = 8 / W;  // canonical groups per region
  constexpr int kPer = Shape<QT>::Reg / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = wave % QT, h = wave / QT;
  // kept entries per canonical group of each of this member's regions
#pragma unroll
  for (int rr = 0; rr < QT; ++rr) {
    const int w = h * QT + rr;
#pragma unroll
    for (int sv = 0; sv < VPW; ++sv) {
      uint32_t c = 0u;
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int sl = rr * kPer + m;
        // with one group per region (8 waves) every entry of region w is in group w
        const bool ing = VPW == 1 || ((ir[sl] >> 5) & 7u) == (uint32_t)(w + sv * W);
        c += (uint32_t)__builtin_popcountll(ballot(((keep >> sl) & 1u) && ing));
      }
      if (lane == 0) sm.vcnt[j][w + sv * W] = c;
    }
  }
  __syncthreads();
  uint32_t vb[8];  // first position of each group
  uint32_t acc = 0u;
#pragma unroll
  for (int v = 0; v < 8; ++v) {
    vb[v] = acc;
    acc += sm.vcnt[j][v];
  }
  if (!live) return;
#pragma unroll
  for (int rr = 0; rr < QT; ++rr) {
    const int w = h * QT + rr;
#pragma unroll
    for (int sv = 0; sv < VPW; ++sv) {
      const int v = w + sv * W;
      uint32_t run = vb[v];
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int sl = rr * kPer + m;
        const bool in = ((keep >> sl) & 1u) && (VPW == 1 || ((ir[sl] >> 5) & 7u) == (uint32_t)v);
        const uint64_t bal = ballot(in);
        const uint32_t pos = run + __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (in && pos < (uint32_t)k) o[pos] = (int32_t)ir[sl];
        run += (uint32_t)__builtin_popcountll(bal);
      }
    }
  }
  for (int i = kk + h * 64 + lane; i < k; i += G * 64) o[i] = -1;
}

// ----------------------------------------------------------------------------
// Scores of one 32-column tile for the work-group's tokens.  Lane column
// lane % 32 is entry e (any entry index; e >= N gives a zero column).

template <int FMT>
struct BTile;
template <>
struct BTile<1> {  // MXFP4: 16 code bytes + one e8m0 scale per lane
  u32x4 cw;
  int sc;
};
template <>
struct BTile<0> {  // bf16: four 8-element pieces per lane
  bf16x8 v[4];
};

template <int FMT>
struct Scorer {
  i32x8 A_fp4;
  int a_scale;
  bf16x8 A_bf[4];
  float wv[2][8];
  __amdgpu_buffer_rsrc_t rk;  // this batch's entry keys (MXFP4 codes or bf16 rows)
  __amdgpu_buffer_rsrc_t rs;  // this batch's MXFP4 block scales
  int voff_k, voff_s;         // the lane's byte offsets inside an entry's row

  // B operand of entry column e (lane % 32).  Buffer loads are range-checked
  // by the hardware: entries at or past the end of the array read as zero, so
  // the loads need no clamp or branch (callers never select e >= n_vis).
  __device__ __forceinline__ BTile<FMT> load(int e) const {
    BTile<FMT> t;
    if constexpr (FMT == 1) {
      t.cw = __builtin_amdgcn_raw_buffer_load_b128(rk, e * 32 + voff_k, 0, 0);
      t.sc = __builtin_amdgcn_raw_buffer_load_b8(rs, e * 2 + voff_s, 0, 0);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        t.v[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rk, e * 128 + ks * 32 + voff_k, 0, 0));
    }
    return t;
  }

  __device__ __forceinline__ f32x16 mfma(const BTile<FMT>& t) const {
    f32x16 C;
#pragma unroll
    for (int i = 0; i < 16; ++i) C[i] = 0.0f;
    if constexpr (FMT == 1) {
      i32x8 B;
#pragma unroll
      for (int i = 0; i < 4; ++i) { B[i] = (int)t.cw[i]; B[4 + i] = 0; }
      C = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(A_fp4, B, C, 4, 4, 0, a_scale, 0, t.sc);
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
        C = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A_bf[ks], t.v[ks], C, 0, 0, 0);
    }
    return C;
  }

  // C rows: heads 0..7 of the lane's token jl0 (i = 0..7) and of token
  // jl0 + 2 (i = 8..15); TPL = 1 scores only the first.
  // The chain starts from +0 and can never produce -0.
  template <int TPL = 2>
  __device__ __forceinline__ void epilogue(const f32x16& C, float I[2]) const {
#pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      float s = 0.0f;
#pragma unroll
      for (int h = 0; h < 8; ++h) s = __builtin_fmaf(wv[tt][h], fmaxf(C[tt * 8 + h], 0.0f), s);
      I[tt] = s;
    }
  }

  template <int TPL = 2>
  __device__ __forceinline__ void score(int e, float I[2]) const { epilogue<TPL>(mfma(load(e)), I); }
};

// Appends the passing lanes of each half-wave to their token's buffer
// (exact fallback: shared count, LDS atomic).
template <int QT>
__device__ __forceinline__ void append(TopkSmem<QT>& sm, const bool pass[2], const uint32_t val[2], int e, int jl0) {
  constexpr int TPL = Shape<QT>::TPL;
  const int lane = threadIdx.x & 63;
  const int leader = (lane < 32) ? 0 : 32;
  const uint64_t halfmask = (lane < 32) ? 0x00000000ffffffffull : 0xffffffff00000000ull;
#pragma unroll
  for (int tt = 0; tt < TPL; ++tt) {
    const uint64_t mine = ballot(pass[tt]) & halfmask;
    const int pc = __builtin_popcountll(mine);
    const int rank = __builtin_popcountll(mine & ((1ull << lane) - 1ull));
    const int j = jl0 + 2 * tt;
    int basepos = 0;
    if (lane == leader && pc > 0) basepos = atomicAdd(&sm.cnt[j < QT ? j : 0], pc);
    basepos = __shfl(basepos, leader);
    const int pos = basepos + rank;
    if (pass[tt]) sm.cand[j][pos] = make_uint2(val[tt], (uint32_t)e);
  }
}

// Appends the passing lanes of a half-wave (token j) to this wave's private
// region of the token's buffer.  The running counts of the two half-waves
// (wc[0]: lanes 0..31, wc[1]: lanes 32..63) are wave-uniform and stay on the
// scalar unit: no LDS atomic, no cross-lane round trip.
template <int QT>
__device__ __forceinline__ void append_private(TopkSmem<QT>& sm, bool vis, bool ge, uint32_t val, int e, int j,
                                               uint32_t (&wc)[2]) {
  constexpr int kReg = Shape<QT>::Reg;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  // the two compares' lane masks, combined on the scalar unit
  const uint64_t bal = ballot(vis) & ballot(ge);
  const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
  const uint32_t nlo = (uint32_t)__builtin_popcount(lo), nhi = (uint32_t)__builtin_popcount(hi);
  // position = count + passing lanes below this one in its half-wave; the
  // upper half's mbcnt_lo counts every bit of lo, taken off its count first
  const uint32_t base = lane < 32 ? wc[0] : wc[1] - nlo;
  const int pos = (int)__builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, base));
  if (vis && ge && pos < kReg) sm.cand[j][wave * kReg + pos] = make_uint2(val, (uint32_t)e);
  wc[0] += nlo;
  wc[1] += nhi;
}

// append_private for a tile every entry of which is visible to both of the
// lane's tokens and which cannot overflow a region (the caller checks both
// on the scalar unit): no per-lane visibility or bound test.  Token j0 (lanes
// 0..31) and j0 + 1 (lanes 32..63) have adjacent buffers, so one position
// serves both halves: the upper lanes add the buffer length plus their
// half's count less everything mbcnt_lo counted below them.
template <int QT>
__device__ __forceinline__ void append_full(TopkSmem<QT>& sm, bool ge, uint32_t val, int e, int j0, int wave,
                                            uint32_t upper, uint32_t (&wc)[2]) {
  constexpr int kReg = Shape<QT>::Reg;
  const uint64_t bal = ballot(ge);
  const uint32_t lo = (uint32_t)bal, hi = (uint32_t)(bal >> 32);
  const uint32_t nlo = (uint32_t)__builtin_popcount(lo), nhi = (uint32_t)__builtin_popcount(hi);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readfirstlane((int)(kCap + wc[1] - wc[0] - nlo));
  const uint32_t pos = __builtin_amdgcn_mbcnt_hi(hi, __builtin_amdgcn_mbcnt_lo(lo, upper & d));
  const uint32_t s0 = (uint32_t)__builtin_amdgcn_readfirstlane((int)((uint32_t)(j0 * kCap + wave * kReg) + wc[0]));
  if (ge) (&sm.cand[0][0])[pos + s0] = make_uint2(val, (uint32_t)e);
  wc[0] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(wc[0] + nlo));
  wc[1] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(wc[1] + nhi));
}

// Scorer of a work-group's QT query tokens q0 .. q0+QT-1 of batch row b:
// the MFMA A operand (rows = (token, head); MXFP4 quantised in-kernel from
// bf16 q when no scales are given), the head weights, and the entry-key
// buffer descriptors.  nvq[j]: visible entries of token q0 + j (0 past n),
// work-group uniform; nvl[tt]: the same for this lane's token jl0 + 2 tt.
template <int QT, int FMT>
__device__ __forceinline__ void init_scorer(Scorer<FMT>& sc, const IndexParams& p, int b, int q0,
                                            const int (&nvq)[QT], int nvl[2]) {
  const int lane = threadIdx.x & 63;

  {
    int arow_j, arow_h;
    row_to_token_head(lane & 31, arow_j, arow_h);
    const int aq = q0 + arow_j;
    const bool arow_ok = (arow_j < QT) && (aq < p.n) && (arow_h < p.H_I);
    const int64_t qrow = ((int64_t)b * p.n + aq) * p.H_I + arow_h;
    sc.a_scale = 127;
    if (FMT == 1) {
#pragma unroll
      for (int i = 0; i < 8; ++i) sc.A_fp4[i] = 0;
      if (arow_ok) {
        if (p.q_scale) {
          const u32x4 cw = *(const u32x4*)((const uint8_t*)p.q + qrow * 32 + (lane >> 5) * 16);
#pragma unroll
          for (int i = 0; i < 4; ++i) sc.A_fp4[i] = (int)cw[i];
          sc.a_scale = p.q_scale[qrow * 2 + (lane >> 5)];
        } else {
          // quantise this (row, 32-element block) of the bf16 query to MXFP4.
          // The block maximum is taken on the bf16 bit patterns (sign
          // cleared, the integer order of finite values is their order), two
          // halves at a time.  v_cvt_scalef32_pk_fp4_f32 divides by the
          // scale 2^E and rounds to the nearest e2m1 value, ties to even,
          // saturating at 6: the same codes as the bit-level encoder for
          // every finite bf16 value and every E (a -0 code where that gives
          // +0, which scores alike).  Word e of load i holds elements
          // 8i + 2e (low half) and 8i + 2e + 1: they become byte e of code
          // word i.
          const u32x4* src = (const u32x4*)((const uint16_t*)p.q + qrow * 64 + (lane >> 5) * 32);
          u32x4 v[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] = src[i];
          u16x2 am = {0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int e = 0; e < 4; ++e) am = __builtin_elementwise_max(am, __builtin_bit_cast(u16x2, v[i][e] & 0x7fff7fffu));
          const uint32_t abits = am[0] > am[1] ? am[0] : am[1];
          if (abits != 0u) {
            const int E = mxfp4_exponent(bf16_to_f32(abits));
            sc.a_scale = E + 127;
            const float scale = __builtin_ldexpf(1.0f, E);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              uint32_t w = 0u;
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16lo(v[i][0]), bf16hi(v[i][0]), scale, 0);
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16lo(v[i][1]), bf16hi(v[i][1]), scale, 1);
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16lo(v[i][2]), bf16hi(v[i][2]), scale, 2);
              w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, bf16lo(v[i][3]), bf16hi(v[i][3]), scale, 3);
              sc.A_fp4[i] = (int)w;
            }
          } else {
            sc.a_scale = 0;
          }
        }
      }
    } else {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        if (arow_ok) {
          sc.A_bf[ks] = *(const bf16x8*)((const uint16_t*)p.q + qrow * 64 + ks * 16 + (lane >> 5) * 8);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) sc.A_bf[ks][e] = (__bf16)0.0f;
        }
      }
    }
  }
  const int jl0 = lane >> 5;  // this lane scores tokens jl0 and jl0 + 2
#pragma unroll
  for (int tt = 0; tt < 2; ++tt) {
    const int q = q0 + jl0 + 2 * tt;
    int v = 0;
#pragma unroll
    for (int jj = 0; jj < QT; ++jj)
      if (jj == jl0 + 2 * tt) v = nvq[jj];
    nvl[tt] = v;
#pragma unroll
    for (int h = 0; h < 8; ++h)
      sc.wv[tt][h] = (v > 0 && h < p.H_I) ? p.w[((int64_t)b * p.n + q) * p.H_I + h] : 0.0f;
  }
  {
    // the descriptors are uniform: build them from scalar values so that the
    // loads take them from SGPRs
    auto uniform_ptr = [](const void* ptr) {
      const uint64_t v = (uint64_t)ptr;
      const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
      const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
      return (void*)(((uint64_t)hi << 32) | lo);
    };
    const int nrec = __builtin_amdgcn_readfirstlane(p.N * (FMT == 1 ? 32 : 128));
    sc.rk = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr((const uint8_t*)p.kidx + (int64_t)b * nrec), (short)0, nrec,
                                              0x00020000);
    sc.rs = sc.rk;
    if (FMT == 1)
      sc.rs = __builtin_amdgcn_make_buffer_rsrc(uniform_ptr(p.kidx_scale + (int64_t)b * p.N * 2), (short)0,
                                                __builtin_amdgcn_readfirstlane(p.N * 2), 0x00020000);
    sc.voff_k = (lane >> 5) * 16;
    sc.voff_s = lane >> 5;
  }
}

// Threshold sample of a work-group whose longest row sees maxnv > kCap
// entries: one entry in S, taken in runs of kRun consecutive entries (run r
// starts at entry r * kRun * S), so that a tile of 32 samples reads 4 runs
// of rows rather than 32 scattered ones.  S is chosen so that about
// kMinAbove samples lie above a cut leaving `target` entries of the row
// above it (k + 850, at most kCap - 1024), with at most kCap samples.
constexpr int kRun = 8;
__device__ __forceinline__ int sample_entry(int i, int S) {
  return (int)(((uint32_t)i / kRun) * (uint32_t)(kRun * S) + ((uint32_t)i % kRun));
}
// samples of a row of nv entries: those with sample_entry(i) < nv, a prefix
__device__ __forceinline__ int sample_count(int nv, int S) {
  const int full = nv / (kRun * S), rest = nv - full * (kRun * S);
  return full * kRun + (rest < kRun ? rest : kRun);
}
// (The sizes here are work-group uniform, but integer division runs on the
// vector unit, a 64-bit one as about 100 instructions: every division below
// is 32-bit.)
__device__ __forceinline__ int sample_stride(int maxnv, int k, int& target) {
  target = k + 850;
  if (target > kCap - 1024) target = kCap - 1024;
  // want = min(ceil(kMinAbove * maxnv / target), kCap); below the cap the
  // product is under 2^24
  const bool capped = (uint32_t)maxnv * (uint32_t)kMinAbove >= (uint32_t)(kCap - 1) * (uint32_t)target + 1u ||
                      maxnv >= (1 << 23);
  const uint32_t want =
      capped ? (uint32_t)kCap : ((uint32_t)kMinAbove * (uint32_t)maxnv + (uint32_t)target - 1u) / (uint32_t)target;
  return (int)(((uint32_t)maxnv + want - 1u) / want);
}

// Workspace row of the split path (few query rows over long entry lists):
// the row's threshold, then the candidates the partitions append.
struct SplitRow {
  int cnt;
  float thr;      // the sampled threshold (rows scored against one threshold)
  uint32_t tkey;  // order key every entry left out is below (rows cut per partition)
  int pad;
  uint2 cand[kCap];
};
static_assert(sizeof(SplitRow) == kSplitRowBytes, "split workspace row size");

// SPLIT 0: the whole selection.  SPLIT 1: only the threshold of each token
// row, written to its workspace row.  SPLIT 2: the exact selection among the
// candidates the partitions appended to the workspace row.
template <int QT, int FMT, int SPLIT = 0>
__global__ __launch_bounds__(Shape<QT>::T) void index_topk_kernel(IndexParams p) {
  constexpr int kWaves = Shape<QT>::W, kThreads = Shape<QT>::T, kTile = Shape<QT>::Tile, kReg = Shape<QT>::Reg;
  constexpr int TPL = Shape<QT>::TPL;
  __shared__ TopkSmem<QT> sm;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: region offsets stay scalar
  const int nblk = (p.n + QT - 1) / QT;
  const int b = blockIdx.x / nblk;
  const int q0 = (nblk - 1 - (int)(blockIdx.x % nblk)) * QT;  // heavy (late) blocks first

  // visible entries of token q: (q_pos0 + q + 1) / m, capped at N (one
  // division, then stepped token by token)
  int nv[QT];
  int maxnv = 0;
  bool all_small = true;
  // (a shift for a power-of-two m)
  const int64_t xq = p.q_pos0 + q0 + 1;
  int64_t cq;
  if ((p.m & (p.m - 1)) == 0) {
    cq = xq >> __builtin_ctz((uint32_t)p.m);
  } else {
    cq = xq / p.m;
  }
  int rq = (int)(xq - cq * p.m);
#pragma unroll
  for (int j = 0; j < QT; ++j) {
    const int q = q0 + j;
    int v = 0;
    if (q < p.n) {
      v = (int)(cq < p.N ? cq : p.N);
      if (v > p.k) all_small = false;
    }
    nv[j] = v;
    maxnv = v > maxnv ? v : maxnv;
    if (++rq == p.m) { rq = 0; ++cq; }
  }
  SplitRow* srow = SPLIT != 0 ? (SplitRow*)p.ws + ((int64_t)b * p.n + q0) : nullptr;
  if (all_small) {
    if (SPLIT == 1) {  // nothing to score: the selection stage writes 0 .. n_vis-1
      if (tid == 0) { srow->cnt = 0; srow->thr = __builtin_inff(); }
      return;
    }
#pragma unroll
    for (int j = 0; j < QT; ++j) {
      const int q = q0 + j;
      if (q < p.n) {
        int32_t* o = p.idx_out + ((int64_t)b * p.n + q) * p.k;
        for (int i = tid; i < p.k; i += kThreads) o[i] = i < nv[j] ? canon_all(i, nv[j]) : -1;
      }
    }
    return;
  }

  // ---- A operand: rows (token, head); lane row = lane % 32, k-block = lane / 32
  // (the split selection scores only on its exact path: set up there)
  Scorer<FMT> sc;
  int nvl[2];
  if (SPLIT != 2) init_scorer<QT, FMT>(sc, p, b, q0, nv, nvl);
  const int jl0 = lane >> 5;  // this lane's tokens: jl0 + 2 tt, tt < TPL
  const int l32 = lane & 31;
  const int grp_j = wave % QT, grp_h = wave / QT;  // this wave's token group and member index
  constexpr int G = kWaves / QT;                    // waves per token group
  constexpr int NS = kCap / G / 64;                 // register slots per lane in a group selection

  // ---- phase 1: per-token thresholds from a sample (sample_entry(i, S))
  const bool sampling = maxnv > kCap;
  int target = 0;
  const int S = sampling ? sample_stride(maxnv, p.k, target) : 1;
  // Sparser than 1/32, kCap samples leave too few above the cut for a
  // reliable count: the first sample then sets a low cut (about 4 x target
  // entries above it) and a 4x denser second sample, filtered by that cut,
  // sets the final one.
  const bool two_stage = sampling && S >= 32;
  const int target_a = two_stage ? 4 * target : target;
  if (tid < QT) { sm.cnt[tid] = 0; sm.thr[tid] = -__builtin_inff(); }
  if (tid == 0) { sm.fallback = 0; sm.ties = 0; sm.staged = 0; sm.above = 0; }
  if (SPLIT != 2 && sampling) {
    // sample tiles wave, wave + kWaves, ...; kDepth tiles in flight per wave
    const int ntile = (sample_count(maxnv, S) + 31) / 32;
    // sample_entry(tile * 32 + l32, S) = tile * 32 S + sample_entry(l32, S):
    // a uniform tile offset plus a lane constant (no per-tile division)
    const int soff = sample_entry(l32, S), tstride = __builtin_amdgcn_readfirstlane(32 * S);
    BTile<FMT> t[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      t[u] = sc.load((wave + u * kWaves) * tstride + soff);
      __builtin_amdgcn_sched_barrier(0);  // issue order = consumption order (tight waits)
    }
    for (int tile0 = wave; tile0 < ntile; tile0 += kDepth * kWaves) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        // unconditional: tiles past the end store nothing (e >= nvl)
        const int tile = tile0 + u * kWaves;
        const f32x16 C = sc.mfma(t[u]);
        t[u] = sc.load((tile + kDepth * kWaves) * tstride + soff);
        float I[2];
        sc.template epilogue<TPL>(C, I);
        // The MFMA takes operands from all 64 lanes.  Its result must be used
        // outside the lane-masked store below, or the compiler may move the
        // MFMA and its operand set-up under that mask, where the masked-off
        // lanes would feed stale registers.
        asm volatile("" : "+v"(I[0]), "+v"(I[1]));
        const int i = tile * 32 + l32;
        const int e = tile * tstride + soff;  // sample_entry(i, S)
#pragma unroll
        for (int tt = 0; tt < TPL; ++tt) {
          const int j = jl0 + 2 * tt;
          if (j < QT && e < nvl[tt]) sm.cand[j][i].x = __float_as_uint(I[tt]);
        }
      }
    }
    __syncthreads();
    // sample quantile: sample i of token j sits in slot m of member h, lane
    // l with i = (m * G + h) * 64 + l, so every member holds a share
    const int nsj = (q0 + grp_j < p.n && nv[grp_j] > kCap) ? sample_count(nv[grp_j], S) : 0;
    uint32_t kr[NS];
#pragma unroll
    for (int m = 0; m < NS; ++m) {
      const int i = (m * G + grp_h) * 64 + lane;
      kr[m] = i < nsj ? okey(sm.cand[grp_j][i].x) : 0u;
    }
    // target_a * nsj < 2^26: a 32-bit division
    int r = nsj > 0 ? (int)(((uint32_t)target_a * (uint32_t)nsj + (uint32_t)nv[grp_j] - 1u) / (uint32_t)nv[grp_j]) : 0;
    r = r < 1 ? 1 : (r > nsj ? nsj : r);
    // the cut need not be exact (a bin of up to r/16 samples is close enough);
    // never above the r-th sample; at least the order key of -inf
    const uint32_t cut = group_cut<QT, NS>(sm, kr, (uint32_t)r, nsj > 0);
    if (nsj > 0 && grp_h == 0 && lane == 0) sm.thr[grp_j] = key_to_float(max(cut, 0x007fffffu));

    if (two_stage) {
      __syncthreads();  // first cuts visible; the sample buffers are free
      float thr_a[2];
#pragma unroll
      for (int tt = 0; tt < TPL; ++tt) {
        const int j = jl0 + 2 * tt;
        thr_a[tt] = (j < QT) ? sm.thr[j < QT ? j : 0] : 0.0f;
        asm volatile("" : "+v"(thr_a[tt]));
      }
      // second sample (sample_entry(i, SB)) filtered by the first cut into the
      // wave-private regions of the token buffers
      const int SB = S / 4;
      const int ntile_b = (sample_count(maxnv, SB) + 31) / 32;
      const int soffb = sample_entry(l32, SB), tstrideb = __builtin_amdgcn_readfirstlane(32 * SB);
      uint32_t wc2[2][2] = {{0u, 0u}, {0u, 0u}};
      BTile<FMT> t[kDepth];
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        t[u] = sc.load((wave + u * kWaves) * tstrideb + soffb);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int tile0 = wave; tile0 < ntile_b; tile0 += kDepth * kWaves) {
#pragma unroll
        for (int u = 0; u < kDepth; ++u) {
          const int tile = tile0 + u * kWaves;
          const f32x16 C = sc.mfma(t[u]);
          t[u] = sc.load((tile + kDepth * kWaves) * tstrideb + soffb);
          float I[2];
          sc.template epilogue<TPL>(C, I);
          const int e = tile * tstrideb + soffb;  // sample_entry(tile * 32 + l32, SB)
#pragma unroll
          for (int tt = 0; tt < TPL; ++tt)
            append_private<QT>(sm, e < nvl[tt], I[tt] >= thr_a[tt], __float_as_uint(I[tt]), e, jl0 + 2 * tt, wc2[tt]);
        }
      }
      if (lane == 0) {
#pragma unroll
        for (int tt = 0; tt < TPL; ++tt)
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            if (hf + 2 * tt < QT) sm.wcnt[wave][hf + 2 * tt] = (int)wc2[tt][hf];
      }
      __syncthreads();
      // cut of the second sample among the kept ones (regions as in the final selection)
      constexpr int kPer = kReg / 64;
      uint32_t kb[NS];
      uint32_t smb = 0u;
      int kept = 0;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) kept += min(sm.wcnt[w][grp_j], kReg);
#pragma unroll
      for (int rr = 0; rr < QT; ++rr) {
        const int w = grp_h * QT + rr;
        const int cw = min(sm.wcnt[w][grp_j], kReg);
#pragma unroll
        for (int m = 0; m < kPer; ++m) {
          const int sl = rr * kPer + m;
          const int pos = lane + 64 * m;
          smb |= (64 * m < cw ? 1u : 0u) << sl;
          const uint32_t x = sm.cand[grp_j][w * kReg + (pos < cw ? pos : 0)].x;
          kb[sl] = pos < cw ? okey(x) : 0u;
        }
      }
      const int nsb = nsj > 0 ? sample_count(nv[grp_j], SB) : 0;
      const int rb = nsb > 0 ? (int)(((uint32_t)target * (uint32_t)nsb + (uint32_t)nv[grp_j] - 1u) / (uint32_t)nv[grp_j]) : 0;
      // too few kept (the first cut was too high): keep the first cut
      const bool act = nsj > 0 && rb >= 1 && kept >= rb;
      const RadixOut rob = group_radix<QT, NS>(sm, kb, smb, (uint32_t)(rb < 1 ? 1 : rb), (uint32_t)kept, act,
                                               (uint32_t)(rb >> 4));
      if (act && grp_h == 0 && lane == 0) sm.thr[grp_j] = key_to_float(max(rob.T, 0x007fffffu));
    }
  }
  __syncthreads();
  if constexpr (SPLIT == 1) {
    if (tid == 0) { srow->cnt = 0; srow->thr = sm.thr[0]; srow->tkey = 0u; }
    return;
  }

  if constexpr (SPLIT == 2) {
    // ---- the candidates appended by the partitions, laid out as the regions;
    // count those at or above the row's bound (every entry left out lies
    // below it, so with k of them the top-k are all candidates).  Every load
    // is issued before the first use (one memory round trip); the slots past
    // the count hold stale values and are not used.
    constexpr int kPerT = kCap / kThreads;
    uint2 v[kPerT];
#pragma unroll
    for (int u = 0; u < kPerT; ++u) v[u] = srow->cand[tid + u * kThreads];
    const int cnt = srow->cnt;
    const uint32_t tkey = srow->tkey;
    const int cc = cnt < kCap ? cnt : kCap;
    int ab = 0;
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      const int i = tid + u * kThreads;
      if (i < cc) {
        sm.cand[0][i] = v[u];
        ab += okey(v[u].x) >= tkey ? 1 : 0;
      }
    }
    for (int off = 32; off >= 1; off >>= 1) ab += __shfl_xor(ab, off);
    if (lane == 0 && ab) atomicAdd(&sm.above, ab);
    if (tid < kWaves) {
      const int c0 = cc - tid * kReg;
      sm.wcnt[tid][0] = c0 < 0 ? 0 : (c0 > kReg ? kReg : c0);
    }
    if (tid == 0 && cnt > kCap) sm.fallback = 1;  // candidates were dropped
  } else {
  // ---- phase 2: every entry scored once; candidates >= threshold appended
    float thr2[2];
  #pragma unroll
    for (int tt = 0; tt < TPL; ++tt) {
      const int j = jl0 + 2 * tt;
      // rows past n (or slots past QT) never pass: the full tiles below do
      // not test visibility
      thr2[tt] = (j < QT && nvl[tt] > 0) ? sm.thr[j < QT ? j : 0] : __builtin_inff();
      // the LDS read completes here, not inside the scoring loop (whose LDS
      // stores would otherwise be waited for on every tile)
      asm volatile("" : "+v"(thr2[tt]));
    }
    {
      // kDepth tiles in flight per wave; each tile's registers are reloaded
      // right after its MFMA has read them.  Wave w scores the tiles
      // T = e / 32 with T % kWaves == w, in ascending order, so its region of
      // a token's buffer holds that token's candidates of those tiles in
      // ascending entry order.
      const int ecol = wave * 32 + l32;
      uint32_t wcnt[2][2] = {{0u, 0u}, {0u, 0u}};
      BTile<FMT> t[kDepth];
  #pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        t[u] = sc.load(u * kTile + ecol);
        __builtin_amdgcn_sched_barrier(0);  // issue order = consumption order (tight waits)
      }
      int base = 0;
      // Groups every entry of which every token sees, while no region can
      // fill within a group (both tested on the scalar unit): append_full.
      // Work-groups with a slot past QT or past the last row (QT = 1, the
      // batch row's end) take the checked loop only.
      int nvmin = nv[0];
  #pragma unroll
      for (int j = 1; j < QT; ++j) nvmin = nv[j] < nvmin ? nv[j] : nvmin;
      if (QT < 2 || q0 + QT > p.n) nvmin = 0;
      const int nfull = __builtin_amdgcn_readfirstlane(nvmin / (kDepth * kTile));
      uint32_t upper = lane >= 32 ? 0xffffffffu : 0u;
      asm volatile("" : "+v"(upper));  // an opaque mask: one v_and per tile, not a move and a select
      for (int g = 0; g < nfull; ++g, base += kDepth * kTile) {
        uint32_t wmax = 0;
  #pragma unroll
        for (int tt = 0; tt < TPL; ++tt) wmax = max(wmax, max(wcnt[tt][0], wcnt[tt][1]));
        if (__builtin_amdgcn_readfirstlane((int)wmax) > kReg - kDepth * 32) break;
  #pragma unroll
        for (int u = 0; u < kDepth; ++u) {
          const f32x16 C = sc.mfma(t[u]);
          t[u] = sc.load(base + (u + kDepth) * kTile + ecol);
          const int e = base + u * kTile + ecol;
          float I[2];
          sc.template epilogue<TPL>(C, I);
  #pragma unroll
          for (int tt = 0; tt < TPL; ++tt)
            append_full<QT>(sm, I[tt] >= thr2[tt], __float_as_uint(I[tt]), e, 2 * tt, wave, upper, wcnt[tt]);
        }
      }
      for (; base < maxnv; base += kDepth * kTile) {
  #pragma unroll
        for (int u = 0; u < kDepth; ++u) {  // unconditional: tiles past the end never pass
          const f32x16 C = sc.mfma(t[u]);
          t[u] = sc.load(base + (u + kDepth) * kTile + ecol);
          const int e = base + u * kTile + ecol;
          float I[2];
          sc.template epilogue<TPL>(C, I);
  #pragma unroll
          for (int tt = 0; tt < TPL; ++tt)
            append_private<QT>(sm, e < nvl[tt], I[tt] >= thr2[tt], __float_as_uint(I[tt]), e, jl0 + 2 * tt, wcnt[tt]);
        }
      }
      if (lane == 0) {
  #pragma unroll
        for (int tt = 0; tt < TPL; ++tt)
  #pragma unroll
          for (int hf = 0; hf < 2; ++hf)
            if (hf + 2 * tt < QT) sm.wcnt[wave][hf + 2 * tt] = (int)wcnt[tt][hf];
      }
    }
  }
  __syncthreads();
  if (wave < QT && lane == 0) {
    int c = 0;
    bool over = false;
    for (int w = 0; w < kWaves; ++w) {
      c += sm.wcnt[w][wave];
      over |= sm.wcnt[w][wave] > kReg;
    }
    sm.cnt[wave] = c;
    const int want = nv[wave] < p.k ? nv[wave] : p.k;
    if (over || c < want || (SPLIT == 2 && sm.above < want)) atomicOr(&sm.fallback, 1);
  }
  __syncthreads();

  if (sm.fallback) {
    // ---- exact streaming fallback for every token of this work-group
    if (SPLIT == 2) init_scorer<QT, FMT>(sc, p, b, q0, nv, nvl);
    if (tid == 0 && p.fallback_count) atomicAdd(p.fallback_count, 1u);
    if (tid < QT) { sm.cnt[tid] = 0; sm.thr[tid] = __uint_as_float(0u); }
    __syncthreads();
    for (int base = 0; base < maxnv; base += kTile) {
      const int e0 = base + wave * 32;
      const int e = e0 + l32;
      bool pass[2] = {false, false};
      uint32_t val[2] = {0u, 0u};
      if (e0 < maxnv) {
        float I[2];
        sc.template score<TPL>(e, I);
#pragma unroll
        for (int tt = 0; tt < TPL; ++tt) {
          const int j = jl0 + 2 * tt;
          const uint32_t u = okey(__float_as_uint(I[tt]));
          val[tt] = u;
          pass[tt] = (j < QT) && (e < nvl[tt]) && (u >= __float_as_uint(sm.thr[j < QT ? j : 0]));
        }
      }
      append<QT>(sm, pass, val, e, jl0);
      __syncthreads();
      int cnow[QT];
#pragma unroll
      for (int j = 0; j < QT; ++j) cnow[j] = sm.cnt[j];
      __syncthreads();  // every thread has read the counts before any can change
#pragma unroll
      for (int j = 0; j < QT; ++j)
        if (cnow[j] > kCap - kTile) wg_shrink_exact(sm, j, p.k);
    }
    for (int j = 0; j < QT; ++j) {
      const int q = q0 + j;
      if (q >= p.n) break;
      wg_shrink_exact(sm, j, p.k);
      const int cnt = sm.cnt[j];
      wg_bitonic_sort(sm, j, cnt);
      int32_t* o = p.idx_out + ((int64_t)b * p.n + q) * p.k;
      for (int i = tid; i < p.k; i += kThreads) o[i] = i < cnt ? (int32_t)sm.cand[j][i].y : -1;
      __syncthreads();
    }
    return;
  }

  // ---- phase 3: each token's group selects its exact top-k among the
  // candidates and writes their indices
  {
    const int j = grp_j;
    const int q = q0 + j;
    const bool live = q < p.n;
    const int kk = nv[j] < p.k ? nv[j] : p.k;
    // member h holds regions h*QT .. h*QT + QT - 1; slot s = (region, m) <-> position lane + 64m
    constexpr int kPer = kReg / 64;
    uint32_t kr[NS];
    uint32_t ir[NS];
    uint32_t smask = 0u;
#pragma unroll
    for (int rr = 0; rr < QT; ++rr) {
      const int w = grp_h * QT + rr;
      const int cw = sm.wcnt[w][j];
#pragma unroll
      for (int m = 0; m < kPer; ++m) {
        const int sl = rr * kPer + m;
        const int pos = lane + 64 * m;
        smask |= (64 * m < cw ? 1u : 0u) << sl;
        const uint2 v = sm.cand[j][w * kReg + (pos < cw ? pos : 0)];
        kr[sl] = pos < cw ? okey(v.x) : 0u;
        ir[sl] = v.y;
      }
    }
    const int c = sm.cnt[j];
    const bool sel = live && c > kk;
    uint32_t keep = 0u;
    {
      const RadixOut ro = group_radix<QT, NS>(sm, kr, smask, (uint32_t)kk, (uint32_t)c, sel);
      const bool need_ties = sel && ro.exact && (uint32_t)kk - ro.above < ro.inbin;
      if (need_ties && grp_h == 0 && lane == 0) sm.ties = 1;
      __syncthreads();
      uint32_t tinv = 0u;
      if (sm.ties) {
        // ties at the k-th score: keep the (kk - above) smallest entry indices among them
        uint32_t k2[NS];
#pragma unroll
        for (int sl = 0; sl < NS; ++sl) k2[sl] = (need_ties && kr[sl] == ro.T) ? ~ir[sl] : 0u;
        const RadixOut r2 = group_radix<QT, NS>(sm, k2, smask, (uint32_t)kk - ro.above, ro.inbin, need_ties);
        tinv = r2.T;
      }
      const uint32_t Tr = sel ? max(ro.T, 1u) : 1u;  // empty slots (key 0) are never kept
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        bool kp = kr[sl] >= Tr;
        if (need_ties && kr[sl] == ro.T) kp = ~ir[sl] >= tinv;
        keep |= (kp ? 1u : 0u) << sl;
      }
    }
    // output in the canonical order, then -1 padding
    int32_t* o = p.idx_out + ((int64_t)b * p.n + (live ? q : 0)) * p.k;
    if constexpr (SPLIT == 0) {
      emit_canonical<QT, NS>(sm, live, ir, keep, kk, p.k, o);
    } else if (nv[0] <= 64 * kCap) {
      // the split path's candidates arrived in atomic order.  Rows of at
      // most 64 kCap entries: the kept entries become a bitmap in the (free)
      // candidate buffer, one 32-bit word per 32-entry tile, read in the
      // canonical order: wave v takes the tiles T = 8 i + v, each lane a run
      // of consecutive i, and writes their set bits in ascending order.
      static_assert(kWaves == 8 && sizeof(sm.cand[0]) == 64 * kCap / 8, "one wave per canonical group, 32 entries a word");
      uint32_t* bm = (uint32_t*)&sm.cand[0][0];
      const int nw = (nv[0] + 31) >> 5;
      __syncthreads();  // the selection's lists in the buffer are read
      for (int i = tid; i < nw; i += kThreads) bm[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int sl = 0; sl < NS; ++sl)
        if ((keep >> sl) & 1u) atomicOr(&bm[ir[sl] >> 5], 1u << (ir[sl] & 31u));
      __syncthreads();
      const int v = wave;
      const int nwv = nw > v ? (nw - v + 7) >> 3 : 0;  // tiles of group v
      const int per = (nwv + 63) >> 6;                 // per lane, at most 2 kCap / 512
      const int i0 = lane * per;
      uint32_t c = 0u;
      for (int t = 0; t < per; ++t)
        if (i0 + t < nwv) c += (uint32_t)__builtin_popcount(bm[8 * (i0 + t) + v]);
      const uint32_t incl = wave_prefix_sum(c);
      if (lane == 63) sm.vcnt[0][v] = incl;
      __syncthreads();
      uint32_t pos = incl - c;
      for (int u = 0; u < v; ++u) pos += sm.vcnt[0][u];
      if (live) {
        for (int t = 0; t < per; ++t) {
          const int i = i0 + t;
          if (i >= nwv) break;
          uint32_t w = bm[8 * i + v];
          while (w) {
            if (pos < (uint32_t)p.k) o[pos] = 32 * (8 * i + v) + __builtin_ctz(w);
            ++pos;
            w &= w - 1u;
          }
        }
        for (int i = kk + tid; i < p.k; i += kThreads) o[i] = -1;
      }
    } else {
      // longer rows: stage the kept entries and sort them into the canonical
      // order
      int mine = 0;
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) mine += __builtin_popcountll(ballot((keep >> sl) & 1u));
      int pos = 0;
      if (lane == 0 && mine) pos = atomicAdd(&sm.staged, mine);  // this wave's range of the staging area
      pos = __builtin_amdgcn_readfirstlane(pos);
#pragma unroll
      for (int sl = 0; sl < NS; ++sl) {
        const bool kp = (keep >> sl) & 1u;
        const uint64_t bal = ballot(kp);
        const int rank = (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u));
        if (kp && pos + rank < kCap) sm.cand[0][pos + rank].y = ir[sl];
        pos += __builtin_popcountll(bal);
      }
      __syncthreads();
      wg_bitonic_sort(sm, 0, kk);
      if (live)
        for (int i = tid; i < p.k; i += kThreads) o[i] = i < kk ? (int32_t)sm.cand[0][i].y : -1;
    }
  }
}

// Split path, partition stage: one work-group of 4 waves scores entries
// [part*part_len, (part+1)*part_len) of one token row against the row's
// threshold and appends the passing ones to the row's workspace candidates
// (one atomic per wave and tile with a passing lane).
template <int FMT>
__global__ __launch_bounds__(256) void index_split_score_kernel(IndexParams p, int parts, int part_len) {
  constexpr int W = 4;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t row = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const int b = (int)(row / p.n), q = (int)(row % p.n);
  SplitRow* srow = (SplitRow*)p.ws + row;
  const float thr = srow->thr;
  if (!(thr < __builtin_inff())) return;  // n_vis <= k: nothing to select
  const int64_t c = (p.q_pos0 + q + 1) / p.m;
  const int nv = (int)(c < p.N ? c : p.N);
  const int e0 = part * part_len;
  const int e1 = nv < e0 + part_len ? nv : e0 + part_len;
  if (e0 >= e1) return;
  Scorer<FMT> sc;
  int nvl[2];
  const int nvq[1] = {nv};
  init_scorer<1, FMT>(sc, p, b, q, nvq, nvl);
  const int l32 = lane & 31;
  const int ntile = (e1 - e0 + 31) / 32;
  BTile<FMT> t[kDepth];
#pragma unroll
  for (int u = 0; u < kDepth; ++u) {
    t[u] = sc.load(e0 + (wave + u * W) * 32 + l32);
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int tile0 = wave; tile0 < ntile; tile0 += kDepth * W) {
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      const int tile = tile0 + u * W;
      const f32x16 C = sc.mfma(t[u]);
      t[u] = sc.load(e0 + (tile + kDepth * W) * 32 + l32);
      float I[2];
      sc.template epilogue<1>(C, I);
      const int e = e0 + tile * 32 + l32;
      const bool pass = lane < 32 && e < e1 && I[0] >= thr;  // token 0 lives in lanes 0..31
      const uint64_t bal = ballot(pass);
      if (bal) {
        int base = 0;
        if (lane == 0) base = atomicAdd(&srow->cnt, __builtin_popcountll(bal));
        base = __builtin_amdgcn_readfirstlane(base);
        const int rank = (int)__builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0u);
        if (pass && base + rank < kCap) srow->cand[base + rank] = make_uint2(__float_as_uint(I[0]), (uint32_t)e);
      }
    }
  }
}

// Split path, one-pass partition stage (rows of at most kCutMaxN entries):
// one work-group of 8 waves scores entries [part * kCutPart, ...) of one
// token row into LDS and keeps about r_keep of its highest: a 256-bin
// histogram over the part's score range [lo, hi] (one more level over the
// cut bin when that bin is crowded) gives a cut, and every entry at or above
// the cut is appended to the row's candidates with one atomic per
// work-group.  The bin of a score is monotone in the score, so every entry
// left out lies below the smallest kept one, t_p; the row's maximum of the
// t_p goes to the workspace row, and the selection stage takes the row's
// exact path unless at least k candidates reach it (then every member of the
// row's top-k is a candidate, ties included).
constexpr int kCutPart = 16384;
constexpr int kCutMaxN = 16 * kCutPart;
constexpr int kCutKeep = 1024;  // kept entries per part staged in LDS

__global__ __launch_bounds__(256) void index_split_init_kernel(IndexParams p, int64_t rows) {
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (r < rows) {
    SplitRow* s = (SplitRow*)p.ws + r;
    s->cnt = 0;
    s->thr = 0.0f;
    s->tkey = 0u;
  }
}

// Bin of score x in [lo, hi] (256 bins of width 1 / inv), monotone in x:
// (x - lo) * inv is rounded monotonically, then clamped to [0, 255].
__device__ __forceinline__ int cut_bin(float x, float lo, float inv) {
  const float f = (x - lo) * inv;
  return !(f > 0.0f) ? 0 : (f >= 255.0f ? 255 : (int)f);
}

template <int FMT>
__global__ __launch_bounds__(512) void index_split_cut_kernel(IndexParams p, int parts, int r_keep) {
  constexpr int W = 8, T = 64 * W;
  __shared__ __attribute__((aligned(16))) float ssc[kCutPart];
  __shared__ uint2 kept[kCutKeep];
  __shared__ uint32_t hist[256];
  __shared__ float red[2][W];
  __shared__ int s_cut[2], s_nkept, s_base;
  __shared__ uint32_t s_tmin;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t row = blockIdx.x / parts;
  const int part = (int)(blockIdx.x % parts);
  const int b = (int)(row / p.n), q = (int)(row % p.n);
  SplitRow* srow = (SplitRow*)p.ws + row;
  const int64_t c = (p.q_pos0 + q + 1) / p.m;
  const int nv = (int)(c < p.N ? c : p.N);
  const int e0 = part * kCutPart;
  const int e1 = nv < e0 + kCutPart ? nv : e0 + kCutPart;
  if (nv <= p.k || e0 >= e1) return;  // the selection stage writes 0 .. nv-1 / past the row
  const int n = e1 - e0;
  Scorer<FMT> sc;
  int nvl[2];
  const int nvq[1] = {nv};
  init_scorer<1, FMT>(sc, p, b, q, nvq, nvl);
  const int l32 = lane & 31;
  if (tid < 256) hist[tid] = 0u;
  if (tid == 0) { s_nkept = 0; s_tmin = 0xffffffffu; }

  // ---- score the part into LDS (token 0 lives in lanes 0..31)
  float lo = __builtin_inff(), hi = -__builtin_inff();
  {
    const int ntile = (n + 31) >> 5;
    BTile<FMT> t[kDepth];
#pragma unroll
    for (int u = 0; u < kDepth; ++u) {
      t[u] = sc.load(e0 + (wave + u * W) * 32 + l32);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int tile0 = wave; tile0 < ntile; tile0 += kDepth * W) {
#pragma unroll
      for (int u = 0; u < kDepth; ++u) {
        const int tile = tile0 + u * W;
        const f32x16 C = sc.mfma(t[u]);
        t[u] = sc.load(e0 + (tile + kDepth * W) * 32 + l32);
        float I[2];
        sc.template epilogue<1>(C, I);
        // the MFMA's result is used outside the lane mask below (see the
        // sampling loop of index_topk_kernel)
        asm volatile("" : "+v"(I[0]));
        const int i = tile * 32 + l32;
        if (lane < 32 && i < n) {
          ssc[i] = I[0];
          lo = fminf(lo, I[0]);
          hi = fmaxf(hi, I[0]);
        }
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, off));
    hi = fmaxf(hi, __shfl_xor(hi, off));
  }
  if (lane == 0) { red[0][wave] = lo; red[1][wave] = hi; }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < W; ++w) { lo = fminf(lo, red[0][w]); hi = fmaxf(hi, red[1][w]); }
  const float inv = 256.0f / (hi - lo);
  const bool spread = hi > lo && inv < __builtin_inff();

  // highest bin b with (bins >= b) + base >= need; -1 if none (wave 0)
  auto find_cut = [&](int need, int& above) -> int {
    uint32_t h[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) h[i] = hist[4 * lane + i];
    const uint32_t s4 = h[0] + h[1] + h[2] + h[3];
    uint32_t suf = s4;  // bins 4 * lane and above
    for (int off = 1; off < 64; off <<= 1) {
      const uint32_t y = __shfl_down(suf, off);
      if (lane + off < 64) suf += y;
    }
    uint32_t S = suf - s4;  // bins above this lane's four
    int bl = -1, ab = 0;
#pragma unroll
    for (int i = 3; i >= 0; --i) {
      if (bl < 0 && S + h[i] >= (uint32_t)need) { bl = 4 * lane + i; ab = (int)S; }
      S += h[i];
    }
    int best = bl;
    for (int off = 32; off >= 1; off >>= 1) best = max(best, __shfl_xor(best, off));
    above = best >= 0 ? __shfl(ab, best >> 2) : 0;
    return best;
  };

  int cut = 0, sub = 0;
  float lo2 = 0.0f, inv2 = 0.0f;
  // the passes below read 4 consecutive scores per thread (n4 of them; the
  // scores at n .. n4-1 are never read as entries)
  const int n4 = (n + 3) & ~3;
  if (spread) {
    for (int i = 4 * tid; i < n4; i += 4 * T) {
      const f32x4 x = *(const f32x4*)&ssc[i];
#pragma unroll
      for (int k = 0; k < 4; ++k)
        if (i + k < n) atomicAdd(&hist[cut_bin(x[k], lo, inv)], 1u);
    }
    __syncthreads();
    if (wave == 0) {
      int above = 0;
      const int cb = find_cut(r_keep, above);
      const int crowd = cb >= 0 ? (int)hist[cb] + above - r_keep : 0;
      // still needed from the cut bin when it holds more than 16 extra
      if (lane == 0) { s_cut[0] = cb < 0 ? 0 : cb; s_cut[1] = (cb >= 0 && crowd > 16) ? r_keep - above : 0; }
    }
    __syncthreads();
    cut = s_cut[0];
    const int need2 = inv * 256.0f < __builtin_inff() ? s_cut[1] : 0;
    if (need2 > 0) {
      // the cut bin is crowded: a second histogram over its range
      lo2 = lo + (float)cut / inv;
      inv2 = inv * 256.0f;
      if (tid < 256) hist[tid] = 0u;
      __syncthreads();
      for (int i = 4 * tid; i < n4; i += 4 * T) {
        const f32x4 x = *(const f32x4*)&ssc[i];
#pragma unroll
        for (int k = 0; k < 4; ++k)
          if (i + k < n && cut_bin(x[k], lo, inv) == cut) atomicAdd(&hist[cut_bin(x[k], lo2, inv2)], 1u);
      }
      __syncthreads();
      if (wave == 0) {
        int above = 0;
        const int sb = find_cut(need2, above);
        if (lane == 0) s_cut[1] = sb < 0 ? 0 : sb;
      }
      __syncthreads();
      sub = s_cut[1];
    }
  }
  const bool drops = spread && (cut > 0 || sub > 0);

  // ---- append the kept entries to LDS (one LDS atomic per wave and pass),
  // then to the row with one atomic
  uint32_t tmin = 0xffffffffu;
  for (int i0 = 0; i0 < n4; i0 += 4 * T) {  // every lane takes every pass (cross-lane sums below)
    const int i = i0 + 4 * tid;
    const f32x4 x = *(const f32x4*)&ssc[i < n4 ? i : 0];
    uint32_t kb = 0u;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      bool kp = i + k < n;
      if (spread && kp) {
        const int b1 = cut_bin(x[k], lo, inv);
        kp = b1 > cut || (b1 == cut && (sub == 0 || cut_bin(x[k], lo2, inv2) >= sub));
      }
      kb |= (kp ? 1u : 0u) << k;
    }
    const uint32_t mine = (uint32_t)__builtin_popcount(kb);
    if (!__builtin_amdgcn_ballot_w64(mine != 0u)) continue;  // nothing kept in this wave's 256 scores
    const uint32_t incl = wave_prefix_sum(mine);
    int base = 0;
    if (lane == 63) base = atomicAdd(&s_nkept, (int)incl);
    int pos = __builtin_amdgcn_readlane(base, 63) + (int)(incl - mine);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      if ((kb >> k) & 1u) {
        if (pos < kCutKeep) kept[pos] = make_uint2(__float_as_uint(x[k]), (uint32_t)(e0 + i + k));
        tmin = min(tmin, okey(__float_as_uint(x[k])));
        ++pos;
      }
    }
  }
  for (int off = 32; off >= 1; off >>= 1) tmin = min(tmin, (uint32_t)__shfl_xor((int)tmin, off));
  if (lane == 0) atomicMin(&s_tmin, tmin);
  __syncthreads();
  if (tid == 0) {
    const int m = s_nkept;
    // too many kept for the staging area: count past the row's capacity (exact path)
    s_base = m > kCutKeep ? -1 : atomicAdd(&srow->cnt, m);
    if (m > kCutKeep) atomicAdd(&srow->cnt, kCap + 1);
    if (drops) atomicMax(&srow->tkey, s_tmin);
  }
  __syncthreads();
  const int m = s_nkept, base = s_base;
  if (base >= 0)
    for (int i = tid; i < m && base + i < kCap; i += T) srow->cand[base + i] = kept[i];
}

// Few query rows over long entry lists (decode): the split path keeps every
// CU busy (entries scored by partitions, selection per row).
constexpr int kSplitPart = 8192;
// The choice depends on the rows of one batch entry only, never on B.
static bool split_path(int B, int n, int64_t q_pos0, int N, int m) {
  (void)B;
  if (n > 4) return false;
  int64_t nv = (q_pos0 + n) / m;
  if (nv > N) nv = N;
  return nv >= 65536;
}

size_t index_topk_workspace(int B, int n, int64_t q_pos0, int N, int m, int) {
  return split_path(B, n, q_pos0, N, m) ? (size_t)B * n * sizeof(SplitRow) : 0;
}

template <int QT>
static hipError_t launch_q(const IndexParams& p, hipStream_t stream) {
  const int nblk = (p.n + QT - 1) / QT;
  dim3 grid((unsigned)((int64_t)p.B * nblk)), block(Shape<QT>::T);
  if (p.fmt == 1)
    hipLaunchKernelGGL((index_topk_kernel<QT, 1>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((index_topk_kernel<QT, 0>), grid, block, 0, stream, p);
  return hipGetLastError();
}

template <int FMT>
static hipError_t launch_split(const IndexParams& p, hipStream_t stream) {
  const int64_t rows = (int64_t)p.B * p.n;
  int64_t nv = (p.q_pos0 + p.n) / p.m;
  if (nv > p.N) nv = p.N;
  if (nv <= kCutMaxN) {
    // one pass: each partition cuts its own scores; r_keep covers the part's
    // expected share of the top-k plus six standard deviations
    const int parts = (int)((nv + kCutPart - 1) / kCutPart);
    const double share = (double)p.k * kCutPart / (double)nv;
    const int r_keep = (int)std::ceil(share + 6.0 * std::sqrt(share) + 8.0);
    hipLaunchKernelGGL(index_split_init_kernel, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, stream, p, rows);
    hipLaunchKernelGGL((index_split_cut_kernel<FMT>), dim3((unsigned)(rows * parts)), dim3(512), 0, stream, p, parts,
                       r_keep);
  } else {
    // sampled threshold per row, then partitions scored against it
    const int parts = (int)((nv + kSplitPart - 1) / kSplitPart);
    hipLaunchKernelGGL((index_topk_kernel<1, FMT, 1>), dim3((unsigned)rows), dim3(Shape<1>::T), 0, stream, p);
    hipLaunchKernelGGL((index_split_score_kernel<FMT>), dim3((unsigned)(rows * parts)), dim3(256), 0, stream, p,
                       parts, kSplitPart);
  }
  hipLaunchKernelGGL((index_topk_kernel<1, FMT, 2>), dim3((unsigned)rows), dim3(Shape<1>::T), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_index_topk(const IndexParams& p, hipStream_t stream) {
  if ((int64_t)p.B * p.n == 0) return hipSuccess;
  if (split_path(p.B, p.n, p.q_pos0, p.N, p.m)) return p.fmt == 1 ? launch_split<1>(p, stream) : launch_split<0>(p, stream);
  if (p.n == 1) return launch_q<1>(p, stream);
  // Rows of up to 64K entries: 2-token work-groups, two per CU, so one
  // work-group's selections overlap the other's scoring.  Longer rows are
  // dominated by scoring, where 4 tokens per loaded key tile are cheaper.
  int64_t nv = (p.q_pos0 + p.n) / p.m;
  if (nv > p.N) nv = p.N;
  if (nv <= 65536) return launch_q<2>(p, stream);
  return launch_q<4>(p, stream);
}

}  // namespace csa
