// attn_plan.h -- the forward's host-side planning and argument checks: tile
// choice, GQA head packing, the split-KV plan and the validation of shapes,
// strides, alignment and aliasing.  Plain C++ (no HIP): the library uses it
// through attn_fwd.hip, and a host-only build (with AddressSanitizer and
// UBSan) exercises it on the CPU.
#ifndef ATTN_PLAN_H_
#define ATTN_PLAN_H_

#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>

#include "attn.h"
#include "attn_tiles.h"

namespace attn_planner {

using namespace attn_tiles;

// The tile every call of head dimension D may take (masked calls always do).
inline int narrow_cfg(int D) {
  if (D == 192) return kCfgD192;
  if (D == 256) return kCfgD256;
  if (D == 96 || D == 80) return kCfgD96;
  return D == 128 ? kCfgD128Narrow : kCfgD64Narrow;
}

// The wide tiles of each head dimension are used without a causal mask or an
// attention mask when they still fill every slot of the device at least
// once; at D = 128 a query range of at most 128 rows per head (decode, or a
// packed GQA group) takes the 128-row decode tile, unless masked.
inline int select_cfg(int B, int Hq, int Nq, int D, int causal, bool masked, int num_cus) {
  const int narrow = narrow_cfg(D);
  if (D != 128 && D != 64) return narrow;
  if (D == 128 && !masked && Nq <= kCfgs[kCfgD128Decode].BM()) return kCfgD128Decode;
  const int wide = D == 128 ? kCfgD128Wide : kCfgD64Wide;
  const TileCfg& w = kCfgs[wide];
  const long long wide_wgs = (long long)B * Hq * ((Nq + w.BM() - 1) / w.BM());
  const long long slots = (long long)w.resident_per_cu() * (num_cus > 0 ? num_cus : 256);
  return (!causal && !masked && wide_wgs >= slots) ? wide : narrow;
}

inline bool head_dim_ok(int D) { return D == 64 || D == 80 || D == 96 || D == 128 || D == 256; }

// Head dimensions of Q/K (D) and V/O (Dv): equal and supported, or the
// (192, 128) pair.
inline bool head_dims_ok(int D, int Dv) { return Dv == D ? head_dim_ok(D) : (D == 192 && Dv == 128); }

// Element strides of one tensor's batch, head and sequence dimensions; the
// head dimension (D) is contiguous.
struct Strides {
  int64_t b, h, n;
};
struct Layout {
  Strides q, k, v, o;
};

inline Layout contiguous_layout(int Hq, int Hkv, int Nq, int Nkv, int D, int Dv) {
  const Strides qs{(int64_t)Hq * Nq * D, (int64_t)Nq * D, D};
  const Strides ks{(int64_t)Hkv * Nkv * D, (int64_t)Nkv * D, D};
  const Strides vs{(int64_t)Hkv * Nkv * Dv, (int64_t)Nkv * Dv, Dv};
  const Strides os{(int64_t)Hq * Nq * Dv, (int64_t)Nq * Dv, Dv};
  return Layout{qs, ks, vs, os};
}

// Bytes from a tensor's base to the end of its last element.
inline __int128 extent_bytes(const Strides& s, int B, int H, int N, int D) {
  return 2 * ((__int128)(B - 1) * s.b + (__int128)(H - 1) * s.h + (__int128)(N - 1) * s.n + D);
}

inline bool overlaps128(const void* a, __int128 na, const void* b, __int128 nb) {
  const __int128 x = (__int128)(uintptr_t)a, y = (__int128)(uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Strides the kernels can take: non-negative multiples of 8 elements (so
// every row starts 16-byte aligned), row strides of at least one row (the
// K/V copies rely on rows past the last key starting beyond its end) and at
// most 2^24 elements (per-lane copy offsets are 32-bit).
inline bool strides_ok(const Strides& s, int D) {
  if (s.b < 0 || s.h < 0 || s.n < D || s.n > (1 << 24)) return false;
  return ((s.b | s.h | s.n) & 7) == 0;
}

// No two elements of the output share an address: ordered by stride, each
// dimension of extent > 1 must step over everything the smaller ones span.
inline bool dense_enough(const Strides& s, int B, int H, int N, int D) {
  int64_t st[3] = {s.b, s.h, s.n};
  int64_t sz[3] = {B, H, N};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        std::swap(st[i], st[j]);
        std::swap(sz[i], sz[j]);
      }
  __int128 span = D;  // the contiguous head dimension
  for (int i = 0; i < 3; ++i) {
    if (sz[i] == 1) continue;
    if ((__int128)st[i] < span) return false;
    span = (__int128)st[i] * sz[i];
  }
  return true;
}

// An attention mask: element (b, h, i, j) at ptr + b*sb + h*sh + i*sq + j.
struct MaskArgs {
  const void* ptr = nullptr;
  int type = ATTN_MASK_NONE;
  int64_t sb = 0, sh = 0, sq = 0;
};

inline int validate(const void* q, const void* k, const void* v, const void* out, const float* lse,
             int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv, float scale, int causal,
             int dtype, const Layout& L, const MaskArgs& M = MaskArgs()) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dims_ok(D, Dv)) return ATTN_EINVAL;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  if (!isfinite(scale)) return ATTN_EINVAL;
  if (!q || !k || !v || !out) return ATTN_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_EINVAL;
  if (((uintptr_t)lse) & 3) return ATTN_EINVAL;
  // Grid and row counts are held in 32-bit integers on the device.
  const size_t rows = (size_t)B * Hq * Nq;
  const size_t krows = (size_t)B * Hkv * Nkv;
  if (rows > (size_t)INT32_MAX || krows > (size_t)INT32_MAX) return ATTN_EINVAL;
  if (!strides_ok(L.q, D) || !strides_ok(L.k, D) || !strides_ok(L.v, Dv) ||
      !strides_ok(L.o, Dv))
    return ATTN_EINVAL;
  if (!dense_enough(L.o, B, Hq, Nq, Dv)) return ATTN_EINVAL;
  const __int128 qb = extent_bytes(L.q, B, Hq, Nq, D), ob = extent_bytes(L.o, B, Hq, Nq, Dv);
  const __int128 kb = extent_bytes(L.k, B, Hkv, Nkv, D), vb = extent_bytes(L.v, B, Hkv, Nkv, Dv);
  if (overlaps128(out, ob, q, qb) || overlaps128(out, ob, k, kb) || overlaps128(out, ob, v, vb))
    return ATTN_EINVAL;
  if (lse) {
    const __int128 lb = (__int128)rows * 4;
    if (overlaps128(lse, lb, q, qb) || overlaps128(lse, lb, k, kb) ||
        overlaps128(lse, lb, v, vb) || overlaps128(lse, lb, out, ob))
      return ATTN_EINVAL;
  }
  if (M.type != ATTN_MASK_NONE) {
    if (M.type != ATTN_MASK_BOOL && M.type != ATTN_MASK_ADD) return ATTN_EINVAL;
    if (!M.ptr || ((uintptr_t)M.ptr & 7)) return ATTN_EINVAL;
    if (M.sb < 0 || M.sh < 0 || M.sq < 0 || ((M.sb | M.sh | M.sq) & 3)) return ATTN_EINVAL;
    const int esz = M.type == ATTN_MASK_BOOL ? 1 : 2;
    const __int128 mb = esz * ((__int128)(B - 1) * M.sb + (__int128)(Hq - 1) * M.sh +
                               (__int128)(Nq - 1) * M.sq + Nkv);
    if (mb > ((__int128)1 << 62)) return ATTN_EINVAL;
    if (overlaps128(out, ob, M.ptr, mb)) return ATTN_EINVAL;
    if (lse && overlaps128(lse, (__int128)rows * 4, M.ptr, mb)) return ATTN_EINVAL;
  }
  return ATTN_OK;
}

// How one call covers its query tiles (tile index (b * Hq + h) * n_qtiles +
// qt): tiles [0, first_split) run whole and write the output directly; the
// key range of each tile in [first_split, tiles) is cut into `splits`
// pieces of `split_len` keys, computed into fp32 partials (in the same
// launch, after the whole tiles) and merged by their log-sum-exp.  Those tiles are the last ones,
// so their rows are one contiguous range [row0, rows).
struct Plan {
  int cfg;
  int Dv;  // width of the fp32 partial rows
  int n_qtiles;
  int splits;
  int split_len;
  long long tiles;
  long long first_split;
  long long row0, rows;
  size_t workspace_bytes() const {
    return splits > 1 ? (size_t)splits * (size_t)(rows - row0) * (Dv + 1) * sizeof(float) : 0;
  }
};

// Cost model for cutting `rem` equal tiles of `ktiles` key steps into s
// pieces on `slots` workgroup slots, in key steps of one workgroup: the
// pieces run in ceil(s * rem / slots) rounds, each piece spends about
// kPieceFillSteps steps filling its pipeline and writing fp32 partials, and
// the merge streams ~8 (Dv + 1) bytes per row and piece through HBM, about
// kMergeStepsPerPiece steps of the whole chip per tile and piece (a 64-key
// step of a 256-row tile is ~8 MFLOP, ~2 us on one CU).
// The merge term scales with the tile's live rows (row_frac of its BM;
// below 1 for short query ranges, e.g. decode).
constexpr double kPieceFillSteps = 2.0;
constexpr double kMergeStepsPerPiece = 0.03;
constexpr int kMaxSplits = 256;
constexpr int kMinStepsPerPiece = 4;

inline int balanced_splits(long long rem, long long slots, int ktiles, double row_frac) {
  int best = 1;
  double best_cost = (double)((rem + slots - 1) / slots) * ktiles;
  const int smax = std::min(kMaxSplits, ktiles / kMinStepsPerPiece);
  for (int s = 2; s <= smax; ++s) {
    const int steps = (ktiles + s - 1) / s;
    const double rounds = (double)((s * rem + slots - 1) / slots);
    const double cost =
        rounds * (steps + kPieceFillSteps) + kMergeStepsPerPiece * s * rem * row_frac;
    if (cost < best_cost) {
      best = s;
      best_cost = cost;
    }
  }
  return best;
}

// Causal tiles differ in length and are launched longest first, which the
// hardware's dynamic dispatch balances, so only a grid smaller than the chip
// is split, into enough pieces to fill every slot -- and only when that
// pays: a launch lasts about as long as its longest piece or its mean load
// per slot, whichever is more, and a split call adds the merge and a fixed
// cost for the second launch and the workspace.  In microseconds,
// calibrated on MI355X with forced piece counts (eager calls; e.g. causal
// GQA 14/2 at 4096 tokens, D = 64: 54-58 us whole, 80-102 us in 2-8
// pieces; 16 heads x 1024: 18 us whole, 38-44 us in 2-16; 4 heads x 2048
// at D = 128: 57 us whole, 38-45 us in 2-8): a key step of a workgroup
// takes its flops at 1 PFLOP/s over the slots, a split call costs
// kSplitFixedUs more, and the merge moves the partials (written once, read
// once) at kMergeBytesPerUs.  Query tile qt of a head (rows up to
// min((qt + 1) BM, Nq)) reaches keys below that row + coff.
constexpr double kChipFlopsPerUs = 1.0e9;
constexpr double kSplitFixedUs = 30.0;
constexpr double kMergeBytesPerUs = 3.0e6;
// A non-causal grid smaller than the device: an eager call that splits
// costs at least kSplitFloorUs (38-45 us measured over such shapes, pieces
// of 4-16 key steps included), so a grid that runs whole in less never
// splits.  Its workgroups, fewer than the CUs, run their key steps at
// about kLoneStepFactor of the shared-CU time (e.g. one
// head of 1000 tokens at D = 64: 18 us whole, 42-47 us in 2-8 pieces; four
// heads of 1000 x 3000: 32 us whole, 43-45 us in 2-16).
constexpr double kSplitFloorUs = 40.0;
constexpr double kLoneStepFactor = 0.6;

inline int causal_splits(long long bh, int n_qtiles, int BM, int BN, int D, int Dv, int Nq,
                         int Nkv, int coff, long long slots, int ktiles) {
  const long long tiles = bh * n_qtiles;
  if (tiles >= slots) return 1;
  const int s = (int)std::min<long long>((slots + tiles - 1) / tiles,
                                         std::min(kMaxSplits, ktiles / kMinStepsPerPiece));
  if (s < 2) return 1;
  long long sum = 0;
  int lmax = 0;
  for (int qt = 0; qt < n_qtiles; ++qt) {
    const long long end =
        std::min<long long>(std::min<long long>((long long)(qt + 1) * BM, Nq) + coff, Nkv);
    const int len = end > 0 ? (int)((end + BN - 1) / BN) : 0;
    sum += len;
    lmax = std::max(lmax, len);
  }
  const double work = (double)sum * bh;
  const double step_us = 2.0 * BM * BN * (double)(D + Dv) * slots / kChipFlopsPerUs;
  const double whole =
      std::max(lmax + kPieceFillSteps, (work + kPieceFillSteps * tiles) / slots) * step_us;
  const int steps = (ktiles + s - 1) / s;
  const double cut = std::max(std::min(lmax, steps) + kPieceFillSteps,
                              (work + kPieceFillSteps * tiles * s) / slots) * step_us +
                     kSplitFixedUs + s * (double)bh * Nq * (Dv + 1) * 8.0 / kMergeBytesPerUs;
  return cut < whole ? s : 1;
}

// num_splits > 0 cuts every tile into that many pieces (at most one per key
// tile).  Otherwise, without a mask, the grid runs in rounds of `slots`
// equal workgroups and only the tiles of the last, partial round are cut,
// so that they finish in a fraction of a round.
inline Plan make_plan(int B, int Hq, int Nq, int Nkv, int D, int Dv, int causal, int num_splits,
               int num_cus, bool masked = false) {
  Plan pl;
  pl.cfg = select_cfg(B, Hq, Nq, D, causal, masked, num_cus);
  pl.Dv = Dv;
  const TileCfg c = kCfgs[pl.cfg];
  pl.n_qtiles = (Nq + c.BM() - 1) / c.BM();
  pl.tiles = (long long)B * Hq * pl.n_qtiles;
  pl.rows = (long long)B * Hq * Nq;
  const long long slots = (long long)c.resident_per_cu() * (num_cus > 0 ? num_cus : 256);
  const int ktiles = (Nkv + c.BN - 1) / c.BN;
  long long first = 0;
  int S;
  if (num_splits > 0) {
    S = num_splits;
  } else if (causal) {
    S = causal_splits((long long)B * Hq, pl.n_qtiles, c.BM(), c.BN, D, Dv, Nq, Nkv,
                      causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq : 0, slots, ktiles);
  } else {
    const long long rem = pl.tiles % slots;
    first = pl.tiles - rem;
    S = rem ? balanced_splits(rem, slots, ktiles, std::min(1.0, (double)Nq / c.BM())) : 1;
    if (S > 1 && first == 0) {
      const double step_us = 2.0 * c.BM() * c.BN * (double)(D + Dv) * slots / kChipFlopsPerUs;
      if ((ktiles + kPieceFillSteps) * step_us * kLoneStepFactor < kSplitFloorUs) S = 1;
    }
  }
  if (S > ktiles) S = ktiles;
  const int tps = (ktiles + S - 1) / S;
  S = (ktiles + tps - 1) / tps;  // drop empty trailing pieces
  pl.splits = S;
  pl.split_len = tps * c.BN;
  pl.first_split = S > 1 ? first : pl.tiles;
  const long long bh = pl.first_split / pl.n_qtiles, qt = pl.first_split % pl.n_qtiles;
  pl.row0 = S > 1 ? bh * Nq + qt * c.BM() : pl.rows;
  return pl;
}

// GQA head packing (the English noflash-attention post's "flattened GQA
// GEMMs", section "The DIY approach").  The G = Hq / Hkv query heads of a KV
// head read the same keys, so when each head's query range is shorter than
// a tile, the G ranges are computed as one range of G * Nq rows of the KV
// head: K and V stream once per group instead of once per head, and the
// tiles fill.  Row r of that range is query head hk * G + r / Nq at
// position r % Nq (the kernel takes the position for the causal mask).
// That is a plain re-indexing when each head's rows follow the previous
// head's (head stride = Nq * row stride, or Nq = 1) in Q, the output and
// the mask; other layouts are not packed.
struct Packing {
  bool on = false;
  int Hq = 0, Nq = 0;  // the launch's heads and rows (packed or not)
  Layout L;
  MaskArgs M;
};

inline Packing packing(int Hq, int Hkv, int Nq, int D, int Dv, const Layout& L, const MaskArgs& M) {
  Packing pk;
  pk.Hq = Hq;
  pk.Nq = Nq;
  pk.L = L;
  pk.M = M;
  const int G = Hq / Hkv;
  if (G <= 1 || Nq >= kCfgs[narrow_cfg(D)].BM()) return pk;
  auto flat = [&](Strides s, Strides* out) {
    if (Nq == 1)
      s.n = s.h;
    else if (s.h != (int64_t)Nq * s.n)
      return false;
    s.h *= G;
    *out = s;
    return true;
  };
  Layout P = L;
  if (!flat(L.q, &P.q) || !flat(L.o, &P.o) || !strides_ok(P.q, D) || !strides_ok(P.o, Dv))
    return pk;
  MaskArgs PM = M;
  if (M.type != ATTN_MASK_NONE) {
    if (Nq == 1)
      PM.sq = M.sh;
    else if (M.sh != (int64_t)Nq * M.sq)
      return pk;
    PM.sh = M.sh * G;
  }
  pk.on = true;
  pk.Hq = Hkv;
  pk.Nq = G * Nq;
  pk.L = P;
  pk.M = PM;
  return pk;
}

// The plan of a call on contiguous tensors, packing included (the planning
// queries describe attn_fwd, whose tensors are contiguous).
inline Plan contiguous_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv, int causal,
                     int num_splits, int num_cus) {
  const Packing pk = packing(Hq, Hkv, Nq, D, Dv, contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv),
                             MaskArgs());
  return make_plan(B, pk.Hq, pk.Nq, Nkv, D, Dv, causal, num_splits, num_cus);
}

}  // namespace attn_planner

#endif  // ATTN_PLAN_H_
