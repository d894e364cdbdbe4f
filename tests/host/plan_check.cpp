// Host-only checks of the forward's planner and argument validation
// (csrc/attn_plan.h), built with AddressSanitizer and UBSan by
// tests/test_host_plan.py.  Seeded random shapes, strides and pointer values
// (plain integers: nothing is dereferenced) drive validate(), packing(),
// make_plan() and contiguous_plan(); each result is checked against
// invariants restated here independently:
//  * a plan covers every key of every query tile exactly once (whole tiles,
//    or pieces of split_len keys of which none is empty), its split rows are
//    the rows of the tiles from first_split on, and its workspace holds
//    splits x those rows x (Dv + 1) floats;
//  * a packed layout addresses, for every packed row, the element of the
//    query head and position it stands for;
//  * validate() accepts only shapes whose rows fit 32 bits, aligned
//    pointers and strides, and outputs that overlap no input.
// Prints "plan checks passed: N cases" and exits 0, or lists failures and
// exits 1.
#include <stdio.h>

#include <random>

#include "attn_plan.h"

using namespace attn_planner;

namespace {

long long g_fail = 0;

#define CHECK(cond, ...)                                            \
  do {                                                              \
    if (!(cond)) {                                                  \
      if (++g_fail <= 20) {                                         \
        fprintf(stderr, "FAIL line %d: %s | ", __LINE__, #cond);    \
        fprintf(stderr, __VA_ARGS__);                               \
        fprintf(stderr, "\n");                                      \
      }                                                             \
    }                                                               \
  } while (0)

const int kDims[][2] = {{64, 64}, {80, 80}, {96, 96}, {128, 128}, {256, 256}, {192, 128}};

bool cfg_allowed(int cfg, int D) {
  switch (D) {
    case 64: return cfg == kCfgD64Narrow || cfg == kCfgD64Wide;
    case 80:
    case 96: return cfg == kCfgD96;
    case 128: return cfg == kCfgD128Narrow || cfg == kCfgD128Wide || cfg == kCfgD128Decode;
    case 192: return cfg == kCfgD192;
    case 256: return cfg == kCfgD256;
  }
  return false;
}

void check_plan(const Plan& pl, int B, int Hq, int Nq, int Nkv, int D, int Dv, int causal,
                int num_splits, int cus) {
  CHECK(pl.cfg >= 0 && pl.cfg < (int)(sizeof(kCfgs) / sizeof(kCfgs[0])), "cfg %d", pl.cfg);
  if (g_fail) return;
  const TileCfg c = kCfgs[pl.cfg];
  CHECK(cfg_allowed(pl.cfg, D), "cfg %d for D %d", pl.cfg, D);
  const int ktiles = (Nkv + c.BN - 1) / c.BN;
  const long long tiles = (long long)B * Hq * ((Nq + c.BM() - 1) / c.BM());
  CHECK(pl.n_qtiles == (Nq + c.BM() - 1) / c.BM(), "n_qtiles %d", pl.n_qtiles);
  CHECK(pl.tiles == tiles, "tiles %lld vs %lld", pl.tiles, tiles);
  CHECK(pl.rows == (long long)B * Hq * Nq, "rows %lld", pl.rows);
  CHECK(pl.Dv == Dv, "Dv");
  CHECK(pl.splits >= 1 && pl.splits <= ktiles, "splits %d ktiles %d", pl.splits, ktiles);
  if (num_splits > 0) CHECK(pl.splits <= num_splits, "splits %d > asked %d", pl.splits, num_splits);
  else CHECK(pl.splits <= kMaxSplits, "splits %d", pl.splits);
  if (pl.splits > 1) {
    CHECK(pl.split_len > 0 && pl.split_len % c.BN == 0, "split_len %d", pl.split_len);
    CHECK((long long)pl.splits * pl.split_len >= Nkv, "pieces end before Nkv");
    CHECK((long long)(pl.splits - 1) * pl.split_len < Nkv, "empty last piece");
    CHECK(pl.first_split >= 0 && pl.first_split < pl.tiles, "first_split %lld", pl.first_split);
    const long long bh = pl.first_split / pl.n_qtiles, qt = pl.first_split % pl.n_qtiles;
    CHECK(pl.row0 == bh * Nq + (long long)qt * c.BM(), "row0 %lld", pl.row0);
    CHECK(pl.row0 < pl.rows, "row0 past rows");
    CHECK(pl.workspace_bytes() ==
              (size_t)pl.splits * (size_t)(pl.rows - pl.row0) * (size_t)(Dv + 1) * 4,
          "workspace bytes");
    if (num_splits == 0 && !causal) {
      // only the last, partial round of equal tiles is cut
      const long long slots = (long long)c.resident_per_cu() * (cus > 0 ? cus : 256);
      CHECK(pl.first_split % slots == 0 && pl.tiles - pl.first_split < slots,
            "split tiles %lld..%lld slots %lld", pl.first_split, pl.tiles, slots);
    }
  } else {
    CHECK(pl.first_split == pl.tiles && pl.row0 == pl.rows, "unsplit plan bounds");
    CHECK(pl.workspace_bytes() == 0, "unsplit workspace");
  }
}

// Element offset of (b, h, n) in a layout.
__int128 at(const Strides& s, long long b, long long h, long long n) {
  return (__int128)b * s.b + (__int128)h * s.h + (__int128)n * s.n;
}

void check_packing(int B, int Hq, int Hkv, int Nq, int D, int Dv, const Layout& L) {
  const Packing pk = packing(Hq, Hkv, Nq, D, Dv, L, MaskArgs());
  const int G = Hq / Hkv;
  if (!pk.on) {
    CHECK(pk.Hq == Hq && pk.Nq == Nq, "unpacked shape changed");
    return;
  }
  CHECK(G > 1 && pk.Hq == Hkv && pk.Nq == G * Nq, "packed shape");
  CHECK(strides_ok(pk.L.q, D) && strides_ok(pk.L.o, Dv), "packed strides");
  for (int b = 0; b < B; ++b)
    for (int hk = 0; hk < Hkv; ++hk)
      for (int r = 0; r < G * Nq; ++r) {
        const int h = hk * G + r / Nq, n = r % Nq;
        CHECK(at(pk.L.q, b, hk, r) == at(L.q, b, h, n), "q row %d of kv head %d", r, hk);
        CHECK(at(pk.L.o, b, hk, r) == at(L.o, b, h, n), "o row %d of kv head %d", r, hk);
        if (g_fail) return;
      }
}

}  // namespace

int main() {
  std::mt19937_64 rng(20261202);
  auto pick = [&](long long lo, long long hi) {
    return std::uniform_int_distribution<long long>(lo, hi)(rng);
  };
  long long cases = 0, split_plans = 0, packed = 0, accepted = 0;

  // Plans over shapes from one row to the largest grids.
  for (int it = 0; it < 20000; ++it) {
    const auto& dd = kDims[pick(0, 5)];
    const int D = dd[0], Dv = dd[1];
    const int Hkv = (int)pick(1, 16), G = (int)(pick(0, 3) == 0 ? 1 : pick(1, 16));
    const int Hq = Hkv * G;
    const int B = (int)pick(1, 8);
    const int Nq = (int)(pick(0, 4) == 0 ? pick(1, 8) : pick(1, 1 << pick(1, 17)));
    const int Nkv = (int)pick(1, 1 << pick(1, 20));
    if ((long long)B * Hq * Nq > INT32_MAX) continue;
    const int causal = (int)pick(0, 2);
    const int ns = pick(0, 2) ? 0 : (int)pick(1, 300);
    const int cus = (int)(pick(0, 3) == 0 ? pick(1, 320) : 256);
    const bool masked = pick(0, 5) == 0;
    const Plan pl = make_plan(B, Hq, Nq, Nkv, D, Dv, causal, ns, cus, masked);
    check_plan(pl, B, Hq, Nq, Nkv, D, Dv, causal, ns, cus);
    split_plans += pl.splits > 1;
    const Plan cp = contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, Dv, causal, ns, cus);
    const Packing pk = packing(Hq, Hkv, Nq, D, Dv, contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv),
                               MaskArgs());
    check_plan(cp, B, pk.Hq, pk.Nq, Nkv, D, Dv, causal, ns, cus);
    ++cases;
  }

  // Packing on contiguous and on [B, N, H, D] (transposed) layouts, small
  // enough to enumerate every row.
  for (int it = 0; it < 3000; ++it) {
    const auto& dd = kDims[pick(0, 5)];
    const int D = dd[0], Dv = dd[1];
    const int Hkv = (int)pick(1, 4), G = (int)pick(1, 8), Hq = Hkv * G;
    const int B = (int)pick(1, 3), Nq = (int)pick(1, 300), Nkv = (int)pick(1, 500);
    Layout L = contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv);
    if (pick(0, 1)) {  // [B, N, H, D] storage viewed as [B, H, N, D]
      L.q = Strides{(int64_t)Nq * Hq * D, D, (int64_t)Hq * D};
      L.o = Strides{(int64_t)Nq * Hq * Dv, Dv, (int64_t)Hq * Dv};
    }
    check_packing(B, Hq, Hkv, Nq, D, Dv, L);
    packed += packing(Hq, Hkv, Nq, D, Dv, L, MaskArgs()).on;
    ++cases;
  }

  // validate(): random (often invalid) arguments; what it accepts must hold
  // the stated conditions.
  for (int it = 0; it < 200000; ++it) {
    const auto& dd = kDims[pick(0, 5)];
    const int D = pick(0, 20) ? dd[0] : (int)pick(-4, 300);
    const int Dv = pick(0, 20) ? dd[1] : (int)pick(-4, 300);
    const int B = (int)pick(-1, 4), Hkv = (int)pick(-1, 8), Hq = Hkv * (int)pick(0, 4);
    const int Nq = (int)(pick(0, 10) ? pick(-1, 5000) : pick(1, INT32_MAX));
    const int Nkv = (int)(pick(0, 10) ? pick(-1, 5000) : pick(1, INT32_MAX));
    const int dtype = (int)pick(-1, 3), causal = (int)pick(-1, 3);
    const float scale = pick(0, 50) ? 0.125f : (pick(0, 1) ? NAN : INFINITY);
    auto ptr = [&]() -> uintptr_t {
      if (!pick(0, 40)) return 0;
      return (uintptr_t)pick(1, 1LL << 44) * (pick(0, 10) ? 256 : 1) + (pick(0, 20) ? 0 : pick(1, 15));
    };
    const uintptr_t q = ptr(), k = ptr(), v = ptr(), o = pick(0, 10) ? ptr() : q;
    const uintptr_t l = pick(0, 3) ? 0 : ptr();
    Layout L = contiguous_layout(std::max(Hq, 1), std::max(Hkv, 1), std::max(Nq, 1),
                                 std::max(Nkv, 1), std::max(D, 1), std::max(Dv, 1));
    if (!pick(0, 4)) {
      auto rnd = [&]() { return (int64_t)(pick(0, 3) ? pick(-8, 1 << 20) * 8 : pick(-100, 1LL << 40)); };
      L.q = Strides{rnd(), rnd(), rnd()};
      L.o = Strides{rnd(), rnd(), rnd()};
    }
    MaskArgs M;
    if (!pick(0, 5)) {
      M.type = (int)pick(0, 3);
      M.ptr = (const void*)ptr();
      M.sb = pick(-4, 1 << 20) * 4;
      M.sh = pick(-4, 1 << 20) * 4;
      M.sq = pick(-4, 1 << 16) * 4;
    }
    const int rc = validate((const void*)q, (const void*)k, (const void*)v, (const void*)o,
                            (const float*)l, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal, dtype,
                            L, M);
    if (rc == ATTN_OK) {
      ++accepted;
      CHECK(B > 0 && Hq > 0 && Hkv > 0 && Nq > 0 && Nkv > 0 && Hq % Hkv == 0, "shape");
      CHECK((long long)B * Hq * Nq <= INT32_MAX && (long long)B * Hkv * Nkv <= INT32_MAX,
            "rows fit 32 bits");
      CHECK(((q | k | v | o) & 15) == 0 && (l & 3) == 0, "alignment");
      CHECK(o != q && o != k && o != v, "output aliases an input");
      CHECK(std::isfinite(scale), "scale");
      CHECK(head_dims_ok(D, Dv), "head dims");
    }
    ++cases;
  }

  if (g_fail) {
    fprintf(stderr, "plan checks failed: %lld of %lld cases\n", g_fail, cases);
    return 1;
  }
  printf("plan checks passed: %lld cases (%lld split plans, %lld packed layouts, %lld "
         "accepted argument sets)\n", cases, split_plans, packed, accepted);
  return 0;
}
