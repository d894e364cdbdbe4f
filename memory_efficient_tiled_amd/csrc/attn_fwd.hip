// attn_fwd.hip -- host side of the attention forward: argument checks, the
// tile and split plan, workspace, launches, and the C entry points.  The
// kernels are in attn_fwd_kernel.h (one translation unit per head
// dimension: attn_fwd_d<D>.hip).

#include "attn_fwd_kernel.h"

#include <stdlib.h>

#include <algorithm>
#include <mutex>

namespace {

using namespace attn_fwd_detail;

// The tile every call of head dimension D may take (masked calls always do).
int narrow_cfg(int D) {
  if (D == 192) return kCfgD192;
  if (D == 256) return kCfgD256;
  if (D == 96 || D == 80) return kCfgD96;
  return D == 128 ? kCfgD128Narrow : kCfgD64Narrow;
}

// The wide tiles of each head dimension are used without a causal mask or an
// attention mask when they still fill every slot of the device at least
// once; at D = 128 a query range of at most 128 rows per head (decode, or a
// packed GQA group) takes the 128-row decode tile, unless masked.
int select_cfg(int B, int Hq, int Nq, int D, int causal, bool masked, int num_cus) {
  const int narrow = narrow_cfg(D);
  if (D != 128 && D != 64) return narrow;
  if (D == 128 && !masked && Nq <= kCfgs[kCfgD128Decode].BM()) return kCfgD128Decode;
  const int wide = D == 128 ? kCfgD128Wide : kCfgD64Wide;
  const TileCfg& w = kCfgs[wide];
  const long long wide_wgs = (long long)B * Hq * ((Nq + w.BM() - 1) / w.BM());
  const long long slots = (long long)w.resident_per_cu() * (num_cus > 0 ? num_cus : 256);
  return (!causal && !masked && wide_wgs >= slots) ? wide : narrow;
}

thread_local int g_last_hip_error = 0;

bool head_dim_ok(int D) { return D == 64 || D == 80 || D == 96 || D == 128 || D == 256; }

// Head dimensions of Q/K (D) and V/O (Dv): equal and supported, or the
// (192, 128) pair.
bool head_dims_ok(int D, int Dv) { return Dv == D ? head_dim_ok(D) : (D == 192 && Dv == 128); }

struct DeviceInfo {
  bool init = false;
  bool gfx950 = false;
  int cus = 0;
  void* scratch = nullptr;  // this device's address of `scratch` (attn_fwd_noalloc)
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

// Split-KV partials of attn_fwd_noalloc, for callers that cannot allocate
// device memory.  Every device the library runs on holds its own copy, from
// the library's load until the process ends.  In host code this name is not
// a device address: host code uses only the address hipGetSymbolAddress
// returns on each device (scratch_address below).
static __device__ __align__(256) unsigned char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

int device_info(DeviceInfo* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= 64) return ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.init) {
    hipDeviceProp_t prop;
    e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      g_last_hip_error = (int)e;
      return ATTN_EHIP;
    }
    d.gfx950 = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    d.cus = prop.multiProcessorCount;
    d.init = true;
  }
  *out = d;
  return d.gfx950 ? ATTN_OK : ATTN_EUNSUPPORTED;
}

// The current device's address of `scratch`, looked up once per device
// (with that device current) and kept.  ATTN_EHIP if the lookup fails.
int scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  if (dev < 0 || dev >= 64) return ATTN_EUNSUPPORTED;
  std::lock_guard<std::mutex> lk(g_dev_mu);
  DeviceInfo& d = g_dev[dev];
  if (!d.scratch) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_EHIP;
    }
    d.scratch = ptr;
  }
  *out = d.scratch;
  return ATTN_OK;
}

// Element strides of one tensor's batch, head and sequence dimensions; the
// head dimension (D) is contiguous.
struct Strides {
  int64_t b, h, n;
};
struct Layout {
  Strides q, k, v, o;
};

Layout contiguous_layout(int Hq, int Hkv, int Nq, int Nkv, int D, int Dv) {
  const Strides qs{(int64_t)Hq * Nq * D, (int64_t)Nq * D, D};
  const Strides ks{(int64_t)Hkv * Nkv * D, (int64_t)Nkv * D, D};
  const Strides vs{(int64_t)Hkv * Nkv * Dv, (int64_t)Nkv * Dv, Dv};
  const Strides os{(int64_t)Hq * Nq * Dv, (int64_t)Nq * Dv, Dv};
  return Layout{qs, ks, vs, os};
}

// Bytes from a tensor's base to the end of its last element.
__int128 extent_bytes(const Strides& s, int B, int H, int N, int D) {
  return 2 * ((__int128)(B - 1) * s.b + (__int128)(H - 1) * s.h + (__int128)(N - 1) * s.n + D);
}

bool overlaps128(const void* a, __int128 na, const void* b, __int128 nb) {
  const __int128 x = (__int128)(uintptr_t)a, y = (__int128)(uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Strides the kernels can take: non-negative multiples of 8 elements (so
// every row starts 16-byte aligned), row strides of at least one row (the
// K/V copies rely on rows past the last key starting beyond its end) and at
// most 2^24 elements (per-lane copy offsets are 32-bit).
bool strides_ok(const Strides& s, int D) {
  if (s.b < 0 || s.h < 0 || s.n < D || s.n > (1 << 24)) return false;
  return ((s.b | s.h | s.n) & 7) == 0;
}

// No two elements of the output share an address: ordered by stride, each
// dimension of extent > 1 must step over everything the smaller ones span.
bool dense_enough(const Strides& s, int B, int H, int N, int D) {
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

int validate(const void* q, const void* k, const void* v, const void* out, const float* lse,
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
// qt): tiles [0, first_split) run whole in a launch that writes the output
// directly; the key range of each tile in [first_split, tiles) is cut into
// `splits` pieces of `split_len` keys, computed by a second launch into fp32
// partials and merged by their log-sum-exp.  Those tiles are the last ones,
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

int balanced_splits(long long rem, long long slots, int ktiles, double row_frac) {
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

// Causal tiles differ in length and are launched longest first, so the
// hardware's dynamic dispatch balances them; only a grid smaller than the
// chip is split, into enough pieces to fill every slot.
int causal_splits(long long tiles, long long slots, int ktiles) {
  if (tiles >= slots) return 1;
  long long s = (slots + tiles - 1) / tiles;
  s = std::min<long long>(s, std::min(kMaxSplits, ktiles / kMinStepsPerPiece));
  return s < 1 ? 1 : (int)s;
}

// num_splits > 0 cuts every tile into that many pieces (at most one per key
// tile).  Otherwise, without a mask, the grid runs in rounds of `slots`
// equal workgroups and only the tiles of the last, partial round are cut,
// so that they finish in a fraction of a round.
Plan make_plan(int B, int Hq, int Nq, int Nkv, int D, int Dv, int causal, int num_splits,
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
    S = causal_splits(pl.tiles, slots, ktiles);
  } else {
    const long long rem = pl.tiles % slots;
    first = pl.tiles - rem;
    S = rem ? balanced_splits(rem, slots, ktiles, std::min(1.0, (double)Nq / c.BM())) : 1;
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

Packing packing(int Hq, int Hkv, int Nq, int D, int Dv, const Layout& L, const MaskArgs& M) {
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
Plan contiguous_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv, int causal,
                     int num_splits, int num_cus) {
  const Packing pk = packing(Hq, Hkv, Nq, D, Dv, contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv),
                             MaskArgs());
  return make_plan(B, pk.Hq, pk.Nq, Nkv, D, Dv, causal, num_splits, num_cus);
}

hipError_t launch_fwd(int D, int Dv, const Params& p, int cfg, bool causal, bool split,
                      bool strided, bool masked, bool bf16, hipStream_t st) {
  if (Dv != D)  // the (192, 128) pair
    return launch_fwd_d<192, 128>(p, cfg, causal, split, strided, masked, bf16, st);
  switch (D) {
    case 64: return launch_fwd_d<64, 64>(p, cfg, causal, split, strided, masked, bf16, st);
    case 80: return launch_fwd_d<80, 80>(p, cfg, causal, split, strided, masked, bf16, st);
    case 96: return launch_fwd_d<96, 96>(p, cfg, causal, split, strided, masked, bf16, st);
    case 256: return launch_fwd_d<256, 256>(p, cfg, causal, split, strided, masked, bf16, st);
    default: return launch_fwd_d<128, 128>(p, cfg, causal, split, strided, masked, bf16, st);
  }
}

// The merge of split partials, for output rows of Dv elements.
hipError_t launch_combine(int Dv, const Params& p, bool strided, bool bf16, hipStream_t st) {
  switch (Dv) {
    case 64: return launch_combine_d<64>(p, strided, bf16, st);
    case 80: return launch_combine_d<80>(p, strided, bf16, st);
    case 96: return launch_combine_d<96>(p, strided, bf16, st);
    case 256: return launch_combine_d<256>(p, strided, bf16, st);
    default: return launch_combine_d<128>(p, strided, bf16, st);
  }
}

// `noalloc`: take the split workspace from this device's `scratch` array
// (ATTN_ESCRATCH, before any launch, when the plan needs more) instead of
// hipMallocAsync.
int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
        int Nq, int Nkv, int D, int Dv, const Layout& L, float scale, int causal, int dtype,
        int num_splits, hipStream_t stream, const MaskArgs& M = MaskArgs(),
        bool noalloc = false) {
  int rc = validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal, dtype, L, M);
  const bool masked = M.type != ATTN_MASK_NONE;
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_EINVAL;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != ATTN_OK) return rc;

  // From here on the launch's heads, rows and strides are the packed ones
  // when the G query heads of a KV head are packed.
  const Packing pk = packing(Hq, Hkv, Nq, D, Dv, L, M);
  const int Nq0 = Nq;
  Hq = pk.Hq;
  Nq = pk.Nq;
  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, Dv, causal, num_splits, di.cus, masked);
  const long long split_wgs = (pl.tiles - pl.first_split) * pl.splits;
  if (pl.first_split > INT32_MAX || split_wgs > INT32_MAX) return ATTN_EINVAL;

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  const Layout& PL = pk.L;
  p.qsb = PL.q.b, p.qsh = PL.q.h, p.qsn = (int)PL.q.n;
  p.ksb = PL.k.b, p.ksh = PL.k.h, p.ksn = (int)PL.k.n;
  p.vsb = PL.v.b, p.vsh = PL.v.h, p.vsn = (int)PL.v.n;
  p.osb = PL.o.b, p.osh = PL.o.h, p.osn = (int)PL.o.n;
  p.lse = lse;
  p.opart = nullptr;
  p.lsepart = nullptr;
  p.Hq = Hq;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = Hq / Hkv;  // 1 when packed
  p.Hkv = Hkv;
  p.n_qtiles = pl.n_qtiles;
  p.n_splits = pl.splits;
  p.split_len = pl.split_len;
  p.row0 = (int)pl.row0;
  p.prows = (int)(pl.rows - pl.row0);
  // A masked score is -inf and must give a probability of exactly 0, so the
  // factor applied to scores stays positive: for scale 0 every finite score
  // times FLT_MIN rounds to a base-2 exponent of 0, as it should.
  p.c = fmaxf(fabsf(scale) * kLog2e, FLT_MIN);
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  p.coff = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq0 : 0;
  p.pos_nq = pk.on ? Nq0 : 0;
  p.mask = (const uint8_t*)pk.M.ptr;
  p.msb = pk.M.sb, p.msh = pk.M.sh, p.msq = pk.M.sq;
  p.mask_mode = pk.M.type;
  p.cm = p.c;
  if (M.type == ATTN_MASK_ADD) p.c = 1.f;  // the mask step forms base-2 scores

  void* ws = nullptr;
  if (noalloc) {
    void* sp = nullptr;
    rc = scratch_address(&sp);
    if (rc != ATTN_OK) return rc;
    if (split_wgs > 0) {
      if (pl.workspace_bytes() > (size_t)ATTN_NOALLOC_SCRATCH_BYTES) return ATTN_ESCRATCH;
      p.opart = (float*)sp;
      p.lsepart = p.opart + (size_t)pl.splits * p.prows * Dv;
    }
  } else if (split_wgs > 0) {
    hipError_t e = attn_host::workspace_alloc(&ws, pl.workspace_bytes(), stream);
    if (e != hipSuccess || !ws) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_ENOMEM;
    }
    p.opart = (float*)ws;
    p.lsepart = p.opart + (size_t)pl.splits * p.prows * Dv;
  }

  const bool cz = causal != 0;
  const Layout C = contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv);
  auto same = [](const Strides& a, const Strides& b) { return a.b == b.b && a.h == b.h && a.n == b.n; };
  const bool strided =
      !(same(PL.q, C.q) && same(PL.k, C.k) && same(PL.v, C.v) && same(PL.o, C.o));
  const bool bf16 = dtype == ATTN_BF16;
  auto launch = [&](bool split) {
    return launch_fwd(D, Dv, p, pl.cfg, cz, split, strided, masked, bf16, stream);
  };

  hipError_t e = hipSuccess;
  if (pl.first_split > 0) {  // whole tiles
    p.total = (int)pl.first_split;
    p.tile0 = 0;
    e = launch(false);
  }
  if (e == hipSuccess && split_wgs > 0) {  // pieces of the remaining tiles, then the merge
    p.total = (int)split_wgs;
    p.tile0 = (int)pl.first_split;
    e = launch(true);
    if (e == hipSuccess) {
      e = launch_combine(Dv, p, strided, bf16, stream);
    }
  }
  if (ws) {
    hipError_t ef = hipFreeAsync(ws, stream);
    if (e == hipSuccess) e = ef;
  }
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  return ATTN_OK;
}

}  // namespace

namespace attn_host {
int check_device(int* cus) {
  DeviceInfo di;
  const int rc = device_info(&di);
  if (cus) *cus = di.cus;
  return rc;
}
void set_last_hip_error(int e) { g_last_hip_error = e; }
hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t st) {
  const char* f = getenv("ATTN_FAIL_WORKSPACE");
  if (f && f[0] == '1' && f[1] == '\0') {
    *p = nullptr;
    return hipErrorOutOfMemory;
  }
  return hipMallocAsync(p, bytes, st);
}
void narrow_plan(int B, int Hq, int Nq, int Nkv, int D, int causal, int num_splits, int cus,
                 NarrowPlan* out) {
  // the masked plan always takes the narrow tile of its head dimension
  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, D, causal, num_splits, cus, true);
  out->n_qtiles = pl.n_qtiles;
  out->splits = pl.splits;
  out->split_len = pl.split_len;
  out->tiles = pl.tiles;
  out->first_split = pl.first_split;
  out->row0 = pl.row0;
  out->rows = pl.rows;
}
}  // namespace attn_host

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, 0,
             (hipStream_t)stream);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                   int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                     int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D,
             contiguous_layout(Hq, Hkv, Nq, Nkv, D, D), scale, causal, dtype, num_splits,
             (hipStream_t)stream, MaskArgs(), true);
}

}  // extern "C"

namespace {
// Strides from the C arrays (batch, head, sequence); NULL = contiguous.
Layout strided_layout(int Hq, int Hkv, int Nq, int Nkv, int D, int Dv, const long long* qs,
                      const long long* ks, const long long* vs, const long long* os) {
  Layout L = contiguous_layout(Hq, Hkv, Nq, Nkv, D, Dv);
  auto take = [](Strides& s, const long long* a) {
    if (a) s = Strides{a[0], a[1], a[2]};
  };
  take(L.q, qs);
  take(L.k, ks);
  take(L.v, vs);
  take(L.o, os);
  return L;
}
}  // namespace

extern "C" {

int attn_fwd_strided(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                     int Hq, int Hkv, int Nq, int Nkv, int D, const long long* q_stride,
                     const long long* k_stride, const long long* v_stride,
                     const long long* o_stride, float scale, int causal, int dtype,
                     int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                   int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  contiguous_layout(Hq, Hkv, Nq, Nkv, D, D));
}

int attn_fwd_strided_check(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                           const long long* q_stride, const long long* k_stride,
                           const long long* v_stride, const long long* o_stride, float scale,
                           int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride));
}

static MaskArgs mask_args(const void* mask, int mask_type, const long long* mask_stride) {
  MaskArgs m;
  m.ptr = mask;
  m.type = mask_type;
  if (mask_type != ATTN_MASK_NONE) {
    if (!mask_stride) {
      m.type = -1;  // rejected by validation
    } else {
      m.sb = mask_stride[0];
      m.sh = mask_stride[1];
      m.sq = mask_stride[2];
    }
  }
  return m;
}

int attn_fwd_masked(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                    int Hq, int Hkv, int Nq, int Nkv, int D, const long long* q_stride,
                    const long long* k_stride, const long long* v_stride,
                    const long long* o_stride, const void* mask, int mask_type,
                    const long long* mask_stride, float scale, int causal, int dtype,
                    int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream, mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_masked_check(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                          const long long* q_stride, const long long* k_stride,
                          const long long* v_stride, const long long* o_stride,
                          const void* mask, int mask_type, const long long* mask_stride,
                          float scale, int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, D, q_stride, k_stride, v_stride, o_stride),
                  mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_dv(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
                int Hkv, int Nq, int Nkv, int D, int Dv, const long long* q_stride,
                const long long* k_stride, const long long* v_stride, const long long* o_stride,
                const void* mask, int mask_type, const long long* mask_stride, float scale,
                int causal, int dtype, int num_splits, void* stream) {
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, Dv, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream, mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_dv_check(const void* q, const void* k, const void* v, const void* out,
                      const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv,
                      const long long* q_stride, const long long* k_stride,
                      const long long* v_stride, const long long* o_stride, const void* mask,
                      int mask_type, const long long* mask_stride, float scale, int causal,
                      int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, Dv, q_stride, k_stride, v_stride, o_stride),
                  mask_args(mask, mask_type, mask_stride));
}

// The planning queries take one head dimension: D = 192 stands for the
// (192, 128) pair, whose partial rows have 128 columns.
static int plan_dv(int D) { return D == 192 ? 128 : D; }

// Compute units of an MI355X, for the host-only workspace query.
constexpr int kMi355xCus = 256;

int attn_fwd_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                        int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dims_ok(D, plan_dv(D)) || (dtype != ATTN_F16 && dtype != ATTN_BF16))
    return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  return contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, 0, num_cus).splits;
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                  int num_splits, int num_cus, attn_plan* plan) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dims_ok(D, plan_dv(D)) || (dtype != ATTN_F16 && dtype != ATTN_BF16))
    return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT || num_splits < 0 || !plan)
    return ATTN_EINVAL;
  if ((long long)B * Hq * Nq > INT32_MAX || (long long)B * Hkv * Nkv > INT32_MAX)
    return ATTN_EINVAL;
  const Plan pl = contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, num_splits, num_cus);
  plan->tile_rows = kCfgs[pl.cfg].BM();
  plan->num_splits = pl.splits;
  plan->split_rows = pl.rows - pl.row0;
  plan->workspace_bytes = pl.workspace_bytes();
  return ATTN_OK;
}

// The plan depends on the number of KV heads only through GQA head
// packing; without it the query returns the largest workspace over every
// Hkv that divides Hq.
size_t attn_fwd_workspace_bytes(int B, int Hq, int Nq, int Nkv, int D, int causal) {
  if (B <= 0 || Hq <= 0 || Nq <= 0 || Nkv <= 0 || !head_dims_ok(D, plan_dv(D))) return 0;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return 0;
  if ((long long)B * Hq * Nq > INT32_MAX) return 0;
  size_t most = 0;
  for (int Hkv = 1; Hkv <= Hq; ++Hkv)
    if (Hq % Hkv == 0)
      most = std::max(most, contiguous_plan(B, Hq, Hkv, Nq, Nkv, D, plan_dv(D), causal, 0,
                                            kMi355xCus).workspace_bytes());
  return most;
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case ATTN_ENOMEM: return "device workspace allocation failed";
    case ATTN_EHIP: return "HIP launch or runtime error";
    case ATTN_ESCRATCH:
      return "the split workspace exceeds the no-allocation scratch (ATTN_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown error code";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
