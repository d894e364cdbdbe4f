// attn_bwd.hip -- gradients of the attention forward (dQ, dK, dV) for gfx950.
//
// The English noflash-attention post keeps autograd through its tiled
// forward (first tier, section "The DIY approach").  With the forward's row
// log-sum-exp saved, the probabilities are recomputed tile by tile and the
// gradients never need the Nq x Nkv matrices either:
//
//   P_ij  = exp(s_ij - lse_i),  s_ij = scale <q_i, k_j>   (0 where masked)
//   dV_j  = sum_i P_ij dO_i            dP_ij = <dO_i, V_j>
//   Delta_i = sum_d dO_id O_id  (= sum_j P_ij dP_ij)
//   dS_ij = P_ij (dP_ij - Delta_i)
//   dQ_i  = scale sum_j dS_ij K_j      dK_j = scale sum_i dS_ij Q_i
//
// K/V gradients of a KV head sum over the Hq / Hkv query heads that read it.
// Kernels, no atomics (results are bitwise reproducible):
//  * attn_delta_kernel: Delta and lse log2(e), one fp32 each per query row;
//  * attn_dkdv_pair_kernel: one workgroup per block of 128 keys of one KV
//    head, looping over every query tile of the query heads it covers, with
//    dK and dV accumulated in registers (dV in one wave of a pair, dK in the
//    other); at D = 64, 80 and 96 attn_dkdv_solo_kernel instead, where
//    each wave does all four products for its keys.  When the KV heads alone
//    give too few workgroups, the query heads of a group are split over
//    several workgroups that write fp32 partial sums, and attn_dkdv_reduce
//    adds them;
//  * attn_dq_kernel: one workgroup per 128 query rows, looping over key tiles
//    like the forward, with dQ accumulated in registers.
// The matrix products use the forward's operand layouts (see attn_fwd.hip):
// a 32x32 accumulator tile is packed in place as the B operand of the next
// product, and the other operand is read from LDS either row-wise (16-byte
// reads, k_swz layout) or transposed (ds_read_b64_tr_b16, v_swz layout).
//
// Padding rows need no masks: rows past Nq (queries) or Nkv (keys) are read
// as zeros, so a padded query row has dO = 0 and Delta = 0 and adds nothing
// to dK and dV, and a padded key has K = V = 0 and adds nothing to dQ; the
// gradients of padded rows themselves are never stored.  Only the causal
// mask is applied, and only on the tiles that straddle the diagonal.

#include "attn_common.h"
#include "attn_plan.h"

#include <mutex>
#include <type_traits>

namespace {

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;     // natural log, [B, Hq, Nq]
  float* delta;         // [B, Hq, Nq]
  float* lse2;          // lse * log2(e), [B, Hq, Nq]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* dkp;           // fp32 partial dK / dV, [hsplit, B, Hkv, Nkv, D], when hsplit > 1
  float* dvp;
  int B, Hq, Hkv, Nq, Nkv, G;
  int hsplit;           // workgroups sharing the query heads of one KV head
  int coff;             // causal: row i sees keys j <= i + coff
  int n_tiles;          // per head: query tiles (dQ) or key blocks (dK/dV)
  int total;            // workgroups of the launch
  float cs;             // scale * log2(e) (signed)
  float scale;
  // Attention mask of the forward (MASKED kernels): element (b, h, i, j) at
  // mask + b*msb + h*msh + i*msq + j, ATTN_MASK_BOOL or ATTN_MASK_ADD.
  const uint8_t* mask;
  int64_t msb, msh, msq;
  int mask_mode;
  // dQ launch without a causal mask, when its grid ends in a partial round:
  // workgroups [0, dq_whole) take whole query tiles 0 .. dq_whole - 1, and
  // each later tile is cut into dq_splits key ranges of dq_split_len keys,
  // whose workgroups write unscaled fp32 partial dQ rows (dqp:
  // [dq_splits][dq_rows][D], row (tile - dq_whole) * rows per tile + row in
  // tile),
  // added by attn_dq_reduce.  dq_splits = 1: every tile whole.
  int dq_whole, dq_splits, dq_split_len, dq_rows;
  float* dqp;
};

// Lanes per row of the delta kernel: D / 8 rounded up to a power of two.
constexpr int bwd_delta_lanes(int D) { return D / 8 <= 8 ? 8 : D / 8 <= 16 ? 16 : 32; }

// Delta_r = sum_d dO[r, d] O[r, d] in fp32: L lanes per row (D / 8 rounded
// up to a power of two; lanes past the row add nothing), one 16-byte load of
// each tensor per lane, a butterfly over the row's lanes.
template <int D, class Tag>
__global__ __launch_bounds__(256) void attn_delta_kernel(BwdParams p, int rows) {
  constexpr int L = bwd_delta_lanes(D);  // lanes per row
  static_assert(D / 8 <= L, "row fits its lanes");
  const int gid = blockIdx.x * 256 + threadIdx.x;
  const int row = gid / L, part = gid % L;
  float acc = 0.f;
  if (row < rows && part * 8 < D) {
    const u32x4 a = *(const u32x4*)(p.o + (size_t)row * D + part * 8);
    const u32x4 g = *(const u32x4*)(p.dout + (size_t)row * D + part * 8);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc += lo_f32<Tag>(a[i]) * lo_f32<Tag>(g[i]) + hi_f32<Tag>(a[i]) * hi_f32<Tag>(g[i]);
  }
#pragma unroll
  for (int w = 1; w < L; w <<= 1) acc += __shfl_xor(acc, w, L);
  if (row < rows && part == 0) {
    p.delta[row] = acc;
    // a row that saw no key (LSE -inf) gets +inf, so exp2(s - lse2) = 0
    const float l = p.lse[row];
    p.lse2[row] = l == -INFINITY ? INFINITY : l * kLog2e;
  }
}

// Copies of a ROWS-row tile into LDS: NI = ROWS * DP / 512 wave
// instructions of 1 KB (DP: the compute dimension), instruction n by wave
// n % NW (a wave-uniform count per wave).  Per-lane byte offsets in memory
// (rows of D elements) for either swizzle; chunks past the row in memory
// (D = 80) get an offset past the buffer and read zeros.
template <int D, int ROWS, int NW>
struct TileCopy {
  static constexpr int DP = compute_dim(D);
  static constexpr int CPR = DP / 8;
  static constexpr int NI = ROWS * CPR / 64;
  static constexpr int PER_WAVE = (NI + NW - 1) / NW;
  static_assert(NI * 64 == ROWS * CPR, "tile copy shape");
};

// How a staged tile is read: along rows (16-byte reads, k_swz), transposed
// (ds_read_b64_tr_b16, v_swz), or both from one copy (u_swz).
enum { kReadRows = 0, kReadCols = 1, kReadBoth = 2 };

// One LDS layout that serves both reads without bank conflicts, for rows
// of 128 bytes (D = 64), 192 bytes (compute dimension 96) and 256 bytes
// (D = 128): the 16-byte chunk index is XORed with a permutation of row
// bits.  Row reads (16 lanes, 16 consecutive rows, one chunk) need
// distinct bank groups over any 16 consecutive rows; transposing reads (32
// lanes, 4 consecutive rows x 64 bytes) need those 4 rows in disjoint
// 64-byte quarters of the banks.  At D = 128 rows r & 3 pick the quarter
// (XOR bits 3:2) and (r >> 2) & 3 the chunk within it (bits 1:0); at
// D = 64, where rows r and r + 1 share the banks, (r >> 1) & 1 picks the
// quarter within the half-row and (r >> 2) & 3 the chunk.  192-byte rows
// start in a different quarter for each r % 4, so the row swizzle
// (r >> 2) & 3, which permutes chunks within a quarter, serves both.
template <int D>
constexpr bool has_both_swz() { return D == 64 || D == 96 || D == 128; }
template <int D>
__device__ __forceinline__ int u_swz(int r) {
  static_assert(has_both_swz<D>(), "one-copy layout only at D = 64, 96 and 128");
  return D == 128  ? (((r & 3) << 2) | ((r >> 2) & 3))
         : D == 96 ? ((r >> 2) & 3)
                   : ((((r >> 1) & 1) << 2) | ((r >> 2) & 3));
}
template <int D, int RD>
__device__ __forceinline__ int tile_swz(int r) {
  if constexpr (RD == kReadRows) return k_swz<D>(r);
  else if constexpr (RD == kReadCols) return v_swz<D>(r);
  else return u_swz<D>(r);
}

template <int D, int ROWS, int NW, int RD>
__device__ __forceinline__ void copy_offsets(int wave, int lane, uint32_t* off) {
  using C = TileCopy<D, ROWS, NW>;
#pragma unroll
  for (int j = 0; j < C::PER_WAVE; ++j) {
    const int slot = (wave + NW * j) * 64 + lane;
    const int row = slot / C::CPR, pc = slot % C::CPR;
    const int ch = pc ^ tile_swz<C::DP, RD>(row);
    off[j] = ch < D / 8 ? row * D * 2 + (ch << 4) : kPadOffset;
  }
}

// Copies the ROWS-row tile starting at row r0 of a [rows_total x D] matrix
// at `base` into LDS (rows past rows_total read as zero; r0 < rows_total).
template <int D, int ROWS, int NW>
__device__ __forceinline__ void copy_tile(const uint16_t* base, int r0, int rows_total,
                                          uint16_t* dst, int wave, const uint32_t* off) {
  using C = TileCopy<D, ROWS, NW>;
  const int n = min(ROWS, rows_total - r0);
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(base + (size_t)r0 * D), 0, (uint32_t)(n * D * 2), kRawBufferFlags);
#pragma unroll
  for (int j = 0; j < C::PER_WAVE; ++j)
    if (wave + NW * j < C::NI) buf2lds16(r, dst + (wave + NW * j) * 512, off[j]);
}

// s_waitcnt immediate that waits for lgkmcnt 0 only (vmcnt 63 and expcnt 7
// are the no-wait values: vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8).
constexpr int kWaitLgkm0 = 0xC07F;

// Buffer B (0 or 1) of a double-buffered LDS tile of N elements.  With SEP
// each buffer is an LDS variable of its own (b0, b1): the compiler then
// sees that a copy still in flight into one buffer cannot alias reads of
// the other, and does not wait for the next tile's copies before the
// current tile's reads.  Without SEP both buffers are halves of b0 and it
// must wait; head dimensions 256 and the (192, 128) pair keep that form,
// whose kernels spill more registers when the compiler may move LDS reads
// above the copies.
template <int B, bool SEP, int N, class T>
__device__ __forceinline__ T* buf_at(T* b0, T* b1) {
  if constexpr (!SEP) return b0 + B * N;
  else if constexpr (B == 0) return b0;
  else return b1;
}
constexpr bool bwd_sep_buffers(int D, int DV) { return D != 256 && D == DV; }

// Query rows per wave (32 x) and per workgroup of the dQ kernel: 64 per wave
// at D = 64 without a causal mask, where Q, dO and dQ of 64 rows fit the
// registers and each K and V operand read from LDS serves two row blocks
// (with a causal mask 64-row waves ran slower); 32 elsewhere.
constexpr int dq_row_blocks(int D, bool causal) { return D == 64 && !causal ? 2 : 1; }
constexpr int dq_block_rows(int D, bool causal) { return 4 * 32 * dq_row_blocks(D, causal); }

// The Q (g = 0) or dO (g = 1) tile of buffer B when both are staged per
// buffer: with SEP buffer B's variable holds [Q | dO], else one variable
// holds [Q0 | Q1 | dO0 | dO1] (TQ, TG: elements of a Q and a dO tile).
template <int B, bool SEP, int TQ, int TG, class T>
__device__ __forceinline__ T* qg_tile(T* b0, T* b1, int g) {
  if constexpr (SEP) return (B == 0 ? b0 : b1) + g * TQ;
  else return b0 + (g ? 2 * TQ + B * TG : B * TQ);
}

// A operand read along rows (16 bytes: chunk 2 kc + hl of row `row`) of a
// tile staged for reads RD (kReadRows or kReadBoth).
template <int D, int RD = kReadRows>
__device__ __forceinline__ u32x4 read_rows(const uint16_t* t, int row, int kc, int hl) {
  return *(const u32x4*)(t + row * D + (((2 * kc + hl) ^ tile_swz<D, RD>(row)) << 3));
}

// A operand read transposed: 8 consecutive rows (in the accumulator's
// interleaving) of columns db*32 + v_d .. + 3, rows from `row` (swizzle
// sw_lo) and row + 8 (sw_hi; the two differ only for kReadBoth tiles).
template <int D>
__device__ __forceinline__ u32x4 read_cols(const uint16_t* t, int row, int db, int v_d,
                                           int sw_lo, int sw_hi) {
  const int d = db * 32 + v_d;
  const u32x2 lo = lds_read_tr16(t + row * D + (((d >> 3) ^ sw_lo) << 3) + (d & 7));
  const u32x2 hi = lds_read_tr16(t + (row + 8) * D + (((d >> 3) ^ sw_hi) << 3) + (d & 7));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Pack accumulator tile `s` (16 values per lane) as two B operands of
// 16 reduction rows each.
template <class Tag>
__device__ __forceinline__ void pack_tile(const f32x16& s, u32x4* out) {
  using N = Num<Tag>;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    u32x4 y;
#pragma unroll
    for (int w = 0; w < 4; ++w) y[w] = N::pack2(s[8 * hf + 2 * w], s[8 * hf + 2 * w + 1]);
    out[hf] = y;
  }
}

// Store accumulator tiles acc[db] (rows = d, column = this lane's row r) as
// row r of a 16-bit [*, D] matrix, times `mul` (columns past D not stored).
template <int D, class Tag>
__device__ __forceinline__ void store_row(uint16_t* dst, const f32x16* acc, float mul, int hl) {
  using N = Num<Tag>;
#pragma unroll
  for (int db = 0; db < compute_dim(D) / 32; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = db * 32 + 8 * i + 4 * hl;
      const f32x16& o = acc[db];
      u32x2 y = {N::pack2(o[4 * i] * mul, o[4 * i + 1] * mul),
                 N::pack2(o[4 * i + 2] * mul, o[4 * i + 3] * mul)};
      if (col < D) *(u32x2*)(dst + col) = y;
    }
}

// Stores a wave's dK^T or dV^T accumulators (column = this lane's key):
// 16-bit rows times `mul`, or the fp32 partial of head split `hs`.
template <int D, class Tag>
__device__ __forceinline__ void store_kv_grad(const BwdParams& p, uint16_t* dst, float* part,
                                              const f32x16* acc, float mul, size_t krow, int hs,
                                              int hl) {
  constexpr int NDB = compute_dim(D) / 32;
  if (p.hsplit == 1) {
    store_row<D, Tag>(dst + krow * D, acc, mul, hl);
    return;
  }
  float* r = part + ((size_t)hs * p.B * p.Hkv * p.Nkv + krow) * D;
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int col = db * 32 + 8 * i + 4 * hl;
      if (col < D)
        *(f32x4*)(r + col) =
            f32x4{acc[db][4 * i], acc[db][4 * i + 1], acc[db][4 * i + 2], acc[db][4 * i + 3]};
    }
}

// dK, dV with paired waves: 8 waves over 128 keys; waves w and w + 4 (which
// share a SIMD) own keys k0 + 32 (w % 4).  K and V of those keys stay in
// registers, K in wave w, V in wave w + 4.  Per query tile of 64 rows:
//   1. wave w:     S = Q K^T, P = exp2(cs S - lse2) (0 above the causal
//                  diagonal), written to LDS packed as a B operand;
//      wave w + 4: dP = dO V^T.
//   2. wave w:     dV^T += dO^T P;
//      wave w + 4: reads P, dS = P (dP - Delta), dK^T += Q^T dS.
// Each wave needs half the registers of one that does all four products,
// so two waves fit on a SIMD and one wave's softmax work overlaps the
// other's matrix products.  Q and dO tiles are in LDS two buffers deep,
// with lse2 and Delta: once each in the layout of both reads at D = 64 and
// 128, else twice each (row-read and transposed layouts).
//
// With V rows of DV != D elements (the (192, 128) pair) the two waves of a
// pair differ: the P wave holds K (D) and accumulates dV^T (DV rows), the
// dS wave holds V (DV) and accumulates dK^T (D rows); Q tiles are D wide
// and dO tiles DV wide.
template <int D, int DV, class Tag, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(512, 2) void attn_dkdv_pair_kernel(BwdParams p) {
  // 64-row query tiles; 32 at D = 256, whose K (or V) operands and dK (or
  // dV) accumulators alone take 192 registers, and for the (192, 128) pair
  // (the same registers; 64-row Q and dO tiles would not fit LDS)
  constexpr bool SQ = D == DV;
  constexpr int NQB = D == 256 || !SQ ? 1 : 2;
  constexpr int NW = 8, BK = 128, BQ = NQB * 32;
  constexpr int DP = compute_dim(D), DVP = compute_dim(DV);
  constexpr int DC = DP / 16, NDB = DP / 32, NKC = BQ / 16;
  constexpr int DCV = DVP / 16, NDBV = DVP / 32;
  constexpr int DCM = DC > DCV ? DC : DCV, NDBM = NDB > NDBV ? NDB : NDBV;
  constexpr int TILE = BQ * DP, TILEV = BQ * DVP;
  constexpr int IPW = TileCopy<D, BQ, NW>::PER_WAVE;
  constexpr int IPWV = TileCopy<DV, BQ, NW>::PER_WAVE;
  using N = Num<Tag>;

  // per buffer: Q then dO tiles read along rows (rows) and transposed
  // (cols); a wave picks its tile by an offset within the buffer.  With
  // UNI one copy in the layout of both reads (rows) serves both.
  constexpr bool SEP = bwd_sep_buffers(D, DV);
  constexpr bool UNI = SEP && (D == 64 || D == 128);  // (at 96: 5% slower here)
  constexpr int RDR = UNI ? kReadBoth : kReadRows;
  constexpr int TQG = TILE + TILEV;
  __shared__ __attribute__((aligned(1024))) uint16_t rows0[SEP ? TQG : 2 * TQG], rows1[SEP ? TQG : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t cols0[UNI ? 1 : SEP ? TQG : 2 * TQG],
      cols1[SEP && !UNI ? TQG : 1];
  __shared__ __attribute__((aligned(1024))) u32x4 xp[4][NKC][64];
  // lse2 and Delta of a tile: one dword per lane of a 64-lane copy (lanes
  // past the tile's rows write zeros), so 64 entries even when BQ = 32
  // (lse2 at 0, Delta at 64 of each buffer)
  __shared__ __attribute__((aligned(256))) float ld0[SEP ? 128 : 256], ld1[SEP ? 128 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;
  const int kw = wave & 3;
  const bool pw = wave < 4;  // computes P (else dS)

  // (causal: key tile 0 sees the most query tiles)
  int bid = CAUSAL ? longest_first(blockIdx.x, p.n_tiles, p.total) : xcd_remap(blockIdx.x, p.total);
  const int kt = bid % p.n_tiles;
  bid /= p.n_tiles;
  const int hs = bid % p.hsplit;
  bid /= p.hsplit;
  const int hk = bid % p.Hkv;
  const int b = bid / p.Hkv;
  const int k0 = kt * BK;
  const int kw0 = k0 + kw * 32;
  const int key = kw0 + l32;
  const int hpw = p.G / p.hsplit;
  const int h0 = hk * p.G + hs * hpw;

  const size_t krow0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* kv = pw ? p.k : p.v;
  const int kvw = pw ? D : DV;  // row length of K (P waves) or V (dS waves)
  u32x4 bf[DCM];
#pragma unroll
  for (int kc = 0; kc < DCM; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u};
    if (key < p.Nkv && kc * 16 + hl * 8 < kvw)
      x = *(const u32x4*)(kv + (krow0 + key) * kvw + kc * 16 + hl * 8);
    bf[kc] = x;
  }
  f32x16 acc[NDBM];
#pragma unroll
  for (int i = 0; i < NDBM; ++i) acc[i] = f32x16{};

  // copy offsets of the Q tiles and (DV != D) of the dO tiles
  uint32_t roff[IPW], toff[UNI ? 1 : IPW], groff[SQ ? 1 : IPWV], gtoff[SQ ? 1 : IPWV];
  copy_offsets<D, BQ, NW, RDR>(wave, lane, roff);
  if constexpr (!UNI) copy_offsets<D, BQ, NW, kReadCols>(wave, lane, toff);
  if constexpr (!SQ) {
    copy_offsets<DV, BQ, NW, kReadRows>(wave, lane, groff);
    copy_offsets<DV, BQ, NW, kReadCols>(wave, lane, gtoff);
  }

  const int nqt = (p.Nq + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? min(nqt, max(0, k0 - p.coff) / BQ) : 0;
  const int per_head = nqt - qt0;
  const int steps = hpw * per_head;

  auto tile_start = [&](int u, int* hq, int* q0) {
    *hq = h0 + u / per_head;
    *q0 = (qt0 + u % per_head) * BQ;
  };
  auto issue = [&](int u, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    int hq, q0;
    tile_start(u, &hq, &q0);
    const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    const uint16_t* qb = p.q + qrow0 * D;
    const uint16_t* gb = p.dout + qrow0 * DV;
    copy_tile<D, BQ, NW>(qb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, 0), wave,
                         roff);
    if constexpr (!UNI)
      copy_tile<D, BQ, NW>(qb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, 0), wave,
                           toff);
    if constexpr (SQ) {
      copy_tile<D, BQ, NW>(gb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, 1), wave,
                           roff);
      if constexpr (!UNI)
        copy_tile<D, BQ, NW>(gb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, 1), wave,
                             toff);
    } else {
      copy_tile<DV, BQ, NW>(gb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, 1), wave,
                            groff);
      copy_tile<DV, BQ, NW>(gb, q0, p.Nq, qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, 1), wave,
                            gtoff);
    }
    if (wave < 2) {  // lse2 (wave 0) and Delta (wave 1): one dword per lane
      const float* src = (wave == 0 ? p.lse2 : p.delta) + qrow0 + q0;
      const int n = min(BQ, p.Nq - q0);
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 4, kRawBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(buf_at<buf, SEP, 128>(ld0, ld1) + wave * 64),
          4, lane * 4, 0, 0, 0);
    }
  };

  const int v_g = lane >> 4, v_r = lane & 15;
  const int v_key = 4 * hl + (v_r >> 2);
  const int v_d = 16 * (v_g & 1) + 4 * (v_r & 3);
  // swizzles of the transposed reads' rows v_key (+ 16 kc) and v_key + 8
  const int v_sw = UNI ? u_swz<UNI ? DP : 64>(v_key) : v_swz<DP>(v_key);
  const int v_sw8 = UNI ? u_swz<UNI ? DP : 64>(v_key + 8) : v_sw;
  const int v_swv = v_swz<DVP>(v_key);

  // P in place of S (P waves); accumulator register e of block qb is query
  // row q0 + qb*32 + 8 (e / 4) + 4 hl + e % 4.  With a mask, its base-2
  // bias joins the exponent; rows past Nq and rows that saw no key in the
  // forward (lse -inf) get P = 0.
  // A mask with row stride 0 (a key-padding mask, or any mask broadcast
  // over the query rows) has one value per key of a head: read once, on
  // every tile whose rows all lie below Nq.  The last tile of a head, which
  // may hold rows past Nq, takes the per-row path: such rows have Q = 0 and
  // a zero lse2 slot, so without the row check P would be exp2(bias), which
  // overflows the 16-bit P operand for large additive biases and turns
  // 0 * inf into NaN in dV and dK.
  auto probs_impl = [&](auto mskc, auto bufc, auto rowc, f32x16* s, int q0, int hq)
      __attribute__((always_inline)) {
    constexpr bool MSK = decltype(mskc)::value;
    constexpr int buf = decltype(bufc)::value;
    constexpr bool ROWMASK = decltype(rowc)::value;  // the mask varies along rows
    const uint8_t* mbase = nullptr;
    if constexpr (MASKED) mbase = p.mask;
    const int64_t mrow0 = MASKED ? b * p.msb + hq * p.msh : 0;
    float kbias = 0.f;
    if constexpr (MASKED && !ROWMASK)
      kbias = key < p.Nkv ? mask_bias1<Tag>(mbase, p.mask_mode, mrow0 + key) : 0.f;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = qb * 32 + 8 * j + 4 * hl;
        const f32x4 ls = *(const f32x4*)(buf_at<buf, SEP, 128>(ld0, ld1) + r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv;
          if constexpr (MASKED && ROWMASK) {
            const int row = q0 + r + e;
            const float bias =
                row < p.Nq && key < p.Nkv
                    ? mask_bias1<Tag>(mbase, p.mask_mode, mrow0 + row * p.msq + key)
                    : 0.f;
            pv = (row < p.Nq && ls[e] != INFINITY)
                     ? fast_exp2(fmaf(p.cs, s[qb][4 * j + e], bias) - ls[e])
                     : 0.f;
          } else if constexpr (MASKED) {
            // one bias per key; every row is below Nq here, and rows that
            // saw no key have lse2 = +inf
            pv = fast_exp2(fmaf(p.cs, s[qb][4 * j + e], kbias - ls[e]));
          } else {
            pv = fast_exp2(fmaf(p.cs, s[qb][4 * j + e], -ls[e]));
          }
          if (MSK && key > q0 + r + e + p.coff) pv = 0.f;
          s[qb][4 * j + e] = pv;
        }
      }
  };
  auto probs = [&](auto mskc, auto bufc, f32x16* s, int q0, int hq)
      __attribute__((always_inline)) {
    if (MASKED && p.msq == 0 && q0 + BQ <= p.Nq)
      probs_impl(mskc, bufc, std::false_type{}, s, q0, hq);
    else
      probs_impl(mskc, bufc, std::true_type{}, s, q0, hq);
  };

  auto tile = [&](int u, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (u + 1 < steps) issue(u + 1, std::integral_constant<int, buf ^ 1>{});
    int hq, q0;
    tile_start(u, &hq, &q0);

    // 1. S (P waves) or dP (dS waves)
    f32x16 s[NQB];
    auto prod1 = [&](auto dcc, auto rwc, const uint16_t* ra) {
      constexpr int DCX = decltype(dcc)::value, RW = decltype(rwc)::value;
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        s[qb] = f32x16{};
#pragma unroll
        for (int kc = 0; kc < DCX; ++kc)
          s[qb] = N::mfma(read_rows<RW, RDR>(ra, qb * 32 + l32, kc, hl), bf[kc], s[qb]);
      }
    };
    if constexpr (SQ)
      prod1(std::integral_constant<int, DC>{}, std::integral_constant<int, DP>{},
            qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, pw ? 0 : 1));
    else if (pw)
      prod1(std::integral_constant<int, DC>{}, std::integral_constant<int, DP>{},
            qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, 0));
    else
      prod1(std::integral_constant<int, DCV>{}, std::integral_constant<int, DVP>{},
            qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, 1));
    u32x4 bop[NKC];
    if (pw) {
      if (CAUSAL && kw0 + 31 > q0 + p.coff)
        probs(std::true_type{}, bufc, s, q0, hq);
      else
        probs(std::false_type{}, bufc, s, q0, hq);
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) pack_tile<Tag>(s[qb], &bop[qb * 2]);
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) xp[kw][kc][lane] = bop[kc];
    }
    // P is in LDS for the partner wave: this wave's LDS stores are done
    // (lgkmcnt 0), then the barrier.  Not __syncthreads, whose fence would
    // also wait for the next tile's copies still in flight into the other
    // buffers; the empty asm statements keep the compiler from moving LDS
    // accesses across the barrier.
    if constexpr (SEP) {
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
    } else {
      __syncthreads();
    }
    if (!pw) {
      // dS = P (dP - Delta) from the partner's P
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          const u32x4 w = xp[kw][qb * 2 + hf][lane];
#pragma unroll
          for (int jj = 0; jj < 2; ++jj) {
            const int j = 2 * hf + jj;
            const f32x4 dl =
                *(const f32x4*)(buf_at<buf, SEP, 128>(ld0, ld1) + 64 + qb * 32 + 8 * j + 4 * hl);
            const float pv[4] = {lo_f32<Tag>(w[2 * jj]), hi_f32<Tag>(w[2 * jj]),
                                 lo_f32<Tag>(w[2 * jj + 1]), hi_f32<Tag>(w[2 * jj + 1])};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              s[qb][4 * j + e] = pv[e] * (s[qb][4 * j + e] - dl[e]);
          }
        }
        pack_tile<Tag>(s[qb], &bop[qb * 2]);
      }
    }
    // 2. dV^T += dO^T P (P waves) or dK^T += Q^T dS (dS waves)
    auto prod2 = [&](auto ndc, auto rwc, const uint16_t* rb, int sw, int sw8) {
      constexpr int NDX = decltype(ndc)::value, RW = decltype(rwc)::value;
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const int row = kc * 16 + v_key;
#pragma unroll
        for (int db = 0; db < NDX; ++db)
          acc[db] = N::mfma(read_cols<RW>(rb, row, db, v_d, sw, sw8), bop[kc], acc[db]);
      }
    };
    if constexpr (UNI)
      prod2(std::integral_constant<int, NDB>{}, std::integral_constant<int, DP>{},
            qg_tile<buf, SEP, TILE, TILEV>(rows0, rows1, pw ? 1 : 0), v_sw, v_sw8);
    else if constexpr (SQ)
      prod2(std::integral_constant<int, NDB>{}, std::integral_constant<int, DP>{},
            qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, pw ? 1 : 0), v_sw, v_sw);
    else if (pw)
      prod2(std::integral_constant<int, NDBV>{}, std::integral_constant<int, DVP>{},
            qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, 1), v_swv, v_swv);
    else
      prod2(std::integral_constant<int, NDB>{}, std::integral_constant<int, DP>{},
            qg_tile<buf, SEP, TILE, TILEV>(cols0, cols1, 0), v_sw, v_sw);
  };

  if (steps > 0) issue(0, std::integral_constant<int, 0>{});
  for (int u = 0; u < steps; u += 2) {
    tile(u, std::integral_constant<int, 0>{});
    if (u + 1 < steps) tile(u + 1, std::integral_constant<int, 1>{});
  }

  if (key < p.Nkv) {
    if (pw)
      store_kv_grad<DV, Tag>(p, p.dv, p.dvp, acc, 1.f, krow0 + key, hs, hl);
    else
      store_kv_grad<D, Tag>(p, p.dk, p.dkp, acc, p.scale, krow0 + key, hs, hl);
  }
}

// dK, dV with each wave doing all four products for its own 32 keys
// (D = 64, 80 and 96; written for D = 128 too, where it spills): 4 waves
// over 128 keys, K and V of the wave's keys in registers.
// Per query tile of BQ rows (64 at D = 64; 32 at 80, 96 and 128, where K,
// V and the two accumulators take 144 or 192 registers):
//   S = Q K^T and dP = dO V^T (row reads of the Q and dO tiles),
//   P = exp2(cs S - lse2) (0 above the causal diagonal), dS = P (dP - Delta),
//   dV^T += dO^T P and dK^T += Q^T dS (transposed reads of the same tiles,
//   staged once in the layout of both reads).
// Nothing passes between waves, so a tile needs only the copies' barrier,
// and the two workgroups on a CU overlap one another's vector and matrix
// work.
template <int D, class Tag, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, 2) void attn_dkdv_solo_kernel(BwdParams p) {
  constexpr int DP = compute_dim(D);
  static_assert(has_both_swz<DP>(), "one-copy tile layout");
  constexpr int NW = 4, BK = 128;
  constexpr int NQB = D == 64 ? 2 : 1, BQ = NQB * 32;
  constexpr int DC = DP / 16, NDB = DP / 32, NKC = BQ / 16;
  constexpr int TILE = BQ * DP;
  constexpr int IPW = TileCopy<D, BQ, NW>::PER_WAVE;
  using N = Num<Tag>;

  // per buffer: the Q tile, then the dO tile; lse2 at 0 and Delta at 64
  // (one dword per lane of a 64-lane copy, zeros past the tile's rows)
  __shared__ __attribute__((aligned(1024))) uint16_t tq0[2 * TILE], tq1[2 * TILE];
  __shared__ __attribute__((aligned(256))) float ld0[128], ld1[128];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;

  int bid = CAUSAL ? longest_first(blockIdx.x, p.n_tiles, p.total) : xcd_remap(blockIdx.x, p.total);
  const int kt = bid % p.n_tiles;
  bid /= p.n_tiles;
  const int hs = bid % p.hsplit;
  bid /= p.hsplit;
  const int hk = bid % p.Hkv;
  const int b = bid / p.Hkv;
  const int k0 = kt * BK;
  const int kw0 = k0 + wave * 32;
  const int key = kw0 + l32;
  const int hpw = p.G / p.hsplit;
  const int h0 = hk * p.G + hs * hpw;

  const size_t krow0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  u32x4 kf[DC], vf[DC];
#pragma unroll
  for (int kc = 0; kc < DC; ++kc) {
    u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
    if (key < p.Nkv && kc * 16 + hl * 8 < D) {
      x = *(const u32x4*)(p.k + (krow0 + key) * D + kc * 16 + hl * 8);
      y = *(const u32x4*)(p.v + (krow0 + key) * D + kc * 16 + hl * 8);
    }
    kf[kc] = x;
    vf[kc] = y;
  }
  f32x16 acck[NDB], accv[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) acck[i] = accv[i] = f32x16{};

  uint32_t roff[IPW];
  copy_offsets<D, BQ, NW, kReadBoth>(wave, lane, roff);

  const int nqt = (p.Nq + BQ - 1) / BQ;
  const int qt0 = CAUSAL ? min(nqt, max(0, k0 - p.coff) / BQ) : 0;
  const int per_head = nqt - qt0;
  const int steps = hpw * per_head;

  auto tile_start = [&](int u, int* hq, int* q0) {
    *hq = h0 + u / per_head;
    *q0 = (qt0 + u % per_head) * BQ;
  };
  auto issue = [&](int u, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    int hq, q0;
    tile_start(u, &hq, &q0);
    const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
    uint16_t* const tb = buf_at<buf, true, 0>(tq0, tq1);
    copy_tile<D, BQ, NW>(p.q + qrow0 * D, q0, p.Nq, tb, wave, roff);
    copy_tile<D, BQ, NW>(p.dout + qrow0 * D, q0, p.Nq, tb + TILE, wave, roff);
    if (wave < 2) {  // lse2 (wave 0) and Delta (wave 1)
      const float* src = (wave == 0 ? p.lse2 : p.delta) + qrow0 + q0;
      const int n = min(BQ, p.Nq - q0);
      const __amdgpu_buffer_rsrc_t r =
          __builtin_amdgcn_make_buffer_rsrc((void*)src, 0, n * 4, kRawBufferFlags);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          r, (__attribute__((address_space(3))) void*)(buf_at<buf, true, 0>(ld0, ld1) + wave * 64),
          4, lane * 4, 0, 0, 0);
    }
  };

  const int v_g = lane >> 4, v_r = lane & 15;
  const int v_key = 4 * hl + (v_r >> 2);
  const int v_d = 16 * (v_g & 1) + 4 * (v_r & 3);
  const int v_sw = u_swz<DP>(v_key), v_sw8 = u_swz<DP>(v_key + 8);

  // P and dS in place of S and dP; accumulator register e of block qb is
  // query row q0 + qb*32 + 8 (e / 4) + 4 hl + e % 4.  A mask enters as in
  // the wave pairs: its base-2 bias joins the exponent, read once per key
  // when it does not vary along rows and the tile holds no row past Nq,
  // else per element with rows past Nq and rows that saw no key (lse2
  // +inf) getting P = 0.
  auto grads_impl = [&](auto mskc, auto rowc, const float* lsb, f32x16* s, f32x16* dp, int q0,
                        int hq) __attribute__((always_inline)) {
    constexpr bool MSK = decltype(mskc)::value;
    constexpr bool ROWMASK = decltype(rowc)::value;
    const uint8_t* mbase = nullptr;
    if constexpr (MASKED) mbase = p.mask;
    const int64_t mrow0 = MASKED ? b * p.msb + hq * p.msh : 0;
    float kbias = 0.f;
    if constexpr (MASKED && !ROWMASK)
      kbias = key < p.Nkv ? mask_bias1<Tag>(mbase, p.mask_mode, mrow0 + key) : 0.f;
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = qb * 32 + 8 * j + 4 * hl;
        const f32x4 ls = *(const f32x4*)(lsb + r);
        const f32x4 dl = *(const f32x4*)(lsb + 64 + r);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          float pv;
          if constexpr (MASKED && ROWMASK) {
            const int row = q0 + r + e;
            const float bias =
                row < p.Nq && key < p.Nkv
                    ? mask_bias1<Tag>(mbase, p.mask_mode, mrow0 + row * p.msq + key)
                    : 0.f;
            pv = (row < p.Nq && ls[e] != INFINITY)
                     ? fast_exp2(fmaf(p.cs, s[qb][4 * j + e], bias) - ls[e])
                     : 0.f;
          } else if constexpr (MASKED) {
            pv = fast_exp2(fmaf(p.cs, s[qb][4 * j + e], kbias - ls[e]));
          } else {
            pv = fast_exp2(fmaf(p.cs, s[qb][4 * j + e], -ls[e]));
          }
          if (MSK && key > q0 + r + e + p.coff) pv = 0.f;
          s[qb][4 * j + e] = pv;
          dp[qb][4 * j + e] = pv * (dp[qb][4 * j + e] - dl[e]);
        }
      }
  };
  auto grads = [&](auto mskc, const float* lsb, f32x16* s, f32x16* dp, int q0, int hq)
      __attribute__((always_inline)) {
    if (MASKED && p.msq == 0 && q0 + BQ <= p.Nq)
      grads_impl(mskc, std::false_type{}, lsb, s, dp, q0, hq);
    else
      grads_impl(mskc, std::true_type{}, lsb, s, dp, q0, hq);
  };

  auto tile = [&](int u, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (u + 1 < steps) issue(u + 1, std::integral_constant<int, buf ^ 1>{});
    int hq, q0;
    tile_start(u, &hq, &q0);
    const uint16_t* const tq = buf_at<buf, true, 0>(tq0, tq1);
    const uint16_t* const tg = tq + TILE;
    f32x16 s[NQB], dp[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      s[qb] = f32x16{};
      dp[qb] = f32x16{};
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        s[qb] = N::mfma(read_rows<DP, kReadBoth>(tq, qb * 32 + l32, kc, hl), kf[kc], s[qb]);
        dp[qb] = N::mfma(read_rows<DP, kReadBoth>(tg, qb * 32 + l32, kc, hl), vf[kc], dp[qb]);
      }
    }
    const float* const lsb = buf_at<buf, true, 0>(ld0, ld1);
    if (CAUSAL && kw0 + 31 > q0 + p.coff)
      grads(std::true_type{}, lsb, s, dp, q0, hq);
    else
      grads(std::false_type{}, lsb, s, dp, q0, hq);
    u32x4 bp[NKC], bs[NKC];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
      pack_tile<Tag>(s[qb], &bp[qb * 2]);
      pack_tile<Tag>(dp[qb], &bs[qb * 2]);
    }
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int row = kc * 16 + v_key;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        accv[db] = N::mfma(read_cols<DP>(tg, row, db, v_d, v_sw, v_sw8), bp[kc], accv[db]);
        acck[db] = N::mfma(read_cols<DP>(tq, row, db, v_d, v_sw, v_sw8), bs[kc], acck[db]);
      }
    }
  };

  if (steps > 0) issue(0, std::integral_constant<int, 0>{});
  for (int u = 0; u < steps; u += 2) {
    tile(u, std::integral_constant<int, 0>{});
    if (u + 1 < steps) tile(u + 1, std::integral_constant<int, 1>{});
  }

  if (key < p.Nkv) {
    store_kv_grad<D, Tag>(p, p.dv, p.dvp, accv, 1.f, krow0 + key, hs, hl);
    store_kv_grad<D, Tag>(p, p.dk, p.dkp, acck, p.scale, krow0 + key, hs, hl);
  }
}

// dK, dV = sums of the hsplit partials (dK times scale), rounded to 16 bits;
// four elements per thread.  n4k (n4v): float4s per partial of dK (dV).
template <class Tag>
__global__ __launch_bounds__(256) void attn_dkdv_reduce(BwdParams p, size_t n4k, size_t n4v) {
  using N = Num<Tag>;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n4k) {
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < p.hsplit; ++h) a += ((const f32x4*)p.dkp)[h * n4k + i];
    a *= p.scale;
    ((u32x2*)p.dk)[i] = u32x2{N::pack2(a[0], a[1]), N::pack2(a[2], a[3])};
  }
  if (i < n4v) {
    f32x4 c = {0.f, 0.f, 0.f, 0.f};
    for (int h = 0; h < p.hsplit; ++h) c += ((const f32x4*)p.dvp)[h * n4v + i];
    ((u32x2*)p.dv)[i] = u32x2{N::pack2(c[0], c[1]), N::pack2(c[2], c[3])};
  }
}

// dQ for 128 query rows (4 waves x 32) of query head hq: loop over key
// tiles (32 keys) like the forward.  Per tile and wave:
//   S^T = K Q^T, dP^T = V dO^T      (rows: 32 keys, columns: 32 queries)
//   P, dS as above (lse2 and Delta: one value per lane)
//   dQ^T += K^T dS^T                (rows: D, columns: 32 queries)
// Q and dO stay in registers; K is copied into LDS once in the layout of
// both reads at D = 64 and 128, else twice (row-read and transposed
// layouts), and V once, two buffers deep, the loop unrolled by two.
// One wave per SIMD at D = 256: Q, dO and the dQ accumulators take 256
// registers (the (192, 128) pair's 208 still fit two waves).  With V rows
// of DV != D elements, dO and V tiles are DV wide and dP reduces over DV.
template <int D, int DV, class Tag, bool CAUSAL, bool MASKED>
__global__ __launch_bounds__(256, D == 256 ? 1 : 2) void attn_dq_kernel(BwdParams p) {
  constexpr bool SQ = D == DV;
  constexpr int QB = dq_row_blocks(D, CAUSAL);
  constexpr int NW = 4, BM = dq_block_rows(D, CAUSAL), BN = 32;
  static_assert(BM == NW * 32 * QB, "dQ tile rows");
  constexpr int DP = compute_dim(D), DVP = compute_dim(DV);
  constexpr int DC = DP / 16, NDB = DP / 32, DCV = DVP / 16;
  constexpr int TILE = BN * DP, TILEV = BN * DVP;
  constexpr int IPW = TileCopy<D, BN, NW>::PER_WAVE;
  constexpr int IPWV = TileCopy<DV, BN, NW>::PER_WAVE;
  using N = Num<Tag>;

  // With UNI one copy of K in the layout of both reads (kr) serves the row
  // reads of S and the transposed reads of dQ, and V shares that layout.
  constexpr bool SEP = bwd_sep_buffers(D, DV);
  constexpr bool UNI = SEP && (D == 64 || D == 128);  // (at 96: 5% slower here)
  constexpr int RDR = UNI ? kReadBoth : kReadRows;
  __shared__ __attribute__((aligned(1024))) uint16_t kr0[SEP ? TILE : 2 * TILE], kr1[SEP ? TILE : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t ktr0[UNI ? 1 : SEP ? TILE : 2 * TILE],
      ktr1[SEP && !UNI ? TILE : 1];
  __shared__ __attribute__((aligned(1024))) uint16_t vr0[SEP ? TILEV : 2 * TILEV], vr1[SEP ? TILEV : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, l32 = lane & 31, hl = lane >> 5;

  // (a split launch renumbers its whole tiles and its pieces separately, as
  // the forward does)
  int bid, sp = 0;
  bool piece = false;
  if (!CAUSAL && p.dq_splits > 1 && (int)blockIdx.x >= p.dq_whole) {
    const int j = xcd_remap(blockIdx.x - p.dq_whole, p.total - p.dq_whole);
    piece = true;
    sp = j % p.dq_splits;
    bid = p.dq_whole + j / p.dq_splits;
  } else if (!CAUSAL && p.dq_splits > 1) {
    bid = xcd_remap(blockIdx.x, p.dq_whole);
  } else {
    bid = CAUSAL ? longest_first(blockIdx.x, p.n_tiles, p.total) : xcd_remap(blockIdx.x, p.total);
  }
  const int tile_id = bid;
  int qt = bid % p.n_tiles;
  bid /= p.n_tiles;
  const int hq = bid % p.Hq;
  const int b = bid / p.Hq;
  if (CAUSAL) qt = p.n_tiles - 1 - qt;  // longest first
  const int hk = hq / p.G;
  const int q0 = qt * BM;
  const int qw0 = q0 + wave * 32 * QB;    // the wave's first query row
  // this lane's query (accumulator column) in row block qb: qw0 + 32 qb + l32
  const int kend = CAUSAL ? max(0, min(p.Nkv, q0 + BM + p.coff)) : p.Nkv;
  // key tiles [t0, t1): every tile, or this piece's key range
  const int t0 = piece ? sp * (p.dq_split_len / BN) : 0;
  const int t1 = piece ? min((kend + BN - 1) / BN, (sp + 1) * (p.dq_split_len / BN))
                       : (kend + BN - 1) / BN;

  const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const size_t krow0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  u32x4 qf[QB][DC], gf[QB][DCV];
  float nl2[QB], dl[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
    if constexpr (SQ) {
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        u32x4 x = {0u, 0u, 0u, 0u}, y = {0u, 0u, 0u, 0u};
        if (qrow < p.Nq && kc * 16 + hl * 8 < D) {
          x = *(const u32x4*)(p.q + (qrow0 + qrow) * D + kc * 16 + hl * 8);
          y = *(const u32x4*)(p.dout + (qrow0 + qrow) * D + kc * 16 + hl * 8);
        }
        qf[qb][kc] = x;
        gf[qb][kc < DCV ? kc : 0] = y;
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (qrow < p.Nq && kc * 16 + hl * 8 < D)
          x = *(const u32x4*)(p.q + (qrow0 + qrow) * D + kc * 16 + hl * 8);
        qf[qb][kc] = x;
      }
#pragma unroll
      for (int kc = 0; kc < DCV; ++kc) {
        u32x4 y = {0u, 0u, 0u, 0u};
        if (qrow < p.Nq && kc * 16 + hl * 8 < DV)
          y = *(const u32x4*)(p.dout + (qrow0 + qrow) * DV + kc * 16 + hl * 8);
        gf[qb][kc] = y;
      }
    }
    nl2[qb] = qrow < p.Nq ? -p.lse2[qrow0 + qrow] : 0.f;
    dl[qb] = qrow < p.Nq ? p.delta[qrow0 + qrow] : 0.f;
  }
  f32x16 dq[QB][NDB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < NDB; ++i) dq[qb][i] = f32x16{};

  uint32_t roff[IPW], toff[UNI ? 1 : IPW], vroff[SQ ? 1 : IPWV];
  copy_offsets<D, BN, NW, RDR>(wave, lane, roff);
  if constexpr (!UNI) copy_offsets<D, BN, NW, kReadCols>(wave, lane, toff);
  if constexpr (!SQ) copy_offsets<DV, BN, NW, kReadRows>(wave, lane, vroff);
  const uint16_t* Kg = p.k + krow0 * D;
  const uint16_t* Vg = p.v + krow0 * DV;
  auto issue = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    copy_tile<D, BN, NW>(Kg, t * BN, p.Nkv, buf_at<buf, SEP, TILE>(kr0, kr1), wave, roff);
    if constexpr (!UNI)
      copy_tile<D, BN, NW>(Kg, t * BN, p.Nkv, buf_at<buf, SEP, TILE>(ktr0, ktr1), wave, toff);
    if constexpr (SQ)
      copy_tile<D, BN, NW>(Vg, t * BN, p.Nkv, buf_at<buf, SEP, TILEV>(vr0, vr1), wave, roff);
    else
      copy_tile<DV, BN, NW>(Vg, t * BN, p.Nkv, buf_at<buf, SEP, TILEV>(vr0, vr1), wave, vroff);
  };

  const int v_g = lane >> 4, v_r = lane & 15;
  const int v_key = 4 * hl + (v_r >> 2);
  const int v_d = 16 * (v_g & 1) + 4 * (v_r & 3);
  const int v_sw = UNI ? u_swz<UNI ? DP : 64>(v_key) : v_swz<DP>(v_key);
  const int v_sw8 = UNI ? u_swz<UNI ? DP : 64>(v_key + 8) : v_sw;

  // register e of the score tile is key t*BN + 8 (e / 4) + 4 hl + e % 4.
  // With a mask, its base-2 bias joins the exponent; rows past Nq and rows
  // that saw no key in the forward (lse -inf) get P = 0.
  const uint8_t* mrow[QB] = {};
  if constexpr (MASKED) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int qrow = qw0 + 32 * qb + l32;
      const int64_t off = b * p.msb + hq * p.msh + (int64_t)min(qrow, p.Nq - 1) * p.msq;
      mrow[qb] = p.mask + off * (p.mask_mode == ATTN_MASK_BOOL ? 1 : 2);
    }
  }
  // (a row that saw no key has nl2 = -inf: P = 0)
  auto probs = [&](auto mskc, f32x16& s, f32x16& dp, int t, int qb) {
    constexpr bool MSK = decltype(mskc)::value;
    const int qrow = qw0 + 32 * qb + l32;
    const bool row_live = qrow < p.Nq;
    if constexpr (MASKED) {
      // A boolean mask that keeps all of this tile's keys for every row of
      // the wave (most tiles of a key-padding mask) changes nothing: take
      // the unmasked form (has-a-zero-byte test on each word, wave vote).
      // A row that saw no key in the forward has a removed key here, or
      // lies entirely above the causal diagonal (MSK zeroes it), and rows
      // past Nq have Q = dO = 0 and give dS = 0 either way.
      if (p.mask_mode == ATTN_MASK_BOOL) {
        uint32_t zero = 0u;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const uint32_t w = mask_keep4(mrow[qb], t * BN + 8 * g + 4 * hl, p.Nkv);
          zero |= (w - 0x01010101u) & ~w & 0x80808080u;
        }
        if (!__builtin_amdgcn_ballot_w64(zero != 0u)) {
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int e = 4 * g + i;
              float pv = fast_exp2(fmaf(p.cs, s[e], nl2[qb]));
              if (MSK && t * BN + 8 * g + 4 * hl + i > qrow + p.coff) pv = 0.f;
              dp[e] = pv * (dp[e] - dl[qb]);
            }
          return;
        }
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float bias[4] = {0.f, 0.f, 0.f, 0.f};
      if constexpr (MASKED)
        mask_bias4<Tag>(mrow[qb], p.mask_mode, t * BN + 8 * g + 4 * hl, p.Nkv, bias);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = 4 * g + i;
        float pv;
        if constexpr (MASKED)
          pv = row_live ? fast_exp2(fmaf(p.cs, s[e], bias[i]) + nl2[qb]) : 0.f;
        else
          pv = fast_exp2(fmaf(p.cs, s[e], nl2[qb]));
        if (MSK && t * BN + 8 * g + 4 * hl + i > qrow + p.coff) pv = 0.f;
        dp[e] = pv * (dp[e] - dl[qb]);
      }
    }
  };

  auto tile = [&](int t, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (t + 1 < t1) issue(t + 1, std::integral_constant<int, buf ^ 1>{});
    f32x16 s[QB], dp[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) s[qb] = dp[qb] = f32x16{};
    const uint16_t* kb = buf_at<buf, SEP, TILE>(kr0, kr1);
    const uint16_t* vb = buf_at<buf, SEP, TILEV>(vr0, vr1);
    // (each K and V operand read serves every row block)
    if constexpr (SQ) {
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        const u32x4 ak = read_rows<DP, RDR>(kb, l32, kc, hl);
        const u32x4 av = read_rows<DP, RDR>(vb, l32, kc, hl);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          s[qb] = N::mfma(ak, qf[qb][kc], s[qb]);
          dp[qb] = N::mfma(av, gf[qb][kc < DCV ? kc : 0], dp[qb]);
        }
      }
    } else {
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        const u32x4 ak = read_rows<DP>(kb, l32, kc, hl);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = N::mfma(ak, qf[qb][kc], s[qb]);
      }
#pragma unroll
      for (int kc = 0; kc < DCV; ++kc) {
        const u32x4 av = read_rows<DVP>(vb, l32, kc, hl);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dp[qb] = N::mfma(av, gf[qb][kc], dp[qb]);
      }
    }
    u32x4 ps[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      if (CAUSAL && t * BN + 31 > qw0 + 32 * qb + p.coff)
        probs(std::true_type{}, s[qb], dp[qb], t, qb);
      else
        probs(std::false_type{}, s[qb], dp[qb], t, qb);
      pack_tile<Tag>(dp[qb], ps[qb]);
    }
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      const int row = kc * 16 + v_key;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const u32x4 a = read_cols<DP>(UNI ? kb : buf_at<buf, SEP, TILE>(ktr0, ktr1), row, db, v_d,
                                      v_sw, v_sw8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) dq[qb][db] = N::mfma(a, ps[qb][kc], dq[qb][db]);
      }
    }
  };

  if (t0 < t1) issue(t0, std::integral_constant<int, 0>{});
  for (int t = t0; t < t1; t += 2) {
    tile(t, std::integral_constant<int, 0>{});
    if (t + 1 < t1) tile(t + 1, std::integral_constant<int, 1>{});
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = qw0 + 32 * qb + l32;
    if (qrow >= p.Nq) continue;
    if (!piece) {
      store_row<D, Tag>(p.dq + (qrow0 + qrow) * D, dq[qb], p.scale, hl);
      continue;
    }
    float* const dst =
        p.dqp + ((size_t)sp * p.dq_rows + (size_t)(tile_id - p.dq_whole) * BM + (qrow - q0)) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int col = db * 32 + 8 * i + 4 * hl;
        const f32x16& o = dq[qb][db];
        if (col < D)
          *(f32x4*)(dst + col) = f32x4{o[4 * i], o[4 * i + 1], o[4 * i + 2], o[4 * i + 3]};
      }
  }
}

// dQ rows of the split tiles: the sum of the pieces' fp32 partials times
// the scale, rounded to 16 bits; four elements per thread.
template <int D, class Tag>
__global__ __launch_bounds__(256) void attn_dq_reduce(BwdParams p, size_t n4) {
  using N = Num<Tag>;
  constexpr int C4 = D / 4;
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  const size_t r = i / C4;
  const int c = (int)(i % C4) * 4;
  constexpr int BM = dq_block_rows(D, false);  // (only non-causal launches split)
  const long long tile = p.dq_whole + (long long)(r / BM);
  const int q = (int)(tile % p.n_tiles) * BM + (int)(r % BM);
  if (q >= p.Nq) return;
  f32x4 a = *(const f32x4*)(p.dqp + r * D + c);
  for (int s = 1; s < p.dq_splits; ++s) a += *(const f32x4*)(p.dqp + ((size_t)s * p.dq_rows + r) * D + c);
  const u32x2 y = {N::pack2(a[0] * p.scale, a[1] * p.scale), N::pack2(a[2] * p.scale, a[3] * p.scale)};
  *(u32x2*)(p.dq + ((size_t)(tile / p.n_tiles) * p.Nq + q) * D + c) = y;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

bool overlaps_bytes(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

// Q, K, dQ, dK rows have D elements; V, O, dO, dV rows Dv (= D, or the
// (192, 128) pair).
int validate_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout,
                 const float* lse, const void* dq, const void* dk, const void* dv, int B, int Hq,
                 int Hkv, int Nq, int Nkv, int D, int Dv, float scale, int causal, int dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  const bool sq_ok = D == 64 || D == 80 || D == 96 || D == 128 || D == 256;
  if (!(Dv == D ? sq_ok : (D == 192 && Dv == 128))) return ATTN_EINVAL;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  if (!isfinite(scale)) return ATTN_EINVAL;
  const void* ins[6] = {q, k, v, o, dout, lse};
  const void* outs[3] = {dq, dk, dv};
  for (const void* x : ins)
    if (!x || ((uintptr_t)x & 15)) return ATTN_EINVAL;
  for (const void* x : outs)
    if (!x || ((uintptr_t)x & 15)) return ATTN_EINVAL;
  const size_t rows = (size_t)B * Hq * Nq, krows = (size_t)B * Hkv * Nkv;
  if (rows > (size_t)INT32_MAX || krows > (size_t)INT32_MAX) return ATTN_EINVAL;
  const size_t qb = rows * D * 2, kb = krows * D * 2;
  const size_t ob = rows * Dv * 2, vb = krows * Dv * 2;
  const size_t in_bytes[6] = {qb, kb, vb, ob, ob, rows * 4};
  const size_t out_bytes[3] = {qb, kb, vb};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 6; ++j)
      if (overlaps_bytes(outs[i], out_bytes[i], ins[j], in_bytes[j])) return ATTN_EINVAL;
    for (int j = 0; j < i; ++j)
      if (overlaps_bytes(outs[i], out_bytes[i], outs[j], out_bytes[j])) return ATTN_EINVAL;
  }
  return ATTN_OK;
}

// Workgroups over which the query heads of one KV head are split for dK/dV:
// the smallest divisor of G that gives at least two workgroups per compute
// unit (G when none does).
int bwd_head_split(int B, int Hkv, int Nkv, int G, int cus) {
  const long long base = (long long)B * Hkv * ((Nkv + 127) / 128);
  for (int d = 1; d < G; ++d)
    if (G % d == 0 && base * d >= 2LL * cus) return d;
  return G;
}

// The forward's attention mask, as attn_fwd_masked takes it.
struct BwdMask {
  const void* ptr = nullptr;
  int type = ATTN_MASK_NONE;
  int64_t sb = 0, sh = 0, sq = 0;
};

int validate_bwd_mask(const BwdMask& m, const void* dq, const void* dk, const void* dv, int B,
                      int Hq, int Hkv, int Nq, int Nkv, int D, int Dv) {
  if (m.type == ATTN_MASK_NONE) return ATTN_OK;
  if (m.type != ATTN_MASK_BOOL && m.type != ATTN_MASK_ADD) return ATTN_EINVAL;
  if (!m.ptr || ((uintptr_t)m.ptr & 7)) return ATTN_EINVAL;
  if (m.sb < 0 || m.sh < 0 || m.sq < 0 || ((m.sb | m.sh | m.sq) & 3)) return ATTN_EINVAL;
  const int esz = m.type == ATTN_MASK_BOOL ? 1 : 2;
  const __int128 mb = esz * ((__int128)(B - 1) * m.sb + (__int128)(Hq - 1) * m.sh +
                             (__int128)(Nq - 1) * m.sq + Nkv);
  if (mb > ((__int128)1 << 62)) return ATTN_EINVAL;
  const size_t qb = (size_t)B * Hq * Nq * D * 2, kb = (size_t)B * Hkv * Nkv * D * 2;
  const size_t vb = (size_t)B * Hkv * Nkv * Dv * 2;
  if (overlaps_bytes(dq, qb, m.ptr, (size_t)mb) || overlaps_bytes(dk, kb, m.ptr, (size_t)mb) ||
      overlaps_bytes(dv, vb, m.ptr, (size_t)mb))
    return ATTN_EINVAL;
  return ATTN_OK;
}

// dQ and dK/dV need only the Delta rows, not each other: dQ runs on a
// second stream of the library's, forked from the caller's stream after the
// Delta kernel and joined back before the caller's stream goes on, so that
// each kernel's last, partial round of workgroups shares the device with
// the other's instead of leaving CUs idle.  Measured against one stream:
// +3.5% to +21% at D = 64 (sweep and causal GQA, 4096 and 16384 tokens),
// +5.8% at D = 256, neutral at 96 and (192, 128); at D = 128 the two
// kernels' streams through L2 collide (video-DiT 17160 -3.5%, 75600
// neutral), so D = 128 keeps one stream.  One side stream and a pair of
// events per device; the events are recorded and waited on under a host
// lock, so concurrent calls cannot mix up their fork and join points.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
  bool init = false;
};
constexpr int kMaxSideDevices = 64;
std::mutex g_side_mu;
SideStream g_side[kMaxSideDevices];

// With g_side_mu held: the current device's side stream and events.
hipError_t side_stream(SideStream** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxSideDevices) return hipErrorInvalidDevice;
  SideStream& ss = g_side[dev];
  if (!ss.init) {
    e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming);
    if (e != hipSuccess) return e;
    ss.init = true;
  }
  *out = &ss;
  return hipSuccess;
}

// The dK/dV kernel: one wave per 32 keys doing all four products where its
// registers allow (D = 64, 80 and 96, with or without a mask; at D = 128 it
// spills 124-216 bytes per lane and runs 1.5x slower than the wave pairs),
// else the pairs.
constexpr bool bwd_solo_dkdv(int D, int DV, bool) {
  return D == DV && (D == 64 || D == 80 || D == 96);
}

template <int D, int DV, class Tag, bool MASKED>
hipError_t launch_bwd(BwdParams p, bool causal, hipStream_t st, SideStream* side) {
  constexpr bool kFork = D != 128;
  const int rows = p.B * p.Hq * p.Nq;
  const size_t threads = (size_t)rows * bwd_delta_lanes(DV);  // Delta: rows of O and dO
  hipLaunchKernelGGL((attn_delta_kernel<DV, Tag>), dim3((unsigned)((threads + 255) / 256)),
                     dim3(256), 0, st, p, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // dQ on the side stream, after Delta (one stream at D = 128: dQ after dK/dV)
  const hipStream_t sq = kFork ? side->s : st;
  if (kFork) {
    e = hipEventRecord(side->fork, st);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return e;
  }
  BwdParams pq = p;
  const int dq_bm = dq_block_rows(D, causal);
  pq.n_tiles = (p.Nq + dq_bm - 1) / dq_bm;
  pq.total = p.dq_splits > 1 ? p.dq_whole + (p.B * p.Hq * pq.n_tiles - p.dq_whole) * p.dq_splits
                             : p.B * p.Hq * pq.n_tiles;
  auto launch_dq = [&]() {
    if (causal)
      hipLaunchKernelGGL((attn_dq_kernel<D, DV, Tag, true, MASKED>), dim3(pq.total), dim3(256),
                         0, sq, pq);
    else
      hipLaunchKernelGGL((attn_dq_kernel<D, DV, Tag, false, MASKED>), dim3(pq.total), dim3(256),
                         0, sq, pq);
    hipError_t e2 = hipGetLastError();
    if (e2 == hipSuccess && p.dq_splits > 1) {
      const size_t n4 = (size_t)p.dq_rows * (D / 4);
      hipLaunchKernelGGL((attn_dq_reduce<D, Tag>), dim3((unsigned)((n4 + 255) / 256)), dim3(256),
                         0, sq, pq, n4);
      e2 = hipGetLastError();
    }
    return e2;
  };
  if (kFork) {
    e = launch_dq();
    if (e != hipSuccess) return e;
  }
  BwdParams pk = p;
  pk.n_tiles = (p.Nkv + 127) / 128;
  pk.total = p.B * p.Hkv * p.hsplit * pk.n_tiles;
  if constexpr (bwd_solo_dkdv(D, DV, MASKED)) {
    if (causal)
      hipLaunchKernelGGL((attn_dkdv_solo_kernel<D, Tag, true, MASKED>), dim3(pk.total), dim3(256),
                         0, st, pk);
    else
      hipLaunchKernelGGL((attn_dkdv_solo_kernel<D, Tag, false, MASKED>), dim3(pk.total),
                         dim3(256), 0, st, pk);
  } else if (causal) {
    hipLaunchKernelGGL((attn_dkdv_pair_kernel<D, DV, Tag, true, MASKED>), dim3(pk.total),
                       dim3(512), 0, st, pk);
  } else {
    hipLaunchKernelGGL((attn_dkdv_pair_kernel<D, DV, Tag, false, MASKED>), dim3(pk.total),
                       dim3(512), 0, st, pk);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (p.hsplit > 1) {
    const size_t n4k = (size_t)p.B * p.Hkv * p.Nkv * D / 4;
    const size_t n4v = (size_t)p.B * p.Hkv * p.Nkv * DV / 4;
    const size_t n4 = n4k > n4v ? n4k : n4v;
    hipLaunchKernelGGL((attn_dkdv_reduce<Tag>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0,
                       st, p, n4k, n4v);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (!kFork) return launch_dq();
  // join: the caller's stream goes on after dQ too
  e = hipEventRecord(side->join, side->s);
  if (e == hipSuccess) e = hipStreamWaitEvent(st, side->join, 0);
  return e;
}

template <int D, int DV>
hipError_t launch_bwd_masks(bool bf, bool masked, const BwdParams& p, bool cz, hipStream_t st,
                            SideStream* side) {
  if (masked)
    return bf ? launch_bwd<D, DV, TagBF16, true>(p, cz, st, side)
              : launch_bwd<D, DV, TagF16, true>(p, cz, st, side);
  return bf ? launch_bwd<D, DV, TagBF16, false>(p, cz, st, side)
            : launch_bwd<D, DV, TagF16, false>(p, cz, st, side);
}

hipError_t launch_bwd_d(int D, int Dv, bool bf, bool masked, const BwdParams& p, bool cz,
                        hipStream_t st) {
  std::lock_guard<std::mutex> lock(g_side_mu);
  SideStream* side = nullptr;
  const hipError_t e = side_stream(&side);
  if (e != hipSuccess) return e;
  if (Dv != D) return launch_bwd_masks<192, 128>(bf, masked, p, cz, st, side);
  switch (D) {
    case 64: return launch_bwd_masks<64, 64>(bf, masked, p, cz, st, side);
    case 80: return launch_bwd_masks<80, 80>(bf, masked, p, cz, st, side);
    case 96: return launch_bwd_masks<96, 96>(bf, masked, p, cz, st, side);
    case 256: return launch_bwd_masks<256, 256>(bf, masked, p, cz, st, side);
    default: return launch_bwd_masks<128, 128>(bf, masked, p, cz, st, side);
  }
}

int run_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
            const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
            int Nkv, int D, int Dv, float scale, int causal, int dtype, void* stream,
            const BwdMask& m) {
  int rc = validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, Dv, scale,
                        causal, dtype);
  if (rc == ATTN_OK) rc = validate_bwd_mask(m, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, Dv);
  if (rc != ATTN_OK) return rc;
  int cus = 0;
  rc = attn_host::check_device(&cus);
  if (rc != ATTN_OK) return rc;
  const int G = Hq / Hkv;
  const int hsplit = bwd_head_split(B, Hkv, Nkv, G, cus);
  const long long kgrid = (long long)B * Hkv * hsplit * ((Nkv + 127) / 128);
  const int dq_bm = dq_block_rows(D, causal != 0);
  const long long qgrid = (long long)B * Hq * ((Nq + dq_bm - 1) / dq_bm);
  if (kgrid > INT32_MAX || qgrid > INT32_MAX) return ATTN_EINVAL;
  // dQ without a causal mask: the tiles of a last, partial round of
  // workgroups are cut into key ranges (the forward's cost model), so they
  // finish in a fraction of a round.  Two dQ workgroups per CU (one at
  // D = 256).
  int dq_whole = 0, dq_splits = 1, dq_len = 0, dq_rows = 0;
  if (!causal) {
    const long long slots = (long long)(D == 256 ? 1 : 2) * cus;
    const long long rem = qgrid % slots;
    const int ktiles = (Nkv + 31) / 32;
    if (rem > 0 && qgrid > rem) {
      int S = attn_planner::balanced_splits(rem, slots, ktiles, 1.0);
      const int tps = (ktiles + S - 1) / S;
      S = (ktiles + tps - 1) / tps;
      if (S > 1 && qgrid + rem * (S - 1) <= INT32_MAX) {
        dq_splits = S;
        dq_len = tps * 32;
        dq_whole = (int)(qgrid - rem);
        dq_rows = (int)rem * dq_bm;
      }
    }
  }

  // workspace: Delta and lse2 per query row, then (split) the fp32 partials
  hipStream_t st = (hipStream_t)stream;
  void* ws = nullptr;
  const size_t rows = (size_t)B * Hq * Nq;
  const size_t rows_bytes = (rows * sizeof(float) + 255) / 256 * 256;
  const size_t part = hsplit > 1 ? (size_t)hsplit * B * Hkv * Nkv * D * sizeof(float) : 0;
  const size_t partv = hsplit > 1 ? (size_t)hsplit * B * Hkv * Nkv * Dv * sizeof(float) : 0;
  const size_t partq = (size_t)dq_splits * dq_rows * D * sizeof(float);  // 0 unless split
  hipError_t e = attn_host::workspace_alloc(&ws, 2 * rows_bytes + part + partv + partq, st);
  if (e != hipSuccess || !ws) {
    attn_host::set_last_hip_error((int)e);
    (void)hipGetLastError();
    return ATTN_ENOMEM;
  }
  BwdParams p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)out;
  p.dout = (const uint16_t*)dout;
  p.lse = lse;
  p.delta = (float*)ws;
  p.lse2 = (float*)((char*)ws + rows_bytes);
  p.dkp = hsplit > 1 ? (float*)((char*)ws + 2 * rows_bytes) : nullptr;
  p.dvp = hsplit > 1 ? (float*)((char*)ws + 2 * rows_bytes + part) : nullptr;
  p.hsplit = hsplit;
  p.dq_whole = dq_whole;
  p.dq_splits = dq_splits;
  p.dq_split_len = dq_len;
  p.dq_rows = dq_rows;
  p.dqp = dq_splits > 1 ? (float*)((char*)ws + 2 * rows_bytes + part + partv) : nullptr;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = G;
  p.n_tiles = 0;
  p.total = 0;
  p.coff = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq : 0;
  p.cs = scale * kLog2e;
  p.scale = scale;
  p.mask = (const uint8_t*)m.ptr;
  p.msb = m.sb, p.msh = m.sh, p.msq = m.sq;
  p.mask_mode = m.type;
  const bool cz = causal != 0, bf = dtype == ATTN_BF16;
  e = launch_bwd_d(D, Dv, bf, m.type != ATTN_MASK_NONE, p, cz, st);
  const hipError_t ef = hipFreeAsync(ws, st);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) {
    attn_host::set_last_hip_error((int)e);
    return ATTN_EHIP;
  }
  return ATTN_OK;
}

BwdMask bwd_mask(const void* mask, int mask_type, const long long* mask_stride) {
  BwdMask m;
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

}  // namespace

extern "C" {

int attn_bwd_check(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, const void* dq, const void* dk,
                   const void* dv, int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale,
                   int causal, int dtype) {
  return validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, D, scale,
                      causal, dtype);
}

int attn_bwd(const void* q, const void* k, const void* v, const void* out, const void* dout,
             const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
             int Nkv, int D, float scale, int causal, int dtype, void* stream) {
  return run_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal,
                 dtype, stream, BwdMask());
}

int attn_bwd_masked(const void* q, const void* k, const void* v, const void* out,
                    const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                    int Hq, int Hkv, int Nq, int Nkv, int D, const void* mask, int mask_type,
                    const long long* mask_stride, float scale, int causal, int dtype,
                    void* stream) {
  return run_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, D, scale, causal,
                 dtype, stream, bwd_mask(mask, mask_type, mask_stride));
}

int attn_bwd_masked_check(const void* q, const void* k, const void* v, const void* out,
                          const void* dout, const float* lse, const void* dq, const void* dk,
                          const void* dv, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                          const void* mask, int mask_type, const long long* mask_stride,
                          float scale, int causal, int dtype) {
  const int rc = validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, D,
                              scale, causal, dtype);
  if (rc != ATTN_OK) return rc;
  return validate_bwd_mask(bwd_mask(mask, mask_type, mask_stride), dq, dk, dv, B, Hq, Hkv, Nq,
                           Nkv, D, D);
}

int attn_bwd_dv(const void* q, const void* k, const void* v, const void* out, const void* dout,
                const float* lse, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
                int Nkv, int D, int Dv, const void* mask, int mask_type,
                const long long* mask_stride, float scale, int causal, int dtype, void* stream) {
  return run_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, Dv, scale, causal,
                 dtype, stream, bwd_mask(mask, mask_type, mask_stride));
}

int attn_bwd_dv_check(const void* q, const void* k, const void* v, const void* out,
                      const void* dout, const float* lse, const void* dq, const void* dk,
                      const void* dv, int B, int Hq, int Hkv, int Nq, int Nkv, int D, int Dv,
                      const void* mask, int mask_type, const long long* mask_stride, float scale,
                      int causal, int dtype) {
  const int rc = validate_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, D, Dv,
                              scale, causal, dtype);
  if (rc != ATTN_OK) return rc;
  return validate_bwd_mask(bwd_mask(mask, mask_type, mask_stride), dq, dk, dv, B, Hq, Hkv, Nq,
                           Nkv, D, Dv);
}

}  // extern "C"
