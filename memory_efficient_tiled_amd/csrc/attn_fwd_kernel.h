// attn_fwd_kernel.h -- the attention forward kernels for gfx950 and their
// launch templates.  Each head dimension instantiates them in a translation
// unit of its own (attn_fwd_d<D>.hip); attn_fwd.hip holds the host side.
//
// What is computed: exact softmax attention, O = softmax(scale*Q K^T [causal
// mask]) V, plus the row log-sum-exp.  Q and K rows have D elements, V and O
// rows DV (equal to D except for the (192, 128) pair).  The English noflash-attention post
// (ai-navigate-news.com) tiles it over query chunks and, in its second tier,
// over key tiles with a running max and a running sum ("online softmax",
// section "The DIY approach"), so the Nq x Nkv score matrix never exists.
// That post ran on a gfx906 without matrix cores and used one PyTorch matmul
// per chunk; here one workgroup owns a block of query rows and streams the key
// and value tiles of its KV head through LDS, with both products on the
// CDNA4 matrix cores (v_mfma_f32_32x32x16_{bf16,f16}) and the softmax in fp32
// registers.
//
// Layout of the work inside a wave (64 lanes, 32 query rows per block):
//  * Scores are formed transposed, S^T = K Q^T, with K as the MFMA A operand
//    (read from LDS) and Q^T as the B operand (held in registers for the whole
//    key loop).  In the 32x32 accumulator a lane then holds one query row
//    (column lane%32) and 16 of the block's 32 keys; the other 16 keys of that
//    row are in lane lane^32.  Row max and row sum are therefore in-lane plus
//    one exchange between the two wave halves.
//  * The probabilities are already laid out as the B operand of
//    O^T = V^T P^T, so P never leaves registers.  V^T is the A operand: V stays
//    row-major in LDS and each lane gathers its 8 keys of one column with two
//    transposing 8-byte LDS reads (ds_read_b64_tr_b16).
//  * The output accumulator O^T also has one query row per lane, so the
//    per-row rescale by alpha = 2^(m_old - m_new) is a plain multiply.
//
// Softmax runs in base 2: scores are scaled by scale*log2(e) and exponentiated
// with v_exp_f32; the log-sum-exp is converted back to natural log.
//
// Split-KV: query tiles that cannot keep the 256 compute units busy (all of
// a small grid, or the last partial round of a large one) are divided into
// key ranges; each piece writes an fp32 partial output normalised by its own
// row sum, plus its partial log-sum-exp, and a second kernel merges them with
// weights exp(lse_s - lse).

#ifndef ATTN_FWD_KERNEL_H_
#define ATTN_FWD_KERNEL_H_

#include "attn_common.h"
#include "attn_tiles.h"

#include <type_traits>
#include <utility>

namespace attn_fwd_detail {

using namespace attn_tiles;


// Probabilities are formed against a running reference max m that is only
// raised when a tile would otherwise produce a probability above 2^8: the
// final O / l and lse = m + log2(l) are the same function of the scores for
// any reference, so the result is unchanged up to rounding.  The check is
// done on the in-lane partial row sum (each term is at most the sum), which
// the softmax needs anyway, so no per-tile row max is computed unless a tile
// fails it (and on the first tile, where m is still -inf).
constexpr float kMaxPartialSum = 256.0f;


struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;        // final output (non-split) or unused
  float* lse;         // final LSE (non-split), may be null
  float* opart;       // split: [S][prows][DV] fp32, rows from row0 on
  float* lsepart;     // split: [S][prows]
  int Hq, Nq, Nkv, G, Hkv;
  int n_qtiles, n_splits, split_len;
  int total;          // workgroups of this launch
  int tile0;          // first query tile of this launch's pieces (split) or tiles
  int n_whole;        // split launches: the first n_whole workgroups are whole
                      // tiles 0 .. n_whole - 1 (then come the pieces of tiles
                      // tile0 ..); 0 for a launch of pieces only
  int row0, prows;    // split: output rows [row0, row0 + prows) have partials
  float c;            // |scale| * log2(e)
  uint32_t qsign;     // 0x80008000 flips the sign of Q (negative scale)
  int coff;           // causal: row i sees keys j <= i + coff (0 top-left, Nkv - Nq bottom-right)
  int pos_nq;         // > 0 when the G query heads of a KV head are packed into one
                      // [G * Nq] row range: row r is then position r % pos_nq
                      // (pos_nq = the real Nq) for the causal mask; 0 = not packed
  // Element strides of the batch, head and sequence dimensions (the head
  // dimension is contiguous); row strides fit in 32 bits.
  int64_t qsb, qsh, ksb, ksh, vsb, vsh, osb, osh;
  int qsn, ksn, vsn, osn;
  // Attention mask (MASKED kernels): element strides of batch, query head
  // and query row (keys contiguous); mask_mode ATTN_MASK_BOOL (bytes,
  // nonzero keeps the key) or ATTN_MASK_ADD (16-bit values added to the
  // scaled scores).  Scores are then formed in base-2 units in the mask
  // step (score * cm + bias * log2 e) and c is 1.
  const uint8_t* mask;
  int64_t msb, msh, msq;
  int mask_mode;
  float cm;
};

// Launch the forward kernels of one pair of head dimensions (Q/K, V/O),
// defined one pair per translation unit in attn_fwd_d<D>[v<DV>].hip.  The
// merge of split partials depends on DV only.
template <int D, int DV>
hipError_t launch_fwd_d(const Params& p, int cfg, bool causal, bool split, bool strided,
                        bool masked, bool bf16, hipStream_t st);
template <int D>
hipError_t launch_combine_d(const Params& p, bool strided, bool bf16, hipStream_t st);
template <> hipError_t launch_fwd_d<64, 64>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_fwd_d<80, 80>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_fwd_d<96, 96>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_fwd_d<128, 128>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_fwd_d<256, 256>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_fwd_d<192, 128>(const Params&, int, bool, bool, bool, bool, bool, hipStream_t);
template <> hipError_t launch_combine_d<64>(const Params&, bool, bool, hipStream_t);
template <> hipError_t launch_combine_d<80>(const Params&, bool, bool, hipStream_t);
template <> hipError_t launch_combine_d<96>(const Params&, bool, bool, hipStream_t);
template <> hipError_t launch_combine_d<128>(const Params&, bool, bool, hipStream_t);
template <> hipError_t launch_combine_d<256>(const Params&, bool, bool, hipStream_t);

}  // namespace attn_fwd_detail

namespace {

using namespace attn_fwd_detail;


// One workgroup: NW waves x QB x 32 query rows, all on KV head hq / G,
// looping over BN-key tiles of its key range.  Each K or V operand read from
// LDS feeds QB MFMAs (one per 32-row query block of the wave), so LDS read
// traffic per flop falls as 1 / QB.  K and V tiles go from HBM (mostly L2)
// straight into LDS (two buffers each; three for V with SB), in a swizzled
// row-major layout: 16-byte chunk c of key row r is stored at chunk
// c ^ k_swz(r) (K) or c ^ v_swz(r) (V).
//
// Software pipeline, one barrier per key tile t (scores S_t already in
// registers when the step starts):
//   wait for this wave's copies of K_{t+1}, V_t; barrier
//   start copies of K_{t+2} (into the buffer K_t used) and V_{t+1}
//   S_{t+1} = K_{t+1} Q^T on the matrix cores, interleaved with the softmax
//   of S_t on the vector ALUs (the two are independent)
//   O += P_t V_t
// The barrier also certifies that every wave has finished reading the
// buffers the new copies overwrite (K_t in the previous step's product,
// V_{t-1} in the previous step's P V).
//
// With SB (single-buffered scores) a step is instead: barrier; start copies of
// K_{t+1}, V_{t+1}; S_t = K_t Q^T; softmax of S_t; O += P_t V_t.  The scores
// then need one register tile, not two, and the overlap of matrix and vector
// work comes from the other wave on the SIMD, which runs half a step late
// (see the loop).  QL > 0 keeps the last QL of the DC reduction chunks of
// Q^T in LDS (each wave its own rows, read back in operand order) instead of
// registers.
//
// STRIDED takes the tensors' batch, head and sequence strides from Params;
// otherwise the layouts are contiguous and the strides compile-time values.
//
// The products run over DP = compute_dim(D) columns: D itself, except that
// D = 80 (not a multiple of the 32-column output blocks) is computed as 96
// with the last two 16-byte chunks of every Q, K and V row read as zeros and
// the matching output columns not stored.  The V and O widths (DV) are
// handled the same way, independently of D.
template <int D, int DV, class Tag, bool CAUSAL, int NW, int QB, int BN, int QL, bool SB,
          bool PD, bool SPLIT, bool STRIDED, bool MASKED>
__global__ __launch_bounds__(NW * 64, kWavesPerSimd) void attn_fwd_kernel(Params p) {
  constexpr int DP = compute_dim(D);     // columns of Q K^T and of K's LDS rows
  constexpr int DVP = compute_dim(DV);   // columns of P V and of V's LDS rows
  constexpr int WR = QB * 32;            // query rows per wave
  constexpr int BM = NW * WR;
  constexpr int CPR = DP / 8;            // 16-byte chunks per LDS row of K
  constexpr int CPG = D / 8;             // 16-byte chunks per row of K in memory
  constexpr int CPRV = DVP / 8;          // the same for V
  constexpr int CPGV = DV / 8;
  constexpr int TILE = BN * DP;          // elements of one K tile
  constexpr int TILEV = BN * DVP;        // elements of one V tile
  constexpr int INSTR = BN * CPR / 64;   // 1 KB wave copies per K tile
  constexpr int INSTRV = BN * CPRV / 64;  // and per V tile
  static_assert(INSTR % NW == 0 && INSTRV % NW == 0, "tile copies must split evenly over waves");
  constexpr int IPW = INSTR / NW;
  constexpr int IPWV = INSTRV / NW;
  constexpr int DC = DP / 16;            // reduction chunks of Q K^T
  constexpr int NKB = BN / 32;           // 32-key blocks per tile
  constexpr int NDB = DVP / 32;          // 32-wide output column blocks
  constexpr int NKC = BN / 16;           // reduction chunks of P V
  constexpr int ROWB = D * 2;            // bytes per K row in memory
  constexpr int ROWBV = DV * 2;          // bytes per V row in memory
  constexpr int DCR = DC - QL;          // Q^T chunks held in registers
  static_assert(QL >= 0 && QL < DC, "at least one Q^T chunk stays in registers");
  static_assert(!(SB && PD), "the deferred P V step belongs to the double-buffered pipeline");
  using N = Num<Tag>;

  __shared__ __attribute__((aligned(1024))) uint16_t kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf0[TILEV];
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf1[TILEV];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf2[SB || PD ? TILEV : 8];
  __shared__ __attribute__((aligned(1024))) u32x4 qlds[QL > 0 ? NW * QB * QL * 64 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // A split launch may start with whole tiles, so that its pieces take the
  // slots those tiles free (each part renumbered over its own range).
  int bid, sp = 0;
  bool piece = SPLIT;
  if (SPLIT && (int)blockIdx.x < p.n_whole) {
    piece = false;
    bid = xcd_remap(blockIdx.x, p.n_whole);
  } else if (SPLIT) {
    bid = xcd_remap(blockIdx.x - p.n_whole, p.total - p.n_whole);
    sp = bid % p.n_splits;
    bid = bid / p.n_splits + p.tile0;
  } else if (CAUSAL) {
    bid = longest_first(blockIdx.x, p.n_qtiles, p.total);  // (the launch holds every tile)
  } else {
    bid = xcd_remap(blockIdx.x, p.total) + p.tile0;
  }
  int qt = bid % p.n_qtiles;
  bid /= p.n_qtiles;
  const int hq = bid % p.Hq;
  const int b = bid / p.Hq;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  const int hk = hq / p.G;
  const int q0 = qt * BM;
  const int wq0 = q0 + wave * WR;       // first query row of this wave
  // A wave whose rows all lie past Nq (the ragged last tile, or the short
  // row ranges of decode) computes nothing: it only copies its share of
  // every K/V tile and meets every barrier.
  const bool idle = wq0 >= p.Nq;
  // Causal position of this wave's first row (packed rows: the smallest
  // position any of them can have, 0).
  const int wpos0 = p.pos_nq ? 0 : wq0;

  // A split launch covers one key range per piece; otherwise every key.
  const int kbeg = piece ? sp * p.split_len : 0;
  int kend = piece ? min(p.Nkv, kbeg + p.split_len) : p.Nkv;
  // Causal: keys past the reach of the tile's last position are masked.
  // Packed rows hold positions 0 .. pos_nq - 1 of several heads.
  if (CAUSAL) kend = max(0, min(kend, (p.pos_nq ? min(q0 + BM, p.pos_nq) : q0 + BM) + p.coff));
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;  // LSE / partial row of query 0
  const int64_t kh = (int64_t)p.Nkv * D, vh = (int64_t)p.Nkv * DV;
  const int64_t qh = (int64_t)p.Nq * D, oh = (int64_t)p.Nq * DV;
  const int qsn = STRIDED ? p.qsn : D, ksn = STRIDED ? p.ksn : D;
  const int vsn = STRIDED ? p.vsn : DV, osn = STRIDED ? p.osn : DV;
  const uint16_t* Qg = p.q + (STRIDED ? b * p.qsb + hq * p.qsh : ((int64_t)b * p.Hq + hq) * qh);
  const uint16_t* Kg = p.k + (STRIDED ? b * p.ksb + hk * p.ksh : ((int64_t)b * p.Hkv + hk) * kh);
  const uint16_t* Vg = p.v + (STRIDED ? b * p.vsb + hk * p.vsh : ((int64_t)b * p.Hkv + hk) * vh);

  // Per-lane byte offsets of this wave's copy slots within a tile (the same
  // for every tile) and the LDS slot each copy fills.  Padding chunks (past
  // the row in memory) get an offset beyond any buffer, so they read zero.
  uint32_t koff[IPW], voff[IPWV];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int slot = (wave * IPW + j) * 64 + lane;
    const int row = slot / CPR, pc = slot % CPR;
    const int kch = pc ^ k_swz<DP>(row);
    koff[j] = kch < CPG ? row * ksn * 2 + (kch << 4) : kPadOffset;
  }
#pragma unroll
  for (int j = 0; j < IPWV; ++j) {
    const int slot = (wave * IPWV + j) * 64 + lane;
    const int row = slot / CPRV, pc = slot % CPRV;
    const int vch = pc ^ v_swz<DVP>(row);
    voff[j] = vch < CPGV ? row * vsn * 2 + (vch << 4) : kPadOffset;
  }
  // Copy tile `t` of K or V (rows `sn` elements and `rowb` bytes long,
  // IP copies per wave) into LDS.  The buffer ends with the last key's row,
  // so rows past it (which start at or beyond that end, as a row stride is
  // at least a row) read as zero: their scores are masked to -inf and their
  // V rows are multiplied by exactly 0.
  auto copy_tile = [&](auto ip, int rowb, const uint16_t* base, int sn, int t, uint16_t* dst,
                       const uint32_t* off) {
    constexpr int IP = decltype(ip)::value;
    const int k0 = kbeg + t * BN;
    const int nrows = min(BN, p.Nkv - k0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)k0 * sn), 0, (nrows - 1) * sn * 2 + rowb, kRawBufferFlags);
#pragma unroll
    for (int j = 0; j < IP; ++j) buf2lds16(r, dst + (wave * IP + j) * 512, off[j]);
  };
  auto issue_k = [&](int t, uint16_t* dst) {
    copy_tile(std::integral_constant<int, IPW>{}, ROWB, Kg, ksn, t, dst, koff);
  };
  auto issue_v = [&](int t, uint16_t* dst) {
    copy_tile(std::integral_constant<int, IPWV>{}, ROWBV, Vg, vsn, t, dst, voff);
  };

  // Q^T operands for the whole key loop: chunks below DCR in registers, the
  // rest in this wave's LDS slots (written and read by this wave only).
  u32x4 qf[QB][DCR];
  const int qmine = wave * QB * QL * 64 + lane;  // this lane's slot in qlds
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + qb * 32 + l32;
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < p.Nq && kc * 16 + hl * 8 < D)
        x = *(const u32x4*)(Qg + (size_t)row * qsn + kc * 16 + hl * 8);
      if (kc < DCR)
        qf[qb][kc < DCR ? kc : 0] = x ^ p.qsign;
      else
        qlds[qmine + (qb * QL + (kc - DCR)) * 64] = x ^ p.qsign;
    }
  }
  // The LDS chunks are re-read at every use, from index qi: the caller
  // passes it through an empty asm once per tile, which hides it from the
  // compiler, so the (loop-invariant) reads are not hoisted out of the key
  // loop into registers.
  auto qop = [&](int qb, int kc, int qi) -> u32x4 {
    if (kc < DCR) return qf[qb][kc < DCR ? kc : 0];
    return qlds[qi + (qb * QL + (kc - DCR)) * 64];
  };
  auto qindex = [&]() {
    int qi = qmine;
    if constexpr (QL > 0) asm volatile("" : "+v"(qi));
    return qi;
  };

  // O^T accumulators: block (qb, db) at oacc[qb * NDB + db].
  f32x16 oacc[QB * NDB];
#pragma unroll
  for (int i = 0; i < QB * NDB; ++i) oacc[i] = f32x16{};
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
  }

  // Lane-invariant parts of the V^T operand addresses.
  const int v_g = lane >> 4, v_r = lane & 15;
  const int v_key = 4 * hl + (v_r >> 2);          // key within a 16-key chunk (first half)
  const int v_d = 16 * (v_g & 1) + 4 * (v_r & 3);  // column within a 32-wide block
  const int v_sw = v_swz<DVP>(v_key);             // same for key v_key + 16 kc (+ 8)

  // Scores of a tile: s[qb * NKB + kb] (32 keys x 32 rows); probabilities
  // pf[qb * NKC + kc] (16 keys x 32 rows, the P^T operands).

  // S^T = K Q^T for one tile, accumulated into s (zeroed here).
  auto qk = [&](const uint16_t* ks, f32x16* s) {
    const int qi = qindex();
#pragma unroll
    for (int i = 0; i < QB * NKB; ++i) s[i] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
      u32x4 bq[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) bq[qb] = qop(qb, kc, qi);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + l32;
        const u32x4 a = *(const u32x4*)(ks + row * DP + (((2 * kc + hl) ^ k_swz<DP>(row)) << 3));
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb * NKB + kb] = N::mfma(a, bq[qb], s[qb * NKB + kb]);
      }
    }
  };

  // Causal position of query row r of this launch (packed rows: r % pos_nq).
  auto qpos_of = [&](int r) { return p.pos_nq ? r % p.pos_nq : r; };

  // Keys past the valid range, and (causal) keys after the row, get -inf:
  // only on tiles that straddle the end of the key range or the diagonal.
  // With a mask, every tile first goes through the mask: a boolean mask
  // sets the scores of the keys it removes to -inf (the others stay raw; c
  // scales them in the exponent), an additive one forms base-2 scores
  // s * cm + bias * log2(e) (then c is 1).
  // (Always inlined: the score arrays it takes by pointer must stay in
  // registers.)
  auto mask = [&](int t, f32x16* s) __attribute__((always_inline)) {
    const int k0 = kbeg + t * BN;
    const bool edge = (k0 + BN > kend) || (CAUSAL && k0 + BN - 1 > wpos0 + p.coff);
    if constexpr (!MASKED) {
      if (edge) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
          const int qpos = qpos_of(wq0 + qb * 32 + l32);
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int key0 = k0 + kb * 32 + 8 * g + 4 * hl;
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int key = key0 + i;
                const float v = s[qb * NKB + kb][4 * g + i];
                const bool ok = key < kend && (!CAUSAL || key <= qpos + p.coff);
                s[qb * NKB + kb][4 * g + i] = ok ? v : -INFINITY;
              }
            }
        }
      }
      return;
    } else {
      const bool keep_mode = p.mask_mode == ATTN_MASK_BOOL;
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wq0 + qb * 32 + l32;
        const int64_t off = b * p.msb + hq * p.msh + (int64_t)min(qrow, p.Nq - 1) * p.msq;
        const uint8_t* mrow = p.mask + off * (keep_mode ? 1 : 2);
        if (keep_mode) {
          // A tile in which the mask keeps every key of every row of the wave
          // (most tiles of a key-padding mask) skips the per-score selects:
          // any zero byte among a lane's mask words shows in the usual
          // has-a-zero-byte test, and the wave votes.
          uint32_t w[NKB][4];
          uint32_t zero = 0u;
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              w[kb][g] = mask_keep4(mrow, k0 + kb * 32 + 8 * g + 4 * hl, p.Nkv);
              zero |= (w[kb][g] - 0x01010101u) & ~w[kb][g] & 0x80808080u;
            }
          if (__builtin_amdgcn_ballot_w64(zero != 0u)) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
              for (int g = 0; g < 4; ++g)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                  if (((w[kb][g] >> (8 * i)) & 0xffu) == 0u)
                    s[qb * NKB + kb][4 * g + i] = -INFINITY;
          }
        } else {
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              float bias[4];
              mask_bias4<Tag>(mrow, ATTN_MASK_ADD, k0 + kb * 32 + 8 * g + 4 * hl, p.Nkv, bias);
#pragma unroll
              for (int i = 0; i < 4; ++i)
                s[qb * NKB + kb][4 * g + i] = fmaf(s[qb * NKB + kb][4 * g + i], p.cm, bias[i]);
            }
        }
      }
    }
    if (edge) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qpos = qpos_of(wq0 + qb * 32 + l32);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = k0 + kb * 32 + 8 * g + 4 * hl + i;
              const bool ok = key < kend && (!CAUSAL || key <= qpos + p.coff);
              const float v = s[qb * NKB + kb][4 * g + i];
              s[qb * NKB + kb][4 * g + i] = ok ? v : -INFINITY;
            }
      }
    }
  };

  // Scores of query block qb of one tile -> probabilities against reference
  // max mb, in place; returns the lane-partial row sum.
  // (The four partial sums start from their first terms: an add of 0 is
  // not folded away, since 0 + -0 is +0.)
  auto probs = [&](f32x16* s, int qb, float mb) {
    float rs[4];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[qb * NKB + kb][e] = fast_exp2(fmaf(s[qb * NKB + kb][e], p.c, -mb));
        if (kb == 0 && e < 4)
          rs[e] = s[qb * NKB + kb][e];
        else
          rs[e & 3] += s[qb * NKB + kb][e];
      }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  // Raw scores of tile t again, masked: the slow path of the softmax needs
  // them after the fast path has overwritten them.  With SB, K_t is still in
  // LDS (ks); otherwise its buffer is being refilled and K comes from global
  // memory (rows past the key range read as zero).
  auto rescore = [&](int t, f32x16* s, const uint16_t* ks) {
    if constexpr (SB) {
      qk(ks, s);
      mask(t, s);
      return;
    }
    const int k0 = kbeg + t * BN;
#pragma unroll
    for (int i = 0; i < QB * NKB; ++i) s[i] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key = k0 + kb * 32 + l32;
        u32x4 a = {0u, 0u, 0u, 0u};
        if (key < p.Nkv && kc * 16 + hl * 8 < D)
          a = *(const u32x4*)(Kg + (size_t)key * ksn + kc * 16 + hl * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb * NKB + kb] = N::mfma(a, qop(qb, kc, qmine), s[qb * NKB + kb]);
      }
    }
    mask(t, s);
  };

  // Softmax of tile t, in two parts.  softmax_fast: probabilities against
  // the current references, in place; true if some row's reference is still
  // -inf or a partial sum exceeds the bound.  softmax_finish: in that case
  // recompute the scores, raise the references to the true running max,
  // rescale O and l, and redo; then accumulate l and pack the P^T operands.
  auto softmax_fast = [&](f32x16* s, float* rs) {
    bool bad = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      rs[qb] = probs(s, qb, m[qb]);
      bad = bad || !(m[qb] > -INFINITY) || !(rs[qb] <= kMaxPartialSum);
    }
    return bad;
  };
  auto softmax_finish = [&](int t, f32x16* s, float* rs, bool bad, u32x4* pf,
                            const uint16_t* ks) {
    if (__builtin_amdgcn_ballot_w64(bad)) {
      rescore(t, s, ks);
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb * NKB + kb][e]);
        mx = pair_max(mx);
        const float mc = (mx == -INFINITY) ? -INFINITY : mx * p.c;
        const float mnew = fmaxf(m[qb], mc);
        const float alpha = (m[qb] == -INFINITY) ? 0.f : fast_exp2(m[qb] - mnew);
        m[qb] = mnew;
        l[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[qb * NDB + db] *= alpha;
        rs[qb] = probs(s, qb, (mnew == -INFINITY) ? 0.f : mnew);
      }
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      l[qb] += rs[qb];  // lane-partial: lane l^32 holds the rest
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 y;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            y[w] = N::pack2(s[qb * NKB + kb][8 * hf + 2 * w], s[qb * NKB + kb][8 * hf + 2 * w + 1]);
          pf[qb * NKC + kb * 2 + hf] = y;
        }
    }
  };

  // O^T += V^T P^T; V^T operands come from transposing reads of V.
  auto pv = [&](const uint16_t* vs, const u32x4* pf) {
#pragma unroll
    for (int kc = 0; kc < NKC; ++kc) {
      const int key = kc * 16 + v_key;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const int d = db * 32 + v_d;
        const int off = (((d >> 3) ^ v_sw) << 3) + (d & 7);
        const u32x2 lo = lds_read_tr16(vs + key * DVP + off);
        const u32x2 hi = lds_read_tr16(vs + (key + 8) * DVP + off);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          oacc[qb * NDB + db] = N::mfma(a, pf[qb * NKC + kc], oacc[qb * NDB + db]);
      }
    }
  };

  // One pipeline step for tile t whose scores are in `s`; K_t and V_t sit in
  // (kc, vc), tile t + 1 goes to (kn, vn).  LAST: no tile t + 1.
  auto step = [&](auto last, int t, f32x16* s, f32x16* sn, uint16_t* kc, uint16_t* vc,
                  uint16_t* kn, uint16_t* vn) {
    constexpr bool LAST = decltype(last)::value;
    mask(t, s);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!LAST) {
      if (t + 2 < ntiles) issue_k(t + 2, kc);
      issue_v(t + 1, vn);
      qk(kn, sn);
    }
    float rs[QB];
    const bool bad = softmax_fast(s, rs);
    u32x4 pf[QB * NKC];
    softmax_finish(t, s, rs, bad, pf, nullptr);
    pv(vc, pf);
  };
  using Last = std::integral_constant<bool, true>;
  using More = std::integral_constant<bool, false>;

  // Single-buffered steps.  Waves w and w + NW/2 share a SIMD; the second
  // group runs half a step late: after the barrier of step t it first forms
  // O += P_{t-1} V_{t-1}, then S_t and its softmax, so each wave's vector
  // work overlaps the other's matrix work.  K_t sits in kbuf[t % 2] and V_t
  // in vbuf[t % 3]: the copies of step t (K_{t+1}, V_{t+1}) overwrite K_{t-1}
  // and V_{t-2}, which every wave has finished with once past the barrier.
  // Idle waves (no rows below Nq): the copies and barriers of the loops
  // below, in the same order and into the same buffers, and nothing else.
  // Single-buffered: one barrier per tile, after which K_{t+1}, V_{t+1}
  // go to kbuf[(t+1) % 2], vbuf[(t+1) % 3].  Double-buffered: one barrier
  // after the first tile's copies, then one per tile, after which K_{t+2}
  // goes to kbuf[t % 2] and V_{t+1} to vbuf[(t+1) % 2] (with PD, to
  // vbuf[(t+1) % 3]).
  auto idle_loop = [&]() {
    if (ntiles <= 0) return;
    issue_k(0, kbuf0);
    issue_v(0, vbuf0);
    if constexpr (SB) {
      for (int t = 0; t < ntiles; ++t) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < ntiles) {
          const int v3 = (t + 1) % 3;
          issue_k(t + 1, ((t + 1) & 1) ? kbuf1 : kbuf0);
          issue_v(t + 1, v3 == 0 ? vbuf0 : v3 == 1 ? vbuf1 : vbuf2);
        }
      }
    } else {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (ntiles > 1) issue_k(1, kbuf1);
      for (int t = 0; t < ntiles; ++t) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (t + 1 < ntiles) {
          if (t + 2 < ntiles) issue_k(t + 2, (t & 1) ? kbuf1 : kbuf0);
          if constexpr (PD) {
            const int v3 = (t + 1) % 3;
            issue_v(t + 1, v3 == 0 ? vbuf0 : v3 == 1 ? vbuf1 : vbuf2);
          } else {
            issue_v(t + 1, ((t + 1) & 1) ? vbuf1 : vbuf0);
          }
        }
      }
    }
  };

  f32x16 sa[QB * NKB], sb[SB ? 1 : QB * NKB];
  if (idle) {
    idle_loop();
  } else if constexpr (SB) {
    const bool late = NW >= 2 && wave >= NW / 2;
    u32x4 pf[QB * NKC];
    // One step: K_t in kc, V_t in vc, V_{t-1} in vp; K_{t+1}, V_{t+1} go to
    // kn, vn.  Whole loop iterations pass the buffers as distinct LDS arrays,
    // so the compiler sees that the reads do not touch what the copies fill.
    auto sb_step = [&](int t, uint16_t* kc, uint16_t* vc, uint16_t* vp, uint16_t* kn,
                       uint16_t* vn) {
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (t + 1 < ntiles) {
        issue_k(t + 1, kn);
        issue_v(t + 1, vn);
      }
      if (late && t > 0) pv(vp, pf);
      qk(kc, sa);
      mask(t, sa);
      float rs[QB];
      const bool bad = softmax_fast(sa, rs);
      softmax_finish(t, sa, rs, bad, pf, kc);
      if (!late) pv(vc, pf);
    };
    auto kbufs = [&](int i) { return i ? kbuf1 : kbuf0; };
    auto vbufs = [&](int i) { return i == 0 ? vbuf0 : i == 1 ? vbuf1 : vbuf2; };
    if (ntiles > 0) {
      issue_k(0, kbuf0);
      issue_v(0, vbuf0);
    }
    int t = 0;
    for (; t + 6 <= ntiles; t += 6) {  // K_t in kbuf[t % 2], V_t in vbuf[t % 3]
      sb_step(t, kbuf0, vbuf0, vbuf2, kbuf1, vbuf1);
      sb_step(t + 1, kbuf1, vbuf1, vbuf0, kbuf0, vbuf2);
      sb_step(t + 2, kbuf0, vbuf2, vbuf1, kbuf1, vbuf0);
      sb_step(t + 3, kbuf1, vbuf0, vbuf2, kbuf0, vbuf1);
      sb_step(t + 4, kbuf0, vbuf1, vbuf0, kbuf1, vbuf2);
      sb_step(t + 5, kbuf1, vbuf2, vbuf1, kbuf0, vbuf0);
    }
    for (; t < ntiles; ++t) {
      const int v3 = t % 3;
      sb_step(t, kbufs(t & 1), vbufs(v3), vbufs(v3 == 0 ? 2 : v3 - 1), kbufs((t + 1) & 1),
              vbufs(v3 == 2 ? 0 : v3 + 1));
    }
    if (late && ntiles > 0) pv(vbufs((ntiles - 1) % 3), pf);
  } else if constexpr (PD) {
    // Double-buffered with P V deferred by one step: after the barrier of
    // step t the wave issues O += P_{t-1} V_{t-1} and S_{t+1} = K_{t+1} Q^T
    // on the matrix cores and the softmax of S_t on the vector ALUs, all
    // independent of one another, so the in-order instruction stream can
    // interleave them; only the packing of P_t follows the softmax.  V_{t-1}
    // is still read in step t, so V rotates through three LDS buffers:
    // K_t in kbuf[t % 2], V_t in vbuf[t % 3], S_t in sa (t even) or sb.
    if (ntiles > 0) {
      u32x4 pf[QB * NKC];
      // kc: K_t (refilled with K_{t+2}); kn: K_{t+1}; vp: V_{t-1}; vn: gets V_{t+1}.
      // FIRST: t = 0, no P V of a previous tile (a compile-time flag, so that
      // every later step is one basic block from the barrier to the softmax).
      auto pd_step = [&](auto last, auto first, int t, f32x16* s, f32x16* sn, uint16_t* kc,
                         uint16_t* kn, uint16_t* vp, uint16_t* vn) {
        constexpr bool LAST = decltype(last)::value;
        constexpr bool FIRST = decltype(first)::value;
        mask(t, s);
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (!LAST) {
          if (t + 2 < ntiles) issue_k(t + 2, kc);
          issue_v(t + 1, vn);
        }
        if (!FIRST) pv(vp, pf);
        if (!LAST) qk(kn, sn);
        float rs[QB];
        const bool bad = softmax_fast(s, rs);
        softmax_finish(t, s, rs, bad, pf, nullptr);
      };
      auto vbufs = [&](int i) { return i == 0 ? vbuf0 : i == 1 ? vbuf1 : vbuf2; };
      issue_k(0, kbuf0);
      issue_v(0, vbuf0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (ntiles > 1) issue_k(1, kbuf1);
      qk(kbuf0, sa);
      using First = std::integral_constant<bool, true>;
      using Next = std::integral_constant<bool, false>;
      if (ntiles == 1) {
        pd_step(Last{}, First{}, 0, sa, sb, kbuf0, kbuf1, vbuf2, vbuf1);
      } else {
        pd_step(More{}, First{}, 0, sa, sb, kbuf0, kbuf1, vbuf2, vbuf1);
        int t = 1;
        for (; t + 6 < ntiles; t += 6) {  // six steps, each with a successor
          pd_step(More{}, Next{}, t, sb, sa, kbuf1, kbuf0, vbuf0, vbuf2);
          pd_step(More{}, Next{}, t + 1, sa, sb, kbuf0, kbuf1, vbuf1, vbuf0);
          pd_step(More{}, Next{}, t + 2, sb, sa, kbuf1, kbuf0, vbuf2, vbuf1);
          pd_step(More{}, Next{}, t + 3, sa, sb, kbuf0, kbuf1, vbuf0, vbuf2);
          pd_step(More{}, Next{}, t + 4, sb, sa, kbuf1, kbuf0, vbuf1, vbuf0);
          pd_step(More{}, Next{}, t + 5, sa, sb, kbuf0, kbuf1, vbuf2, vbuf1);
        }
        // t is odd here: K_t in kbuf1, S_t in sb
        for (; t + 2 < ntiles; t += 2) {
          pd_step(More{}, Next{}, t, sb, sa, kbuf1, kbuf0, vbufs((t + 2) % 3), vbufs((t + 1) % 3));
          pd_step(More{}, Next{}, t + 1, sa, sb, kbuf0, kbuf1, vbufs(t % 3), vbufs((t + 2) % 3));
        }
        if (t + 1 < ntiles) {
          pd_step(More{}, Next{}, t, sb, sa, kbuf1, kbuf0, vbufs((t + 2) % 3), vbufs((t + 1) % 3));
          pd_step(Last{}, Next{}, t + 1, sa, sb, kbuf0, kbuf1, vbufs(t % 3), vbufs((t + 2) % 3));
        } else {
          pd_step(Last{}, Next{}, t, sb, sa, kbuf1, kbuf0, vbufs((t + 2) % 3), vbufs((t + 1) % 3));
        }
      }
      pv(vbufs((ntiles - 1) % 3), pf);  // O += P_{last} V_{last}
    }
  } else if (ntiles > 0) {
    issue_k(0, kbuf0);
    issue_v(0, vbuf0);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ntiles > 1) issue_k(1, kbuf1);
    qk(kbuf0, sa);
    int t = 0;
    for (; t + 2 < ntiles; t += 2) {
      step(More{}, t, sa, sb, kbuf0, vbuf0, kbuf1, vbuf1);
      step(More{}, t + 1, sb, sa, kbuf1, vbuf1, kbuf0, vbuf0);
    }
    if (t + 1 < ntiles) {
      step(More{}, t, sa, sb, kbuf0, vbuf0, kbuf1, vbuf1);
      step(Last{}, t + 1, sb, sa, kbuf1, vbuf1, kbuf0, vbuf0);
    } else {
      step(Last{}, t, sa, sb, kbuf0, vbuf0, kbuf1, vbuf1);
    }
  }

  // Epilogue: combine the two lane halves' row sums, normalise, store.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int qrow = wq0 + qb * 32 + l32;
    const float lt = pair_sum(l[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
    if (qrow < p.Nq) {
      if (piece) {
        const size_t prow = (size_t)sp * p.prows + (qrow0 + qrow - p.row0);
        float* dst = p.opart + prow * DV;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = db * 32 + 8 * i + 4 * hl;
            const f32x16& o = oacc[qb * NDB + db];
            f32x4 y = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
            if (DVP == DV || col < DV) *(f32x4*)(dst + col) = y;
          }
        if (hl == 0) p.lsepart[prow] = lse_v;
      } else {
        uint16_t* dst = p.o + (STRIDED ? b * p.osb + hq * p.osh : ((int64_t)b * p.Hq + hq) * oh) +
                        (size_t)qrow * osn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = db * 32 + 8 * i + 4 * hl;
            const f32x16& o = oacc[qb * NDB + db];
            u32x2 y = {N::pack2(o[4 * i] * inv, o[4 * i + 1] * inv),
                       N::pack2(o[4 * i + 2] * inv, o[4 * i + 3] * inv)};
            if (DVP == DV || col < DV) *(u32x2*)(dst + col) = y;
          }
        if (hl == 0 && p.lse) p.lse[qrow0 + qrow] = lse_v;
      }
    }
  }
}

// Merge split-KV partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
// Partial row r belongs to output row row0 + r.
template <int D, class Tag, bool STRIDED>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ lsepart,
                                                           uint16_t* __restrict__ o,
                                                           float* __restrict__ lse, int rows,
                                                           int row0, int n_splits, int Hq, int Nq,
                                                           int64_t osb, int64_t osh, int osn) {
  using N = Num<Tag>;
  constexpr int C4 = D / 4;
  const size_t idx = (size_t)blockIdx.x * 256 + threadIdx.x;
  const size_t row = idx / C4;
  const int c4 = (int)(idx % C4);
  if (row >= (size_t)rows) return;
  float mx = -INFINITY;
  for (int s = 0; s < n_splits; ++s) mx = fmaxf(mx, lsepart[(size_t)s * rows + row]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s = 0; s < n_splits; ++s) {
      const float ls = lsepart[(size_t)s * rows + row];
      const float w = (ls == -INFINITY) ? 0.f : expf(ls - mx);
      wsum += w;
      const f32x4 x = *(const f32x4*)(opart + ((size_t)s * rows + row) * D + c4 * 4);
      acc += w * x;
    }
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  u32x2 y = {N::pack2(acc[0] * inv, acc[1] * inv), N::pack2(acc[2] * inv, acc[3] * inv)};
  const int r = row0 + (int)row;
  size_t at = (size_t)r * D;  // contiguous: output row r
  if (STRIDED) {
    const int i = r % Nq, bh = r / Nq;
    at = (bh / Hq) * osb + (bh % Hq) * osh + (size_t)i * osn;
  }
  *(u32x2*)(o + at + c4 * 4) = y;
  if (c4 == 0 && lse) lse[row0 + row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// The same merge for rows cut into many pieces (decode: a few rows, up to
// 256 pieces each): one workgroup of 1024 threads per output row, so that
// every piece's loads are in flight at once (with few rows the merge is
// bound by load latency).  The threads first find the largest piece LSE
// together; then groups of GS threads take every NG-th piece, each thread
// 4 columns, and the groups' sums meet in LDS.
constexpr int kRowMergeThreads = 1024;

template <int D, class Tag, bool STRIDED>
__global__ __launch_bounds__(kRowMergeThreads) void attn_combine_rows_kernel(
    const float* __restrict__ opart, const float* __restrict__ lsepart, uint16_t* __restrict__ o,
    float* __restrict__ lse, int rows, int row0, int n_splits, int Hq, int Nq, int64_t osb,
    int64_t osh, int osn) {
  using N = Num<Tag>;
  constexpr int T = kRowMergeThreads;
  constexpr int C4 = D / 4;
  constexpr int GS = C4 <= 32 ? 32 : 64;
  constexpr int NG = T / GS;
  __shared__ float red[T / 64];
  __shared__ f32x4 part[NG][GS];
  __shared__ float wpart[NG];
  const int row = blockIdx.x;  // grid = rows
  const int t = threadIdx.x;
  const int g = t / GS, c4 = t % GS;
  // The first round of eight pieces per group is loaded before the largest
  // LSE is known (the loads do not depend on it), so the two round trips to
  // memory overlap (few rows: the merge is bound by load latency).
  constexpr int U = 8;
  float ls[U];
  f32x4 x[U];
  auto load_round = [&](int s0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int s = s0 + u * NG;
      ls[u] = s < n_splits ? lsepart[(size_t)s * rows + row] : -INFINITY;
      x[u] = (s < n_splits && c4 < C4)
                 ? *(const f32x4*)(opart + ((size_t)s * rows + row) * D + c4 * 4)
                 : f32x4{0.f, 0.f, 0.f, 0.f};
    }
  };
  load_round(g);
  float mx = -INFINITY;
  for (int s = t; s < n_splits; s += T) mx = fmaxf(mx, lsepart[(size_t)s * rows + row]);
  mx = wave_max(mx);  // then the 16 waves' maxima through LDS
  if ((t & 63) == 0) red[t >> 6] = mx;
  __syncthreads();
  mx = red[0];
#pragma unroll
  for (int w = 1; w < T / 64; ++w) mx = fmaxf(mx, red[w]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -INFINITY) {
    for (int s0 = g;;) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float w = (ls[u] == -INFINITY) ? 0.f : expf(ls[u] - mx);
        wsum += w;
        acc += w * x[u];
      }
      s0 += U * NG;
      if (s0 >= n_splits) break;
      load_round(s0);
    }
  }
  part[g][c4] = acc;
  if (c4 == 0) wpart[g] = wsum;
  __syncthreads();
  if (t >= C4) return;
  f32x4 a = part[0][t];
  float ws = wpart[0];
#pragma unroll
  for (int gg = 1; gg < NG; ++gg) {
    a += part[gg][t];
    ws += wpart[gg];
  }
  const float inv = ws > 0.f ? 1.f / ws : 0.f;
  u32x2 y = {N::pack2(a[0] * inv, a[1] * inv), N::pack2(a[2] * inv, a[3] * inv)};
  const int r = row0 + row;
  size_t at = (size_t)r * D;  // contiguous: output row r
  if (STRIDED) {
    const int i = r % Nq, bh = r / Nq;
    at = (bh / Hq) * osb + (bh % Hq) * osh + (size_t)i * osn;
  }
  *(u32x2*)(o + at + t * 4) = y;
  if (t == 0 && lse) lse[row0 + row] = ws > 0.f ? mx + logf(ws) : -INFINITY;
}

// Pieces per row above which the merge takes a workgroup per row.
constexpr int kRowMergeSplits = 16;

// Masked launches always take the strided kernels (the mask has strides
// of its own) and only the narrow tiles.
template <int D, int DV, int CFG, class Tag, bool CAUSAL, bool SPLIT, bool MASKED>
hipError_t launch_main(const Params& p, bool strided, hipStream_t stream) {
  constexpr TileCfg c = kCfgs[CFG];
  if (MASKED)
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, DV, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, c.PD && !MASKED, SPLIT, true, MASKED>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  else if (strided)
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, DV, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, c.PD, SPLIT, true, false>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, DV, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, c.PD, SPLIT, false, false>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int DV, int CFG, class Tag, bool MASKED>
hipError_t dispatch(const Params& p, bool causal, bool split, bool strided, hipStream_t st) {
  if (causal)
    return split ? launch_main<D, DV, CFG, Tag, true, true, MASKED>(p, strided, st)
                 : launch_main<D, DV, CFG, Tag, true, false, MASKED>(p, strided, st);
  return split ? launch_main<D, DV, CFG, Tag, false, true, MASKED>(p, strided, st)
               : launch_main<D, DV, CFG, Tag, false, false, MASKED>(p, strided, st);
}

// The wide tiles are only selected without a causal mask.
template <int D, int DV, class Tag>
hipError_t dispatch_d(const Params& p, int cfg, bool causal, bool split, bool strided,
                      bool masked, hipStream_t st) {
  constexpr int kNarrow = D == 192             ? kCfgD192
                          : D == 256           ? kCfgD256
                          : D == 96 || D == 80 ? kCfgD96
                          : D == 128           ? kCfgD128Narrow
                                               : kCfgD64Narrow;
  constexpr int kWide = D == 192             ? kCfgD192
                        : D == 256           ? kCfgD256
                        : D == 96 || D == 80 ? kCfgD96
                        : D == 128           ? kCfgD128Wide
                                             : kCfgD64Wide;
  constexpr int kMasked = D == 128 ? kCfgD128Masked : kNarrow;
  if (masked) return dispatch<D, DV, kMasked, Tag, true>(p, causal, split, true, st);
  if constexpr (D == 128 && DV == 128)
    if (cfg == kCfgD128Decode) return dispatch<D, DV, kCfgD128Decode, Tag, false>(p, causal, split, strided, st);
  if (kWide != kNarrow && cfg == kWide && !causal)
    return split ? launch_main<D, DV, kWide, Tag, false, true, false>(p, strided, st)
                 : launch_main<D, DV, kWide, Tag, false, false, false>(p, strided, st);
  return dispatch<D, DV, kNarrow, Tag, false>(p, causal, split, strided, st);
}

template <int D, class Tag>
hipError_t launch_combine(const Params& p, bool strided, hipStream_t st) {
  if (p.n_splits > kRowMergeSplits) {
    if (strided)
      hipLaunchKernelGGL((attn_combine_rows_kernel<D, Tag, true>), dim3(p.prows),
                         dim3(kRowMergeThreads), 0, st, p.opart, p.lsepart, p.o, p.lse, p.prows,
                         p.row0, p.n_splits, p.Hq, p.Nq, p.osb, p.osh, p.osn);
    else
      hipLaunchKernelGGL((attn_combine_rows_kernel<D, Tag, false>), dim3(p.prows),
                         dim3(kRowMergeThreads), 0, st, p.opart, p.lsepart, p.o, p.lse, p.prows,
                         p.row0, p.n_splits, p.Hq, p.Nq, p.osb, p.osh, p.osn);
    return hipGetLastError();
  }
  const size_t threads = (size_t)p.prows * (D / 4);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  if (strided)
    hipLaunchKernelGGL((attn_combine_kernel<D, Tag, true>), dim3(blocks), dim3(256), 0, st,
                       p.opart, p.lsepart, p.o, p.lse, p.prows, p.row0, p.n_splits, p.Hq, p.Nq,
                       p.osb, p.osh, p.osn);
  else
    hipLaunchKernelGGL((attn_combine_kernel<D, Tag, false>), dim3(blocks), dim3(256), 0, st,
                       p.opart, p.lsepart, p.o, p.lse, p.prows, p.row0, p.n_splits, p.Hq, p.Nq,
                       p.osb, p.osh, p.osn);
  return hipGetLastError();
}

}  // namespace

#endif  // ATTN_FWD_KERNEL_H_
