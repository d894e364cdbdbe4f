// attn_fwd.hip -- fused, tiled, online-softmax attention forward for gfx950.
//
// What is computed: exact softmax attention, O = softmax(scale*Q K^T [causal
// mask]) V, plus the row log-sum-exp.  The English noflash-attention post
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

#include "attn_common.h"

#include <mutex>
#include <type_traits>
#include <utility>

namespace {

// Probabilities are formed against a running reference max m that is only
// raised when a tile would otherwise produce a probability above 2^8: the
// final O / l and lse = m + log2(l) are the same function of the scores for
// any reference, so the result is unchanged up to rounding.  The check is
// done on the in-lane partial row sum (each term is at most the sum), which
// the softmax needs anyway, so no per-tile row max is computed unless a tile
// fails it (and on the first tile, where m is still -inf).
constexpr float kMaxPartialSum = 256.0f;

// Columns the products run over for head dimension D (see attn_fwd_kernel).
constexpr int compute_dim(int D) { return D == 80 ? 96 : D; }

// A buffer offset past every tile's buffer size: such a copy reads zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;        // final output (non-split) or unused
  float* lse;         // final LSE (non-split), may be null
  float* opart;       // split: [S][prows][D] fp32, rows from row0 on
  float* lsepart;     // split: [S][prows]
  int Hq, Nq, Nkv, G, Hkv;
  int n_qtiles, n_splits, split_len;
  int total;          // workgroups of this launch
  int tile0;          // first query tile of this launch
  int row0, prows;    // split: output rows [row0, row0 + prows) have partials
  float c;            // |scale| * log2(e)
  uint32_t qsign;     // 0x80008000 flips the sign of Q (negative scale)
  int coff;           // causal: row i sees keys j <= i + coff (0 top-left, Nkv - Nq bottom-right)
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
// the matching output columns not stored.
template <int D, class Tag, bool CAUSAL, int NW, int QB, int BN, int QL, bool SB, bool SPLIT,
          bool STRIDED, bool MASKED>
__global__ __launch_bounds__(NW * 64, kWavesPerSimd) void attn_fwd_kernel(Params p) {
  constexpr int DP = compute_dim(D);    // columns of the products and LDS rows
  constexpr int WR = QB * 32;           // query rows per wave
  constexpr int BM = NW * WR;
  constexpr int CPR = DP / 8;           // 16-byte chunks per LDS row
  constexpr int CPG = D / 8;            // 16-byte chunks per row in memory
  constexpr int TILE = BN * DP;         // elements of one K (or V) tile
  constexpr int INSTR = BN * CPR / 64;  // 1 KB wave copies per tile
  static_assert(INSTR % NW == 0, "tile copies must split evenly over waves");
  constexpr int IPW = INSTR / NW;
  constexpr int DC = DP / 16;           // reduction chunks of Q K^T
  constexpr int NKB = BN / 32;          // 32-key blocks per tile
  constexpr int NDB = DP / 32;          // 32-wide output column blocks
  constexpr int NKC = BN / 16;          // reduction chunks of P V
  constexpr int ROWB = D * 2;           // bytes per K/V row in memory
  constexpr int DCR = DC - QL;          // Q^T chunks held in registers
  static_assert(QL >= 0 && QL < DC, "at least one Q^T chunk stays in registers");
  using N = Num<Tag>;

  __shared__ __attribute__((aligned(1024))) uint16_t kbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf0[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t kbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf1[TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t vbuf2[SB ? TILE : 8];
  __shared__ __attribute__((aligned(1024))) u32x4 qlds[QL > 0 ? NW * QB * QL * 64 : 1];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: keeps LDS bases scalar
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int bid = xcd_remap(blockIdx.x, p.total);
  int sp = 0;
  if (SPLIT) {
    sp = bid % p.n_splits;
    bid /= p.n_splits;
  }
  bid += p.tile0;
  int qt = bid % p.n_qtiles;
  bid /= p.n_qtiles;
  const int hq = bid % p.Hq;
  const int b = bid / p.Hq;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  const int hk = hq / p.G;
  const int q0 = qt * BM;
  const int wq0 = q0 + wave * WR;       // first query row of this wave

  // A split launch covers one key range per piece; otherwise every key.
  const int kbeg = SPLIT ? sp * p.split_len : 0;
  int kend = SPLIT ? min(p.Nkv, kbeg + p.split_len) : p.Nkv;
  if (CAUSAL) kend = max(0, min(kend, q0 + BM + p.coff));  // keys past the last row's are masked
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;  // LSE / partial row of query 0
  const int64_t kvh = (int64_t)p.Nkv * D, qh = (int64_t)p.Nq * D;
  const int qsn = STRIDED ? p.qsn : D, ksn = STRIDED ? p.ksn : D;
  const int vsn = STRIDED ? p.vsn : D, osn = STRIDED ? p.osn : D;
  const uint16_t* Qg = p.q + (STRIDED ? b * p.qsb + hq * p.qsh : ((int64_t)b * p.Hq + hq) * qh);
  const uint16_t* Kg = p.k + (STRIDED ? b * p.ksb + hk * p.ksh : ((int64_t)b * p.Hkv + hk) * kvh);
  const uint16_t* Vg = p.v + (STRIDED ? b * p.vsb + hk * p.vsh : ((int64_t)b * p.Hkv + hk) * kvh);

  // Per-lane byte offsets of this wave's copy slots within a tile (the same
  // for every tile) and the LDS slot each copy fills.  Padding chunks (past
  // the row in memory) get an offset beyond any buffer, so they read zero.
  uint32_t koff[IPW], voff[IPW];
#pragma unroll
  for (int j = 0; j < IPW; ++j) {
    const int slot = (wave * IPW + j) * 64 + lane;
    const int row = slot / CPR, pc = slot % CPR;
    const int kch = pc ^ k_swz<DP>(row), vch = pc ^ v_swz<DP>(row);
    koff[j] = kch < CPG ? row * ksn * 2 + (kch << 4) : kPadOffset;
    voff[j] = vch < CPG ? row * vsn * 2 + (vch << 4) : kPadOffset;
  }
  // Copy tile `t` of K (or V, rows `sn` elements apart) into LDS.  The
  // buffer ends with the last key's row, so rows past it (which start at or
  // beyond that end, as sn >= D) read as zero: their scores are masked to
  // -inf and their V rows are multiplied by exactly 0.
  auto issue = [&](const uint16_t* base, int sn, int t, uint16_t* dst, const uint32_t* off) {
    const int k0 = kbeg + t * BN;
    const int nrows = min(BN, p.Nkv - k0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(base + (size_t)k0 * sn), 0, (nrows - 1) * sn * 2 + ROWB, kRawBufferFlags);
#pragma unroll
    for (int j = 0; j < IPW; ++j) buf2lds16(r, dst + (wave * IPW + j) * 512, off[j]);
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
  const int v_sw = v_swz<DP>(v_key);              // same for key v_key + 16 kc (+ 8)

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

  // Four consecutive mask values of one row as base-2 biases (keys from
  // key0; those past the key range are not read).
  auto mask_bias4 = [&](const uint8_t* mrow, int key0, float* bias) {
    if (p.mask_mode == ATTN_MASK_BOOL) {
      uint32_t w = 0;
      if (key0 + 3 < p.Nkv) {
        w = *(const uint32_t*)(mrow + key0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + i < p.Nkv) w |= (uint32_t)mrow[key0 + i] << (8 * i);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) bias[i] = ((w >> (8 * i)) & 0xffu) ? 0.f : -INFINITY;
    } else {
      const uint16_t* m16 = (const uint16_t*)mrow;
      u32x2 w = {0u, 0u};
      if (key0 + 3 < p.Nkv) {
        w = *(const u32x2*)(m16 + key0);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (key0 + i < p.Nkv) w[i >> 1] |= (uint32_t)m16[key0 + i] << (16 * (i & 1));
      }
      bias[0] = lo_f32<Tag>(w[0]) * kLog2e;
      bias[1] = hi_f32<Tag>(w[0]) * kLog2e;
      bias[2] = lo_f32<Tag>(w[1]) * kLog2e;
      bias[3] = hi_f32<Tag>(w[1]) * kLog2e;
    }
  };

  // Keys past the valid range, and (causal) keys after the row, get -inf.
  // Only tiles that straddle the end of the key range or the diagonal; with
  // a mask, every tile (scores are scaled and biased here).
  auto mask = [&](int t, f32x16* s) {
    const int k0 = kbeg + t * BN;
    const bool need = MASKED || (k0 + BN > kend) || (CAUSAL && k0 + BN - 1 > wq0 + p.coff);
    if (need) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int qrow = wq0 + qb * 32 + l32;
        const uint8_t* mrow = nullptr;
        if constexpr (MASKED) {
          const int64_t off = b * p.msb + hq * p.msh + (int64_t)min(qrow, p.Nq - 1) * p.msq;
          mrow = p.mask + off * (p.mask_mode == ATTN_MASK_BOOL ? 1 : 2);
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int key0 = k0 + kb * 32 + 8 * g + 4 * hl;
            float bias[4] = {0.f, 0.f, 0.f, 0.f};
            if constexpr (MASKED) mask_bias4(mrow, key0, bias);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int key = key0 + i;
              float v = s[qb * NKB + kb][4 * g + i];
              if constexpr (MASKED) v = fmaf(v, p.cm, bias[i]);
              const bool ok = key < kend && (!CAUSAL || key <= qrow + p.coff);
              s[qb * NKB + kb][4 * g + i] = ok ? v : -INFINITY;
            }
          }
      }
    }
  };

  // Scores of query block qb of one tile -> probabilities against reference
  // max mb, in place; returns the lane-partial row sum.
  auto probs = [&](f32x16* s, int qb, float mb) {
    float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[qb * NKB + kb][e] = fast_exp2(fmaf(s[qb * NKB + kb][e], p.c, -mb));
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
        const u32x2 lo = lds_read_tr16(vs + key * DP + off);
        const u32x2 hi = lds_read_tr16(vs + (key + 8) * DP + off);
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
      if (t + 2 < ntiles) issue(Kg, ksn, t + 2, kc, koff);
      issue(Vg, vsn, t + 1, vn, voff);
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
  f32x16 sa[QB * NKB], sb[SB ? 1 : QB * NKB];
  if constexpr (SB) {
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
        issue(Kg, ksn, t + 1, kn, koff);
        issue(Vg, vsn, t + 1, vn, voff);
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
      issue(Kg, ksn, 0, kbuf0, koff);
      issue(Vg, vsn, 0, vbuf0, voff);
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
  } else if (ntiles > 0) {
    issue(Kg, ksn, 0, kbuf0, koff);
    issue(Vg, vsn, 0, vbuf0, voff);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (ntiles > 1) issue(Kg, ksn, 1, kbuf1, koff);
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
      if (SPLIT) {
        const size_t prow = (size_t)sp * p.prows + (qrow0 + qrow - p.row0);
        float* dst = p.opart + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = db * 32 + 8 * i + 4 * hl;
            const f32x16& o = oacc[qb * NDB + db];
            f32x4 y = {o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
            if (DP == D || col < D) *(f32x4*)(dst + col) = y;
          }
        if (hl == 0) p.lsepart[prow] = lse_v;
      } else {
        uint16_t* dst = p.o + (STRIDED ? b * p.osb + hq * p.osh : ((int64_t)b * p.Hq + hq) * qh) +
                        (size_t)qrow * osn;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int col = db * 32 + 8 * i + 4 * hl;
            const f32x16& o = oacc[qb * NDB + db];
            u32x2 y = {N::pack2(o[4 * i] * inv, o[4 * i + 1] * inv),
                       N::pack2(o[4 * i + 2] * inv, o[4 * i + 3] * inv)};
            if (DP == D || col < D) *(u32x2*)(dst + col) = y;
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

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

// Tile table: waves per workgroup, 32-row query blocks per wave, keys per
// tile, Q^T chunks kept in LDS, pipeline.  Every kernel runs two waves per
// SIMD (8 per CU), so a CU holds 8 / NW workgroups.  At D = 128 the
// workgroup has 8 waves, so each K/V tile copied into LDS serves 256 or 512
// query rows.  64 rows per wave halve the LDS and L2 traffic per flop; at
// D = 128 that needs the single-buffered pipeline and part of Q^T in LDS to
// fit the registers.  The wide tiles pay when they still give every slot of
// the device a workgroup and no causal diagonal is wasted; otherwise the
// 32-row waves are faster.  At D = 256 a wave's 32 rows of O take 128
// registers, so there is one tile: 32-row waves, 32-key tiles, the
// single-buffered pipeline and half of Q^T (8 of 16 chunks) in LDS.  At
// D = 96 (12 chunks per row) the copies split evenly over 4 waves with
// 64-key tiles: the D = 64 narrow tile.  D = 80 runs the D = 96 tile with
// two zero chunks per row.
struct TileCfg {
  int NW, QB, BN, QL;
  bool SB;
  constexpr int BM() const { return NW * QB * 32; }
  constexpr int resident_per_cu() const { return 4 * kWavesPerSimd / NW; }
};
enum {
  kCfgD64Narrow = 0,
  kCfgD64Wide = 1,
  kCfgD128Narrow = 2,
  kCfgD128Wide = 3,
  kCfgD256 = 4,
  kCfgD96 = 5
};
constexpr TileCfg kCfgs[6] = {{4, 1, 64, 0, false},
                              {4, 2, 32, 0, false},
                              {8, 1, 64, 0, false},
                              {8, 2, 32, 3, true},
                              {8, 1, 32, 8, true},
                              {4, 1, 64, 0, false}};

// The wide tiles of each head dimension are used without a causal mask when
// they still fill every slot of the device at least once.
int select_cfg(int B, int Hq, int Nq, int D, int causal, int num_cus) {
  if (D == 256) return kCfgD256;
  if (D == 96 || D == 80) return kCfgD96;
  const int narrow = D == 128 ? kCfgD128Narrow : kCfgD64Narrow;
  const int wide = D == 128 ? kCfgD128Wide : kCfgD64Wide;
  const TileCfg& w = kCfgs[wide];
  const long long wide_wgs = (long long)B * Hq * ((Nq + w.BM() - 1) / w.BM());
  const long long slots = (long long)w.resident_per_cu() * (num_cus > 0 ? num_cus : 256);
  return (!causal && wide_wgs >= slots) ? wide : narrow;
}

thread_local int g_last_hip_error = 0;

bool head_dim_ok(int D) { return D == 64 || D == 80 || D == 96 || D == 128 || D == 256; }

struct DeviceInfo {
  bool init = false;
  bool gfx950 = false;
  int cus = 0;
};
std::mutex g_dev_mu;
DeviceInfo g_dev[64];

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

// Element strides of one tensor's batch, head and sequence dimensions; the
// head dimension (D) is contiguous.
struct Strides {
  int64_t b, h, n;
};
struct Layout {
  Strides q, k, v, o;
};

Layout contiguous_layout(int Hq, int Hkv, int Nq, int Nkv, int D) {
  const Strides qs{(int64_t)Hq * Nq * D, (int64_t)Nq * D, D};
  const Strides ks{(int64_t)Hkv * Nkv * D, (int64_t)Nkv * D, D};
  return Layout{qs, ks, ks, qs};
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
             int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
             int dtype, const Layout& L, const MaskArgs& M = MaskArgs()) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dim_ok(D)) return ATTN_EINVAL;
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
  if (!strides_ok(L.q, D) || !strides_ok(L.k, D) || !strides_ok(L.v, D) || !strides_ok(L.o, D))
    return ATTN_EINVAL;
  if (!dense_enough(L.o, B, Hq, Nq, D)) return ATTN_EINVAL;
  const __int128 qb = extent_bytes(L.q, B, Hq, Nq, D), ob = extent_bytes(L.o, B, Hq, Nq, D);
  const __int128 kb = extent_bytes(L.k, B, Hkv, Nkv, D), vb = extent_bytes(L.v, B, Hkv, Nkv, D);
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
  int D;
  int n_qtiles;
  int splits;
  int split_len;
  long long tiles;
  long long first_split;
  long long row0, rows;
  size_t workspace_bytes() const {
    return splits > 1 ? (size_t)splits * (size_t)(rows - row0) * (D + 1) * sizeof(float) : 0;
  }
};

// Cost model for cutting `rem` equal tiles of `ktiles` key steps into s
// pieces on `slots` workgroup slots, in key steps of one workgroup: the
// pieces run in ceil(s * rem / slots) rounds, each piece spends about
// kPieceFillSteps steps filling its pipeline and writing fp32 partials, and
// the merge streams ~8 (D + 1) bytes per row and piece through HBM, about
// kMergeStepsPerPiece steps of the whole chip per tile and piece (a 64-key
// step of a 256-row tile is ~8 MFLOP, ~2 us on one CU).
constexpr double kPieceFillSteps = 2.0;
constexpr double kMergeStepsPerPiece = 0.03;
constexpr int kMaxSplits = 64;
constexpr int kMinStepsPerPiece = 8;

int balanced_splits(long long rem, long long slots, int ktiles) {
  int best = 1;
  double best_cost = (double)((rem + slots - 1) / slots) * ktiles;
  const int smax = std::min(kMaxSplits, ktiles / kMinStepsPerPiece);
  for (int s = 2; s <= smax; ++s) {
    const int steps = (ktiles + s - 1) / s;
    const double rounds = (double)((s * rem + slots - 1) / slots);
    const double cost = rounds * (steps + kPieceFillSteps) + kMergeStepsPerPiece * s * rem;
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
Plan make_plan(int B, int Hq, int Nq, int Nkv, int D, int causal, int num_splits, int num_cus,
               bool masked = false) {
  Plan pl;
  pl.cfg = select_cfg(B, Hq, Nq, D, causal || masked, num_cus);
  pl.D = D;
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
    S = rem ? balanced_splits(rem, slots, ktiles) : 1;
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

// Masked launches always take the strided kernels (the mask has strides
// of its own) and only the narrow tiles.
template <int D, int CFG, class Tag, bool CAUSAL, bool SPLIT, bool MASKED>
hipError_t launch_main(const Params& p, bool strided, hipStream_t stream) {
  constexpr TileCfg c = kCfgs[CFG];
  if (MASKED)
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, SPLIT, true, MASKED>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  else if (strided)
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, SPLIT, true, false>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(
        (attn_fwd_kernel<D, Tag, CAUSAL, c.NW, c.QB, c.BN, c.QL, c.SB, SPLIT, false, false>),
        dim3(p.total), dim3(c.NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, int CFG, class Tag, bool MASKED>
hipError_t dispatch(const Params& p, bool causal, bool split, bool strided, hipStream_t st) {
  if (causal)
    return split ? launch_main<D, CFG, Tag, true, true, MASKED>(p, strided, st)
                 : launch_main<D, CFG, Tag, true, false, MASKED>(p, strided, st);
  return split ? launch_main<D, CFG, Tag, false, true, MASKED>(p, strided, st)
               : launch_main<D, CFG, Tag, false, false, MASKED>(p, strided, st);
}

// The wide tiles are only selected without a causal mask.
template <int D, class Tag>
hipError_t dispatch_d(const Params& p, int cfg, bool causal, bool split, bool strided,
                      bool masked, hipStream_t st) {
  constexpr int kNarrow = D == 256 ? kCfgD256
                          : D == 96 || D == 80 ? kCfgD96
                          : D == 128           ? kCfgD128Narrow
                                               : kCfgD64Narrow;
  constexpr int kWide = D == 256 ? kCfgD256
                        : D == 96 || D == 80 ? kCfgD96
                        : D == 128           ? kCfgD128Wide
                                             : kCfgD64Wide;
  if (masked) return dispatch<D, kNarrow, Tag, true>(p, causal, split, true, st);
  if (cfg == kWide && !causal)
    return split ? launch_main<D, kWide, Tag, false, true, false>(p, strided, st)
                 : launch_main<D, kWide, Tag, false, false, false>(p, strided, st);
  return dispatch<D, kNarrow, Tag, false>(p, causal, split, strided, st);
}

template <int D, class Tag>
hipError_t launch_combine(const Params& p, bool strided, hipStream_t st) {
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

int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
        int Nq, int Nkv, int D, const Layout& L, float scale, int causal, int dtype,
        int num_splits, hipStream_t stream, const MaskArgs& M = MaskArgs()) {
  int rc = validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype, L, M);
  const bool masked = M.type != ATTN_MASK_NONE;
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_EINVAL;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != ATTN_OK) return rc;

  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, causal, num_splits, di.cus, masked);
  const long long split_wgs = (pl.tiles - pl.first_split) * pl.splits;
  if (pl.first_split > INT32_MAX || split_wgs > INT32_MAX) return ATTN_EINVAL;

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  p.qsb = L.q.b, p.qsh = L.q.h, p.qsn = (int)L.q.n;
  p.ksb = L.k.b, p.ksh = L.k.h, p.ksn = (int)L.k.n;
  p.vsb = L.v.b, p.vsh = L.v.h, p.vsn = (int)L.v.n;
  p.osb = L.o.b, p.osh = L.o.h, p.osn = (int)L.o.n;
  p.lse = lse;
  p.opart = nullptr;
  p.lsepart = nullptr;
  p.Hq = Hq;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = Hq / Hkv;
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
  p.coff = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq : 0;
  p.mask = (const uint8_t*)M.ptr;
  p.msb = M.sb, p.msh = M.sh, p.msq = M.sq;
  p.mask_mode = M.type;
  p.cm = p.c;
  if (masked) p.c = 1.f;  // the mask step forms base-2 scores

  void* ws = nullptr;
  if (split_wgs > 0) {
    hipError_t e = hipMallocAsync(&ws, pl.workspace_bytes(), stream);
    if (e != hipSuccess || !ws) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_ENOMEM;
    }
    p.opart = (float*)ws;
    p.lsepart = p.opart + (size_t)pl.splits * p.prows * D;
  }

  const bool cz = causal != 0;
  const Layout C = contiguous_layout(Hq, Hkv, Nq, Nkv, D);
  auto same = [](const Strides& a, const Strides& b) { return a.b == b.b && a.h == b.h && a.n == b.n; };
  const bool strided = !(same(L.q, C.q) && same(L.k, C.k) && same(L.v, C.v) && same(L.o, C.o));
  auto launch = [&](bool split) {
    if (D == 64)
      return dtype == ATTN_BF16 ? dispatch_d<64, TagBF16>(p, pl.cfg, cz, split, strided, masked, stream)
                                : dispatch_d<64, TagF16>(p, pl.cfg, cz, split, strided, masked, stream);
    if (D == 256)
      return dtype == ATTN_BF16 ? dispatch_d<256, TagBF16>(p, pl.cfg, cz, split, strided, masked, stream)
                                : dispatch_d<256, TagF16>(p, pl.cfg, cz, split, strided, masked, stream);
    if (D == 96)
      return dtype == ATTN_BF16 ? dispatch_d<96, TagBF16>(p, pl.cfg, cz, split, strided, masked, stream)
                                : dispatch_d<96, TagF16>(p, pl.cfg, cz, split, strided, masked, stream);
    if (D == 80)
      return dtype == ATTN_BF16 ? dispatch_d<80, TagBF16>(p, pl.cfg, cz, split, strided, masked, stream)
                                : dispatch_d<80, TagF16>(p, pl.cfg, cz, split, strided, masked, stream);
    return dtype == ATTN_BF16 ? dispatch_d<128, TagBF16>(p, pl.cfg, cz, split, strided, masked, stream)
                              : dispatch_d<128, TagF16>(p, pl.cfg, cz, split, strided, masked, stream);
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
      if (D == 64)
        e = dtype == ATTN_BF16 ? launch_combine<64, TagBF16>(p, strided, stream)
                               : launch_combine<64, TagF16>(p, strided, stream);
      else if (D == 256)
        e = dtype == ATTN_BF16 ? launch_combine<256, TagBF16>(p, strided, stream)
                               : launch_combine<256, TagF16>(p, strided, stream);
      else if (D == 96)
        e = dtype == ATTN_BF16 ? launch_combine<96, TagBF16>(p, strided, stream)
                               : launch_combine<96, TagF16>(p, strided, stream);
      else if (D == 80)
        e = dtype == ATTN_BF16 ? launch_combine<80, TagBF16>(p, strided, stream)
                               : launch_combine<80, TagF16>(p, strided, stream);
      else
        e = dtype == ATTN_BF16 ? launch_combine<128, TagBF16>(p, strided, stream)
                               : launch_combine<128, TagF16>(p, strided, stream);
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
}  // namespace attn_host

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, contiguous_layout(Hq, Hkv, Nq, Nkv, D),
             scale, causal, dtype, 0, (hipStream_t)stream);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                   int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, contiguous_layout(Hq, Hkv, Nq, Nkv, D),
             scale, causal, dtype, num_splits, (hipStream_t)stream);
}

}  // extern "C"

namespace {
// Strides from the C arrays (batch, head, sequence); NULL = contiguous.
Layout strided_layout(int Hq, int Hkv, int Nq, int Nkv, int D, const long long* qs,
                      const long long* ks, const long long* vs, const long long* os) {
  Layout L = contiguous_layout(Hq, Hkv, Nq, Nkv, D);
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
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                   int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype,
                  contiguous_layout(Hq, Hkv, Nq, Nkv, D));
}

int attn_fwd_strided_check(const void* q, const void* k, const void* v, const void* out,
                           const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                           const long long* q_stride, const long long* k_stride,
                           const long long* v_stride, const long long* o_stride, float scale,
                           int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride));
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
  const Layout L = strided_layout(Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride);
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, L, scale, causal, dtype, num_splits,
             (hipStream_t)stream, mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_masked_check(const void* q, const void* k, const void* v, const void* out,
                          const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                          const long long* q_stride, const long long* k_stride,
                          const long long* v_stride, const long long* o_stride,
                          const void* mask, int mask_type, const long long* mask_stride,
                          float scale, int causal, int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype,
                  strided_layout(Hq, Hkv, Nq, Nkv, D, q_stride, k_stride, v_stride, o_stride),
                  mask_args(mask, mask_type, mask_stride));
}

int attn_fwd_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                        int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dim_ok(D) || (dtype != ATTN_F16 && dtype != ATTN_BF16)) return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  return make_plan(B, Hq, Nq, Nkv, D, causal, 0, num_cus).splits;
}

int attn_fwd_plan(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                  int num_splits, int num_cus, attn_plan* plan) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (!head_dim_ok(D) || (dtype != ATTN_F16 && dtype != ATTN_BF16)) return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT || num_splits < 0 || !plan)
    return ATTN_EINVAL;
  if ((long long)B * Hq * Nq > INT32_MAX || (long long)B * Hkv * Nkv > INT32_MAX)
    return ATTN_EINVAL;
  const Plan pl = make_plan(B, Hq, Nq, Nkv, D, causal, num_splits, num_cus);
  plan->tile_rows = kCfgs[pl.cfg].BM();
  plan->num_splits = pl.splits;
  plan->split_rows = pl.rows - pl.row0;
  plan->workspace_bytes = pl.workspace_bytes();
  return ATTN_OK;
}

size_t attn_fwd_workspace_bytes(int B, int Hq, int Nq, int Nkv, int D, int num_splits) {
  (void)Nkv;
  if (num_splits <= 1 || B <= 0 || Hq <= 0 || Nq <= 0 || D <= 0) return 0;
  const size_t rows = (size_t)B * Hq * Nq;
  return (size_t)num_splits * rows * ((size_t)D + 1) * sizeof(float);
}

const char* attn_strerror(int code) {
  switch (code) {
    case ATTN_OK: return "success";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported device (gfx950 required)";
    case ATTN_ENOMEM: return "device workspace allocation failed";
    case ATTN_EHIP: return "HIP launch or runtime error";
    default: return "unknown error code";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
