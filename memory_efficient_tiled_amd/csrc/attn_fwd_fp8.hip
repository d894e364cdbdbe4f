// attn_fwd_fp8.hip -- the attention forward on FP8 inputs (OCP E4M3, one
// descale factor per tensor), head dimension 128, for gfx950.
//
// What is computed: the forward of attn_fwd.hip on the values
// q8 * q_descale, k8 * k_descale, v8 * v_descale, with the output in
// bf16 or fp16 and the row log-sum-exp in fp32.  Both products run on the
// 8-bit matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 x E4M3,
// fp32 accumulation, block scales fixed at 1), at twice the 16-bit rate:
//  * S^T = K Q^T: K (A operand) from LDS, Q^T (B operand) in registers; a
//    lane holds 32 consecutive bytes of a row for both, so each reduction
//    slot pairs the same head-dimension element.
//  * O^T = V^T P^T: P is rounded to E4M3 (the running reference max keeps
//    every probability at most 2^8, inside E4M3's range of 448).  The
//    instruction pairs operand byte s of lane group g (lanes 32g..32g+31)
//    of A with byte s of lane group g of B, so P^T and V^T only have to
//    agree on which key each (g, s) holds: lane group g takes keys
//    32g..32g+31 of the 64-key tile in order.  A lane's scores cover half
//    of those keys (the 32x32 accumulator interleaves the two lane groups
//    in blocks of 4 keys); one v_permlane32_swap per 4 packed probabilities
//    exchanges the halves.  V is transposed once per call into a workspace
//    ([B, Hkv, D, Nkv rounded up to 64], zero padded), so a lane's 32 keys
//    of one column are 32 contiguous bytes.
// Softmax, masking, split-KV and the merge are those of the 16-bit kernel.

#include "attn_fwd_kernel.h"

namespace {

using namespace attn_fwd_detail;

typedef int i32x8 __attribute__((ext_vector_type(8)));

constexpr int kD8 = 128;   // head dimension
constexpr int kBN8 = 64;   // keys per tile
constexpr int kNW8 = 8;    // waves per workgroup, 32 query rows each

// S (32 x 32, fp32) += A (32 x 64) B (64 x 32) on E4M3 operands, block
// scales 2^0 (E8M0 127).
__device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}

__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
               (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// Four fp32 -> four E4M3 bytes (round to nearest even), byte i from x_i.
__device__ __forceinline__ uint32_t pack4_fp8(float a, float b, float c, float d) {
  const uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
}

// V [B*Hkv, Nkv, 128] -> V^T [B*Hkv, 128, nkv_pad] (bytes), keys past Nkv
// zero.  One workgroup per 64 keys of one head, through LDS.
__global__ __launch_bounds__(256) void attn_fp8_transpose_v(const uint8_t* __restrict__ v,
                                                            uint8_t* __restrict__ vt, int Nkv,
                                                            int nkv_pad, int tiles_per_head) {
  __shared__ __attribute__((aligned(16))) uint8_t t[64][kD8 + 16];
  const int bh = blockIdx.x / tiles_per_head, k0 = (blockIdx.x % tiles_per_head) * 64;
  const uint8_t* src = v + (size_t)bh * Nkv * kD8;
  uint8_t* dst = vt + (size_t)bh * kD8 * nkv_pad;
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 64 rows x 8 chunks of 16 bytes
    const int c = threadIdx.x + 256 * i, r = c >> 3, ch = c & 7;
    u32x4 x = {0u, 0u, 0u, 0u};
    if (k0 + r < Nkv) x = *(const u32x4*)(src + (size_t)(k0 + r) * kD8 + ch * 16);
    *(u32x4*)(&t[r][ch * 16]) = x;
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 2; ++i) {  // 128 rows x 4 chunks of 16 keys
    const int c = threadIdx.x + 256 * i, d = c >> 2, ch = c & 3;
    u32x4 y;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int r = ch * 16 + 4 * w;
      y[w] = (uint32_t)t[r][d] | ((uint32_t)t[r + 1][d] << 8) | ((uint32_t)t[r + 2][d] << 16) |
             ((uint32_t)t[r + 3][d] << 24);
    }
    *(u32x4*)(dst + (size_t)d * nkv_pad + k0 + ch * 16) = y;
  }
}

// One workgroup: 8 waves x 32 query rows of query head hq, over the 64-key
// tiles of its key range; K and V^T tiles double-buffered in LDS (8 KB
// each), scores double-buffered in registers (the pipeline of the 16-bit
// kernel's narrow tiles).  K rows are 128 bytes, stored with 16-byte chunk
// c at c ^ ((r >> 1) & 7); V^T rows are 64 bytes, chunk c at
// c ^ ((d >> 2) & 3): the 16 lanes that read one chunk of 16 consecutive
// rows then hit 16 distinct bank groups.
template <class Tag, bool CAUSAL, bool SPLIT>
__global__ __launch_bounds__(kNW8 * 64, kWavesPerSimd) void attn_fwd_fp8_kernel(
    Params p, const uint8_t* __restrict__ vt, int nkv_pad, float v_descale) {
  constexpr int D = kD8, BN = kBN8, NW = kNW8;
  constexpr int BM = NW * 32;
  constexpr int NKB = BN / 32;  // 32-key score blocks per tile
  constexpr int NDB = D / 32;   // 32-wide output column blocks
  constexpr int DC = D / 64;    // reduction chunks of Q K^T
  using N = Num<Tag>;

  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[BN * D];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[BN * D];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf0[D * BN];
  __shared__ __attribute__((aligned(1024))) uint8_t vbuf1[D * BN];

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // A split launch may start with whole tiles (as in the 16-bit path): its
  // pieces then take the slots of the whole tiles that finish first.
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
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;
  const int hk = hq / p.G;
  const int q0 = qt * BM;
  const int wq0 = q0 + wave * 32;
  const int qrow = wq0 + l32;

  const int kbeg = piece ? sp * p.split_len : 0;
  int kend = piece ? min(p.Nkv, kbeg + p.split_len) : p.Nkv;
  if (CAUSAL) kend = max(0, min(kend, q0 + BM + p.coff));
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const uint8_t* Qg = (const uint8_t*)p.q + qrow0 * D;
  const uint8_t* Kg = (const uint8_t*)p.k + ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv * D;
  const uint8_t* VTg = vt + ((size_t)b * p.Hkv + hk) * (size_t)D * nkv_pad;

  // One 1 KB copy per wave and tile of each: slot wave * 64 + lane.
  const int slot = wave * 64 + lane;
  const int krow = slot >> 3, vd = slot >> 2;
  const uint32_t koff = krow * D + (((slot & 7) ^ ((krow >> 1) & 7)) << 4);
  const uint32_t voff = vd * nkv_pad + (((slot & 3) ^ ((vd >> 2) & 3)) << 4);
  // K rows past the key range read as zero (their scores are masked); the
  // V^T workspace is zero past Nkv and covers every tile.
  auto issue_k = [&](int t, uint8_t* dst) {
    const int k0 = kbeg + t * BN;
    const int nrows = min(BN, p.Nkv - k0);
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(Kg + (size_t)k0 * D), 0, nrows * D, kRawBufferFlags);
    buf2lds16(r, (uint16_t*)(dst + wave * 1024), koff);
  };
  auto issue_v = [&](int t, uint8_t* dst) {
    const int k0 = kbeg + t * BN;
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(VTg + k0), 0, (D - 1) * nkv_pad + BN, kRawBufferFlags);
    buf2lds16(r, (uint16_t*)(dst + wave * 1024), voff);
  };

  // Q^T operands: bytes 64 kc + 32 hl .. + 31 of this lane's query row.
  i32x8 qf[DC];
#pragma unroll
  for (int kc = 0; kc < DC; ++kc) {
    u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
    if (qrow < p.Nq) {
      lo = *(const u32x4*)(Qg + (size_t)qrow * D + kc * 64 + hl * 32);
      hi = *(const u32x4*)(Qg + (size_t)qrow * D + kc * 64 + hl * 32 + 16);
    }
    qf[kc] = cat8(lo ^ p.qsign, hi ^ p.qsign);
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // S^T = K Q^T for one tile (LDS).
  auto qk = [&](const uint8_t* ks, f32x16* s) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < DC; ++kc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int row = kb * 32 + l32, sw = (row >> 1) & 7, c0 = 4 * kc + 2 * hl;
        const u32x4 lo = *(const u32x4*)(ks + row * D + ((c0 ^ sw) << 4));
        const u32x4 hi = *(const u32x4*)(ks + row * D + (((c0 + 1) ^ sw) << 4));
        s[kb] = mfma_fp8(cat8(lo, hi), qf[kc], s[kb]);
      }
  };

  // Keys past the range, and (causal) keys after the row, get -inf.
  auto mask = [&](int t, f32x16* s) {
    const int k0 = kbeg + t * BN;
    if ((k0 + BN > kend) || (CAUSAL && k0 + BN - 1 > wq0 + p.coff)) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
          const bool ok = key < kend && (!CAUSAL || key <= qrow + p.coff);
          if (!ok) s[kb][e] = -INFINITY;
        }
    }
  };

  auto probs = [&](f32x16* s, float mb) {
    float rs[4];   // started from their first terms (an add of 0 is not folded)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[kb][e] = fast_exp2(fmaf(s[kb][e], p.c, -mb));
        if (kb == 0 && e < 4)
          rs[e] = s[kb][e];
        else
          rs[e & 3] += s[kb][e];
      }
    return (rs[0] + rs[1]) + (rs[2] + rs[3]);
  };

  // The slow path needs tile t's raw scores again; its K buffer is being
  // refilled, so K comes from global memory (rows past Nkv read as zero).
  auto rescore = [&](int t, f32x16* s) {
    const int k0 = kbeg + t * BN;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kc = 0; kc < DC; ++kc)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const int key = k0 + kb * 32 + l32;
        u32x4 lo = {0u, 0u, 0u, 0u}, hi = {0u, 0u, 0u, 0u};
        if (key < p.Nkv) {
          lo = *(const u32x4*)(Kg + (size_t)key * D + kc * 64 + hl * 32);
          hi = *(const u32x4*)(Kg + (size_t)key * D + kc * 64 + hl * 32 + 16);
        }
        s[kb] = mfma_fp8(cat8(lo, hi), qf[kc], s[kb]);
      }
    mask(t, s);
  };

  // Probabilities of tile t (scores s) against the running reference max,
  // raised from recomputed scores when a partial sum exceeds 2^8 or the
  // reference is still -inf; then P^T as the E4M3 B operand of P V.
  auto softmax = [&](int t, f32x16* s, i32x8* pb) {
    float rs = probs(s, m);
    const bool bad = !(m > -INFINITY) || !(rs <= kMaxPartialSum);
    if (__builtin_amdgcn_ballot_w64(bad)) {
      rescore(t, s);
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
      mx = pair_max(mx);
      const float mc = (mx == -INFINITY) ? -INFINITY : mx * p.c;
      const float mnew = fmaxf(m, mc);
      const float alpha = (m == -INFINITY) ? 0.f : fast_exp2(m - mnew);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      rs = probs(s, (mnew == -INFINITY) ? 0.f : mnew);
    }
    l += rs;  // lane-partial: lane l ^ 32 holds the rest
    // dword a of block kb: keys kb*32 + 8a + 4hl .. + 3 of this lane
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const uint32_t d0 = pack4_fp8(s[0][4 * a], s[0][4 * a + 1], s[0][4 * a + 2], s[0][4 * a + 3]);
      const uint32_t d1 = pack4_fp8(s[1][4 * a], s[1][4 * a + 1], s[1][4 * a + 2], s[1][4 * a + 3]);
      // lanes 32..63 of d0 trade with lanes 0..31 of d1: lane group g then
      // holds keys 32g + 8a .. + 3 (r[0]) and 32g + 8a + 4 .. + 7 (r[1])
      const auto r = __builtin_amdgcn_permlane32_swap(d0, d1, false, false);
      (*pb)[2 * a] = (int)r[0];
      (*pb)[2 * a + 1] = (int)r[1];
    }
  };

  // O^T += V^T P^T: lane (d + 32 g) reads keys 32g .. 32g + 31 of column d.
  auto pv = [&](const uint8_t* vs, const i32x8& pb) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 32 + l32, sw = (d >> 2) & 3;
      const u32x4 lo = *(const u32x4*)(vs + d * BN + (((2 * hl) ^ sw) << 4));
      const u32x4 hi = *(const u32x4*)(vs + d * BN + (((2 * hl + 1) ^ sw) << 4));
      oacc[db] = mfma_fp8(cat8(lo, hi), pb, oacc[db]);
    }
  };

  // One step for tile t (scores in s): K_t, V_t in (kc, vc); K_{t+2} and
  // V_{t+1} are copied into kc and vn after the barrier, S_{t+1} = K_{t+1} Q^T
  // (kn) is formed while the softmax of S_t runs.
  auto step = [&](auto last, int t, f32x16* s, f32x16* sn, uint8_t* kc, uint8_t* vc,
                  uint8_t* kn, uint8_t* vn) {
    constexpr bool LAST = decltype(last)::value;
    mask(t, s);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (!LAST) {
      if (t + 2 < ntiles) issue_k(t + 2, kc);
      issue_v(t + 1, vn);
      qk(kn, sn);
    }
    i32x8 pb;
    softmax(t, s, &pb);
    pv(vc, pb);
  };
  using Last = std::integral_constant<bool, true>;
  using More = std::integral_constant<bool, false>;

  f32x16 sa[NKB], sb[NKB];
  if (ntiles > 0) {
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

  // Epilogue: row sum over both lane halves, normalise, apply V's descale.
  const float lt = pair_sum(l);
  const float inv = lt > 0.f ? v_descale / lt : 0.f;
  const float lse_v = lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  if (qrow < p.Nq) {
    if (piece) {
      const size_t prow = (size_t)sp * p.prows + (qrow0 + qrow - p.row0);
      float* dst = p.opart + prow * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& o = oacc[db];
          *(f32x4*)(dst + db * 32 + 8 * i + 4 * hl) =
              f32x4{o[4 * i] * inv, o[4 * i + 1] * inv, o[4 * i + 2] * inv, o[4 * i + 3] * inv};
        }
      if (hl == 0) p.lsepart[prow] = lse_v;
    } else {
      uint16_t* dst = p.o + (qrow0 + qrow) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const f32x16& o = oacc[db];
          *(u32x2*)(dst + db * 32 + 8 * i + 4 * hl) =
              u32x2{N::pack2(o[4 * i] * inv, o[4 * i + 1] * inv),
                    N::pack2(o[4 * i + 2] * inv, o[4 * i + 3] * inv)};
        }
      if (hl == 0 && p.lse) p.lse[qrow0 + qrow] = lse_v;
    }
  }
}

template <class Tag, bool SPLIT>
hipError_t launch_fp8_main(const Params& p, bool causal, const uint8_t* vt, int nkv_pad,
                           float vds, hipStream_t st) {
  if (causal)
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<Tag, true, SPLIT>), dim3(p.total), dim3(kNW8 * 64),
                       0, st, p, vt, nkv_pad, vds);
  else
    hipLaunchKernelGGL((attn_fwd_fp8_kernel<Tag, false, SPLIT>), dim3(p.total), dim3(kNW8 * 64),
                       0, st, p, vt, nkv_pad, vds);
  return hipGetLastError();
}

hipError_t launch_fp8(const Params& p, bool bf16, bool causal, bool split, const uint8_t* vt,
                      int nkv_pad, float vds, hipStream_t st) {
  if (bf16)
    return split ? launch_fp8_main<TagBF16, true>(p, causal, vt, nkv_pad, vds, st)
                 : launch_fp8_main<TagBF16, false>(p, causal, vt, nkv_pad, vds, st);
  return split ? launch_fp8_main<TagF16, true>(p, causal, vt, nkv_pad, vds, st)
               : launch_fp8_main<TagF16, false>(p, causal, vt, nkv_pad, vds, st);
}

bool overlaps_fp8(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int validate_fp8(const void* q, const void* k, const void* v, const void* out, const float* lse,
                 int B, int Hq, int Hkv, int Nq, int Nkv, int D, float qds, float kds, float vds,
                 float scale, int causal, int out_dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if (D != kD8) return ATTN_EINVAL;
  if (out_dtype != ATTN_F16 && out_dtype != ATTN_BF16) return ATTN_EINVAL;
  if (causal < 0 || causal > ATTN_CAUSAL_BOTTOM_RIGHT) return ATTN_EINVAL;
  if (!isfinite(scale) || !isfinite(qds) || !isfinite(kds) || !isfinite(vds)) return ATTN_EINVAL;
  if (!(qds > 0.f) || !(kds > 0.f) || !(vds > 0.f)) return ATTN_EINVAL;
  if (!q || !k || !v || !out) return ATTN_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_EINVAL;
  if ((uintptr_t)lse & 3) return ATTN_EINVAL;
  const size_t rows = (size_t)B * Hq * Nq, krows = (size_t)B * Hkv * Nkv;
  if (rows > (size_t)INT32_MAX || krows > (size_t)INT32_MAX) return ATTN_EINVAL;
  if (Nkv > (1 << 24)) return ATTN_EINVAL;  // V^T row offsets are 32-bit
  const size_t qb = rows * D, kb = krows * D, ob = rows * D * 2;
  if (overlaps_fp8(out, ob, q, qb) || overlaps_fp8(out, ob, k, kb) || overlaps_fp8(out, ob, v, kb))
    return ATTN_EINVAL;
  if (lse && (overlaps_fp8(lse, rows * 4, q, qb) || overlaps_fp8(lse, rows * 4, k, kb) ||
              overlaps_fp8(lse, rows * 4, v, kb) || overlaps_fp8(lse, rows * 4, out, ob)))
    return ATTN_EINVAL;
  return ATTN_OK;
}

int run_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
            int Hkv, int Nq, int Nkv, int D, float qds, float kds, float vds, float scale,
            int causal, int out_dtype, int num_splits, hipStream_t st) {
  int rc = validate_fp8(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, qds, kds, vds, scale, causal,
                        out_dtype);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_EINVAL;
  int cus = 0;
  rc = attn_host::check_device(&cus);
  if (rc != ATTN_OK) return rc;
  attn_host::NarrowPlan pl;
  attn_host::narrow_plan(B, Hq, Nq, Nkv, D, causal, num_splits, cus, &pl);
  const long long split_wgs = (pl.tiles - pl.first_split) * pl.splits;
  // grid sizes are ints: whole tiles and pieces share one launch
  if (pl.first_split + split_wgs > INT32_MAX) return ATTN_EINVAL;

  const int nkv_pad = (Nkv + kBN8 - 1) / kBN8 * kBN8;
  const size_t vt_bytes = ((size_t)B * Hkv * D * nkv_pad + 255) / 256 * 256;
  const size_t part_bytes =
      split_wgs > 0 ? (size_t)pl.splits * (size_t)(pl.rows - pl.row0) * (D + 1) * sizeof(float) : 0;
  void* ws = nullptr;
  hipError_t e = attn_host::workspace_alloc(&ws, vt_bytes + part_bytes, st);
  if (e != hipSuccess || !ws) {
    attn_host::set_last_hip_error((int)e);
    (void)hipGetLastError();
    return ATTN_ENOMEM;
  }
  uint8_t* vt = (uint8_t*)ws;

  Params p = {};
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  p.lse = lse;
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
  // scores of the 8-bit values times the descales, scale and log2(e); kept
  // positive (a masked score must give exactly 0) as in the 16-bit path
  p.c = fmaxf(fabsf(scale) * qds * kds * kLog2e, FLT_MIN);
  p.qsign = scale < 0.f ? 0x80808080u : 0u;  // E4M3 sign bits of Q
  p.coff = causal == ATTN_CAUSAL_BOTTOM_RIGHT ? Nkv - Nq : 0;
  if (split_wgs > 0) {
    p.opart = (float*)((char*)ws + vt_bytes);
    p.lsepart = p.opart + (size_t)pl.splits * p.prows * D;
  }

  const int tph = nkv_pad / kBN8;
  hipLaunchKernelGGL(attn_fp8_transpose_v, dim3((unsigned)((long long)B * Hkv * tph)), dim3(256),
                     0, st, (const uint8_t*)v, vt, Nkv, nkv_pad, tph);
  e = hipGetLastError();
  const bool bf16 = out_dtype == ATTN_BF16, cz = causal != 0;
  // whole tiles and the pieces of the rest in one launch, whole tiles first
  p.n_whole = 0;
  if (e == hipSuccess && split_wgs > 0) {
    p.n_whole = (int)pl.first_split;
    p.total = (int)(pl.first_split + split_wgs);
    p.tile0 = (int)pl.first_split;
    e = launch_fp8(p, bf16, cz, true, vt, nkv_pad, vds, st);
    if (e == hipSuccess) e = launch_combine_d<kD8>(p, false, bf16, st);
  } else if (e == hipSuccess && pl.first_split > 0) {
    p.total = (int)pl.first_split;
    p.tile0 = 0;
    e = launch_fp8(p, bf16, cz, false, vt, nkv_pad, vds, st);
  }
  const hipError_t ef = hipFreeAsync(ws, st);
  if (e == hipSuccess) e = ef;
  if (e != hipSuccess) {
    attn_host::set_last_hip_error((int)e);
    return ATTN_EHIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

int attn_fwd_fp8(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                 int Hq, int Hkv, int Nq, int Nkv, int D, float q_descale, float k_descale,
                 float v_descale, float scale, int causal, int out_dtype, int num_splits,
                 void* stream) {
  return run_fp8(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, q_descale, k_descale, v_descale,
                 scale, causal, out_dtype, num_splits, (hipStream_t)stream);
}

int attn_fwd_fp8_check(const void* q, const void* k, const void* v, const void* out,
                       const float* lse, int B, int Hq, int Hkv, int Nq, int Nkv, int D,
                       float q_descale, float k_descale, float v_descale, float scale,
                       int causal, int out_dtype) {
  return validate_fp8(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, q_descale, k_descale, v_descale,
                      scale, causal, out_dtype);
}

}  // extern "C"
