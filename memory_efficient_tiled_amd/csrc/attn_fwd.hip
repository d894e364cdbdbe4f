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
//    O^T = V^T P^T, so P never leaves registers.  V^T is the A operand: V is
//    written to LDS transposed ([d][key]) so each lane reads its operand with
//    two 8-byte loads.
//  * The output accumulator O^T also has one query row per lane, so the
//    per-row rescale by alpha = 2^(m_old - m_new) is a plain multiply.
//
// Softmax runs in base 2: scores are scaled by scale*log2(e) and exponentiated
// with v_exp_f32; the log-sum-exp is converted back to natural log.
//
// Split-KV: when query tiles alone cannot fill the 256 compute units, the key
// range is divided into splits; each writes an fp32 partial output normalised
// by its own row sum, plus its partial log-sum-exp, and a second kernel merges
// them with weights exp(lse_s - lse).

#include <hip/hip_runtime.h>

#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "attn.h"

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

struct TagF16 {};
struct TagBF16 {};

template <class Tag>
struct Num;

template <>
struct Num<TagBF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
  // Two fp32 -> two bf16 (round to nearest even) in one 32-bit word.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
};

template <>
struct Num<TagF16> {
  static __device__ __forceinline__ f32x16 mfma(u32x4 a, u32x4 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
};

struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;        // final output (non-split) or unused
  float* lse;         // final LSE (non-split), may be null
  float* opart;       // split: [S][B*Hq*Nq][D] fp32
  float* lsepart;     // split: [S][B*Hq*Nq]
  int Hq, Nq, Nkv, G, Hkv;
  int n_qtiles, n_splits, split_len, total;
  int rows;           // B*Hq*Nq
  float c;            // |scale| * log2(e)
  uint32_t qsign;     // 0x80008000 flips the sign of Q (negative scale)
};

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Renumber
// so that each XCD receives a contiguous range of logical tiles: the query
// tiles of one head then share that XCD's L2 for their K/V stream.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, s = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

template <int D, class Tag, bool CAUSAL, int NW, int QB, int BN, bool SPLIT>
__global__ __launch_bounds__(NW * 64) void attn_fwd_kernel(Params p) {
  constexpr int NT = NW * 64;
  constexpr int BM = NW * QB * 32;
  constexpr int KRS = D + 8;       // K tile row stride in LDS (elements): +16 B breaks bank aliasing
  constexpr int VRS = BN + 4;      // V^T tile row stride in LDS (elements)
  constexpr int KTILE = BN * KRS;
  constexpr int VTILE = D * VRS;
  constexpr int DC = D / 16;       // 16-wide reduction chunks of Q K^T
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr int NDB = D / 32;      // 32-wide output column blocks
  constexpr int NKC = BN / 16;     // 16-key reduction chunks of P V
  constexpr int KCH = BN * D / 8;  // 16-byte chunks per K (or V) tile
  static_assert(KCH % NT == 0, "tile must split evenly over threads");
  constexpr int KLD = KCH / NT;
  constexpr int KG = KLD >= 4 ? 4 : KLD;  // keys packed per transposed V store
  constexpr int VPAIRS = KLD / KG;
  static_assert(VPAIRS * KG == KLD, "V staging must cover the tile");
  static_assert(KG == 4 || KG == 2, "unsupported V staging width");
  using N = Num<Tag>;

  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * (KTILE + VTILE)];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int bid = xcd_remap(blockIdx.x, p.total);
  int sp = 0;
  if (SPLIT) {
    sp = bid % p.n_splits;
    bid /= p.n_splits;
  }
  int qt = bid % p.n_qtiles;
  bid /= p.n_qtiles;
  const int hq = bid % p.Hq;
  const int b = bid / p.Hq;
  if (CAUSAL) qt = p.n_qtiles - 1 - qt;  // longest causal rows first
  const int hk = hq / p.G;
  const int q0 = qt * BM;

  const int kbeg = sp * p.split_len;
  int kend = min(p.Nkv, kbeg + p.split_len);
  if (CAUSAL) kend = min(kend, q0 + BM);  // keys past the tile's last row are all masked
  const int ntiles = kend > kbeg ? (kend - kbeg + BN - 1) / BN : 0;

  const size_t qrow0 = ((size_t)b * p.Hq + hq) * (size_t)p.Nq;
  const size_t krow0 = ((size_t)b * p.Hkv + hk) * (size_t)p.Nkv;
  const uint16_t* __restrict__ Kg = p.k + krow0 * D;
  const uint16_t* __restrict__ Vg = p.v + krow0 * D;

  // Q^T operands for the whole key loop.
  u32x4 qf[QB][DC];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = q0 + (wave * QB + qb) * 32 + l32;
#pragma unroll
    for (int kc = 0; kc < DC; ++kc) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (row < p.Nq)
        x = *(const u32x4*)(p.q + (qrow0 + row) * D + kc * 16 + hl * 8);
      qf[qb][kc] = x ^ p.qsign;
    }
  }

  f32x16 oacc[QB][NDB];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[qb][db] = f32x16{};
  }

  u32x4 kst[KLD];
  u32x4 vst[VPAIRS][KG];

  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = i * NT + tid;
      const int row = c / (D / 8), col = c % (D / 8);
      const int key = k0 + row;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < p.Nkv) x = *(const u32x4*)(Kg + (size_t)key * D + col * 8);
      kst[i] = x;
    }
#pragma unroll
    for (int pr = 0; pr < VPAIRS; ++pr) {
      const int pi = pr * NT + tid;
      const int g = pi % (BN / KG), dc = pi / (BN / KG);
#pragma unroll
      for (int r = 0; r < KG; ++r) {
        const int key = k0 + g * KG + r;
        u32x4 x = {0u, 0u, 0u, 0u};
        if (key < p.Nkv) x = *(const u32x4*)(Vg + (size_t)key * D + dc * 8);
        vst[pr][r] = x;
      }
    }
  };

  auto lstore = [&](int buf) {
    uint16_t* Ks = smem + buf * (KTILE + VTILE);
    uint16_t* Vs = Ks + KTILE;
#pragma unroll
    for (int i = 0; i < KLD; ++i) {
      const int c = i * NT + tid;
      const int row = c / (D / 8), col = c % (D / 8);
      *(u32x4*)(Ks + row * KRS + col * 8) = kst[i];
    }
#pragma unroll
    for (int pr = 0; pr < VPAIRS; ++pr) {
      const int pi = pr * NT + tid;
      const int g = pi % (BN / KG), dc = pi / (BN / KG);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int w = e >> 1;
        uint16_t* dst = Vs + (dc * 8 + e) * VRS + g * KG;
        if (KG == 4) {
          uint32_t a0 = vst[pr][0][w], a1 = vst[pr][1][w], a2 = vst[pr][2][w], a3 = vst[pr][3][w];
          u32x2 y;
          if (e & 1) {
            y[0] = (a0 >> 16) | (a1 & 0xffff0000u);
            y[1] = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            y[0] = (a0 & 0xffffu) | (a1 << 16);
            y[1] = (a2 & 0xffffu) | (a3 << 16);
          }
          *(u32x2*)dst = y;
        } else {
          uint32_t a0 = vst[pr][0][w], a1 = vst[pr][1][w];
          *(uint32_t*)dst = (e & 1) ? ((a0 >> 16) | (a1 & 0xffff0000u)) : ((a0 & 0xffffu) | (a1 << 16));
        }
      }
    }
  };

  if (ntiles > 0) {
    gload(kbeg);
    lstore(0);
    __syncthreads();
  }

  const int wq0 = q0 + wave * QB * 32;  // first query row of this wave

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = kbeg + t * BN;
    const bool more = t + 1 < ntiles;
    if (more) gload(k0 + BN);

    const uint16_t* Ks = smem + (t & 1) * (KTILE + VTILE);
    const uint16_t* Vs = Ks + KTILE;

    // S^T = K Q^T for this tile.
    f32x16 s[QB][NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int kc = 0; kc < DC; ++kc) {
        const u32x4 a = *(const u32x4*)(Ks + (kb * 32 + l32) * KRS + kc * 16 + hl * 8);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb][kb] = N::mfma(a, qf[qb][kc], s[qb][kb]);
      }
    }

    // Keys past the valid range, and (causal) keys after the row, get -inf.
    const bool need_mask = (k0 + BN > kend) || (CAUSAL && k0 + BN - 1 > wq0);
    if (need_mask) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int row = wq0 + qb * 32 + l32;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = k0 + kb * 32 + 8 * (e >> 2) + 4 * hl + (e & 3);
            const bool ok = key < kend && (!CAUSAL || key <= row);
            if (!ok) s[qb][kb][e] = -INFINITY;
          }
      }
    }

    // Online softmax (base 2), then P in the input type as the B operand.
    u32x4 pf[QB][NKC];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[qb][kb][e]);
      mx = fmaxf(mx, xor32(mx));
      const float mc = (mx == -INFINITY) ? -INFINITY : mx * p.c;
      const float mnew = fmaxf(m[qb], mc);
      const float mb = (mnew == -INFINITY) ? 0.f : mnew;
      const float alpha = fast_exp2(m[qb] - mb);
      m[qb] = mnew;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float sv = s[qb][kb][e];
          float x = fast_exp2(fmaf(sv, p.c, -mb));
          if (need_mask && sv == -INFINITY) x = 0.f;
          s[qb][kb][e] = x;
          rs += x;
        }
      l[qb] = l[qb] * alpha + rs;  // lane-partial: the partner lane holds the other keys
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[qb][db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
          u32x4 y;
#pragma unroll
          for (int w = 0; w < 4; ++w)
            y[w] = N::pack2(s[qb][kb][8 * hf + 2 * w], s[qb][kb][8 * hf + 2 * w + 1]);
          pf[qb][kb * 2 + hf] = y;
        }
    }

    // O^T += V^T P^T.
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int kc = 0; kc < NKC; ++kc) {
        const uint16_t* src = Vs + (db * 32 + l32) * VRS + kc * 16 + 4 * hl;
        const u32x2 lo = *(const u32x2*)src;
        const u32x2 hi = *(const u32x2*)(src + 8);
        const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = N::mfma(a, pf[qb][kc], oacc[qb][db]);
      }
    }

    if (more) lstore((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: combine the two lane halves' row sums, normalise, store.
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = wq0 + qb * 32 + l32;
    const float lt = l[qb] + xor32(l[qb]);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse_v = lt > 0.f ? (m[qb] + __log2f(lt)) * kLn2 : -INFINITY;
    if (row < p.Nq) {
      if (SPLIT) {
        const size_t prow = (size_t)sp * p.rows + qrow0 + row;
        float* dst = p.opart + prow * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 y = {oacc[qb][db][4 * i] * inv, oacc[qb][db][4 * i + 1] * inv,
                       oacc[qb][db][4 * i + 2] * inv, oacc[qb][db][4 * i + 3] * inv};
            *(f32x4*)(dst + db * 32 + 8 * i + 4 * hl) = y;
          }
        if (hl == 0) p.lsepart[prow] = lse_v;
      } else {
        uint16_t* dst = p.o + (qrow0 + row) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            u32x2 y = {N::pack2(oacc[qb][db][4 * i] * inv, oacc[qb][db][4 * i + 1] * inv),
                       N::pack2(oacc[qb][db][4 * i + 2] * inv, oacc[qb][db][4 * i + 3] * inv)};
            *(u32x2*)(dst + db * 32 + 8 * i + 4 * hl) = y;
          }
        if (hl == 0 && p.lse) p.lse[qrow0 + row] = lse_v;
      }
    }
  }
}

// Merge split-KV partials: lse = log sum_s exp(lse_s), O = sum_s exp(lse_s - lse) O_s.
template <int D, class Tag>
__global__ __launch_bounds__(256) void attn_combine_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ lsepart,
                                                           uint16_t* __restrict__ o,
                                                           float* __restrict__ lse, int rows,
                                                           int n_splits) {
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
  *(u32x2*)(o + row * D + c4 * 4) = y;
  if (c4 == 0 && lse) lse[row] = wsum > 0.f ? mx + logf(wsum) : -INFINITY;
}

// ---------------------------------------------------------------------------
// Host side.
// ---------------------------------------------------------------------------

// Tile table per head dimension.
struct TileCfg {
  int NW, QB, BN;
  int BM() const { return NW * QB * 32; }
};
constexpr TileCfg kCfgD64 = {4, 1, 64};
constexpr TileCfg kCfgD128 = {4, 1, 64};
constexpr int kResidentWgPerCu = 2;

inline TileCfg cfg_for(int D) { return D == 64 ? kCfgD64 : kCfgD128; }

thread_local int g_last_hip_error = 0;

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

bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

int validate(const void* q, const void* k, const void* v, const void* out, const float* lse,
             int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
             int dtype) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0) return ATTN_EINVAL;
  if (Hq % Hkv != 0) return ATTN_EINVAL;
  if (D != 64 && D != 128) return ATTN_EINVAL;
  if (dtype != ATTN_F16 && dtype != ATTN_BF16) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  if (!isfinite(scale)) return ATTN_EINVAL;
  if (!q || !k || !v || !out) return ATTN_EINVAL;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15) return ATTN_EINVAL;
  if (((uintptr_t)lse) & 3) return ATTN_EINVAL;
  // Grid and row counts are held in 32-bit integers on the device.
  const size_t rows = (size_t)B * Hq * Nq;
  const size_t krows = (size_t)B * Hkv * Nkv;
  if (rows > (size_t)INT32_MAX || krows > (size_t)INT32_MAX) return ATTN_EINVAL;
  const size_t qbytes = rows * D * 2, kbytes = krows * D * 2;
  if (overlaps(out, qbytes, q, qbytes) || overlaps(out, qbytes, k, kbytes) ||
      overlaps(out, qbytes, v, kbytes))
    return ATTN_EINVAL;
  if (lse) {
    const size_t lbytes = rows * 4;
    if (overlaps(lse, lbytes, q, qbytes) || overlaps(lse, lbytes, k, kbytes) ||
        overlaps(lse, lbytes, v, kbytes) || overlaps(lse, lbytes, out, qbytes))
      return ATTN_EINVAL;
  }
  return ATTN_OK;
}

// Split-KV count: enough workgroups for every CU to hold kResidentWgPerCu of
// them, with each split keeping at least 8 key tiles.
int choose_splits(int B, int Hq, int Nq, int Nkv, int D, int num_cus) {
  const TileCfg c = cfg_for(D);
  const long long wgs = (long long)B * Hq * ((Nq + c.BM() - 1) / c.BM());
  const long long target = (long long)kResidentWgPerCu * (num_cus > 0 ? num_cus : 256);
  if (wgs >= target) return 1;
  const int ktiles = (Nkv + c.BN - 1) / c.BN;
  long long s = (target + wgs - 1) / wgs;
  const long long by_keys = ktiles / 8;
  if (s > by_keys) s = by_keys;
  if (s > 64) s = 64;
  return s < 1 ? 1 : (int)s;
}

template <int D, class Tag, bool CAUSAL, bool SPLIT>
hipError_t launch_main(const Params& p, hipStream_t stream) {
  constexpr TileCfg c = (D == 64) ? kCfgD64 : kCfgD128;
  hipLaunchKernelGGL((attn_fwd_kernel<D, Tag, CAUSAL, c.NW, c.QB, c.BN, SPLIT>), dim3(p.total),
                     dim3(c.NW * 64), 0, stream, p);
  return hipGetLastError();
}

template <int D, class Tag>
hipError_t dispatch(const Params& p, bool causal, bool split, hipStream_t st) {
  if (causal)
    return split ? launch_main<D, Tag, true, true>(p, st) : launch_main<D, Tag, true, false>(p, st);
  return split ? launch_main<D, Tag, false, true>(p, st) : launch_main<D, Tag, false, false>(p, st);
}

template <int D, class Tag>
hipError_t launch_combine(const Params& p, hipStream_t st) {
  const size_t threads = (size_t)p.rows * (D / 4);
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL((attn_combine_kernel<D, Tag>), dim3(blocks), dim3(256), 0, st, p.opart,
                     p.lsepart, p.o, p.lse, p.rows, p.n_splits);
  return hipGetLastError();
}

int run(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq, int Hkv,
        int Nq, int Nkv, int D, float scale, int causal, int dtype, int num_splits,
        hipStream_t stream) {
  int rc = validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype);
  if (rc != ATTN_OK) return rc;
  if (num_splits < 0) return ATTN_EINVAL;
  DeviceInfo di;
  rc = device_info(&di);
  if (rc != ATTN_OK) return rc;

  const TileCfg c = cfg_for(D);
  const int ktiles = (Nkv + c.BN - 1) / c.BN;
  int S = num_splits > 0 ? num_splits : choose_splits(B, Hq, Nq, Nkv, D, di.cus);
  if (S > ktiles) S = ktiles;
  const int tiles_per_split = (ktiles + S - 1) / S;
  S = (ktiles + tiles_per_split - 1) / tiles_per_split;  // drop empty trailing splits

  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)out;
  p.lse = lse;
  p.opart = nullptr;
  p.lsepart = nullptr;
  p.Hq = Hq;
  p.Nq = Nq;
  p.Nkv = Nkv;
  p.G = Hq / Hkv;
  p.Hkv = Hkv;
  p.n_qtiles = (Nq + c.BM() - 1) / c.BM();
  p.n_splits = S;
  p.split_len = tiles_per_split * c.BN;
  p.rows = B * Hq * Nq;
  p.c = fabsf(scale) * kLog2e;
  p.qsign = scale < 0.f ? 0x80008000u : 0u;
  const long long total = (long long)B * Hq * p.n_qtiles * S;
  if (total > INT32_MAX) return ATTN_EINVAL;
  p.total = (int)total;

  const bool split = S > 1;
  void* ws = nullptr;
  if (split) {
    const size_t bytes = attn_fwd_workspace_bytes(B, Hq, Nq, Nkv, D, S);
    hipError_t e = hipMallocAsync(&ws, bytes, stream);
    if (e != hipSuccess || !ws) {
      g_last_hip_error = (int)e;
      (void)hipGetLastError();
      return ATTN_ENOMEM;
    }
    p.opart = (float*)ws;
    p.lsepart = p.opart + (size_t)S * p.rows * D;
  }

  hipError_t e;
  const bool cz = causal != 0;
  if (D == 64)
    e = dtype == ATTN_BF16 ? dispatch<64, TagBF16>(p, cz, split, stream)
                           : dispatch<64, TagF16>(p, cz, split, stream);
  else
    e = dtype == ATTN_BF16 ? dispatch<128, TagBF16>(p, cz, split, stream)
                           : dispatch<128, TagF16>(p, cz, split, stream);
  if (e == hipSuccess && split) {
    if (D == 64)
      e = dtype == ATTN_BF16 ? launch_combine<64, TagBF16>(p, stream)
                             : launch_combine<64, TagF16>(p, stream);
    else
      e = dtype == ATTN_BF16 ? launch_combine<128, TagBF16>(p, stream)
                             : launch_combine<128, TagF16>(p, stream);
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

extern "C" {

int attn_fwd(const void* q, const void* k, const void* v, void* out, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype, 0,
             (hipStream_t)stream);
}

int attn_fwd_split(const void* q, const void* k, const void* v, void* out, float* lse, int B,
                   int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal, int dtype,
                   int num_splits, void* stream) {
  return run(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype, num_splits,
             (hipStream_t)stream);
}

int attn_fwd_check(const void* q, const void* k, const void* v, const void* out, const float* lse,
                   int B, int Hq, int Hkv, int Nq, int Nkv, int D, float scale, int causal,
                   int dtype) {
  return validate(q, k, v, out, lse, B, Hq, Hkv, Nq, Nkv, D, scale, causal, dtype);
}

int attn_fwd_num_splits(int B, int Hq, int Hkv, int Nq, int Nkv, int D, int causal, int dtype,
                        int num_cus) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || Nq <= 0 || Nkv <= 0 || Hq % Hkv != 0) return ATTN_EINVAL;
  if ((D != 64 && D != 128) || (dtype != ATTN_F16 && dtype != ATTN_BF16)) return ATTN_EINVAL;
  if (causal != 0 && causal != 1) return ATTN_EINVAL;
  const TileCfg c = cfg_for(D);
  const int ktiles = (Nkv + c.BN - 1) / c.BN;
  int S = choose_splits(B, Hq, Nq, Nkv, D, num_cus);
  if (S > ktiles) S = ktiles;
  const int tps = (ktiles + S - 1) / S;
  return (ktiles + tps - 1) / tps;
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
    case ATTN_ENOMEM: return "split-KV workspace allocation failed";
    case ATTN_EHIP: return "HIP launch or runtime error";
    default: return "unknown error code";
  }
}

int attn_last_hip_error(void) { return g_last_hip_error; }

}  // extern "C"
