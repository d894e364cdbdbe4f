// attn_common.h -- device helpers shared by the attention kernels (forward
// and gradients) and the host hooks they share; included by both sources.
#ifndef ATTN_COMMON_H_
#define ATTN_COMMON_H_

#include <hip/hip_runtime.h>

#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "attn.h"
#include "attn_tiles.h"

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

// The low / high 16-bit value of a 32-bit word as fp32.
template <class Tag>
__device__ __forceinline__ float lo_f32(uint32_t w);
template <class Tag>
__device__ __forceinline__ float hi_f32(uint32_t w);
template <>
__device__ __forceinline__ float lo_f32<TagBF16>(uint32_t w) { return __uint_as_float(w << 16); }
template <>
__device__ __forceinline__ float hi_f32<TagBF16>(uint32_t w) {
  return __uint_as_float(w & 0xFFFF0000u);
}
template <>
__device__ __forceinline__ float lo_f32<TagF16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[0];
}
template <>
__device__ __forceinline__ float hi_f32<TagF16>(uint32_t w) {
  return (float)__builtin_bit_cast(f16x2, w)[1];
}

// Attention-mask values as base-2 biases.  ATTN_MASK_BOOL: bytes, zero
// removes the key (-inf), nonzero keeps it (0).  ATTN_MASK_ADD: values of
// the input type, added to the scaled scores (times log2 e here).
// mask_keep4: the bytes of keys key0 .. key0 + 3 of one boolean mask row
// (byte i nonzero keeps key key0 + i); keys at or past nkv are not read
// and come back kept.
__device__ __forceinline__ uint32_t mask_keep4(const uint8_t* mrow, int key0, int nkv) {
  if (key0 + 3 < nkv) return *(const uint32_t*)(mrow + key0);
  uint32_t w = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (key0 + i < nkv) w |= (uint32_t)mrow[key0 + i] << (8 * i);
  return w | (~0u << (8 * max(0, min(4, nkv - key0))));
}

// mask_bias4: keys key0 .. key0 + 3 of one mask row (16-bit mask rows at
// `mrow` as bytes); keys at or past nkv are not read (bias 0).
template <class Tag>
__device__ __forceinline__ void mask_bias4(const uint8_t* mrow, int mode, int key0, int nkv,
                                           float* bias) {
  if (mode == ATTN_MASK_BOOL) {
    const uint32_t w = mask_keep4(mrow, key0, nkv);
#pragma unroll
    for (int i = 0; i < 4; ++i) bias[i] = ((w >> (8 * i)) & 0xffu) ? 0.f : -INFINITY;
  } else {
    const uint16_t* m16 = (const uint16_t*)mrow;
    u32x2 w = {0u, 0u};
    if (key0 + 3 < nkv) {
      w = *(const u32x2*)(m16 + key0);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (key0 + i < nkv) w[i >> 1] |= (uint32_t)m16[key0 + i] << (16 * (i & 1));
    }
    bias[0] = lo_f32<Tag>(w[0]) * kLog2e;
    bias[1] = hi_f32<Tag>(w[0]) * kLog2e;
    bias[2] = lo_f32<Tag>(w[1]) * kLog2e;
    bias[3] = hi_f32<Tag>(w[1]) * kLog2e;
  }
}

// One mask value (element `idx` of the mask) as a base-2 bias.
template <class Tag>
__device__ __forceinline__ float mask_bias1(const uint8_t* mask, int mode, int64_t idx) {
  if (mode == ATTN_MASK_BOOL) return mask[idx] ? 0.f : -INFINITY;
  const uint32_t h = ((const uint16_t*)mask)[idx];
  return lo_f32<Tag>(h) * kLog2e;
}

// Columns the matrix products run over for head dimension D: D itself,
// except that D = 80 (not a whole number of 32-column output blocks) is
// computed as 96 with the last two 16-byte chunks of every row zero.
constexpr int compute_dim(int D) { return D == 80 ? 96 : D; }

// A buffer offset past every tile's buffer size: such a copy reads zeros.
constexpr uint32_t kPadOffset = 0x80000000u;

// Hardware hands consecutive workgroup ids to the 8 XCDs in turn.  Renumber
// so that each XCD receives a contiguous range of logical tiles: the query
// tiles of one head then share that XCD's L2 for their K/V stream.
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int q = total >> 3, r = total & 7;
  const int x = bid & 7, s = bid >> 3;
  return (x < r ? x * (q + 1) : r * (q + 1) + (x - r) * q) + s;
}

// Causal grids, whose tiles differ in length: workgroup j of a launch of
// `total` = count x ntiles tiles (tile index fastest in the logical order)
// takes logical tile (j % count) * ntiles + j / count, so the launch runs
// tile index 0 of every head first, then index 1, and so on.  The caller
// orders tile indices longest first.  Dealt round-robin over the 8 XCDs,
// every XCD then gets an equal share of each length and runs its share
// longest first; xcd_remap would give each XCD a contiguous range of heads
// instead, whose long tiles some XCDs would reach only late.
__device__ __forceinline__ int longest_first(int j, int ntiles, int total) {
  const int count = total / ntiles;
  return (j % count) * ntiles + j / count;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposing LDS read: in each 16-lane group, lane i receives element i%4 of
// the 4-element (8-byte) words addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const uint16_t* p) {
  typedef short i16x4 __attribute__((ext_vector_type(4)));
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(u32x2, r);
}

// Both halves of the wave exchange a value; the max (sum) of the two results
// is the max (sum) over lanes l and l^32, identical in both lanes.
__device__ __forceinline__ float pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// Max over the 64 lanes of a wave, in every lane.
__device__ __forceinline__ float wave_max(float x) {
  x = pair_max(x);
#pragma unroll
  for (int o = 16; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}

// LDS swizzles.  gfx950 serves a 16-byte LDS read 16 lanes (256 bytes, all
// 64 banks) at a time and an 8-byte read 32 lanes at a time, so a pattern is
// conflict-free when those lanes cover 16 distinct 16-byte bank groups.
//  * K operand reads: the 16 lanes of a group read the same chunk of 16
//    consecutive key rows.  With 256-byte rows (D = 128) the chunk is XORed
//    with r & 15; with 128-byte rows (D = 64) two rows share the 64 banks and
//    the chunk is XORed with (r >> 1) & 7.
//  * V^T operand reads (transposing, 8 bytes per lane): 32 lanes read 4 keys
//    x 64 contiguous bytes.  With 256-byte rows the 4 keys go to 4 disjoint
//    64-byte quarters (XOR 4 * (r & 3)); with 128-byte rows keys r and r + 2
//    share banks and are separated by XOR 4 * ((r >> 1) & 1).
//  Rows of 512 bytes (D = 256) start on bank 0 like 256-byte rows and use
//  the same two swizzles.  Rows of 192 bytes (D = 96, 12 chunks) start on
//  bank groups 0, 12, 8, 4 for r % 4 = 0..3: XOR-ing the chunk with
//  (r >> 2) & 3 (which keeps it below 12) spreads 16 consecutive rows over
//  all 16 groups, and 4 consecutive keys already cover four disjoint
//  quarters for the transposing reads.
//  Rows of 384 bytes (D = 192, 24 chunks) start on bank group 0 or 8 for
//  even and odd r, as 128-byte rows do, and take their swizzles: XOR-ing
//  the chunk with (r >> 1) & 7 (row reads) or 4 * ((r >> 1) & 1)
//  (transposing reads) keeps it in its aligned group of 8, so below 24.
template <int D>
__device__ __forceinline__ int k_swz(int r) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256,
                "K swizzles cover D = 64, 96, 128, 192, 256");
  return D == 192 ? ((r >> 1) & 7)
         : D >= 128 ? (r & 15)
         : D == 96  ? ((r >> 2) & 3)
                    : ((r >> 1) & 7);
}
template <int D>
__device__ __forceinline__ int v_swz(int r) {
  static_assert(D == 64 || D == 96 || D == 128 || D == 192 || D == 256,
                "transposed-read swizzles cover D = 64, 96, 128, 192, 256");
  return D == 192 ? 4 * ((r >> 1) & 1)
         : D >= 128 ? 4 * (r & 3)
         : D == 96  ? 0
                    : 4 * ((r >> 1) & 1);
}

// Buffer resource word 3 for raw (untyped, stride 0) buffer loads on gfx9.
constexpr int kRawBufferFlags = 0x00020000;

using attn_tiles::kWavesPerSimd;

// Copy 16 bytes per lane from a buffer into LDS: lane i writes lds + 16 i
// (lds wave-uniform).  Offsets at or beyond the buffer's size read zero.
__device__ __forceinline__ void buf2lds16(__amdgpu_buffer_rsrc_t r, uint16_t* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

}  // namespace

// Host side, defined in attn_fwd.hip.
namespace attn_host {
// ATTN_OK when the current device is a gfx950 (its CU count in *cus), else
// ATTN_EUNSUPPORTED or ATTN_EHIP.
int check_device(int* cus);
// Records the hipError_t behind an ATTN_EHIP / ATTN_ENOMEM return.
void set_last_hip_error(int e);
// Stream-ordered workspace on `st`, from the library's memory pool of the
// current device (hipMallocFromPoolAsync; the pool keeps its memory between
// calls, see attn_workspace_pool).  With the environment
// variable ATTN_FAIL_WORKSPACE set to 1 the request fails with
// hipErrorOutOfMemory without allocating: failure injection for tests of
// the ATTN_ENOMEM paths (read at every call; nothing has been launched
// when a workspace request fails).
hipError_t workspace_alloc(void** p, size_t bytes, hipStream_t st);
// How a call on the D = 128 narrow tiles (256 query rows, 64-key tiles)
// covers its query tiles: tiles [0, first_split) whole, the rest cut into
// `splits` key ranges of split_len keys whose rows [row0, rows) are merged.
struct NarrowPlan {
  int n_qtiles, splits, split_len;
  long long tiles, first_split, row0, rows;
};
void narrow_plan(int B, int Hq, int Nq, int Nkv, int D, int causal, int num_splits, int cus,
                 NarrowPlan* out);
}  // namespace attn_host

#endif  // ATTN_COMMON_H_
