// attn_tiles.h -- the forward's tile table, shared by the kernels and the
// host planner.  Plain C++ (no HIP), so the planner also builds on the host
// alone.
#ifndef ATTN_TILES_H_
#define ATTN_TILES_H_

namespace attn_tiles {

// Waves per SIMD that every kernel is compiled for: each wave may use up to
// 256 of the SIMD's 512 vector registers (arch + accumulation).
constexpr int kWavesPerSimd = 2;

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
// two zero chunks per row.  D = 192 with DV = 128 (24-chunk K rows, 16-chunk
// V rows): 64-key tiles (the copies of a 32-key K tile would not split over
// 8 waves), 32-row waves, the single-buffered pipeline and 4 of the 12 Q^T
// chunks in LDS (double-buffered scores and all of Q^T in registers spill).
// Masked calls at D = 128 take that pipeline too (same 256 rows and 64-key
// tiles as the narrow tile): the mask step's registers then fit.
struct TileCfg {
  int NW, QB, BN, QL;
  bool SB;
  bool PD;  // double-buffered pipeline with P V deferred by one step (see the kernel)
  constexpr int BM() const { return NW * QB * 32; }
  constexpr int resident_per_cu() const { return 4 * kWavesPerSimd / NW; }
};
// Short query ranges at D = 128 (decode, or the packed query heads of a
// GQA group: at most 128 rows) take a 4-wave, 128-row tile: two workgroups
// per CU then stream two key ranges at once, and waves without rows skip
// the arithmetic.
enum {
  kCfgD64Narrow = 0,
  kCfgD64Wide = 1,
  kCfgD128Narrow = 2,
  kCfgD128Wide = 3,
  kCfgD256 = 4,
  kCfgD96 = 5,
  kCfgD192 = 6,
  kCfgD128Masked = 7,
  kCfgD128Decode = 8
};
constexpr TileCfg kCfgs[9] = {{4, 1, 64, 0, false, true},
                              {4, 2, 32, 0, false, false},
                              {8, 1, 64, 0, false, false},
                              {8, 2, 32, 3, true, false},
                              {8, 1, 32, 8, true, false},
                              {4, 1, 64, 0, false, false},
                              {8, 1, 64, 4, true, false},
                              {8, 1, 64, 4, true, false},
                              {4, 1, 64, 0, false, false}};

}  // namespace attn_tiles

#endif  // ATTN_TILES_H_
