// Host-only launch planning of the expert GEMMs: which kernel a shape runs
// on and the limits that kernel relies on.  Plain C++ (no HIP), so the
// limits can be checked on the host alone.
#pragma once

#include <stdint.h>

#include <algorithm>

namespace moe {
namespace plan {

inline long cdiv(long a, long b) { return (a + b - 1) / b; }

// Rows per m-tile of the many-row kernel, its n-tile widths per mode (gate
// and up rows are interleaved in one 256-row weight tile, so a gate/up tile
// writes 128 H columns; a down tile writes 256 output columns) and the
// number of tiles one workgroup can track (four 64-lane registers).
constexpr int kBigTileRows = 256;
constexpr int kBigGateUpCols = 128;
constexpr int kBigDownCols = 256;
constexpr long kBigMaxTilesPerWg = 256;
constexpr int kBigMaxGroups = 1024;
// The first m-tile of a tile's group is packed into 22 bits.
constexpr long kBigMaxMTiles = 1l << 22;

// Largest m-tile count of ngroups groups holding at most `rows` rows in
// total: every group that holds any row takes one m-tile, and every further
// 256 rows one more.
inline long big_mtiles_max(long rows, long ngroups) {
  if (rows <= ngroups) return rows;
  return ngroups + (rows - ngroups) / kBigTileRows;
}

// n-tiles of the many-row kernel per m-tile: mode 1 gate/up, mode 2 down.
inline long big_ntiles(int mode, long d_model, long d_ff) {
  return mode == 1 ? cdiv(d_ff, kBigGateUpCols) : cdiv(d_model, kBigDownCols);
}

// Experts with 257..320 rows run on a second tile shape, 320 x 192 (gate/up
// tiles write 96 H columns, down tiles 192 output columns), one tile each
// instead of two 256-row tiles that would each stream the weight slice.
constexpr int kR320Lo = 257, kR320Hi = 320;
inline long big320_ntiles(int mode, long d_model, long d_ff) {
  return mode == 1 ? cdiv(d_ff, 96) : cdiv(d_model, 192);
}

// Upper bound on the work items one workgroup of a G-workgroup grid runs.
// The kernel's items are the tiles, except that a last round at most half
// full has its tiles cut into f <= G / rem row slices; then the items are
// full + rem * f <= full + G, so every workgroup runs at most ceil(tiles/G).
inline long big_items_per_wg_max(long tiles, long G) { return cdiv(tiles, G); }

// A tall-tile shape: rows per expert (T*k/E) of at least 32 make tall tiles
// worth it if there are enough of them to spread over the chip; with 64 or
// more rows per FFN expert they are used regardless (16-row tiles would
// re-read every weight slice 4 or more times).
constexpr long kMinTiles = 64;
inline bool ffn_tall_tiles(long T, long top_k, long n_ffn, long n_zero, long d_model,
                           long d_ff) {
  const long E = n_ffn + n_zero;
  const long Tk = T * top_k;
  return (Tk / E >= 32 && cdiv(Tk, 128) * cdiv(std::min(d_ff, d_model), 128) >= kMinTiles) ||
         Tk / n_ffn >= 64;
}

// Workgroups of a many-row launch are G (one per CU) times the smallest
// multiple m that keeps every workgroup within kBigMaxTilesPerWg items for
// the worst spread of rows over experts, in both modes.  One workgroup fills
// a CU's LDS, so a grid of G * m runs as m waves of persistent workgroups
// (same work, same tile order within an XCD); the kernel takes its grid size
// from the launch.  Returns 0 when no m up to kBigMaxGridMult does.
constexpr long kBigMaxGridMult = 64;
inline long big_grid_mult(long T, long top_k, long n_ffn, long d_model, long d_ff, long G) {
  if (G < 1) return 0;
  const long mt = big_mtiles_max(T * top_k, n_ffn);
  const long nt = std::max(big_ntiles(1, d_model, d_ff), big_ntiles(2, d_model, d_ff));
  for (long m = 1; m <= kBigMaxGridMult; ++m)
    if (big_items_per_wg_max(mt * nt, G * m) <= kBigMaxTilesPerWg) return m;
  return 0;
}

// Whether the expert GEMMs of a bf16 shape run on the many-row kernel
// (256x256 direct-to-LDS tiles, with 320x192 ones beside them:
// ffn_use_r320), for G workgroups per wave (big_grid_mult waves).  `gather`:
// gate/up reads x rows through perm (token rows anywhere in x, addressed by
// 32-bit offsets from x, so x must stay below 4 GiB); otherwise token rows
// (x_perm or H) are contiguous per tile and addressed from a 64-bit tile
// base.  Each expert's weights are addressed by 32-bit offsets.
inline bool ffn_use_big(long T, long top_k, long n_ffn, long n_zero, long d_model, long d_ff,
                        bool bf16, bool gather, long G) {
  const long Tk = T * top_k;
  if (!bf16 || !ffn_tall_tiles(T, top_k, n_ffn, n_zero, d_model, d_ff)) return false;
  if (d_model % 128 != 0 || d_ff % 128 != 0) return false;
  if ((uint64_t)d_ff * d_model * 2 >= (1ull << 32)) return false;
  if (gather && (uint64_t)T * d_model * 2 >= (1ull << 32)) return false;
  if (n_ffn > kBigMaxGroups || G < 1) return false;
  // enough tiles to spread over the chip
  const long nt_min = std::min(big_ntiles(1, d_model, d_ff), big_ntiles(2, d_model, d_ff));
  if (cdiv(Tk, kBigTileRows) * nt_min < kMinTiles) return false;
  // every workgroup tracks at most 256 items, in both modes, on a grid of
  // G * big_grid_mult workgroups
  if (big_mtiles_max(Tk, n_ffn) >= kBigMaxMTiles) return false;
  return big_grid_mult(T, top_k, n_ffn, d_model, d_ff, G) > 0;
}

// Whether a many-row shape also uses the 320-row tiles: at most
// min(n_ffn, T*k / 257) groups take one such tile each, and every workgroup
// tracks at most 256 items of that launch too, in both modes, on G
// workgroups (the launch runs on the same G * big_grid_mult grid as the
// 256-row one, which only lowers that count).  (The kernel uses them only
// when the groups in range fill four rounds of the grid.)
inline bool ffn_use_r320(long T, long top_k, long n_ffn, long d_model, long d_ff, long G) {
  const long groups = std::min(n_ffn, T * top_k / kR320Lo);
  if (groups < 1 || G < 1) return false;
  const long nt = std::max(big320_ntiles(1, d_model, d_ff), big320_ntiles(2, d_model, d_ff));
  return big_items_per_wg_max(groups * nt, G) <= kBigMaxTilesPerWg;
}

}  // namespace plan
}  // namespace moe
