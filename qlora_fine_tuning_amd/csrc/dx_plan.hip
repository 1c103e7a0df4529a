// Host-side plan of the input-gradient grid (no device code): output tiles, the split of the
// contraction N for outputs with few tiles, and the workspace the split partials need.  Kept
// apart from the kernel source so that the kernel's recorded HBM counters (keyed by a hash of
// that source) stay valid when this launch policy changes.
#include "common.hpp"
#include "launch.hpp"

namespace lora {

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return kNormCUs;
  return n;
}

int dx_tiles(int64_t M, int64_t K) { return (int)(((M + kTile - 1) / kTile) * ((K + kTile - 1) / kTile)); }

// Number of N ranges per output tile (1..32, at least 8 steps of 64 each), minimising an
// estimate in tile-steps (x 256): rounds of 256 resident workgroups x steps per unit, plus the
// units' partials, each a 256 KB fp32 store that the tile's last unit reads back, at about 40
// tile-steps per unit on each CU (measured on the QLoRA FFN input gradient, 320 tiles x 432
// steps: S = 2, 3, 4, 8 took 1.13, 1.09, 1.15, 1.73 ms; a flat 4 steps per unit chose 4).  More
// than 8 ranges only pay for a handful of tiles over a long N (a 256-token chunk of an LM head's
// gradient: 16 tiles, 2000 steps, S = 16).
int dx_splits(int64_t M, int64_t N, int64_t K, int R) {
  const int64_t tiles = dx_tiles(M, K), steps = N / kStep;
  int best = 1;
  (void)R;
  int64_t best_cost = ((tiles + 255) / 256) * steps * 256;
  for (int64_t s = 2; s <= 32 && steps / s >= 8; ++s) {
    const int64_t cost = ((tiles * s + 255) / 256) * ((steps + s - 1) / s) * 256 + 40 * tiles * s;
    if (cost < best_cost) best = (int)s, best_cost = cost;
  }
  return best;
}

// How many tiles (the first ones) take S + 1 units instead of S: the count that makes the units a
// whole number of rounds of the persistent grid, used only when those (S + 1)-way units also
// fill whole rounds by themselves (so they form the last round and every CU runs the same
// number of steps) and still have at least 8 steps each; else 0.  The QLoRA FFN input gradient:
// 320 tiles x 3 = 960 units on 256 CUs, 64 tiles x 4 = 256 units fill the fourth round (1.07 ->
// ~1.0 ms measured).
int dx_split_hi(int64_t M, int64_t N, int64_t K, int R) {
  const int s = dx_splits(M, N, K, R);
  if (s < 2) return 0;
  const int64_t tiles = dx_tiles(M, K), units = tiles * s;
  const int64_t cus = device_cus() & ~7;
  if (cus <= 0 || units <= cus || units % cus == 0) return 0;
  const int64_t hi = cus - units % cus;
  if (hi > tiles || (hi * (s + 1)) % cus != 0 || (N / kStep) / (s + 1) < 8) return 0;
  return (int)hi;
}

size_t dx_part_bytes(int64_t M, int64_t N, int64_t K, int R) {
  const int s = dx_splits(M, N, K, R);
  if (s == 1) return 0;
  const int rp = R <= 16 ? 16 : (R <= 32 ? 32 : 64);
  return (size_t)dx_tiles(M, K) * (s + (dx_split_hi(M, N, K, R) > 0)) * dx_slot_bytes(rp);
}

}  // namespace lora
