// Host-side check of the grouped GEMMs' workgroup-to-tile maps, compiled from
// the library's own header: over the launch grid each map must hand out
// every tile exactly once and nothing out of range.
#include <cstdio>
#include <vector>

#include "moe_internal.h"

using namespace moe;

static int check(const char* what, int total, int grid, int (*tile_of)(int, const int*), const int* arg) {
  std::vector<int> seen(total, 0);
  for (int wg = 0; wg < grid; ++wg) {
    const int t = tile_of(wg, arg);
    if (t < -1 || (t >= total && t != -1)) {
      // the XCD-blocked plan order leaves tiles past the plan to the kernel's own bound check
      if (arg[0] == 0 && t >= total) continue;
      printf("%s: workgroup %d -> tile %d of %d\n", what, wg, t, total);
      return 1;
    }
    if (t >= 0 && t < total) seen[t]++;
  }
  for (int i = 0; i < total; ++i)
    if (seen[i] != 1) {
      printf("%s: tile %d handed out %d times (total %d, grid %d)\n", what, i, seen[i], total, grid);
      return 1;
    }
  return 0;
}

static int plan_map(int wg, const int*) { return xcd_tile_of(wg); }
static int wgrad_map(int wg, const int* a) { return wgrad_tile_of(wg, a[1], a[2], a[3]); }

int main() {
  long cases = 0;
  for (int tiles = 1; tiles <= 3000; tiles += (tiles < 300 ? 1 : 97)) {
    const int arg[4] = {0, 0, 0, 0};
    if (check("xcd_tile_of", tiles, xcd_grid(tiles), plan_map, arg)) return 1;
    ++cases;
  }
  for (int E = 0; E <= 1024; E += (E < 20 ? 1 : (E < 200 ? 13 : 205)))
    for (int tpr : {0, 1, 3, 8, 88, 165})
      for (int tps : {0, 1, 7, 8, 9, 165, 300}) {
        const int total = E * tpr + tps;
        if (total == 0) continue;
        const int arg[4] = {1, E, tpr, tps};
        if (check("wgrad_tile_of", total, wgrad_grid(E, tpr, tps), wgrad_map, arg)) return 1;
        ++cases;
      }
  printf("ok %ld cases\n", cases);
  return 0;
}
