// Host-side sizing of the kernels' grids and workspaces, shared by the
// launchers and the C ABI's workspace arithmetic. No device code: the same
// file builds into the library and into the host-only checks of the ABI.
#include "kvc_internal.h"

namespace kvc {

int csr_blocks(int L) { return (L + CSR_BLOCK_TOKENS - 1) / CSR_BLOCK_TOKENS; }

int fused_blocks_per_head(int heads) { return heads >= 128 ? 2 : (heads >= 64 ? 4 : 8); }

// 4 (64 tokens) while the budget's 64-token slices give each of the P blocks
// at least 8 (one per wave), then 2 and 1.
int fused_slice_tiles(int B, int P) {
  if ((B + 63) / 64 >= 8 * P) return 4;
  if ((B + 31) / 32 >= 8 * P) return 2;
  return 1;
}

// 64-token multiples, at most DEC_MAX_PAIRS / G splits.
void dense_split(int n, int G, int* nsplit, int* T) {
  int ns = (n + 511) / 512;
  const int cap = DEC_MAX_PAIRS / G;
  if (ns > cap) ns = cap;
  if (ns < 1) ns = 1;
  int t = (n + ns - 1) / ns;
  t = (t + 63) / 64 * 64;
  *T = t;
  *nsplit = (n + t - 1) / t;
}

bool window_kmeans_fits(int m, int nc) { return nc <= WINDOW_KMEANS_MAX_C && (size_t)m * sizeof(int) <= 64 * 1024; }

}  // namespace kvc
