// Host-side helpers of the C ABI: status text, probe-row selection and sliding-tile labels.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <vector>

#include "bsa.h"

extern "C" const char* bsa_status_string(int status) {
  switch (status) {
    case BSA_OK: return "ok";
    case BSA_E_ARG: return "invalid argument (null pointer or scalar out of range)";
    case BSA_E_SHAPE: return "inconsistent sizes";
    case BSA_E_DTYPE: return "unknown element type";
    case BSA_E_UNSUPPORTED: return "request not supported by this library";
    case BSA_E_WORKSPACE: return "workspace missing or too small";
    case BSA_E_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

extern "C" int bsa_abi_version(void) { return 4; }

// "Sparse-block compensation", API table (select_probe_rows: head-agnostic, round-robin over
// query clusters, weights |G_a| / m_a) and "Deviations from the papers" (middle-out member;
// weights normalized to 1).  "Partition the Support, Reconstruct the Residual": probes are
// stratified across query groups, so a single partial round is spread over the clusters.
extern "C" bsa_status bsa_select_probe_rows(const int32_t* labels, int S, int C, int M, int32_t* probe_idx,
                                            float* weights) {
  if (!labels || !probe_idx || !weights || S < 1 || C < 1 || M < 1 || M > S) return BSA_E_ARG;
  std::vector<std::vector<int32_t>> members(C);
  for (int i = 0; i < S; ++i) {
    if (labels[i] < 0 || labels[i] >= C) return BSA_E_ARG;
    members[labels[i]].push_back(i);
  }
  // Middle-out order inside each cluster: m, m-1, m+1, m-2, m+2, ... with m = n / 2.
  std::vector<std::vector<int32_t>> queue(C);
  for (int a = 0; a < C; ++a) {
    const int n = static_cast<int>(members[a].size());
    const int m = n / 2;
    if (n == 0) continue;
    queue[a].push_back(members[a][m]);
    for (int d = 1; static_cast<int>(queue[a].size()) < n; ++d) {
      if (m - d >= 0) queue[a].push_back(members[a][m - d]);
      if (m + d < n) queue[a].push_back(members[a][m + d]);
    }
  }
  std::vector<int> nonempty;
  for (int a = 0; a < C; ++a)
    if (!members[a].empty()) nonempty.push_back(a);
  const int nne = static_cast<int>(nonempty.size());
  std::vector<int> visit;
  if (M >= nne) {
    visit = nonempty;
  } else {
    for (int j = 0; j < M; ++j) {
      const int k = static_cast<int>(std::floor((j + 0.5) * static_cast<double>(nne) / M));
      visit.push_back(nonempty[k]);
    }
  }
  std::vector<int> cursor(C, 0), from;
  int taken = 0;
  while (taken < M) {
    for (int a : visit) {
      if (taken == M) break;
      if (cursor[a] < static_cast<int>(queue[a].size())) {
        probe_idx[taken++] = queue[a][cursor[a]++];
        from.push_back(a);
      }
    }
    visit = nonempty;
  }
  double total = 0.0;
  std::vector<double> w(M);
  for (int p = 0; p < M; ++p) {
    const int a = from[p];
    w[p] = static_cast<double>(members[a].size()) / static_cast<double>(cursor[a]);
    total += w[p];
  }
  for (int p = 0; p < M; ++p) weights[p] = static_cast<float>(w[p] / total);
  return BSA_OK;
}

// "Sparse-block compensation", API table: labels matching Sliding Tile Attention tiles.
extern "C" bsa_status bsa_tile_labels(int T, int H, int W, int tt, int th, int tw, int chunk, int32_t* labels) {
  if (!labels || T < 1 || H < 1 || W < 1 || tt < 1 || th < 1 || tw < 1 || chunk < 0) return BSA_E_ARG;
  const long long S = static_cast<long long>(T) * H * W;
  if (S > 0x7fffffffLL) return BSA_E_UNSUPPORTED;
  const int ny = (H + th - 1) / th, nx = (W + tw - 1) / tw;
  std::vector<int32_t> tile(static_cast<size_t>(S));
  for (int t = 0; t < T; ++t)
    for (int y = 0; y < H; ++y)
      for (int x = 0; x < W; ++x) tile[(static_cast<size_t>(t) * H + y) * W + x] = ((t / tt) * ny + y / th) * nx + x / tw;
  if (chunk == 0) {
    std::copy(tile.begin(), tile.end(), labels);
    return BSA_OK;
  }
  // Tile-major rank: count tokens per tile, then place tokens in raster order within tiles.
  const int ntiles = ((T + tt - 1) / tt) * ny * nx;
  std::vector<long long> start(static_cast<size_t>(ntiles) + 1, 0);
  for (long long i = 0; i < S; ++i) ++start[tile[i] + 1];
  for (int k = 0; k < ntiles; ++k) start[k + 1] += start[k];
  for (long long i = 0; i < S; ++i) labels[i] = static_cast<int32_t>(start[tile[i]]++ / chunk);
  return BSA_OK;
}

// Sliding-tile block mask over the cells of an nT x nH x nW raster grid grouped into tiles of
// (tt, th, tw) cells: cell i keeps cell j when j's tile lies in the window of i's tile; along
// each axis the window of `w` tiles around coordinate a starts at min(max(a - w/2, 0),
// max(n - w, 0)) for n tiles on that axis.
extern "C" bsa_status bsa_sliding_tile_mask(int nT, int nH, int nW, int tt, int th, int tw, int wt, int wh, int ww,
                                            uint8_t* keep) {
  if (!keep || nT < 1 || nH < 1 || nW < 1 || tt < 1 || th < 1 || tw < 1 || wt < 1 || wh < 1 || ww < 1)
    return BSA_E_ARG;
  const long long N = static_cast<long long>(nT) * nH * nW;
  if (N > 65535) return BSA_E_UNSUPPORTED;
  const int n[3] = {(nT + tt - 1) / tt, (nH + th - 1) / th, (nW + tw - 1) / tw};
  const int w[3] = {wt, wh, ww};
  std::vector<int> coord[3];
  for (int a = 0; a < 3; ++a) coord[a].resize(static_cast<size_t>(N));
  for (int t = 0; t < nT; ++t)
    for (int y = 0; y < nH; ++y)
      for (int x = 0; x < nW; ++x) {
        const size_t i = (static_cast<size_t>(t) * nH + y) * nW + x;
        coord[0][i] = t / tt;
        coord[1][i] = y / th;
        coord[2][i] = x / tw;
      }
  for (long long i = 0; i < N; ++i) {
    int lo[3];
    for (int a = 0; a < 3; ++a) lo[a] = std::min(std::max(coord[a][i] - w[a] / 2, 0), std::max(n[a] - w[a], 0));
    uint8_t* row = keep + static_cast<size_t>(i) * N;
    for (long long j = 0; j < N; ++j) {
      bool in = true;
      for (int a = 0; a < 3; ++a) in = in && coord[a][j] >= lo[a] && coord[a][j] < lo[a] + w[a];
      row[j] = in ? 1 : 0;
    }
  }
  return BSA_OK;
}
