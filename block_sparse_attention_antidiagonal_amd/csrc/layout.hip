// Cluster layout (stable counting sort of labels) and per-cluster centroids.
//
// Layout: "Partition the Support, Reconstruct the Residual" (summary page), group-major
// permutation of Q, K, V.  Centroids: "Sparse-block compensation", section "SVG-EAR --
// centroid compensation" (key and value means of each cluster, cluster size n_c).
#include "layout.hpp"

namespace bsa {
namespace {

// Centroids: one workgroup per (cluster, batch x K/V head); 16 lanes cover a row of D=128
// (8 elements each), 16 rows in flight per pass.
template <typename T, int D>
__global__ __launch_bounds__(256) void centroid_kernel(const T* __restrict__ K, const T* __restrict__ V, int S,
                                                        const int32_t* __restrict__ perm,
                                                        const int32_t* __restrict__ offsets, int C,
                                                        float* __restrict__ Kbar, float* __restrict__ Vbar) {
  constexpr int kLanesPerRow = D / 8;          // 8 or 16
  constexpr int kRowsPerPass = 256 / kLanesPerRow;  // 32 or 16
  const int c = blockIdx.x;
  const size_t bh = blockIdx.y;
  const int lo = offsets[c], hi = offsets[c + 1];
  const int sub = threadIdx.x % kLanesPerRow, rr = threadIdx.x / kLanesPerRow;
  const T* Kh = K + bh * static_cast<size_t>(S) * D;
  const T* Vh = V + bh * static_cast<size_t>(S) * D;
  float ka[8] = {}, va[8] = {};
  // Rows go kBatch passes at a time: their cluster-order token indices first, then all their
  // K and V loads, so that 2 kBatch row loads per thread are in flight; the sums take the rows
  // in the same order as one pass at a time would.
  constexpr int kBatch = 4;
  for (int r0 = lo + rr; r0 < hi; r0 += kBatch * kRowsPerPass) {
    int tok[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const int r = r0 + i * kRowsPerPass;
      tok[i] = r < hi ? perm[r] : -1;
    }
    float kx[kBatch][8], vx[kBatch][8];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      const bool ok = tok[i] >= 0 && tok[i] < S;
      const size_t off = static_cast<size_t>(ok ? tok[i] : 0) * D + sub * 8;
      if constexpr (sizeof(T) == 2) {
        uint4 kq = make_uint4(0u, 0u, 0u, 0u), vq = make_uint4(0u, 0u, 0u, 0u);
        if (ok) {
          kq = *reinterpret_cast<const uint4*>(Kh + off);
          vq = *reinterpret_cast<const uint4*>(Vh + off);
        }
        const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w}, vw[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          kx[i][2 * j] = __uint_as_float(kw[j] << 16);
          kx[i][2 * j + 1] = __uint_as_float(kw[j] & 0xffff0000u);
          vx[i][2 * j] = __uint_as_float(vw[j] << 16);
          vx[i][2 * j + 1] = __uint_as_float(vw[j] & 0xffff0000u);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          kx[i][j] = ok ? to_f32(Kh[off + j]) : 0.0f;
          vx[i][j] = ok ? to_f32(Vh[off + j]) : 0.0f;
        }
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (tok[i] < 0 || tok[i] >= S) continue;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        ka[j] += kx[i][j];
        va[j] += vx[i][j];
      }
    }
  }
  __shared__ float red[2][kRowsPerPass][D];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    red[0][rr][sub * 8 + i] = ka[i];
    red[1][rr][sub * 8 + i] = va[i];
  }
  __syncthreads();
  const int n = hi - lo;
  const float inv = n > 0 ? 1.0f / static_cast<float>(n) : 0.0f;
  for (int e = threadIdx.x; e < 2 * D; e += blockDim.x) {
    const int which = e / D, d = e % D;
    float s = 0.0f;
    for (int j = 0; j < kRowsPerPass; ++j) s += red[which][j][d];
    float* out = which == 0 ? Kbar : Vbar;
    out[(bh * C + c) * D + d] = s * inv;
  }
}

// Member of cluster position k in the middle-out order of a cluster of n members: m = n / 2
// first, then m-1, m+1, m-2, m+2, ... while both sides last, then the longer side outwards.
__device__ __forceinline__ int middle_out_member(int n, int k) {
  const int m = n / 2, below = m, above = n - 1 - m;
  if (k == 0) return m;
  const int both = below < above ? below : above;
  const int j = k - 1;
  if (j < 2 * both) return (j % 2 == 0) ? m - (j / 2 + 1) : m + (j / 2 + 1);
  const int d = both + 1 + (j - 2 * both);
  return below > above ? m - d : m + d;
}

// Probe rows of every layout from its cluster layout (the rule of bsa_select_probe_rows, the
// members in the layout's stable order), one workgroup per layout.  Cluster sizes and the list
// of non-empty clusters (a block scan) go to LDS; a partial round (fewer probes than non-empty
// clusters: one probe from each of M evenly spaced ones) is taken by M threads at once; full
// rounds (round r takes member r, middle-out, of every cluster with more than r members, in
// cluster order) are walked by one thread over the LDS copy.  Dynamic LDS: 2 C + 256 ints.
constexpr int kSelThreads = 256;
__global__ __launch_bounds__(kSelThreads) void select_probes_kernel(int S, int C, int M,
                                                                    const int32_t* __restrict__ perm,
                                                                    const int32_t* __restrict__ offsets,
                                                                    int32_t* __restrict__ probe_idx,
                                                                    float* __restrict__ weights) {
  extern __shared__ int32_t sel_lds[];
  int32_t* n_s = sel_lds;           // [C] cluster sizes
  int32_t* ne_s = sel_lds + C;      // [C] the non-empty clusters in order
  int32_t* part = sel_lds + 2 * C;  // [kSelThreads] scan of per-thread non-empty counts
  const size_t p = blockIdx.x;
  const int t = threadIdx.x;
  const int32_t* off = offsets + p * (C + 1);
  const int32_t* pp = perm + p * S;
  int32_t* idx = probe_idx + p * M;
  float* w = weights + p * M;
  const int per = (C + kSelThreads - 1) / kSelThreads, c0 = t * per, c1 = min(C, c0 + per);
  int mine = 0;
  for (int a = c0; a < c1; ++a) {
    const int n = off[a + 1] - off[a];
    n_s[a] = n;
    mine += n > 0 ? 1 : 0;
  }
  part[t] = mine;
  __syncthreads();
  for (int d = 1; d < kSelThreads; d <<= 1) {  // inclusive scan of the counts
    const int add = t >= d ? part[t - d] : 0;
    __syncthreads();
    part[t] += add;
    __syncthreads();
  }
  int rank = part[t] - mine;
  for (int a = c0; a < c1; ++a)
    if (n_s[a] > 0) ne_s[rank++] = a;
  const int nne = part[kSelThreads - 1];
  __syncthreads();
  if (M < nne) {
    for (int j = t; j < M; j += kSelThreads) {
      const int a = ne_s[static_cast<int>(floor((j + 0.5) * static_cast<double>(nne) / M))];
      idx[j] = pp[off[a] + middle_out_member(n_s[a], 0)];
      w[j] = static_cast<float>(n_s[a]);  // |G_a| / 1
    }
  } else if (t == 0) {
    int largest = 0;
    for (int a = 0; a < C; ++a) largest = max(largest, n_s[a]);
    int taken = 0, R = 0, a_last = 0;  // the last probe comes from cluster a_last in round R
    for (int r = 0; r < largest && taken < M; ++r)
      for (int a = 0; a < C && taken < M; ++a)
        if (n_s[a] > r) {
          idx[taken++] = pp[off[a] + middle_out_member(n_s[a], r)];
          R = r;
          a_last = a;
        }
    // Weights |G_a| / m_a, m_a = the rounds cluster a took part in: every round before R it had
    // members for, and round R if it came up before the last probe.
    int k = 0;
    for (int r = 0; r < largest && k < M; ++r)
      for (int a = 0; a < C && k < M; ++a)
        if (n_s[a] > r) {
          const int m_a = min(n_s[a], R) + ((n_s[a] > R && a <= a_last) ? 1 : 0);
          w[k++] = static_cast<float>(static_cast<double>(n_s[a]) / m_a);
        }
    for (; taken < M; ++taken) {  // fewer members than probes (labels outside [0, C)): padding
      idx[taken] = 0;
      w[taken] = 0.0f;
    }
  }
  __syncthreads();  // the weights are written (global memory, visible to the workgroup)
  if (t == 0) {  // normalized to sum to 1
    double total = 0.0;
    for (int j = 0; j < M; ++j) total += static_cast<double>(w[j]);
    for (int j = 0; j < M; ++j) w[j] = total > 0.0 ? static_cast<float>(static_cast<double>(w[j]) / total) : 0.0f;
  }
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_cluster_layout_workspace_size(int P, int S, int C, size_t* bytes) {
  if (!bytes || P < 1 || S < 1 || C < 1) return BSA_E_ARG;
  if (C > kMaxC || P > 65535) return BSA_E_UNSUPPORTED;
  *bytes = static_cast<size_t>(P) * layout_chunks(S) * static_cast<size_t>(C) * sizeof(int32_t);
  return BSA_OK;
}

extern "C" bsa_status bsa_cluster_layout(int P, const int32_t* labels, int S, int C, int32_t* perm, int32_t* offsets,
                                         int32_t* counts, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  bsa_status st = bsa_cluster_layout_workspace_size(P, S, C, &need);
  if (st != BSA_OK) return st;
  if (!labels || !perm || !offsets || !counts) return BSA_E_ARG;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  launch_layouts(labels, S, C, P, static_cast<int32_t*>(ws), perm, offsets, counts, stream);
  return launch_status();
}

extern "C" bsa_status bsa_select_probe_rows_layouts(int P, int S, int C, int M, const int32_t* perm,
                                                    const int32_t* offsets, int32_t* probe_idx, float* weights,
                                                    hipStream_t stream) {
  if (!perm || !offsets || !probe_idx || !weights || P < 1 || S < 1 || C < 1 || M < 1 || M > S) return BSA_E_ARG;
  if (C > kMaxC || P > 65535) return BSA_E_UNSUPPORTED;
  const size_t lds = (2 * static_cast<size_t>(C) + kSelThreads) * sizeof(int32_t);
  hipFuncSetAttribute(reinterpret_cast<const void*>(select_probes_kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                      static_cast<int>(lds));
  hipLaunchKernelGGL(select_probes_kernel, dim3(P), dim3(kSelThreads), lds, stream, S, C, M, perm, offsets, probe_idx,
                     weights);
  return launch_status();
}

extern "C" bsa_status bsa_centroids(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V,
                                    const int32_t* perm, const int32_t* offsets, int C, float* Kbar, float* Vbar,
                                    hipStream_t stream) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  if (B < 1 || Hkv < 1 || S < 1 || C < 1) return BSA_E_ARG;
  if (!K || !V || !perm || !offsets || !Kbar || !Vbar) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (static_cast<long long>(B) * Hkv > 65535) return BSA_E_UNSUPPORTED;
  const dim3 grid(C, B * Hkv);
  if (dtype == BSA_BF16) {
    if (D == 128)
      hipLaunchKernelGGL((centroid_kernel<bf16_t, 128>), grid, dim3(256), 0, stream, static_cast<const bf16_t*>(K),
                         static_cast<const bf16_t*>(V), S, perm, offsets, C, Kbar, Vbar);
    else
      hipLaunchKernelGGL((centroid_kernel<bf16_t, 64>), grid, dim3(256), 0, stream, static_cast<const bf16_t*>(K),
                         static_cast<const bf16_t*>(V), S, perm, offsets, C, Kbar, Vbar);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((centroid_kernel<float, 128>), grid, dim3(256), 0, stream, static_cast<const float*>(K),
                         static_cast<const float*>(V), S, perm, offsets, C, Kbar, Vbar);
    else
      hipLaunchKernelGGL((centroid_kernel<float, 64>), grid, dim3(256), 0, stream, static_cast<const float*>(K),
                         static_cast<const float*>(V), S, perm, offsets, C, Kbar, Vbar);
  }
  return launch_status();
}
