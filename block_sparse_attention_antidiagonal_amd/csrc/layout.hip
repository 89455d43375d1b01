// Cluster layout (stable counting sort of labels) and per-cluster centroids.
//
// Layout: "Partition the Support, Reconstruct the Residual" (summary page), group-major
// permutation of Q, K, V.  Centroids: "Sparse-block compensation", section "SVG-EAR --
// centroid compensation" (key and value means of each cluster, cluster size n_c).
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kChunk = 1024;  // tokens per chunk of the counting sort
constexpr int kMaxC = 8192;   // clusters per layout (LDS histogram)

// Per-chunk histograms: hist[chunk][c].
__global__ __launch_bounds__(256) void layout_hist(const int32_t* __restrict__ labels, int S, int C,
                                                    int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxC];
  for (int c = threadIdx.x; c < C; c += blockDim.x) h[c] = 0;
  __syncthreads();
  const int base = blockIdx.x * kChunk;
  for (int i = threadIdx.x; i < kChunk; i += blockDim.x) {
    const int p = base + i;
    if (p < S) {
      const int lab = labels[p];
      if (lab >= 0 && lab < C) atomicAdd(&h[lab], 1);
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < C; c += blockDim.x) hist[static_cast<size_t>(blockIdx.x) * C + c] = h[c];
}

// counts, offsets, and per-chunk bases (hist is rewritten in place as base[chunk][c]).
__global__ __launch_bounds__(1024) void layout_scan(int C, int nchunks, int32_t* __restrict__ hist,
                                                     int32_t* __restrict__ offsets, int32_t* __restrict__ counts) {
  __shared__ int32_t part[1024];
  // Each thread owns a contiguous run of clusters.
  const int per = (C + blockDim.x - 1) / blockDim.x;
  const int c0 = threadIdx.x * per;
  int32_t run = 0;
  for (int c = c0; c < c0 + per && c < C; ++c) {
    int32_t n = 0;
#pragma unroll 8
    for (int k = 0; k < nchunks; ++k) n += hist[static_cast<size_t>(k) * C + c];
    counts[c] = n;
    run += n;
  }
  part[threadIdx.x] = run;
  __syncthreads();
  // Inclusive scan of per-thread totals (Hillis-Steele).
  for (int d = 1; d < static_cast<int>(blockDim.x); d <<= 1) {
    const int32_t add = threadIdx.x >= static_cast<unsigned>(d) ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t off = part[threadIdx.x] - run;
  for (int c = c0; c < c0 + per && c < C; ++c) {
    offsets[c] = off;
    int32_t within = off;
#pragma unroll 8
    for (int k = 0; k < nchunks; ++k) {
      const size_t idx = static_cast<size_t>(k) * C + c;
      const int32_t n = hist[idx];
      hist[idx] = within;
      within += n;
    }
    off = within;
  }
  if (threadIdx.x == blockDim.x - 1) offsets[C] = part[blockDim.x - 1];
}

// Stable scatter: the rank of token p among earlier tokens of its chunk with the same label.
// The chunk is cut into 64-token segments, one wave each: inside a segment, one ballot per
// distinct label gives every lane its rank among earlier lanes and the label's count, which
// the segment lists in LDS; a token's rank adds the counts of its label in earlier segments.
// The work grows with the number of distinct labels per segment (a few for tile labels).
constexpr int kSeg = 64;
constexpr int kSegs = kChunk / kSeg;
__global__ __launch_bounds__(256) void layout_scatter(const int32_t* __restrict__ labels, int S, int C,
                                                       const int32_t* __restrict__ base, int32_t* __restrict__ perm) {
  __shared__ int32_t seg_lab[kSegs][kSeg];  // distinct labels of each segment
  __shared__ int32_t seg_cnt[kSegs][kSeg];  // and their counts
  __shared__ int32_t seg_n[kSegs];
  constexpr int kWaves = 256 / 64;
  const int start = blockIdx.x * kChunk;
  const int n = min(kChunk, S - start);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  int lab_r[kSegs / kWaves], rank_r[kSegs / kWaves];
#pragma unroll
  for (int k = 0; k < kSegs / kWaves; ++k) {
    const int seg = wave + k * kWaves;
    const int i = seg * kSeg + lane;
    int li = i < n ? labels[start + i] : -1;
    if (li < 0 || li >= C) li = -1;
    int rank = 0, nd = 0;
    unsigned long long left = __ballot(li >= 0);
    while (left) {
      const int leader = __ffsll(static_cast<long long>(left)) - 1;
      const int l = __builtin_amdgcn_readlane(li, leader);
      const unsigned long long m = __ballot(li == l);
      if (li == l) rank = __popcll(m & below);
      if (lane == 0) {
        seg_lab[seg][nd] = l;
        seg_cnt[seg][nd] = __popcll(m);
      }
      ++nd;
      left &= ~m;
    }
    if (lane == 0) seg_n[seg] = nd;
    lab_r[k] = li;
    rank_r[k] = rank;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSegs / kWaves; ++k) {
    const int seg = wave + k * kWaves;
    const int li = lab_r[k];
    int pre = 0;
    for (int s2 = 0; s2 < seg; ++s2) {
      const int nd = seg_n[s2];
      for (int d = 0; d < nd; ++d) pre += seg_lab[s2][d] == li ? seg_cnt[s2][d] : 0;
    }
    if (li >= 0) perm[base[static_cast<size_t>(blockIdx.x) * C + li] + pre + rank_r[k]] = start + seg * kSeg + lane;
  }
}

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
  for (int r = lo + rr; r < hi; r += kRowsPerPass) {
    const int tok = perm[r];
    if (tok < 0 || tok >= S) continue;
    const T* kp = Kh + static_cast<size_t>(tok) * D + sub * 8;
    const T* vp = Vh + static_cast<size_t>(tok) * D + sub * 8;
    if constexpr (sizeof(T) == 2) {
      const uint4 kq = *reinterpret_cast<const uint4*>(kp);
      const uint4 vq = *reinterpret_cast<const uint4*>(vp);
      const uint32_t kw[4] = {kq.x, kq.y, kq.z, kq.w}, vw[4] = {vq.x, vq.y, vq.z, vq.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ka[2 * i] += __uint_as_float(kw[i] << 16);
        ka[2 * i + 1] += __uint_as_float(kw[i] & 0xffff0000u);
        va[2 * i] += __uint_as_float(vw[i] << 16);
        va[2 * i + 1] += __uint_as_float(vw[i] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        ka[i] += to_f32(kp[i]);
        va[i] += to_f32(vp[i]);
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

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_cluster_layout_workspace_size(int S, int C, size_t* bytes) {
  if (!bytes || S < 1 || C < 1) return BSA_E_ARG;
  if (C > kMaxC) return BSA_E_UNSUPPORTED;
  const size_t nchunks = (static_cast<size_t>(S) + kChunk - 1) / kChunk;
  *bytes = nchunks * static_cast<size_t>(C) * sizeof(int32_t);
  return BSA_OK;
}

extern "C" bsa_status bsa_cluster_layout(const int32_t* labels, int S, int C, int32_t* perm, int32_t* offsets,
                                         int32_t* counts, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  bsa_status st = bsa_cluster_layout_workspace_size(S, C, &need);
  if (st != BSA_OK) return st;
  if (!labels || !perm || !offsets || !counts) return BSA_E_ARG;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  const int nchunks = (S + kChunk - 1) / kChunk;
  int32_t* hist = static_cast<int32_t*>(ws);
  hipLaunchKernelGGL(layout_hist, dim3(nchunks), dim3(256), 0, stream, labels, S, C, hist);
  hipLaunchKernelGGL(layout_scan, dim3(1), dim3(1024), 0, stream, C, nchunks, hist, offsets, counts);
  hipLaunchKernelGGL(layout_scatter, dim3(nchunks), dim3(256), 0, stream, labels, S, C, hist, perm);
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
