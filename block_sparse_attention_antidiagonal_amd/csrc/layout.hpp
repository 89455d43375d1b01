// Stable counting sort of cluster labels (the cluster layout), for one layout or a batch of
// independent layouts: layout p reads labels[p][S] and writes perm[p][S], offsets[p][C+1],
// counts[p][C], using hist[p][nchunks][C].  Included by every source that sorts labels.
#pragma once

#include "common.hpp"

namespace bsa {
namespace {

constexpr int kChunk = 1024;  // tokens per chunk of the counting sort
constexpr int kMaxC = 8192;   // clusters per layout (LDS histogram)

// Per-chunk histograms: hist[chunk][c].
__global__ __launch_bounds__(256) void layout_hist(const int32_t* __restrict__ labels, int S, int C, int nchunks,
                                                    int32_t* __restrict__ hist) {
  __shared__ int32_t h[kMaxC];
  labels += static_cast<size_t>(blockIdx.y) * S;  // layout blockIdx.y of a batch of layouts
  hist += static_cast<size_t>(blockIdx.y) * nchunks * C;
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
  hist += static_cast<size_t>(blockIdx.x) * nchunks * C;  // layout blockIdx.x of a batch
  offsets += static_cast<size_t>(blockIdx.x) * (C + 1);
  counts += static_cast<size_t>(blockIdx.x) * C;
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

// Stable scatter: a token's place is its chunk's base for its label plus the number of earlier
// tokens of the chunk with the same label.  Wave w owns sub-chunk w (256 tokens, 4 segments
// of 64) and walks its segments in order: one ballot per distinct label of a segment gives
// every lane its rank among the earlier lanes with its label, to which it adds the wave's
// running count of that label (LDS), which the label's first lane then advances.  After all
// waves are done, a token adds the counts of its label in the earlier sub-chunks.  Dynamic
// LDS: 4 C ints.
constexpr int kSub = 256;
__global__ __launch_bounds__(256) void layout_scatter(const int32_t* __restrict__ labels, int S, int C,
                                                       int nchunks, const int32_t* __restrict__ base,
                                                       int32_t* __restrict__ perm) {
  extern __shared__ int32_t sub_counts[];  // [4][C]: running, then total, counts per sub-chunk
  labels += static_cast<size_t>(blockIdx.y) * S;
  base += static_cast<size_t>(blockIdx.y) * nchunks * C;
  perm += static_cast<size_t>(blockIdx.y) * S;
  const int start = blockIdx.x * kChunk;
  const int n = min(kChunk, S - start);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const unsigned long long below = (1ull << lane) - 1ull;
  for (int e = threadIdx.x; e < (kChunk / kSub) * C; e += kSub) sub_counts[e] = 0;
  __syncthreads();
  int32_t* run = sub_counts + wave * C;
  int lab_r[kSub / 64], rank_r[kSub / 64];
#pragma unroll
  for (int k = 0; k < kSub / 64; ++k) {
    const int i = wave * kSub + k * 64 + lane;
    int li = i < n ? labels[start + i] : -1;
    if (li < 0 || li >= C) li = -1;
    int rank = 0;
    unsigned long long left = __ballot(li >= 0);
    while (left) {
      const int leader = __ffsll(static_cast<long long>(left)) - 1;
      const int l = __builtin_amdgcn_readlane(li, leader);
      const unsigned long long m = __ballot(li == l);
      const int before = run[l];  // uniform: every lane reads the same count
      if (li == l) rank = before + __popcll(m & below);
      if (lane == leader) run[l] = before + __popcll(m);
      left &= ~m;
    }
    lab_r[k] = li;
    rank_r[k] = rank;
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < kSub / 64; ++k) {
    const int li = lab_r[k];
    if (li < 0) continue;
    int r = rank_r[k];
    for (int w2 = 0; w2 < wave; ++w2) r += sub_counts[w2 * C + li];
    perm[base[static_cast<size_t>(blockIdx.x) * C + li] + r] = start + wave * kSub + k * 64 + lane;
  }
}

inline int layout_chunks(int S) { return (S + kChunk - 1) / kChunk; }

// P layouts of S labels into C clusters; hist holds P * layout_chunks(S) * C ints.
inline void launch_layouts(const int32_t* labels, int S, int C, int P, int32_t* hist, int32_t* perm,
                           int32_t* offsets, int32_t* counts, hipStream_t stream) {
  const int nchunks = layout_chunks(S);
  hipLaunchKernelGGL(layout_hist, dim3(nchunks, P), dim3(256), 0, stream, labels, S, C, nchunks, hist);
  hipLaunchKernelGGL(layout_scan, dim3(P), dim3(1024), 0, stream, C, nchunks, hist, offsets, counts);
  const size_t lds = static_cast<size_t>((kChunk / kSub) * C) * sizeof(int32_t);
  hipFuncSetAttribute(reinterpret_cast<const void*>(layout_scatter), hipFuncAttributeMaxDynamicSharedMemorySize,
                      static_cast<int>(lds));
  hipLaunchKernelGGL(layout_scatter, dim3(nchunks, P), dim3(kSub), lds, stream, labels, S, C, nchunks, hist, perm);
}

}  // namespace
}  // namespace bsa
