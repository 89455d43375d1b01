// Per-row top-p block selection and kept-block lists.
//
// "Dynamic block masks and head-wise mask reuse", section "XAttention -- anti-diagonal block
// scoring": each query block keeps the smallest set of key blocks whose mass reaches tau of
// the row total; section "Deviations from the papers": at least one block per row, key
// block 0 not forced.  Equal scores are taken by lower key-block index.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kMaxCk = 1024;

__device__ __forceinline__ uint32_t sortable(float x) {
  const uint32_t u = __float_as_uint(x);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Block-wide exclusive scan of one int per thread (256 threads).
__device__ int block_excl_scan(int v, int* tmp, int* total) {
  const int t = threadIdx.x;
  tmp[t] = v;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const int add = t >= d ? tmp[t - d] : 0;
    __syncthreads();
    tmp[t] += add;
    __syncthreads();
  }
  const int incl = tmp[t];
  *total = tmp[255];
  __syncthreads();
  return incl - v;
}

// One workgroup (256 threads) per score row.
__global__ __launch_bounds__(256) void top_p_kernel(const float* __restrict__ scores, int Cq, int Ck,
                                                     const float* __restrict__ tau, int n_tau, int Hs,
                                                     uint8_t* __restrict__ keep, int32_t* __restrict__ kv_count,
                                                     int16_t* __restrict__ kv_idx) {
  __shared__ uint64_t key[kMaxCk];
  __shared__ float csum[kMaxCk];
  __shared__ int tmpi[256];
  __shared__ float tmpf[256];
  __shared__ uint8_t kb[kMaxCk];
  const size_t row = blockIdx.x;
  const int g = static_cast<int>(row / Cq);
  const float tau_r = n_tau == 1 ? tau[0] : tau[g % Hs];
  const float* srow = scores + row * Ck;
  int n2 = 1;
  while (n2 < Ck) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256) {
    // Descending by score, then ascending by index: the low word is the inverted index.
    key[i] = i < Ck ? (static_cast<uint64_t>(sortable(srow[i])) << 32) | static_cast<uint32_t>(0xffffffffu - i) : 0ull;
  }
  __syncthreads();
  // Bitonic sort, descending.
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += 256) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t a = key[i], b = key[p];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            key[i] = b;
            key[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // Inclusive prefix sum of the sorted scores: 4 consecutive entries per thread, then a
  // scan over the thread totals.
  float loc[4];
  float run = 0.0f;
  const int b0 = threadIdx.x * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = b0 + e;
    float s = 0.0f;
    if (i < Ck) s = srow[0xffffffffu - static_cast<uint32_t>(key[i])];
    run += s;
    loc[e] = run;
  }
  tmpf[threadIdx.x] = run;
  __syncthreads();
  for (int d = 1; d < 256; d <<= 1) {
    const float add = threadIdx.x >= static_cast<unsigned>(d) ? tmpf[threadIdx.x - d] : 0.0f;
    __syncthreads();
    tmpf[threadIdx.x] += add;
    __syncthreads();
  }
  const float before = tmpf[threadIdx.x] - run;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (b0 + e < kMaxCk) csum[b0 + e] = before + loc[e];
  __syncthreads();
  const float target = tau_r * csum[Ck - 1];
  // Shortest prefix reaching the target: the first rank whose cumulative mass >= target.
  int first = Ck - 1;
  for (int i = threadIdx.x; i < Ck; i += 256)
    if (csum[i] >= target) first = min(first, i);
  tmpi[threadIdx.x] = first;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (threadIdx.x < static_cast<unsigned>(d)) tmpi[threadIdx.x] = min(tmpi[threadIdx.x], tmpi[threadIdx.x + d]);
    __syncthreads();
  }
  const int last = tmpi[0];
  __syncthreads();
  for (int i = threadIdx.x; i < Ck; i += 256) kb[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i <= last; i += 256) kb[0xffffffffu - static_cast<uint32_t>(key[i])] = 1;
  __syncthreads();
  uint8_t* krow = keep + row * Ck;
  for (int i = threadIdx.x; i < Ck; i += 256) krow[i] = kb[i];
  // Ascending kept list.
  int16_t* lrow = kv_idx + row * Ck;
  int offset = 0;
  for (int c0 = 0; c0 < Ck; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int bit = c < Ck ? kb[c] : 0;
    int total;
    const int pos = block_excl_scan(bit, tmpi, &total);
    if (bit) lrow[offset + pos] = static_cast<int16_t>(c);
    offset += total;
  }
  if (threadIdx.x == 0) kv_count[row] = offset;
}

// Rows of at most 256 clusters: one wave per row, four keys per lane (lane l holds sorted
// positions 4l .. 4l+3), so the bitonic sort runs in registers -- partners one to three
// positions away within the lane, farther ones in another lane by a shuffle -- and the
// prefix sum, the cut and the kept list use wave scans, without barriers.  The keys, the
// order and the cut rule are those of top_p_kernel.
constexpr int kWaveCk = 256;
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t x, int m) {
  const int lo = __shfl_xor(static_cast<int>(x & 0xffffffffu), m);
  const int hi = __shfl_xor(static_cast<int>(x >> 32), m);
  return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}
__device__ __forceinline__ float wave_incl_scan(float x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const float y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}
__device__ __forceinline__ int wave_incl_scan_i(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  return x;
}

// Bitonic sort of 256 keys held four per lane (position i = 4 lane + j), descending.
__device__ __forceinline__ void wave_sort_desc(uint64_t (&key)[4]) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int k = 2; k <= kWaveCk; k <<= 1) {
#pragma unroll
    for (int d = k >> 1; d > 0; d >>= 1) {
      if (d >= 4) {
        const int dl = d >> 2;
        const bool lower = (lane & dl) == 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const uint64_t other = shfl_xor_u64(key[j], dl);
          const bool desc = ((lane * 4 + j) & k) == 0;
          const bool keep_max = desc == lower;
          key[j] = keep_max ? (key[j] > other ? key[j] : other) : (key[j] < other ? key[j] : other);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if ((j & d) != 0) continue;
          const int p = j | d;
          const bool desc = ((lane * 4 + j) & k) == 0;
          const uint64_t a = key[j], b = key[p];
          if (desc ? (a < b) : (a > b)) {
            key[j] = b;
            key[p] = a;
          }
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void top_p_wave_kernel(const float* __restrict__ scores, int rows, int Cq, int Ck,
                                                          const float* __restrict__ tau, int n_tau, int Hs,
                                                          uint8_t* __restrict__ keep, int32_t* __restrict__ kv_count,
                                                          int16_t* __restrict__ kv_idx) {
  __shared__ uint8_t kb_s[4][kWaveCk];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<size_t>(rows)) return;  // whole waves only; no barrier below
  const int g = static_cast<int>(row / Cq);
  const float tau_r = n_tau == 1 ? tau[0] : tau[g % Hs];
  const float* srow = scores + row * Ck;
  uint64_t key[4];
  float sv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane * 4 + j;
    sv[j] = i < Ck ? srow[i] : 0.0f;
    key[j] = i < Ck ? (static_cast<uint64_t>(sortable(sv[j])) << 32) | static_cast<uint32_t>(0xffffffffu - i) : 0ull;
  }
  wave_sort_desc(key);
  // Inclusive prefix sum of the sorted scores: 4 per lane, then over the lanes.
  float loc[4];
  float run = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane * 4 + j;
    float x = 0.0f;
    if (i < Ck) x = srow[0xffffffffu - static_cast<uint32_t>(key[j])];
    run += x;
    loc[j] = run;
  }
  const float incl = wave_incl_scan(run);
  const float before = incl - run;
  const float total = __shfl(incl, 63);
  const float target = tau_r * total;
  // The first rank whose cumulative mass reaches the target (Ck - 1 if none does).
  int mine = kWaveCk;
#pragma unroll
  for (int j = 3; j >= 0; --j)
    if (lane * 4 + j < Ck && before + loc[j] >= target) mine = lane * 4 + j;
  const unsigned long long hit = __ballot(mine < kWaveCk);
  int last = Ck - 1;
  if (hit) last = __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1);
  uint8_t* kb = kb_s[wave];
#pragma unroll
  for (int j = 0; j < 4; ++j) kb[lane * 4 + j] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane * 4 + j <= last) kb[0xffffffffu - static_cast<uint32_t>(key[j])] = 1;
  __builtin_amdgcn_wave_barrier();
  uint8_t* krow = keep + row * Ck;
  int bits[4], nb = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane * 4 + j;
    bits[j] = c < Ck ? kb[c] : 0;
    if (c < Ck) krow[c] = static_cast<uint8_t>(bits[j]);
    nb += bits[j];
  }
  // Ascending kept list.
  const int ni = wave_incl_scan_i(nb);
  int pos = ni - nb;
  int16_t* lrow = kv_idx + row * Ck;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (bits[j]) lrow[pos++] = static_cast<int16_t>(lane * 4 + j);
  if (lane == 63) kv_count[row] = ni;
}

// Error-aware routes for rows of at most 256 clusters: one wave per row, as top_p_wave_kernel
// (keys: err / n_c as in error_route_kernel; the prefix sum counts keys).
__global__ __launch_bounds__(256) void error_route_wave_kernel(const float* __restrict__ err, int rows, int Ck,
                                                               const int32_t* __restrict__ k_off, int rows_per_layout,
                                                               int budget, uint8_t* __restrict__ keep,
                                                               int32_t* __restrict__ kv_count,
                                                               int16_t* __restrict__ kv_idx) {
  __shared__ uint8_t kb_s[4][kWaveCk];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + wave;
  if (row >= static_cast<size_t>(rows)) return;  // whole waves only; no barrier below
  if (rows_per_layout > 0) k_off += (row / rows_per_layout) * (Ck + 1);  // the row's key layout
  const float* erow = err + row * Ck;
  uint64_t key[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int i = lane * 4 + j;
    key[j] = 0;  // empty clusters (and padding) sort last
    if (i < Ck) {
      const int n = k_off[i + 1] - k_off[i];
      if (n > 0)
        key[j] = (static_cast<uint64_t>(sortable(__fdiv_rn(erow[i], static_cast<float>(n)))) << 32) |
                 static_cast<uint32_t>(0xffffffffu - i);
    }
  }
  wave_sort_desc(key);
  int loc[4];
  int run = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int n = 0;
    if (key[j] != 0) {
      const int c = static_cast<int>(0xffffffffu - static_cast<uint32_t>(key[j]));
      n = k_off[c + 1] - k_off[c];
    }
    run += n;
    loc[j] = run;
  }
  const int before = wave_incl_scan_i(run) - run;
  // Last kept rank: the first non-empty rank whose cumulative count reaches the budget, else
  // the last non-empty rank.
  int mine = kWaveCk, last_ne = -1;
#pragma unroll
  for (int j = 3; j >= 0; --j) {
    if (key[j] == 0) continue;
    last_ne = max(last_ne, lane * 4 + j);
    if (before + loc[j] >= budget) mine = lane * 4 + j;
  }
  const unsigned long long hit = __ballot(mine < kWaveCk);
  int last = -1;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) last_ne = max(last_ne, __shfl_xor(last_ne, o));
  last = last_ne;
  if (hit) last = min(last, __shfl(mine, __ffsll(static_cast<long long>(hit)) - 1));
  uint8_t* kb = kb_s[wave];
#pragma unroll
  for (int j = 0; j < 4; ++j) kb[lane * 4 + j] = 0;
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (lane * 4 + j <= last) kb[0xffffffffu - static_cast<uint32_t>(key[j])] = 1;
  __builtin_amdgcn_wave_barrier();
  uint8_t* krow = keep + row * Ck;
  int bits[4], nb = 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = lane * 4 + j;
    bits[j] = c < Ck ? kb[c] : 0;
    if (c < Ck) krow[c] = static_cast<uint8_t>(bits[j]);
    nb += bits[j];
  }
  const int ni = wave_incl_scan_i(nb);
  int pos = ni - nb;
  int16_t* lrow = kv_idx + row * Ck;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    if (bits[j]) lrow[pos++] = static_cast<int16_t>(lane * 4 + j);
  if (lane == 63) kv_count[row] = ni;
}

__global__ __launch_bounds__(256) void mask_lists_kernel(const uint8_t* __restrict__ keep, int Ck,
                                                          int32_t* __restrict__ kv_count,
                                                          int16_t* __restrict__ kv_idx) {
  __shared__ int tmpi[256];
  const size_t row = blockIdx.x;
  const uint8_t* krow = keep + row * Ck;
  int16_t* lrow = kv_idx + row * Ck;
  int offset = 0;
  for (int c0 = 0; c0 < Ck; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int bit = (c < Ck && krow[c] != 0) ? 1 : 0;
    int total;
    const int pos = block_excl_scan(bit, tmpi, &total);
    if (bit) lrow[offset + pos] = static_cast<int16_t>(c);
    offset += total;
  }
  if (threadIdx.x == 0) kv_count[row] = offset;
}

// Error-aware routes ("Block-sparse attention" topic page, SVG-EAR card: the blocks with the
// highest error-to-cost ratio are computed exactly, the rest compensated).  One workgroup per
// mask row: the row's non-empty key clusters in order of err / n_c (float32, correctly
// rounded; descending, ties by lower index) -- the cost of block (a, c) is n_a n_c, and n_a
// is the same along the row -- and the shortest prefix whose key count reaches `budget`
// tokens, at least one cluster.  Empty clusters are never kept.
__global__ __launch_bounds__(256) void error_route_kernel(const float* __restrict__ err, int Ck,
                                                          const int32_t* __restrict__ k_off, int rows_per_layout,
                                                          int budget, uint8_t* __restrict__ keep,
                                                          int32_t* __restrict__ kv_count,
                                                          int16_t* __restrict__ kv_idx) {
  __shared__ uint64_t key[kMaxCk];
  __shared__ int csum[kMaxCk];
  __shared__ int tmpi[256];
  __shared__ uint8_t kb[kMaxCk];
  const size_t row = blockIdx.x;
  if (rows_per_layout > 0) k_off += (row / rows_per_layout) * (Ck + 1);  // the row's key layout
  const float* erow = err + row * Ck;
  int n2 = 1;
  while (n2 < Ck) n2 <<= 1;
  for (int i = threadIdx.x; i < n2; i += 256) {
    uint64_t k = 0;  // empty clusters (and padding) sort last
    if (i < Ck) {
      const int n = k_off[i + 1] - k_off[i];
      if (n > 0)
        k = (static_cast<uint64_t>(sortable(__fdiv_rn(erow[i], static_cast<float>(n)))) << 32) |
            static_cast<uint32_t>(0xffffffffu - i);
    }
    key[i] = k;
  }
  __syncthreads();
  for (int k = 2; k <= n2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int i = threadIdx.x; i < n2; i += 256) {
        const int p = i ^ j;
        if (p > i) {
          const uint64_t a = key[i], b = key[p];
          const bool desc = (i & k) == 0;
          if (desc ? (a < b) : (a > b)) {
            key[i] = b;
            key[p] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // Inclusive prefix sum of the key counts in sorted order (4 entries per thread).
  int loc[4];
  int run = 0;
  const int b0 = threadIdx.x * 4;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int i = b0 + e;
    int n = 0;
    if (i < Ck && key[i] != 0) {
      const int c = static_cast<int>(0xffffffffu - static_cast<uint32_t>(key[i]));
      n = k_off[c + 1] - k_off[c];
    }
    run += n;
    loc[e] = run;
  }
  int total;
  const int before = block_excl_scan(run, tmpi, &total);
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (b0 + e < kMaxCk) csum[b0 + e] = before + loc[e];
  __syncthreads();
  // Last kept rank: the first non-empty rank whose cumulative count reaches the budget, else
  // the last non-empty rank.
  int first = 0x7fffffff, last_ne = -1;
  for (int i = threadIdx.x; i < Ck; i += 256) {
    if (key[i] == 0) continue;
    last_ne = max(last_ne, i);
    if (csum[i] >= budget) first = min(first, i);
  }
  tmpi[threadIdx.x] = first;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (threadIdx.x < static_cast<unsigned>(d)) tmpi[threadIdx.x] = min(tmpi[threadIdx.x], tmpi[threadIdx.x + d]);
    __syncthreads();
  }
  const int first_all = tmpi[0];
  __syncthreads();
  tmpi[threadIdx.x] = last_ne;
  __syncthreads();
  for (int d = 128; d > 0; d >>= 1) {
    if (threadIdx.x < static_cast<unsigned>(d)) tmpi[threadIdx.x] = max(tmpi[threadIdx.x], tmpi[threadIdx.x + d]);
    __syncthreads();
  }
  const int last = min(first_all, tmpi[0]);
  __syncthreads();
  for (int i = threadIdx.x; i < Ck; i += 256) kb[i] = 0;
  __syncthreads();
  for (int i = threadIdx.x; i <= last; i += 256) kb[0xffffffffu - static_cast<uint32_t>(key[i])] = 1;
  __syncthreads();
  uint8_t* krow = keep + row * Ck;
  for (int i = threadIdx.x; i < Ck; i += 256) krow[i] = kb[i];
  int16_t* lrow = kv_idx + row * Ck;
  int offset = 0;
  for (int c0 = 0; c0 < Ck; c0 += 256) {
    const int c = c0 + threadIdx.x;
    const int bit = c < Ck ? kb[c] : 0;
    int tot;
    const int pos = block_excl_scan(bit, tmpi, &tot);
    if (bit) lrow[offset + pos] = static_cast<int16_t>(c);
    offset += tot;
  }
  if (threadIdx.x == 0) kv_count[row] = offset;
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_top_p_mask(const float* scores, int G, int Cq, int Ck, const float* tau, int n_tau, int Hs,
                                     uint8_t* keep, int32_t* kv_count, int16_t* kv_idx, hipStream_t stream) {
  if (!scores || !tau || !keep || !kv_count || !kv_idx) return BSA_E_ARG;
  if (G < 1 || Cq < 1 || Ck < 1 || Hs < 1) return BSA_E_ARG;
  if (n_tau != 1 && n_tau != Hs) return BSA_E_SHAPE;
  if (G % Hs != 0) return BSA_E_SHAPE;
  if (Ck > kMaxCk) return BSA_E_UNSUPPORTED;
  const long long rows = static_cast<long long>(G) * Cq;
  if (rows > 0x7fffffffLL) return BSA_E_UNSUPPORTED;
  if (Ck <= kWaveCk) {
    hipLaunchKernelGGL(top_p_wave_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream, scores,
                       static_cast<int>(rows), Cq, Ck, tau, n_tau, Hs, keep, kv_count, kv_idx);
    return launch_status();
  }
  hipLaunchKernelGGL(top_p_kernel, dim3(static_cast<unsigned>(rows)), dim3(256), 0, stream, scores, Cq, Ck, tau, n_tau,
                     Hs, keep, kv_count, kv_idx);
  return launch_status();
}

extern "C" bsa_status bsa_mask_lists(const uint8_t* keep, int rows, int Ck, int32_t* kv_count, int16_t* kv_idx,
                                     hipStream_t stream) {
  if (!keep || !kv_count || !kv_idx || rows < 1 || Ck < 1) return BSA_E_ARG;
  if (Ck > 32767) return BSA_E_UNSUPPORTED;
  hipLaunchKernelGGL(mask_lists_kernel, dim3(rows), dim3(256), 0, stream, keep, Ck, kv_count, kv_idx);
  return launch_status();
}

extern "C" bsa_status bsa_error_route(const float* err, int rows, int Ck, const int32_t* k_offsets, int rows_per_layout,
                                      int budget, uint8_t* keep, int32_t* kv_count, int16_t* kv_idx,
                                      hipStream_t stream) {
  if (!err || !k_offsets || !keep || !kv_count || !kv_idx || rows < 1 || Ck < 1) return BSA_E_ARG;
  if (rows_per_layout < 0 || (rows_per_layout > 0 && rows % rows_per_layout != 0)) return BSA_E_ARG;
  if (Ck > kMaxCk) return BSA_E_UNSUPPORTED;
  if (Ck <= kWaveCk) {
    hipLaunchKernelGGL(error_route_wave_kernel, dim3((rows + 3) / 4), dim3(256), 0, stream, err, rows, Ck, k_offsets,
                       rows_per_layout, budget, keep, kv_count, kv_idx);
    return launch_status();
  }
  hipLaunchKernelGGL(error_route_kernel, dim3(rows), dim3(256), 0, stream, err, Ck, k_offsets, rows_per_layout, budget,
                     keep, kv_count, kv_idx);
  return launch_status();
}
