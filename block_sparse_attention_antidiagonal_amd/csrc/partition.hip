// Response-coupled partitioning: key groups from the keys' responses to sampled queries, query
// groups from the queries' responses to the key-group centroids.
//
// "Partition the Support, Reconstruct the Residual" (summary page), the Response-Coupled
// Partitioning paragraph: queries sampled from the call, keys grouped by their pre-softmax
// response profiles (feature rank rK = 48), key-group centroids defining the query coordinates
// (rank rQ = 64), one asymmetric pass; the grouped-query paragraph: partitions are shared by
// the query heads of a K/V group; the timing paragraph: the grouping is an online k-means
// inside the call.  Readings of what the page leaves open (one partition pair per (batch, K/V
// head); evenly spaced samples and starting centres; Lloyd iterations, ties to the lower
// centre, a centre without points stays; query coordinates as unit directions of the group's
// mean query) are the oracle's, stated in include/bsa.h.
//
// Every feature vector is stored with kF = 64 floats (zero past its rank), so one k-means
// serves both the key profiles and the query coordinates.  k-means on the GPU: the nearest
// centre from |c|^2 - 2 x.c with x.c as split-bfloat16 MFMA products, the update as segment
// means over a counting sort of the labels (a fixed summation order, so runs repeat bit for
// bit).  For bfloat16 inputs the key profiles and query coordinates are MFMA products too.
#include "layout.hpp"

namespace bsa {
namespace {

constexpr int kF = 64;          // stored feature width
inline size_t pack_align_up(size_t x) { return (x + 255) / 256 * 256; }
constexpr int kCenChunk = 256;  // centres staged in LDS at a time (one per thread)

__device__ __forceinline__ int evenly_spaced(int j, int n_items, int n_pick) {
  return static_cast<int>(((2LL * j + 1) * n_items) / (2LL * n_pick));
}

// qs[p][j][d]: the rK sampled query rows of layout p = b * Hkv + kvh (token floor((j + 1/2)
// S / rK) of query head kvh * G + j % G); rows past rK are zero.  One workgroup per p.
template <typename T, int D>
__global__ __launch_bounds__(D) void sample_queries_kernel(const T* __restrict__ Q, int Hq, int Hkv, int S, int rK,
                                                           float* __restrict__ qs) {
  const int p = blockIdx.x, b = p / Hkv, kvh = p % Hkv, G = Hq / Hkv, d = threadIdx.x;
  for (int j = 0; j < kF; ++j) {
    float v = 0.0f;
    if (j < rK) {
      const int h = kvh * G + j % G, tok = evenly_spaced(j, S, rK);
      v = to_f32(Q[((static_cast<size_t>(b) * Hq + h) * S + tok) * D + d]);
    }
    qs[(static_cast<size_t>(p) * kF + j) * D + d] = v;
  }
}

// X[p][i][j] = (k_i . qs_j) * scale for j < rK, 0 past it: each key's response profile.
template <typename T, int D>
__global__ __launch_bounds__(256) void key_profile_kernel(const T* __restrict__ K, int S, const float* __restrict__ qs,
                                                          int rK, float scale, float* __restrict__ X) {
  __shared__ float qsh[kF][D];
  const int p = blockIdx.y;
  for (int e = threadIdx.x; e < kF * D; e += 256) qsh[e / D][e % D] = qs[static_cast<size_t>(p) * kF * D + e];
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= S) return;
  float k[D];
  const T* kr = K + (static_cast<size_t>(p) * S + i) * D;
#pragma unroll
  for (int d = 0; d < D; ++d) k[d] = to_f32(kr[d]);
  float* xr = X + (static_cast<size_t>(p) * S + i) * kF;
  for (int j = 0; j < kF; ++j) {
    float acc = 0.0f;
    if (j < rK) {
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(k[d], qsh[j][d], acc);
    }
    xr[j] = acc * scale;
  }
}

// Starting centres: cen[p][c] = X[p][floor((c + 1/2) N / C)].
__global__ __launch_bounds__(kF) void init_centres_kernel(const float* __restrict__ X, int N, int C,
                                                          float* __restrict__ cen) {
  const int c = blockIdx.x, p = blockIdx.y;
  const int i = evenly_spaced(c, N, C);
  cen[(static_cast<size_t>(p) * C + c) * kF + threadIdx.x] = X[(static_cast<size_t>(p) * N + i) * kF + threadIdx.x];
}

// Split of float values into bfloat16 high and low parts (x = hi + lo + a residual of at most
// 2^-17 |x|): three bfloat16 products hi.hi + hi.lo + lo.hi give a dot product to about
// 2^-15 of |x| |c|, with the MFMA cores' rate.
__device__ __forceinline__ void split_frag(const float* x, Frag<bf16_t>& hi, Frag<bf16_t>& lo) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const __bf16 hb = static_cast<__bf16>(x[i]);
    hi.v[i] = hb;
    lo.v[i] = static_cast<__bf16>(x[i] - static_cast<float>(hb));
  }
}

__device__ __forceinline__ void load8(const float* p, float* v) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[i] = a[i];
    v[4 + i] = b[i];
  }
}

__device__ __forceinline__ int swap_halves_i(int x) { return __float_as_int(swap_halves(__int_as_float(x))); }

// Nearest centre of every point: argmin_c |c|^2 - 2 x . c over the first 16 NK features (the
// rest are zero on both sides), equal values to the lower index.  The products x . c run on
// the MFMA cores as split-bfloat16 products: centres (A, rows = centres, staged in LDS per
// chunk of 256 with their float32 norms) against points (B, columns = points, held in
// registers by the wave that owns them); each lane keeps the best centre of its point over
// the accumulator rows it holds, and the two lane halves are merged at the end.
constexpr int kAssignTiles = 4;                    // 32-point tiles per wave
constexpr int kAssignPts = 4 * kAssignTiles * 32;  // points per workgroup
template <int NK>
__global__ __launch_bounds__(256) void assign_kernel(const float* __restrict__ X, int N, const float* __restrict__ cen,
                                                     int C, int32_t* __restrict__ labels) {
  __shared__ uint4 chi[kCenChunk][8];  // 16-byte pieces of the high parts, piece q at q ^ (c & 7)
  __shared__ uint4 clo[kCenChunk][8];
  __shared__ float cn[kCenChunk];
  const int p = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  Frag<bf16_t> bh[kAssignTiles][NK], bl[kAssignTiles][NK];
  int pt[kAssignTiles];
#pragma unroll
  for (int t = 0; t < kAssignTiles; ++t) {
    pt[t] = blockIdx.x * kAssignPts + (wave * kAssignTiles + t) * 32 + (lane & 31);
    const float* xr = X + (static_cast<size_t>(p) * N + min(pt[t], N - 1)) * kF + 8 * h;
#pragma unroll
    for (int s = 0; s < NK; ++s) {
      float v[8];
      load8(xr + 16 * s, v);
      split_frag(v, bh[t][s], bl[t][s]);
    }
  }
  float best[kAssignTiles];
  int arg[kAssignTiles];
#pragma unroll
  for (int t = 0; t < kAssignTiles; ++t) {
    best[t] = INFINITY;
    arg[t] = 0;
  }
  const float* cp = cen + static_cast<size_t>(p) * C * kF;
  for (int c0 = 0; c0 < C; c0 += kCenChunk) {
    const int nc = min(kCenChunk, C - c0);
    __syncthreads();  // the previous chunk's reads are done
    {
      const int c = threadIdx.x;  // one centre per thread (kCenChunk == blockDim.x)
      float n2 = 0.0f;
#pragma unroll
      for (int q = 0; q < 2 * NK; ++q) {
        float v[8] = {};
        if (c < nc) load8(cp + static_cast<size_t>(c0 + c) * kF + 8 * q, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) n2 = __builtin_fmaf(v[i], v[i], n2);
        Frag<bf16_t> hi, lo;
        split_frag(v, hi, lo);
        chi[c][q ^ (c & 7)] = __builtin_bit_cast(uint4, hi.v);
        clo[c][q ^ (c & 7)] = __builtin_bit_cast(uint4, lo.v);
      }
      cn[c] = c < nc ? n2 : INFINITY;  // padding rows never win
    }
    __syncthreads();
    const int nblk = (nc + 31) >> 5;
    for (int blk = 0; blk < nblk; ++blk) {
      const int c = blk * 32 + (lane & 31);
      Frag<bf16_t> ah[NK], al[NK];
#pragma unroll
      for (int s = 0; s < NK; ++s) {
        ah[s].v = __builtin_bit_cast(bf16x8, chi[c][(2 * s + h) ^ (c & 7)]);
        al[s].v = __builtin_bit_cast(bf16x8, clo[c][(2 * s + h) ^ (c & 7)]);
      }
#pragma unroll
      for (int t = 0; t < kAssignTiles; ++t) {
        f32x16 acc = {};
#pragma unroll
        for (int s = 0; s < NK; ++s) {
          acc = mma(ah[s], bh[t][s], acc);
          acc = mma(ah[s], bl[t][s], acc);
          acc = mma(al[s], bh[t][s], acc);
        }
#pragma unroll
        for (int j = 0; j < 16; ++j) {  // rows in increasing order: the first minimum stays
          const int row = blk * 32 + 8 * (j >> 2) + 4 * h + (j & 3);
          const float d = __builtin_fmaf(-2.0f, acc[j], cn[row]);
          if (d < best[t]) {
            best[t] = d;
            arg[t] = c0 + row;
          }
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < kAssignTiles; ++t) {
    const float ob = swap_halves(best[t]);
    const int oa = swap_halves_i(arg[t]);
    if (ob < best[t] || (ob == best[t] && oa < arg[t])) arg[t] = oa;
    if (h == 0 && pt[t] < N) labels[static_cast<size_t>(p) * N + pt[t]] = arg[t];
  }
}

// Sixteen-byte loads of float or bfloat16 rows, widened to float.
template <typename T>
struct Vec16;
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  static __device__ __forceinline__ void add(const float* p, float* acc) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(p);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += v[i];
  }
};
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  static __device__ __forceinline__ void add(const bf16_t* p, float* acc) {
    const uint4 v = *reinterpret_cast<const uint4*>(p);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      acc[2 * i] += __uint_as_float(w[i] << 16);
      acc[2 * i + 1] += __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};

// out[p][c] = mean of the W-wide rows of segment c (rows[p][perm[p][r]] for offsets[p][c] <= r
// < offsets[p][c + 1]).  An empty segment keeps out[p][c] (KEEP_EMPTY: k-means centres) or
// writes zeros (key-group centroids).  The rows are summed in a fixed order: slot
// r % RPS of the workgroup takes every RPS-th row, and the slots are added in order.
template <typename T, int W, bool KEEP_EMPTY>
__global__ __launch_bounds__(256) void segment_mean_kernel(const T* __restrict__ rows, int N,
                                                           const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ offsets, int C,
                                                           float* __restrict__ out) {
  constexpr int VEC = Vec16<T>::N, LPR = W / VEC, RPS = 256 / LPR;
  __shared__ float part[RPS][W];
  const int c = blockIdx.x, p = blockIdx.y;
  const int32_t* off = offsets + static_cast<size_t>(p) * (C + 1);
  const int lo = off[c], hi = off[c + 1];
  float* dst = out + (static_cast<size_t>(p) * C + c) * W;
  if (hi <= lo) {
    if (!KEEP_EMPTY)
      for (int e = threadIdx.x; e < W; e += 256) dst[e] = 0.0f;
    return;
  }
  const int slot = threadIdx.x / LPR, q = threadIdx.x % LPR;
  const T* base = rows + static_cast<size_t>(p) * N * W + q * VEC;
  const int32_t* pp = perm + static_cast<size_t>(p) * N;
  float a[VEC] = {}, b[VEC] = {};
  int r = lo + slot;
  for (; r + RPS < hi; r += 2 * RPS) {  // two rows in flight per thread
    Vec16<T>::add(base + static_cast<size_t>(pp[r]) * W, a);
    Vec16<T>::add(base + static_cast<size_t>(pp[r + RPS]) * W, b);
  }
  if (r < hi) Vec16<T>::add(base + static_cast<size_t>(pp[r]) * W, a);
#pragma unroll
  for (int v = 0; v < VEC; ++v) part[slot][q * VEC + v] = a[v] + b[v];
  __syncthreads();
  const float inv_n = 1.0f / static_cast<float>(hi - lo);
  for (int e = threadIdx.x; e < W; e += 256) {
    float s = 0.0f;
#pragma unroll 8
    for (int sl = 0; sl < RPS; ++sl) s += part[sl][e];
    dst[e] = s * inv_n;
  }
}

// Key profiles of bfloat16 keys on the MFMA cores: X[p][i][j] = (k_i . qs_j) * scale, with the
// sampled queries (exact in bfloat16) as the A operand (rows = the 64 features) and 32-key
// tiles as the B operand; products are exact, sums in float32.  Each wave takes kProfTiles
// tiles of its workgroup's 512 keys.
constexpr int kProfTiles = 4;
template <int D>
__global__ __launch_bounds__(256) void key_profile_mfma_kernel(const bf16_t* __restrict__ K, int S,
                                                               const float* __restrict__ qs, float scale,
                                                               float* __restrict__ X) {
  const int p = blockIdx.y, lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  Frag<bf16_t> a[2][D / 16];
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      float v[8];
      load8(qs + (static_cast<size_t>(p) * kF + 32 * b + (lane & 31)) * D + 16 * s + 8 * h, v);
      frag_from_f32(a[b][s], v);
    }
  for (int tt = 0; tt < kProfTiles; ++tt) {
    const int tok0 = ((blockIdx.x * 4 + wave) * kProfTiles + tt) * 32;
    if (tok0 >= S) break;
    const int tok = tok0 + (lane & 31);
    const bf16_t* kr = K + (static_cast<size_t>(p) * S + min(tok, S - 1)) * D + 8 * h;
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      Frag<bf16_t> bk;
      load_frag(bk, kr + 16 * s);
      acc0 = mma(a[0][s], bk, acc0);
      acc1 = mma(a[1][s], bk, acc1);
    }
    if (tok < S) {
      float* xr = X + (static_cast<size_t>(p) * S + tok) * kF + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<f32x4*>(xr + 8 * q) =
            f32x4{acc0[4 * q] * scale, acc0[4 * q + 1] * scale, acc0[4 * q + 2] * scale, acc0[4 * q + 3] * scale};
        *reinterpret_cast<f32x4*>(xr + 32 + 8 * q) =
            f32x4{acc1[4 * q] * scale, acc1[4 * q + 1] * scale, acc1[4 * q + 2] * scale, acc1[4 * q + 3] * scale};
      }
    }
  }
}

// Query coordinates of bfloat16 queries on the MFMA cores: the key-group centroids (split
// into bfloat16 high and low parts) as the A operand (rows = the coordinates), 32-token tiles
// of each of the group's query heads as the B operand, summed over the heads; then scaled by
// scale / G and to unit length (the two lane halves hold the two halves of a token's
// coordinates).
template <int D>
__global__ __launch_bounds__(256) void query_coord_mfma_kernel(const bf16_t* __restrict__ Q, int Hq, int Hkv, int S,
                                                               const float* __restrict__ kbar, int Ck, int rQ,
                                                               float scale, float* __restrict__ X) {
  const int p = blockIdx.y, b = p / Hkv, kvh = p % Hkv, G = Hq / Hkv;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, h = lane >> 5;
  Frag<bf16_t> ah[2][D / 16], al[2][D / 16];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const int j = 32 * blk + (lane & 31);
    const float* kr = kbar + (static_cast<size_t>(p) * Ck + (j < rQ ? evenly_spaced(j, Ck, rQ) : 0)) * D + 8 * h;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      float v[8] = {};
      if (j < rQ) load8(kr + 16 * s, v);
      split_frag(v, ah[blk][s], al[blk][s]);
    }
  }
  const float f = scale / static_cast<float>(G);
  for (int tt = 0; tt < kProfTiles; ++tt) {
    const int tok0 = ((blockIdx.x * 4 + wave) * kProfTiles + tt) * 32;
    if (tok0 >= S) break;
    const int tok = tok0 + (lane & 31);
    f32x16 acc0 = {}, acc1 = {};
    for (int g = 0; g < G; ++g) {
      const bf16_t* qr = Q + ((static_cast<size_t>(b) * Hq + kvh * G + g) * S + min(tok, S - 1)) * D + 8 * h;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
        Frag<bf16_t> bq;
        load_frag(bq, qr + 16 * s);
        acc0 = mma(ah[0][s], bq, acc0);
        acc0 = mma(al[0][s], bq, acc0);
        acc1 = mma(ah[1][s], bq, acc1);
        acc1 = mma(al[1][s], bq, acc1);
      }
    }
    float n2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      acc0[j] *= f;
      acc1[j] *= f;
      n2 = __builtin_fmaf(acc0[j], acc0[j], n2);
      n2 = __builtin_fmaf(acc1[j], acc1[j], n2);
    }
    n2 += swap_halves(n2);
    const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
    if (tok < S) {
      float* xr = X + (static_cast<size_t>(p) * S + tok) * kF + 4 * h;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        *reinterpret_cast<f32x4*>(xr + 8 * q) =
            f32x4{acc0[4 * q] * inv, acc0[4 * q + 1] * inv, acc0[4 * q + 2] * inv, acc0[4 * q + 3] * inv};
        *reinterpret_cast<f32x4*>(xr + 32 + 8 * q) =
            f32x4{acc1[4 * q] * inv, acc1[4 * q + 1] * inv, acc1[4 * q + 2] * inv, acc1[4 * q + 3] * inv};
      }
    }
  }
}

// X[p][i] = the unit direction of token i's responses (its mean query over the group's heads,
// dotted with the centroids of key groups floor((j + 1/2) Ck / rQ'), times scale); a zero
// vector stays zero; zero past rQ'.
template <typename T, int D>
__global__ __launch_bounds__(256) void query_coord_kernel(const T* __restrict__ Q, int Hq, int Hkv, int S,
                                                          const float* __restrict__ kbar, int Ck, int rQ, float scale,
                                                          float* __restrict__ X) {
  __shared__ float kb[kF][D];
  const int p = blockIdx.y, b = p / Hkv, kvh = p % Hkv, G = Hq / Hkv;
  for (int e = threadIdx.x; e < kF * D; e += 256) {
    const int j = e / D, d = e % D;
    kb[j][d] = j < rQ ? kbar[(static_cast<size_t>(p) * Ck + evenly_spaced(j, Ck, rQ)) * D + d] : 0.0f;
  }
  __syncthreads();
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= S) return;
  float q[D];
#pragma unroll
  for (int d = 0; d < D; ++d) q[d] = 0.0f;
  for (int g = 0; g < G; ++g) {
    const T* qr = Q + ((static_cast<size_t>(b) * Hq + kvh * G + g) * S + i) * D;
#pragma unroll
    for (int d = 0; d < D; ++d) q[d] += to_f32(qr[d]);
  }
  const float invg = 1.0f / static_cast<float>(G);
  // The responses go out as they are formed (the query row holds the registers), then the
  // thread scales its own row to unit length.
  float* xr = X + (static_cast<size_t>(p) * S + i) * kF;
  float n2 = 0.0f;
  for (int j = 0; j < kF; ++j) {
    float acc = 0.0f;
    if (j < rQ) {
#pragma unroll
      for (int d = 0; d < D; ++d) acc = __builtin_fmaf(q[d], kb[j][d], acc);
    }
    const float g = acc * invg * scale;
    n2 = __builtin_fmaf(g, g, n2);
    xr[j] = g;
  }
  const float inv = n2 > 0.0f ? 1.0f / sqrtf(n2) : 0.0f;
#pragma unroll
  for (int j = 0; j < kF; j += 4) {
    f32x4 v = *reinterpret_cast<const f32x4*>(xr + j);
    *reinterpret_cast<f32x4*>(xr + j) = f32x4{v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv};
  }
}

// Scratch of the k-means: the counting sort of the labels.
struct KmWs {
  int32_t *hist, *perm, *offsets, *counts;
};
inline size_t km_ws_ints(int P, int N, int C) {
  return static_cast<size_t>(P) * (static_cast<size_t>(layout_chunks(N)) * C + N + (C + 1) + C);
}
inline KmWs km_ws(int32_t* base, int P, int N, int C) {
  KmWs w;
  w.hist = base;
  w.perm = w.hist + static_cast<size_t>(P) * layout_chunks(N) * C;
  w.offsets = w.perm + static_cast<size_t>(P) * N;
  w.counts = w.offsets + static_cast<size_t>(P) * (C + 1);
  return w;
}

template <int NK>
void launch_assign(const float* X, int N, const float* cen, int C, int P, int32_t* labels, hipStream_t stream) {
  hipLaunchKernelGGL((assign_kernel<NK>), dim3((N + kAssignPts - 1) / kAssignPts, P), dim3(256), 0, stream, X, N,
                     cen, C, labels);
}

// P independent k-means runs of N points (kF-float rows of X, the first nf features nonzero)
// into C centres; labels [P][N], centres [P][C][kF].  The counting sort of the labels orders
// the points of every centre for the means.
void launch_kmeans(const float* X, int N, int nf, int C, int P, int iters, int32_t* labels, float* cen,
                   const KmWs& w, hipStream_t stream) {
  auto assign = [&]() {
    if (nf <= 16)
      launch_assign<1>(X, N, cen, C, P, labels, stream);
    else if (nf <= 32)
      launch_assign<2>(X, N, cen, C, P, labels, stream);
    else if (nf <= 48)
      launch_assign<3>(X, N, cen, C, P, labels, stream);
    else
      launch_assign<4>(X, N, cen, C, P, labels, stream);
  };
  hipLaunchKernelGGL(init_centres_kernel, dim3(C, P), dim3(kF), 0, stream, X, N, C, cen);
  for (int it = 0; it < iters; ++it) {
    assign();
    launch_layouts(labels, N, C, P, w.hist, w.perm, w.offsets, w.counts, stream);
    hipLaunchKernelGGL((segment_mean_kernel<float, kF, true>), dim3(C, P), dim3(256), 0, stream, X, N, w.perm,
                       w.offsets, C, cen);
  }
  assign();
}

// Scratch of the whole partition: the features (kF floats per token), the sampled queries,
// the key-group centroids, the centres of both runs, the k-means sort.
struct RcpWs {
  size_t X, qs, kbar, kcen, qcen, km, total;
};
inline RcpWs rcp_ws(int P, int S, int D, int Cq, int Ck) {
  RcpWs w;
  w.X = 0;
  w.qs = pack_align_up(static_cast<size_t>(P) * S * kF * 4);
  w.kbar = w.qs + pack_align_up(static_cast<size_t>(P) * kF * D * 4);
  w.kcen = w.kbar + pack_align_up(static_cast<size_t>(P) * Ck * D * 4);
  w.qcen = w.kcen + pack_align_up(static_cast<size_t>(P) * Ck * kF * 4);
  w.km = w.qcen + pack_align_up(static_cast<size_t>(P) * Cq * kF * 4);
  w.total = w.km + pack_align_up(km_ws_ints(P, S, Ck > Cq ? Ck : Cq) * 4);
  return w;
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_kmeans_workspace_size(int P, int N, int C, size_t* bytes) {
  if (!bytes || P < 1 || N < 1 || C < 1) return BSA_E_ARG;
  if (C > kMaxC || C > N) return BSA_E_UNSUPPORTED;
  *bytes = km_ws_ints(P, N, C) * 4;
  return BSA_OK;
}

extern "C" bsa_status bsa_kmeans(int P, int N, int nf, const float* X, int C, int iters, int32_t* labels,
                                 float* centres, void* ws, size_t ws_bytes, hipStream_t stream) {
  size_t need = 0;
  const bsa_status st = bsa_kmeans_workspace_size(P, N, C, &need);
  if (st != BSA_OK) return st;
  if (!X || !labels || !centres || nf < 1 || nf > kF || iters < 0) return BSA_E_ARG;
  if (P > 65535) return BSA_E_UNSUPPORTED;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  launch_kmeans(X, N, nf, C, P, iters, labels, centres, km_ws(static_cast<int32_t*>(ws), P, N, C), stream);
  return launch_status();
}

extern "C" bsa_status bsa_response_partition_workspace_size(int B, int Hkv, int S, int D, int Cq, int Ck,
                                                            size_t* bytes) {
  if (!bytes || B < 1 || Hkv < 1 || S < 1 || Cq < 1 || Ck < 1) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (Cq > kMaxC || Ck > kMaxC || Cq > S || Ck > S) return BSA_E_UNSUPPORTED;
  *bytes = rcp_ws(B * Hkv, S, D, Cq, Ck).total;
  return BSA_OK;
}

extern "C" bsa_status bsa_response_partition(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                             const void* K, float scale, int rK, int rQ, int Cq, int Ck, int iters,
                                             int32_t* k_labels, int32_t* q_labels, float* k_centres,
                                             float* q_centres, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  size_t need = 0;
  const bsa_status st = bsa_response_partition_workspace_size(B, Hkv, S, D, Cq, Ck, &need);
  if (st != BSA_OK) return st;
  if (Hq < 1 || Hq % Hkv != 0) return BSA_E_SHAPE;
  if (!Q || !K || !k_labels || !q_labels) return BSA_E_ARG;
  if (rK < 1 || rK > kF || rQ < 1 || rQ > kF || iters < 0) return BSA_E_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return BSA_E_ARG;
  if (static_cast<long long>(B) * Hkv > 65535) return BSA_E_UNSUPPORTED;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  const int P = B * Hkv;
  const RcpWs W = rcp_ws(P, S, D, Cq, Ck);
  unsigned char* base = static_cast<unsigned char*>(ws);
  float* X = reinterpret_cast<float*>(base + W.X);
  float* qs = reinterpret_cast<float*>(base + W.qs);
  float* kbar = reinterpret_cast<float*>(base + W.kbar);
  float* kcen = k_centres != nullptr ? k_centres : reinterpret_cast<float*>(base + W.kcen);
  float* qcen = q_centres != nullptr ? q_centres : reinterpret_cast<float*>(base + W.qcen);
  const KmWs kw = km_ws(reinterpret_cast<int32_t*>(base + W.km), P, S, Ck);
  const KmWs qw = km_ws(reinterpret_cast<int32_t*>(base + W.km), P, S, Cq);
  const int rq = rQ < Ck ? rQ : Ck;  // coordinates: at most one per key group
  const dim3 tok_grid((S + 255) / 256, P);
#define BSA_RCP(T, DD, PROFILE, COORDS)                                                                              \
  do {                                                                                                               \
    const T* Qt = static_cast<const T*>(Q);                                                                         \
    const T* Kt = static_cast<const T*>(K);                                                                         \
    hipLaunchKernelGGL((sample_queries_kernel<T, DD>), dim3(P), dim3(DD), 0, stream, Qt, Hq, Hkv, S, rK, qs);        \
    PROFILE;                                                                                                         \
    launch_kmeans(X, S, rK, Ck, P, iters, k_labels, kcen, kw, stream);                                               \
    launch_layouts(k_labels, S, Ck, P, kw.hist, kw.perm, kw.offsets, kw.counts, stream);                      \
    hipLaunchKernelGGL((segment_mean_kernel<T, DD, false>), dim3(Ck, P), dim3(256), 0, stream, Kt, S, kw.perm,       \
                       kw.offsets, Ck, kbar);                                                                        \
    COORDS;                                                                                                          \
    launch_kmeans(X, S, rq, Cq, P, iters, q_labels, qcen, qw, stream);                                               \
  } while (0)
  const dim3 mfma_grid((S + 4 * kProfTiles * 32 - 1) / (4 * kProfTiles * 32), P);
#define BSA_RCP_BF16(DD)                                                                                             \
  BSA_RCP(bf16_t, DD,                                                                                                \
          hipLaunchKernelGGL((key_profile_mfma_kernel<DD>), mfma_grid, dim3(256), 0, stream, Kt, S, qs, scale, X),   \
          hipLaunchKernelGGL((query_coord_mfma_kernel<DD>), mfma_grid, dim3(256), 0, stream, Qt, Hq, Hkv, S, kbar,   \
                             Ck, rq, scale, X))
#define BSA_RCP_F32(DD)                                                                                              \
  BSA_RCP(float, DD,                                                                                                 \
          hipLaunchKernelGGL((key_profile_kernel<float, DD>), tok_grid, dim3(256), 0, stream, Kt, S, qs, rK, scale,  \
                             X),                                                                                     \
          hipLaunchKernelGGL((query_coord_kernel<float, DD>), tok_grid, dim3(256), 0, stream, Qt, Hq, Hkv, S, kbar,  \
                             Ck, rq, scale, X))
  if (dtype == BSA_BF16) {
    if (D == 128) BSA_RCP_BF16(128); else BSA_RCP_BF16(64);
  } else {
    if (D == 128) BSA_RCP_F32(128); else BSA_RCP_F32(64);
  }
#undef BSA_RCP_BF16
#undef BSA_RCP_F32
#undef BSA_RCP
  return launch_status();
}
