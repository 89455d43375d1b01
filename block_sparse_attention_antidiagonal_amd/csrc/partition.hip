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
// serves both the key profiles and the query coordinates.  k-means on the GPU: assignment with
// one thread per point against the centres staged in LDS (|c|^2 - 2 x.c in float32), update
// as segment means over a counting sort of the labels (deterministic order).
#include "layout.hpp"

namespace bsa {
namespace {

constexpr int kF = 64;          // stored feature width
inline size_t pack_align_up(size_t x) { return (x + 255) / 256 * 256; }
constexpr int kAssignPts = 256;  // points per assignment workgroup
constexpr int kCenChunk = 256;  // centres staged in LDS at a time

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

// Nearest centre of every point: argmin_c |c|^2 - 2 x . c over the first NF features (the
// rest are zero on both sides), equal values to the lower index.
template <int NF>
__global__ __launch_bounds__(kAssignPts) void assign_kernel(const float* __restrict__ X, int N,
                                                            const float* __restrict__ cen, int C,
                                                            int32_t* __restrict__ labels) {
  __shared__ float ch[kCenChunk][NF];
  __shared__ float cn[kCenChunk];
  const int p = blockIdx.y;
  const int i = blockIdx.x * kAssignPts + threadIdx.x;
  float x[NF];
  const float* xr = X + (static_cast<size_t>(p) * N + (i < N ? i : 0)) * kF;
#pragma unroll
  for (int f = 0; f < NF; f += 4) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(xr + f);
    x[f] = v[0];
    x[f + 1] = v[1];
    x[f + 2] = v[2];
    x[f + 3] = v[3];
  }
  float best = INFINITY;
  int arg = 0;
  const float* cp = cen + static_cast<size_t>(p) * C * kF;
  for (int c0 = 0; c0 < C; c0 += kCenChunk) {
    const int nc = min(kCenChunk, C - c0);
    __syncthreads();  // the previous chunk's reads are done
    for (int e = threadIdx.x; e < nc * NF; e += kAssignPts) ch[e / NF][e % NF] = cp[(c0 + e / NF) * kF + e % NF];
    __syncthreads();
    for (int c = threadIdx.x; c < nc; c += kAssignPts) {
      float s = 0.0f;
#pragma unroll
      for (int f = 0; f < NF; ++f) s = __builtin_fmaf(ch[c][f], ch[c][f], s);
      cn[c] = s;
    }
    __syncthreads();
    for (int c = 0; c < nc; ++c) {
      float dot = 0.0f;
#pragma unroll
      for (int f = 0; f < NF; ++f) dot = __builtin_fmaf(x[f], ch[c][f], dot);
      const float dist = __builtin_fmaf(-2.0f, dot, cn[c]);
      if (dist < best) {
        best = dist;
        arg = c0 + c;
      }
    }
  }
  if (i < N) labels[static_cast<size_t>(p) * N + i] = arg;
}

// cen[p][c] = mean of the points of centre c (in the counting-sort order of the labels); a
// centre without points keeps its value.
__global__ __launch_bounds__(kF) void centre_mean_kernel(const float* __restrict__ X, int N,
                                                         const int32_t* __restrict__ perm,
                                                         const int32_t* __restrict__ offsets, int C,
                                                         float* __restrict__ cen) {
  const int c = blockIdx.x, p = blockIdx.y, f = threadIdx.x;
  const int32_t* off = offsets + static_cast<size_t>(p) * (C + 1);
  const int lo = off[c], hi = off[c + 1];
  if (hi <= lo) return;
  const int32_t* pp = perm + static_cast<size_t>(p) * N;
  const float* Xp = X + static_cast<size_t>(p) * N * kF;
  float s = 0.0f;
  for (int r = lo; r < hi; ++r) s += Xp[static_cast<size_t>(pp[r]) * kF + f];
  cen[(static_cast<size_t>(p) * C + c) * kF + f] = s / static_cast<float>(hi - lo);
}

// kbar[p][c] = mean of the keys of key group c in key space (zero for an empty group).
template <typename T, int D>
__global__ __launch_bounds__(D) void group_key_mean_kernel(const T* __restrict__ K, int S,
                                                           const int32_t* __restrict__ perm,
                                                           const int32_t* __restrict__ offsets, int C,
                                                           float* __restrict__ kbar) {
  const int c = blockIdx.x, p = blockIdx.y, d = threadIdx.x;
  const int32_t* off = offsets + static_cast<size_t>(p) * (C + 1);
  const int lo = off[c], hi = off[c + 1];
  const int32_t* pp = perm + static_cast<size_t>(p) * S;
  const T* Kp = K + static_cast<size_t>(p) * S * D;
  float s = 0.0f;
  for (int r = lo; r < hi; ++r) s += to_f32(Kp[static_cast<size_t>(pp[r]) * D + d]);
  kbar[(static_cast<size_t>(p) * C + c) * D + d] = hi > lo ? s / static_cast<float>(hi - lo) : 0.0f;
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

template <int NF>
void launch_assign(const float* X, int N, const float* cen, int C, int P, int32_t* labels, hipStream_t stream) {
  hipLaunchKernelGGL((assign_kernel<NF>), dim3((N + kAssignPts - 1) / kAssignPts, P), dim3(kAssignPts), 0, stream, X,
                     N, cen, C, labels);
}

// P independent k-means runs of N points (kF-float rows of X, the first nf features nonzero)
// into C centres; labels [P][N], centres [P][C][kF].  The counting sort leaves the layout of
// the final labels in w (perm, offsets).
void launch_kmeans(const float* X, int N, int nf, int C, int P, int iters, int32_t* labels, float* cen,
                   const KmWs& w, hipStream_t stream) {
  auto assign = [&]() {
    if (nf <= 16)
      launch_assign<16>(X, N, cen, C, P, labels, stream);
    else if (nf <= 32)
      launch_assign<32>(X, N, cen, C, P, labels, stream);
    else if (nf <= 48)
      launch_assign<48>(X, N, cen, C, P, labels, stream);
    else
      launch_assign<64>(X, N, cen, C, P, labels, stream);
  };
  hipLaunchKernelGGL(init_centres_kernel, dim3(C, P), dim3(kF), 0, stream, X, N, C, cen);
  for (int it = 0; it < iters; ++it) {
    assign();
    launch_layouts(labels, N, C, P, w.hist, w.perm, w.offsets, w.counts, stream);
    hipLaunchKernelGGL(centre_mean_kernel, dim3(C, P), dim3(kF), 0, stream, X, N, w.perm, w.offsets, C, cen);
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
#define BSA_RCP(T, DD)                                                                                               \
  do {                                                                                                               \
    const T* Qt = static_cast<const T*>(Q);                                                                         \
    const T* Kt = static_cast<const T*>(K);                                                                         \
    hipLaunchKernelGGL((sample_queries_kernel<T, DD>), dim3(P), dim3(DD), 0, stream, Qt, Hq, Hkv, S, rK, qs);        \
    hipLaunchKernelGGL((key_profile_kernel<T, DD>), tok_grid, dim3(256), 0, stream, Kt, S, qs, rK, scale, X);        \
    launch_kmeans(X, S, rK, Ck, P, iters, k_labels, kcen, kw, stream);                                               \
    launch_layouts(k_labels, S, Ck, P, kw.hist, kw.perm, kw.offsets, kw.counts, stream);                            \
    hipLaunchKernelGGL((group_key_mean_kernel<T, DD>), dim3(Ck, P), dim3(DD), 0, stream, Kt, S, kw.perm, kw.offsets, \
                       Ck, kbar);                                                                                    \
    hipLaunchKernelGGL((query_coord_kernel<T, DD>), tok_grid, dim3(256), 0, stream, Qt, Hq, Hkv, S, kbar, Ck, rq,    \
                       scale, X);                                                                                    \
    launch_kmeans(X, S, rq, Cq, P, iters, q_labels, qcen, qw, stream);                                               \
  } while (0)
  if (dtype == BSA_BF16) {
    if (D == 128) BSA_RCP(bf16_t, 128); else BSA_RCP(bf16_t, 64);
  } else {
    if (D == 128) BSA_RCP(float, 128); else BSA_RCP(float, 64);
  }
#undef BSA_RCP
  return launch_status();
}
