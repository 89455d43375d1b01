// Probe rows of the error-aware router: the mean query row of every query cluster.
//
// "Block-sparse attention" topic page, SVG-EAR card: a light probe estimates each block's
// compensation error.  "Sparse-block compensation", section "SVG-EAR -- centroid
// compensation": skipped keys are stood in for by their cluster mean; the router's probe for
// a block row is the same statistic on the query side, q_bar_a = (1 / n_a) sum_{i in a} q_i,
// rounded to the input type (as the centroid keys are in the attention).  An empty cluster
// gets a zero row.
//
// One workgroup per (query cluster, batch x head): 16-byte loads with a row's chunks on
// consecutive lanes, float32 sums per thread, then over the row slots in a fixed order.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kQcThreads = 256;

template <typename T, int D>
__global__ __launch_bounds__(kQcThreads) void query_centroid_kernel(const T* __restrict__ Q, int S,
                                                                    const int32_t* __restrict__ perm,
                                                                    const int32_t* __restrict__ offsets, int Cq,
                                                                    int Hq, int Hkv, int nl, T* __restrict__ qbar) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                            // chunks per row
  constexpr int SLOTS = kQcThreads / CPR;                 // rows read side by side
  __shared__ float red[SLOTS][D + 1];
  const int a = blockIdx.x;
  const size_t bh = blockIdx.y;
  if (nl > 1) {  // the query layout of this head's (batch, K/V head)
    const size_t lay = (bh / Hq) * Hkv + (bh % Hq) / (Hq / Hkv);
    perm += lay * S;
    offsets += lay * (Cq + 1);
  }
  const int lo = offsets[a], n = offsets[a + 1] - lo;
  const int c = threadIdx.x % CPR, slot = threadIdx.x / CPR;
  const T* Qh = Q + bh * static_cast<size_t>(S) * D;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
  for (int r = slot; r < n; r += SLOTS) {
    const uint4 v = *reinterpret_cast<const uint4*>(Qh + static_cast<size_t>(perm[lo + r]) * D + c * EPC);
    const T* x = reinterpret_cast<const T*>(&v);
#pragma unroll
    for (int e = 0; e < EPC; ++e) acc[e] += to_f32(x[e]);
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[slot][c * EPC + e] = acc[e];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += kQcThreads) {
    float s = 0.0f;
    for (int k = 0; k < SLOTS; ++k) s += red[k][d];
    qbar[(bh * Cq + a) * D + d] = from_f32<T>(n > 0 ? s / static_cast<float>(n) : 0.0f);
  }
}

template <typename T, int D>
bsa_status launch_query_centroids(int B, int Hq, int Hkv, int S, const void* Q, const int32_t* perm,
                                  const int32_t* offsets, int Cq, int nl, void* qbar, hipStream_t stream) {
  hipLaunchKernelGGL((query_centroid_kernel<T, D>), dim3(Cq, B * Hq), dim3(kQcThreads), 0, stream,
                     static_cast<const T*>(Q), S, perm, offsets, Cq, Hq, Hkv, nl, static_cast<T*>(qbar));
  return launch_status();
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_query_centroids(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                          const int32_t* q_perm, const int32_t* q_offsets, int Cq, int n_layouts,
                                          void* qbar, hipStream_t stream) {
  if (!Q || !q_perm || !q_offsets || !qbar || B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Cq < 1) return BSA_E_ARG;
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
#define BSA_QC_ARGS B, Hq, Hkv, S, Q, q_perm, q_offsets, Cq, n_layouts, qbar, stream
  if (dtype == BSA_BF16)
    return D == 128 ? launch_query_centroids<bf16_t, 128>(BSA_QC_ARGS) : launch_query_centroids<bf16_t, 64>(BSA_QC_ARGS);
  return D == 128 ? launch_query_centroids<float, 128>(BSA_QC_ARGS) : launch_query_centroids<float, 64>(BSA_QC_ARGS);
#undef BSA_QC_ARGS
}
