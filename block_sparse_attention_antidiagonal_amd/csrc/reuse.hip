// Head-wise temporal mask reuse: pooled Q/K summaries, drift and refresh decision, cache update.
//
// "Dynamic block masks and head-wise mask reuse", section "HEART -- head-wise temporal mask
// reuse" (Temporal Mask Reuse): a head keeps the token means of Q and K from the step where
// its mask was last built; its drift is the L1 distance of the current means from those,
// summed over Q and K; above a threshold the mask is rebuilt and the anchor moves.  A layer
// override refreshes no head when fewer than 40% of the heads ask, every head when more than
// 80% do.  Section "What mlx-arsenal ships": the summary, the drift (optionally relative) and
// a two-phase cache as separate steps.  Section "Deviations from the papers": the relative
// drift divides by the anchor's L1 norm.
//
// The summary pass is bound by HBM: it reads Q and K once.  Workgroups own a chunk of 2048 rows
// of one head; 16-byte loads, a row's chunks on consecutive lanes, float32 sums; the chunk
// partials are summed by a second kernel in a fixed order, so results do not depend on timing.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kPoolThreads = 256;
constexpr int kPoolRows = 2048;  // rows of one head per workgroup

// Partial sums over one chunk of rows of one head (heads 0..Hq-1 of Q, then Hkv heads of K):
// part[(head * nchunk + chunk) * D + d].
template <typename T, int D>
__global__ __launch_bounds__(kPoolThreads) void pooled_partial_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                                      int Hq, int Hkv, int S, int nchunk,
                                                                      float* __restrict__ part) {
  constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;                            // chunks per row
  constexpr int SLOTS = kPoolThreads / CPR;               // rows read side by side
  __shared__ float red[SLOTS][D + 1];
  const int chunk = blockIdx.x;
  const int hh = blockIdx.y;  // b * (Hq + Hkv) + head
  const int Ht = Hq + Hkv;
  const int b = hh / Ht, head = hh % Ht;
  const T* base = head < Hq ? Q + (static_cast<size_t>(b) * Hq + head) * S * D
                            : K + (static_cast<size_t>(b) * Hkv + (head - Hq)) * S * D;
  const int c = threadIdx.x % CPR, slot = threadIdx.x / CPR;
  const int r0 = chunk * kPoolRows;
  const int r1 = min(S, r0 + kPoolRows);
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
#pragma unroll 4
  for (int r = r0 + slot; r < r1; r += SLOTS) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + static_cast<size_t>(r) * D + c * EPC);
    if constexpr (sizeof(T) == 2) {
      const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        acc[2 * p] += __uint_as_float(w[p] << 16);
        acc[2 * p + 1] += __uint_as_float(w[p] & 0xffff0000u);
      }
    } else {
      acc[0] += __uint_as_float(v.x);
      acc[1] += __uint_as_float(v.y);
      acc[2] += __uint_as_float(v.z);
      acc[3] += __uint_as_float(v.w);
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) red[slot][c * EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float s = 0.0f;
#pragma unroll 4
    for (int k = 0; k < SLOTS; ++k) s += red[k][threadIdx.x];
    part[(static_cast<size_t>(hh) * nchunk + chunk) * D + threadIdx.x] = s;
  }
}

// One workgroup per (batch, mask head), one thread per feature: the summary of mask head m is
// the mean over the tokens of the query heads (and key heads) its mask serves.
__global__ void pooled_finalize_kernel(const float* __restrict__ part, int Hq, int Hkv, int Hm, int S, int D,
                                       int nchunk, float* __restrict__ qbar, float* __restrict__ kbar) {
  const int bm = blockIdx.x;
  const int b = bm / Hm, m = bm % Hm;
  const int d = threadIdx.x;
  if (d >= D) return;
  const int G = Hq / Hkv;
  int q0, q1, k0, k1;  // query heads [q0, q1), key heads [k0, k1)
  if (Hm == Hq) {
    q0 = m; q1 = m + 1; k0 = m / G; k1 = k0 + 1;
  } else if (Hm == Hkv) {
    q0 = m * G; q1 = q0 + G; k0 = m; k1 = m + 1;
  } else {
    q0 = 0; q1 = Hq; k0 = 0; k1 = Hkv;
  }
  const int Ht = Hq + Hkv;
  auto head_sum = [&](int head) {
    const float* p = part + (static_cast<size_t>(b) * Ht + head) * nchunk * D + d;
    float s = 0.0f;
    for (int c = 0; c < nchunk; ++c) s += p[static_cast<size_t>(c) * D];
    return s;
  };
  float sq = 0.0f, sk = 0.0f;
  for (int h = q0; h < q1; ++h) sq += head_sum(h);
  for (int h = k0; h < k1; ++h) sk += head_sum(Hq + h);
  qbar[static_cast<size_t>(bm) * D + d] = sq / (static_cast<float>(q1 - q0) * static_cast<float>(S));
  kbar[static_cast<size_t>(bm) * D + d] = sk / (static_cast<float>(k1 - k0) * static_cast<float>(S));
}

// One workgroup per batch entry: drift of every mask head from its anchor, the per-head
// request (drift > delta) and the layer override over the entry's Hm heads.  The override
// compares counts, 10 * asking < 4 * Hm and 10 * asking > 8 * Hm, which is the 40% / 80%
// test without rounding the fraction.  Each thread revisits only the heads it wrote.
constexpr int kDecideThreads = 256;
__global__ __launch_bounds__(kDecideThreads) void reuse_decide_kernel(
    int Hm, int D, const float* __restrict__ qbar, const float* __restrict__ kbar, const float* __restrict__ anchor_q,
    const float* __restrict__ anchor_k, int have_anchor, float delta, int relative, int gate, float* __restrict__ drift,
    uint8_t* __restrict__ refresh) {
  __shared__ int asking;
  const int b = blockIdx.x;
  if (threadIdx.x == 0) asking = 0;
  __syncthreads();
  for (int m = threadIdx.x; m < Hm; m += kDecideThreads) {
    const size_t i = static_cast<size_t>(b) * Hm + m;
    float dist = 0.0f;
    if (have_anchor) {
      float norm = 0.0f;
      const size_t o = i * D;
      for (int d = 0; d < D; ++d) {
        dist += fabsf(qbar[o + d] - anchor_q[o + d]) + fabsf(kbar[o + d] - anchor_k[o + d]);
        norm += fabsf(anchor_q[o + d]) + fabsf(anchor_k[o + d]);
      }
      if (relative) dist = norm > 0.0f ? dist / norm : (dist > 0.0f ? INFINITY : 0.0f);
    }
    if (drift != nullptr) drift[i] = dist;
    const bool want = !have_anchor || dist > delta;
    refresh[i] = want ? 1 : 0;
    if (have_anchor && want) atomicAdd(&asking, 1);
  }
  __syncthreads();
  if (!have_anchor || !gate) return;
  const int n = asking;
  const bool none = 10 * n < 4 * Hm;
  const bool all = 10 * n > 8 * Hm;
  if (!none && !all) return;
  for (int m = threadIdx.x; m < Hm; m += kDecideThreads) refresh[static_cast<size_t>(b) * Hm + m] = all ? 1 : 0;
}

// Cache update, one workgroup slice per (batch, mask head): heads with refresh[bm] take the new
// mask rows and their anchors move to the current summaries; the others are left as they are.
constexpr int kUpdateThreads = 256;
constexpr int kUpdateSplit = 8;  // workgroups per head
__device__ __forceinline__ void copy_bytes(unsigned char* __restrict__ dst, const unsigned char* __restrict__ src,
                                           size_t n, int part, int parts) {
  const bool vec = ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src) | n) & 15) == 0;
  if (vec) {
    const size_t n16 = n / 16;
    for (size_t i = static_cast<size_t>(part) * kUpdateThreads + threadIdx.x; i < n16;
         i += static_cast<size_t>(parts) * kUpdateThreads)
      reinterpret_cast<uint4*>(dst)[i] = reinterpret_cast<const uint4*>(src)[i];
  } else {
    for (size_t i = static_cast<size_t>(part) * kUpdateThreads + threadIdx.x; i < n;
         i += static_cast<size_t>(parts) * kUpdateThreads)
      dst[i] = src[i];
  }
}
__global__ __launch_bounds__(kUpdateThreads) void reuse_update_kernel(
    int Cq, int Ck, int D, const uint8_t* __restrict__ refresh, const float* __restrict__ qbar,
    const float* __restrict__ kbar, const uint8_t* __restrict__ new_keep, const int32_t* __restrict__ new_count,
    const int16_t* __restrict__ new_idx, uint8_t* __restrict__ keep, int32_t* __restrict__ kv_count,
    int16_t* __restrict__ kv_idx, float* __restrict__ anchor_q, float* __restrict__ anchor_k) {
  const int bm = blockIdx.x, part = blockIdx.y;
  if (!refresh[bm]) return;
  const size_t rows = static_cast<size_t>(Cq) * Ck;
  if (new_keep != nullptr) {
    copy_bytes(keep + bm * rows, new_keep + bm * rows, rows, part, kUpdateSplit);
    copy_bytes(reinterpret_cast<unsigned char*>(kv_idx + bm * rows),
               reinterpret_cast<const unsigned char*>(new_idx + bm * rows), rows * sizeof(int16_t), part,
               kUpdateSplit);
    copy_bytes(reinterpret_cast<unsigned char*>(kv_count + static_cast<size_t>(bm) * Cq),
               reinterpret_cast<const unsigned char*>(new_count + static_cast<size_t>(bm) * Cq),
               static_cast<size_t>(Cq) * sizeof(int32_t), part, kUpdateSplit);
  }
  if (part == 0) {
    for (int d = threadIdx.x; d < D; d += kUpdateThreads) {
      anchor_q[static_cast<size_t>(bm) * D + d] = qbar[static_cast<size_t>(bm) * D + d];
      anchor_k[static_cast<size_t>(bm) * D + d] = kbar[static_cast<size_t>(bm) * D + d];
    }
  }
}

inline int pool_chunks(int S) { return (S + kPoolRows - 1) / kPoolRows; }

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_pooled_qk_workspace_size(int B, int Hq, int Hkv, int S, int D, size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || S < 1) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  *bytes = static_cast<size_t>(B) * (Hq + Hkv) * pool_chunks(S) * D * sizeof(float);
  return BSA_OK;
}

extern "C" bsa_status bsa_pooled_qk(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                                    int Hm, float* qbar, float* kbar, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  size_t need = 0;
  const bsa_status st = bsa_pooled_qk_workspace_size(B, Hq, Hkv, S, D, &need);
  if (st != BSA_OK) return st;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (Hm != Hq && Hm != Hkv && Hm != 1) return BSA_E_SHAPE;
  if (!Q || !K || !qbar || !kbar) return BSA_E_ARG;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * (Hq + Hkv) > 65535 || static_cast<long long>(B) * Hm > 0x7fffffff)
    return BSA_E_UNSUPPORTED;
  const int nchunk = pool_chunks(S);
  float* part = static_cast<float*>(ws);
  const dim3 grid(nchunk, B * (Hq + Hkv));
  if (dtype == BSA_BF16) {
    if (D == 128)
      hipLaunchKernelGGL((pooled_partial_kernel<bf16_t, 128>), grid, dim3(kPoolThreads), 0, stream,
                         static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), Hq, Hkv, S, nchunk, part);
    else
      hipLaunchKernelGGL((pooled_partial_kernel<bf16_t, 64>), grid, dim3(kPoolThreads), 0, stream,
                         static_cast<const bf16_t*>(Q), static_cast<const bf16_t*>(K), Hq, Hkv, S, nchunk, part);
  } else {
    if (D == 128)
      hipLaunchKernelGGL((pooled_partial_kernel<float, 128>), grid, dim3(kPoolThreads), 0, stream,
                         static_cast<const float*>(Q), static_cast<const float*>(K), Hq, Hkv, S, nchunk, part);
    else
      hipLaunchKernelGGL((pooled_partial_kernel<float, 64>), grid, dim3(kPoolThreads), 0, stream,
                         static_cast<const float*>(Q), static_cast<const float*>(K), Hq, Hkv, S, nchunk, part);
  }
  hipLaunchKernelGGL(pooled_finalize_kernel, dim3(B * Hm), dim3(D), 0, stream, part, Hq, Hkv, Hm, S, D, nchunk, qbar,
                     kbar);
  return launch_status();
}

extern "C" bsa_status bsa_mask_reuse_decide(int B, int Hm, int D, const float* qbar, const float* kbar,
                                            const float* anchor_q, const float* anchor_k, int have_anchor, float delta,
                                            int relative, int gate, float* drift, uint8_t* refresh,
                                            hipStream_t stream) {
  if (B < 1 || Hm < 1 || D < 1) return BSA_E_ARG;
  if ((have_anchor != 0 && have_anchor != 1) || (relative != 0 && relative != 1) || (gate != 0 && gate != 1))
    return BSA_E_ARG;
  if (!refresh || !qbar || !kbar) return BSA_E_ARG;
  if (have_anchor && (!anchor_q || !anchor_k)) return BSA_E_ARG;
  if (delta != delta) return BSA_E_ARG;  // NaN threshold
  if (Hm > 0x7fffffff / 10) return BSA_E_UNSUPPORTED;
  hipLaunchKernelGGL(reuse_decide_kernel, dim3(B), dim3(kDecideThreads), 0, stream, Hm, D, qbar, kbar, anchor_q,
                     anchor_k, have_anchor, delta, relative, gate, drift, refresh);
  return launch_status();
}

extern "C" bsa_status bsa_mask_reuse_update(int B, int Hm, int Cq, int Ck, int D, const uint8_t* refresh,
                                            const float* qbar, const float* kbar, const uint8_t* new_keep,
                                            const int32_t* new_count, const int16_t* new_idx, uint8_t* keep,
                                            int32_t* kv_count, int16_t* kv_idx, float* anchor_q, float* anchor_k,
                                            hipStream_t stream) {
  if (B < 1 || Hm < 1 || Cq < 1 || Ck < 1 || D < 1) return BSA_E_ARG;
  if (!refresh || !qbar || !kbar || !anchor_q || !anchor_k) return BSA_E_ARG;
  const bool masks = new_keep != nullptr;
  if (masks && (!new_count || !new_idx || !keep || !kv_count || !kv_idx)) return BSA_E_ARG;
  if (!masks && (new_count || new_idx)) return BSA_E_ARG;
  if (static_cast<long long>(B) * Hm > 0x7fffffff) return BSA_E_UNSUPPORTED;
  hipLaunchKernelGGL(reuse_update_kernel, dim3(B * Hm, kUpdateSplit), dim3(kUpdateThreads), 0, stream, Cq, Ck, D,
                     refresh, qbar, kbar, new_keep, new_count, new_idx, keep, kv_count, kv_idx, anchor_q, anchor_k);
  return launch_status();
}
