// Key/value packing for block-sparse attention, fused with the cluster centroids.
//
// "Partition the Support, Reconstruct the Residual" (summary page): keys and values are
// permuted into group-major order before the sparse kernel.  "Sparse-block compensation",
// section "SVG-EAR -- centroid compensation": each key cluster's key and value means and its
// size.
//
// One pass over K and V per (batch, K/V head) writes, for every key cluster, its keys in
// tiles of 64 (the last tile of a cluster zero-filled), in the layout the attention kernel
// copies straight into LDS:
//   K tile   [64 keys][D]   (input element type)
//   V^T tile [D][64 keys]   (keys of each 16-key group in the order 0-3, 8-11, 4-7, 12-15,
//                            the order in which the attention kernel's P V product takes
//                            them; bfloat16 inputs: float16 when every value of the tile is
//                            below 2^16 in magnitude -- bfloat16 values there are at most
//                            65280, inside the float16 range -- and some is at least 2^-8,
//                            so that values losing float16 precision are negligible next to
//                            the tile's largest; else bfloat16.  float32 inputs: float32)
// and the per-tile format flag.  The same pass sums each cluster's keys and values for the
// centroids, which are packed afterwards as extra tiles (K-bar rounded to the input type,
// V-bar like V), with log2 n_c for each centroid column.  A caller holding its own centroids
// and counts (the page API takes them as inputs) packs the token tiles alone and has its
// centroids and counts packed instead.
#include "pack.hpp"

#include <type_traits>

namespace bsa {
namespace {

constexpr int kPackThreads = 256;

// tile_off[c] = first tile of cluster c (exclusive prefix of ceil(n_c / 64)); clears the
// per-head format summary hmix[nh]; clog2n[c] = log2 of the centroid count (the caller's
// counts when given, else the cluster size), -inf for 0.  One workgroup per key layout.
__global__ __launch_bounds__(1024) void tile_offsets_kernel(const int32_t* __restrict__ offsets, int C,
                                                             const int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ tile_off, int32_t* __restrict__ hmix,
                                                             int nh, float* __restrict__ clog2n) {
  __shared__ int32_t part[1024];
  const size_t lay = blockIdx.x;
  offsets += lay * (C + 1);
  tile_off += lay * (C + 1);
  clog2n += lay * C;
  if (counts != nullptr) counts += lay * C;
  if (lay == 0)
    for (int i = threadIdx.x; i < nh; i += blockDim.x) hmix[i] = 0;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    const int n = counts != nullptr ? counts[c] : offsets[c + 1] - offsets[c];
    clog2n[c] = n > 0 ? __log2f(static_cast<float>(n)) : -INFINITY;
  }
  const int per = (C + blockDim.x - 1) / blockDim.x;
  const int c0 = threadIdx.x * per;
  int32_t run = 0;
  for (int c = c0; c < c0 + per && c < C; ++c) run += (offsets[c + 1] - offsets[c] + kPackTile - 1) / kPackTile;
  part[threadIdx.x] = run;
  __syncthreads();
  for (int d = 1; d < static_cast<int>(blockDim.x); d <<= 1) {
    const int32_t add = threadIdx.x >= static_cast<unsigned>(d) ? part[threadIdx.x - d] : 0;
    __syncthreads();
    part[threadIdx.x] += add;
    __syncthreads();
  }
  int32_t off = part[threadIdx.x] - run;
  for (int c = c0; c < c0 + per && c < C; ++c) {
    tile_off[c] = off;
    off += (offsets[c + 1] - offsets[c] + kPackTile - 1) / kPackTile;
  }
  if (threadIdx.x == blockDim.x - 1) tile_off[C] = part[blockDim.x - 1];
}

__device__ __forceinline__ uint32_t bf16_exp(uint16_t b) { return (b >> 7) & 0xffu; }

// Key held at position `pos` of a V^T row: positions 4-7 and 8-11 of each 16-key group are
// swapped (order 0-3, 8-11, 4-7, 12-15), an involution.
__device__ __forceinline__ int vt_key(int pos) { return (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1); }

// One workgroup per (key cluster, batch x K/V head).  V is staged in LDS in its own 16-bit
// encoding for bfloat16 inputs (float32 otherwise); the buffer for the centroid reduction
// reuses that memory once the last tile is written, so a workgroup needs about 17 KB of LDS
// (bfloat16, D = 128) and many are resident per CU.
template <typename T, int D>
struct PackSmem {
  using VS = std::conditional_t<sizeof(T) == 2, uint16_t, float>;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  static constexpr int CPR = D / EPC;
  static constexpr int kKeyGroups = kPackThreads / CPR;
  static constexpr int VROW = D + 16 / static_cast<int>(sizeof(VS));  // padded row (elements)
  static constexpr int V_BYTES = kPackTile * VROW * static_cast<int>(sizeof(VS));
  static constexpr int RED_BYTES = 2 * kKeyGroups * D * 4;
  static constexpr int BYTES = V_BYTES > RED_BYTES ? V_BYTES : RED_BYTES;
};

template <typename T, int D>
__global__ __launch_bounds__(kPackThreads) void pack_cluster_kernel(
    const T* __restrict__ K, const T* __restrict__ V, int S, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ offsets, int C, int nl, const int32_t* __restrict__ tile_off, int tiles_per_head,
    T* __restrict__ Kp, uint16_t* __restrict__ Vtp16, float* __restrict__ Vtp32, uint8_t* __restrict__ flags,
    int32_t* __restrict__ hmix, float* __restrict__ Kbar, float* __restrict__ Vbar) {
  // Kbar == nullptr: the caller gives the centroids; only the token tiles are written.
  using M = PackSmem<T, D>;
  using VS = typename M::VS;
  constexpr int EPC = M::EPC;                             // elements per 16-byte chunk
  constexpr int CPR = M::CPR;                             // chunks per row
  constexpr int kItems = kPackTile * CPR / kPackThreads;  // (key, chunk) items per thread
  constexpr int kKeyGroups = M::kKeyGroups;               // keys covered in one pass
  __shared__ __align__(16) unsigned char smem[M::BYTES];
  // Largest bfloat16 exponent of the tile's values, one slot per tile parity: slot j & 1 is
  // cleared at the top of tile j, when every wave has passed tile j-1's first barrier and so
  // has finished reading the slot's value of tile j-2.  (With one slot, a wave still reading
  // tile j's value after the second barrier could see thread 0's reset for tile j+1.)
  __shared__ uint32_t emax_s[2];
  VS* vt = reinterpret_cast<VS*>(smem);                      // [kPackTile][VROW]: the tile's V
  float* red = reinterpret_cast<float*>(smem);               // [2][kKeyGroups][D], after the tiles
  const int c = blockIdx.x;
  const size_t bh = blockIdx.y;
  const size_t lay = layout_of(nl, bh);  // this head's key layout
  perm += lay * S;
  offsets += lay * (C + 1);
  tile_off += lay * (C + 1);
  const int lo = offsets[c], n = offsets[c + 1] - lo;
  const int t = threadIdx.x, ch = t % CPR, kg = t / CPR;
  const T* Kh = K + bh * static_cast<size_t>(S) * D;
  const T* Vh = V + bh * static_cast<size_t>(S) * D;
  float ks[EPC], vs[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) ks[e] = vs[e] = 0.0f;
  const int ntiles = (n + kPackTile - 1) / kPackTile;
  // Loads are issued in batches: the token indices of all of a thread's rows of a tile, then
  // all their K and V chunks, so that each tile costs one round trip for the indices and one
  // for the rows.  The rows of tile j+1 are requested before tile j is processed.
  auto load_idx = [&](int j, int (&p)[kItems]) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int r = j * kPackTile + kg + i * kKeyGroups;
      p[i] = r < n ? perm[lo + r] : -1;
    }
  };
  // Rows past the cluster read token 0 (always present) and are replaced by zeros where they
  // are used: the loads are unconditional, so none of them waits behind a branch.
  auto load_rows = [&](const int (&p)[kItems], uint4 (&kv)[kItems], uint4 (&vv)[kItems]) {
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const size_t row = static_cast<size_t>(p[i] >= 0 ? p[i] : 0) * D + ch * EPC;
      kv[i] = *reinterpret_cast<const uint4*>(Kh + row);
      vv[i] = *reinterpret_cast<const uint4*>(Vh + row);
    }
  };
  uint4 kv[kItems], vv[kItems];
  if (ntiles > 0) {
    int p0[kItems];
    load_idx(0, p0);
    load_rows(p0, kv, vv);
  }
  for (int j = 0; j < ntiles; ++j) {
    const size_t tile = bh * tiles_per_head + tile_off[c] + j;
    uint32_t* emax_slot = &emax_s[j & 1];
    if (t == 0) *emax_slot = 0;
    uint4 kn[kItems], vn[kItems];
    if (j + 1 < ntiles) {
      int p1[kItems];
      load_idx(j + 1, p1);
      load_rows(p1, kn, vn);
    }
    // LDS-only barriers in the loop: the compiler's barrier would also wait for the loads of
    // tile j+1 (the registers of tile j are awaited where they are used).
    pipe_barrier();  // the slot cleared; the previous tile's V^T reads are done
    uint32_t emax = 0;
#pragma unroll
    for (int i = 0; i < kItems; ++i) {
      const int key = kg + i * kKeyGroups;
      const bool in = j * kPackTile + key < n;
      const uint4 zero = make_uint4(0, 0, 0, 0);
      const uint4 kq = in ? kv[i] : zero, vq = in ? vv[i] : zero;
      *reinterpret_cast<uint4*>(Kp + (tile * kPackTile + key) * D + ch * EPC) = kq;
      const T* ke = reinterpret_cast<const T*>(&kq);
      const T* ve = reinterpret_cast<const T*>(&vq);
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        ks[e] += to_f32(ke[e]);
        vs[e] += to_f32(ve[e]);
      }
      if constexpr (sizeof(T) == 2) {
        *reinterpret_cast<uint4*>(vt + key * M::VROW + ch * EPC) = vq;
#pragma unroll
        for (int e = 0; e < EPC; ++e) emax = max(emax, bf16_exp(ve[e].bits));
      } else {
        *reinterpret_cast<uint4*>(vt + key * M::VROW + ch * EPC) = vq;
      }
    }
    if constexpr (sizeof(T) == 2) atomicMax(emax_slot, emax);
    pipe_barrier();
    // V^T rows: [d][64 keys], 16-bit (8 keys per 16-byte chunk) or float32 (4 keys).  A wave
    // takes 32 (16) consecutive d and 2 (4) neighbouring chunks of keys: its LDS reads then
    // fall in distinct banks (key rows are D + 8 (D + 4) elements apart), and each V^T row
    // gets 32 (64) contiguous bytes per store.
    if constexpr (sizeof(T) == 2) {
      const uint32_t tile_emax = *emax_slot;
      const bool f16 = tile_emax <= 142u && tile_emax >= 119u;  // bfloat16 exponent 142: [2^15, 2^16); 119: 2^-8
      if (t == 0) {
        flags[tile] = f16 ? 1 : 0;
        if (!f16) atomicOr(&hmix[bh], 1);
      }
      for (int idx = t; idx < D * (kPackTile / 8); idx += kPackThreads) {
        const int d = (idx / 2) % D, k0 = (2 * (idx / (2 * D)) + idx % 2) * 8;
        uint32_t w[4];
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const uint32_t a = vt[vt_key(k0 + 2 * p) * M::VROW + d], b = vt[vt_key(k0 + 2 * p + 1) * M::VROW + d];
          w[p] = f16 ? pack_f16x2(__uint_as_float(a << 16), __uint_as_float(b << 16)) : (a | (b << 16));
        }
        *reinterpret_cast<uint4*>(Vtp16 + (tile * D + d) * kPackTile + k0) = make_uint4(w[0], w[1], w[2], w[3]);
      }
    } else {
      if (t == 0) flags[tile] = 1;
      for (int idx = t; idx < D * (kPackTile / 4); idx += kPackThreads) {
        const int d = (idx / 4) % D, k0 = (4 * (idx / (4 * D)) + idx % 4) * 4;
        *reinterpret_cast<f32x4*>(Vtp32 + (tile * D + d) * kPackTile + k0) =
            f32x4{vt[vt_key(k0) * M::VROW + d], vt[vt_key(k0 + 1) * M::VROW + d], vt[vt_key(k0 + 2) * M::VROW + d],
                  vt[vt_key(k0 + 3) * M::VROW + d]};
      }
    }
    if (j + 1 < ntiles) {
#pragma unroll
      for (int i = 0; i < kItems; ++i) {
        kv[i] = kn[i];
        vv[i] = vn[i];
      }
    }
  }
  if (Kbar == nullptr) return;  // (uniform over the workgroup)
  __syncthreads();  // the last tile's V^T reads are done before red reuses the memory
  // Centroid means: reduce the per-thread column sums over the key groups.
#pragma unroll
  for (int e = 0; e < EPC; ++e) {
    red[kg * D + ch * EPC + e] = ks[e];
    red[(kKeyGroups + kg) * D + ch * EPC + e] = vs[e];
  }
  __syncthreads();
  const float inv = n > 0 ? 1.0f / static_cast<float>(n) : 0.0f;
  for (int e = t; e < 2 * D; e += kPackThreads) {
    const int which = e / D, d = e % D;
    float s = 0.0f;
    for (int g = 0; g < kKeyGroups; ++g) s += red[(which * kKeyGroups + g) * D + d];
    (which == 0 ? Kbar : Vbar)[(bh * C + c) * D + d] = s * inv;
  }
}

// Centroid tiles: K-bar rounded to the input type, V-bar^T like value tiles.  One workgroup
// per (64-centroid tile, batch x K/V head).
template <typename T, int D>
__global__ __launch_bounds__(kPackThreads) void pack_centroid_kernel(
    const float* __restrict__ Kbar, const float* __restrict__ Vbar, int C, int tiles_per_head, int first_tile,
    T* __restrict__ Kp, uint16_t* __restrict__ Vtp16, float* __restrict__ Vtp32, uint8_t* __restrict__ flags,
    int32_t* __restrict__ hmix) {
  __shared__ float vmax_s;
  const int j = blockIdx.x;
  const size_t bh = blockIdx.y;
  const size_t tile = bh * tiles_per_head + first_tile + j;
  const float* Kb = Kbar + bh * C * D;
  const float* Vb = Vbar + bh * C * D;
  const int t = threadIdx.x;
  if (t == 0) vmax_s = 0.0f;
  __syncthreads();
  float vmax = 0.0f;
  for (int idx = t; idx < kPackTile * D; idx += kPackThreads) {
    const int key = idx / D, d = idx % D;
    const int cc = j * kPackTile + key;
    Kp[(tile * kPackTile + key) * D + d] = from_f32<T>(cc < C ? Kb[static_cast<size_t>(cc) * D + d] : 0.0f);
    if (cc < C) vmax = fmaxf(vmax, fabsf(Vb[static_cast<size_t>(cc) * D + d]));
  }
  // The range test is on float values here: every |v| at most the float16 maximum, some
  // |v| >= 2^-8.
  atomicMax(reinterpret_cast<unsigned int*>(&vmax_s), __float_as_uint(vmax));  // non-negative floats order as uints
  __syncthreads();
  if constexpr (sizeof(T) == 2) {
    const bool f16 = vmax_s <= 65504.0f && vmax_s >= 0.00390625f;
    if (t == 0) {
      flags[tile] = f16 ? 1 : 0;
      if (!f16) atomicOr(&hmix[bh], 1);
    }
    for (int idx = t; idx < D * kPackTile; idx += kPackThreads) {
      const int d = idx / kPackTile, pos = idx % kPackTile;
      const int cc = j * kPackTile + vt_key(pos);
      const float x = cc < C ? Vb[static_cast<size_t>(cc) * D + d] : 0.0f;
      Vtp16[(tile * D + d) * kPackTile + pos] =
          f16 ? __builtin_bit_cast(uint16_t, static_cast<_Float16>(x)) : f32_to_bf16(x);
    }
  } else {
    if (t == 0) flags[tile] = 1;
    for (int idx = t; idx < D * kPackTile; idx += kPackThreads) {
      const int d = idx / kPackTile, pos = idx % kPackTile;
      const int cc = j * kPackTile + vt_key(pos);
      Vtp32[(tile * D + d) * kPackTile + pos] = cc < C ? Vb[static_cast<size_t>(cc) * D + d] : 0.0f;
    }
  }
}

// given == true: Kbar, Vbar and counts are the caller's (read only).  nl key layouts (1 or
// B * Hkv): perm [nl][S], offsets [nl][C + 1], counts [nl][C].
template <typename T, int D>
bsa_status launch_pack(int B, int Hkv, int S, const void* K, const void* V, const int32_t* perm,
                       const int32_t* offsets, int C, int nl, const float* Kbar, const float* Vbar,
                       const int32_t* counts, bool given, void* packed, hipStream_t stream) {
  const PackLayout L = pack_layout(B, Hkv, S, D, C, sizeof(T), nl);
  unsigned char* base = static_cast<unsigned char*>(packed);
  int32_t* tile_off = reinterpret_cast<int32_t*>(base + L.tile_off);
  uint8_t* flags = base + L.flags;
  int32_t* hmix = reinterpret_cast<int32_t*>(base + L.hmix);
  T* Kp = reinterpret_cast<T*>(base + L.k);
  uint16_t* V16 = reinterpret_cast<uint16_t*>(base + L.v);
  float* V32 = reinterpret_cast<float*>(base + L.v);
  float* clog2n = reinterpret_cast<float*>(base + L.clog2n);
  hipLaunchKernelGGL(tile_offsets_kernel, dim3(nl), dim3(1024), 0, stream, offsets, C, given ? counts : nullptr,
                     tile_off, hmix, B * Hkv, clog2n);
  hipLaunchKernelGGL((pack_cluster_kernel<T, D>), dim3(C, B * Hkv), dim3(kPackThreads), 0, stream,
                     static_cast<const T*>(K), static_cast<const T*>(V), S, perm, offsets, C, nl, tile_off,
                     L.tiles_per_head,
                     Kp, V16, V32, flags, hmix, given ? nullptr : const_cast<float*>(Kbar),
                     given ? nullptr : const_cast<float*>(Vbar));
  hipLaunchKernelGGL((pack_centroid_kernel<T, D>), dim3(L.centroid_tiles, B * Hkv), dim3(kPackThreads), 0, stream,
                     Kbar, Vbar, C, L.tiles_per_head, L.first_centroid_tile, Kp, V16, V32, flags, hmix);
  return launch_status();
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_kv_pack_workspace_size(int B, int Hkv, int S, int D, int dtype, int C, int n_layouts,
                                                 size_t* bytes) {
  if (!bytes || B < 1 || Hkv < 1 || S < 1 || C < 1) return BSA_E_ARG;
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (C > 32767) return BSA_E_UNSUPPORTED;
  *bytes = pack_layout(B, Hkv, S, D, C, dtype_size(dtype), n_layouts).total;
  return BSA_OK;
}

extern "C" bsa_status bsa_kv_pack(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V,
                                  const int32_t* perm, const int32_t* offsets, int C, int n_layouts, float* Kbar,
                                  float* Vbar, void* packed, size_t packed_bytes, hipStream_t stream) {
  size_t need = 0;
  bsa_status st = bsa_kv_pack_workspace_size(B, Hkv, S, D, dtype, C, n_layouts, &need);
  if (st != BSA_OK) return st;
  if (!K || !V || !perm || !offsets || !Kbar || !Vbar) return BSA_E_ARG;
  if (!packed || packed_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hkv > 65535) return BSA_E_UNSUPPORTED;
#define BSA_PACK_ARGS B, Hkv, S, K, V, perm, offsets, C, n_layouts, Kbar, Vbar, nullptr, false, packed, stream
  if (dtype == BSA_BF16)
    return D == 128 ? launch_pack<bf16_t, 128>(BSA_PACK_ARGS) : launch_pack<bf16_t, 64>(BSA_PACK_ARGS);
  return D == 128 ? launch_pack<float, 128>(BSA_PACK_ARGS) : launch_pack<float, 64>(BSA_PACK_ARGS);
#undef BSA_PACK_ARGS
}

extern "C" bsa_status bsa_kv_pack_centroids(int B, int Hkv, int S, int D, int dtype, const void* K, const void* V,
                                            const int32_t* perm, const int32_t* offsets, int C, int n_layouts,
                                            const float* Kbar, const float* Vbar, const int32_t* counts,
                                            void* packed, size_t packed_bytes, hipStream_t stream) {
  size_t need = 0;
  bsa_status st = bsa_kv_pack_workspace_size(B, Hkv, S, D, dtype, C, n_layouts, &need);
  if (st != BSA_OK) return st;
  if (!K || !V || !perm || !offsets || !Kbar || !Vbar || !counts) return BSA_E_ARG;
  if (!packed || packed_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hkv > 65535) return BSA_E_UNSUPPORTED;
#define BSA_PACK_ARGS B, Hkv, S, K, V, perm, offsets, C, n_layouts, Kbar, Vbar, counts, true, packed, stream
  if (dtype == BSA_BF16)
    return D == 128 ? launch_pack<bf16_t, 128>(BSA_PACK_ARGS) : launch_pack<bf16_t, 64>(BSA_PACK_ARGS);
  return D == 128 ? launch_pack<float, 128>(BSA_PACK_ARGS) : launch_pack<float, 64>(BSA_PACK_ARGS);
#undef BSA_PACK_ARGS
}
