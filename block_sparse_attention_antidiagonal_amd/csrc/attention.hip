// Block-sparse flash attention with centroid compensation, and exact dense probe rows.
//
// "Sparse-block compensation", sections "The problem" (kept blocks only; hard drop
// renormalizes over kept keys), "SVG-EAR -- centroid compensation" (each skipped key
// cluster adds one column with logit q.kbar_c*scale + log n_c and value vbar_c) and "No LSE
// needed" (the result is one softmax over the extended keys).  Here that softmax is one
// online softmax per query row: centroid columns and kept key tiles stream through the
// same running max and sum, so no mask or log-sum-exp merge is ever materialised.
// "Partition the Support, Reconstruct the Residual" (summary page), Probe-Fitted Residual
// Reconstruction: probe rows attend to every key (bsa_probe_attention); when a correction
// follows, the attention keeps its rows in float32 so that the fit reads the probes' sparse
// rows from them and the correction (bsa_correct) rounds each row once.
//
// Work decomposition (gfx950): a workgroup of 4 waves owns 128 query rows of one query
// cluster (the cluster's rows are gathered through the cluster layout); each wave owns 32
// rows.  Keys stream through LDS in tiles of 64 rows.  Products are computed transposed,
// S^T = K Q^T and O^T += V^T P^T, with 32x32 MFMA tiles, so that in the accumulator layout
// every lane holds one query row's values: the row max/sum need one exchange between the
// two 32-lane halves and the P tile feeds the second product without leaving registers.
#include "common.hpp"
#include "pack.hpp"

#include <mutex>
#include <type_traits>

namespace bsa {
namespace {

constexpr int kNK = 64;        // keys per LDS tile
constexpr int kRowsWG = 128;   // query rows per workgroup
constexpr int kThreads = 256;  // 4 waves
constexpr float kRescaleSlack = 8.0f;  // log2 units the running max may lag (p <= 256)
constexpr int kFlagBytes = 32;         // per-wave tile flags at the end of LDS (4 waves x 2 ints)
// Instruction classes of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedMfma = 0x008;
constexpr int kSchedDsRead = 0x100;

template <typename T, int D>
struct Cfg {
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));  // elements per 16-byte chunk
  static constexpr int CPR = D / EPC;                            // chunks per row
  static constexpr int KPAD = EPC;                               // K row padding (16 B)
  static constexpr int VPAD = sizeof(T) == 2 ? 4 : 4;            // V^T row padding (8 B bf16, 16 B fp32)
  static constexpr int KROW = D + KPAD;
  static constexpr int VROW = kNK + VPAD;
  static constexpr int K_ELEMS = kNK * KROW;
  static constexpr int V_ELEMS = D * VROW;
  static constexpr int ZROW = D + KPAD;  // output staging row
  static constexpr int KV_BYTES = (K_ELEMS + V_ELEMS) * static_cast<int>(sizeof(T));
  static constexpr int Z_BYTES = kRowsWG * ZROW * static_cast<int>(sizeof(T));
  static constexpr int LDS_BYTES = (KV_BYTES > Z_BYTES ? KV_BYTES : Z_BYTES) + kNK * 4;
  static constexpr int DT = D / 32;  // 32-wide output tiles
  static constexpr int KK = D / 16;  // contraction steps of Q K^T
};

// Running softmax state of one wave (32 query rows; lane l holds row l % 32).
template <int D>
struct RowState {
  f32x16 o[D / 32];
  float m;  // running max, log2 units (may lag the true max: < kRescaleSlack, < 14 in tile_step16)
  float l;  // this lane's partial sum (its 16 keys of every 32-key tile)
};

// ----------------------------------------------------------------- tile loaders

// For bfloat16 inputs the V^T tile is stored as float16 when every value fits it (|v| < 2^15)
// and the tile holds at least one value >= 2^-8 (so values that lose float16 precision are
// negligible next to the tile's largest); otherwise the tile is stored as bfloat16.  Each
// wave publishes two flags (any value too large, any value large enough) in LDS; after the
// next barrier every wave reads the same decision.
__device__ __forceinline__ void publish_tile_flags(int* flags, bool big, bool normal) {
  const unsigned long long b = __ballot(big), n = __ballot(normal);
  if ((threadIdx.x & 63) == 0) {
    flags[2 * (threadIdx.x >> 6)] = b != 0;
    flags[2 * (threadIdx.x >> 6) + 1] = n != 0;
  }
}
__device__ __forceinline__ bool tile_fits_f16(const int* flags) {
  const bool big = flags[0] | flags[2] | flags[4] | flags[6];
  const bool normal = flags[1] | flags[3] | flags[5] | flags[7];
  return !big && normal;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// V^T store of one thread's 4 keys x 8 columns (bfloat16 words w[key][pair]).
__device__ __forceinline__ void store_vt_bf16(bf16_t* Vt, int vrow, int d0, int k0, const uint32_t (&w)[4][4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {  // column pair (2p, 2p+1): low halves -> 2p, high halves -> 2p+1
    const uint32_t lo01 = __builtin_amdgcn_perm(w[1][p], w[0][p], 0x05040100u);
    const uint32_t lo23 = __builtin_amdgcn_perm(w[3][p], w[2][p], 0x05040100u);
    const uint32_t hi01 = __builtin_amdgcn_perm(w[1][p], w[0][p], 0x07060302u);
    const uint32_t hi23 = __builtin_amdgcn_perm(w[3][p], w[2][p], 0x07060302u);
    *reinterpret_cast<uint2*>(Vt + (d0 + 2 * p) * vrow + k0) = make_uint2(lo01, lo23);
    *reinterpret_cast<uint2*>(Vt + (d0 + 2 * p + 1) * vrow + k0) = make_uint2(hi01, hi23);
  }
}
__device__ __forceinline__ void store_vt_f16(bf16_t* Vt, int vrow, int d0, int k0, const uint32_t (&w)[4][4]) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    *reinterpret_cast<uint2*>(Vt + (d0 + 2 * p) * vrow + k0) =
        make_uint2(pack_f16x2(bf16_lo(w[0][p]), bf16_lo(w[1][p])), pack_f16x2(bf16_lo(w[2][p]), bf16_lo(w[3][p])));
    *reinterpret_cast<uint2*>(Vt + (d0 + 2 * p + 1) * vrow + k0) =
        make_uint2(pack_f16x2(bf16_hi(w[0][p]), bf16_hi(w[1][p])), pack_f16x2(bf16_hi(w[2][p]), bf16_hi(w[3][p])));
  }
}

// K rows -> Ks[key][d] and V rows -> Vt[d][key] (transposed), zero rows past `nvalid`.
// `row_of(key)` gives the source row offset (in elements) of tile key `key`.  Pass 1 of a
// bfloat16 tile writes V^T as float16 and publishes the fits-float16 flags; if the tile does
// not fit, load_kv_tile_fallback rewrites V^T as bfloat16 after the barrier.
template <typename T, int D, typename RowFn>
__device__ __forceinline__ void load_kv_tile(T* Ks, T* Vt, int* flags, const T* __restrict__ Kh,
                                             const T* __restrict__ Vh, int nvalid, RowFn row_of) {
  using C = Cfg<T, D>;
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < kNK * C::CPR / kThreads; ++i) {
    const int idx = t + i * kThreads;
    const int key = idx / C::CPR, ch = idx % C::CPR;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (key < nvalid) v = *reinterpret_cast<const uint4*>(Kh + row_of(key) + ch * C::EPC);
    *reinterpret_cast<uint4*>(Ks + key * C::KROW + ch * C::EPC) = v;
  }
  // V: each thread transposes a block of 4 keys x EPC columns.
  constexpr int kBlocks = (kNK / 4) * C::CPR;
  uint32_t emax = 0;  // largest exponent field among this thread's bfloat16 values
#pragma unroll
  for (int i = 0; i < (kBlocks + kThreads - 1) / kThreads; ++i) {
    const int idx = t + i * kThreads;
    if (kBlocks % kThreads != 0 && idx >= kBlocks) break;
    const int kq = idx / C::CPR, ch = idx % C::CPR;
    uint4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int key = kq * 4 + k;
      r[k] = key < nvalid ? *reinterpret_cast<const uint4*>(Vh + row_of(key) + ch * C::EPC) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t w[4][4] = {{r[0].x, r[0].y, r[0].z, r[0].w},
                              {r[1].x, r[1].y, r[1].z, r[1].w},
                              {r[2].x, r[2].y, r[2].z, r[2].w},
                              {r[3].x, r[3].y, r[3].z, r[3].w}};
    const int d0 = ch * C::EPC;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int k = 0; k < 4; ++k)
#pragma unroll
        for (int p = 0; p < 4; ++p) emax = max(emax, max((w[k][p] >> 7) & 0xffu, (w[k][p] >> 23) & 0xffu));
      store_vt_f16(Vt, C::VROW, d0, kq * 4, w);
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p)
        *reinterpret_cast<uint4*>(Vt + (d0 + p) * C::VROW + kq * 4) = make_uint4(w[0][p], w[1][p], w[2][p], w[3][p]);
    }
  }
  // bfloat16 exponent 143 is 2^16 > float16 max; exponent 119 is 2^-8.
  if constexpr (sizeof(T) == 2) publish_tile_flags(flags, emax >= 143u, emax >= 119u);
}

template <typename T, int D, typename RowFn>
__device__ __forceinline__ void load_kv_tile_fallback(T* Vt, const T* __restrict__ Vh, int nvalid, RowFn row_of) {
  using C = Cfg<T, D>;
  constexpr int kBlocks = (kNK / 4) * C::CPR;
#pragma unroll 1
  for (int idx = threadIdx.x; idx < kBlocks; idx += kThreads) {
    const int kq = idx / C::CPR, ch = idx % C::CPR;
    uint4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int key = kq * 4 + k;
      r[k] = key < nvalid ? *reinterpret_cast<const uint4*>(Vh + row_of(key) + ch * C::EPC) : make_uint4(0, 0, 0, 0);
    }
    const uint32_t w[4][4] = {{r[0].x, r[0].y, r[0].z, r[0].w},
                              {r[1].x, r[1].y, r[1].z, r[1].w},
                              {r[2].x, r[2].y, r[2].z, r[2].w},
                              {r[3].x, r[3].y, r[3].z, r[3].w}};
    store_vt_bf16(reinterpret_cast<bf16_t*>(Vt), C::VROW, ch * C::EPC, kq * 4, w);
  }
}

// Centroid rows (float32) -> the same LDS layout; bias[key] (log2 units) is log2 n_c for a
// skipped non-empty cluster and -inf otherwise (keep_row == nullptr: every non-empty cluster
// counts as skipped).  bfloat16 inputs: K-bar is rounded to bfloat16; V-bar is stored as
// float16 when the tile fits it (flags as for token tiles), else as bfloat16 by
// load_centroid_fallback.
template <typename T, int D>
__device__ __forceinline__ void load_centroid_tile(T* Ks, T* Vt, float* bias, int* flags, const float* __restrict__ Kb,
                                                   const float* __restrict__ Vb, int c0, int Ck,
                                                   const int32_t* __restrict__ k_offsets,
                                                   const uint8_t* __restrict__ keep_row) {
  using C = Cfg<T, D>;
  const int t = threadIdx.x;
  constexpr int kGroups = D / 8;  // 8 floats per item
#pragma unroll 1
  for (int idx = t; idx < kNK * kGroups; idx += kThreads) {
    const int key = idx / kGroups, g = idx % kGroups;
    const int c = c0 + key;
    float x[8];
    if (c < Ck) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(Kb + static_cast<size_t>(c) * D + g * 8);
      const f32x4 b = *reinterpret_cast<const f32x4*>(Kb + static_cast<size_t>(c) * D + g * 8 + 4);
      x[0] = a[0]; x[1] = a[1]; x[2] = a[2]; x[3] = a[3];
      x[4] = b[0]; x[5] = b[1]; x[6] = b[2]; x[7] = b[3];
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) x[i] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) Ks[key * C::KROW + g * 8 + i] = from_f32<T>(x[i]);
  }
  float vmax = 0.0f;
#pragma unroll 2
  for (int idx = t; idx < kNK * D; idx += kThreads) {
    const int key = idx % kNK, d = idx / kNK;
    const int c = c0 + key;
    const float x = c < Ck ? Vb[static_cast<size_t>(c) * D + d] : 0.0f;
    if constexpr (sizeof(T) == 2) {
      vmax = fmaxf(vmax, fabsf(x));
      const _Float16 hx = static_cast<_Float16>(x);
      Vt[d * C::VROW + key].bits = __builtin_bit_cast(uint16_t, hx);
    } else {
      Vt[d * C::VROW + key] = from_f32<T>(x);
    }
  }
  if constexpr (sizeof(T) == 2) publish_tile_flags(flags, !(vmax < 32768.0f), vmax >= 0.00390625f);
  if (t < kNK) {
    const int c = c0 + t;
    float b = -INFINITY;
    if (c < Ck) {
      const int n = k_offsets[c + 1] - k_offsets[c];
      if (n > 0 && (keep_row == nullptr || keep_row[c] == 0)) b = __log2f(static_cast<float>(n));
    }
    bias[t] = b;
  }
}

template <typename T, int D>
__device__ __forceinline__ void load_centroid_fallback(T* Vt, const float* __restrict__ Vb, int c0, int Ck) {
  using C = Cfg<T, D>;
#pragma unroll 2
  for (int idx = threadIdx.x; idx < kNK * D; idx += kThreads) {
    const int key = idx % kNK, d = idx / kNK;
    const int c = c0 + key;
    Vt[d * C::VROW + key] = from_f32<T>(c < Ck ? Vb[static_cast<size_t>(c) * D + d] : 0.0f);
  }
}

// ----------------------------------------------------------------- LDS tile layouts

// Padded rows (tiles stored by the threads themselves): K rows of D + 16 B, V^T rows of
// 64 keys + 8 B (bfloat16) or 16 B (float32), keys in natural order.
template <typename T, int D>
struct PaddedLds {
  using C = Cfg<T, D>;
  static __device__ __forceinline__ void kfrag(Frag<T>& f, const T* Ks, int row, int kk, int h) {
    load_frag(f, Ks + row * C::KROW + kk * 16 + 8 * h);
  }
  static __device__ __forceinline__ void vfrag(Frag<T>& f, const T* Vt, int d, int ks, int h) {
    load_frag_split(f, Vt + d * C::VROW + ks * 16 + 4 * h);
  }
  static __device__ __forceinline__ void vfrag16(Frag16& f, const T* Vt, int d, int ks, int h) {
    load_frag_split(f, reinterpret_cast<const bf16_t*>(Vt + d * C::VROW + ks * 16 + 4 * h));
  }
};

// Unpadded rows with the XOR chunk swizzle (tiles copied from the packed buffer straight
// into LDS).  V^T rows hold the keys of each 16-key group in the order 0-3, 8-11, 4-7,
// 12-15, so the eight keys one lane needs in a P V step are one contiguous 16 bytes.
template <typename T, int D>
struct SwzLds {
  static constexpr int KROWB = D * static_cast<int>(sizeof(T));
  static constexpr int VROWB = kNK * static_cast<int>(sizeof(T));
  static constexpr int K_BYTES = kNK * KROWB;
  static constexpr int V_BYTES = D * VROWB;
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  using SK = Swz<KROWB>;
  using SV = Swz<VROWB>;
  template <typename S, typename F>
  static __device__ __forceinline__ void frag(F& f, const void* base, int row, int e0) {
    if constexpr (sizeof(T) == 2) {
      f.v = __builtin_bit_cast(decltype(f.v), *S::chunk(base, row, e0 / EPC));
    } else {
      const f32x4 lo = __builtin_bit_cast(f32x4, *S::chunk(base, row, e0 / EPC));
      const f32x4 hi = __builtin_bit_cast(f32x4, *S::chunk(base, row, e0 / EPC + 1));
      f.v = f32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  static __device__ __forceinline__ void kfrag(Frag<T>& f, const T* Ks, int row, int kk, int h) {
    frag<SK>(f, Ks, row, kk * 16 + 8 * h);
  }
  static __device__ __forceinline__ void vfrag(Frag<T>& f, const T* Vt, int d, int ks, int h) {
    frag<SV>(f, Vt, d, ks * 16 + 8 * h);
  }
  static __device__ __forceinline__ void vfrag16(Frag16& f, const T* Vt, int d, int ks, int h) {
    f.v = __builtin_bit_cast(f16x8, *SV::chunk(Vt, d, (ks * 16 + 8 * h) / EPC));
  }
};

// ----------------------------------------------------------------- tile compute

// Logit bias policies for one 64-key tile (values in log2 units, added to the scaled logits).
// `key` is the tile-local key index, `lane` the caller's lane (its query row).
struct NoBias {
  __device__ bool active() const { return false; }
  __device__ float operator()(int) const { return 0.0f; }
};
struct KeyBias {  // one bias per key from LDS (centroid columns: log2 n_c or -inf); null = none
  const float* bias;
  __device__ bool active() const { return bias != nullptr; }
  __device__ float operator()(int key) const { return bias[key]; }
};

// One 64-key tile for one wave, in three parts: S^T = K Q^T (tile_qk), the online softmax
// (tile_softmax) and O^T += V^T P^T (tile_pv).  qf: this wave's Q fragments; c2 = scale *
// log2(e); keys at or past `nvalid` do not exist.  pv16: for bfloat16 inputs the tile's V^T in
// LDS is float16 and P is rounded to float16 (else both are bfloat16).  Bias, nvalid and pv16
// are uniform over the workgroup, so the branches on them cost no divergence.
template <typename T, int D, typename Lds, int AHEAD = 1>
__device__ __forceinline__ void tile_qk(const T* Ks, const Frag<T>* qf, f32x16& s0, f32x16& s1) {
  using C = Cfg<T, D>;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
  s0 = f32x16{};
  s1 = f32x16{};
  // Fragments are read AHEAD steps before the products that use them.  The sparse attention's
  // float16 loop reads two ahead (one ahead leaves each product waiting for its own LDS read),
  // with group barriers that keep the compiler's schedule in that order; the other kernels,
  // with less room in their registers, read one ahead.
  Frag<T> a0[AHEAD + 1], a1[AHEAD + 1];
#pragma unroll
  for (int i = 0; i < AHEAD; ++i) {
    Lds::kfrag(a0[i], Ks, r, i, h);
    Lds::kfrag(a1[i], Ks, 32 + r, i, h);
  }
  if constexpr (AHEAD > 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2 * AHEAD, 0);
#pragma unroll
  for (int kk = 0; kk < C::KK; ++kk) {
    if (kk + AHEAD < C::KK) {
      Lds::kfrag(a0[(kk + AHEAD) % (AHEAD + 1)], Ks, r, kk + AHEAD, h);
      Lds::kfrag(a1[(kk + AHEAD) % (AHEAD + 1)], Ks, 32 + r, kk + AHEAD, h);
    }
    s0 = mma(a0[kk % (AHEAD + 1)], qf[kk], s0);
    s1 = mma(a1[kk % (AHEAD + 1)], qf[kk], s1);
    if constexpr (AHEAD > 1) {
      if (kk + AHEAD < C::KK) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 2, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 2, 0);
    }
  }
}

// Online softmax of one tile's logits, in place: s[0], s[1] hold S^T in, P out (log2 units).
// Key of s[mt][j]: mt*32 + 8*(j/4) + 4*h + j%4.  Without a bias the max is taken on the raw
// products (c2 > 0) and the scale folds into the exponent's FMA.  The running max may lag the
// true max by up to kRescaleSlack, so P <= 2^kRescaleSlack; O and l are rescaled only when a
// row exceeds that (a wave-uniform branch, rarely taken after the first tiles).
template <typename T, int D, typename Bias>
__device__ __forceinline__ void tile_softmax(f32x16 (&s)[2], RowState<D>& st, float c2, const Bias& bias,
                                             int nvalid) {
  using C = Cfg<T, D>;
  const int h = (threadIdx.x & 63) >> 5;
  float xs = c2;  // scale still to apply to s
  if (__builtin_expect(bias.active(), 0)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mt][j] = s[mt][j] * c2 + bias(mt * 32 + 8 * (j / 4) + 4 * h + (j % 4));
    xs = 1.0f;
  }
  if (__builtin_expect(nvalid < kNK, 0)) {  // ragged last tile of a cluster
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (mt * 32 + 8 * (j / 4) + 4 * h + (j % 4) >= nvalid) s[mt][j] = -INFINITY;
  }
  // Tree reductions keep the dependency chains short.
  float t8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x16& v = s[i / 4];
    const int o = 4 * (i % 4);
    t8[i] = fmaxf(fmaxf(v[o], v[o + 1]), fmaxf(v[o + 2], v[o + 3]));
  }
  float mx = fmaxf(fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3])), fmaxf(fmaxf(t8[4], t8[5]), fmaxf(t8[6], t8[7])));
  mx = fmaxf(mx, swap_halves(mx)) * xs;
  if (__builtin_expect(__ballot(mx > st.m + kRescaleSlack) != 0, 0)) {
    const float m_new = fmaxf(st.m, mx);
    const float alpha = (st.m == -INFINITY) ? 0.0f : fast_exp2(st.m - m_new);
    st.m = m_new;
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[dt][j] *= alpha;
  }
  const float m_use = st.m == -INFINITY ? 0.0f : st.m;
#pragma unroll
  for (int mt = 0; mt < 2; ++mt)
#pragma unroll
    for (int j = 0; j < 16; ++j) s[mt][j] = fast_exp2(__builtin_fmaf(s[mt][j], xs, -m_use));
  float s8[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const f32x16& v = s[i / 4];
    const int o = 4 * (i % 4);
    s8[i] = (v[o] + v[o + 1]) + (v[o + 2] + v[o + 3]);
  }
  st.l += ((s8[0] + s8[1]) + (s8[2] + s8[3])) + ((s8[4] + s8[5]) + (s8[6] + s8[7]));
}

// P fragment of contraction step ks (keys ks*16 .. ks*16+15): elements s[ks/2][(ks%2)*8 + i].
__device__ __forceinline__ void p_frag16(Frag16& f, const f32x16 (&s)[2], int ks) {
#pragma unroll
  for (int i = 0; i < 8; ++i) f.v[i] = static_cast<_Float16>(s[ks >> 1][(ks & 1) * 8 + i]);
}
template <typename T>
__device__ __forceinline__ void p_frag(Frag<T>& f, const f32x16 (&s)[2], int ks) {
  float x[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) x[i] = s[ks >> 1][(ks & 1) * 8 + i];
  frag_from_f32(f, x);
}

// O^T += V^T P^T over four 16-key steps with a float16 V^T tile; pfrag(ks, f) supplies the P
// fragment of step ks.  Fragment n = ks * DT + dt of V^T is read PF products ahead (the
// sparse attention's float16 loop: three, in the order the group barriers fix).
template <typename T, int D, typename Lds, int PF = 1, typename PFrag>
__device__ __forceinline__ void pv16_steps(const T* Vt, RowState<D>& st, PFrag&& pfrag) {
  using C = Cfg<T, D>;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31, h = lane >> 5;
  constexpr int NF = 4 * C::DT;
  Frag16 va[PF + 1];
#pragma unroll
  for (int n = 0; n < PF; ++n) Lds::vfrag16(va[n], Vt, (n % C::DT) * 32 + r, n / C::DT, h);
  if constexpr (PF > 1) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, PF, 0);
  Frag16 pb;
#pragma unroll
  for (int n = 0; n < NF; ++n) {
    const int ks = n / C::DT, dt = n % C::DT;
    if (n + PF < NF) Lds::vfrag16(va[(n + PF) % (PF + 1)], Vt, ((n + PF) % C::DT) * 32 + r, (n + PF) / C::DT, h);
    if (dt == 0) pfrag(ks, pb);
    st.o[dt] = mma(va[n % (PF + 1)], pb, st.o[dt]);
    if constexpr (PF > 1) {
      if (n + PF < NF) __builtin_amdgcn_sched_group_barrier(kSchedDsRead, 1, 0);
      __builtin_amdgcn_sched_group_barrier(kSchedMfma, 1, 0);
    }
  }
}

// O^T += V^T P^T over four 16-key steps.  B fragment element i of step ks holds the key
// ks*16 + 8*(i/4) + 4*h + i%4; the V^T fragment reads the same keys.
template <typename T, int D, typename Lds>
__device__ __forceinline__ void tile_pv(const T* Vt, const f32x16 (&s)[2], RowState<D>& st, bool pv16) {
  using C = Cfg<T, D>;
  const int lane = threadIdx.x & 63;
  const int r = lane & 31;
  const int h = lane >> 5;
  if (sizeof(T) == 2 && __builtin_expect(pv16, 1)) {
    pv16_steps<T, D, Lds>(Vt, st, [&](int ks, Frag16& f) { p_frag16(f, s, ks); });
  } else {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      Frag<T> pb;
      p_frag(pb, s, ks);
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt) {
        Frag<T> va;
        Lds::vfrag(va, Vt, dt * 32 + r, ks, h);
        st.o[dt] = mma(va, pb, st.o[dt]);
      }
    }
  }
}

template <typename T, int D, typename Lds, typename Bias>
__device__ __forceinline__ void tile_step(const T* Ks, const T* Vt, const Frag<T>* qf, RowState<D>& st, float c2,
                                          const Bias& bias, int nvalid, bool pv16) {
  f32x16 s[2];
  // The Q K^T products issue at raised wave priority, so that of the two waves sharing a SIMD
  // the one entering its products goes first and the other's softmax fills in beside them.
  __builtin_amdgcn_s_setprio(1);
  tile_qk<T, D, Lds>(Ks, qf, s[0], s[1]);
  __builtin_amdgcn_s_setprio(0);
  tile_softmax<T, D>(s, st, c2, bias, nvalid);
  tile_pv<T, D, Lds>(Vt, s, st, pv16);
}

// Tile step of the float16 loop (bfloat16 inputs, every V^T tile float16).  The logits are
// exponentiated against the running max as it stands, straight into the float16 P fragments,
// and the row sums are taken from those fragments with float32 dot products, so the
// normalisation adds exactly the weights that the P V product multiplies.  The tile's own max
// is computed only when the running max is unset (first tile) or when some lane's sum of its 32
// weights reaches 2^14 -- a logit at least 9 log2 units above the running max, with float16
// range at stake; then the running max moves up to the tile's (O and l rescaled) and the
// weights are formed again from the logits, which the first pass left intact.  Weights thus
// stay below 2^14, and without the max the common tile saves its reduction.
template <int D, typename Bias>
__device__ __forceinline__ void tile_step16(const bf16_t* Ks, const bf16_t* Vt, const Frag<bf16_t>* qf,
                                           RowState<D>& st, float c2, const Bias& bias, int nvalid) {
  using C = Cfg<bf16_t, D>;
  using Lds = SwzLds<bf16_t, D>;
  const int h = (threadIdx.x & 63) >> 5;
  f32x16 s[2];
  __builtin_amdgcn_s_setprio(1);
  tile_qk<bf16_t, D, Lds, 2>(Ks, qf, s[0], s[1]);
  __builtin_amdgcn_s_setprio(0);
  float xs = c2;  // scale still to apply to s
  if (__builtin_expect(bias.active(), 0)) {
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) s[mt][j] = s[mt][j] * c2 + bias(mt * 32 + 8 * (j / 4) + 4 * h + (j % 4));
    xs = 1.0f;
  }
  if (__builtin_expect(nvalid < kNK, 0)) {  // ragged last tile of a cluster
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        if (mt * 32 + 8 * (j / 4) + 4 * h + (j % 4) >= nvalid) s[mt][j] = -INFINITY;
  }
  Frag16 pf[4];  // P of the four 16-key steps
  const f16x2 ones = {static_cast<_Float16>(1.0f), static_cast<_Float16>(1.0f)};
  auto weights = [&]() {
    const float m_use = st.m == -INFINITY ? 0.0f : st.m;
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int i = 0; i < 8; i += 2) {
        const float e0 = fast_exp2(__builtin_fmaf(s[ks >> 1][(ks & 1) * 8 + i], xs, -m_use));
        const float e1 = fast_exp2(__builtin_fmaf(s[ks >> 1][(ks & 1) * 8 + i + 1], xs, -m_use));
        pf[ks].v[i] = static_cast<_Float16>(e0);
        pf[ks].v[i + 1] = static_cast<_Float16>(e1);
        const f16x2 pr = {pf[ks].v[i], pf[ks].v[i + 1]};
        acc[ks] = __builtin_amdgcn_fdot2(pr, ones, acc[ks], false);
      }
    return (acc[0] + acc[1]) + (acc[2] + acc[3]);
  };
  float lsum = 0.0f;
  bool need_max = __ballot(st.m == -INFINITY) != 0;
  if (!need_max) {
    lsum = weights();
    need_max = __ballot(!(lsum < 16384.0f)) != 0;  // also catches an infinite weight
  }
  if (__builtin_expect(need_max, 0)) {
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x16& v = s[i / 4];
      const int o = 4 * (i % 4);
      t8[i] = fmaxf(fmaxf(v[o], v[o + 1]), fmaxf(v[o + 2], v[o + 3]));
    }
    float mx = fmaxf(fmaxf(fmaxf(t8[0], t8[1]), fmaxf(t8[2], t8[3])), fmaxf(fmaxf(t8[4], t8[5]), fmaxf(t8[6], t8[7])));
    mx = fmaxf(mx, swap_halves(mx)) * xs;
    if (mx > st.m) {
      const float alpha = (st.m == -INFINITY) ? 0.0f : fast_exp2(st.m - mx);
      st.m = mx;
      st.l *= alpha;
#pragma unroll
      for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
        for (int j = 0; j < 16; ++j) st.o[dt][j] *= alpha;
    }
    lsum = weights();
  }
  st.l += lsum;
  // Wave priorities (the two waves of a SIMD belong to different workgroups): the P V products
  // that end a wave's tile go first, then Q K^T products, then the softmax arithmetic, so a
  // wave near its workgroup's barrier is not held back by the other wave's exponentials
  // (measured: 2% faster than raising only the Q K^T products).
  __builtin_amdgcn_s_setprio(2);
  pv16_steps<bf16_t, D, Lds, 3>(Vt, st, [&](int ks, Frag16& f) { f = pf[ks]; });
  __builtin_amdgcn_s_setprio(0);
}

template <typename T, int D>
__device__ __forceinline__ void load_q_frags(Frag<T>* qf, const T* __restrict__ qrow) {
  const int h = (threadIdx.x & 63) >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) load_frag(qf[kk], qrow + kk * 16 + 8 * h);
}

template <int D>
__device__ __forceinline__ void init_state(RowState<D>& st) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) st.o[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.0f;
}

// Work unit -> (batch x K/V head, query cluster, head in group): unit = ((b Hkv + kvh) Cq + a) G + g,
// so the query heads that share a K/V head (and a mask) are adjacent.
__device__ __forceinline__ void decode_unit(int u, int Cq, int G, int& bk, int& a, int& g) {
  g = u % G;
  const int r = u / G;
  a = r % Cq;
  bk = r / Cq;
}

template <typename T, int D>
constexpr int attn_lds_bytes() {
  using C = Cfg<T, D>;
  const int base = C::KV_BYTES > C::Z_BYTES ? C::KV_BYTES : C::Z_BYTES;
  return base + kNK * 4 + kFlagBytes;
}

// ----------------------------------------------------------------- sparse attention

// Packed tiles go from global memory straight into LDS (16 bytes per lane, no registers):
// one wave instruction fills 1 KB of LDS, lane l writing bytes [16 l, 16 l + 16).  Each lane
// fetches the global chunk that the swizzle puts in its LDS slot; these per-lane byte offsets
// are the same for every tile.
template <typename T, int D>
struct TileDma {
  using S = SwzLds<T, D>;
  static constexpr int NK = S::K_BYTES / 16 / kThreads;  // K chunks per thread
  static constexpr int NV = S::V_BYTES / 16 / kThreads;  // V^T chunks per thread
  static_assert(S::K_BYTES % (16 * kThreads) == 0 && S::V_BYTES % (16 * kThreads) == 0, "tile split");
  // Copy j of a thread fills LDS slot (4 j + wave) * 64 + lane.  Successive copies are 4 KB
  // apart in both LDS and global memory: they move whole rows (16 rows of 256 B, 32 of 128 B
  // ...), and the swizzle pattern repeats every 16 rows, so one per-lane offset serves all.
  static constexpr int kStep = kThreads * 16;
  // Whether the swizzle of a row repeats kStep bytes further on (else each copy computes its
  // own offset).
  template <typename W>
  static constexpr bool repeats() {
    return ((kThreads / W::CPR) / W::RP) % (W::MASK + 1) == 0;
  }
  template <typename W, int ROWB>
  static __device__ __forceinline__ int offset(int j) {
    const int slot = (j * 4 + (static_cast<int>(threadIdx.x) >> 6)) * 64 + (threadIdx.x & 63);
    const int r = slot / W::CPR;
    return r * ROWB + W::pos(r, slot % W::CPR) * 16;
  }
  int koff, voff;
  __device__ __forceinline__ void init() {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int slot = wave * 64 + lane;
    const int rk = slot / S::SK::CPR, rv = slot / S::SV::CPR;
    koff = rk * S::KROWB + S::SK::pos(rk, slot % S::SK::CPR) * 16;
    voff = rv * S::VROWB + S::SV::pos(rv, slot % S::SV::CPR) * 16;
  }
  // Start copying a K tile (gk) into LDS at Ks, or a V^T tile (gv) into LDS at Vt.
  __device__ __forceinline__ void issue_k(const unsigned char* gk, T* Ks) const {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass only needs the kernel's launch stub
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    unsigned char* lk = reinterpret_cast<unsigned char*>(Ks) + wave * 1024;
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int off = repeats<typename S::SK>() ? j * kStep + koff : offset<typename S::SK, S::KROWB>(j);
      __builtin_amdgcn_global_load_lds(gk + off, lk + j * kStep, 16, 0, 0);
    }
#endif
  }
  __device__ __forceinline__ void issue_v(const unsigned char* gv, T* Vt) const {
#if defined(__HIP_DEVICE_COMPILE__)
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    unsigned char* lv = reinterpret_cast<unsigned char*>(Vt) + wave * 1024;
#pragma unroll
    for (int j = 0; j < NV; ++j) {
      const int off = repeats<typename S::SV>() ? j * kStep + voff : offset<typename S::SV, S::VROWB>(j);
      __builtin_amdgcn_global_load_lds(gv + off, lv + j * kStep, 16, 0, 0);
    }
#endif
  }
  // The same copies by buffer loads: the head's tiles are a buffer resource, the tile's byte
  // offset a scalar, the per-lane offsets the constants above, so a tile costs no address
  // arithmetic (16-bit tiles, whose swizzle repeats every kStep bytes).
  static constexpr bool kBuffer = repeats<typename S::SK>() && repeats<typename S::SV>();
  __device__ __forceinline__ void issue_kv_buf(__amdgpu_buffer_rsrc_t kr, __amdgpu_buffer_rsrc_t vr, int toff, T* Ks,
                                               T* Vt) const {
#if defined(__HIP_DEVICE_COMPILE__)
    typedef __attribute__((address_space(3))) unsigned char lds_u8;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
    lds_u8* lk = (lds_u8*)(reinterpret_cast<unsigned char*>(Ks) + wave * 1024);
    lds_u8* lv = (lds_u8*)(reinterpret_cast<unsigned char*>(Vt) + wave * 1024);
#pragma unroll
    for (int j = 0; j < NK; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, lk + j * kStep, 16, koff + j * kStep, toff, 0, 0);
#pragma unroll
    for (int j = 0; j < NV; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, lv + j * kStep, 16, voff + j * kStep, toff, 0, 0);
#endif
  }
};
// Buffer resource over `bytes` bytes at p (raw buffer, 32-bit elements; offsets past the end
// read as zero).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_buffer(const void* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, bytes, 0x00020000);
}

// The tile sequence of one mask row, expanded ahead of the attention by tile_list_wave_kernel:
// the centroid tiles (compensation), then the tiles of every kept key cluster in list order,
// one int32 entry per tile: bits 0-22 the packed tile index, bits 23-28 the tile's key count
// minus one, bit 29 set for centroid tiles.  A cluster's tile count is clamped to the tiles
// the packed buffer gives it, so keys past it are never read.
constexpr int kEntryTileBits = 23;
constexpr int kEntryCentroid = 1 << 29;
__device__ __forceinline__ int entry_make(int tile, int nvalid, bool centroid) {
  return tile | ((nvalid - 1) << kEntryTileBits) | (centroid ? kEntryCentroid : 0);
}
__device__ __forceinline__ int entry_tile(int e) { return e & ((1 << kEntryTileBits) - 1); }
__device__ __forceinline__ int entry_nvalid(int e) { return ((e >> kEntryTileBits) & 63) + 1; }
__device__ __forceinline__ bool entry_centroid(int e) { return (e & kEntryCentroid) != 0; }

// One wave per mask row (four rows per workgroup): writes the row's entries (at most maxe)
// and their count.  The row's clusters go 64 at a time, one per lane, and a wave scan of their
// tile counts places their entries.  Mask row (b Hm + hm) Cq + a reads the key layout of its
// (batch, K/V head) when there is one per head (nl > 1, Hm in {Hkv, Hq}).
__global__ __launch_bounds__(256) void tile_list_wave_kernel(const int32_t* __restrict__ kv_count,
                                                             const int16_t* __restrict__ kv_idx, int rows, int Ck,
                                                             const int32_t* __restrict__ k_off,
                                                             const int32_t* __restrict__ tile_off, int nl, int Hq,
                                                             int Hkv, int Hm, int Cq, int first_ctile, int ctiles,
                                                             int comp, int maxe, int32_t* __restrict__ entries,
                                                             int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const size_t row = static_cast<size_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (row >= static_cast<size_t>(rows)) return;  // whole waves only; no barrier below
  if (nl > 1) {
    const size_t bh = row / Cq;
    const int b = static_cast<int>(bh / Hm), hm = static_cast<int>(bh % Hm);
    const size_t lay = static_cast<size_t>(b) * Hkv + (Hm == Hq ? hm / (Hq / Hkv) : hm);
    k_off += lay * (Ck + 1);
    tile_off += lay * (Ck + 1);
  }
  const int cnt = kv_count[row];
  const int16_t* list = kv_idx + row * Ck;
  int32_t* out = entries + row * maxe;
  int base = 0;
  if (comp) {
    for (int e = lane; e < ctiles && e < maxe; e += 64) out[e] = entry_make(first_ctile + e, kNK, true);
    base = min(ctiles, maxe);
  }
  for (int p0 = 0; p0 < cnt; p0 += 64) {
    const int p = p0 + lane;
    int nt = 0, n = 0, t0 = 0;
    if (p < cnt) {
      const int cl = list[p];
      if (cl >= 0 && cl < Ck) {
        n = k_off[cl + 1] - k_off[cl];
        t0 = tile_off[cl];
        nt = min((n + kNK - 1) / kNK, min(tile_off[cl + 1], first_ctile) - t0);
        if (n <= 0 || t0 < 0 || nt < 0) nt = 0;
      }
    }
    int incl = nt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int first = base + incl - nt;
    for (int j = 0; j < nt && first + j < maxe; ++j) out[first + j] = entry_make(t0 + j, min(kNK, n - j * kNK), false);
    base += __shfl(incl, 63);
  }
  if (lane == 0) counts[row] = min(base, maxe);
}

// Work order for the attention.  Workgroups are dispatched to the 8 XCDs round-robin, and
// each XCD has its own L2.  The units of one K/V group -- every query cluster of its query
// heads, which read the same key tiles and (for GQA) share masks -- go to one XCD, query
// cluster by query cluster, so that workgroups running together on an XCD sweep nearby
// tiles and hit its L2.  Groups are spread over the XCDs longest-processing-time first by
// their total tile count.  There are two queues: groups whose V^T tiles are all float16
// (hmix[group] == 0 with fast_ok) for the float16 kernel, the others for the general one.
// Queue q uses ctl[32 q + x] as XCD x's unit counter and ctl[32 q + 8 + x] as the start of
// its segment of `order` (ctl[32 q + 16] = end).  One workgroup.
// Per K/V group (one workgroup each): the group's work, the sum over its units of their tile
// counts + 1, and with sort_ok the rank of each unit within its group by descending tile count
// (ties by unit index), else its index.  Unit u of group bk is u = bk * per + j with
// j = a * G + g (decode_unit).  Dynamic LDS: the group's counts (per ints, sort_ok only).
constexpr int kGroupThreads = 256;
constexpr int kMaxSortUnits = 12288;  // units per group ranked in LDS (48 KB)
__global__ __launch_bounds__(kGroupThreads) void group_rank_kernel(const int32_t* __restrict__ counts, int Hq,
                                                                   int Hkv, int Hm, int Cq, int sort_ok,
                                                                   int32_t* __restrict__ rank,
                                                                   int32_t* __restrict__ gsum) {
  extern __shared__ int ucnt[];
  __shared__ int red[kGroupThreads / 64];
  const int bk = blockIdx.x;
  const int G = Hq / Hkv;
  const int per = Cq * G;
  const int b = bk / Hkv, kvh = bk % Hkv;
  int local = 0;
  for (int j = threadIdx.x; j < per; j += kGroupThreads) {
    const int a = j / G, g = j % G, hq = kvh * G + g;
    const int hm = Hm == 1 ? 0 : (Hm == Hq ? hq : kvh);
    const int c = counts[(static_cast<size_t>(b) * Hm + hm) * Cq + a];
    local += c + 1;
    if (sort_ok) ucnt[j] = c;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) local += __shfl_xor(local, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = local;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
#pragma unroll
    for (int w = 0; w < kGroupThreads / 64; ++w) tot += red[w];
    gsum[bk] = tot;
  }
  int32_t* rk = rank + static_cast<size_t>(bk) * per;
  for (int j = threadIdx.x; j < per; j += kGroupThreads) {
    int r = j;
    if (sort_ok) {
      const int c = ucnt[j];
      r = 0;
      for (int j2 = 0; j2 < per; ++j2) {
        const int c2 = ucnt[j2];  // the same address for every lane: a broadcast read
        r += (c2 > c) | ((c2 == c) & (j2 < j));
      }
    }
    rk[j] = r;
  }
}

// Work order of the attention units, from the group totals and ranks above.  K/V groups go
// to the 8 XCDs longest processing time first (the float16 and the general queue apart);
// inside an XCD's segment the groups follow in assignment order and a group's units by rank:
// workgroups that run side by side then sweep the key tiles of one head at similar rates and
// meet in the L2 more often, and the longest units start first.  ctl: queue q's counters at
// ctl[32 q + x], its segment starts at ctl[32 q + 8 + x] (x <= 8).
constexpr int kOrderThreads = 1024;
constexpr int kMaxGroups = 2048;
constexpr int kQueueCtl = 32;  // ints of ctl per queue
__global__ __launch_bounds__(kOrderThreads) void order_kernel(const int32_t* __restrict__ gsum,
                                                               const int32_t* __restrict__ rank, int B, int Hq,
                                                               int Hkv, int Cq, const int32_t* __restrict__ hmix,
                                                               int fast_ok, int32_t* __restrict__ order,
                                                               int32_t* __restrict__ ctl) {
  __shared__ int wsum[kMaxGroups];
  __shared__ int place[kMaxGroups];  // first the group of each rank, then the slot of each group
  __shared__ int8_t gq[kMaxGroups];  // the queue of each group (read by the serial loop below)
  __shared__ int seg[2][kXcds + 1];
  const int t = threadIdx.x;
  const int G = Hq / Hkv;
  const int ng = B * Hkv;
  const int per = Cq * G;  // units per group, contiguous in unit numbering
  const int units = ng * per;
  if (ng > kMaxGroups) {  // too many groups to balance here: plain order in the general queue
    for (int u = t; u < units; u += kOrderThreads) order[u] = u;
    if (t <= kXcds) {
      ctl[8 + t] = 0;  // empty float16 queue
      if (t < kXcds) ctl[t] = 0;
      ctl[kQueueCtl + 8 + t] = static_cast<int>((static_cast<long long>(units) * t) / kXcds);
      if (t < kXcds) ctl[kQueueCtl + t] = 0;
    }
    return;
  }
  for (int i = t; i < ng; i += kOrderThreads) {
    wsum[i] = gsum[i];
    gq[i] = (fast_ok && hmix[i] == 0) ? 0 : 1;
  }
  __syncthreads();
  // Rank the groups by descending work (ties by index).
  for (int i = t; i < ng; i += kOrderThreads) {
    const int w = wsum[i];
    int r = 0;
    for (int j = 0; j < ng; ++j) r += (wsum[j] > w) | ((wsum[j] == w) & (j < i));
    place[r] = i;
  }
  __syncthreads();
  if (t == 0) {
    // Longest processing time first: each group to the least loaded XCD of its queue.  The
    // per-XCD loads and group counts of both queues stay in registers (the loops over XCDs
    // are unrolled), so the serial loop waits on no memory but the group's own entries.
    long long ld[2][kXcds];
    int cnt[2][kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x) ld[0][x] = ld[1][x] = cnt[0][x] = cnt[1][x] = 0;
    for (int r = 0; r < ng; ++r) {
      const int gi = place[r];
      const bool q1 = gq[gi] != 0;
      const long long w = wsum[gi];
      int xs = 0;
      long long best = q1 ? ld[1][0] : ld[0][0];
#pragma unroll
      for (int x = 1; x < kXcds; ++x) {
        const long long lx = q1 ? ld[1][x] : ld[0][x];
        if (lx < best) {
          best = lx;
          xs = x;
        }
      }
      int slot = 0;
#pragma unroll
      for (int x = 0; x < kXcds; ++x) {
        if (x == xs) {
          if (q1) {
            ld[1][x] += w;
            slot = cnt[1][x]++;
          } else {
            ld[0][x] += w;
            slot = cnt[0][x]++;
          }
        }
      }
      wsum[gi] = ((q1 ? kXcds : 0) + xs) * kMaxGroups + slot;  // queue, XCD and slot of the group
    }
    int run = 0;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
#pragma unroll
      for (int x = 0; x < kXcds; ++x) {
        seg[q][x] = run;
        ctl[q * kQueueCtl + 8 + x] = run;
        ctl[q * kQueueCtl + x] = 0;
        run += cnt[q][x] * per;
      }
      seg[q][kXcds] = run;
      ctl[q * kQueueCtl + 8 + kXcds] = run;
    }
  }
  __syncthreads();
  // Each thread's ranks are loaded together before any store depends on them.
  constexpr int kOrderBatch = 16;
  for (int u0 = t; u0 < units; u0 += kOrderThreads * kOrderBatch) {
    int rk[kOrderBatch];
#pragma unroll
    for (int i = 0; i < kOrderBatch; ++i) {
      const int u = u0 + i * kOrderThreads;
      rk[i] = u < units ? rank[u] : 0;
    }
#pragma unroll
    for (int i = 0; i < kOrderBatch; ++i) {
      const int u = u0 + i * kOrderThreads;
      if (u < units) {
        const int bk = u / per;
        const int qx = wsum[bk] / kMaxGroups, slot = wsum[bk] % kMaxGroups;
        order[seg[qx / kXcds][qx % kXcds] + slot * per + rk[i]] = u;
      }
    }
  }
}

// The correction o + o A + c applied in the attention's epilogue ("Partition the Support,
// Reconstruct the Residual", Probe-Fitted Residual Reconstruction: the fitted map corrects
// every row).  A is staged in LDS transposed, with each 16-feature group of a row in the
// order 0-3, 8-11, 4-7, 12-15 -- the order in which the output accumulators hold a row's
// features, so they feed the product as they are -- as bfloat16 high and low parts for
// bfloat16 inputs (o A by three products, hi*hi + hi*lo + lo*hi: float32 accuracy) or float32
// for float32 inputs; then c.  The image is built once per head by corr_image_kernel and
// copied into LDS per row block.
template <typename T, int D>
struct CorrImage {
  static constexpr bool kSplit = sizeof(T) == 2;
  static constexpr int ROW = kSplit ? D + 8 : D + 4;  // elements per A^T row (16-byte aligned)
  static constexpr int A_BYTES = (kSplit ? 2 : 1) * D * ROW * static_cast<int>(sizeof(T));
  static constexpr int BYTES = A_BYTES + D * 4;  // + c
  // Whole 1 KB blocks: one wave instruction copies 1 KB from global memory into LDS.
  static constexpr int STRIDE = (BYTES + 1023) / 1024 * 1024;
};
__host__ __device__ constexpr int corr_pos(int f) { return (f & ~12) | ((f & 4) << 1) | ((f & 8) >> 1); }
// Largest image of any instantiation (the workspace reserves it per (batch, query head)).
constexpr size_t kCorrImageStride = CorrImage<bf16_t, 128>::STRIDE > CorrImage<float, 128>::STRIDE
                                        ? CorrImage<bf16_t, 128>::STRIDE
                                        : CorrImage<float, 128>::STRIDE;

template <typename T, int D>
__global__ __launch_bounds__(256) void corr_image_kernel(const float* __restrict__ A, const float* __restrict__ cvec,
                                                         unsigned char* __restrict__ img) {
  using I = CorrImage<T, D>;
  const size_t bh = blockIdx.x;
  const float* Ah = A + bh * D * D;
  unsigned char* out = img + bh * kCorrImageStride;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int i = e / D, j = e % D;  // A[i][j] -> row j (output feature), position corr_pos(i)
    const float x = Ah[e];
    if constexpr (I::kSplit) {
      bf16_t* hi = reinterpret_cast<bf16_t*>(out);
      bf16_t* lo = hi + D * I::ROW;
      const __bf16 hb = static_cast<__bf16>(x);
      hi[j * I::ROW + corr_pos(i)].bits = __builtin_bit_cast(uint16_t, hb);
      lo[j * I::ROW + corr_pos(i)].bits = f32_to_bf16(x - static_cast<float>(hb));
    } else {
      reinterpret_cast<float*>(out)[j * I::ROW + corr_pos(i)] = x;
    }
  }
  for (int d = threadIdx.x; d < D; d += 256)
    reinterpret_cast<float*>(out + I::A_BYTES)[d] = cvec[bh * D + d];
}

// o (the accumulator layout of a wave's 32 rows) += o A + c, with the image in LDS at `img`.
// The product accumulates straight into o: the operand fragments of o are taken first.
template <typename T, int D>
__device__ __forceinline__ void apply_correction(f32x16 (&o)[D / 32], const unsigned char* img) {
  using I = CorrImage<T, D>;
  constexpr int DT = D / 32, KK = D / 16;
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  // Contraction positions 16 kk + 8 h + e hold features 16 kk + 4 h + (e % 4) + 8 (e / 4):
  // entries 8 (kk % 2) + e of accumulator kk / 2.
  if constexpr (I::kSplit) {
    const bf16_t* AtH = reinterpret_cast<const bf16_t*>(img);
    const bf16_t* AtL = AtH + D * I::ROW;
    Frag<bf16_t> oh[KK], ol[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = o[kk / 2][8 * (kk % 2) + e];
        const __bf16 hb = static_cast<__bf16>(x);
        oh[kk].v[e] = hb;
        ol[kk].v[e] = static_cast<__bf16>(x - static_cast<float>(hb));
      }
#pragma unroll
    for (int jt = 0; jt < DT; ++jt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frag<bf16_t> ah, al;
        load_frag(ah, AtH + (jt * 32 + r) * I::ROW + kk * 16 + 8 * h);
        load_frag(al, AtL + (jt * 32 + r) * I::ROW + kk * 16 + 8 * h);
        o[jt] = mma(ah, oh[kk], o[jt]);
        o[jt] = mma(ah, ol[kk], o[jt]);
        o[jt] = mma(al, oh[kk], o[jt]);
      }
  } else {
    const float* At = reinterpret_cast<const float*>(img);
    Frag<float> of[KK];
#pragma unroll
    for (int kk = 0; kk < KK; ++kk)
#pragma unroll
      for (int e = 0; e < 8; ++e) of[kk].v[e] = o[kk / 2][8 * (kk % 2) + e];
#pragma unroll
    for (int jt = 0; jt < DT; ++jt)
#pragma unroll
      for (int kk = 0; kk < KK; ++kk) {
        Frag<float> af;
        load_frag(af, At + (jt * 32 + r) * I::ROW + kk * 16 + 8 * h);
        o[jt] = mma(af, of[kk], o[jt]);
      }
  }
  const float* cs = reinterpret_cast<const float*>(img + I::A_BYTES);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int j = 0; j < 16; ++j) o[dt][j] += cs[dt * 32 + 8 * (j / 4) + 4 * h + (j % 4)];
}

// Copy this head's correction image into LDS (1 KB per wave instruction, straight into LDS).
template <typename T, int D>
__device__ __forceinline__ void load_correction_image(const unsigned char* src, unsigned char* lds) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int NB = CorrImage<T, D>::STRIDE / 1024;
  const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int lane = threadIdx.x & 63;
  for (int blk = wave; blk < NB; blk += kThreads / 64)
    __builtin_amdgcn_global_load_lds(src + blk * 1024 + lane * 16, lds + blk * 1024, 16, 0, 0);
#endif
}

template <typename T, int D, typename TO, bool CORR = false>
struct AttnLds {
  using C = Cfg<T, D>;
  static constexpr int KB = SwzLds<T, D>::K_BYTES;  // one K tile
  static constexpr int VB = SwzLds<T, D>::V_BYTES;  // one V^T tile
  static constexpr int K0 = 0;                      // K buffers [2]
  static constexpr int V0 = 2 * KB;                 // V^T buffers [2]
  static constexpr int TILES = 2 * KB + 2 * VB;
  static constexpr int ZEPC = 16 / static_cast<int>(sizeof(TO));  // output elements per 16-byte chunk
  static constexpr int ZROW = D + ZEPC;                             // output staging row (elements)
  static constexpr int Z_BYTES = kRowsWG * ZROW * static_cast<int>(sizeof(TO));
  static constexpr int MAIN0 = TILES > Z_BYTES ? TILES : Z_BYTES;
  static constexpr int MAIN = (CORR && CorrImage<T, D>::STRIDE > MAIN0) ? CorrImage<T, D>::STRIDE : MAIN0;
  static constexpr int BIAS = MAIN;                // float[2 buffers][kNK]
  static constexpr int UNIT = BIAS + 2 * kNK * 4;  // the workgroup's current work unit
  static constexpr int TOTAL = UNIT + 16;
};

// Workgroups resident per CU: bfloat16 kernels keep two (eight waves, two per SIMD, so
// one wave's softmax overlaps the other's MFMAs); float32 tiles need the LDS of one.
template <typename T, bool FAST = true>
constexpr int attn_occupancy() {
  return (sizeof(T) == 2 && FAST) ? 2 : 1;
}

// TO: output element type (the input type, or float32 when a correction pass follows).
// FAST: the kernel for heads whose V^T tiles are all float16 (bfloat16 inputs only); the
// general kernel handles the others with a per-tile format switch.  Each takes its units
// from its own queue, and keeping the two apart gives each its own register allocation.
template <typename T, int D, bool COMP, typename TO, bool FAST, bool CORR>
__global__ __launch_bounds__(kThreads, (attn_occupancy<T, FAST>())) void sparse_attn_kernel(
    const T* __restrict__ Q, TO* __restrict__ O, float* __restrict__ lse, int B, int Hq, int Hkv, int S, float c2,
    const int32_t* __restrict__ q_perm, const int32_t* __restrict__ q_off, int Cq, const int32_t* __restrict__ k_off,
    int Ck, const uint8_t* __restrict__ keep, const int32_t* __restrict__ entries, const int32_t* __restrict__ counts,
    int maxe, int Hm, const uint8_t* __restrict__ tile_flags, const int32_t* __restrict__ hmix,
    const T* __restrict__ Kp, const void* __restrict__ Vtp, int tiles_per_head, int first_ctile,
    const float* __restrict__ clog2n, int nl, const int32_t* __restrict__ order, int32_t* __restrict__ ctl,
    const unsigned char* __restrict__ corr_img) {
  using C = Cfg<T, D>;
  using L = AttnLds<T, D, TO, CORR>;
  constexpr size_t kTileBytes = static_cast<size_t>(kNK) * D * sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];
  TO* Z = reinterpret_cast<TO*>(smem);
  float* bias0 = reinterpret_cast<float*>(smem + L::BIAS);

  const int G = Hq / Hkv;
  int* unit_slot = reinterpret_cast<int*>(smem + L::UNIT);
  TileDma<T, D> dma;
  dma.init();
  // Persistent workgroups: each takes units from its XCD's segment of the work order, then
  // helps the other XCDs once its own is exhausted; -1 ends the loop for every wave at once.
  const int x0 = static_cast<int>(blockIdx.x % kXcds);  // dispatch is round-robin over XCDs
  int tries = 0;                                        // used by thread 0 only
  int32_t* qctl = ctl + (FAST ? 0 : kQueueCtl);
  for (;;) {
  if (threadIdx.x == 0) {
    int got = -1;
    while (tries < kXcds) {
      const int q = (x0 + tries) % kXcds;
      const int n = qctl[8 + q + 1] - qctl[8 + q];
      // A plain read first: a queue already drained (or empty) costs no atomic.
      if (__hip_atomic_load(&qctl[q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < n) {
        const int i = atomicAdd(&qctl[q], 1);
        if (i < n) {
          got = qctl[8 + q] + i;
          break;
        }
      }
      ++tries;
    }
    *unit_slot = got;
  }
  __syncthreads();
  const int idx = *unit_slot;
  __syncthreads();
  if (idx < 0) break;
  int bk, a, g;
  decode_unit(order[idx], Cq, G, bk, a, g);
  const int b = bk / Hkv, kvh = bk % Hkv;
  const int hq = kvh * G + g;
  const int hm = Hm == 1 ? 0 : (Hm == Hq ? hq : kvh);
  const size_t mrow = (static_cast<size_t>(b) * Hm + hm) * Cq + a;
  const size_t bhq = static_cast<size_t>(b) * Hq + hq;
  const size_t bkv = static_cast<size_t>(b) * Hkv + kvh;
  const T* Qh = Q + bhq * S * D;
  TO* Oh = O + bhq * S * D;
  const unsigned char* Kph = reinterpret_cast<const unsigned char*>(Kp) + bkv * tiles_per_head * kTileBytes;
  const unsigned char* Vph = static_cast<const unsigned char*>(Vtp) + bkv * tiles_per_head * kTileBytes;
  const uint8_t* flags_h = tile_flags + bkv * tiles_per_head;
  const uint8_t* keep_row = keep + mrow * Ck;
  // The query and key layouts of this (batch, K/V head): one shared layout (nl = 1) or its own.
  const size_t lay = layout_of(nl, bkv);
  const int32_t* qperm_h = q_perm + lay * S;
  const int32_t* qoff_h = q_off + lay * (Cq + 1);
  const float* clog2n_h = clog2n + lay * Ck;
  const int32_t* ent = entries + mrow * maxe;
  const int ecount = counts[mrow];

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int q_lo = qoff_h[a], q_hi = qoff_h[a + 1];

  // Centroid bias of a tile (log2 n_c where this row's cluster skipped c, -inf otherwise;
  // log2 n_c comes from the pack, -inf for a count of 0).
  auto write_bias = [&](float* dst, int ct) {
    if (threadIdx.x < kNK) {
      const int cc = ct * kNK + static_cast<int>(threadIdx.x);
      float bv = -INFINITY;
      if (cc < Ck && keep_row[cc] == 0) bv = clog2n_h[cc];
      dst[threadIdx.x] = bv;
    }
  };

  for (int rt = q_lo; rt < q_hi; rt += kRowsWG) {
    const int nrows = min(kRowsWG, q_hi - rt);
    // This lane's query row; rows past the cluster reuse row 0 and are not stored.  A wave
    // with no row of the cluster (a cluster's last block of fewer than 128 rows) only copies
    // its share of the tiles and meets the barriers: its SIMD is left to the other workgroup.
    const int my = wave * 32 + r;
    const bool wave_rows = wave * 32 < nrows;  // uniform over the wave
    const int qtok = qperm_h[rt + (my < nrows ? my : 0)];
    Frag<T> qf[C::KK];
    load_q_frags<T, D>(qf, Qh + static_cast<size_t>(qtok) * D);
    // Wait for Q here: otherwise the loop's wait counters, merged over the loop entry, make
    // every tile wait for its own prefetch before the first MFMA.
    __builtin_amdgcn_s_waitcnt(0);
    RowState<D> st;
    init_state<D>(st);

    // Tiles (centroid tiles, then kept tiles) stream through two LDS buffers: while tile j is
    // computed, tile j+1 is copied from global memory into the other buffer; one wait and one
    // barrier per tile.  The row's tile entries are read 64 at a time, one per lane, and each
    // tile takes its entry from a lane; its V^T format flag is fetched one tile ahead.
    auto kbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::K0 + i * L::KB); };
    auto vbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::V0 + i * L::VB); };
    // ALL16: every V^T tile of this head is float16 (the usual case), so the tile loop needs
    // neither the format flags nor the bfloat16 product; it is compiled separately from the
    // general loop so that the rare format switch does not burden its registers.
    // The head's packed K and V^T tiles as buffer resources (one head: at most 772 tiles of
    // 16 KB, well inside 32-bit offsets).
    const __amdgpu_buffer_rsrc_t krsrc = raw_buffer(Kph, static_cast<int>(tiles_per_head * kTileBytes));
    const __amdgpu_buffer_rsrc_t vrsrc = raw_buffer(Vph, static_cast<int>(tiles_per_head * kTileBytes));
    auto tile_loop = [&](auto all16_tag) {
    constexpr bool ALL16 = decltype(all16_tag)::value;
    int chunk = lane < ecount ? ent[lane] : 0;
    int chunk_next = 64 + lane < ecount ? ent[64 + lane] : 0;
    int e0 = ecount > 0 ? __builtin_amdgcn_readlane(chunk, 0) : 0;
    int pv0 = 0;
    if (ecount > 0) {
      const int tl = entry_tile(e0);
      dma.issue_k(Kph + tl * kTileBytes, kbuf(0));
      dma.issue_v(Vph + tl * kTileBytes, vbuf(0));
      if (entry_centroid(e0)) write_bias(bias0, tl - first_ctile);
      if (!ALL16) pv0 = __builtin_amdgcn_readfirstlane(static_cast<int>(flags_h[tl]));
    }
    wait_vmem();
    __syncthreads();
    // One tile step on buffer BJ.  The float16 loop passes BJ as a compile-time constant (two
    // steps per iteration), so LDS addresses fold into the instructions' offsets; the general
    // loop keeps one step per iteration, which costs it fewer registers.
    auto step = [&](int p, int BJ) {
      const int pn = p + 1;
      const bool have1 = pn < ecount;
      if ((pn & 63) == 0) {  // entries pn .. pn+63 move in; fetch the block after them
        chunk = chunk_next;
        const int q = pn + 64 + lane;
        chunk_next = q < ecount ? ent[q] : 0;
      }
      int e1 = 0, pv1 = 0;
      if (have1) {
        e1 = __builtin_amdgcn_readlane(chunk, pn & 63);
        const int tl = entry_tile(e1);
        if constexpr (TileDma<T, D>::kBuffer) {
          dma.issue_kv_buf(krsrc, vrsrc, tl * static_cast<int>(kTileBytes), kbuf(BJ ^ 1), vbuf(BJ ^ 1));
        } else {
          dma.issue_k(Kph + tl * kTileBytes, kbuf(BJ ^ 1));
          dma.issue_v(Vph + tl * kTileBytes, vbuf(BJ ^ 1));
        }
        if (entry_centroid(e1)) write_bias(bias0 + (BJ ^ 1) * kNK, tl - first_ctile);
        if (!ALL16) pv1 = flags_h[tl];
      }
      if (wave_rows) {
        const KeyBias kb{entry_centroid(e0) ? bias0 + BJ * kNK : nullptr};
        if constexpr (ALL16)
          tile_step16<D>(reinterpret_cast<const bf16_t*>(kbuf(BJ)), reinterpret_cast<const bf16_t*>(vbuf(BJ)),
                         reinterpret_cast<const Frag<bf16_t>*>(qf), st, c2, kb, entry_nvalid(e0));
        else
          tile_step<T, D, SwzLds<T, D>>(kbuf(BJ), vbuf(BJ), qf, st, c2, kb, entry_nvalid(e0), pv0 != 0);
      }
      wait_vmem();
      __syncthreads();
      e0 = e1;
      if (!ALL16) pv0 = __builtin_amdgcn_readfirstlane(pv1);
    };
    if constexpr (ALL16) {
      for (int p = 0; p < ecount; p += 2) {
        step(p, 0);
        if (p + 1 < ecount) step(p + 1, 1);
      }
    } else {
      for (int p = 0; p < ecount; ++p) step(p, p & 1);
    }
    };
    tile_loop(std::integral_constant<bool, FAST && sizeof(T) == 2>{});

    const float l_tot = st.l + swap_halves(st.l);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) st.o[dt][j] *= inv;
    if constexpr (CORR) {
      // The tile buffers are free (the loop ended on a barrier): copy this head's image of A
      // and c into them, then every row gets o + o A + c before its single rounding.
      load_correction_image<T, D>(corr_img + bhq * kCorrImageStride, smem);
      wait_vmem();
      __syncthreads();
      if (wave_rows) apply_correction<T, D>(st.o, smem);
      __syncthreads();  // every wave is done with the image before the rows are staged over it
    }
    // Stage the tile as rows in LDS, then store rows with 16-byte writes.
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int d = dt * 32 + 8 * (j / 4) + 4 * h + (j % 4);
        Z[my * L::ZROW + d] = from_f32<TO>(st.o[dt][j]);
      }
    if (lse != nullptr && h == 0 && my < nrows) {
      const float v = l_tot > 0.0f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
      lse[bhq * S + qtok] = v;
    }
    // Each wave stores its own 32 rows, 64 / ZCPR whole rows per instruction; a row's token
    // comes from the lane that loaded its query (a lane shuffle, not a global load).
    constexpr int ZCPR = D / L::ZEPC;  // 16-byte chunks per output row
    constexpr int RPI = 64 / ZCPR;     // rows per store instruction
#pragma unroll 1
    for (int k = 0; k < 32 / RPI; ++k) {
      const int rw = k * RPI + lane / ZCPR, ch = lane % ZCPR;  // row within the wave
      const int row = wave * 32 + rw;
      const int tok = __shfl(qtok, rw);
      if (row < nrows)
        *reinterpret_cast<uint4*>(Oh + static_cast<size_t>(tok) * D + ch * L::ZEPC) =
            *reinterpret_cast<const uint4*>(Z + row * L::ZROW + ch * L::ZEPC);
    }
    __syncthreads();
  }
  }  // units
}

// ----------------------------------------------------------------- probe rows

// Per (query row, key) mask of a probe tile: the key's cluster must be kept for the query's
// cluster.  Keep bits of the workgroup's probe rows are packed in LDS (one bit per key
// cluster); the tile's key-cluster labels are in LDS too.
struct ProbeMask {
  __device__ bool active() const { return true; }
  const uint32_t* bits;  // this lane's row of packed keep bits
  const int* klab;       // tile key -> key cluster
  int nvalid;
  __device__ float operator()(int key) const {
    if (key >= nvalid) return -INFINITY;
    const int c = klab[key];
    if (c < 0) return -INFINITY;
    return ((bits[c >> 5] >> (c & 31)) & 1u) ? 0.0f : -INFINITY;
  }
};
// Centroid columns of a probe row: log2 n_c where the row's cluster skipped c, else -inf.
struct ProbeCentroids {
  __device__ bool active() const { return true; }
  const uint32_t* bits;
  const float* log2n;  // tile centroid -> log2 n_c (-inf for empty / out of range)
  int c0;
  __device__ float operator()(int key) const {
    const int c = c0 + key;
    const float b = log2n[key];
    if (b == -INFINITY) return -INFINITY;
    return ((bits[c >> 5] >> (c & 31)) & 1u) ? -INFINITY : b;
  }
};

constexpr int kMaxCkProbe = 2048;  // packed keep bits per probe row in LDS

// Partial attention of up to 128 probe rows against one chunk of keys, written unnormalized
// with the running max (log2 units) and sum for a later merge.  DENSE: every key.  Sparse:
// only keys of kept clusters of the row's own query cluster, and (with centroids) one extra
// chunk index holding the centroid columns of its skipped clusters, which is the row of the
// block-sparse output computed in float32.
template <typename T, int D, bool SPARSE>
__global__ __launch_bounds__(kThreads, 2) void probe_partial_kernel(
    const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V, int Hq, int Hkv, int S, float c2,
    const int32_t* __restrict__ probe_idx, int M, int chunk, int ntok_chunks, int nchunks,
    const int32_t* __restrict__ q_labels, const int32_t* __restrict__ k_labels, const uint8_t* __restrict__ keep,
    int Hm, int Cq, int Ck, const int32_t* __restrict__ k_off, const float* __restrict__ Kbar,
    const float* __restrict__ Vbar, float* __restrict__ Opart, float* __restrict__ mpart,
    float* __restrict__ lpart) {
  using C = Cfg<T, D>;
  constexpr int LDS = attn_lds_bytes<T, D>();
  extern __shared__ __align__(16) unsigned char smem[];
  T* Ks = reinterpret_cast<T*>(smem);
  T* Vt = Ks + C::K_ELEMS;
  float* bias = reinterpret_cast<float*>(smem + (LDS - kNK * 4 - kFlagBytes));
  int* flags = reinterpret_cast<int*>(smem + (LDS - kFlagBytes));
  int* klab = reinterpret_cast<int*>(smem + LDS);
  uint32_t* bits = reinterpret_cast<uint32_t*>(smem + LDS + kNK * 4);
  const int ci = blockIdx.x, qt = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hq, hq = bh % Hq, kvh = hq / (Hq / Hkv);
  const T* Qh = Q + static_cast<size_t>(bh) * S * D;
  const T* Kh = K + (static_cast<size_t>(b) * Hkv + kvh) * S * D;
  const T* Vh = V + (static_cast<size_t>(b) * Hkv + kvh) * S * D;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int my = qt * kRowsWG + wave * 32 + r;
  const int qtok = probe_idx[my < M ? my : 0];
  const int words = (Ck + 31) / 32;
  if constexpr (SPARSE) {
    // Pack the keep bits of every probe row of this workgroup.
    const int hm = Hm == 1 ? 0 : (Hm == Hq ? hq : kvh);
    for (int e = threadIdx.x; e < kRowsWG * words; e += kThreads) {
      const int row = e / words, w = e % words;
      const int pr = qt * kRowsWG + row;
      uint32_t v = 0;
      if (pr < M) {
        const int a = q_labels[probe_idx[pr]];
        if (a >= 0 && a < Cq) {
          const uint8_t* krow = keep + ((static_cast<size_t>(b) * Hm + hm) * Cq + a) * Ck;
          for (int k = 0; k < 32; ++k) {
            const int c = w * 32 + k;
            if (c < Ck && krow[c] != 0) v |= 1u << k;
          }
        }
      }
      bits[row * words + w] = v;
    }
    __syncthreads();
  }
  const uint32_t* mybits = bits + (wave * 32 + r) * words;
  Frag<T> qf[C::KK];
  load_q_frags<T, D>(qf, Qh + static_cast<size_t>(qtok) * D);
  RowState<D> st;
  init_state<D>(st);
  if (ci < ntok_chunks) {
    const int k_lo = ci * chunk, k_hi = min(S, k_lo + chunk);
    for (int kt = k_lo; kt < k_hi; kt += kNK) {
      const int nvalid = min(kNK, k_hi - kt);
      auto row_of = [&](int key) { return static_cast<size_t>(kt + key) * D; };
      load_kv_tile<T, D>(Ks, Vt, flags, Kh, Vh, nvalid, row_of);
      if constexpr (SPARSE) {
        if (threadIdx.x < kNK) {
          const int key = kt + threadIdx.x;
          const int c = key < k_hi ? k_labels[key] : -1;
          klab[threadIdx.x] = (c >= 0 && c < Ck) ? c : -1;  // tokens outside every cluster stay masked
        }
      }
      __syncthreads();
      const bool f16 = sizeof(T) != 2 || tile_fits_f16(flags);
      if (!f16) {
        load_kv_tile_fallback<T, D>(Vt, Vh, nvalid, row_of);
        __syncthreads();
      }
      if constexpr (SPARSE)
        tile_step<T, D, PaddedLds<T, D>>(Ks, Vt, qf, st, c2, ProbeMask{mybits, klab, nvalid}, nvalid, f16);
      else
        tile_step<T, D, PaddedLds<T, D>>(Ks, Vt, qf, st, c2, NoBias{}, nvalid, f16);
      __syncthreads();
    }
  } else if constexpr (SPARSE) {
    // Centroid columns (the chunk past the token chunks).
    const float* Kb = Kbar + (static_cast<size_t>(b) * Hkv + kvh) * Ck * D;
    const float* Vb = Vbar + (static_cast<size_t>(b) * Hkv + kvh) * Ck * D;
    for (int c0 = 0; c0 < Ck; c0 += kNK) {
      // With an all-zero keep row the per-tile bias is log2 n_c for every non-empty cluster.
      load_centroid_tile<T, D>(Ks, Vt, bias, flags, Kb, Vb, c0, Ck, k_off, nullptr);
      __syncthreads();
      const bool f16 = sizeof(T) != 2 || tile_fits_f16(flags);
      if (!f16) {
        load_centroid_fallback<T, D>(Vt, Vb, c0, Ck);
        __syncthreads();
      }
      tile_step<T, D, PaddedLds<T, D>>(Ks, Vt, qf, st, c2, ProbeCentroids{mybits, bias, c0}, kNK, f16);
      __syncthreads();
    }
  }
  const float l_tot = st.l + swap_halves(st.l);
  if (my < M) {
    const size_t prow = (static_cast<size_t>(bh) * nchunks + ci) * M + my;
#pragma unroll
    for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4*>(Opart + prow * D + d) =
            f32x4{st.o[dt][4 * g4], st.o[dt][4 * g4 + 1], st.o[dt][4 * g4 + 2], st.o[dt][4 * g4 + 3]};
      }
    if (h == 0) {
      mpart[prow] = st.m;
      lpart[prow] = l_tot;
    }
  }
}

// One lane-uniform logit bias for a whole tile (log2 units): 0 where the lane's row takes the
// tile, -inf where it does not.
struct LaneBias {
  float b;
  __device__ bool active() const { return true; }
  __device__ float operator()(int) const { return b; }
};
// Centroid columns of a tile for a lane's row: log2 n_c where the row's query cluster skipped
// key cluster c (keep bits in LDS), -inf where it kept c or for a row without centroids.
struct RowCentroids {
  const uint32_t* bits;  // the row's keep bits (nullptr: no centroid columns)
  const float* log2n;    // tile column -> log2 n_c (-inf for a count of 0 or a column past Ck)
  int c0;
  __device__ bool active() const { return true; }
  __device__ float operator()(int key) const {
    if (bits == nullptr) return -INFINITY;
    const int c = c0 + key;
    const float b = log2n[key];
    if (b == -INFINITY) return -INFINITY;
    return ((bits[c >> 5] >> (c & 31)) & 1u) ? -INFINITY : b;
  }
};

// Probe rows from the packed K/V tiles of bsa_kv_pack (bfloat16).  Dense rows attend to
// every key: the softmax over all keys does not depend on their order, so a workgroup streams
// a run of `tpc` consecutive token tiles of one head through two LDS buffers with
// global-to-LDS copies, exactly as the attention does, for up to 128 rows; a tile's key count
// comes from its cluster (the last tile of a cluster is ragged) and its V^T format from the
// pack's flags.  SPARSE: rows [M, 2M) repeat the M probes under the block-sparse rule of the
// attention -- a token tile counts for a row only when the row's query cluster keeps the
// tile's key cluster (keep bits in LDS) -- and one more chunk, index nchunks, holds the
// centroid tiles, whose columns count for the sparse rows of the clusters that skipped them
// (with compensation; the chunk is empty without).  That chunk is a launch of its own (CEN):
// one kernel holding both kinds of tile step spilled registers inside its tile loop (0.55 ms
// against 0.19 ms for the repair's probe pass on the video workload).  Partial rows, running
// max and sum go to probe_merge_kernel.  Chunks past the head's last tile write empty
// partials.
template <int D, bool SPARSE, bool CEN = false>
__global__ __launch_bounds__(kThreads, 2) void probe_packed_kernel(
    const bf16_t* __restrict__ Q, int Hq, int Hkv, int Sq, float c2, const int32_t* __restrict__ probe_idx, int M,
    const int32_t* __restrict__ tile_off, const int32_t* __restrict__ k_off, int C, int nl,
    const uint8_t* __restrict__ tile_flags, const bf16_t* __restrict__ Kp, const void* __restrict__ Vtp,
    int tiles_per_head, int tpc, int nchunks, const int32_t* __restrict__ q_labels, const uint8_t* __restrict__ keep,
    int Hm, int Cq, const float* __restrict__ clog2n, int first_ctile, int ctiles, int comp, int words,
    float* __restrict__ Opart, float* __restrict__ mpart, float* __restrict__ lpart) {
  using T = bf16_t;
  using L = AttnLds<T, D, float>;
  constexpr size_t kTileBytes = static_cast<size_t>(kNK) * D * sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];
  int* nv = reinterpret_cast<int*>(smem + L::BIAS);   // key count of each tile of the chunk (tpc <= 2 kNK)
  int* clus = nv + 2 * kNK;                            // key cluster of each tile of the chunk
  float* cbias = reinterpret_cast<float*>(clus + 2 * kNK);  // log2 n_c of a centroid tile's columns
  uint32_t* bits = reinterpret_cast<uint32_t*>(cbias + kNK);  // [128 rows][words]: sparse rows' keep bits
  static_assert(SPARSE || !CEN, "the centroid chunk belongs to the sparse rows");
  // CEN: this launch takes the centroid chunk (index nchunks) alone, so that each kernel holds
  // one kind of tile step.
  const int ci = CEN ? nchunks : static_cast<int>(blockIdx.x), qt = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hq, hq = bh % Hq, kvh = hq / (Hq / Hkv);
  const size_t bkv = static_cast<size_t>(b) * Hkv + kvh;
  const unsigned char* Kph = reinterpret_cast<const unsigned char*>(Kp) + bkv * tiles_per_head * kTileBytes;
  const unsigned char* Vph = static_cast<const unsigned char*>(Vtp) + bkv * tiles_per_head * kTileBytes;
  const uint8_t* flags_h = tile_flags + bkv * tiles_per_head;
  // This head's layouts (nl > 1: one per (batch, K/V head), with its own probe rows).
  const size_t lay = layout_of(nl, bkv);
  tile_off += lay * (C + 1);
  k_off += lay * (C + 1);
  clog2n += lay * C;
  if (q_labels != nullptr) q_labels += lay * Sq;
  if (probe_idx != nullptr) probe_idx += lay * M;
  constexpr bool cen = CEN;  // the centroid chunk
  const int nrows = SPARSE ? 2 * M : M;
  const int nch = SPARSE ? nchunks + 1 : nchunks;
  int t0, t1;
  if (cen) {
    t0 = first_ctile;
    t1 = comp ? first_ctile + ctiles : first_ctile;
  } else {
    const int ntiles = tile_off[C];
    // tpc == 0: the head's tiles are split evenly over the chunks (at most 2 kNK each).
    const int per = tpc > 0 ? tpc : (ntiles + nchunks - 1) / nchunks;
    t0 = ci * per;
    t1 = min(ntiles, t0 + per);
  }
  // Tile t belongs to cluster c with tile_off[c] <= t < tile_off[c + 1].
  if (!cen && static_cast<int>(threadIdx.x) < t1 - t0) {
    const int t = t0 + static_cast<int>(threadIdx.x);
    int lo = 0, hi = C;  // invariant: tile_off[lo] <= t < tile_off[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (tile_off[mid] <= t) lo = mid; else hi = mid;
    }
    const int n = k_off[lo + 1] - k_off[lo];
    nv[threadIdx.x] = min(kNK, n - kNK * (t - tile_off[lo]));
    clus[threadIdx.x] = lo;
  }
  if (cen && static_cast<int>(threadIdx.x) < t1 - t0) {
    const int jt = static_cast<int>(threadIdx.x);
    nv[jt] = min(kNK, C - kNK * jt);
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int R = qt * kRowsWG + wave * 32 + r;  // this lane's row
  const bool sparse_row = SPARSE && R >= M && R < nrows;
  const int pj = SPARSE && R >= M ? R - M : R;  // its probe
  const int qtok = probe_idx != nullptr ? probe_idx[pj < M ? pj : 0] : (pj < M ? pj : 0);
  if constexpr (SPARSE) {
    // Keep bits of the sparse rows' query clusters (a dense row, or a row past the probes,
    // keeps every cluster: its bits are never read).
    const int hm = Hm == 1 ? 0 : (Hm == Hq ? hq : kvh);
    for (int e = threadIdx.x; e < kRowsWG * words; e += kThreads) {
      const int row = e / words, w = e % words;
      const int Rr = qt * kRowsWG + row;
      uint32_t v = 0;
      if (Rr >= M && Rr < nrows) {
        const int tok = probe_idx != nullptr ? probe_idx[Rr - M] : Rr - M;
        const int a = q_labels[tok];
        if (a >= 0 && a < Cq) {
          const uint8_t* kr = keep + ((static_cast<size_t>(b) * Hm + hm) * Cq + a) * C;
          for (int i = 0; i < 32; ++i) {
            const int c = w * 32 + i;
            if (c < C && kr[c] != 0) v |= 1u << i;
          }
        }
      }
      bits[row * words + w] = v;
    }
  }
  const uint32_t* mybits = bits + (wave * 32 + r) * words;
  Frag<T> qf[D / 16];
  load_q_frags<T, D>(qf, Q + static_cast<size_t>(bh) * Sq * D + static_cast<size_t>(qtok) * D);
  __builtin_amdgcn_s_waitcnt(0);
  RowState<D> st;
  init_state<D>(st);
  TileDma<T, D> dma;
  dma.init();
  auto kbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::K0 + i * L::KB); };
  auto vbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::V0 + i * L::VB); };
  if (t0 < t1) {
    dma.issue_k(Kph + t0 * kTileBytes, kbuf(0));
    dma.issue_v(Vph + t0 * kTileBytes, vbuf(0));
  }
  wait_vmem();
  __syncthreads();
  for (int t = t0; t < t1; ++t) {
    const int bj = (t - t0) & 1;
    if (cen && threadIdx.x < kNK) {  // this centroid tile's log2 n_c (read before the barrier below)
      const int c = (t - first_ctile) * kNK + static_cast<int>(threadIdx.x);
      cbias[threadIdx.x] = c < C ? clog2n[c] : -INFINITY;
    }
    if (cen) __syncthreads();
    if (t + 1 < t1) {
      dma.issue_k(Kph + (t + 1) * kTileBytes, kbuf(bj ^ 1));
      dma.issue_v(Vph + (t + 1) * kTileBytes, vbuf(bj ^ 1));
    }
    const bool pv16 = flags_h[t] != 0;
    if (cen) {
      tile_step<T, D, SwzLds<T, D>>(kbuf(bj), vbuf(bj), qf, st, c2,
                                    RowCentroids{sparse_row ? mybits : nullptr, cbias, (t - first_ctile) * kNK},
                                    nv[t - t0], pv16);
    } else if (SPARSE) {
      const int c = clus[t - t0];
      const bool take = !sparse_row || ((mybits[c >> 5] >> (c & 31)) & 1u);
      tile_step<T, D, SwzLds<T, D>>(kbuf(bj), vbuf(bj), qf, st, c2, LaneBias{take ? 0.0f : -INFINITY}, nv[t - t0],
                                    pv16);
    } else {
      tile_step<T, D, SwzLds<T, D>>(kbuf(bj), vbuf(bj), qf, st, c2, NoBias{}, nv[t - t0], pv16);
    }
    wait_vmem();
    __syncthreads();
  }
  const float l_tot = st.l + swap_halves(st.l);
  if (R < nrows) {
    const size_t prow = (static_cast<size_t>(bh) * nch + ci) * nrows + R;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int d = dt * 32 + 8 * g4 + 4 * h;
        *reinterpret_cast<f32x4*>(Opart + prow * D + d) =
            f32x4{st.o[dt][4 * g4], st.o[dt][4 * g4 + 1], st.o[dt][4 * g4 + 2], st.o[dt][4 * g4 + 3]};
      }
    if (h == 0) {
      mpart[prow] = st.m;
      lpart[prow] = l_tot;
    }
  }
}

// Rows m < split go to Od[bh][m], rows m >= split to Os[bh][m - split] (both with `split`
// rows per head).
template <int D>
__global__ __launch_bounds__(D) void probe_merge_kernel(const float* __restrict__ Opart,
                                                        const float* __restrict__ mpart,
                                                        const float* __restrict__ lpart, int M, int nchunks,
                                                        float* __restrict__ Od, float* __restrict__ lse2, int split,
                                                        float* __restrict__ Os) {
  const int m = blockIdx.x, bh = blockIdx.y, d = threadIdx.x;
  float mx = -INFINITY;
  // Unrolled so that the loads of several chunks are in flight together.
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) mx = fmaxf(mx, mpart[(static_cast<size_t>(bh) * nchunks + c) * M + m]);
  float l = 0.0f, o = 0.0f;
#pragma unroll 8
  for (int c = 0; c < nchunks; ++c) {
    const size_t prow = (static_cast<size_t>(bh) * nchunks + c) * M + m;
    const float mc = mpart[prow];
    if (mc == -INFINITY) continue;
    const float w = fast_exp2(mc - mx);
    l += lpart[prow] * w;
    o += Opart[prow * D + d] * w;
  }
  const float val = l > 0.0f ? o / l : 0.0f;
  if (m < split)
    Od[(static_cast<size_t>(bh) * split + m) * D + d] = val;
  else
    Os[(static_cast<size_t>(bh) * split + (m - split)) * D + d] = val;
  // Log-sum-exp of the scaled logits in log2 units (running max plus log2 of the sum).
  if (lse2 != nullptr && d == 0 && m < split)
    lse2[static_cast<size_t>(bh) * split + m] = l > 0.0f ? mx + __log2f(l) : -INFINITY;
}

// ----------------------------------------------------------------- block compensation error

// Compensation error of every block for the error-aware router ("Block-sparse attention"
// topic page, SVG-EAR card: a light probe estimates each block's compensation error; the
// probe of query cluster a is its mean row q_bar_a).  With the probe's dense output O_a and
// log-sum-exp lse_a (log2 units, from the dense probe pass), weights p_j = 2^(s_j c2 - lse_a)
// and, for key cluster c, N_c = sum_{j in c} p_j v_j, Z_c = sum_{j in c} p_j and
// z_hat = 2^(q_bar_a . k_bar_c c2 + log2 n_c - lse_a), the error is the norm of the
// first-order change of O_a when the block is compensated: ||z_hat v_bar_c - N_c - O_a
// (z_hat - Z_c)||_2.  Workgroup (chunk of kErrClusters key clusters, 128 probe rows, batch x
// query head): the chunk's tiles, contiguous in the packed buffer, stream through two LDS
// buffers; N_c and Z_c accumulate over a cluster's tiles and the error is formed after its
// last tile.  N_c and O_a Z_c nearly cancel where a centroid is accurate, so the P V product
// takes P as a high and a low float16 (or bfloat16) part.
constexpr int kErrClusters = 8;

template <int D>
__device__ __forceinline__ void tile_pv_split(const bf16_t* Vt, const f32x16 (&s)[2], RowState<D>& st, bool pv16) {
  using Lds = SwzLds<bf16_t, D>;
  const int lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (pv16) {
      Frag16 hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = s[ks >> 1][(ks & 1) * 8 + i];
        const _Float16 xh = static_cast<_Float16>(x);
        hi.v[i] = xh;
        lo.v[i] = static_cast<_Float16>(x - static_cast<float>(xh));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        Frag16 va;
        Lds::vfrag16(va, Vt, dt * 32 + r, ks, h);
        st.o[dt] = mma(va, hi, st.o[dt]);
        st.o[dt] = mma(va, lo, st.o[dt]);
      }
    } else {
      Frag<bf16_t> hi, lo;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float x = s[ks >> 1][(ks & 1) * 8 + i];
        const __bf16 xh = static_cast<__bf16>(x);
        hi.v[i] = xh;
        lo.v[i] = static_cast<__bf16>(x - static_cast<float>(xh));
      }
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        Frag<bf16_t> va;
        Lds::vfrag(va, Vt, dt * 32 + r, ks, h);
        st.o[dt] = mma(va, hi, st.o[dt]);
        st.o[dt] = mma(va, lo, st.o[dt]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void block_error_kernel(
    const bf16_t* __restrict__ Qb, int Hq, int Hkv, int Cq, float c2, const float* __restrict__ O1,
    const float* __restrict__ lse2, const int32_t* __restrict__ tile_off, const int32_t* __restrict__ k_off, int Ck,
    int nl, const uint8_t* __restrict__ tile_flags, const bf16_t* __restrict__ Kp, const void* __restrict__ Vtp,
    int tiles_per_head, const float* __restrict__ Kbar, const float* __restrict__ Vbar, float* __restrict__ err) {
  using T = bf16_t;
  using L = AttnLds<T, D, float>;
  constexpr size_t kTileBytes = static_cast<size_t>(kNK) * D * sizeof(T);
  extern __shared__ __align__(16) unsigned char smem[];
  float* kb_s = reinterpret_cast<float*>(smem + L::TILES);   // [kErrClusters][D] centroid keys
  float* vb_s = kb_s + kErrClusters * D;                     // [kErrClusters][D] centroid values
  int* toff_s = reinterpret_cast<int*>(vb_s + kErrClusters * D);  // first tile of each cluster (+ end)
  int* n_s = toff_s + kErrClusters + 1;                      // cluster sizes
  const int chunk = blockIdx.x, qt = blockIdx.y, bh = blockIdx.z;
  const int b = bh / Hq, hq = bh % Hq, kvh = hq / (Hq / Hkv);
  const size_t bkv = static_cast<size_t>(b) * Hkv + kvh;
  tile_off += layout_of(nl, bkv) * (Ck + 1);  // this head's key layout
  k_off += layout_of(nl, bkv) * (Ck + 1);
  const int c0 = chunk * kErrClusters, nc = min(kErrClusters, Ck - c0);
  const int t = threadIdx.x;
  for (int i = t; i < nc * D; i += kThreads) {
    kb_s[i] = Kbar[(bkv * Ck + c0) * D + i];
    vb_s[i] = Vbar[(bkv * Ck + c0) * D + i];
  }
  if (t <= nc) toff_s[t] = tile_off[c0 + t];
  if (t < nc) n_s[t] = k_off[c0 + t + 1] - k_off[c0 + t];
  const int wave = t >> 6, lane = t & 63, r = lane & 31, h = lane >> 5;
  const int my = qt * kRowsWG + wave * 32 + r;
  const size_t prow = static_cast<size_t>(bh) * Cq + (my < Cq ? my : Cq - 1);
  Frag<T> qf[D / 16];
  load_q_frags<T, D>(qf, Qb + prow * D);
  const float lse_r = lse2[prow];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  const bool store = h == 0 && my < Cq;
  float* err_row = err + (static_cast<size_t>(bh) * Cq + (my < Cq ? my : 0)) * Ck + c0;  // used only with store
  for (int ci = 0; ci < nc; ++ci)
    if (store && n_s[ci] <= 0) err_row[ci] = 0.0f;  // an empty cluster: no tiles, no error
  const int T0 = toff_s[0], T1 = toff_s[nc];
  const unsigned char* Kph = reinterpret_cast<const unsigned char*>(Kp) + bkv * tiles_per_head * kTileBytes;
  const unsigned char* Vph = static_cast<const unsigned char*>(Vtp) + bkv * tiles_per_head * kTileBytes;
  const uint8_t* flags_h = tile_flags + bkv * tiles_per_head;
  RowState<D> st;
  init_state<D>(st);
  float zl = 0.0f;  // this lane's part of Z_c
  TileDma<T, D> dma;
  dma.init();
  auto kbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::K0 + i * L::KB); };
  auto vbuf = [&](int i) { return reinterpret_cast<T*>(smem + L::V0 + i * L::VB); };
  if (T0 < T1) {
    dma.issue_k(Kph + T0 * kTileBytes, kbuf(0));
    dma.issue_v(Vph + T0 * kTileBytes, vbuf(0));
  }
  wait_vmem();
  __syncthreads();
  int ci = 0;
  for (int tt = T0; tt < T1; ++tt) {
    const int bj = (tt - T0) & 1;
    if (tt + 1 < T1) {
      dma.issue_k(Kph + (tt + 1) * kTileBytes, kbuf(bj ^ 1));
      dma.issue_v(Vph + (tt + 1) * kTileBytes, vbuf(bj ^ 1));
    }
    while (tt >= toff_s[ci + 1]) ++ci;  // the same for every lane; skips empty clusters
    const int nv = min(kNK, n_s[ci] - kNK * (tt - toff_s[ci]));
    f32x16 s[2];
    tile_qk<T, D, SwzLds<T, D>>(kbuf(bj), qf, s[0], s[1]);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = mt * 32 + 8 * (j / 4) + 4 * h + (j % 4);
        const float p = key < nv ? fast_exp2(__builtin_fmaf(s[mt][j], c2, -lse_r)) : 0.0f;
        s[mt][j] = p;
        zl += p;
      }
    tile_pv_split<D>(vbuf(bj), s, st, flags_h[tt] != 0);
    if (tt == toff_s[ci + 1] - 1) {  // the cluster's last tile: its error
      const float zc = zl + swap_halves(zl);
      float dot = 0.0f;  // q_bar . k_bar_c over this lane's half of D, then both halves
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
#pragma unroll
        for (int i = 0; i < 8; ++i) dot += static_cast<float>(qf[kk].v[i]) * kb_s[ci * D + kk * 16 + 8 * h + i];
      dot += swap_halves(dot);
      const float zh = fast_exp2(__builtin_fmaf(dot, c2, __log2f(static_cast<float>(n_s[ci])) - lse_r));
      const float dz = zh - zc;
      const float* orow = O1 + prow * D;
      float e2 = 0.0f;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int d = dt * 32 + 8 * g4 + 4 * h;
          const f32x4 o = *reinterpret_cast<const f32x4*>(orow + d);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float delta = zh * vb_s[ci * D + d + i] - st.o[dt][4 * g4 + i] - o[i] * dz;
            e2 += delta * delta;
          }
        }
      e2 += swap_halves(e2);
      if (store) err_row[ci] = sqrtf(e2);
      init_state<D>(st);
      zl = 0.0f;
    }
    wait_vmem();
    __syncthreads();
  }
}

constexpr int kProbeChunk = 2048;

struct PackedKV {
  const int32_t* tile_off;
  const int32_t* hmix;
  const uint8_t* flags;
  const void* k;
  const void* v;
  const float* clog2n;
  int tiles_per_head, first_ctile, ctiles;
};

// Tile entries per mask row: the centroid tiles plus at most every token tile of the head.
inline int list_stride(int S, int Ck) {
  const PackLayout L = pack_layout(1, 1, S, 64, Ck, 2);
  return L.centroid_tiles + L.first_centroid_tile;
}
// Workspace of the attention: tile entries [rows][stride], counts [rows], the work order
// [units] and the unit counter.
struct AttnWs {
  size_t entries, counts, order, rank, gsum, counter, aimg, total;
};
inline AttnWs attn_ws(int B, int Hq, int Hm, int Cq, int S, int Ck) {
  const size_t rows = static_cast<size_t>(B) * Hm * Cq;
  const size_t units = static_cast<size_t>(B) * Hq * Cq;
  AttnWs w;
  w.entries = 0;
  w.counts = pack_align(rows * list_stride(S, Ck) * sizeof(int32_t));
  w.order = w.counts + pack_align(rows * sizeof(int32_t));
  w.rank = w.order + pack_align(units * sizeof(int32_t));
  w.gsum = w.rank + pack_align(units * sizeof(int32_t));  // one int per K/V group (<= B * Hq)
  w.counter = w.gsum + pack_align(static_cast<size_t>(B) * Hq * sizeof(int32_t));
  w.aimg = w.counter + 256;  // correction images, one per (batch, query head)
  w.total = w.aimg + static_cast<size_t>(B) * Hq * kCorrImageStride;
  return w;
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static int cus[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cus[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cus[dev] = n;
  }
  return cus[dev];
}

template <typename T, int D, bool COMP, typename TO, bool FAST, bool CORR>
void launch_sparse_variant(hipStream_t stream, const void* Q, void* O, float* lse, int B, int Hq, int Hkv, int S,
                           float c2, const int32_t* q_perm, const int32_t* q_off, int Cq, const int32_t* k_off, int Ck,
                           const uint8_t* keep, const int32_t* entries, const int32_t* counts, int maxe, int Hm,
                           const PackedKV& P, int nl, const int32_t* order, int32_t* ctl, int units,
                           const unsigned char* corr_img) {
  constexpr int LDS = AttnLds<T, D, TO, CORR>::TOTAL;
  auto kern = sparse_attn_kernel<T, D, COMP, TO, FAST, CORR>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  const int grid = min(units, device_cus() * attn_occupancy<T, FAST>());
  hipLaunchKernelGGL(kern, dim3(grid), dim3(kThreads), LDS, stream, static_cast<const T*>(Q), static_cast<TO*>(O), lse,
                     B, Hq, Hkv, S, c2, q_perm, q_off, Cq, k_off, Ck, keep, entries, counts, maxe, Hm, P.flags, P.hmix,
                     static_cast<const T*>(P.k), P.v, P.tiles_per_head, P.first_ctile, P.clog2n, nl, order, ctl,
                     corr_img);
}

template <typename T, int D>
bsa_status launch_sparse(int B, int Hq, int Hkv, int S, const void* Q, float scale, const int32_t* q_perm,
                         const int32_t* q_off, int Cq, const int32_t* k_off, int Ck, int nl, const uint8_t* keep,
                         const int32_t* kv_count, const int16_t* kv_idx, int Hm, const void* packed, bool comp,
                         bool out_f32, const float* A, const float* cvec, void* O, float* lse, void* ws,
                         hipStream_t stream) {
  const long long nunits = static_cast<long long>(B) * Hq * Cq;
  if (nunits > 0x7fffffffLL) return BSA_E_UNSUPPORTED;
  const int units = static_cast<int>(nunits);
  const float c2 = scale * kLog2e;
  const PackLayout L = pack_layout(B, Hkv, S, D, Ck, sizeof(T), nl);
  const unsigned char* base = static_cast<const unsigned char*>(packed);
  const PackedKV P{reinterpret_cast<const int32_t*>(base + L.tile_off),
                   reinterpret_cast<const int32_t*>(base + L.hmix), base + L.flags, base + L.k, base + L.v,
                   reinterpret_cast<const float*>(base + L.clog2n), L.tiles_per_head, L.first_centroid_tile,
                   L.centroid_tiles};
  const size_t rows = static_cast<size_t>(B) * Hm * Cq;
  const int maxe = list_stride(S, Ck);
  const AttnWs W = attn_ws(B, Hq, Hm, Cq, S, Ck);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  int32_t* entries = reinterpret_cast<int32_t*>(wsb + W.entries);
  int32_t* counts = reinterpret_cast<int32_t*>(wsb + W.counts);
  int32_t* order = reinterpret_cast<int32_t*>(wsb + W.order);
  int32_t* rank = reinterpret_cast<int32_t*>(wsb + W.rank);
  int32_t* gsum = reinterpret_cast<int32_t*>(wsb + W.gsum);
  int32_t* counter = reinterpret_cast<int32_t*>(wsb + W.counter);
  unsigned char* aimg = wsb + W.aimg;
  const bool corr = A != nullptr;
  if (corr)
    hipLaunchKernelGGL((corr_image_kernel<T, D>), dim3(static_cast<unsigned>(B * Hq)), dim3(256), 0, stream, A, cvec,
                       aimg);
  hipLaunchKernelGGL(tile_list_wave_kernel, dim3(static_cast<unsigned>((rows + 3) / 4)), dim3(256), 0, stream,
                     kv_count, kv_idx, static_cast<int>(rows), Ck, k_off, P.tile_off, nl, Hq, Hkv, Hm, Cq,
                     P.first_ctile, P.ctiles, comp ? 1 : 0, maxe, entries, counts);
  constexpr bool kHalf = sizeof(T) == 2;  // float16 products exist for bfloat16 inputs only
  const int per = Cq * (Hq / Hkv);
  const bool sort_ok = per <= kMaxSortUnits;
  hipLaunchKernelGGL(group_rank_kernel, dim3(static_cast<unsigned>(B * Hkv)), dim3(kGroupThreads),
                     sort_ok ? per * 4 : 0, stream, counts, Hq, Hkv, Hm, Cq, sort_ok ? 1 : 0, rank, gsum);
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, stream, gsum, rank, B, Hq, Hkv, Cq, P.hmix,
                     kHalf ? 1 : 0, order, counter);
  // The general kernel first (usually without work), then the float16 one.
#define BSA_LAUNCH(COMP, TO, CORR)                                                                                    \
  do {                                                                                                                 \
    launch_sparse_variant<T, D, COMP, TO, false, CORR>(stream, Q, O, lse, B, Hq, Hkv, S, c2, q_perm, q_off, Cq,       \
                                                       k_off, Ck, keep, entries, counts, maxe, Hm, P, nl, order,      \
                                                       counter, units, aimg);                                         \
    if (kHalf)                                                                                                         \
      launch_sparse_variant<T, D, COMP, TO, kHalf, CORR>(stream, Q, O, lse, B, Hq, Hkv, S, c2, q_perm, q_off, Cq,     \
                                                         k_off, Ck, keep, entries, counts, maxe, Hm, P, nl, order,    \
                                                         counter, units, aimg);                                       \
  } while (0)
  if (comp) {
    if (corr) BSA_LAUNCH(true, T, true); else if (out_f32) BSA_LAUNCH(true, float, false); else BSA_LAUNCH(true, T, false);
  } else {
    if (corr) BSA_LAUNCH(false, T, true); else if (out_f32) BSA_LAUNCH(false, float, false); else BSA_LAUNCH(false, T, false);
  }
#undef BSA_LAUNCH
  return launch_status();
}

template <typename T, int D, bool SPARSE>
void launch_probe_pass(int B, int Hq, int Hkv, int S, const void* Q, const void* K, const void* V, float c2,
                       const int32_t* probe_idx, int M, const int32_t* q_labels, const int32_t* k_labels,
                       const uint8_t* keep, int Hm, int Cq, int Ck, const int32_t* k_off, const float* Kbar,
                       const float* Vbar, float* out, float* ws, hipStream_t stream) {
  constexpr int LDS = attn_lds_bytes<T, D>();
  const int ntok = (S + kProbeChunk - 1) / kProbeChunk;
  const int nchunks = ntok + ((SPARSE && Kbar != nullptr) ? 1 : 0);
  const int qtiles = (M + kRowsWG - 1) / kRowsWG;
  float* Opart = ws;
  float* mpart = Opart + static_cast<size_t>(B) * Hq * nchunks * M * D;
  float* lpart = mpart + static_cast<size_t>(B) * Hq * nchunks * M;
  const int extra = SPARSE ? kNK * 4 + kRowsWG * ((Ck + 31) / 32) * 4 : 0;
  auto kern = probe_partial_kernel<T, D, SPARSE>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS + extra);
  hipLaunchKernelGGL(kern, dim3(nchunks, qtiles, B * Hq), dim3(kThreads), LDS + extra, stream,
                     static_cast<const T*>(Q), static_cast<const T*>(K), static_cast<const T*>(V), Hq, Hkv, S, c2,
                     probe_idx, M, kProbeChunk, ntok, nchunks, q_labels, k_labels, keep, Hm, Cq, Ck, k_off, Kbar,
                     Vbar, Opart, mpart, lpart);
  hipLaunchKernelGGL((probe_merge_kernel<D>), dim3(M, B * Hq), dim3(D), 0, stream, Opart, mpart, lpart, M, nchunks,
                     out, nullptr, M, nullptr);
}

size_t probe_ws_floats(int B, int Hq, int S, int D, int M) {
  const size_t nchunks = (static_cast<size_t>(S) + kProbeChunk - 1) / kProbeChunk + 1;
  return static_cast<size_t>(B) * Hq * nchunks * M * (D + 2);
}

// Dense probe rows from the packed tiles: chunks of tpc tiles, sized so that about 24 chunks
// cover the largest possible token-tile count of a head (measured on the video workload,
// 768 tiles per head: 32 tiles per chunk 207 us, 24 tiles 226 us, 16 tiles 219 us, 48 tiles
// 243 us).
inline int packed_probe_tpc(int first_ctile) { return max(4, min(2 * kNK, (first_ctile + 23) / 24)); }
inline int packed_probe_chunks(int first_ctile) {
  const int tpc = packed_probe_tpc(first_ctile);
  return (first_ctile + tpc - 1) / tpc;
}

// Partial rows of the packed probe pass: per (batch x query head) up to nchunks + 1 chunks of
// 2 M rows (dense and sparse), D + 2 floats each.
inline size_t packed_probe_ws_bytes(int B, int Hq, int D, int M, int first_ctile) {
  return static_cast<size_t>(B) * Hq * (packed_probe_chunks(first_ctile) + 1) * 2 * M * (D + 2) * sizeof(float);
}

// Q holds Sq rows per head; probe_idx == nullptr takes rows 0 .. M-1; lse2 (log2 units) is
// optional.  Os != nullptr: also the sparse rows (q_labels, keep with Hm mask heads of Cq rows,
// compensate), from the same pass.
template <int D>
bsa_status launch_probe_packed(int B, int Hq, int Hkv, int S, int Sq, const void* Q, float scale,
                               const int32_t* probe_idx, int M, const void* packed, const int32_t* k_off, int C,
                               float* Od, float* lse2, void* ws, hipStream_t stream, int nl,
                               const int32_t* q_labels = nullptr, const uint8_t* keep = nullptr, int Hm = 1,
                               int Cq = 1, bool comp = false, float* Os = nullptr) {
  const PackLayout PL = pack_layout(B, Hkv, S, D, C, sizeof(bf16_t), nl);
  const unsigned char* base = static_cast<const unsigned char*>(packed);
  const bool sparse = Os != nullptr;
  const int nrows = sparse ? 2 * M : M;
  int tpc = packed_probe_tpc(PL.first_centroid_tile);
  int nchunks = packed_probe_chunks(PL.first_centroid_tile);  // the most chunks (sizes the workspace)
  if (sparse && nrows <= kRowsWG) {
    // The repair's pass (dense and sparse rows of up to 64 probes in one row tile): as many
    // chunks per head as one round of the workgroups the device runs at once takes, each
    // splitting the head's filled tiles (tile_off[C], read by the kernel) evenly.  On the
    // video workload (40 heads): 11 chunks per head 0.19 ms; 12, which leaves a partial second
    // round, 0.26 ms; 23 (two rounds) 0.23 ms.
    const int slots = device_cus() * 2 * 9 / 10;
    const int want = max(1, slots / (B * Hq));
    const int least = (PL.first_centroid_tile + 2 * kNK - 1) / (2 * kNK);  // chunks of at most 2 kNK tiles
    nchunks = max(least, min(nchunks, want));
    tpc = 0;
  }
  const int nch = sparse ? nchunks + 1 : nchunks;
  const int qtiles = (nrows + kRowsWG - 1) / kRowsWG;
  const int words = sparse ? (C + 31) / 32 : 0;
  float* Opart = static_cast<float*>(ws);
  float* mpart = Opart + static_cast<size_t>(B) * Hq * nch * nrows * D;
  float* lpart = mpart + static_cast<size_t>(B) * Hq * nch * nrows;
  const int LDS = AttnLds<bf16_t, D, float>::BIAS + (4 * kNK + kNK) * 4 + kRowsWG * words * 4;
#define BSA_PROBE_ARGS                                                                                                \
  static_cast<const bf16_t*>(Q), Hq, Hkv, Sq, scale * kLog2e, probe_idx, M,                                         \
      reinterpret_cast<const int32_t*>(base + PL.tile_off), k_off, C, nl, base + PL.flags,                          \
      reinterpret_cast<const bf16_t*>(base + PL.k), base + PL.v, PL.tiles_per_head, tpc, nchunks, q_labels, keep, Hm, \
      Cq, reinterpret_cast<const float*>(base + PL.clog2n), PL.first_centroid_tile, PL.centroid_tiles, comp ? 1 : 0, \
      words, Opart, mpart, lpart
  if (sparse) {
    auto kern = probe_packed_kernel<D, true, false>;
    hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    hipLaunchKernelGGL(kern, dim3(nchunks, qtiles, B * Hq), dim3(kThreads), LDS, stream, BSA_PROBE_ARGS);
    auto kcen = probe_packed_kernel<D, true, true>;
    hipFuncSetAttribute(reinterpret_cast<const void*>(kcen), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    hipLaunchKernelGGL(kcen, dim3(1, qtiles, B * Hq), dim3(kThreads), LDS, stream, BSA_PROBE_ARGS);
  } else {
    auto kern = probe_packed_kernel<D, false>;
    hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
    hipLaunchKernelGGL(kern, dim3(nch, qtiles, B * Hq), dim3(kThreads), LDS, stream, BSA_PROBE_ARGS);
  }
#undef BSA_PROBE_ARGS
  hipLaunchKernelGGL((probe_merge_kernel<D>), dim3(nrows, B * Hq), dim3(D), 0, stream, Opart, mpart, lpart, nrows,
                     nch, Od, lse2, M, Os);
  return launch_status();
}

template <typename T, int D>
bsa_status launch_probe(int B, int Hq, int Hkv, int S, const void* Q, const void* K, const void* V, float scale,
                        const int32_t* probe_idx, int M, const int32_t* q_labels, const int32_t* k_labels,
                        const uint8_t* keep, int Hm, int Cq, int Ck, const int32_t* k_off, const float* Kbar,
                        const float* Vbar, float* Od, float* Os, void* ws, hipStream_t stream) {
  const float c2 = scale * kLog2e;
  float* w = static_cast<float*>(ws);
  launch_probe_pass<T, D, false>(B, Hq, Hkv, S, Q, K, V, c2, probe_idx, M, nullptr, nullptr, nullptr, 1, 1, 1, nullptr,
                                 nullptr, nullptr, Od, w, stream);
  if (Os != nullptr)
    launch_probe_pass<T, D, true>(B, Hq, Hkv, S, Q, K, V, c2, probe_idx, M, q_labels, k_labels, keep, Hm, Cq, Ck,
                                  k_off, Kbar, Vbar, Os, w, stream);
  return launch_status();
}


// ----------------------------------------------------------------- error-aware routing: block errors

// Workspace of bsa_block_error: the dense probe pass's partials, its rows O_a [B, Hq, Cq, D]
// and log-sum-exp [B, Hq, Cq] (float32).
struct ErrWs {
  size_t part, o1, lse, total;
};
inline ErrWs err_ws(int B, int Hq, int Hkv, int S, int D, int Cq, int Ck) {
  const PackLayout PL = pack_layout(B, Hkv, S, D, Ck, sizeof(bf16_t));  // (tile counts do not depend on layouts)
  ErrWs w;
  w.part = 0;
  w.o1 = pack_align(static_cast<size_t>(B) * Hq * packed_probe_chunks(PL.first_centroid_tile) * Cq * (D + 2) *
                    sizeof(float));
  w.lse = w.o1 + pack_align(static_cast<size_t>(B) * Hq * Cq * D * sizeof(float));
  w.total = w.lse + pack_align(static_cast<size_t>(B) * Hq * Cq * sizeof(float));
  return w;
}

template <int D>
bsa_status launch_block_error(int B, int Hq, int Hkv, int S, const void* qbar, int Cq, float scale, const void* packed,
                              const int32_t* k_off, int Ck, int nl, const float* Kbar, const float* Vbar, float* err,
                              void* ws, hipStream_t stream) {
  const ErrWs W = err_ws(B, Hq, Hkv, S, D, Cq, Ck);
  unsigned char* wsb = static_cast<unsigned char*>(ws);
  float* O1 = reinterpret_cast<float*>(wsb + W.o1);
  float* lse2 = reinterpret_cast<float*>(wsb + W.lse);
  // Pass 1: the probes' dense rows and log-sum-exp (rows 0 .. Cq-1 of qbar).
  const bsa_status st = launch_probe_packed<D>(B, Hq, Hkv, S, Cq, qbar, scale, nullptr, Cq, packed, k_off, Ck, O1,
                                               lse2, wsb + W.part, stream, nl);
  if (st != BSA_OK) return st;
  // Pass 2: the per-block errors.
  const PackLayout PL = pack_layout(B, Hkv, S, D, Ck, sizeof(bf16_t), nl);
  const unsigned char* base = static_cast<const unsigned char*>(packed);
  constexpr int LDS = AttnLds<bf16_t, D, float>::TILES + 2 * kErrClusters * D * 4 + (2 * kErrClusters + 1) * 4;
  auto kern = block_error_kernel<D>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, LDS);
  hipLaunchKernelGGL(kern, dim3((Ck + kErrClusters - 1) / kErrClusters, (Cq + kRowsWG - 1) / kRowsWG, B * Hq),
                     dim3(kThreads), LDS, stream, static_cast<const bf16_t*>(qbar), Hq, Hkv, Cq, scale * kLog2e, O1,
                     lse2, reinterpret_cast<const int32_t*>(base + PL.tile_off), k_off, Ck, nl, base + PL.flags,
                     reinterpret_cast<const bf16_t*>(base + PL.k), base + PL.v, PL.tiles_per_head, Kbar, Vbar, err);
  return launch_status();
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_sparse_attention_workspace_size(int B, int Hq, int Hm, int Cq, int S, int Ck,
                                                          size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hm < 1 || Cq < 1 || S < 1 || Ck < 1) return BSA_E_ARG;
  if (Ck > 32767) return BSA_E_UNSUPPORTED;
  if (list_stride(S, Ck) >= (1 << kEntryTileBits)) return BSA_E_UNSUPPORTED;
  *bytes = attn_ws(B, Hq, Hm, Cq, S, Ck).total;
  return BSA_OK;
}

extern "C" bsa_status bsa_sparse_attention(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                           float scale, const int32_t* q_perm, const int32_t* q_offsets, int Cq,
                                           const int32_t* k_offsets, int Ck, int n_layouts, const uint8_t* keep,
                                           const int32_t* kv_count, const int16_t* kv_idx, int Hm,
                                           const void* packed, size_t packed_bytes, int compensate,
                                           const float* A, const float* c, int out_dtype, void* O, float* lse,
                                           void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype) || !valid_dtype(out_dtype)) return BSA_E_DTYPE;
  if (out_dtype != dtype && out_dtype != BSA_F32) return BSA_E_DTYPE;
  if ((A == nullptr) != (c == nullptr)) return BSA_E_ARG;
  if (A != nullptr && out_dtype != dtype) return BSA_E_UNSUPPORTED;  // the epilogue writes the input type
  if (A != nullptr && static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  if (B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Cq < 1 || Ck < 1) return BSA_E_ARG;
  if (!Q || !O || !q_perm || !q_offsets || !k_offsets || !keep || !kv_count || !kv_idx || !packed) return BSA_E_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return BSA_E_ARG;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (Hm != 1 && Hm != Hkv && Hm != Hq) return BSA_E_SHAPE;
  // Layouts per (batch, K/V head): every mask row then belongs to one of them.
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (n_layouts > 1 && Hm == 1 && Hkv > 1) return BSA_E_SHAPE;  // Hm must be Hkv or Hq
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  size_t need = 0;
  const bsa_status st = bsa_sparse_attention_workspace_size(B, Hq, Hm, Cq, S, Ck, &need);
  if (st != BSA_OK) return st;
  const PackLayout PL = pack_layout(B, Hkv, S, D, Ck, dtype_size(dtype), n_layouts);
  if (packed_bytes < PL.total) return BSA_E_WORKSPACE;
  // One head's tiles are addressed with 32-bit byte offsets.
  if (static_cast<size_t>(PL.tiles_per_head) * 64 * D * dtype_size(dtype) > 0x7fffffffu) return BSA_E_UNSUPPORTED;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  const bool out_f32 = out_dtype == BSA_F32 && dtype != BSA_F32;
#define BSA_ARGS B, Hq, Hkv, S, Q, scale, q_perm, q_offsets, Cq, k_offsets, Ck, n_layouts, keep, kv_count, kv_idx, Hm, \
                 packed, compensate != 0, out_f32, A, c, O, lse, ws, stream
  if (dtype == BSA_BF16) return D == 128 ? launch_sparse<bf16_t, 128>(BSA_ARGS) : launch_sparse<bf16_t, 64>(BSA_ARGS);
  return D == 128 ? launch_sparse<float, 128>(BSA_ARGS) : launch_sparse<float, 64>(BSA_ARGS);
#undef BSA_ARGS
}

// ----------------------------------------------------------------- allocation-free variant

// The attention's scratch memory (tile lists, work order, unit ranks, queue counters, staged
// corrections) for callers that cannot allocate: a file-scope device array, one copy per GPU
// for the life of the process.  Host code never passes the array's name to a kernel (on the
// host it is a stand-in, not a device address): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current.
constexpr size_t kStaticScratchBytes = size_t{48} << 20;
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch array, or nullptr if it cannot be had.
void* static_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) return nullptr;
    g_scratch_ptr[dev] = ptr;
  }
  return g_scratch_ptr[dev];
}
}  // namespace

extern "C" size_t bsa_sparse_attention_static_scratch_bytes(void) { return kStaticScratchBytes; }

extern "C" bsa_status bsa_sparse_attention_noalloc(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                                   float scale, const int32_t* q_perm, const int32_t* q_offsets,
                                                   int Cq, const int32_t* k_offsets, int Ck, int n_layouts,
                                                   const uint8_t* keep, const int32_t* kv_count,
                                                   const int16_t* kv_idx, int Hm,
                                                   const void* packed, size_t packed_bytes, int compensate,
                                                   const float* A, const float* c, int out_dtype, void* O,
                                                   float* lse, hipStream_t stream) {
  size_t need = 0;
  if (B < 1 || Hq < 1 || Hm < 1 || Cq < 1 || S < 1 || Ck < 1) return BSA_E_ARG;
  const bsa_status st = bsa_sparse_attention_workspace_size(B, Hq, Hm, Cq, S, Ck, &need);
  if (st != BSA_OK) return st;
  if (need > kStaticScratchBytes) return BSA_E_WORKSPACE;  // larger than the static scratch
  void* ws = static_scratch();
  if (ws == nullptr) return BSA_E_HIP;
  // Every scratch section is written by the call's own kernels before it is read (the lists,
  // ranks, totals, order and queue counters by the list and order kernels, the corrections by
  // corr_image_kernel), so nothing needs clearing between calls.
  return bsa_sparse_attention(B, Hq, Hkv, S, D, dtype, Q, scale, q_perm, q_offsets, Cq, k_offsets, Ck, n_layouts,
                              keep, kv_count, kv_idx, Hm, packed, packed_bytes, compensate, A, c, out_dtype, O, lse,
                              ws, kStaticScratchBytes, stream);
}

extern "C" bsa_status bsa_probe_attention_workspace_size(int B, int Hq, int S, int D, int M, size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || S < 1 || M < 1) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (M > 1024) return BSA_E_UNSUPPORTED;
  *bytes = probe_ws_floats(B, Hq, S, D, M) * sizeof(float);
  return BSA_OK;
}

extern "C" bsa_status bsa_probe_attention_packed_workspace_size(int B, int Hq, int Hkv, int S, int D, int M, int C,
                                                                 size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || S < 1 || M < 1 || C < 1) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  const PackLayout PL = pack_layout(B, Hkv, S, D, C, sizeof(bf16_t));
  *bytes = packed_probe_ws_bytes(B, Hq, D, M, PL.first_centroid_tile);
  return BSA_OK;
}

extern "C" bsa_status bsa_probe_attention_packed(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                                 float scale, const int32_t* probe_idx, int M, const void* packed,
                                                 size_t packed_bytes, const int32_t* k_offsets, int C,
                                                 int n_layouts, const int32_t* q_labels, const uint8_t* keep, int Hm,
                                                 int Cq, int compensate, float* O_dense_probe,
                                                 float* O_sparse_probe, void* ws, size_t ws_bytes,
                                                 hipStream_t stream) {
  if (dtype != BSA_BF16) return valid_dtype(dtype) ? BSA_E_UNSUPPORTED : BSA_E_DTYPE;
  size_t need = 0;
  const bsa_status st = bsa_probe_attention_packed_workspace_size(B, Hq, Hkv, S, D, M, C, &need);
  if (st != BSA_OK) return st;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (!Q || !probe_idx || !packed || !k_offsets || !O_dense_probe) return BSA_E_ARG;
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (O_sparse_probe != nullptr) {
    if (!q_labels || !keep || Cq < 1) return BSA_E_ARG;
    if (Hm != 1 && Hm != Hkv && Hm != Hq) return BSA_E_SHAPE;
    if (n_layouts > 1 && Hm == 1 && Hkv > 1) return BSA_E_SHAPE;  // Hm must be Hkv or Hq
    if (C > 1024) return BSA_E_UNSUPPORTED;  // keep bits of 128 rows in LDS
  }
  if (M > 1024) return BSA_E_UNSUPPORTED;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return BSA_E_ARG;
  if (packed_bytes < pack_layout(B, Hkv, S, D, C, sizeof(bf16_t), n_layouts).total) return BSA_E_WORKSPACE;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  return D == 128 ? launch_probe_packed<128>(B, Hq, Hkv, S, S, Q, scale, probe_idx, M, packed, k_offsets, C,
                                             O_dense_probe, nullptr, ws, stream, n_layouts, q_labels, keep, Hm, Cq,
                                             compensate != 0, O_sparse_probe)
                  : launch_probe_packed<64>(B, Hq, Hkv, S, S, Q, scale, probe_idx, M, packed, k_offsets, C,
                                            O_dense_probe, nullptr, ws, stream, n_layouts, q_labels, keep, Hm, Cq,
                                            compensate != 0, O_sparse_probe);
}

extern "C" bsa_status bsa_probe_attention(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                          const void* K, const void* V, float scale, const int32_t* probe_idx, int M,
                                          const int32_t* q_labels, const int32_t* k_labels, const uint8_t* keep,
                                          int Hm, int Cq, int Ck, const int32_t* k_offsets, const float* Kbar,
                                          const float* Vbar, float* O_dense_probe, float* O_sparse_probe, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  size_t need = 0;
  bsa_status st = bsa_probe_attention_workspace_size(B, Hq, S, D, M, &need);
  if (st != BSA_OK) return st;
  if (Hkv < 1 || Hq % Hkv != 0) return BSA_E_SHAPE;
  if (!Q || !K || !V || !probe_idx || !O_dense_probe) return BSA_E_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return BSA_E_ARG;
  if (O_sparse_probe != nullptr) {
    if (!q_labels || !k_labels || !keep || !k_offsets || Cq < 1 || Ck < 1) return BSA_E_ARG;
    if ((Kbar == nullptr) != (Vbar == nullptr)) return BSA_E_ARG;
    if (Hm != 1 && Hm != Hkv && Hm != Hq) return BSA_E_SHAPE;
    if (Ck > kMaxCkProbe) return BSA_E_UNSUPPORTED;
  }
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
#define BSA_ARGS B, Hq, Hkv, S, Q, K, V, scale, probe_idx, M, q_labels, k_labels, keep, Hm, Cq, Ck, k_offsets, Kbar, \
                 Vbar, O_dense_probe, O_sparse_probe, ws, stream
  if (dtype == BSA_BF16) return D == 128 ? launch_probe<bf16_t, 128>(BSA_ARGS) : launch_probe<bf16_t, 64>(BSA_ARGS);
  return D == 128 ? launch_probe<float, 128>(BSA_ARGS) : launch_probe<float, 64>(BSA_ARGS);
#undef BSA_ARGS
}

extern "C" bsa_status bsa_block_error_workspace_size(int B, int Hq, int Hkv, int S, int D, int Cq, int Ck,
                                                      size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || S < 1 || Cq < 1 || Ck < 1) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (Cq > 4096 || Ck > 32767) return BSA_E_UNSUPPORTED;
  *bytes = bsa::err_ws(B, Hq, Hkv, S, D, Cq, Ck).total;
  return BSA_OK;
}

extern "C" bsa_status bsa_block_error(int B, int Hq, int Hkv, int S, int D, int dtype, const void* qbar, int Cq,
                                      float scale, const void* packed, size_t packed_bytes, const int32_t* k_offsets,
                                      int Ck, int n_layouts, const float* Kbar, const float* Vbar, float* err,
                                      void* ws, size_t ws_bytes, hipStream_t stream) {
  if (dtype != BSA_BF16) return valid_dtype(dtype) ? BSA_E_UNSUPPORTED : BSA_E_DTYPE;
  size_t need = 0;
  const bsa_status st = bsa_block_error_workspace_size(B, Hq, Hkv, S, D, Cq, Ck, &need);
  if (st != BSA_OK) return st;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (!qbar || !packed || !k_offsets || !Kbar || !Vbar || !err) return BSA_E_ARG;
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (!(scale > 0.0f) || !(scale < INFINITY)) return BSA_E_ARG;
  if (packed_bytes < pack_layout(B, Hkv, S, D, Ck, sizeof(bf16_t), n_layouts).total) return BSA_E_WORKSPACE;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  return D == 128 ? launch_block_error<128>(B, Hq, Hkv, S, qbar, Cq, scale, packed, k_offsets, Ck, n_layouts, Kbar,
                                            Vbar, err, ws, stream)
                  : launch_block_error<64>(B, Hq, Hkv, S, qbar, Cq, scale, packed, k_offsets, Ck, n_layouts, Kbar,
                                           Vbar, err, ws, stream);
}
