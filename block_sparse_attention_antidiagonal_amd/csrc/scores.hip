// XAttention antidiagonal block scores.
//
// "Dynamic block masks and head-wise mask reuse", section "XAttention -- anti-diagonal block
// scoring": every stride x stride sub-block of Q K^T is summarized by the sum along its
// anti-diagonal; the strided logits are softmaxed per row and summed per block x block
// tile; section "Deviations from the papers": rows are divided by their total; section
// "Out of scope, and why": the sequence is zero-padded to a multiple of the block size and
// padded keys take softmax mass.
//
// The anti-diagonal sum of sub-block (i', j') is the dot product of two length stride*D
// vectors: strided query row i' lists tokens i'*s+s-1, ..., i'*s (reverse order) and strided
// key row j' lists tokens j'*s, ..., j'*s+s-1.  So the strided logits are one GEMM with
// contraction length stride*D, computed here with MFMA in tiles of 256 x 256 strided rows
// (8 waves of 128 keys x 64 queries), the operands streaming through LDS in stages of one
// token column (tt) and 64 bytes of head dimension, copied straight from global memory
// (gathered through the cluster order) into XOR-swizzled LDS rows through a ring of four
// stage buffers, copies three stages ahead of the products, and each wave reads the first
// fragments of the next stage before the barrier that ends the current one.
// Its epilogue keeps, per strided query row, the tile max, the tile sum of exponentials and
// the per-block sums relative to that max; a second pass merges the tiles of a row (the
// full-row softmax), sums the rows of a query block and normalizes.
// Workspace: part[bh][key block][strided row], mstat/lstat[bh][key tile][strided row].
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kTile = 256;      // strided rows per tile side
constexpr int kSThreads = 512;  // 8 waves: 2 (keys) x 4 (queries)
constexpr int kRowB = 64;       // bytes of one strided row per stage
constexpr int kNBuf = 4;        // stage buffers in LDS (kNBuf - 1 stages copied ahead)
using SRow = Swz<kRowB>;
static_assert(kNBuf == 4, "the stage waits assume at most two later stages in flight");
// Source of the zero padding copies: one token row of the widest input (128 float32).
__device__ const uint4 kZeroRow[32] = {};

template <typename T>
struct SStage {
  static constexpr int KCE = kRowB / static_cast<int>(sizeof(T));  // elements per row per stage
  static constexpr int KS = KCE / 16;                              // 16-wide MFMA steps per stage
  static constexpr int OP_BYTES = kTile * kRowB;                   // one operand of a stage
  static constexpr int BUF_BYTES = 2 * OP_BYTES;                   // keys + queries
  static constexpr int NCH = OP_BYTES / 16 / kSThreads;            // 16-byte chunks per thread per operand
  static constexpr int EPC = 16 / static_cast<int>(sizeof(T));
  static constexpr int LDS_BYTES = kNBuf * BUF_BYTES + 2 * kTile * 4 + 3 * 2 * kTile * 4;  // stages, reductions, tokens
};

// S^T tile: keys (A operand) x queries (B operand).  Wave w: keys 128*(w/4).., queries 64*(w%4)..
template <typename T, int D, int R>
__global__ __launch_bounds__(kSThreads, 1) void score_gemm_kernel(const T* __restrict__ Q, const T* __restrict__ K,
                                                                   const int32_t* __restrict__ perm, int Hq, int Hkv,
                                                                   int S, int stride, int Ns, int nb, int ntk, float c2,
                                                                   float* __restrict__ part, float* __restrict__ mstat,
                                                                   float* __restrict__ lstat,
                                                                   const uint8_t* __restrict__ heads, int Hs) {
  using C = SStage<T>;
  extern __shared__ __align__(16) unsigned char smem[];
  float* red = reinterpret_cast<float*>(smem + kNBuf * C::BUF_BYTES);  // [2][kTile]
  // Workgroups are dispatched to the 8 XCDs round-robin in linear order, and each XCD has its
  // own L2: the tiles of one (batch, head) are mapped to one XCD, query strip by query strip,
  // so that the workgroups running together there read the same strided rows at about the
  // same contraction step.  Heads beyond a multiple of 8 keep the plain order.
  int kt, qt, bh;
  {
    const int ntt = ntk * ntk;
    const int L = static_cast<int>(blockIdx.x + ntk * (blockIdx.y + ntk * blockIdx.z));
    const int nbh = static_cast<int>(gridDim.z), full = (nbh / kXcds) * kXcds;
    int tile;
    if (L < full * ntt) {
      const int x = L % kXcds, slot = L / kXcds;
      bh = (slot / ntt) * kXcds + x;
      tile = slot % ntt;
    } else {
      bh = L / ntt;
      tile = L % ntt;
    }
    qt = tile / ntk;
    kt = tile % ntk;
  }
  const int b = bh / Hq, hq = bh % Hq, kvh = hq / (Hq / Hkv);
  // Score heads whose mask is kept from an earlier call are not scored (the whole workgroup
  // leaves before any barrier).
  if (heads != nullptr && heads[static_cast<size_t>(b) * Hs + (Hs == Hq ? hq : kvh)] == 0) return;
  const unsigned char* Qh = reinterpret_cast<const unsigned char*>(Q + static_cast<size_t>(bh) * S * D);
  const unsigned char* Kh = reinterpret_cast<const unsigned char*>(K + (static_cast<size_t>(b) * Hkv + kvh) * S * D);
  const int t = threadIdx.x, wave = t >> 6, lane = t & 63, r = lane & 31, h = lane >> 5;
  const int kw = wave >> 2, qw = wave & 3;

  // This thread's copy slots: chunk j of each operand is LDS slot (8 j + wave) * 64 + lane,
  // i.e. row slot / 8 and swizzled chunk position slot % 8 of that row.
  int srow[C::NCH], scol[C::NCH];
#pragma unroll
  for (int j = 0; j < C::NCH; ++j) {
    const int slot = (j * 8 + wave) * 64 + lane;
    srow[j] = slot / SRow::CPR;
    scol[j] = SRow::pos(srow[j], slot % SRow::CPR);  // the global chunk that lands in this slot
  }
  // Tokens of the tile's strided rows, one token column at a time, in an LDS ring of three
  // columns: tok[c % 3][operand][row] = perm of the row's token in column c.  Each thread
  // copies one entry (4 bytes) straight from perm, two columns ahead of use, so the token
  // lookups never wait on a register load.  Rows past the sequence copy perm[0] and are
  // recognized as padding when used.  Without perm the token is the position itself.
  int* tok = reinterpret_cast<int*>(smem + kNBuf * C::BUF_BYTES + 2 * kTile * 4);  // [3][2][kTile]
  auto copy_tokens = [&](int tt) {
#if defined(__HIP_DEVICE_COMPILE__)
    if (perm != nullptr) {
      const int op = t / kTile, i = t % kTile;  // operand 0 = keys, 1 = queries
      const int row = (op == 0 ? kt : qt) * kTile + i;
      const int pos = op == 0 ? row * stride + tt : row * stride + stride - 1 - tt;
      const int* src = (row < Ns && pos < S) ? perm + pos : perm;
      __builtin_amdgcn_global_load_lds(src, tok + ((tt % 3) * 2 + op) * kTile + (t & ~63) % kTile, 4, 0, 0);
    }
#endif
  };
  constexpr int kDC = D * static_cast<int>(sizeof(T)) / kRowB;  // stages per token column
  // Copy sources of this thread's chunks for one token column: row address plus chunk offset,
  // or the zero row for padding.  Computed once per column; each stage adds a constant.
  const unsigned char* ksrc[C::NCH];
  const unsigned char* qsrc[C::NCH];
  auto column_sources = [&](int tt) {
    const int* ktab = tok + ((tt % 3) * 2) * kTile;
    const int* qtab = ktab + kTile;
#pragma unroll
    for (int j = 0; j < C::NCH; ++j) {
      const int jk = kt * kTile + srow[j], iq = qt * kTile + srow[j];
      const int pk = jk * stride + tt, pq = iq * stride + stride - 1 - tt;
      const bool kval = jk < Ns && pk < S, qval = iq < Ns && pq < S;
      const int ktk = perm ? ktab[srow[j]] : pk, qtk = perm ? qtab[srow[j]] : pq;
      const size_t off = scol[j] * 16;
      // Padding copies zeros from kZeroRow, so that every thread issues the same number of
      // copies per stage (the stage waits count them).
      ksrc[j] = (kval ? Kh + static_cast<size_t>(ktk) * D * sizeof(T) : reinterpret_cast<const unsigned char*>(kZeroRow)) + off;
      qsrc[j] = (qval ? Qh + static_cast<size_t>(qtk) * D * sizeof(T) : reinterpret_cast<const unsigned char*>(kZeroRow)) + off;
    }
  };
  // Stage x (token column x / kDC, bytes (x % kDC) * kRowB of each token row) goes to buffer
  // x % kNBuf.  Entering token column tt, the tokens of column tt + 2 are copied (into the
  // ring slot column tt - 1 used).
  auto issue = [&](int x) {
    const int xb = x % kNBuf, xd = x % kDC;
    if (xd == 0) {
      const int tt = x / kDC;
      if (tt + 2 < stride) copy_tokens(tt + 2);
      column_sources(tt);
    }
    unsigned char* As = smem + xb * C::BUF_BYTES;
    unsigned char* Bs = As + C::OP_BYTES;
#pragma unroll
    for (int j = 0; j < C::NCH; ++j) {
      const int slot_base = (j * 8 + wave) * 64;
#if defined(__HIP_DEVICE_COMPILE__)
      __builtin_amdgcn_global_load_lds(ksrc[j] + xd * kRowB, As + slot_base * 16, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(qsrc[j] + xd * kRowB, Bs + slot_base * 16, 16, 0, 0);
#endif
    }
  };

  f32x16 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = f32x16{};

  constexpr int kG = kDC > kNBuf ? kDC : kNBuf;  // stages per unrolled group
  const int nst = stride * kDC;  // a multiple of kG (stride >= 4)
  copy_tokens(0);
  if (stride > 1) copy_tokens(1);
  wait_vmem();
  __syncthreads();
  constexpr int kPerStage = 2 * C::NCH;  // tile copies per thread per stage
  // Software pipeline across the barriers: at the barrier that ends stage st every stage up to
  // st + 2 is in LDS for every wave, so a wave reads the first fragments of stage st + 1 before
  // that barrier and starts its products right after it.  Copies run three stages ahead of
  // the products (stage st + 4 is issued into the buffer stage st has just freed).
  issue(0);
  issue(1);
  issue(2);
  issue(3);
  wait_vmem_n<2 * kPerStage>();  // stages 0 and 1 (the copies of 2 and 3 may be in flight)
  pipe_barrier();
  Frag<T> fa[4], fb[2];
  auto load_frags = [&](const unsigned char* As, int ks) {
    const unsigned char* Bs = As + C::OP_BYTES;
#pragma unroll
    for (int m = 0; m < 4; ++m) swz_frag<SRow>(fa[m], As, kw * 128 + m * 32 + r, ks * 16 + 8 * h);
#pragma unroll
    for (int n = 0; n < 2; ++n) swz_frag<SRow>(fb[n], Bs, qw * 64 + n * 32 + r, ks * 16 + 8 * h);
  };
  auto products = [&]() {
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 2; ++n) acc[m][n] = mma(fa[m], fb[n], acc[m][n]);
  };
  load_frags(smem, 0);
  for (int base = 0; base < nst; base += kG) {
#pragma unroll
    for (int u = 0; u < kG; ++u) {
      const int st = base + u;
      const unsigned char* As = smem + (u % kNBuf) * C::BUF_BYTES;
#pragma unroll
      for (int ks = 0; ks < C::KS; ++ks) {
        products();
        if (ks + 1 < C::KS) load_frags(As, ks + 1);
      }
      if (st + 1 < nst) load_frags(smem + ((u + 1) % kNBuf) * C::BUF_BYTES, 0);
      // The barrier ending stage st: stages up to st + 2 landed (st + 3 may be in flight);
      // every wave is done with stage st's buffer, which stage st + 4 then refills.
      const int later = min(1, nst - 3 - st);
      if (later >= 1)
        wait_vmem_n<kPerStage>();
      else
        wait_vmem_n<0>();
      pipe_barrier();
      if (st + 4 < nst) issue(st + 4);
    }
  }
  wait_vmem();
  __syncthreads();

  // Epilogue.  acc[m][n][j]: key kt*256 + kw*128 + m*32 + 8*(j/4) + 4*h + j%4,
  //                          query qt*256 + qw*64 + n*32 + r.
  float mx[2];
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    float v = -INFINITY;
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int key = kt * kTile + kw * 128 + m * 32 + 8 * (j / 4) + 4 * h + (j % 4);
        const float y = key < Ns ? acc[m][n][j] * c2 : -INFINITY;
        acc[m][n][j] = y;
        v = fmaxf(v, y);
      }
    v = fmaxf(v, swap_halves(v));
    mx[n] = v;
  }
  if (h == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) red[kw * kTile + qw * 64 + n * 32 + r] = mx[n];
  }
  __syncthreads();
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int ql = qw * 64 + n * 32 + r;
    mx[n] = fmaxf(red[ql], red[kTile + ql]);
  }
  __syncthreads();
  float ls[2] = {0.0f, 0.0f};
#pragma unroll
  for (int n = 0; n < 2; ++n)
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float e = fast_exp2(acc[m][n][j] - mx[n]);
        acc[m][n][j] = e;
        ls[n] += e;
      }
  // Block sums over R consecutive keys.
  const size_t pbase = static_cast<size_t>(bh) * nb;
#pragma unroll
  for (int n = 0; n < 2; ++n) {
    const int query = qt * kTile + qw * 64 + n * 32 + r;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int kbase = kt * kTile + kw * 128 + m * 32;  // first key of this 32-key group
      if constexpr (R <= 4) {
        // Blocks lie inside one lane's 4-key runs.
#pragma unroll
        for (int g = 0; g < 4; ++g)
#pragma unroll
          for (int q0 = 0; q0 < 4; q0 += R) {
            float s = 0.0f;
#pragma unroll
            for (int e = 0; e < R; ++e) s += acc[m][n][4 * g + q0 + e];
            const int key0 = kbase + 8 * g + 4 * h + q0;
            if (query < Ns && key0 < Ns) part[(pbase + key0 / R) * Ns + query] = s;
          }
      } else {
        // A block spans R/8 run pairs: runs 8*g..8*g+3 (lower half) and 8*g+4.. (upper half).
        constexpr int kRunsPer = R / 8;
#pragma unroll
        for (int g0 = 0; g0 < 4; g0 += kRunsPer) {
          float s = 0.0f;
#pragma unroll
          for (int g = g0; g < g0 + kRunsPer; ++g)
#pragma unroll
            for (int e = 0; e < 4; ++e) s += acc[m][n][4 * g + e];
          s += swap_halves(s);
          const int key0 = kbase + 8 * g0;
          if (h == 0 && query < Ns && key0 < Ns) part[(pbase + key0 / R) * Ns + query] = s;
        }
      }
    }
    ls[n] += swap_halves(ls[n]);
  }
  if (h == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) red[kw * kTile + qw * 64 + n * 32 + r] = ls[n];
  }
  __syncthreads();
  if (kw == 0 && h == 0) {
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int ql = qw * 64 + n * 32 + r;
      const int query = qt * kTile + ql;
      if (query < Ns) {
        const size_t s_idx = (static_cast<size_t>(bh) * ntk + kt) * Ns + query;
        mstat[s_idx] = mx[n];
        lstat[s_idx] = red[ql] + red[kTile + ql];
      }
    }
  }
}

// One workgroup per (batch, score head, kFinQB query blocks): merge the key tiles of each
// strided row (full-row softmax), sum each block's rows, normalize, and average over the query
// heads of a group when pooling.  A thread owns key blocks c and reads, for each, the kFinQB R
// consecutive strided rows of the workgroup (128 contiguous bytes for R = 8), so the rows
// 8 KB apart in the partial sums are read in whole cache lines.  Per query block the
// arithmetic and its order are those of one block per workgroup.
constexpr int kFinQB = 4;
template <int R>
__global__ __launch_bounds__(256) void score_finalize_kernel(const float* __restrict__ part,
                                                              const float* __restrict__ mstat,
                                                              const float* __restrict__ lstat, int Hq, int Hs,
                                                              int Ns, int nb, int ntk, float* __restrict__ scores,
                                                              const uint8_t* __restrict__ heads) {
  constexpr int QR = kFinQB * R;  // strided rows of the workgroup
  __shared__ float Mrow[QR], Lrow[QR];
  __shared__ float red[kFinQB][256];
  const int a0 = blockIdx.x * kFinQB, bhs = blockIdx.y;
  if (heads != nullptr && heads[bhs] == 0) return;  // rows kept from an earlier call
  const int nq = min(kFinQB, nb - a0);              // query blocks of this workgroup
  const int b = bhs / Hs, hs = bhs % Hs;
  const int G = Hq / Hs;
  constexpr int kPerT = 4;  // key blocks per thread (nb <= 1024)
  float acc[kFinQB][kPerT] = {};
  for (int gi = 0; gi < G; ++gi) {
    const int hq = hs * G + gi;
    const size_t bh = static_cast<size_t>(b) * Hq + hq;
    if (threadIdx.x < QR && static_cast<int>(threadIdx.x) < nq * R) {
      const int row = a0 * R + threadIdx.x;
      float M = -INFINITY;
#pragma unroll 8
      for (int k = 0; k < ntk; ++k) M = fmaxf(M, mstat[(bh * ntk + k) * Ns + row]);
      float L = 0.0f;
#pragma unroll 8
      for (int k = 0; k < ntk; ++k) {
        const size_t s = (bh * ntk + k) * Ns + row;
        L += lstat[s] * fast_exp2(mstat[s] - M);
      }
      Mrow[threadIdx.x] = M;
      Lrow[threadIdx.x] = L;
    }
    __syncthreads();
    float mass[kFinQB][kPerT];
#pragma unroll
    for (int e = 0; e < kPerT; ++e) {
      const int c = threadIdx.x + e * 256;
#pragma unroll
      for (int q = 0; q < kFinQB; ++q) mass[q][e] = 0.0f;
      if (c < nb) {
        const int k = c * R / kTile;
        const float* prow = part + (bh * nb + c) * Ns + a0 * R;
        const float* mrow = mstat + (bh * ntk + k) * Ns + a0 * R;
#pragma unroll
        for (int q = 0; q < kFinQB; ++q) {
          if (q < nq) {
#pragma unroll
            for (int i = 0; i < R; ++i) {
              const float w = fast_exp2(mrow[q * R + i] - Mrow[q * R + i]) / Lrow[q * R + i];
              mass[q][e] += prow[q * R + i] * w;
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < kFinQB; ++q) {
      float tot = 0.0f;
#pragma unroll
      for (int e = 0; e < kPerT; ++e) tot += mass[q][e];
      red[q][threadIdx.x] = tot;
    }
    __syncthreads();
    for (int d = 128; d > 0; d >>= 1) {
      if (threadIdx.x < static_cast<unsigned>(d))
#pragma unroll
        for (int q = 0; q < kFinQB; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + d];
      __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < kFinQB; ++q) {
      const float inv = 1.0f / red[q][0];
#pragma unroll
      for (int e = 0; e < kPerT; ++e) acc[q][e] += mass[q][e] * inv;
    }
    __syncthreads();
  }
  const float invG = 1.0f / static_cast<float>(G);
#pragma unroll
  for (int q = 0; q < kFinQB; ++q) {
    if (q >= nq) break;
    float* out = scores + (static_cast<size_t>(bhs) * nb + a0 + q) * nb;
#pragma unroll
    for (int e = 0; e < kPerT; ++e) {
      const int c = threadIdx.x + e * 256;
      if (c < nb) out[c] = G == 1 ? acc[q][e] : acc[q][e] * invG;
    }
  }
}

struct ScoreDims {
  int nb, Ns, ntk;
};

inline ScoreDims score_dims(int S, int block, int stride) {
  ScoreDims d;
  d.nb = (S + block - 1) / block;
  d.Ns = d.nb * (block / stride);
  d.ntk = (d.Ns + kTile - 1) / kTile;
  return d;
}

template <typename T, int D, int R>
void launch_scores(int B, int Hq, int Hkv, int S, const void* Q, const void* K, const int32_t* perm, int stride,
                   float score_scale, int pool_gqa, float* scores, void* ws, hipStream_t stream, const ScoreDims& sd,
                   const uint8_t* heads) {
  const int Hs = pool_gqa ? Hkv : Hq;
  float* part = static_cast<float*>(ws);
  float* mstat = part + static_cast<size_t>(B) * Hq * sd.nb * sd.Ns;
  float* lstat = mstat + static_cast<size_t>(B) * Hq * sd.ntk * sd.Ns;
  auto kern = score_gemm_kernel<T, D, R>;
  hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize,
                      SStage<T>::LDS_BYTES);
  hipLaunchKernelGGL(kern, dim3(sd.ntk, sd.ntk, B * Hq), dim3(kSThreads), SStage<T>::LDS_BYTES, stream,
                     static_cast<const T*>(Q), static_cast<const T*>(K), perm, Hq, Hkv, S, stride, sd.Ns, sd.nb, sd.ntk,
                     score_scale * kLog2e, part, mstat, lstat, heads, Hs);
  hipLaunchKernelGGL((score_finalize_kernel<R>), dim3((sd.nb + kFinQB - 1) / kFinQB, B * Hs), dim3(256), 0, stream,
                     part, mstat, lstat, Hq, Hs, sd.Ns, sd.nb, sd.ntk, scores, heads);
}

template <typename T, int D>
bsa_status dispatch_r(int R, int B, int Hq, int Hkv, int S, const void* Q, const void* K, const int32_t* perm,
                      int stride, float score_scale, int pool_gqa, float* scores, void* ws, hipStream_t stream,
                      const ScoreDims& sd, const uint8_t* heads) {
#define BSA_R(RR) launch_scores<T, D, RR>(B, Hq, Hkv, S, Q, K, perm, stride, score_scale, pool_gqa, scores, ws, stream, sd, heads)
  switch (R) {
    case 2: BSA_R(2); break;
    case 4: BSA_R(4); break;
    case 8: BSA_R(8); break;
    case 16: BSA_R(16); break;
    default: return BSA_E_UNSUPPORTED;
  }
#undef BSA_R
  return launch_status();
}

bsa_status scores_entry(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                        const int32_t* perm, int block, int stride, float score_scale, int pool_gqa, float* scores,
                        void* ws, size_t ws_bytes, hipStream_t stream, const uint8_t* heads) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  size_t need = 0;
  bsa_status st = bsa_antidiag_scores_workspace_size(B, Hq, Hkv, S, D, block, stride, &need);
  if (st != BSA_OK) return st;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (!Q || !K || !scores) return BSA_E_ARG;
  if (!(score_scale > 0.0f) || !(score_scale < INFINITY)) return BSA_E_ARG;
  if (pool_gqa != 0 && pool_gqa != 1) return BSA_E_ARG;
  if (!ws || ws_bytes < need) return BSA_E_WORKSPACE;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  const ScoreDims sd = score_dims(S, block, stride);
  const int R = block / stride;
  if (dtype == BSA_BF16) {
    if (D == 128) return dispatch_r<bf16_t, 128>(R, B, Hq, Hkv, S, Q, K, perm, stride, score_scale, pool_gqa, scores, ws, stream, sd, heads);
    return dispatch_r<bf16_t, 64>(R, B, Hq, Hkv, S, Q, K, perm, stride, score_scale, pool_gqa, scores, ws, stream, sd, heads);
  }
  if (D == 128) return dispatch_r<float, 128>(R, B, Hq, Hkv, S, Q, K, perm, stride, score_scale, pool_gqa, scores, ws, stream, sd, heads);
  return dispatch_r<float, 64>(R, B, Hq, Hkv, S, Q, K, perm, stride, score_scale, pool_gqa, scores, ws, stream, sd, heads);
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_antidiag_scores_workspace_size(int B, int Hq, int Hkv, int S, int D, int block, int stride,
                                                         size_t* bytes) {
  if (!bytes || B < 1 || Hq < 1 || Hkv < 1 || S < 1 || block < 1 || stride < 1) return BSA_E_ARG;
  if (block % stride != 0) return BSA_E_ARG;
  const int R = block / stride;
  if (R != 2 && R != 4 && R != 8 && R != 16) return BSA_E_UNSUPPORTED;
  if (stride != 4 && stride != 8 && stride != 16 && stride != 32) return BSA_E_UNSUPPORTED;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  const ScoreDims sd = score_dims(S, block, stride);
  if (sd.nb > 1024) return BSA_E_UNSUPPORTED;
  *bytes = static_cast<size_t>(B) * Hq * sd.Ns * (static_cast<size_t>(sd.nb) + 2 * sd.ntk) * sizeof(float);
  return BSA_OK;
}

extern "C" bsa_status bsa_antidiag_scores(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q, const void* K,
                                          const int32_t* perm, int block, int stride, float score_scale, int pool_gqa,
                                          float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  return scores_entry(B, Hq, Hkv, S, D, dtype, Q, K, perm, block, stride, score_scale, pool_gqa, scores, ws, ws_bytes,
                      stream, nullptr);
}

extern "C" bsa_status bsa_antidiag_scores_heads(int B, int Hq, int Hkv, int S, int D, int dtype, const void* Q,
                                                const void* K, const int32_t* perm, int block, int stride,
                                                float score_scale, int pool_gqa, const uint8_t* heads, float* scores,
                                                void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!heads) return BSA_E_ARG;
  return scores_entry(B, Hq, Hkv, S, D, dtype, Q, K, perm, block, stride, score_scale, pool_gqa, scores, ws, ws_bytes,
                      stream, heads);
}
