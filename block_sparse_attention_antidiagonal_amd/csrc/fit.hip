// SparsePR probe-fitted residual repair: the ridge fit and the correction of every row.
//
// "Partition the Support, Reconstruct the Residual" (summary page), Probe-Fitted Residual
// Reconstruction: the residual R = O_dense - O_sparse of M probe rows is fitted by a
// weighted ridge regression (lambda = 0.1) from the standardized sparse output; the
// feature-dependent correction is projected on the top r = 16 principal residual
// directions and applied to every row.  "Sparse-block compensation", section "Deviations
// from the papers": probe weights are normalized to sum to 1.
//
// One workgroup per (batch, head) computes the fit in float64.  With M <= D probes the ridge
// system is solved in its M x M dual form, which gives the same W:
//   W = (Y^T Y + lambda I)^-1 Y^T T  =  Y^T (Y Y^T + lambda I)^-1 T,
// with Y = Omega^1/2 X and T = Omega^1/2 Rc.  The principal directions of Rc^T Omega Rc = T^T T
// come from the eigenvectors U of the M x M Gram matrix T T^T (cyclic Jacobi): V_r =
// T^T U_r Lambda_r^-1/2, and T V_r = U_r Lambda_r^1/2, so W V_r = Y^T (Y Y^T + lambda I)^-1 U_r
// Lambda_r^1/2.  The folded map is A = diag(1/sigma) (W V_r) V_r^T, c = rbar - mu A.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kMaxM = 64;
constexpr int kFitThreads = 256;

struct FitSmem {
  float Y[kMaxM][128 + 1];       // Omega^1/2 X (float32 copy of the float64 values)
  double G[kMaxM][kMaxM + 1];    // T T^T; later Y Y^T + lambda I and its Cholesky factor
  union {
    float T[kMaxM][128 + 1];     // Omega^1/2 Rc, until T T^T is formed
    double E[kMaxM][kMaxM + 1];  // eigenvectors of T T^T (columns)
    double WV[128][17];          // W V_r, once the eigenvectors are consumed
  } u;
  double Zr[kMaxM][17];          // U_r Lambda_r^1/2, then (Y Y^T + lambda I)^-1 of it
  double Vr[16][128 + 1];        // V_r^T
  double mu[128], sig[128], rbar[128];
  double w[kMaxM], sw[kMaxM];
  double eval[kMaxM];
  int order[kMaxM];
  double rot_c[kMaxM / 2], rot_s[kMaxM / 2];
  int pair_p[kMaxM / 2], pair_q[kMaxM / 2];
  double scratch[kFitThreads];
  int r_eff;
};

__device__ double block_sum(double v, double* scratch) {
  scratch[threadIdx.x] = v;
  __syncthreads();
  for (int d = kFitThreads / 2; d > 0; d >>= 1) {
    if (threadIdx.x < static_cast<unsigned>(d)) scratch[threadIdx.x] += scratch[threadIdx.x + d];
    __syncthreads();
  }
  const double s = scratch[0];
  __syncthreads();
  return s;
}

__global__ __launch_bounds__(kFitThreads) void probe_fit_kernel(const float* __restrict__ Os,
                                                                 const float* __restrict__ Od,
                                                                 const float* __restrict__ weights, int D, int M,
                                                                 float lambda, int rank, float* __restrict__ Aout,
                                                                 float* __restrict__ cout) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FitSmem& sm = *reinterpret_cast<FitSmem*>(smem_raw);
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const float* Osh = Os + static_cast<size_t>(bh) * M * D;
  const float* Odh = Od + static_cast<size_t>(bh) * M * D;
  // Pad the problem to an even size n for the round-robin Jacobi ordering; padded rows are 0.
  const int n = (M + 1) & ~1;

  // Normalized weights.
  double wsum_part = 0.0;
  for (int m = t; m < M; m += kFitThreads) wsum_part += static_cast<double>(weights[m]);
  const double wsum = block_sum(wsum_part, sm.scratch);
  for (int m = t; m < kMaxM; m += kFitThreads) {
    const double wm = m < M ? static_cast<double>(weights[m]) / wsum : 0.0;
    sm.w[m] = wm;
    sm.sw[m] = sqrt(wm);
  }
  __syncthreads();
  // Weighted mean and deviation of X0 = O[probe]; weighted mean residual.
  for (int d = t; d < D; d += kFitThreads) {
    double mu = 0.0, rb = 0.0;
    for (int m = 0; m < M; ++m) {
      const double x = static_cast<double>(Osh[m * D + d]);
      mu += sm.w[m] * x;
      rb += sm.w[m] * (static_cast<double>(Odh[m * D + d]) - x);
    }
    double var = 0.0;
    for (int m = 0; m < M; ++m) {
      const double x = static_cast<double>(Osh[m * D + d]);
      var += sm.w[m] * (x - mu) * (x - mu);
    }
    double sg = sqrt(var);
    if (sg < 1e-6) sg = 1.0;
    sm.mu[d] = mu;
    sm.sig[d] = sg;
    sm.rbar[d] = rb;
  }
  __syncthreads();
  // Y = sqrt(w) (X0 - mu) / sigma,  T = sqrt(w) (R - rbar); rows past M are zero.
  for (int e = t; e < kMaxM * D; e += kFitThreads) {
    const int m = e / D, d = e % D;
    float y = 0.0f, tr = 0.0f;
    if (m < M) {
      const double x = static_cast<double>(Osh[m * D + d]);
      const double rres = static_cast<double>(Odh[m * D + d]) - x;
      y = static_cast<float>(sm.sw[m] * (x - sm.mu[d]) / sm.sig[d]);
      tr = static_cast<float>(sm.sw[m] * (rres - sm.rbar[d]));
    }
    sm.Y[m][d] = y;
    sm.u.T[m][d] = tr;
  }
  __syncthreads();
  // G = T T^T (n x n).
  for (int e = t; e < n * n; e += kFitThreads) {
    const int i = e / n, j = e % n;
    double g = 0.0;
    for (int d = 0; d < D; ++d) g += static_cast<double>(sm.u.T[i][d]) * sm.u.T[j][d];
    sm.G[i][j] = g;
  }
  __syncthreads();
  for (int e = t; e < n * n; e += kFitThreads) sm.u.E[e / n][e % n] = (e / n == e % n) ? 1.0 : 0.0;
  __syncthreads();

  // Cyclic Jacobi on G (round-robin pairing of n indices, n/2 disjoint rotations a round).
  double fro_part = 0.0;
  for (int e = t; e < n * n; e += kFitThreads) fro_part += sm.G[e / n][e % n] * sm.G[e / n][e % n];
  const double fro = sqrt(block_sum(fro_part, sm.scratch));
  const int half = n / 2;
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off_part = 0.0;
    for (int e = t; e < n * n; e += kFitThreads) {
      const int i = e / n, j = e % n;
      if (i != j) off_part += sm.G[i][j] * sm.G[i][j];
    }
    const double off = sqrt(block_sum(off_part, sm.scratch));
    if (!(off > 1e-15 * fro)) break;
    for (int round = 0; round < n - 1; ++round) {
      if (t < half) {
        // Position 0 holds index 0; positions 1..n-1 rotate by one each round.
        const int pos_a = t, pos_b = n - 1 - t;
        int p = pos_a == 0 ? 0 : 1 + (pos_a - 1 + round) % (n - 1);
        int q = pos_b == 0 ? 0 : 1 + (pos_b - 1 + round) % (n - 1);
        if (p > q) {
          const int tmp = p;
          p = q;
          q = tmp;
        }
        const double apq = sm.G[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double theta = (sm.G[q][q] - sm.G[p][p]) / (2.0 * apq);
          const double tt = (theta >= 0.0 ? 1.0 : -1.0) / (fabs(theta) + sqrt(theta * theta + 1.0));
          c = 1.0 / sqrt(tt * tt + 1.0);
          s = tt * c;
        }
        sm.pair_p[t] = p;
        sm.pair_q[t] = q;
        sm.rot_c[t] = c;
        sm.rot_s[t] = s;
      }
      __syncthreads();
      // Columns of G and E: (G J)_ip = c G_ip - s G_iq, (G J)_iq = s G_ip + c G_iq.
      for (int e = t; e < half * n; e += kFitThreads) {
        const int k = e / n, i = e % n;
        const int p = sm.pair_p[k], q = sm.pair_q[k];
        const double c = sm.rot_c[k], s = sm.rot_s[k];
        const double gp = sm.G[i][p], gq = sm.G[i][q];
        sm.G[i][p] = c * gp - s * gq;
        sm.G[i][q] = s * gp + c * gq;
        const double ep = sm.u.E[i][p], eq = sm.u.E[i][q];
        sm.u.E[i][p] = c * ep - s * eq;
        sm.u.E[i][q] = s * ep + c * eq;
      }
      __syncthreads();
      // Rows: (J^T G)_pj = c G_pj - s G_qj, (J^T G)_qj = s G_pj + c G_qj.
      for (int e = t; e < half * n; e += kFitThreads) {
        const int k = e / n, j = e % n;
        const int p = sm.pair_p[k], q = sm.pair_q[k];
        const double c = sm.rot_c[k], s = sm.rot_s[k];
        const double gp = sm.G[p][j], gq = sm.G[q][j];
        sm.G[p][j] = c * gp - s * gq;
        sm.G[q][j] = s * gp + c * gq;
      }
      __syncthreads();
    }
  }
  // Eigenvalues sorted descending; kept directions have eigenvalue > 1e-12 of the largest.
  if (t == 0) {
    for (int i = 0; i < n; ++i) {
      sm.eval[i] = sm.G[i][i];
      sm.order[i] = i;
    }
    for (int i = 0; i < n; ++i)
      for (int j = i + 1; j < n; ++j)
        if (sm.eval[sm.order[j]] > sm.eval[sm.order[i]]) {
          const int tmp = sm.order[i];
          sm.order[i] = sm.order[j];
          sm.order[j] = tmp;
        }
    const double emax = sm.eval[sm.order[0]];
    int r_eff = 0;
    if (emax > 0.0)
      for (int i = 0; i < n && r_eff < rank; ++i)
        if (sm.eval[sm.order[i]] > 1e-12 * emax) ++r_eff;
    sm.r_eff = r_eff;
  }
  __syncthreads();
  const int r_eff = sm.r_eff;
  // Zr = U_r Lambda_r^1/2 (M x r);  V_r^T row k = T^T u_k / sqrt(lambda_k), with T
  // recomputed from the inputs (its LDS copy was overwritten by the eigenvectors).
  for (int e = t; e < M * r_eff; e += kFitThreads) {
    const int m = e / r_eff, k = e % r_eff;
    const int col = sm.order[k];
    sm.Zr[m][k] = sm.u.E[m][col] * sqrt(sm.eval[col]);
  }
  for (int e = t; e < r_eff * D; e += kFitThreads) {
    const int k = e / D, d = e % D;
    const int col = sm.order[k];
    double v = 0.0;
    for (int m = 0; m < M; ++m) {
      const double x = static_cast<double>(Osh[m * D + d]);
      const double tr = sm.sw[m] * ((static_cast<double>(Odh[m * D + d]) - x) - sm.rbar[d]);
      v += tr * sm.u.E[m][col];
    }
    sm.Vr[k][d] = v / sqrt(sm.eval[col]);
  }
  __syncthreads();
  // G <- Y Y^T + lambda I (M x M), then its Cholesky factor (lower, right-looking).
  for (int e = t; e < M * M; e += kFitThreads) {
    const int i = e / M, j = e % M;
    double g = 0.0;
    for (int d = 0; d < D; ++d) g += static_cast<double>(sm.Y[i][d]) * sm.Y[j][d];
    sm.G[i][j] = g + (i == j ? static_cast<double>(lambda) : 0.0);
  }
  __syncthreads();
  for (int k = 0; k < M; ++k) {
    if (t == 0) sm.G[k][k] = sqrt(sm.G[k][k]);
    __syncthreads();
    const double dkk = sm.G[k][k];
    for (int i = k + 1 + t; i < M; i += kFitThreads) sm.G[i][k] /= dkk;
    __syncthreads();
    const int rem = M - k - 1;
    for (int e = t; e < rem * rem; e += kFitThreads) {
      const int i = k + 1 + e / rem, j = k + 1 + e % rem;
      if (j <= i) sm.G[i][j] -= sm.G[i][k] * sm.G[j][k];
    }
    __syncthreads();
  }
  // Solve (L L^T) z = Zr, one right-hand side per thread.
  if (t < r_eff) {
    for (int i = 0; i < M; ++i) {
      double v = sm.Zr[i][t];
      for (int j = 0; j < i; ++j) v -= sm.G[i][j] * sm.Zr[j][t];
      sm.Zr[i][t] = v / sm.G[i][i];
    }
    for (int i = M - 1; i >= 0; --i) {
      double v = sm.Zr[i][t];
      for (int j = i + 1; j < M; ++j) v -= sm.G[j][i] * sm.Zr[j][t];
      sm.Zr[i][t] = v / sm.G[i][i];
    }
  }
  __syncthreads();
  // W V_r = Y^T z (D x r), stored over the eigenvectors (no longer needed).
  for (int e = t; e < D * r_eff; e += kFitThreads) {
    const int d = e / r_eff, k = e % r_eff;
    double v = 0.0;
    for (int m = 0; m < M; ++m) v += static_cast<double>(sm.Y[m][d]) * sm.Zr[m][k];
    sm.u.WV[d][k] = v;
  }
  __syncthreads();
  // A = diag(1/sigma) (W V_r) V_r^T;  c = rbar - mu A.  One thread per output column j.
  float* Ah = Aout + static_cast<size_t>(bh) * D * D;
  for (int j = t; j < D; j += kFitThreads) {
    double cj = sm.rbar[j];
    for (int i = 0; i < D; ++i) {
      double a = 0.0;
      for (int k = 0; k < r_eff; ++k) a += sm.u.WV[i][k] * sm.Vr[k][j];
      a /= sm.sig[i];
      Ah[static_cast<size_t>(i) * D + j] = static_cast<float>(a);
      cj -= sm.mu[i] * a;
    }
    cout[static_cast<size_t>(bh) * D + j] = static_cast<float>(cj);
  }
}

// O <- O + O A + c for 128 rows per workgroup: (O A) on bf16 MFMA into LDS, then a
// row-parallel pass adds O and c in float32 and rounds once.  O is exact in bfloat16; A is
// split into high and low bfloat16 parts so the product keeps float32 accuracy.
template <int D>
__global__ __launch_bounds__(256) void apply_bf16_kernel(bf16_t* __restrict__ O, const float* __restrict__ A,
                                                          const float* __restrict__ cvec, int S) {
  constexpr int ROW = D + 8;
  extern __shared__ __align__(16) unsigned char smem_apply[];
  bf16_t* AtH = reinterpret_cast<bf16_t*>(smem_apply);  // A^T rows: At[j][i] = A[i][j]
  bf16_t* AtL = AtH + D * ROW;
  float* Z = reinterpret_cast<float*>(AtL + D * ROW);  // [128][D + 4]
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * 128;
  const float* Ah = A + static_cast<size_t>(bh) * D * D;
  bf16_t* Oh = O + static_cast<size_t>(bh) * S * D;
  for (int e = threadIdx.x; e < D * D; e += 256) {
    const int i = e / D, j = e % D;
    const float a = Ah[e];
    const __bf16 hi = static_cast<__bf16>(a);
    AtH[j * ROW + i].bits = __builtin_bit_cast(uint16_t, hi);
    AtL[j * ROW + i] = from_f32<bf16_t>(a - static_cast<float>(hi));
  }
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  // Output^T tile (D x 32 rows of this wave): A-operand = A^T rows, B-operand = O rows.
  const int my = row0 + wave * 32 + r;
  const int src = my < S ? my : S - 1;
  f32x16 acc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    Frag<bf16_t> ob;
    load_frag(ob, Oh + static_cast<size_t>(src) * D + kk * 16 + 8 * h);
#pragma unroll
    for (int jt = 0; jt < D / 32; ++jt) {
      Frag<bf16_t> ah, al;
      load_frag(ah, AtH + (jt * 32 + r) * ROW + kk * 16 + 8 * h);
      load_frag(al, AtL + (jt * 32 + r) * ROW + kk * 16 + 8 * h);
      acc[jt] = mma(ah, ob, acc[jt]);
      acc[jt] = mma(al, ob, acc[jt]);
    }
  }
#pragma unroll
  for (int jt = 0; jt < D / 32; ++jt)
#pragma unroll
    for (int j = 0; j < 16; ++j) Z[(wave * 32 + r) * (D + 4) + jt * 32 + 8 * (j / 4) + 4 * h + (j % 4)] = acc[jt][j];
  __syncthreads();
  const float* ch = cvec + static_cast<size_t>(bh) * D;
  for (int e = threadIdx.x; e < 128 * (D / 8); e += 256) {
    const int rr = e / (D / 8), g = e % (D / 8);
    const int row = row0 + rr;
    if (row >= S) continue;
    bf16_t* p = Oh + static_cast<size_t>(row) * D + g * 8;
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t wv[4] = {q.x, q.y, q.z, q.w};
    uint32_t outw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = g * 8 + 2 * i;
      const float lo = __uint_as_float(wv[i] << 16) + Z[rr * (D + 4) + d] + ch[d];
      const float hi = __uint_as_float(wv[i] & 0xffff0000u) + Z[rr * (D + 4) + d + 1] + ch[d + 1];
      outw[i] = pack_bf16x2(lo, hi);
    }
    *reinterpret_cast<uint4*>(p) = make_uint4(outw[0], outw[1], outw[2], outw[3]);
  }
}

// Float32 outputs: plain float32 arithmetic, one row per thread pass.
__global__ __launch_bounds__(256) void apply_f32_kernel(float* __restrict__ O, const float* __restrict__ A,
                                                        const float* __restrict__ cvec, int S, int D) {
  extern __shared__ float rows[];  // 8 rows x D
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * 8;
  float* Oh = O + static_cast<size_t>(bh) * S * D;
  const float* Ah = A + static_cast<size_t>(bh) * D * D;
  for (int e = threadIdx.x; e < 8 * D; e += 256) {
    const int rr = e / D, d = e % D;
    rows[e] = row0 + rr < S ? Oh[static_cast<size_t>(row0 + rr) * D + d] : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 8 * D; e += 256) {
    const int rr = e / D, j = e % D;
    if (row0 + rr >= S) continue;
    float v = rows[e] + cvec[static_cast<size_t>(bh) * D + j];
    for (int i = 0; i < D; ++i) v += rows[rr * D + i] * Ah[static_cast<size_t>(i) * D + j];
    Oh[static_cast<size_t>(row0 + rr) * D + j] = v;
  }
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_probe_fit(int B, int Hq, int D, const float* O_sparse_probe, const float* O_dense_probe,
                                    const float* weights, int M, float lambda, int rank, float* A, float* c,
                                    hipStream_t stream) {
  if (B < 1 || Hq < 1 || !O_sparse_probe || !O_dense_probe || !weights || !A || !c) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (M < 2) return BSA_E_ARG;
  if (M > kMaxM) return BSA_E_UNSUPPORTED;
  if (!(lambda > 0.0f) || !(lambda < INFINITY)) return BSA_E_ARG;
  if (rank < 1 || rank > D) return BSA_E_ARG;
  if (rank > 16) return BSA_E_UNSUPPORTED;
  const int smem = static_cast<int>(sizeof(FitSmem));
  hipFuncSetAttribute(reinterpret_cast<const void*>(probe_fit_kernel), hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  hipLaunchKernelGGL(probe_fit_kernel, dim3(B * Hq), dim3(kFitThreads), smem, stream, O_sparse_probe, O_dense_probe,
                     weights, D, M, lambda, rank, A, c);
  return launch_status();
}

extern "C" bsa_status bsa_probe_apply(int B, int Hq, int S, int D, int dtype, void* O, const float* A, const float* c,
                                      hipStream_t stream) {
  if (!valid_dtype(dtype)) return BSA_E_DTYPE;
  if (B < 1 || Hq < 1 || S < 1 || !O || !A || !c) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  if (dtype == BSA_BF16) {
    const dim3 grid((S + 127) / 128, B * Hq);
    const int smem128 = 2 * 128 * (128 + 8) * 2 + 128 * (128 + 4) * 4;
    const int smem64 = 2 * 64 * (64 + 8) * 2 + 128 * (64 + 4) * 4;
    if (D == 128) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(apply_bf16_kernel<128>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, smem128);
      hipLaunchKernelGGL((apply_bf16_kernel<128>), grid, dim3(256), smem128, stream, static_cast<bf16_t*>(O), A, c, S);
    } else {
      hipFuncSetAttribute(reinterpret_cast<const void*>(apply_bf16_kernel<64>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, smem64);
      hipLaunchKernelGGL((apply_bf16_kernel<64>), grid, dim3(256), smem64, stream, static_cast<bf16_t*>(O), A, c, S);
    }
  } else {
    const dim3 grid((S + 7) / 8, B * Hq);
    hipLaunchKernelGGL(apply_f32_kernel, grid, dim3(256), 8 * D * sizeof(float), stream, static_cast<float*>(O), A, c,
                       S, D);
  }
  return launch_status();
}
