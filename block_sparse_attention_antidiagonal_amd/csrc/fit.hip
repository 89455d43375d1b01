// SparsePR probe-fitted residual repair: the ridge fit and the correction of every row.
//
// "Partition the Support, Reconstruct the Residual" (summary page), Probe-Fitted Residual
// Reconstruction: the residual R = O_dense - O_sparse of M probe rows is fitted by a
// weighted ridge regression (lambda = 0.1) from the standardized sparse output; the
// feature-dependent correction is projected on the top r = 16 principal residual
// directions and applied to every row.  "Sparse-block compensation", section "Deviations
// from the papers": probe weights are normalized to sum to 1.
//
// One workgroup per (batch, head) computes the fit in float64.  With M <= 64 probes the ridge
// system is solved in its M x M dual form, which gives the same W (more probes: the D x D
// primal form further below):
//   W = (Y^T Y + lambda I)^-1 Y^T T  =  Y^T (Y Y^T + lambda I)^-1 T,
// with Y = Omega^1/2 X and T = Omega^1/2 Rc.  The principal directions of Rc^T Omega Rc = T^T T
// come from the eigenvectors U of the M x M Gram matrix T T^T (Householder tridiagonalization,
// multisection on Sturm counts, inverse iteration, back-transformation): V_r =
// T^T U_r Lambda_r^-1/2, and T V_r = U_r Lambda_r^1/2, so W V_r = Y^T (Y Y^T + lambda I)^-1 U_r
// Lambda_r^1/2.  The folded map is A = diag(1/sigma) (W V_r) V_r^T, c = rbar - mu A.
#include "common.hpp"

namespace bsa {
namespace {

constexpr int kMaxM = 64;
constexpr int kN = 64;  // eigenproblem size: the M x M Gram matrix padded with zero rows
constexpr int kFitThreads = 256;
constexpr int kMaxRank = 16;

struct FitSmem {
  float Y[kN][128 + 1];  // raw sparse rows, then Omega^1/2 X (float32 of the float64 values)
  union {
    float T[kN][128 + 1];          // raw dense rows, then Omega^1/2 Rc
    double Vr[kMaxRank][128 + 1];  // V_r^T, once T is consumed
  } t;
  double G[kN][kN + 1];  // T T^T; later Y Y^T + lambda I and its Cholesky factor
  union {
    double E[kN][kN + 1];          // eigenvectors of T T^T (columns)
    double WV[128][kMaxRank + 1];  // diag(1/sigma) W V_r, once the eigenvectors are consumed
    struct {                       // exchange buffers of the reduction steps (by step parity)
      double colH[2][kN];          // column k of T T^T
      double colL[2][kN];          // column k of Y Y^T + lambda I
      double p[2][kN];             // p = G v
      double vp[2][kFitThreads / 64];  // per-wave partial sums of v^T p
    } hh;
  } e;
  double Zr[kN][kMaxRank + 1];  // U_r Lambda_r^1/2, then (Y Y^T + lambda I)^-1 of it
  double mu[128], sig[128], rbar[128];
  double w[kN], sw[kN];
  double eval[kN];
  double u[kMaxRank];  // (mu / sigma)^T W V_r
  double dg[kN], od[kN], e2[kN];  // tridiagonal form: diagonal, off-diagonal, off-diagonal squared
  double lam[kMaxRank];           // the largest eigenvalues, descending
  int order[kN];
  double wave_part[kFitThreads / 64];
  int r_eff;
};

// Cross-lane moves of a double with DPP (VALU, no LDS round trip): CTRL is the DPP control.
template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const unsigned long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp(static_cast<int>(b & 0xffffffffu), CTRL, 0xf, 0xf, false);
  const int hi = __builtin_amdgcn_mov_dpp(static_cast<int>(b >> 32), CTRL, 0xf, 0xf, false);
  return __longlong_as_double((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                              static_cast<unsigned>(lo));
}
__device__ __forceinline__ double readlane_f64(double v, int lane) {
  const unsigned long long b = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_readlane(static_cast<int>(b & 0xffffffffu), lane);
  const int hi = __builtin_amdgcn_readlane(static_cast<int>(b >> 32), lane);
  return __longlong_as_double((static_cast<unsigned long long>(static_cast<unsigned>(hi)) << 32) |
                              static_cast<unsigned>(lo));
}
// Sum over each 16-lane row: lane pairs, quads, half rows, rows (every lane gets its row's sum).
__device__ __forceinline__ double row16_sum(double v) {
  v += dpp_f64<0xB1>(v);   // quad_perm [1, 0, 3, 2]
  v += dpp_f64<0x4E>(v);   // quad_perm [2, 3, 0, 1]
  v += dpp_f64<0x141>(v);  // row_half_mirror
  v += dpp_f64<0x140>(v);  // row_mirror
  return v;
}
// Sum over the wave (every lane gets the total).
__device__ __forceinline__ double wave_sum_f64(double v) {
  v = row16_sum(v);
  return (readlane_f64(v, 0) + readlane_f64(v, 16)) + (readlane_f64(v, 32) + readlane_f64(v, 48));
}

// Sum over the workgroup (every thread gets the total).
__device__ double block_sum(double v, double* part) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();  // earlier readers of `part` are done
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = v;
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < kFitThreads / 64; ++i) s += part[i];
  return s;
}

// acc[r][c] = sum_d X[i0+r][d] X[j0+c][d] (i0 = 4 (t / 16), j0 = 4 (t % 16)): thread t's 4 x 4
// block of the 64 x 64 Gram matrix of the rows of X (in LDS, float32), float64 sums, plus
// diag_add on the diagonal.
__device__ __forceinline__ void gram64_block(const float (*X)[128 + 1], int D, double (&acc)[4][4], double diag_add) {
  const int i0 = (threadIdx.x / 16) * 4, j0 = (threadIdx.x % 16) * 4;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[r][c] = 0.0;
  for (int d = 0; d < D; ++d) {
    double a[4], b[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      a[r] = static_cast<double>(X[i0 + r][d]);
      b[r] = static_cast<double>(X[j0 + r][d]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[r][c] += a[r] * b[c];
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) acc[r][r] += i0 == j0 ? diag_add : 0.0;
}

__global__ __launch_bounds__(kFitThreads) void probe_fit_kernel(const float* __restrict__ Os,
                                                                 const float* __restrict__ Od,
                                                                 const float* __restrict__ weights, int D, int M,
                                                                 int Hq, int Hkv, int nl, float lambda, int rank,
                                                                 float* __restrict__ Aout, float* __restrict__ cout) {
  static_assert(kFitThreads == 256, "the 4 x 4 blocking assumes 256 threads");
  extern __shared__ __align__(16) unsigned char smem_raw[];
  FitSmem& sm = *reinterpret_cast<FitSmem*>(smem_raw);
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const float* Osh = Os + static_cast<size_t>(bh) * M * D;
  const float* Odh = Od + static_cast<size_t>(bh) * M * D;
  if (nl > 1) weights += ((bh / Hq) * static_cast<size_t>(Hkv) + (bh % Hq) / (Hq / Hkv)) * M;  // the head's layout

  // Raw rows into LDS (rows past M are zero), normalized weights.
  for (int e = t; e < kN * D; e += kFitThreads) {
    const int m = e / D, d = e % D;
    sm.Y[m][d] = m < M ? Osh[e] : 0.0f;
    sm.t.T[m][d] = m < M ? Odh[e] : 0.0f;
  }
  double wsum_part = 0.0;
  for (int m = t; m < M; m += kFitThreads) wsum_part += static_cast<double>(weights[m]);
  const double wsum = block_sum(wsum_part, sm.wave_part);
  for (int m = t; m < kN; m += kFitThreads) {
    const double wm = m < M ? static_cast<double>(weights[m]) / wsum : 0.0;
    sm.w[m] = wm;
    sm.sw[m] = sqrt(wm);
  }
  __syncthreads();
  // Weighted mean and deviation of X0 = O[probe]; weighted mean residual.
  for (int d = t; d < D; d += kFitThreads) {
    double mu = 0.0, rb = 0.0;
    for (int m = 0; m < M; ++m) {
      const double x = static_cast<double>(sm.Y[m][d]);
      mu += sm.w[m] * x;
      rb += sm.w[m] * (static_cast<double>(sm.t.T[m][d]) - x);
    }
    double var = 0.0;
    for (int m = 0; m < M; ++m) {
      const double x = static_cast<double>(sm.Y[m][d]) - mu;
      var += sm.w[m] * x * x;
    }
    double sg = sqrt(var);
    if (sg < 1e-6) sg = 1.0;
    sm.mu[d] = mu;
    sm.sig[d] = sg;
    sm.rbar[d] = rb;
  }
  __syncthreads();
  // Y = sqrt(w) (X0 - mu) / sigma,  T = sqrt(w) (R - rbar), in place; rows past M stay zero.
  for (int e = t; e < M * D; e += kFitThreads) {
    const int m = e / D, d = e % D;
    const double x = static_cast<double>(sm.Y[m][d]);
    const double rres = static_cast<double>(sm.t.T[m][d]) - x;
    sm.Y[m][d] = static_cast<float>(sm.sw[m] * (x - sm.mu[d]) / sm.sig[d]);
    sm.t.T[m][d] = static_cast<float>(sm.sw[m] * (rres - sm.rbar[d]));
  }
  __syncthreads();
  // G = T T^T and G2 = Y Y^T + lambda I (64 x 64): thread t holds the 4 x 4 blocks of both at
  // rows i0.., columns j0.. in registers.  G2 runs over all 64 rows: the zero rows past M give
  // the block sqrt(lambda) I in its factor, which the zero right-hand sides there leave at zero.
  const int i0 = (t / 16) * 4, j0 = (t % 16) * 4;
  double g[4][4], g2[4][4], qb[4][4];  // qb: this thread's block of Q = H_0 H_1 ... (starts at I)
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) qb[r][c] = i0 + r == j0 + c ? 1.0 : 0.0;
  gram64_block(sm.t.T, D, g, 0.0);
  gram64_block(sm.Y, D, g2, static_cast<double>(lambda));
  auto& hh = sm.e.hh;
  // Column 0 of G and of G2 into the exchange buffers (by the threads holding it).
  if (j0 == 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      hh.colH[0][i0 + r] = g[r][0];
      hh.colL[0][i0 + r] = g2[r][0];
    }
  }
  __syncthreads();

  // Leading eigenpairs of G, in four steps: Householder reduction to tridiagonal form, the
  // largest kMaxRank eigenvalues by multisection on Sturm counts, their eigenvectors by inverse
  // iteration on the tridiagonal matrix (orthogonalized), and the back-transformation.
  //
  // (1) Step k reflects rows and columns k+1.. so that column k has zeros below the
  // subdiagonal: H = I - 2 v v^T with |v| = 1; the trailing block becomes G - v w^T - w v^T with
  // w = 2 G v - 2 (v^T G v) v.  Every wave forms the reflector from column k (lane = element);
  // each thread then forms p = G v on its block, summed over the 16 lanes of its row block, and
  // after one barrier (for v^T p and p by column) updates its block.  The product of the
  // reflectors, Q = H_0 H_1 ..., is accumulated on the same blocks (Q <- Q - 2 (Q v) v^T, no
  // barrier of its own), so the eigenvectors of G are Q times those of the tridiagonal form.  The
  // same steps eliminate G2 = L D L^T (L unit lower triangular, D the pivots): step k subtracts
  // G2[i][k] G2[k][j] / G2[k][k] from the trailing block, so G2 stays symmetric and afterwards
  // G2[k][k] = d_k and G2[i][k] = G2[k][i] = L[i][k] d_k for i > k.  Two barriers per step.
  {
    const int wave = t >> 6, lane = t & 63;
    for (int k = 0; k < kN - 2; ++k) {
      const int b = k & 1;
      const double xl = lane > k ? hh.colH[b][lane] : 0.0;
      const double s2 = wave_sum_f64(xl * xl);
      const double x0 = hh.colH[b][k + 1];
      double alpha = 0.0, vn2 = 0.0;
      if (s2 > 0.0) {
        alpha = x0 >= 0.0 ? -sqrt(s2) : sqrt(s2);
        vn2 = 2.0 * s2 - 2.0 * x0 * alpha;
      }
      const double vinv = vn2 > 0.0 ? 1.0 / sqrt(vn2) : 0.0;
      if (t == 0) {
        sm.dg[k] = hh.colH[b][k];
        sm.od[k] = alpha;
      }
      double vr[4], vc[4], lr[4], lc[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = i0 + r, j = j0 + r;
        vr[r] = i > k ? (hh.colH[b][i] - (i == k + 1 ? alpha : 0.0)) * vinv : 0.0;
        vc[r] = j > k ? (hh.colH[b][j] - (j == k + 1 ? alpha : 0.0)) * vinv : 0.0;
        lr[r] = hh.colL[b][i];
        lc[r] = hh.colL[b][j];
      }
      const double rpiv = 1.0 / hh.colL[b][k];
      double p[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc += g[r][c] * vc[c];
        p[r] = row16_sum(acc);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        double acc = 0.0;
#pragma unroll
        for (int c = 0; c < 4; ++c) acc += qb[r][c] * vc[c];
        const double qv2 = 2.0 * row16_sum(acc);
#pragma unroll
        for (int c = 0; c < 4; ++c) qb[r][c] -= qv2 * vc[c];
      }
      double part = (t & 15) == 0 ? (vr[0] * p[0] + vr[1] * p[1]) + (vr[2] * p[2] + vr[3] * p[3]) : 0.0;
      part = (readlane_f64(part, 0) + readlane_f64(part, 16)) + (readlane_f64(part, 32) + readlane_f64(part, 48));
      if (lane == 0) hh.vp[b][wave] = part;
      if ((t & 15) == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) hh.p[b][i0 + r] = p[r];
      }
      __syncthreads();  // v^T p partials and p are in LDS
      const double vp = (hh.vp[b][0] + hh.vp[b][1]) + (hh.vp[b][2] + hh.vp[b][3]);
      if (vn2 > 0.0) {  // else the column is already zero: H = I
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          const double wc = 2.0 * hh.p[b][j0 + c] - 2.0 * vp * vc[c];
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const double wr = 2.0 * p[r] - 2.0 * vp * vr[r];
            if (i0 + r > k && j0 + c > k) g[r][c] -= vr[r] * wc + wr * vc[c];
          }
        }
      }
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double rk = lc[c] * rpiv;
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (i0 + r > k && j0 + c > k) g2[r][c] -= lr[r] * rk;
      }
      if (j0 == ((k + 1) & ~3)) {
        const int c = (k + 1) & 3;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          hh.colH[b ^ 1][i0 + r] = c == 0 ? g[r][0] : c == 1 ? g[r][1] : c == 2 ? g[r][2] : g[r][3];
          hh.colL[b ^ 1][i0 + r] = c == 0 ? g2[r][0] : c == 1 ? g2[r][1] : c == 2 ? g2[r][2] : g2[r][3];
        }
      }
      __syncthreads();  // column k+1 is in LDS
    }
  }
  // The last 2 x 2 block of the tridiagonal form, and the last elimination step of G2.
  if (t == 0) {
    sm.dg[kN - 2] = hh.colH[0][kN - 2];
    sm.od[kN - 2] = hh.colH[0][kN - 1];
    sm.od[kN - 1] = 0.0;
  }
  if (t == kFitThreads - 1) {
    sm.dg[kN - 1] = g[3][3];
    g2[3][3] -= hh.colL[0][kN - 1] * (hh.colL[0][kN - 1] * (1.0 / hh.colL[0][kN - 2]));
  }
  // Q into the LDS matrix, for the back-transformation.
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) sm.G[i0 + r][j0 + c] = qb[r][c];
  __syncthreads();
  if (t < kN) sm.e2[t] = sm.od[t] * sm.od[t];
  __syncthreads();

  // (2) Sturm count: eigenvalues below x = sign changes of the LDL^T pivots of T - x I.
  double emax2 = 0.0, glo = INFINITY, ghi = -INFINITY;
  for (int i = 0; i < kN; ++i) {
    const double r0 = i > 0 ? fabs(sm.od[i - 1]) : 0.0;
    const double r1 = i < kN - 1 ? fabs(sm.od[i]) : 0.0;
    glo = fmin(glo, sm.dg[i] - r0 - r1);
    ghi = fmax(ghi, sm.dg[i] + r0 + r1);
    emax2 = fmax(emax2, sm.e2[i]);
  }
  const double span = fmax(ghi - glo, 1e-300);
  const double pivmin = 1e-290 * fmax(1.0, emax2);
  // Only the signs of the pivots matter, so the hardware reciprocal stands in for division.
  auto below = [&](double x) {
    int neg = 0;
    double q = 1.0;
    for (int i = 0; i < kN; ++i) {
      q = (sm.dg[i] - x) - (i > 0 ? sm.e2[i - 1] * __builtin_amdgcn_rcp(q) : 0.0);
      if (fabs(q) < pivmin) q = -pivmin;
      neg += q < 0.0 ? 1 : 0;
    }
    return neg;
  };
  {  // 16 eigenvalues at once: lanes of a 16-lane group probe 16 points of its interval
    const int k = t >> 4, j = t & 15;
    double a = glo - 1e-3 * span, b = ghi + 1e-3 * span;
    // 17^10 > 2e12: each eigenvalue to about 1e-12 of the spectrum's span, close enough for
    // the inverse iteration below (the fit itself uses only the eigenvectors: lambda^1/2 in
    // Zr and lambda^-1/2 in V_r cancel in A).
    for (int it = 0; it < 10; ++it) {
      const double x = a + (b - a) * static_cast<double>(j + 1) / 17.0;
      const bool ok = (kN - below(x)) <= k;  // at most k eigenvalues above x: lambda_k <= x
      const unsigned long long mask = __ballot(ok);
      const unsigned bits = static_cast<unsigned>(mask >> (16 * ((threadIdx.x & 63) >> 4))) & 0xffffu;
      const int f = bits ? __builtin_ctz(bits) : 16;
      const double na = f == 0 ? a : a + (b - a) * static_cast<double>(f) / 17.0;
      const double nb = f == 16 ? b : a + (b - a) * static_cast<double>(f + 1) / 17.0;
      a = na;
      b = nb;
    }
    if (j == 0) sm.lam[k] = 0.5 * (a + b);
  }
  __syncthreads();
  if (t == 0) {
    const double lmax = sm.lam[0];
    int r_eff = 0;
    if (lmax > 0.0) r_eff = min(rank, kN - below(1e-12 * lmax));
    sm.r_eff = r_eff;
  }
  __syncthreads();
  const int nvec = sm.r_eff;

  // (3) Inverse iteration on T for each kept eigenvalue (one thread per vector): LU of
  // T - lambda I without pivoting (tiny pivots replaced), two solves from a fixed start,
  // normalized each time.  The vector lives in registers (the loops are unrolled); column
  // 16+k of E holds the reciprocal pivots and column 32+k the multipliers; the result goes
  // to column k.
  if (t < nvec) {
    const int k = t;
    const double lk = sm.lam[k];
    const double tiny = 1e-14 * fmax(fabs(glo), fabs(ghi)) + pivmin;
    double u = sm.dg[0] - lk;
    if (fabs(u) < tiny) u = tiny;
    sm.e.E[0][16 + k] = 1.0 / u;
    for (int i = 1; i < kN; ++i) {
      const double l = sm.od[i - 1] / u;
      u = (sm.dg[i] - lk) - l * sm.od[i - 1];
      if (fabs(u) < tiny) u = tiny;
      sm.e.E[i][16 + k] = 1.0 / u;
      sm.e.E[i][32 + k] = l;
    }
    double* x = &sm.e.E[0][k];  // x[i * (kN + 1)] = element i
    constexpr int RS = kN + 1;
    for (int i = 0; i < kN; ++i) x[i * RS] = 1.0 + static_cast<double>((i * 7 + k * 13) % 11) / 11.0;
    // The recurrences run through registers; elements and factors move in blocks of 8 so
    // their LDS accesses overlap.
    for (int iter = 0; iter < 2; ++iter) {
      double prev = x[0];
      for (int i0 = 0; i0 < kN; i0 += 8) {
        double xb[8], lb[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xb[j] = x[(i0 + j) * RS];
          lb[j] = sm.e.E[i0 + j][32 + k];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          if (i0 + j > 0) xb[j] -= lb[j] * prev;
          prev = xb[j];
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) x[(i0 + j) * RS] = xb[j];
      }
      double next = 0.0, nrm = 0.0;
      for (int i0 = kN - 8; i0 >= 0; i0 -= 8) {
        double xb[8], ub[8], ob[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          xb[j] = x[(i0 + j) * RS];
          ub[j] = sm.e.E[i0 + j][16 + k];
          ob[j] = sm.od[i0 + j];
        }
#pragma unroll
        for (int j = 7; j >= 0; --j) {
          const double v = (i0 + j == kN - 1) ? xb[j] * ub[j] : (xb[j] - ob[j] * next) * ub[j];
          xb[j] = v;
          next = v;
          nrm += v * v;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) x[(i0 + j) * RS] = xb[j];
      }
      const double inv = 1.0 / sqrt(nrm);
      for (int i = 0; i < kN; ++i) x[i * RS] *= inv;
    }
  }
  __syncthreads();
  // Modified Gram-Schmidt over the vectors in eigenvalue order (one wave, lane = element).
  if (t < 64) {
    for (int k = 0; k < nvec; ++k) {
      for (int j = 0; j < k; ++j) {
        const double dot = wave_sum_f64(sm.e.E[t][j] * sm.e.E[t][k]);
        sm.e.E[t][k] -= dot * sm.e.E[t][j];
      }
      const double nrm = wave_sum_f64(sm.e.E[t][k] * sm.e.E[t][k]);
      sm.e.E[t][k] *= 1.0 / sqrt(nrm);
    }
  }
  __syncthreads();
  // (4) Eigenvectors of G: Q y for each tridiagonal eigenvector y (16-lane groups, one vector
  // each, four rows per lane), written over y once every group has read its vector.
  {
    const int k = t >> 4, q = t & 15;
    double x[kN / 16];
#pragma unroll
    for (int c = 0; c < kN / 16; ++c) x[c] = 0.0;
    if (k < nvec) {
      for (int j = 0; j < kN; ++j) {
        const double y = sm.e.E[j][k];
#pragma unroll
        for (int c = 0; c < kN / 16; ++c) x[c] += sm.G[q + 16 * c][j] * y;
      }
    }
    __syncthreads();
    if (k < nvec) {
#pragma unroll
      for (int c = 0; c < kN / 16; ++c) sm.e.E[q + 16 * c][k] = x[c];
    }
  }
  if (t < kN) {
    sm.eval[t] = t < kMaxRank ? sm.lam[t] : 0.0;
    sm.order[t] = t;
  }
  __syncthreads();
  const int r_eff = sm.r_eff;
  // Zr = U_r Lambda_r^1/2 (rows past M are zero);  V_r^T row k = T^T u_k / sqrt(lambda_k),
  // staged in registers while T is still read, then stored over T.
  for (int e = t; e < kN * kMaxRank; e += kFitThreads) {
    const int m = e / kMaxRank, k = e % kMaxRank;
    double z = 0.0;
    if (k < r_eff && m < M) {
      const int col = sm.order[k];
      z = sm.e.E[m][col] * sqrt(sm.eval[col]);
    }
    sm.Zr[m][k] = z;
  }
  constexpr int kVrPer = kMaxRank * 128 / kFitThreads;
  double vr[kVrPer];
#pragma unroll
  for (int i = 0; i < kVrPer; ++i) {
    const int e = t + i * kFitThreads;
    const int k = e / D, d = e % D;
    double v = 0.0;
    if (k < r_eff) {
      const int col = sm.order[k];
      for (int m = 0; m < M; ++m) v += static_cast<double>(sm.t.T[m][d]) * sm.e.E[m][col];
      v /= sqrt(sm.eval[col]);
    }
    vr[i] = v;
  }
  // G <- the factor of Y Y^T + lambda I, from the registers that eliminated it.
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int c = 0; c < 4; ++c) sm.G[i0 + r][j0 + c] = g2[r][c];
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kVrPer; ++i) {
    const int e = t + i * kFitThreads;
    const int k = e / D, d = e % D;
    if (k < kMaxRank) sm.t.Vr[k][d] = vr[i];
  }
  {
    const int wave = t >> 6, lane = t & 63;
    // z = G2^-1 Zr: wave q solves right-hand sides 4q .. 4q+3 with lane = row, in registers,
    // without barriers: L a = Zr (a_k broadcast from lane k), b = D^-1 a, then L^T z = b.
    constexpr int kRhsPerWave = kMaxRank / (kFitThreads / 64);
    const double rdl = 1.0 / sm.G[lane][lane];
    double z[kRhsPerWave];
#pragma unroll
    for (int r = 0; r < kRhsPerWave; ++r) z[r] = sm.Zr[lane][kRhsPerWave * wave + r];
    for (int k = 0; k < kN - 1; ++k) {
      const double g = lane > k ? sm.G[k][lane] * readlane_f64(rdl, k) : 0.0;  // L[lane][k]
#pragma unroll
      for (int r = 0; r < kRhsPerWave; ++r) z[r] -= g * readlane_f64(z[r], k);
    }
#pragma unroll
    for (int r = 0; r < kRhsPerWave; ++r) z[r] *= rdl;
    for (int k = kN - 1; k > 0; --k) {
      const double g = lane < k ? sm.G[k][lane] * rdl : 0.0;  // L[k][lane]
#pragma unroll
      for (int r = 0; r < kRhsPerWave; ++r) z[r] -= g * readlane_f64(z[r], k);
    }
    __syncthreads();  // every wave is done reading Zr
#pragma unroll
    for (int r = 0; r < kRhsPerWave; ++r) sm.Zr[lane][kRhsPerWave * wave + r] = z[r];
  }
  __syncthreads();
  // diag(1/sigma) W V_r = diag(1/sigma) Y^T z (D x r), stored over the eigenvectors.
  for (int e = t; e < D * kMaxRank; e += kFitThreads) {  // columns past r_eff are zero
    const int d = e / kMaxRank, k = e % kMaxRank;
    double v = 0.0;
    if (k < r_eff)
      for (int m = 0; m < M; ++m) v += static_cast<double>(sm.Y[m][d]) * sm.Zr[m][k];
    sm.e.WV[d][k] = v / sm.sig[d];
  }
  __syncthreads();
  // u = mu^T diag(1/sigma) W V_r, so that c = rbar - mu A = rbar - u V_r^T.
  if (t < r_eff) {
    double v = 0.0;
    for (int d = 0; d < D; ++d) v += sm.mu[d] * sm.e.WV[d][t];
    sm.u[t] = v;
  }
  __syncthreads();
  // A = diag(1/sigma) (W V_r) V_r^T: each thread keeps its column of V_r^T in registers (its
  // column index is the same for all its outputs), rows coalesced.
  float* Ah = Aout + static_cast<size_t>(bh) * D * D;
  {
    static_assert(kFitThreads % 128 == 0, "one column per thread for D up to 128");
    const int j = t % D;
    double vcol[kMaxRank];
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) vcol[k] = k < r_eff ? sm.t.Vr[k][j] : 0.0;
    for (int i = t / D; i < D; i += kFitThreads / D) {
      double a = 0.0;
#pragma unroll
      for (int k = 0; k < kMaxRank; ++k) a += sm.e.WV[i][k] * vcol[k];
      Ah[i * D + j] = static_cast<float>(a);
    }
  }
  for (int j = t; j < D; j += kFitThreads) {
    double cj = sm.rbar[j];
    for (int k = 0; k < r_eff; ++k) cj -= sm.u[k] * sm.t.Vr[k][j];
    cout[static_cast<size_t>(bh) * D + j] = static_cast<float>(cj);
  }
}

// ---------------------------------------------------------------- the fit for M > 64 probes
//
// The same fit in its D x D primal form, for more probes than the dual form's 64 (any M up
// to kMaxPrimalM): with Y = Omega^1/2 X and T = Omega^1/2 Rc (rows y_m, t_m),
//   C = T^T T = Rc^T Omega Rc  ->  V_r, its top eigenvectors (the principal residual directions);
//   W V_r = (Y^T Y + lambda I)^-1 Y^T T V_r = (Y^T Y + lambda I)^-1 sum_m y_m (t_m^T V_r);
//   A = diag(1/sigma) (W V_r) V_r^T,  c = rbar - mu A.
// The probe rows stream from global memory in chunks of kChunkRows through LDS (three passes:
// the weighted statistics, C, then Y^T Y and the right-hand sides), so M is not bounded by LDS;
// the two N x N float64 matrices (N = D) take turns in one LDS array, each accumulated in
// registers (a block of (N/16)^2 entries per thread) and stored when complete.  The eigenpairs
// follow the dual kernel's four steps (Householder tridiagonalization, multisection on Sturm
// counts, inverse iteration, back-transformation), with lanes holding N/64 columns each; the
// Householder vector of step k is kept in row k right of the diagonal, the inverse iteration's
// pivots and multipliers (for N = 128) in the lower-left block of the matrix, which the
// reduction no longer reads.
constexpr int kMaxPrimalM = 65536;
constexpr int kChunkRows = 16;

template <int N>
struct PrimalSmem {
  static constexpr int VS = kMaxRank + 1;  // row stride of the vector array
  double G[N][N];  // C, then its reduction; later Y^T Y + lambda I and its factor; finally diag(1/sigma) W V_r
  double V[N][VS];  // eigenvectors (column k = vector k); during the reduction, p = G v partial sums
  double pv[N == 128 ? 1 : N][N == 128 ? 1 : 2 * kMaxRank];  // N = 64: pivots and multipliers
  double mu[N], sig[N], rbar[N];
  double dg[N], od[N], e2[N];
  double lam[kMaxRank], u[kMaxRank];
  double wave_part[kFitThreads / 64];
  double wsum;
  int r_eff;
};

// Reciprocal pivot (j = 0) and multiplier (j = 1) of element i of inverse-iteration vector k.
template <int N>
__device__ __forceinline__ double& inv_slot(PrimalSmem<N>& sm, int k, int i, int j) {
  if constexpr (N == 128)
    return sm.G[64 + (i >> 1)][32 * j + 16 * (i & 1) + k];  // row >= 64 > column: below the diagonal
  else
    return sm.pv[i][j * kMaxRank + k];
}

// Element i of a vector held N/64 per lane (lane i % 64, slot i / 64).
template <int EL>
__device__ __forceinline__ double lane_elem(const double (&x)[EL], int i) {
  if constexpr (EL == 1) {
    return readlane_f64(x[0], i);
  } else {
    return i < 64 ? readlane_f64(x[0], i) : readlane_f64(x[1], i - 64);
  }
}

// out = sum over the rows m of f(m)^T g(m) (N x N, float64) with rows produced chunk by chunk:
// fill(m0, rows) writes the rows m0 .. m0+rows-1 of f to stage_f and of g to stage_g
// ([kChunkRows][N] each, float64, in LDS); each thread accumulates its block in registers.
// diag_add is added on the diagonal.  Ends with every thread's block in acc (not stored).
template <int N, typename Fill>
__device__ __forceinline__ void gram_stream(int M, double* stage_f, double* stage_g, Fill&& fill,
                                            double (&acc)[N / 16][N / 16]) {
  constexpr int B = N / 16;
  const int i0 = (threadIdx.x / 16) * B, j0 = (threadIdx.x % 16) * B;
#pragma unroll
  for (int r = 0; r < B; ++r)
#pragma unroll
    for (int c = 0; c < B; ++c) acc[r][c] = 0.0;
  for (int m0 = 0; m0 < M; m0 += kChunkRows) {
    const int rows = min(kChunkRows, M - m0);
    fill(m0, rows);
    __syncthreads();
    for (int m = 0; m < rows; ++m) {
      double a[B], b[B];
#pragma unroll
      for (int r = 0; r < B; ++r) {
        a[r] = stage_f[m * N + i0 + r];
        b[r] = stage_g[m * N + j0 + r];
      }
#pragma unroll
      for (int r = 0; r < B; ++r)
#pragma unroll
        for (int c = 0; c < B; ++c) acc[r][c] += a[r] * b[c];
    }
    __syncthreads();  // the stage is read before the next chunk overwrites it
  }
}

template <int N>
__global__ __launch_bounds__(kFitThreads) void probe_fit_primal_kernel(const float* __restrict__ Os,
                                                                        const float* __restrict__ Od,
                                                                        const float* __restrict__ weights, int M,
                                                                        int Hq, int Hkv, int nl, float lambda,
                                                                        int rank, float* __restrict__ Aout,
                                                                        float* __restrict__ cout) {
  constexpr int D = N;
  constexpr int EL = N / 64;  // columns per lane
  constexpr int B = N / 16;   // Gram block per thread
  extern __shared__ __align__(16) unsigned char smem_raw[];
  PrimalSmem<N>& sm = *reinterpret_cast<PrimalSmem<N>*>(smem_raw);
  const int bh = blockIdx.x;
  const int t = threadIdx.x;
  const int wave = t >> 6, lane = t & 63;
  const float* Osh = Os + static_cast<size_t>(bh) * M * D;
  const float* Odh = Od + static_cast<size_t>(bh) * M * D;
  if (nl > 1) weights += ((bh / Hq) * static_cast<size_t>(Hkv) + (bh % Hq) / (Hq / Hkv)) * M;  // the head's layout

  double wp = 0.0;
  for (int m = t; m < M; m += kFitThreads) wp += static_cast<double>(weights[m]);
  const double wsum = block_sum(wp, sm.wave_part);
  // Weighted mean and deviation of X0 = O[probe], weighted mean residual (one feature per thread).
  for (int d = t; d < D; d += kFitThreads) {
    double mu = 0.0, rb = 0.0;
    for (int m = 0; m < M; ++m) {
      const double wm = static_cast<double>(weights[m]) / wsum;
      const double x = static_cast<double>(Osh[static_cast<size_t>(m) * D + d]);
      mu += wm * x;
      rb += wm * (static_cast<double>(Odh[static_cast<size_t>(m) * D + d]) - x);
    }
    double var = 0.0;
    for (int m = 0; m < M; ++m) {
      const double wm = static_cast<double>(weights[m]) / wsum;
      const double x = static_cast<double>(Osh[static_cast<size_t>(m) * D + d]) - mu;
      var += wm * x * x;
    }
    double sg = sqrt(var);
    if (sg < 1e-6) sg = 1.0;
    sm.mu[d] = mu;
    sm.sig[d] = sg;
    sm.rbar[d] = rb;
  }
  __syncthreads();
  double* stage = &sm.G[0][0];  // the matrix is accumulated in registers while rows pass here
  // t_m = sqrt(w_m) (R_m - rbar) and y_m = sqrt(w_m) (X0_m - mu) / sigma, float64.
  auto row_t = [&](double* dst, int m0, int rows) {
    for (int e = t; e < rows * D; e += kFitThreads) {
      const int m = e / D, d = e % D;
      const size_t g = static_cast<size_t>(m0 + m) * D + d;
      const double sw = sqrt(static_cast<double>(weights[m0 + m]) / wsum);
      dst[e] = sw * ((static_cast<double>(Odh[g]) - static_cast<double>(Osh[g])) - sm.rbar[d]);
    }
  };
  auto row_y = [&](double* dst, int m0, int rows) {
    for (int e = t; e < rows * D; e += kFitThreads) {
      const int m = e / D, d = e % D;
      const size_t g = static_cast<size_t>(m0 + m) * D + d;
      const double sw = sqrt(static_cast<double>(weights[m0 + m]) / wsum);
      dst[e] = sw * (static_cast<double>(Osh[g]) - sm.mu[d]) / sm.sig[d];
    }
  };
  const int i0 = (t / 16) * B, j0 = (t % 16) * B;
  {
    double acc[B][B];
    auto fill = [&](int m0, int rows) { row_t(stage, m0, rows); };
    gram_stream<N>(M, stage, stage, fill, acc);
#pragma unroll
    for (int r = 0; r < B; ++r)
#pragma unroll
      for (int c = 0; c < B; ++c) sm.G[i0 + r][j0 + c] = acc[r][c];
  }
  __syncthreads();

  // (1) Householder reduction of G to tridiagonal form (see the dual kernel); lane holds
  // columns lane + 64 e.  The vector of step k is stored in row k right of the diagonal.
  double (*pw)[N] = reinterpret_cast<double (*)[N]>(&sm.V[0][0]);  // [4][N] partial sums of G v
  for (int k = 0; k < N - 2; ++k) {
    double x[EL], v[EL];
    double s2p = 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      x[e] = j > k ? sm.G[k][j] : 0.0;
      s2p += x[e] * x[e];
    }
    const double s2 = wave_sum_f64(s2p);
    const double x0 = lane_elem<EL>(x, k + 1);
    double alpha = 0.0, vn2 = 0.0;
    if (s2 > 0.0) {
      alpha = x0 >= 0.0 ? -sqrt(s2) : sqrt(s2);
      vn2 = 2.0 * s2 - 2.0 * x0 * alpha;
    }
    const double vinv = vn2 > 0.0 ? 1.0 / sqrt(vn2) : 0.0;
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      v[e] = j > k ? (x[e] - (j == k + 1 ? alpha : 0.0)) * vinv : 0.0;
    }
    double acc[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) acc[e] = 0.0;
    for (int c = k + 1 + wave; c < N; c += kFitThreads / 64) {
      const double vc = lane_elem<EL>(v, c);
#pragma unroll
      for (int e = 0; e < EL; ++e) acc[e] += sm.G[c][lane + 64 * e] * vc;
    }
#pragma unroll
    for (int e = 0; e < EL; ++e) pw[wave][lane + 64 * e] = acc[e];
    __syncthreads();  // partial products complete; every wave has read row k
    if (wave == 0) {
#pragma unroll
      for (int e = 0; e < EL; ++e)
        if (lane + 64 * e > k) sm.G[k][lane + 64 * e] = v[e];
      if (lane == 0) {
        sm.dg[k] = sm.G[k][k];
        sm.od[k] = alpha;
      }
    }
    if (vn2 > 0.0) {
      double pl[EL], w[EL];
      double vpp = 0.0;
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int j = lane + 64 * e;
        pl[e] = 0.0;
        if (j > k) {
#pragma unroll
          for (int q = 0; q < kFitThreads / 64; ++q) pl[e] += pw[q][j];
        }
        vpp += v[e] * pl[e];
      }
      const double vp = wave_sum_f64(vpp);
#pragma unroll
      for (int e = 0; e < EL; ++e) w[e] = 2.0 * pl[e] - 2.0 * vp * v[e];
      for (int c = k + 1 + wave; c < N; c += kFitThreads / 64) {
        const double vc = lane_elem<EL>(v, c), wc = lane_elem<EL>(w, c);
#pragma unroll
        for (int e = 0; e < EL; ++e)
          if (lane + 64 * e > k) sm.G[c][lane + 64 * e] -= vc * w[e] + wc * v[e];
      }
    }
    __syncthreads();  // the trailing block is updated
  }
  if (t == 0) {
    sm.dg[N - 2] = sm.G[N - 2][N - 2];
    sm.od[N - 2] = sm.G[N - 1][N - 2];
    sm.dg[N - 1] = sm.G[N - 1][N - 1];
    sm.od[N - 1] = 0.0;
  }
  __syncthreads();
  if (t < N) sm.e2[t] = sm.od[t] * sm.od[t];
  __syncthreads();

  // (2) The largest kMaxRank eigenvalues by multisection on Sturm counts.
  double emax2 = 0.0, glo = INFINITY, ghi = -INFINITY;
  for (int i = 0; i < N; ++i) {
    const double r0 = i > 0 ? fabs(sm.od[i - 1]) : 0.0;
    const double r1 = i < N - 1 ? fabs(sm.od[i]) : 0.0;
    glo = fmin(glo, sm.dg[i] - r0 - r1);
    ghi = fmax(ghi, sm.dg[i] + r0 + r1);
    emax2 = fmax(emax2, sm.e2[i]);
  }
  const double span = fmax(ghi - glo, 1e-300);
  const double pivmin = 1e-290 * fmax(1.0, emax2);
  auto below = [&](double xv) {
    int neg = 0;
    double q = 1.0;
    for (int i = 0; i < N; ++i) {
      q = (sm.dg[i] - xv) - (i > 0 ? sm.e2[i - 1] * __builtin_amdgcn_rcp(q) : 0.0);
      if (fabs(q) < pivmin) q = -pivmin;
      neg += q < 0.0 ? 1 : 0;
    }
    return neg;
  };
  {
    const int k = t >> 4, j = t & 15;
    double a = glo - 1e-3 * span, b = ghi + 1e-3 * span;
    for (int it = 0; it < 13; ++it) {
      const double xv = a + (b - a) * static_cast<double>(j + 1) / 17.0;
      const bool ok = (N - below(xv)) <= k;
      const unsigned long long mask = __ballot(ok);
      const unsigned bits = static_cast<unsigned>(mask >> (16 * ((threadIdx.x & 63) >> 4))) & 0xffffu;
      const int f = bits ? __builtin_ctz(bits) : 16;
      const double na = f == 0 ? a : a + (b - a) * static_cast<double>(f) / 17.0;
      const double nb = f == 16 ? b : a + (b - a) * static_cast<double>(f + 1) / 17.0;
      a = na;
      b = nb;
    }
    if (j == 0) sm.lam[k] = 0.5 * (a + b);
  }
  __syncthreads();
  if (t == 0) {
    const double lmax = sm.lam[0];
    int r_eff = 0;
    if (lmax > 0.0) r_eff = min(rank, N - below(1e-12 * lmax));
    sm.r_eff = r_eff;
  }
  __syncthreads();
  const int r_eff = sm.r_eff;

  // (3) Inverse iteration (one thread per vector; vector k in column k of V).
  if (t < r_eff) {
    const int k = t;
    const double lk = sm.lam[k];
    const double tiny = 1e-14 * fmax(fabs(glo), fabs(ghi)) + pivmin;
    double uu = sm.dg[0] - lk;
    if (fabs(uu) < tiny) uu = tiny;
    inv_slot<N>(sm, k, 0, 0) = 1.0 / uu;
    for (int i = 1; i < N; ++i) {
      const double l = sm.od[i - 1] / uu;
      uu = (sm.dg[i] - lk) - l * sm.od[i - 1];
      if (fabs(uu) < tiny) uu = tiny;
      inv_slot<N>(sm, k, i, 0) = 1.0 / uu;
      inv_slot<N>(sm, k, i, 1) = l;
    }
    for (int i = 0; i < N; ++i) sm.V[i][k] = 1.0 + static_cast<double>((i * 7 + k * 13) % 11) / 11.0;
    for (int iter = 0; iter < 3; ++iter) {
      double prev = sm.V[0][k];
      for (int i = 1; i < N; ++i) {
        prev = sm.V[i][k] - inv_slot<N>(sm, k, i, 1) * prev;
        sm.V[i][k] = prev;
      }
      double next = 0.0, nrm = 0.0;
      for (int i = N - 1; i >= 0; --i) {
        const double vi = (i == N - 1 ? sm.V[i][k] : sm.V[i][k] - sm.od[i] * next) * inv_slot<N>(sm, k, i, 0);
        sm.V[i][k] = vi;
        next = vi;
        nrm += vi * vi;
      }
      const double inv = 1.0 / sqrt(nrm);
      for (int i = 0; i < N; ++i) sm.V[i][k] *= inv;
    }
  }
  __syncthreads();
  // Modified Gram-Schmidt in eigenvalue order (one wave, N/64 elements per lane).
  if (t < 64) {
    for (int k = 0; k < r_eff; ++k) {
      for (int j = 0; j < k; ++j) {
        double dp = 0.0;
#pragma unroll
        for (int e = 0; e < EL; ++e) dp += sm.V[t + 64 * e][j] * sm.V[t + 64 * e][k];
        const double dot = wave_sum_f64(dp);
#pragma unroll
        for (int e = 0; e < EL; ++e) sm.V[t + 64 * e][k] -= dot * sm.V[t + 64 * e][j];
      }
      double np = 0.0;
#pragma unroll
      for (int e = 0; e < EL; ++e) np += sm.V[t + 64 * e][k] * sm.V[t + 64 * e][k];
      const double inv = 1.0 / sqrt(wave_sum_f64(np));
#pragma unroll
      for (int e = 0; e < EL; ++e) sm.V[t + 64 * e][k] *= inv;
    }
  }
  __syncthreads();
  // (4) Back-transformation, y <- H_s y for s = N-3 .. 0 (16-lane groups, one vector each);
  // the reflector of step s is row s of G right of the diagonal.
  {
    const int k = t >> 4, q = t & 15;
    if (k < r_eff) {
      for (int s = N - 3; s >= 0; --s) {
        double dot = 0.0;
#pragma unroll
        for (int c = 0; c < N / 16; ++c) {
          const int i = q + 16 * c;
          if (i > s) dot += sm.G[s][i] * sm.V[i][k];
        }
        dot = row16_sum(dot);
#pragma unroll
        for (int c = 0; c < N / 16; ++c) {
          const int i = q + 16 * c;
          if (i > s) sm.V[i][k] -= 2.0 * dot * sm.G[s][i];
        }
      }
    }
  }
  __syncthreads();

  // Y^T Y + lambda I and the right-hand sides Z = sum_m y_m (t_m^T V_r), one pass over the rows:
  // each chunk stages y and t rows and the products z_m = t_m^T V_r.  Thread (wave q, lane)
  // keeps Z[lane + 64 e][4 q + r], the layout of the solve below.
  constexpr int kRhs = kMaxRank / (kFitThreads / 64);
  double z[EL][kRhs];
#pragma unroll
  for (int e = 0; e < EL; ++e)
#pragma unroll
    for (int r = 0; r < kRhs; ++r) z[e][r] = 0.0;
  {
    double* sy = stage;
    double* st = stage + kChunkRows * N;
    double* sz = stage + 2 * kChunkRows * N;  // [kChunkRows][kMaxRank]
    double acc[B][B];
    auto fill = [&](int m0, int rows) {
      row_y(sy, m0, rows);
      row_t(st, m0, rows);
      __syncthreads();
      {  // z_m[k] for the chunk's rows: thread (m, k)
        const int m = t / kMaxRank, k = t % kMaxRank;
        if (m < rows) {
          double s = 0.0;
          if (k < r_eff)
            for (int d = 0; d < D; ++d) s += st[m * N + d] * sm.V[d][k];
          sz[m * kMaxRank + k] = s;
        }
      }
      __syncthreads();
      for (int m = 0; m < rows; ++m)
#pragma unroll
        for (int e = 0; e < EL; ++e) {
          const double yv = sy[m * N + lane + 64 * e];
#pragma unroll
          for (int r = 0; r < kRhs; ++r) z[e][r] += yv * sz[m * kMaxRank + kRhs * wave + r];
        }
    };
    static_assert(kChunkRows * kMaxRank == kFitThreads, "one z product per thread");
    gram_stream<N>(M, sy, sy, fill, acc);
#pragma unroll
    for (int r = 0; r < B; ++r)
#pragma unroll
      for (int c = 0; c < B; ++c)
        sm.G[i0 + r][j0 + c] = acc[r][c] + (i0 + r == j0 + c ? static_cast<double>(lambda) : 0.0);
  }
  __syncthreads();
  // L D L^T of G (right-looking, both triangles; see the dual kernel), then the solve.
  for (int k = 0; k < N - 1; ++k) {
#pragma unroll
    for (int e = 0; e < EL; ++e) {
      const int j = lane + 64 * e;
      if (j > k) {
        const double rk = sm.G[k][j] / sm.G[k][k];
        for (int i = k + 1 + wave; i < N; i += kFitThreads / 64) sm.G[i][j] -= sm.G[i][k] * rk;
      }
    }
    __syncthreads();
  }
  {
    double rdl[EL];
#pragma unroll
    for (int e = 0; e < EL; ++e) rdl[e] = 1.0 / sm.G[lane + 64 * e][lane + 64 * e];
    for (int k = 0; k < N - 1; ++k) {
      const double rk = lane_elem<EL>(rdl, k);
      double zk[kRhs];
#pragma unroll
      for (int r = 0; r < kRhs; ++r) {
        double col[EL];
#pragma unroll
        for (int e = 0; e < EL; ++e) col[e] = z[e][r];
        zk[r] = lane_elem<EL>(col, k);
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int j = lane + 64 * e;
        const double g = j > k ? sm.G[k][j] * rk : 0.0;  // L[j][k]
#pragma unroll
        for (int r = 0; r < kRhs; ++r) z[e][r] -= g * zk[r];
      }
    }
#pragma unroll
    for (int e = 0; e < EL; ++e)
#pragma unroll
      for (int r = 0; r < kRhs; ++r) z[e][r] *= rdl[e];
    for (int k = N - 1; k > 0; --k) {
      double zk[kRhs];
#pragma unroll
      for (int r = 0; r < kRhs; ++r) {
        double col[EL];
#pragma unroll
        for (int e = 0; e < EL; ++e) col[e] = z[e][r];
        zk[r] = lane_elem<EL>(col, k);
      }
#pragma unroll
      for (int e = 0; e < EL; ++e) {
        const int j = lane + 64 * e;
        const double g = j < k ? sm.G[k][j] * rdl[e] : 0.0;  // L[k][j]
#pragma unroll
        for (int r = 0; r < kRhs; ++r) z[e][r] -= g * zk[r];
      }
    }
  }
  __syncthreads();  // the factor is read; its storage takes diag(1/sigma) W V_r
  double (*WV)[kMaxRank + 1] = reinterpret_cast<double (*)[kMaxRank + 1]>(&sm.G[0][0]);
#pragma unroll
  for (int e = 0; e < EL; ++e)
#pragma unroll
    for (int r = 0; r < kRhs; ++r) {
      const int d = lane + 64 * e, k = kRhs * wave + r;
      WV[d][k] = k < r_eff ? z[e][r] / sm.sig[d] : 0.0;
    }
  __syncthreads();
  if (t < r_eff) {
    double s = 0.0;
    for (int d = 0; d < D; ++d) s += sm.mu[d] * WV[d][t];
    sm.u[t] = s;
  }
  __syncthreads();
  float* Ah = Aout + static_cast<size_t>(bh) * D * D;
  {
    const int j = t % D;
    double vcol[kMaxRank];
#pragma unroll
    for (int k = 0; k < kMaxRank; ++k) vcol[k] = k < r_eff ? sm.V[j][k] : 0.0;
    for (int i = t / D; i < D; i += kFitThreads / D) {
      double a = 0.0;
#pragma unroll
      for (int k = 0; k < kMaxRank; ++k) a += WV[i][k] * vcol[k];
      Ah[i * D + j] = static_cast<float>(a);
    }
  }
  for (int j = t; j < D; j += kFitThreads) {
    double cj = sm.rbar[j];
    for (int k = 0; k < r_eff; ++k) cj -= sm.u[k] * sm.V[j][k];
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

// O_out <- O + O A + c from float32 rows O (the uncorrected attention output), rounded once to
// bfloat16.  A workgroup stages A^T once (high and low bfloat16 parts, transposed through 4 x 4
// register blocks); then each wave takes blocks of 32 rows on its own: (O A)^T = A^T O^T on MFMA
// with O split into high and low parts as well (hi*hi + hi*lo + lo*hi, float32 accuracy).  The
// contraction runs over each 16-feature group in the order 0-3, 8-11, 4-7, 12-15 (A^T rows are
// stored that way), so the O entries a lane loads for the products are exactly those of the
// output features it holds afterwards: the row is read once, into registers.  Partner lanes
// (same row, other half) swap halves of their results so that each stores 16-byte chunks.
constexpr int kCorrRows = 1024;
__device__ __forceinline__ int corr_pos(int f) { return (f & ~12) | ((f & 4) << 1) | ((f & 8) >> 1); }
template <int D>
__global__ __launch_bounds__(256, 1) void correct_bf16_kernel(const float* __restrict__ Oin,
                                                               const float* __restrict__ A,
                                                               const float* __restrict__ cvec, int S,
                                                               bf16_t* __restrict__ Oout) {
  constexpr int ROWA = D + 8;  // A^T staging row (elements; 16-byte aligned rows)
  extern __shared__ __align__(16) unsigned char smem_corr[];
  bf16_t* AtH = reinterpret_cast<bf16_t*>(smem_corr);  // A^T rows: At[j][corr_pos(i)] = A[i][j]
  bf16_t* AtL = AtH + D * ROWA;
  float* cs = reinterpret_cast<float*>(AtL + D * ROWA);
  const int bh = blockIdx.y;
  const float* Ah = A + static_cast<size_t>(bh) * D * D;
  const float* Oh = Oin + static_cast<size_t>(bh) * S * D;
  bf16_t* Ph = Oout + static_cast<size_t>(bh) * S * D;
  constexpr int kBlk = (D / 4) * (D / 4);
  for (int blk = threadIdx.x; blk < kBlk; blk += 256) {
    const int i0 = (blk / (D / 4)) * 4, j0 = (blk % (D / 4)) * 4;
    f32x4 rowv[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) rowv[k] = *reinterpret_cast<const f32x4*>(Ah + (i0 + k) * D + j0);
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      float hi[4], lo[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const __bf16 hb = static_cast<__bf16>(rowv[k][jj]);
        hi[k] = static_cast<float>(hb);
        lo[k] = rowv[k][jj] - hi[k];
      }
      *reinterpret_cast<uint2*>(AtH + (j0 + jj) * ROWA + corr_pos(i0)) =
          make_uint2(pack_bf16x2(hi[0], hi[1]), pack_bf16x2(hi[2], hi[3]));
      *reinterpret_cast<uint2*>(AtL + (j0 + jj) * ROWA + corr_pos(i0)) =
          make_uint2(pack_bf16x2(lo[0], lo[1]), pack_bf16x2(lo[2], lo[3]));
    }
  }
  for (int d = threadIdx.x; d < D; d += 256) cs[d] = cvec[static_cast<size_t>(bh) * D + d];
  __syncthreads();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, r = lane & 31, h = lane >> 5;
  const int rows_end = min(S, static_cast<int>(blockIdx.x + 1) * kCorrRows);
  for (int row0 = blockIdx.x * kCorrRows + wave * 32; row0 < rows_end; row0 += 4 * 32) {
    const int my = row0 + r;
    const float* orow = Oh + static_cast<size_t>(my < S ? my : S - 1) * D;
    // o[4 jt + q] = features 32 jt + 8 q + 4 h + (0..3) of this lane's row.
    f32x4 o[D / 8];
#pragma unroll
    for (int i = 0; i < D / 8; ++i) o[i] = *reinterpret_cast<const f32x4*>(orow + 8 * i + 4 * h);
    f32x16 acc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) acc[i] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
      Frag<bf16_t> oh, ol;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float x = o[2 * kk + e / 4][e % 4];
        const __bf16 hi = static_cast<__bf16>(x);
        oh.v[e] = hi;
        ol.v[e] = static_cast<__bf16>(x - static_cast<float>(hi));
      }
#pragma unroll
      for (int jt = 0; jt < D / 32; ++jt) {
        Frag<bf16_t> ah, al;
        load_frag(ah, AtH + (jt * 32 + r) * ROWA + kk * 16 + 8 * h);
        load_frag(al, AtL + (jt * 32 + r) * ROWA + kk * 16 + 8 * h);
        acc[jt] = mma(ah, oh, acc[jt]);
        acc[jt] = mma(ah, ol, acc[jt]);
        acc[jt] = mma(al, oh, acc[jt]);
      }
    }
    // Entry 4q+e of acc[jt] is feature 32 jt + 8 q + 4 h + e, as is o[4 jt + q][e].  Chunk
    // pair (2c, 2c+1) of 8 features: the lower half (h = 0) stores chunk 2c, the upper half
    // chunk 2c+1; each gives its partner the 4 values the partner lacks.
    bf16_t* prow = Ph + static_cast<size_t>(my < S ? my : 0) * D;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint32_t w[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int jt = c / 2, q = 2 * (c % 2) + u;
        const int f = jt * 32 + 8 * q + 4 * h;
        const f32x4 ov = o[4 * jt + q];
        w[u][0] = pack_bf16x2(ov[0] + acc[jt][4 * q] + cs[f], ov[1] + acc[jt][4 * q + 1] + cs[f + 1]);
        w[u][1] = pack_bf16x2(ov[2] + acc[jt][4 * q + 2] + cs[f + 2], ov[3] + acc[jt][4 * q + 3] + cs[f + 3]);
      }
      const uint32_t got0 = __float_as_uint(swap_halves(__uint_as_float(h ? w[0][0] : w[1][0])));
      const uint32_t got1 = __float_as_uint(swap_halves(__uint_as_float(h ? w[0][1] : w[1][1])));
      const uint4 v = h ? make_uint4(got0, got1, w[1][0], w[1][1]) : make_uint4(w[0][0], w[0][1], got0, got1);
      if (my < S) *reinterpret_cast<uint4*>(prow + 16 * c + 8 * h) = v;
    }
  }
}

// Float32 rows: plain float32 arithmetic (Oout may be Oin).
__global__ __launch_bounds__(256) void correct_f32_kernel(const float* __restrict__ Oin, const float* __restrict__ A,
                                                          const float* __restrict__ cvec, int S, int D,
                                                          float* Oout) {
  extern __shared__ float rows_c[];  // 8 rows x D
  const int bh = blockIdx.y;
  const int row0 = blockIdx.x * 8;
  const float* Ih = Oin + static_cast<size_t>(bh) * S * D;
  float* Oh = Oout + static_cast<size_t>(bh) * S * D;
  const float* Ah = A + static_cast<size_t>(bh) * D * D;
  for (int e = threadIdx.x; e < 8 * D; e += 256) {
    const int rr = e / D, d = e % D;
    rows_c[e] = row0 + rr < S ? Ih[static_cast<size_t>(row0 + rr) * D + d] : 0.0f;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < 8 * D; e += 256) {
    const int rr = e / D, j = e % D;
    if (row0 + rr >= S) continue;
    float v = rows_c[e] + cvec[static_cast<size_t>(bh) * D + j];
    for (int i = 0; i < D; ++i) v += rows_c[rr * D + i] * Ah[static_cast<size_t>(i) * D + j];
    Oh[static_cast<size_t>(row0 + rr) * D + j] = v;
  }
}

// out[bh][m][:] = X[bh][idx[m]][:] (float32 rows).
__global__ __launch_bounds__(128) void gather_rows_kernel(const float* __restrict__ X, int S, int D,
                                                          const int32_t* __restrict__ idx, int M,
                                                          float* __restrict__ out) {
  const int m = blockIdx.x, bh = blockIdx.y;
  const int i = idx[m];
  if (i < 0 || i >= S) return;
  for (int d = threadIdx.x; d < D; d += blockDim.x)
    out[(static_cast<size_t>(bh) * M + m) * D + d] = X[(static_cast<size_t>(bh) * S + i) * D + d];
}

}  // namespace
}  // namespace bsa

using namespace bsa;

extern "C" bsa_status bsa_probe_fit(int B, int Hq, int Hkv, int D, const float* O_sparse_probe,
                                    const float* O_dense_probe, const float* weights, int M, int n_layouts,
                                    float lambda, int rank, float* A, float* c, hipStream_t stream) {
  if (B < 1 || Hq < 1 || Hkv < 1 || !O_sparse_probe || !O_dense_probe || !weights || !A || !c) return BSA_E_ARG;
  if (Hq % Hkv != 0) return BSA_E_SHAPE;
  if (n_layouts != 1 && static_cast<long long>(n_layouts) != static_cast<long long>(B) * Hkv) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (M < 2) return BSA_E_ARG;
  if (M > kMaxPrimalM) return BSA_E_UNSUPPORTED;
  if (!(lambda > 0.0f) || !(lambda < INFINITY)) return BSA_E_ARG;
  if (rank < 1 || rank > D) return BSA_E_ARG;
  if (rank > kMaxRank) return BSA_E_UNSUPPORTED;
  if (M > kMaxM) {  // the primal form
    auto launch = [&](auto kern, int smem) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(kern), hipFuncAttributeMaxDynamicSharedMemorySize, smem);
      hipLaunchKernelGGL(kern, dim3(B * Hq), dim3(kFitThreads), smem, stream, O_sparse_probe, O_dense_probe, weights,
                         M, Hq, Hkv, n_layouts, lambda, rank, A, c);
    };
    if (D == 128)
      launch(probe_fit_primal_kernel<128>, static_cast<int>(sizeof(PrimalSmem<128>)));
    else
      launch(probe_fit_primal_kernel<64>, static_cast<int>(sizeof(PrimalSmem<64>)));
    return launch_status();
  }
  const int smem = static_cast<int>(sizeof(FitSmem));
  hipFuncSetAttribute(reinterpret_cast<const void*>(probe_fit_kernel), hipFuncAttributeMaxDynamicSharedMemorySize, smem);
  hipLaunchKernelGGL(probe_fit_kernel, dim3(B * Hq), dim3(kFitThreads), smem, stream, O_sparse_probe, O_dense_probe,
                     weights, D, M, Hq, Hkv, n_layouts, lambda, rank, A, c);
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

extern "C" bsa_status bsa_correct(int B, int Hq, int S, int D, int out_dtype, const float* O_in, const float* A,
                                  const float* c, void* O_out, hipStream_t stream) {
  if (!valid_dtype(out_dtype)) return BSA_E_DTYPE;
  if (B < 1 || Hq < 1 || S < 1 || !O_in || !O_out || !A || !c) return BSA_E_ARG;
  if (D != 64 && D != 128) return BSA_E_UNSUPPORTED;
  if (static_cast<long long>(B) * Hq > 65535) return BSA_E_UNSUPPORTED;
  if (out_dtype == BSA_BF16) {
    const dim3 grid((S + kCorrRows - 1) / kCorrRows, B * Hq);
    const int smem = 2 * D * (D + 8) * 2 + D * 4;
    if (D == 128) {
      hipFuncSetAttribute(reinterpret_cast<const void*>(correct_bf16_kernel<128>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, smem);
      hipLaunchKernelGGL((correct_bf16_kernel<128>), grid, dim3(256), smem, stream, O_in, A, c, S,
                         static_cast<bf16_t*>(O_out));
    } else {
      hipFuncSetAttribute(reinterpret_cast<const void*>(correct_bf16_kernel<64>),
                          hipFuncAttributeMaxDynamicSharedMemorySize, smem);
      hipLaunchKernelGGL((correct_bf16_kernel<64>), grid, dim3(256), smem, stream, O_in, A, c, S,
                         static_cast<bf16_t*>(O_out));
    }
  } else {
    const dim3 grid((S + 7) / 8, B * Hq);
    hipLaunchKernelGGL(correct_f32_kernel, grid, dim3(256), 8 * D * sizeof(float), stream, O_in, A, c, S, D,
                       static_cast<float*>(O_out));
  }
  return launch_status();
}

extern "C" bsa_status bsa_gather_rows(int BH, int S, int D, const float* X, const int32_t* idx, int M, float* out,
                                      hipStream_t stream) {
  if (BH < 1 || S < 1 || D < 1 || M < 1 || !X || !idx || !out) return BSA_E_ARG;
  if (BH > 65535) return BSA_E_UNSUPPORTED;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(M, BH), dim3(128), 0, stream, X, S, D, idx, M, out);
  return launch_status();
}
