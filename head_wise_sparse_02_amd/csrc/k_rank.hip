// Effective rank of each query head's query-key kernel, from frozen weights.
//
// [AoH] "Autonomy-of-Heads: Data-Free Sparse Attention from Frozen Query-Key
// Geometry", Methodology §1-§3: the kernel of query head g (KV head h) is
// M_g = W_K^h^T W_Q^g (d_model x d_model); its singular values, normalised to
// sum 1, give eff_rank = exp(-sum s log s); the non-zero singular values come
// from the d_head x d_head matrix C = (W_Q W_Q^T)(W_K W_K^T) (eig C = sigma^2).
//
// Route here, fp64 throughout:
//   gram_kernel   A_g = W_Q^g W_Q^g^T for each query head, B_h = W_K^h W_K^h^T
//                 for each KV head (16 x 16 output tiles, 64-column chunks
//                 of the weight rows staged in LDS);
//   rank_kernel   one workgroup per query head: Cholesky A_g + delta I = L L^T
//                 in LDS (delta = 1e-15 tr(A)/d keeps it defined when W_Q is
//                 rank deficient and moves sigma^2 by a relative 1e-15);
//                 S = L^T B_h L, which is symmetric with eig S = eig(A B) =
//                 sigma(M_g)^2; cyclic Jacobi on S in LDS with the round-robin
//                 ordering (64 disjoint rotations per step, rows then columns);
//                 sigma = sqrt(max(lambda, 0)) and the entropy of sigma / sum.
#include "hws_device.h"

namespace hws {

namespace {

constexpr int DH = D;                 // head dim, 128
constexpr int RT = 256;               // threads of both kernels
constexpr int MAX_SWEEPS = 24;

__global__ __launch_bounds__(RT) void gram_kernel(const float* w, int d_model, double* out) {
  const int mat = blockIdx.z, ti = blockIdx.y * 16, tj = blockIdx.x * 16;
  const float* W = w + (size_t)mat * DH * d_model;
  __shared__ double ra[16][65], rb[16][65];
  const int tid = threadIdx.x, i = tid / 16, j = tid % 16;
  double acc = 0.0;
  for (int k0 = 0; k0 < d_model; k0 += 64) {
    for (int e = tid; e < 16 * 64; e += RT) {
      const int r = e / 64, cc = e % 64, k = k0 + cc;
      ra[r][cc] = k < d_model ? (double)W[(size_t)(ti + r) * d_model + k] : 0.0;
      rb[r][cc] = k < d_model ? (double)W[(size_t)(tj + r) * d_model + k] : 0.0;
    }
    __syncthreads();
#pragma unroll 8
    for (int cc = 0; cc < 64; ++cc) acc = fma(ra[i][cc], rb[j][cc], acc);
    __syncthreads();
  }
  out[(size_t)mat * DH * DH + (size_t)(ti + i) * DH + tj + j] = acc;
}

// Sum of one double per thread over the workgroup (every thread gets it).
__device__ double block_sum(double v, double* red) {
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = v;
  __syncthreads();
  double t = 0.0;
  for (int w = 0; w < RT / 64; ++w) t += red[w];
  return t;
}

// Pair k of round r of the round-robin schedule over 128 indices: index 0
// stays, 1..127 rotate; every pair meets once in 127 rounds.
__device__ __forceinline__ void rr_pair(int r, int k, int& p, int& q) {
  if (k == 0) {
    p = 0;
    q = 1 + r;
  } else {
    p = 1 + (r + k) % (DH - 1);
    q = 1 + (r - k + (DH - 1)) % (DH - 1);
  }
}

__global__ __launch_bounds__(RT) void rank_kernel(const double* A, const double* B, int G, double* Lg,
                                                  double* Sg, float* eff_rank) {
  const int g = blockIdx.x, tid = threadIdx.x;
  const double* Ag = A + (size_t)g * DH * DH;
  const double* Bh = B + (size_t)(g / G) * DH * DH;
  double* L = Lg + (size_t)g * DH * DH;
  double* Sglob = Sg + (size_t)g * DH * DH;
  __shared__ double S[DH][DH + 1];
  __shared__ double cs[DH / 2][2];
  __shared__ int pq[DH / 2][2];
  __shared__ double red[RT / 64];
  __shared__ int stop;

  // ---- A_g + delta I, then Cholesky in place (lower triangle) ----
  for (int e = tid; e < DH * DH; e += RT) S[e / DH][e % DH] = Ag[e];
  __syncthreads();
  const double tr = block_sum(tid < DH ? S[tid][tid] : 0.0, red);
  if (tid < DH) S[tid][tid] += 1e-15 * tr / DH + 1e-300;
  __syncthreads();
  for (int k = 0; k < DH; ++k) {
    if (tid == 0) S[k][k] = sqrt(fmax(S[k][k], 1e-300));
    __syncthreads();
    for (int i = k + 1 + tid; i < DH; i += RT) S[i][k] /= S[k][k];
    __syncthreads();
    const int m = DH - k - 1;
    for (int e = tid; e < m * m; e += RT) {
      const int i = k + 1 + e / m, j = k + 1 + e % m;
      if (j <= i) S[i][j] -= S[i][k] * S[j][k];
    }
    __syncthreads();
  }
  for (int e = tid; e < DH * DH; e += RT) {
    const int i = e / DH, j = e % DH;
    L[e] = j <= i ? S[i][j] : 0.0;
  }
  __threadfence_block();
  __syncthreads();

  // ---- T = B L (in LDS), then S = L^T T (to global, then back to LDS) ----
  for (int e = tid; e < DH * DH; e += RT) {
    const int i = e / DH, j = e % DH;
    double acc = 0.0;
    for (int m = j; m < DH; ++m) acc = fma(Bh[(size_t)i * DH + m], L[(size_t)m * DH + j], acc);
    S[i][j] = acc;
  }
  __syncthreads();
  for (int e = tid; e < DH * DH; e += RT) {
    const int i = e / DH, j = e % DH;
    double acc = 0.0;
    for (int m = i; m < DH; ++m) acc = fma(L[(size_t)m * DH + i], S[m][j], acc);
    Sglob[e] = acc;
  }
  __threadfence_block();
  __syncthreads();
  for (int e = tid; e < DH * DH; e += RT) {
    const int i = e / DH, j = e % DH;
    S[i][j] = 0.5 * (Sglob[(size_t)i * DH + j] + Sglob[(size_t)j * DH + i]);   // exact symmetry
  }
  __syncthreads();

  // ---- cyclic Jacobi: 127 rounds of 64 disjoint rotations per sweep ----
  for (int sweep = 0; sweep < MAX_SWEEPS; ++sweep) {
    for (int r = 0; r < DH - 1; ++r) {
      if (tid < DH / 2) {
        int p, q;
        rr_pair(r, tid, p, q);
        const double apq = S[p][q];
        double c = 1.0, s = 0.0;
        if (fabs(apq) > 1e-300) {
          const double tau = (S[q][q] - S[p][p]) / (2.0 * apq);
          const double t = (tau >= 0.0 ? 1.0 : -1.0) / (fabs(tau) + sqrt(1.0 + tau * tau));
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        cs[tid][0] = c;
        cs[tid][1] = s;
        pq[tid][0] = p;
        pq[tid][1] = q;
      }
      __syncthreads();
      for (int e = tid; e < (DH / 2) * DH; e += RT) {       // rows p, q
        const int k = e / DH, j = e % DH;
        const int p = pq[k][0], q = pq[k][1];
        const double c = cs[k][0], s = cs[k][1];
        const double ap = S[p][j], aq = S[q][j];
        S[p][j] = c * ap - s * aq;
        S[q][j] = s * ap + c * aq;
      }
      __syncthreads();
      for (int e = tid; e < (DH / 2) * DH; e += RT) {       // columns p, q
        const int k = e / DH, i = e % DH;
        const int p = pq[k][0], q = pq[k][1];
        const double c = cs[k][0], s = cs[k][1];
        const double ap = S[i][p], aq = S[i][q];
        S[i][p] = c * ap - s * aq;
        S[i][q] = s * ap + c * aq;
      }
      __syncthreads();
    }
    double off = 0.0, dia = 0.0;
    for (int e = tid; e < DH * DH; e += RT) {
      const int i = e / DH, j = e % DH;
      const double v = S[i][j] * S[i][j];
      if (i == j) dia += v;
      else off += v;
    }
    off = block_sum(off, red);
    dia = block_sum(dia, red);
    if (tid == 0) stop = off <= 1e-30 * dia ? 1 : 0;
    __syncthreads();
    if (stop) break;
  }

  // ---- singular values of M_g and the entropy of their distribution ----
  const double sv = tid < DH ? sqrt(fmax(S[tid][tid], 0.0)) : 0.0;
  const double tot = block_sum(sv, red);
  const double sh = tot > 0.0 ? sv / tot : 0.0;
  const double ent = block_sum(sh > 0.0 ? -sh * log(sh) : 0.0, red);
  if (tid == 0) eff_rank[g] = (float)exp(ent);
}

}  // namespace

size_t rank_workspace_bytes(int hq, int hkv) {
  return (size_t)(3 * hq + hkv) * DH * DH * sizeof(double);
}

hipError_t launch_effective_rank(int hq, int hkv, int d_model, const float* w_q, const float* w_k,
                                 float* eff_rank, void* workspace, hipStream_t s) {
  double* A = static_cast<double*>(workspace);
  double* B = A + (size_t)hq * DH * DH;
  double* L = B + (size_t)hkv * DH * DH;
  double* S = L + (size_t)hq * DH * DH;
  hipLaunchKernelGGL(gram_kernel, dim3(DH / 16, DH / 16, hq), dim3(RT), 0, s, w_q, d_model, A);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gram_kernel, dim3(DH / 16, DH / 16, hkv), dim3(RT), 0, s, w_k, d_model, B);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(rank_kernel, dim3(hq), dim3(RT), 0, s, A, B, hq / hkv, L, S, eff_rank);
  return hipGetLastError();
}

}  // namespace hws
