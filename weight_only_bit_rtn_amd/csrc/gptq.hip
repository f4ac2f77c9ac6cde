// gptq.hip -- error-feedback (GPTQ / OPTQ) quantization in fp64 on gfx950.
//
// Method: the parameters of each output row are quantized one input channel
// after another, and the inverse Hessian built from the layer's input
// activations is used to adjust the parameters not yet quantized, which
// compensates the quantization error (BladeLLM model quantization,
// "Quantization algorithms", GPTQ).  The Hessian is accumulated from
// calibration inputs and the grid is the per-row (or per-group) asymmetric
// min-max grid (OPTQ reproducibility card, "Experiment Setup" row).
//
// The inverse-Hessian update of column i,
//     err_i = (t_i - deq_i) / Hinv_ii,   t_j -= err_i * Hinv_ij  (j > i),
// followed by the removal of column i from Hinv, is carried out here without
// any inverse: with H = R R^T and R upper triangular, the weight that column
// j sees after all earlier updates is
//     t_j = w_j + (sum_{i<j} d_i R_ij) / R_jj,   d_i = w_i - deq_i,
// (w the original weights), because W - deq(Q) = E U with U = R^-1 the upper
// Cholesky factor of H^-1 and E = (W - deq(Q)) R.  R is the Cholesky factor of
// H with the index order reversed: reverse(H) = L L^T gives R_ij =
// L[K-1-i][K-1-j].
//
// Steps, all in fp64 on the caller's stream, in the caller's workspace:
//  1. hessian_kernel: reverse(H) = (2/n) X^T X with both indices reversed;
//  2. damp_kernel: damp * mean(diag) added to the diagonal; status cleared;
//  3. right-looking blocked Cholesky of reverse(H) in place, 64 columns per
//     panel: diagonal block in one workgroup (chol_diag_kernel), the panel
//     below by row-wise substitution (chol_panel_kernel), the trailing lower
//     triangle by 64x64 tiles (chol_update_kernel);
//  4. gptq_rows_kernel: 64 weight rows per workgroup (rows are independent),
//     K in blocks of 64 columns: the contribution of all earlier residuals
//     d_i to the block (a 64 x j0 x 64 product, four waves) and then the
//     block's columns one after another (one lane per row);
//  5. the codes are packed by the packing kernel.
// deq_i = (q_i - z) * s is the exact value code q_i stands for.  The grid
// (scales, zero points) is the RTN grid of the original weights
// (min-max, or signed symmetric with codes from 1), written by the RTN
// quantizer before step 4.
#include "common.h"
#include "kernels.h"

namespace lowbit {

namespace {

constexpr int kNB = 64;    // Cholesky panel width and GPTQ column block
constexpr int kRows = 64;  // weight rows per GPTQ workgroup
constexpr int kChunk = 64;   // earlier columns staged per LDS round in step 4
constexpr int kHChunk = 32;  // calibration rows staged per LDS round in step 1

__device__ __forceinline__ double h_bits_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// Step 1.  Workgroup (bi, bj) computes the 64 x 64 tile of H at rows
// 64 bi.., columns 64 bj.. and stores it with both indices reversed.
// Thread (ty, tx) = (tid / 16, tid % 16) owns rows 4 ty.., columns 4 tx...
__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                      int K, double* __restrict__ Hrev) {
  __shared__ double xi[kHChunk][64];
  __shared__ double xj[kHChunk][64];
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  double acc[4][4] = {};
  for (int64_t t0 = 0; t0 < n; t0 += kHChunk) {
    for (int e = tid; e < kHChunk * 64; e += 256) {
      const int tt = e >> 6, c = e & 63;
      const int64_t t = t0 + tt;
      xi[tt][c] = (t < n && i0 + c < K) ? h_bits_to_f64(x[t * K + i0 + c]) : 0.0;
      xj[tt][c] = (t < n && j0 + c < K) ? h_bits_to_f64(x[t * K + j0 + c]) : 0.0;
    }
    __syncthreads();
#pragma unroll 4
    for (int tt = 0; tt < kHChunk; ++tt) {
      double a[4], b[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[u] = xi[tt][4 * ty + u];
        b[u] = xj[tt][4 * tx + u];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(a[u], b[v], acc[u][v]);
    }
    __syncthreads();
  }
  const double f = 2.0 / (double)n;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + 4 * ty + u, j = j0 + 4 * tx + v;
      if (i < K && j < K) Hrev[(int64_t)(K - 1 - i) * K + (K - 1 - j)] = f * acc[u][v];
    }
}

// Step 2 (one workgroup): diag += damp * trace / K; the status word is cleared.
__global__ __launch_bounds__(1024) void damp_kernel(double* __restrict__ A, int K, double damp,
                                                    int32_t* __restrict__ status) {
  __shared__ double part[1024];
  double s = 0.0;
  for (int i = threadIdx.x; i < K; i += blockDim.x) s += A[(int64_t)i * K + i];
  part[threadIdx.x] = s;
  __syncthreads();
  for (int h = blockDim.x / 2; h > 0; h >>= 1) {
    if ((int)threadIdx.x < h) part[threadIdx.x] += part[threadIdx.x + h];
    __syncthreads();
  }
  const double add = damp * part[0] / (double)K;
  for (int i = threadIdx.x; i < K; i += blockDim.x) A[(int64_t)i * K + i] += add;
  if (threadIdx.x == 0) status[0] = 0;
}

// Step 3a (one workgroup): Cholesky of the nb x nb diagonal block at kb.  A
// non-positive pivot (H not positive definite) sets the status word and is
// replaced by 1 so that the remaining steps stay finite.
// One wave, lane r holding row r of the block in registers.  Step c: the
// pivot comes from lane c, lanes below scale their entry of column c, the
// column goes through LDS, and every lane updates its row (entries right of
// its diagonal are never used).
__global__ __launch_bounds__(64) void chol_diag_kernel(double* __restrict__ A, int K, int kb,
                                                       int nb, int32_t* __restrict__ status) {
  __shared__ double col[kNB];
  const int r = threadIdx.x;
  double a[kNB];
#pragma unroll
  for (int c = 0; c < kNB; ++c)
    a[c] = (r < nb && c < nb) ? A[(int64_t)(kb + r) * K + kb + c] : (c == r ? 1.0 : 0.0);
#pragma unroll
  for (int c = 0; c < kNB; ++c) {
    if (c < nb) {
      double d = __shfl(a[c], c);
      if (!(d > 0.0)) {
        if (r == 0) status[0] = 1;
        d = 1.0;
      }
      const double p = __builtin_sqrt(d);
      const double lrc = r > c ? a[c] / p : (r == c ? p : a[c]);
      a[c] = lrc;
      col[r] = lrc;
      __syncthreads();
#pragma unroll
      for (int k = c + 1; k < kNB; ++k)
        if (r >= k) a[k] -= lrc * col[k];
      __syncthreads();
    }
  }
  if (r < nb) {
#pragma unroll
    for (int c = 0; c < kNB; ++c)
      if (c <= r) A[(int64_t)(kb + r) * K + kb + c] = a[c];
  }
}

// Step 3b: rows below the diagonal block, one row per thread: solve
// x L11^T = a (forward substitution) for the row's nb panel entries.
__global__ __launch_bounds__(256) void chol_panel_kernel(double* __restrict__ A, int K, int kb,
                                                         int nb) {
  __shared__ double l[kNB][kNB + 1];
  const int tid = threadIdx.x;
  for (int e = tid; e < nb * nb; e += 256) {
    const int r = e / nb, c = e % nb;
    l[r][c] = c <= r ? A[(int64_t)(kb + r) * K + kb + c] : 0.0;
  }
  __syncthreads();
  const int r = kb + nb + blockIdx.x * 256 + tid;
  if (r >= K) return;
  double* row = A + (int64_t)r * K + kb;
  double v[kNB];
#pragma unroll
  for (int c = 0; c < kNB; ++c) v[c] = c < nb ? row[c] : 0.0;
#pragma unroll
  for (int c = 0; c < kNB; ++c) {
    if (c < nb) {
      // four partial sums: a quarter of the dependent chain
      double s4[4] = {v[c], 0.0, 0.0, 0.0};
#pragma unroll
      for (int k = 0; k < c; ++k) s4[k & 3] -= v[k] * l[c][k];
      v[c] = ((s4[0] + s4[1]) + (s4[2] + s4[3])) / l[c][c];
    }
  }
#pragma unroll
  for (int c = 0; c < kNB; ++c)
    if (c < nb) row[c] = v[c];
}

// Step 3c: trailing lower triangle from s0 = kb + nb on: A[i][j] -= sum_k
// L[i][kb + k] L[j][kb + k], in 64 x 64 tiles (ti >= tj; the grid is square
// and the upper tiles return at once).
__global__ __launch_bounds__(256) void chol_update_kernel(double* __restrict__ A, int K, int kb,
                                                          int nb) {
  const int ti = blockIdx.x, tj = blockIdx.y;
  if (tj > ti) return;
  __shared__ double li[64][kNB + 1];
  __shared__ double lj[64][kNB + 1];
  const int s0 = kb + nb;
  const int i0 = s0 + 64 * ti, j0 = s0 + 64 * tj;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  for (int e = tid; e < 64 * kNB; e += 256) {
    const int r = e / kNB, k = e % kNB;
    li[r][k] = (i0 + r < K && k < nb) ? A[(int64_t)(i0 + r) * K + kb + k] : 0.0;
    lj[r][k] = (j0 + r < K && k < nb) ? A[(int64_t)(j0 + r) * K + kb + k] : 0.0;
  }
  __syncthreads();
  double acc[4][4] = {};
#pragma unroll 4
  for (int k = 0; k < kNB; ++k) {
    double a[4], b[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      a[u] = li[4 * ty + u][k];
      b[u] = lj[4 * tx + u][k];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(a[u], b[v], acc[u][v]);
  }
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int i = i0 + 4 * ty + u, j = j0 + 4 * tx + v;
      if (i < K && j <= i) A[(int64_t)i * K + j] -= acc[u][v];
    }
}

// Step 4.  Workgroup b owns rows r0 = 64 b .. r0 + 63 (lane = row).  DT is the
// residual matrix transposed, DT[i][n] = d_i of row n, so that a wave's
// loads of one column are contiguous.
__global__ __launch_bounds__(256) void gptq_rows_kernel(
    const uint16_t* __restrict__ w, int N, int K, const double* __restrict__ L,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int G, int gsz,
    int M, int qlo /* lowest code: 0, or 1 on the symmetric grid */, double* __restrict__ DT,
    uint8_t* __restrict__ codes) {
  __shared__ double rs[kChunk][kNB];        // R[i0 + ii][jb + c], earlier columns
  __shared__ double dsm[kChunk][kRows];     // DT[i0 + ii][r0 + lane], their residuals
  __shared__ double cs[kNB][kRows];         // sum_{i < j} d_i R_ij of each (column, row)
  __shared__ double rb[kNB][kNB + 1];       // R[jb + a][jb + c], the block's own rows
  __shared__ uint16_t ws[kRows][kNB + 2];   // the block's original weights
  __shared__ uint32_t qs[kRows][kNB / 4];    // the block's codes, stored together
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = blockIdx.x * kRows;
  const int row = r0 + lane;
  const bool valid = row < N;
  // R_ij = L[K-1-i][K-1-j]
  auto Rat = [&](int i, int j) { return L[(int64_t)(K - 1 - i) * K + (K - 1 - j)]; };

  for (int jb = 0; jb < K; jb += kNB) {
    const int nb = min(kNB, K - jb);
    // contribution of the columns before the block: thread (ty, tx) sums
    // rows 4 ty .. 4 ty + 3 and block columns 4 tx .. 4 tx + 3
    const int ty = tid >> 4, tx = tid & 15;
    double acc[4][4] = {};
    // Chunks of 64 earlier columns: R rows and residuals staged in LDS, the
    // next chunk's loads issued (into registers) before this chunk's products.
    const int nchunks = jb / kChunk;
    double pr[16], pd[16];
    auto fetch = [&](int i0) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = tid + 256 * k, ii = e >> 6, c = e & 63;
        pr[k] = c < nb ? Rat(i0 + ii, jb + c) : 0.0;
        pd[k] = r0 + c < N ? DT[(int64_t)(i0 + ii) * N + r0 + c] : 0.0;
      }
    };
    if (nchunks > 0) fetch(0);
    for (int ch = 0; ch < nchunks; ++ch) {
      __syncthreads();  // the previous chunk has been read
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const int e = tid + 256 * k, ii = e >> 6, c = e & 63;
        rs[ii][c] = pr[k];
        dsm[ii][c] = pd[k];
      }
      __syncthreads();
      if (ch + 1 < nchunks) fetch((ch + 1) * kChunk);
      // operands of step ii + 1 are read while step ii multiplies
      double a[2][4], b[2][4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        a[0][u] = dsm[0][4 * ty + u];
        b[0][u] = rs[0][4 * tx + u];
      }
#pragma unroll
      for (int ii = 0; ii < kChunk; ++ii) {
        const int cur = ii & 1, nxt = cur ^ 1;
        if (ii + 1 < kChunk) {
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            a[nxt][u] = dsm[ii + 1][4 * ty + u];
            b[nxt][u] = rs[ii + 1][4 * tx + u];
          }
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[u][v] = __builtin_fma(a[cur][u], b[cur][v], acc[u][v]);
      }
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int v = 0; v < 4; ++v) cs[4 * tx + v][4 * ty + u] = acc[u][v];
    for (int e = tid; e < kNB * kNB; e += 256) {
      const int a = e / kNB, c = e % kNB;
      rb[a][c] = (a < nb && c < nb && c >= a) ? Rat(jb + a, jb + c) : 0.0;
    }
    for (int e = tid; e < kRows * kNB; e += 256) {
      const int rr = e / kNB, c = e % kNB;
      ws[rr][c] = (r0 + rr < N && c < nb) ? w[(int64_t)(r0 + rr) * K + jb + c] : (uint16_t)0;
    }
    __syncthreads();
    // the block's columns in order, one lane per row; the row's running
    // sums for the block's columns stay in registers
    if (wave == 0) {
      // a 64-column block meets at most two groups (groups are multiples of
      // 32 columns, blocks start on multiples of 64)
      const int g0 = jb / gsz, g1 = min((jb + nb - 1) / gsz, G - 1);
      const double s0 = valid ? h_bits_to_f64(scales[(int64_t)row * G + g0]) : 1.0;
      const double s1 = valid ? h_bits_to_f64(scales[(int64_t)row * G + g1]) : 1.0;
      const int64_t z0 = valid ? zeros[(int64_t)row * G + g0] : 0;
      const int64_t z1 = valid ? zeros[(int64_t)row * G + g1] : 0;
      double cb[kNB];
#pragma unroll
      for (int j = 0; j < kNB; ++j) cb[j] = cs[j][lane];
#pragma unroll
      for (int j = 0; j < kNB; ++j) {
        if (j < nb) {
          const int col = jb + j;
          const bool first = col / gsz == g0;
          const double s = first ? s0 : s1;
          const int64_t z = first ? z0 : z1;
          const double wv = h_bits_to_f64(ws[lane][j]);
          const double t = wv + cb[j] / rb[j][j];
          int64_t q = (int64_t)__builtin_rint(t / s) + z;
          q = q < qlo ? qlo : (q > M ? M : q);
          // the dequantized weight (q - z) * s, exact in fp64
          const double deq = (double)(q - z) * s;
          const double d = wv - deq;
          reinterpret_cast<uint8_t*>(qs[lane])[j] = (uint8_t)q;
          if (valid) DT[(int64_t)col * N + row] = d;
#pragma unroll
          for (int j2 = j + 1; j2 < kNB; ++j2) cb[j2] = __builtin_fma(d, rb[j][j2], cb[j2]);
        }
      }
    }
    __syncthreads();
    // the block's codes, four per store (K is a multiple of 32, jb of 64)
    for (int e = tid; e < kRows * (kNB / 4); e += 256) {
      const int rr = e / (kNB / 4), c4 = e % (kNB / 4);
      if (r0 + rr < N && 4 * c4 < nb)
        *reinterpret_cast<uint32_t*>(codes + (int64_t)(r0 + rr) * K + jb + 4 * c4) = qs[rr][c4];
    }
  }
}

}  // namespace

size_t gptq_workspace_bytes(int64_t N, int64_t K) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return 256 + up((size_t)K * K * 8) + up((size_t)K * N * 8) + up((size_t)N * K);
}

hipError_t launch_gptq(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x,
                       int64_t n_samples, double damp, int bits, int64_t group_size, bool sym,
                       uint8_t* codes, uint32_t* packed, uint16_t* scales, int32_t* zeros,
                       void* workspace, hipStream_t stream) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  uint8_t* base = static_cast<uint8_t*>(workspace);
  int32_t* status = reinterpret_cast<int32_t*>(base);
  double* A = reinterpret_cast<double*>(base + 256);
  double* DT = reinterpret_cast<double*>(base + 256 + up((size_t)K * K * 8));
  uint8_t* wcodes = base + 256 + up((size_t)K * K * 8) + up((size_t)K * N * 8);
  uint8_t* out_codes = codes ? codes : wcodes;
  const int k = (int)K, n = (int)N;

  // the grid of the original weights (and placeholder codes)
  hipError_t e = launch_quantize(w, N, K, bits, group_size, sym, out_codes, nullptr, scales,
                                 zeros, stream);
  if (e != hipSuccess) return e;
  const int tiles = (k + 63) / 64;
  hipLaunchKernelGGL(hessian_kernel, dim3(tiles, tiles), dim3(256), 0, stream, x, n_samples, k,
                     A);
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, stream, A, k, damp, status);
  for (int kb = 0; kb < k; kb += kNB) {
    const int nb = k - kb < kNB ? k - kb : kNB;
    hipLaunchKernelGGL(chol_diag_kernel, dim3(1), dim3(64), 0, stream, A, k, kb, nb, status);
    const int below = k - kb - nb;
    if (below > 0) {
      hipLaunchKernelGGL(chol_panel_kernel, dim3((below + 255) / 256), dim3(256), 0, stream, A,
                         k, kb, nb);
      const int t = (below + 63) / 64;
      hipLaunchKernelGGL(chol_update_kernel, dim3(t, t), dim3(256), 0, stream, A, k, kb, nb);
    }
  }
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  hipLaunchKernelGGL(gptq_rows_kernel, dim3((n + kRows - 1) / kRows), dim3(256), 0, stream, w, n,
                     k, A, scales, zeros, G, gsz, (1 << bits) - 1, sym ? 1 : 0, DT, out_codes);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (packed) return launch_pack(out_codes, N, K, bits, packed, stream);
  return hipSuccess;
}

}  // namespace lowbit
