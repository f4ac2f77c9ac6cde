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
//  1. hessian_kernel: reverse(H) = (2/n) X^T X with both indices reversed
//     (the lower triangle, which is all the later steps read);
//  2. damp_kernel: damp * mean(diag) added to the diagonal; status cleared;
//  3. chol_tiles_kernel: tiled right-looking Cholesky of reverse(H) in
//     place, 64 x 64 tiles, one launch: workgroups take the factor, solve and
//     update tasks in dependency order and wait only for the tiles they read;
//  4. gptq_rows_kernel: 64 weight rows per workgroup (rows are independent),
//     K in blocks of 64 columns: the contribution of all earlier residuals
//     d_i to the block (a 64 x j0 x 64 product on the fp64 matrix cores,
//     eight waves) and then the block's columns one after another (one lane
//     per row);
//  5. the codes are packed by the packing kernel.
// deq_i = (q_i - z) * s is the exact value code q_i stands for.  The grid
// (scales, zero points) is the RTN grid of the original weights
// (min-max, or signed symmetric with codes from 1), written by the RTN
// quantizer before step 4.
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lowbit {

namespace {

constexpr int kNB = 64;    // GPTQ column block
constexpr int kRows = 64;  // weight rows per GPTQ workgroup (32 on shorter layers)
constexpr int kChunk = 64;   // earlier columns staged per LDS round in step 4
constexpr int kHChunk = 32;  // calibration rows staged per LDS round in step 1
constexpr int kRowThreads = 512;  // step 4: eight waves, two per SIMD

typedef double f64x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double h_bits_to_f64(uint16_t b) {
  return (double)__builtin_bit_cast(_Float16, b);
}

// Step 1.  Workgroup (bi, bj) computes the 64 x 64 tile of H at rows
// 64 bi.., columns 64 bj.. and stores it with both indices reversed.  Only
// tiles with bi <= bj are formed: H is symmetric and the later steps read the
// lower triangle of reverse(H) alone (entries i >= j).
// The products run on the fp64 matrix cores (v_mfma_f64_16x16x4f64,
// D = A B + D with A 16 x 4, B 4 x 16): wave w owns the 32 x 32 quarter
// (w / 2, w % 2) as 2 x 2 tiles; lane l supplies A[l % 16][l / 16] and
// B[l / 16][l % 16] (calibration row l / 16 of the 4-row step) and holds
// D[l / 16 + 4 v][l % 16] in element v.  Operands come from the staged rows
// in LDS, one read per lane and tile edge per 4 rows (eight times fewer LDS
// reads per multiply-add than 4 x 4 register tiles on the vector units).
__global__ __launch_bounds__(256) void hessian_kernel(const uint16_t* __restrict__ x, int64_t n,
                                                      int K, double* __restrict__ Hrev) {
  if (blockIdx.x > blockIdx.y) return;
  __shared__ __align__(16) double xi[kHChunk][64];
  __shared__ __align__(16) double xj[kHChunk][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int i0 = blockIdx.x * 64, j0 = blockIdx.y * 64;
  const int ml = lane & 15, kl = lane >> 4;
  const int mb = (wave >> 1) * 32, nbw = (wave & 1) * 32;
  f64x4_t acc[2][2];
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v) acc[u][v] = f64x4_t{0.0, 0.0, 0.0, 0.0};
  // Staging: each thread brings 8 consecutive values (16 bytes) of one
  // calibration row for each operand (K is a multiple of 32 and x 16-byte
  // aligned, so a piece is wholly inside or outside the matrix); the next
  // chunk's pieces are loaded while this chunk multiplies.  Rows past n and
  // columns past K are clamped for the load and replaced by zeros.
  static_assert(kHChunk * 8 == 256, "one 16-byte piece per thread and operand");
  const int tt = tid >> 3, c8 = (tid & 7) * 8;
  const bool in_i = i0 + c8 < K, in_j = j0 + c8 < K;
  const int ci = in_i ? i0 + c8 : 0, cj = in_j ? j0 + c8 : 0;
  uint4 pi, pj;
  auto fetch = [&](int64_t t0) {
    const int64_t t = t0 + tt < n ? t0 + tt : n - 1;
    pi = *reinterpret_cast<const uint4*>(x + t * K + ci);
    pj = *reinterpret_cast<const uint4*>(x + t * K + cj);
  };
  auto put = [&](double (*dst)[64], uint4 p, bool keep) {
    const uint32_t wv[4] = {p.x, p.y, p.z, p.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const double lo = keep ? h_bits_to_f64((uint16_t)(wv[q] & 0xffffu)) : 0.0;
      const double hi = keep ? h_bits_to_f64((uint16_t)(wv[q] >> 16)) : 0.0;
      *reinterpret_cast<double2*>(&dst[tt][c8 + 2 * q]) = double2{lo, hi};
    }
  };
  fetch(0);
  for (int64_t t0 = 0; t0 < n; t0 += kHChunk) {
    const bool row_in = t0 + tt < n;
    __syncthreads();  // the previous chunk has been read
    put(xi, pi, row_in && in_i);
    put(xj, pj, row_in && in_j);
    __syncthreads();
    if (t0 + kHChunk < n) fetch(t0 + kHChunk);
#pragma unroll
    for (int kk = 0; kk < kHChunk / 4; ++kk) {
      const int tt4 = 4 * kk + kl;
      const double a0 = xi[tt4][mb + ml], a1 = xi[tt4][mb + 16 + ml];
      const double b0 = xj[tt4][nbw + ml], b1 = xj[tt4][nbw + 16 + ml];
      acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
      acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
      acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
      acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
    }
  }
  const double f = 2.0 / (double)n;
#pragma unroll
  for (int u = 0; u < 2; ++u)
#pragma unroll
    for (int v = 0; v < 2; ++v)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = i0 + mb + 16 * u + kl + 4 * e, j = j0 + nbw + 16 * v + ml;
        if (i < K && j < K) Hrev[(int64_t)(K - 1 - i) * K + (K - 1 - j)] = f * acc[u][v][e];
      }
}

// Step 2 (one workgroup): diag += damp * trace / K; the status word, the
// task counter and the tile counters of step 3 are cleared.
__global__ __launch_bounds__(1024) void damp_kernel(double* __restrict__ A, int K, double damp,
                                                    int32_t* __restrict__ status,
                                                    int* __restrict__ ver, int nver,
                                                    int* __restrict__ ticket) {
  for (int i = threadIdx.x; i < nver; i += blockDim.x) ver[i] = 0;
  if (threadIdx.x == 0) ticket[0] = 0;
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

// Step 3, as one kernel over 64 x 64 tiles of the lower triangle (nt tiles
// per side): the tasks of the right-looking tiled Cholesky,
//   for k: factor tile (k, k); solve tiles (i, k), i > k, against it;
//          update tiles (i, j), k < j <= i, by tile(i, k) tile(j, k)^T,
// numbered in that order (within step k the updates column by column, so
// that tile (k+1, k+1), which the next factorization needs, comes first).
// Workgroups take task numbers from a counter and wait only for the tiles
// their task reads: ver[i nt + j] counts the updates applied to tile (i, j),
// plus one once it is final.  Every task waits only for tasks with smaller
// numbers, which workgroups that are already running hold, so the waits end;
// each is bounded all the same (status bit 2 if a bound is ever reached, and
// every later wait then gives up at once).
// Tiles move between workgroups through device-coherent loads and stores
// (they bypass the non-coherent caches), so a tile is published by waiting
// for its stores and then storing its counter; no cache-wide write-back or
// invalidation is needed.
constexpr int kT = 64;
constexpr int kTP = kT + 2;  // LDS tile row stride: 16-byte aligned rows
constexpr int kSpinLimit = 1 << 22;

__device__ __forceinline__ double ld_dev(const double* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_dev(double* p, double v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// every earlier memory operation of this wave has completed (vmcnt = 0)
__device__ __forceinline__ void wait_vmem() {
  __builtin_amdgcn_s_waitcnt(0 | (0x7 << 4) | (0xf << 8));
}

__device__ __forceinline__ double readlane_f64(double v, int l) {
  const long long b = __builtin_bit_cast(long long, v);
  const unsigned lo = (unsigned)__builtin_amdgcn_readlane((int)b, l);
  const unsigned hi = (unsigned)__builtin_amdgcn_readlane((int)(b >> 32), l);
  return __builtin_bit_cast(double, ((unsigned long long)hi << 32) | lo);
}

int chol_task_count(int nt) {
  int n = 0;
  for (int k = 0; k < nt; ++k) {
    const int m = nt - 1 - k;
    n += 1 + m + m * (m + 1) / 2;
  }
  return n;
}

// The factor and solve tasks work in panels of kP columns.  For a panel,
// one wave (lane r holding row r's kP panel entries in registers) runs the
// panel's column steps, each touching only the panel's own columns; then the
// four waves apply the panel to the columns right of it as 16 x 16 tiles on
// the fp64 matrix cores.  The serial chain per column is thus short (at most
// kP - 1 multiply-adds), and the bulk of the work is matrix-core work.
constexpr int kP = 16;

// D[16 ti + m][16 tj + n] -= sum_{c < kP} P(16 ti + m, c0 + c) Q(16 tj + n, c0 + c),
// m, n < 16, with P(r, c) = p[r pr + c pc] and Q(s, c) = q[s qr + c qc] in LDS;
// D row-major with stride ldd.  Lane layout of v_mfma_f64_16x16x4f64 as in
// the Hessian (lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16] and
// holds D[l / 16 + 4 e][l % 16] in element e).
__device__ __forceinline__ void tile_sub_product(double* d, int ldd, const double* p, int pr,
                                                 int pc, const double* q, int qr, int qc, int ti,
                                                 int tj, int c0, int lane) {
  const int ml = lane & 15, kl = lane >> 4;
  f64x4_t acc;
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = d[(16 * ti + kl + 4 * e) * ldd + 16 * tj + ml];
#pragma unroll
  for (int kk = 0; kk < kP / 4; ++kk) {
    const int c = c0 + 4 * kk + kl;
    const double av = -p[(16 * ti + ml) * pr + c * pc];
    const double bv = q[(16 * tj + ml) * qr + c * qc];
    acc = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc, 0, 0, 0);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) d[(16 * ti + kl + 4 * e) * ldd + 16 * tj + ml] = acc[e];
}

// 1 / sqrt(d) to fp64 accuracy: the hardware estimate and two Newton steps
__device__ __forceinline__ double rsqrt_f64(double d) {
  double y = __builtin_amdgcn_rsq(d);
  y = y * (1.5 - 0.5 * d * y * y);
  y = y * (1.5 - 0.5 * d * y * y);
  return y;
}

// Factor panel C0 of an LDS tile t (row stride kTP, lower triangle valid,
// earlier panels already applied): one wave, lane r = row r.  Column C0 + c
// goes to every lane through one of two LDS column buffers.  Branch-free (a
// non-positive pivot is replaced by 1 and counted in bad).
template <int C0>
__device__ __forceinline__ void potrf_panel(double* t, int r, double* colA, double* colB,
                                            int& bad) {
  double a[kP];
#pragma unroll
  for (int c = 0; c < kP; ++c) a[c] = t[r * kTP + C0 + c];
#pragma unroll
  for (int c = 0; c < kP; ++c) {
    double d = readlane_f64(a[c], C0 + c);
    const bool ok = d > 0.0;  // d is the same in every lane
    bad |= ok ? 0 : 1;
    d = ok ? d : 1.0;
    // rows r >= C0 + c: the factor's entry (d rp on the diagonal); rows
    // above hold entries right of their diagonal here, which are never read
    const double l = a[c] * rsqrt_f64(d);
    a[c] = l;
    double* col = (c & 1) ? colB : colA;
    col[r] = l;
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int m = c + 1; m < kP; ++m) a[m] = __builtin_fma(-l, col[C0 + m], a[m]);
  }
#pragma unroll
  for (int c = 0; c < kP; ++c) t[r * kTP + C0 + c] = a[c];
}

// Solve panel C0 of the rows x (LDS, row stride kTP) against the factor,
// lt[c][m] = L[m][c] (column c of the factor as an LDS row), rd[c] =
// 1 / L[c][c]: one wave, lane r = row r.
template <int C0>
__device__ __forceinline__ void trsm_panel(double* x, int r, const double* lt, const double* rd) {
  double a[kP];
#pragma unroll
  for (int c = 0; c < kP; ++c) a[c] = x[r * kTP + C0 + c];
#pragma unroll
  for (int c = 0; c < kP; ++c) {
    const double xc = a[c] * rd[C0 + c];
    a[c] = xc;
    // the factor row's offset depends on xc, so that the compiler does not
    // hoist every step's reads to the start
    int off = (C0 + c) * kTP;
    asm volatile("" : "+v"(off) : "v"(xc));
#pragma unroll
    for (int m = c + 1; m < kP; ++m) a[m] = __builtin_fma(-xc, lt[off + C0 + m], a[m]);
  }
#pragma unroll
  for (int c = 0; c < kP; ++c) x[r * kTP + C0 + c] = a[c];
}

__global__ __launch_bounds__(256, 2) void chol_tiles_kernel(double* __restrict__ A, int K, int nt,
                                                            int ntasks, int* __restrict__ ver,
                                                            int* __restrict__ ticket,
                                                            int32_t* __restrict__ status) {
  __shared__ __align__(16) double ta[kT][kTP];
  __shared__ __align__(16) double tb[kT][kTP];
  __shared__ __align__(16) double rd[kT];
  __shared__ int task[4];
  const int tid = threadIdx.x, lane = tid & 63;
  // the wave index in a scalar register: branches on it are wave-uniform
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // No control flow in this loop depends on the lane: wave 0 as a whole
  // takes the task and waits, the other waves wait at the barrier.  (With a
  // thread-0 region at each end of the loop body, the two regions can be
  // merged across the back edge into a loop exit that the other lanes of
  // wave 0 do not take; they then meet the next barrier without thread 0.)
  for (;;) {
    if (wave == 0) {
      int t = 0;
      if (lane == 0) t = atomicAdd(ticket, 1);
      t = __builtin_amdgcn_readfirstlane(t);  // lane 0, the first active lane
      int type = -1, ti = 0, tj = 0, tk = 0;
      if (t < ntasks) {
        int k = 0, base = 0, m = nt - 1;
        for (;;) {
          const int sz = 1 + m + m * (m + 1) / 2;
          if (t < base + sz) break;
          base += sz, ++k, --m;
        }
        const int o = t - base;
        if (o == 0) {
          type = 0, ti = tj = tk = k;
        } else if (o <= m) {
          type = 1, ti = k + o, tj = k, tk = k;
        } else {
          int u = o - 1 - m, j = k + 1;
          while (u >= nt - j) u -= nt - j, ++j;
          type = 2, ti = j + u, tj = j, tk = k;
        }
        // every lane polls the same word; the value is taken from lane 0
        auto wait_ge = [&](int idx, int target) {
          for (int it = 0;; ++it) {
            const int v = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(&ver[idx], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
            if (v >= target) return;
            if ((it & 63) == 63 &&
                (__builtin_amdgcn_readfirstlane(__hip_atomic_load(
                     status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) & 2))
              return;
            if (it >= kSpinLimit) {
              atomicOr(status, 2);
              return;
            }
            __builtin_amdgcn_s_sleep(1);
          }
        };
        wait_ge(ti * nt + tj, tk);  // the earlier updates of the task's own tile
        if (type == 1) wait_ge(tk * nt + tk, tk + 1);
        if (type == 2) {
          wait_ge(ti * nt + tk, tk + 1);
          wait_ge(tj * nt + tk, tk + 1);
        }
        // the tile loads below are issued after the counters were seen
        wait_vmem();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
      }
      // all lanes write the same values
      task[0] = type, task[1] = ti, task[2] = tj, task[3] = tk;
    }
    __syncthreads();
    const int type = __builtin_amdgcn_readfirstlane(task[0]);
    const int ti = __builtin_amdgcn_readfirstlane(task[1]);
    const int tj = __builtin_amdgcn_readfirstlane(task[2]);
    const int tk = __builtin_amdgcn_readfirstlane(task[3]);
    if (type < 0) return;
    const int r0 = ti * kT, c0 = tj * kT, k0 = tk * kT;
    const int nbi = min(kT, K - r0), nbj = min(kT, K - c0);
    // The thread index, opaque per task: values derived from it are
    // recomputed in each task instead of being held (and spilled) across
    // the whole loop.
    int tid_ = tid;
    asm volatile("" : "+v"(tid_));
    const int lane = tid_ & 63;
    // Staging: thread tid handles entries (4 q + tid / 64, tid % 64), q < 16;
    // rows past the matrix are clamped for the load and replaced by 0 (or
    // the identity) afterwards, so every load is issued unconditionally.
    const int er = tid_ >> 6, ec = tid_ & 63;
    if (type == 0) {
      // factor tile (k, k): one wave, lane r holding row r; column c's
      // entries go through LDS to every lane
      double v[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + er;
        v[q] = ld_dev(&A[(int64_t)(r0 + min(r, nbi - 1)) * K + r0 + min(ec, nbi - 1)]);
      }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + er;
        ta[r][ec] = (r < nbi && ec <= r) ? v[q] : (r == ec ? 1.0 : 0.0);
      }
      __syncthreads();
      // panels of kP columns: the panel's column steps on one wave, then the
      // lower tiles right of and below the panel updated on the matrix cores
      int bad = 0;
      auto panel = [&](auto c0v) {
        constexpr int C0 = decltype(c0v)::value;
        if (wave == 0) potrf_panel<C0>(&ta[0][0], lane, rd, &tb[0][0], bad);
        __syncthreads();
        if constexpr (C0 + kP < kT) {
          constexpr int n = (kT - C0 - kP) / 16, p0 = (C0 + kP) / 16;
          for (int t = wave; t < n * (n + 1) / 2; t += 4) {
            int ti = 0;
            while ((ti + 1) * (ti + 2) / 2 <= t) ++ti;
            const int tj = t - ti * (ti + 1) / 2;
            tile_sub_product(&ta[0][0], kTP, &ta[0][0], kTP, 1, &ta[0][0], kTP, 1, p0 + ti, p0 + tj,
                             C0, lane);
          }
          __syncthreads();
        }
      };
      panel(std::integral_constant<int, 0>{});
      panel(std::integral_constant<int, 16>{});
      panel(std::integral_constant<int, 32>{});
      panel(std::integral_constant<int, 48>{});
      if (wave == 0 && bad) atomicOr(status, 1);  // the same in every lane
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + er;
        if (r < nbi && ec <= r) st_dev(&A[(int64_t)(r0 + r) * K + r0 + ec], ta[r][ec]);
      }
    } else if (type == 1) {
      // solve tile (i, k): X L_kk^T = A_ik, one wave, lane r holding row r;
      // ta[c][m] = L_kk[m][c] (column c of the factor as a row)
      double v[16], w[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = 4 * q + er;
        v[q] = ld_dev(&A[(int64_t)(k0 + m) * K + k0 + ec]);
        w[q] = ld_dev(&A[(int64_t)(r0 + min(m, nbi - 1)) * K + k0 + ec]);
      }
      double dg = 1.0;
      if (tid < kT) dg = ld_dev(&A[(int64_t)(k0 + tid) * K + k0 + tid]);
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = 4 * q + er;
        ta[ec][m] = ec <= m ? v[q] : 0.0;
        tb[m][ec] = m < nbi ? w[q] : 0.0;
      }
      if (tid < kT) rd[tid] = 1.0 / dg;
      __syncthreads();
      // panels of kP columns: the panel's column steps on one wave, then the
      // columns right of the panel, all rows, updated on the matrix cores
      auto panel = [&](auto c0v) {
        constexpr int C0 = decltype(c0v)::value;
        if (wave == 0) trsm_panel<C0>(&tb[0][0], lane, &ta[0][0], rd);
        __syncthreads();
        if constexpr (C0 + kP < kT) {
          constexpr int n = (kT - C0 - kP) / 16, p0 = (C0 + kP) / 16;
          for (int t = wave; t < 4 * n; t += 4)
            tile_sub_product(&tb[0][0], kTP, &tb[0][0], kTP, 1, &ta[0][0], 1, kTP, t & 3,
                             p0 + (t >> 2), C0, lane);
          __syncthreads();
        }
      };
      panel(std::integral_constant<int, 0>{});
      panel(std::integral_constant<int, 16>{});
      panel(std::integral_constant<int, 32>{});
      panel(std::integral_constant<int, 48>{});
      __syncthreads();
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int m = 4 * q + er;
        if (m < nbi) st_dev(&A[(int64_t)(r0 + m) * K + k0 + ec], tb[m][ec]);
      }
    } else {
      // update tile (i, j) -= tile(i, k) tile(j, k)^T on the fp64 matrix
      // cores: wave w owns the 32 x 32 quarter (w / 2, w % 2) as 2 x 2 tiles
      const int ml = lane & 15, kl = lane >> 4;
      const int mb = (wave >> 1) * 32, nbw = (wave & 1) * 32;
      double v[16], w[16];
      f64x4_t acc[2][2];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + er;
        v[q] = ld_dev(&A[(int64_t)(r0 + min(r, nbi - 1)) * K + k0 + ec]);
        w[q] = ld_dev(&A[(int64_t)(c0 + min(r, nbj - 1)) * K + k0 + ec]);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int vv = 0; vv < 2; ++vv)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = mb + 16 * u + kl + 4 * e, c = nbw + 16 * vv + ml;
            acc[u][vv][e] =
                ld_dev(&A[(int64_t)(r0 + min(r, nbi - 1)) * K + c0 + min(c, nbj - 1)]);
          }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int r = 4 * q + er;
        ta[r][ec] = r < nbi ? v[q] : 0.0;
        tb[r][ec] = r < nbj ? w[q] : 0.0;
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < kT / 4; ++kk) {
        const int m = 4 * kk + kl;
        const double a0 = -ta[mb + ml][m], a1 = -ta[mb + 16 + ml][m];
        const double b0 = tb[nbw + ml][m], b1 = tb[nbw + 16 + ml][m];
        acc[0][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, acc[0][0], 0, 0, 0);
        acc[0][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b1, acc[0][1], 0, 0, 0);
        acc[1][0] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b0, acc[1][0], 0, 0, 0);
        acc[1][1] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, acc[1][1], 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int vv = 0; vv < 2; ++vv)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int r = mb + 16 * u + kl + 4 * e, c = nbw + 16 * vv + ml;
            if (r < nbi && c < nbj && (ti != tj || c <= r))
              st_dev(&A[(int64_t)(r0 + r) * K + c0 + c], acc[u][vv][e]);
          }
    }
    // publish the tile: every wave's stores have completed before the
    // counter moves
    wait_vmem();
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __syncthreads();
    if (wave == 0)  // every lane stores the same value
      __hip_atomic_store(&ver[ti * nt + tj], tk + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Step 4.  Workgroup b owns rows r0 = RW b .. r0 + RW - 1 (lane = row; RW is
// 16, 32, 48 or 64: the fewest whose workgroups all fit on the CUs at once).
// DT is the residual matrix transposed, DT[i][n] = d_i of row n, so that a
// wave's loads of one column are contiguous.
template <int RW>
__global__ __launch_bounds__(kRowThreads) void gptq_rows_kernel(
    const uint16_t* __restrict__ w, int N, int K, const double* __restrict__ L,
    const uint16_t* __restrict__ scales, const int32_t* __restrict__ zeros, int G, int gsz,
    int M, int qlo /* lowest code: 0, or 1 on the symmetric grid */, double* __restrict__ DT,
    uint8_t* __restrict__ codes) {
  __shared__ double rs[kChunk][kNB];        // R[i0 + ii][jb + c], earlier columns
  static_assert(RW == 16 || RW == 32 || RW == 48 || RW == 64, "16-row tiles, one lane per row");
  static_assert(kRowThreads == 512, "the product tiles are laid out for eight waves");
  constexpr int NRT = RW / 16;               // 16-row product tiles (times 4 column tiles)
  constexpr int CPW = RW <= 32 ? 1 : 2;      // most 16-column product tiles of one wave
  __shared__ double dsm[kChunk][RW];        // DT[i0 + ii][r0 + lane], their residuals
  __shared__ double cs[kNB][RW];            // sum_{i < j} d_i R_ij of each (column, row)
  __shared__ double rb[kNB][kNB + 2];       // R[jb + a][jb + c], the block's own rows (16-byte rows)
  __shared__ double rdi[kNB];               // 1 / R[jb + a][jb + a]
  __shared__ uint16_t ws[RW][kNB + 2];      // the block's original weights
  __shared__ uint32_t qs[RW][kNB / 4];       // the block's codes, stored together
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int ml = lane & 15, kl = lane >> 4;
  // Product tiles of wave w (wave w runs on SIMD w mod 4): rows mb .. mb + 15,
  // ncw column tiles from nbw.  RW = 32 and 64: NRT row tiles times 4 column
  // tiles spread evenly (one or two per wave).  RW = 48: 12 tiles, two for
  // waves 0-3 and one for waves 4-7, so that every SIMD holds three.  RW =
  // 16: 4 tiles, each summed by two waves over the two halves of a chunk
  // (kh), the halves added in LDS.
  int mb, nbw, ncw, kh = 0;
  if constexpr (RW == 16) {
    mb = 0, nbw = (wave & 3) * 16, ncw = 1, kh = wave >> 2;
  } else if constexpr (RW == 48) {
    if (wave < 4) {
      mb = (wave >> 1) * 16, nbw = (wave & 1) * 32, ncw = 2;
    } else {
      mb = 32, nbw = (wave - 4) * 16, ncw = 1;
    }
  } else {
    mb = (wave % NRT) * 16, nbw = (wave / NRT) * 16 * CPW, ncw = CPW;
  }
  const int r0 = blockIdx.x * RW;
  const int row = r0 + lane;
  const bool valid = lane < RW && row < N;
  const int lr = lane < RW ? lane : RW - 1;  // LDS row of the lane (lanes past RW idle)
  // R_ij = L[K-1-i][K-1-j]
  auto Rat = [&](int i, int j) { return L[(int64_t)(K - 1 - i) * K + (K - 1 - j)]; };

  for (int jb = 0; jb < K; jb += kNB) {
    const int nb = min(kNB, K - jb);
    // contribution of the columns before the block, on the fp64 matrix
    // cores: wave w sums rows mb .. mb + 15 and block columns
    // nbw .. nbw + 16 ncw - 1 as 16 x 16 tiles (lane layout as in step 1);
    // two waves per SIMD keep the matrix pipe busier than one
    f64x4_t acc[CPW];
#pragma unroll
    for (int v = 0; v < CPW; ++v) acc[v] = f64x4_t{0.0, 0.0, 0.0, 0.0};
    // Chunks of 64 earlier columns: R rows and residuals staged in LDS, the
    // next chunk's loads issued (into registers) before this chunk's products.
    const int nchunks = jb / kChunk;
    constexpr int PR = kChunk * kNB / kRowThreads, PD = kChunk * RW / kRowThreads;
    double pr[PR], pd[PD];
    auto fetch = [&](int i0) {
#pragma unroll
      for (int k = 0; k < PR; ++k) {
        const int e = tid + kRowThreads * k, ii = e >> 6, c = e & 63;
        pr[k] = c < nb ? Rat(i0 + ii, jb + c) : 0.0;
      }
#pragma unroll
      for (int k = 0; k < PD; ++k) {
        const int e = tid + kRowThreads * k, ii = e / RW, c = e % RW;
        pd[k] = r0 + c < N ? DT[(int64_t)(i0 + ii) * N + r0 + c] : 0.0;
      }
    };
    if (nchunks > 0) fetch(0);
    for (int ch = 0; ch < nchunks; ++ch) {
      __syncthreads();  // the previous chunk has been read
#pragma unroll
      for (int k = 0; k < PR; ++k) {
        const int e = tid + kRowThreads * k, ii = e >> 6, c = e & 63;
        rs[ii][c] = pr[k];
      }
#pragma unroll
      for (int k = 0; k < PD; ++k) {
        const int e = tid + kRowThreads * k, ii = e / RW, c = e % RW;
        dsm[ii][c] = pd[k];
      }
      __syncthreads();
      if (ch + 1 < nchunks) fetch((ch + 1) * kChunk);
      auto mma_chunk = [&](auto nc) {
        constexpr int NC = decltype(nc)::value;
        constexpr int NKK = RW == 16 ? kChunk / 8 : kChunk / 4;
#pragma unroll
        for (int k2 = 0; k2 < NKK; ++k2) {
          const int ii = 4 * (k2 + NKK * kh) + kl;
          const double a = dsm[ii][mb + ml];
          double b[NC];
#pragma unroll
          for (int v = 0; v < NC; ++v) b[v] = rs[ii][nbw + 16 * v + ml];
#pragma unroll
          for (int v = 0; v < NC; ++v)
            acc[v] = __builtin_amdgcn_mfma_f64_16x16x4f64(a, b[v], acc[v], 0, 0, 0);
        }
      };
      if constexpr (CPW == 1) {
        mma_chunk(std::integral_constant<int, 1>{});
      } else {
        if (ncw == 2)
          mma_chunk(std::integral_constant<int, 2>{});
        else
          mma_chunk(std::integral_constant<int, 1>{});
      }
    }
    if constexpr (RW == 16) {
      // waves 4-7 hold the second halves of the chunks' sums
      if (kh == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[nbw + ml][kl + 4 * e] = acc[0][e];
      }
      __syncthreads();
      if (kh == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[nbw + ml][kl + 4 * e] += acc[0][e];
      }
    } else {
#pragma unroll
      for (int v = 0; v < CPW; ++v)
        if (v < ncw) {
#pragma unroll
          for (int e = 0; e < 4; ++e) cs[nbw + 16 * v + ml][mb + kl + 4 * e] = acc[v][e];
        }
    }
    for (int e = tid; e < kNB * kNB; e += kRowThreads) {
      const int a = e / kNB, c = e % kNB;
      rb[a][c] = (a < nb && c < nb && c >= a) ? Rat(jb + a, jb + c) : 0.0;
    }
    // the reciprocals of the block's diagonal, so the column walk's chain
    // holds one division (the code decision) instead of two
    for (int a = tid; a < kNB; a += kRowThreads) rdi[a] = a < nb ? 1.0 / Rat(jb + a, jb + a) : 1.0;
    for (int e = tid; e < RW * kNB; e += kRowThreads) {
      const int rr = e / kNB, c = e % kNB;
      ws[rr][c] = (r0 + rr < N && c < nb) ? w[(int64_t)(r0 + rr) * K + jb + c] : (uint16_t)0;
    }
    __syncthreads();
    // The block's columns in order, one lane per row, the row's running sums
    // in registers, in two halves of kNB / 2 columns: a column's decision
    // updates only the sums of its own half, and between the halves the
    // first half's residuals enter the second half's sums as one small
    // product on the matrix cores (the serial chain per column then carries
    // at most kNB / 2 - 1 multiply-adds instead of kNB - 1).
    constexpr int kH = kNB / 2;
    // a 64-column block meets at most two groups (groups are multiples of
    // 32 columns, blocks start on multiples of 64)
    const int g0 = jb / gsz, g1 = min((jb + nb - 1) / gsz, G - 1);
    // column j's decision for the lane's row from its running sum: code into
    // qs, residual into DT (and returned)
    auto decide = [&](int j, double cbj, double s0, double s1, int64_t z0, int64_t z1) {
      const int col = jb + j;
      const bool first = col / gsz == g0;
      const double s = first ? s0 : s1;
      const int64_t z = first ? z0 : z1;
      const double wv = h_bits_to_f64(ws[lr][j]);
      const double t = wv + cbj * rdi[j];
      int64_t q = (int64_t)__builtin_rint(t / s) + z;
      q = q < qlo ? qlo : (q > M ? M : q);
      // the dequantized weight (q - z) * s, exact in fp64
      const double deq = (double)(q - z) * s;
      const double d = wv - deq;
      if (lane < RW) reinterpret_cast<uint8_t*>(qs[lane])[j] = (uint8_t)q;
      if (valid) DT[(int64_t)col * N + row] = d;
      return d;
    };
    // the half [J0, J0 + kH): running sums cbh, factor rows of the block in
    // 16-byte reads, four entries at a time, issued before their
    // multiply-adds; the residuals go to dh (when given)
    auto walk_half = [&](auto j0v, double (&cbh)[kH], double* dh) {
      constexpr int J0 = decltype(j0v)::value;
      const double s0 = valid ? h_bits_to_f64(scales[(int64_t)row * G + g0]) : 1.0;
      const double s1 = valid ? h_bits_to_f64(scales[(int64_t)row * G + g1]) : 1.0;
      const int64_t z0 = valid ? zeros[(int64_t)row * G + g0] : 0;
      const int64_t z1 = valid ? zeros[(int64_t)row * G + g1] : 0;
#pragma unroll
      for (int jj = 0; jj < kH; ++jj) {
        const int j = J0 + jj;
        if (j < nb) {
          const double d = decide(j, cbh[jj], s0, s1, z0, z1);
          if (dh) dh[jj] = d;
#pragma unroll
          for (int j2b = (jj + 1) & ~1; j2b < kH; j2b += 4) {
            double r8[4];
#pragma unroll
            for (int t = 0; t < 4; t += 2) {
              if (j2b + t < kH) {
                const double2 v = *reinterpret_cast<const double2*>(&rb[j][J0 + j2b + t]);
                r8[t] = v.x, r8[t + 1] = v.y;
              }
            }
#pragma unroll
            for (int t = 0; t < 4; ++t) {
              const int j2 = j2b + t;
              if (j2 > jj && j2 < kH) cbh[j2] = __builtin_fma(d, r8[t], cbh[j2]);
            }
          }
        }
      }
    };
    if (wave == 0) {
      double cbh[kH], dh[kH];
#pragma unroll
      for (int jj = 0; jj < kH; ++jj) cbh[jj] = cs[jj][lr];
      walk_half(std::integral_constant<int, 0>{}, cbh, dh);
      // the first half's residuals for the cross product (dsm is free now)
      if (lane < RW) {
#pragma unroll
        for (int jj = 0; jj < kH; ++jj) dsm[jj][lane] = dh[jj];
      }
    }
    __syncthreads();
    if (nb > kH) {
      // second-half sums += (first-half residuals) x (factor rows 0..kH-1,
      // columns kH..kNB-1): NRT x 2 tiles of 16 x 16, one per wave
      if (wave < 2 * NRT) {
        const int rt = wave % NRT, ct = 2 + wave / NRT;
        f64x4_t acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = cs[16 * ct + ml][16 * rt + kl + 4 * e];
#pragma unroll
        for (int kk = 0; kk < kH / 4; ++kk) {
          const int jj = 4 * kk + kl;
          acc = __builtin_amdgcn_mfma_f64_16x16x4f64(dsm[jj][16 * rt + ml], rb[jj][16 * ct + ml],
                                                     acc, 0, 0, 0);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) cs[16 * ct + ml][16 * rt + kl + 4 * e] = acc[e];
      }
      __syncthreads();
      if (wave == 0) {
        double cbh[kH];
#pragma unroll
        for (int jj = 0; jj < kH; ++jj) cbh[jj] = cs[kH + jj][lr];
        walk_half(std::integral_constant<int, kH>{}, cbh, nullptr);
      }
    }
    __syncthreads();
    // the block's codes, four per store (K is a multiple of 32, jb of 64)
    for (int e = tid; e < RW * (kNB / 4); e += kRowThreads) {
      const int rr = e / (kNB / 4), c4 = e % (kNB / 4);
      if (r0 + rr < N && 4 * c4 < nb)
        *reinterpret_cast<uint32_t*>(codes + (int64_t)(r0 + rr) * K + jb + 4 * c4) = qs[rr][c4];
    }
  }
}

}  // namespace

// The no-allocation entry point's workspace: a file-scope device array of
// kGptqScratchBytes (each GPU the library runs on holds its own copy until the
// process ends).  In host code `gptq_scratch` only names the symbol; its
// device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is passed to kernels.
namespace {

__device__ __align__(256) unsigned char gptq_scratch[kGptqScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Copies the status word of a run into the caller's output.
__global__ void copy_status_kernel(const int32_t* __restrict__ from, int32_t* __restrict__ to) {
  if (threadIdx.x == 0 && blockIdx.x == 0) to[0] = from[0];
}

}  // namespace

hipError_t gptq_scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(gptq_scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_gptq_noalloc(const uint16_t* w, int64_t N, int64_t K, const uint16_t* x,
                               int64_t n_samples, double damp, int bits, int64_t group_size,
                               uint8_t* codes, uint32_t* packed, uint16_t* scales, int32_t* zeros,
                               int32_t* status_out, hipStream_t stream) {
  void* ws = nullptr;
  hipError_t e = gptq_scratch_address(&ws);
  if (e != hipSuccess) return e;
  e = launch_gptq(w, N, K, x, n_samples, damp, bits, group_size, false, codes, packed, scales,
                  zeros, ws, stream);
  if (e != hipSuccess || status_out == nullptr) return e;
  hipLaunchKernelGGL(copy_status_kernel, dim3(1), dim3(64), 0, stream,
                     static_cast<const int32_t*>(ws), status_out);
  return hipGetLastError();
}

size_t gptq_workspace_bytes(int64_t N, int64_t K) {
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t nt = (size_t)((K + kT - 1) / kT);
  return 256 + up((size_t)K * K * 8) + up((size_t)K * N * 8) + up((size_t)N * K) +
         up(nt * nt * 4);
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
  int* ver = reinterpret_cast<int*>(wcodes + up((size_t)N * K));
  int* ticket = reinterpret_cast<int*>(base + 64);
  uint8_t* out_codes = codes ? codes : wcodes;
  const int k = (int)K, n = (int)N;

  // the grid of the original weights (and placeholder codes)
  hipError_t e = launch_quantize(w, N, K, bits, group_size, sym, out_codes, nullptr, scales,
                                 zeros, stream);
  if (e != hipSuccess) return e;
  const int tiles = (k + 63) / 64;
  hipLaunchKernelGGL(hessian_kernel, dim3(tiles, tiles), dim3(256), 0, stream, x, n_samples, k,
                     A);
  const int nt = (k + kT - 1) / kT;
  hipLaunchKernelGGL(damp_kernel, dim3(1), dim3(1024), 0, stream, A, k, damp, status, ver,
                     nt * nt, ticket);
  hipLaunchKernelGGL(chol_tiles_kernel, dim3(2 * device_cu_count()), dim3(256), 0, stream, A, k,
                     nt, chol_task_count(nt), ver, ticket, status);
  const int gsz = (int)(group_size == 0 ? K : group_size);
  const int G = (int)(K / gsz);
  // Rows per workgroup: the fewest of 16, 32, 48 and 64 whose workgroups all
  // run at once (one per CU), so that a layer spreads over as many CUs as it
  // can (the product part shrinks with the rows; the column walk does not
  // change); 64 for taller layers.
  const int qmax = (1 << bits) - 1, qlo = sym ? 1 : 0;
  const int cus = device_cu_count();
  if ((n + 15) / 16 <= cus)
    hipLaunchKernelGGL(gptq_rows_kernel<16>, dim3((n + 15) / 16), dim3(kRowThreads), 0, stream, w,
                       n, k, A, scales, zeros, G, gsz, qmax, qlo, DT, out_codes);
  else if ((n + 31) / 32 <= cus)
    hipLaunchKernelGGL(gptq_rows_kernel<32>, dim3((n + 31) / 32), dim3(kRowThreads), 0, stream, w, n, k, A,
                       scales, zeros, G, gsz, qmax, qlo, DT, out_codes);
  else if ((n + 47) / 48 <= cus)
    hipLaunchKernelGGL(gptq_rows_kernel<48>, dim3((n + 47) / 48), dim3(kRowThreads), 0, stream, w,
                       n, k, A, scales, zeros, G, gsz, qmax, qlo, DT, out_codes);
  else
    hipLaunchKernelGGL(gptq_rows_kernel<kRows>, dim3((n + kRows - 1) / kRows), dim3(kRowThreads), 0,
                       stream, w, n, k, A, scales, zeros, G, gsz, qmax, qlo, DT, out_codes);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (packed) return launch_pack(out_codes, N, K, bits, packed, stream);
  return hipSuccess;
}

}  // namespace lowbit
