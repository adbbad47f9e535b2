// Shared device helpers for the gfx950 GPTQ-2D library: MFMA operand types and a
// 64x64 tile GEMM used by the factor stage and the band updates.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace g2d {

constexpr int kTile = 64;      // output tile edge of the tile GEMM
constexpr int kKc = 32;        // K chunk staged through LDS per iteration
constexpr int kPad = 4;        // LDS row padding (elements)
constexpr int kThreads = 256;  // 4 wave64s per workgroup

template <typename T>
struct Mfma;

// v_mfma_f32_16x16x4_f32: D(16x16) += A(16x4) B(4x16).  Lane l supplies A[l%16][l/16]
// and B[l/16][l%16]; acc[e] holds D[row(l, e)][l%16] with row = 4*(l/16) + e.
template <>
struct Mfma<float> {
  typedef float acc_t __attribute__((ext_vector_type(4)));
  __device__ static inline acc_t run(float a, float b, acc_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline int row(int lane, int e) { return 4 * (lane >> 4) + e; }
};

// v_mfma_f64_16x16x4_f64: same A and B operand layout with doubles, but the
// accumulator is interleaved: acc[e] holds D[4*e + l/16][l%16].
template <>
struct Mfma<double> {
  typedef double acc_t __attribute__((ext_vector_type(4)));
  __device__ static inline acc_t run(double a, double b, acc_t c) {
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
  }
  __device__ static inline int row(int lane, int e) { return 4 * e + (lane >> 4); }
};

template <typename T>
struct TileSmem {
  T a[kKc][kTile + kPad];  // op(A) chunk, stored k-major: a[k][i]
  T b[kKc][kTile + kPad];  // op(B) chunk: b[k][j]
};

// C[0:M,0:N] = beta*C + alpha * sum_{k in [k0,k1)} op(A)[i][k] op(B)[k][j] for one 64x64
// tile.  Pointers are already offset to the tile origin (A at row 0 of the tile, B at
// column 0); M, N <= 64 are the valid extents.  op(A)[i][k] = TA ? A[k*lda+i] :
// A[i*lda+k]; op(B)[k][j] = TB ? B[j*ldb+k] : B[k*ldb+j].  beta == 0 never reads C.
// Called by all 256 threads of the workgroup.
template <typename T, bool TA, bool TB>
__device__ inline void tile_gemm(const T* A, int64_t lda, const T* B,
                                 int64_t ldb, T* C, int64_t ldc, int M, int N, int k0, int k1,
                                 T alpha, T beta, TileSmem<T>& sm) {
  typedef typename Mfma<T>::acc_t acc_t;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int wr = w >> 1, wc = w & 1;
  acc_t acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b) acc[a][b] = acc_t{0, 0, 0, 0};

  for (int kb = k0; kb < k1; kb += kKc) {
    const int kc = (k1 - kb) < kKc ? (k1 - kb) : kKc;
    // stage op(A): 64 x kKc
    if (TA) {
      const int k = tid >> 3, i8 = (tid & 7) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = i8 + u;
        sm.a[k][i] = (k < kc && i < M) ? A[(int64_t)(kb + k) * lda + i] : T(0);
      }
    } else {
      const int i = tid >> 2, k8 = (tid & 3) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k8 + u;
        sm.a[k][i] = (k < kc && i < M) ? A[(int64_t)i * lda + kb + k] : T(0);
      }
    }
    // stage op(B): kKc x 64
    if (TB) {
      const int j = tid >> 2, k8 = (tid & 3) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int k = k8 + u;
        sm.b[k][j] = (k < kc && j < N) ? B[(int64_t)j * ldb + kb + k] : T(0);
      }
    } else {
      const int k = tid >> 3, j8 = (tid & 7) * 8;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int j = j8 + u;
        sm.b[k][j] = (k < kc && j < N) ? B[(int64_t)(kb + k) * ldb + j] : T(0);
      }
    }
    __syncthreads();
    const int kr = lane >> 4, cl = lane & 15;
#pragma unroll 2
    for (int kk = 0; kk < kKc; kk += 4) {
      T av[2], bv[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        av[t] = sm.a[kk + kr][32 * wr + 16 * t + cl];
        bv[t] = sm.b[kk + kr][32 * wc + 16 * t + cl];
      }
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b) acc[a][b] = Mfma<T>::run(av[a], bv[b], acc[a][b]);
    }
    __syncthreads();
  }
  const int cl = lane & 15;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 32 * wr + 16 * a + Mfma<T>::row(lane, e);
        const int j = 32 * wc + 16 * b + cl;
        if (i < M && j < N) {
          T* p = C + (int64_t)i * ldc + j;
          const T v = alpha * acc[a][b][e];
          *p = (beta == T(0)) ? v : v + beta * (*p);
        }
      }
}

__device__ inline void record_info(int* info, int code, int index) {
  if (info == nullptr) return;
  if (atomicCAS(info, 0, code) == 0) info[1] = index;
}

}  // namespace g2d
