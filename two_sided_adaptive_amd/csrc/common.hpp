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

// Raw buffer loads: a descriptor covers [base, base + bytes); element offsets past the
// end read as zero (hardware range check), so guarded loads need no branch and many
// stay in flight.  Word 3 of the descriptor is the gfx9 raw-buffer configuration.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ inline rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0,
                                           (int)(bytes > 0 ? bytes : 0), 0x00020000);
}
template <typename T>
__device__ inline T buf_load(rsrc_t r, uint32_t elem);
template <>
__device__ inline float buf_load<float>(rsrc_t r, uint32_t elem) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, 0, 0));
}
template <>
__device__ inline double buf_load<double>(rsrc_t r, uint32_t elem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, 0, 0);
  return __hiloint2double((int)v[1], (int)v[0]);
}
// Same with a wave-uniform element offset `uelem` added through the scalar offset field.
template <typename T>
__device__ inline T buf_load_s(rsrc_t r, uint32_t elem, uint32_t uelem);
template <>
__device__ inline float buf_load_s<float>(rsrc_t r, uint32_t elem, uint32_t uelem) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, elem * 4u, uelem * 4u, 0));
}
template <>
__device__ inline double buf_load_s<double>(rsrc_t r, uint32_t elem, uint32_t uelem) {
  const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, elem * 8u, uelem * 8u, 0);
  return __hiloint2double((int)v[1], (int)v[0]);
}

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

  // operand ranges end at the last valid element, so k-major reads past row k1 are
  // zero; for i-major views the k-tail is masked explicitly; rows/columns past M/N
  // read neighbouring data that only feeds outputs which are never stored
  const int64_t es = sizeof(T);
  const rsrc_t ra = TA ? make_rsrc(A, ((int64_t)(k1 - 1) * lda + M) * es)
                       : make_rsrc(A, ((int64_t)(M - 1) * lda + k1) * es);
  const rsrc_t rb = TB ? make_rsrc(B, ((int64_t)(N - 1) * ldb + k1) * es)
                       : make_rsrc(B, ((int64_t)(k1 - 1) * ldb + N) * es);
  for (int kb = k0; kb < k1; kb += kKc) {
    // stage op(A): 64 x kKc
    if (TA) {
      const int k = tid >> 3, i8 = (tid & 7) * 8;
      T v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = buf_load<T>(ra, (uint32_t)((int64_t)(kb + k) * lda + i8 + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) sm.a[k][i8 + u] = v[u];
    } else {
      const int i = tid >> 2, k8 = (tid & 3) * 8;
      T v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = buf_load<T>(ra, (uint32_t)((int64_t)i * lda + kb + k8 + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) sm.a[k8 + u][i] = (kb + k8 + u < k1) ? v[u] : T(0);
    }
    // stage op(B): kKc x 64
    if (TB) {
      const int j = tid >> 2, k8 = (tid & 3) * 8;
      T v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = buf_load<T>(rb, (uint32_t)((int64_t)j * ldb + kb + k8 + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) sm.b[k8 + u][j] = (kb + k8 + u < k1) ? v[u] : T(0);
    } else {
      const int k = tid >> 3, j8 = (tid & 7) * 8;
      T v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = buf_load<T>(rb, (uint32_t)((int64_t)(kb + k) * ldb + j8 + u));
#pragma unroll
      for (int u = 0; u < 8; ++u) sm.b[k][j8 + u] = v[u];
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
  const rsrc_t rc = make_rsrc(C, ((int64_t)(M - 1) * ldc + N) * es);
  T old[2][2][4];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 32 * wr + 16 * a + Mfma<T>::row(lane, e), j = 32 * wc + 16 * b + cl;
        old[a][b][e] = (beta == T(0)) ? T(0) : buf_load<T>(rc, (uint32_t)((int64_t)i * ldc + j));
      }
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 32 * wr + 16 * a + Mfma<T>::row(lane, e), j = 32 * wc + 16 * b + cl;
        if (i < M && j < N) C[(int64_t)i * ldc + j] = alpha * acc[a][b][e] + beta * old[a][b][e];
      }
}

__device__ inline void record_info(int* info, int code, int index) {
  if (info == nullptr) return;
  if (atomicCAS(info, 0, code) == 0) info[1] = index;
}

}  // namespace g2d
