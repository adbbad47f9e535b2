// Packed storage of the integer codes and its dequantising consumers.
//
// The quantizer's output is an integer matrix ("GPTQ-2D: Cubic-Time Two-Sided Adaptive
// Rounding", arxivlens page, Abstract); the pages define no storage format.  Format: a code
// z in [lo, hi] = [-2^(bits-1), 2^(bits-1)-1] is the field u = z - lo; row r is one
// little-endian bit string in which code c occupies bits c*bits .. c*bits+bits-1; the row is
// held in wpr = ceil(n*bits/32) uint32 words, padding bits zero.  All three kernels are
// HBM-bound elementwise passes.
#include <hip/hip_runtime.h>

#include "launch.hpp"
#include "prof.hpp"

namespace g2d {
namespace {

// Every kernel takes the field width as a template argument, so the divisions and shifts by
// `bits` compile to constants, and a 2-D grid (x: position in the row, y: rows, strided), so
// no thread divides by the row length.  Rows are at most 2^31 bits long (checked on the
// host), so positions within a row are 32-bit.

// One thread per packed word: the fields that overlap bits [32w, 32w+32) of its row are read
// from the int8 codes (adjacent threads read adjacent code ranges) and assembled; a field
// that straddles two words gives its low part to the first and its high part to the second.
// Codes outside [lo, hi] are stored modulo 2^bits.
// With VEC (bits 2, 4 or 8, whose fields never straddle words, a row length that is a
// multiple of 32/bits and aligned codes, checked on the host) the word's 32/bits codes are
// one vector load.
template <int BITS, bool VEC>
__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ codes,
                                              uint32_t* __restrict__ packed, int64_t rows,
                                              int n, int wpr) {
  constexpr int lo = -(1 << (BITS - 1));
  constexpr unsigned mask = (1u << BITS) - 1u;
  const int w = blockIdx.x * 256 + threadIdx.x;
  if (w >= wpr) return;
  if constexpr (VEC && 32 % BITS == 0) {
    constexpr int K = 32 / BITS;  // codes per word: 16, 8 or 4 bytes
    typedef int8_t vec_t __attribute__((ext_vector_type(K)));
    for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
      const vec_t v = *(const vec_t*)(codes + r * n + (int64_t)w * K);
      uint32_t word = 0;
#pragma unroll
      for (int k = 0; k < K; ++k) word |= ((unsigned)((int)v[k] - lo) & mask) << (k * BITS);
      packed[r * wpr + w] = word;
    }
    return;
  }
  const int bit0 = 32 * w;
  const int c0 = bit0 / BITS;                           // first field overlapping the word
  const int c1 = min((bit0 + 32 + BITS - 1) / BITS, n);  // one past the last one
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    const int8_t* row = codes + r * n;
    uint32_t word = 0;
#pragma unroll
    for (int k = 0; k < 32 / BITS + 2; ++k) {
      const int c = c0 + k;
      if (c < c1) {
        const unsigned u = (unsigned)((int)row[c] - lo) & mask;
        const int off = c * BITS - bit0;  // negative for a field begun in the previous word
        word |= off >= 0 ? u << off : u >> (-off);
      }
    }
    packed[r * wpr + w] = word;
  }
}

// The 64-bit window of words (w, w+1) of a row that holds the four fields from code c on
// (4*bits <= 32 bits starting at bit (c*bits) % 32 of word w), and the offset in it.
template <int BITS>
__device__ inline uint64_t window(const uint32_t* __restrict__ row, int c, int wpr, int& sh) {
  const int pos = c * BITS, w = pos >> 5;
  sh = pos & 31;
  return (uint64_t)row[w] | (w + 1 < wpr ? (uint64_t)row[w + 1] << 32 : 0ull);
}

// Q = s * (u + lo): one thread per two consecutive entries of a row, written with one
// two-element store when VEC (even n and an aligned Q, checked on the host).
template <int BITS, typename T, bool VEC>
__global__ __launch_bounds__(256) void k_unpack(const uint32_t* __restrict__ packed,
                                                const T* __restrict__ scales, T* __restrict__ Q,
                                                int64_t rows, int n, int wpr) {
  constexpr int lo = -(1 << (BITS - 1));
  constexpr unsigned mask = (1u << BITS) - 1u;
  const int c = 2 * (blockIdx.x * 256 + threadIdx.x);
  if (c >= n) return;
  for (int64_t r = blockIdx.y; r < rows; r += gridDim.y) {
    int sh;
    const uint64_t win = window<BITS>(packed + r * wpr, c, wpr, sh);
    const T sr = scales[r];
    const T q0 = sr * (T)((int)((unsigned)(win >> sh) & mask) + lo);
    const T q1 = sr * (T)((int)((unsigned)(win >> (sh + BITS)) & mask) + lo);
    T* q = Q + r * n + c;
    if (VEC) {
      typedef T pair_t __attribute__((ext_vector_type(2)));
      pair_t v;
      v.x = q0;
      v.y = q1;
      *(pair_t*)q = v;
    } else {
      q[0] = q0;
      if (c + 1 < n) q[1] = q1;
    }
  }
}

constexpr int kMaxBatch = 8;

// Y[b][r] = s[r] * sum_c z[r][c] * X[b][c]: one wave per row.  Lane l decodes the four
// consecutive codes c = 4l + 256k .. 4l + 256k + 3, four values of k per trip with the word
// windows of all four loaded first.  With VEC (n a multiple of 4 and X 4-element aligned,
// checked on the host) the four X values of a lane are one vector load, so a wave reads one
// contiguous, fully used range of X per load.  Per-lane sums are combined by a butterfly
// over the wave.
template <int BITS, typename T, bool VEC>
__global__ __launch_bounds__(256) void k_packed_gemv(const uint32_t* __restrict__ packed,
                                                     const T* __restrict__ scales,
                                                     const T* __restrict__ X, T* __restrict__ Y,
                                                     int64_t rows, int n, int wpr, int batch) {
  constexpr int lo = -(1 << (BITS - 1));
  constexpr unsigned mask = (1u << BITS) - 1u;
  typedef T quad_t __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const uint32_t* row = packed + r * wpr;
  T acc[kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) acc[b] = T(0);
  for (int cb = 4 * lane; cb < n; cb += 1024) {
    uint64_t win[4];
    int sh[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = cb + 256 * k;
      win[k] = c < n ? window<BITS>(row, c, wpr, sh[k]) : (sh[k] = 0, 0ull);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int c = cb + 256 * k;
      if (c >= n) continue;
      T z[4];
#pragma unroll
      for (int j = 0; j < 4; ++j)
        z[j] = (T)((int)((unsigned)(win[k] >> (sh[k] + j * BITS)) & mask) + lo);
#pragma unroll
      for (int b = 0; b < kMaxBatch; ++b) {
        if (b < batch) {
          const T* xb = X + (int64_t)b * n + c;
          if (VEC) {
            const quad_t x = *(const quad_t*)xb;
            acc[b] += z[0] * x.x;
            acc[b] += z[1] * x.y;
            acc[b] += z[2] * x.z;
            acc[b] += z[3] * x.w;
          } else {
#pragma unroll
            for (int j = 0; j < 4; ++j)
              if (c + j < n) acc[b] += z[j] * xb[j];
          }
        }
      }
    }
  }
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) {
    T v = acc[b];
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    if (b < batch && lane == 0) Y[(int64_t)b * rows + r] = scales[r] * v;
  }
}

template <template <int> class F, typename... Args>
hipError_t by_bits(int bits, Args... args) {
  switch (bits) {
    case 2: return F<2>::run(args...);
    case 3: return F<3>::run(args...);
    case 4: return F<4>::run(args...);
    case 5: return F<5>::run(args...);
    case 6: return F<6>::run(args...);
    case 7: return F<7>::run(args...);
    case 8: return F<8>::run(args...);
  }
  return hipErrorInvalidValue;
}

unsigned grid_rows(int64_t rows) { return (unsigned)(rows < 65535 ? rows : 65535); }

template <int BITS>
struct PackLaunch {
  static hipError_t run(int64_t rows, int n, int wpr, const int8_t* codes, uint32_t* packed,
                        hipStream_t s) {
    const dim3 grid((unsigned)cdiv(wpr, 256), grid_rows(rows));
    const int K = 32 / BITS;
    if (32 % BITS == 0 && n % K == 0 && (uintptr_t)codes % K == 0)
      k_pack<BITS, true><<<grid, 256, 0, s>>>(codes, packed, rows, n, wpr);
    else
      k_pack<BITS, false><<<grid, 256, 0, s>>>(codes, packed, rows, n, wpr);
    return hipGetLastError();
  }
};

template <int BITS>
struct UnpackLaunch {
  static hipError_t run(int64_t rows, int n, int wpr, int dtype, const uint32_t* packed,
                        const void* scales, void* Q, hipStream_t s) {
    const dim3 grid((unsigned)cdiv(cdiv(n, 2), 256), grid_rows(rows));
    const bool vec = n % 2 == 0 && (uintptr_t)Q % (dtype == 0 ? 8 : 16) == 0;
    if (dtype == 0) {
      if (vec)
        k_unpack<BITS, float, true><<<grid, 256, 0, s>>>(packed, (const float*)scales,
                                                          (float*)Q, rows, n, wpr);
      else
        k_unpack<BITS, float, false><<<grid, 256, 0, s>>>(packed, (const float*)scales,
                                                           (float*)Q, rows, n, wpr);
    } else {
      if (vec)
        k_unpack<BITS, double, true><<<grid, 256, 0, s>>>(packed, (const double*)scales,
                                                           (double*)Q, rows, n, wpr);
      else
        k_unpack<BITS, double, false><<<grid, 256, 0, s>>>(packed, (const double*)scales,
                                                            (double*)Q, rows, n, wpr);
    }
    return hipGetLastError();
  }
};

template <int BITS>
struct GemvLaunch {
  template <typename T, bool VEC>
  static void go(unsigned blocks, const uint32_t* packed, const void* scales, const void* X,
                 void* Y, int64_t rows, int n, int wpr, int batch, hipStream_t s) {
    k_packed_gemv<BITS, T, VEC><<<blocks, 256, 0, s>>>(packed, (const T*)scales, (const T*)X,
                                                       (T*)Y, rows, n, wpr, batch);
  }
  static hipError_t run(int64_t rows, int n, int wpr, int dtype, const uint32_t* packed,
                        const void* scales, int batch, const void* X, void* Y, hipStream_t s) {
    const unsigned blocks = (unsigned)cdiv(rows, 4);
    const bool vec = n % 4 == 0 && (uintptr_t)X % (dtype == 0 ? 16 : 32) == 0;
    if (dtype == 0) {
      if (vec)
        go<float, true>(blocks, packed, scales, X, Y, rows, n, wpr, batch, s);
      else
        go<float, false>(blocks, packed, scales, X, Y, rows, n, wpr, batch, s);
    } else {
      if (vec)
        go<double, true>(blocks, packed, scales, X, Y, rows, n, wpr, batch, s);
      else
        go<double, false>(blocks, packed, scales, X, Y, rows, n, wpr, batch, s);
    }
    return hipGetLastError();
  }
};

}  // namespace

int64_t packed_row_words(int64_t n, int bits) { return (n * bits + 31) / 32; }

// Rows longer than 2^31 - 1 bits, or grids beyond the launch limits, are rejected.
static bool fits(int64_t rows, int64_t n, int bits) {
  return n * bits < ((int64_t)1 << 31) - 32 && cdiv(rows, 4) <= 0x7FFFFFFF;
}

hipError_t pack_enqueue(int64_t rows, int64_t n, int bits, const int8_t* codes,
                        uint32_t* packed, hipStream_t s) {
  if (!fits(rows, n, bits)) return hipErrorInvalidValue;
  const int64_t wpr = packed_row_words(n, bits);
  prof_begin(KC_PACK, s);
  const hipError_t e = by_bits<PackLaunch>(bits, rows, (int)n, (int)wpr, codes, packed, s);
  prof_end(KC_PACK, s, 0.0, (double)rows * (double)n + 4.0 * (double)rows * (double)wpr);
  return e;
}

hipError_t unpack_enqueue(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                          const void* scales, void* Q, hipStream_t s) {
  if (!fits(rows, n, bits)) return hipErrorInvalidValue;
  const int64_t wpr = packed_row_words(n, bits);
  const double es = dtype == 0 ? 4.0 : 8.0;
  prof_begin(KC_PACK, s);
  const hipError_t e =
      by_bits<UnpackLaunch>(bits, rows, (int)n, (int)wpr, dtype, packed, scales, Q, s);
  prof_end(KC_PACK, s, (double)rows * (double)n,
           4.0 * (double)rows * (double)wpr + es * (double)rows * ((double)n + 1.0));
  return e;
}

hipError_t packed_gemv_enqueue(int64_t rows, int64_t n, int bits, int dtype,
                               const uint32_t* packed, const void* scales, int batch,
                               const void* X, void* Y, hipStream_t s) {
  if (batch < 1 || batch > kMaxBatch || !fits(rows, n, bits)) return hipErrorInvalidValue;
  const int64_t wpr = packed_row_words(n, bits);
  const double es = dtype == 0 ? 4.0 : 8.0;
  prof_begin(KC_PACK, s);
  const hipError_t e = by_bits<GemvLaunch>(bits, rows, (int)n, (int)wpr, dtype, packed, scales,
                                           batch, X, Y, s);
  prof_end(KC_PACK, s, 2.0 * (double)batch * (double)rows * (double)n,
           4.0 * (double)rows * (double)wpr +
               es * ((double)rows + (double)batch * ((double)n + (double)rows)));
  return e;
}

}  // namespace g2d
