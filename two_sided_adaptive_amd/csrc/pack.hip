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

// One thread per packed word: the fields that overlap bits [32w, 32w+32) of its row are
// read from the int8 codes (adjacent threads read adjacent code ranges) and assembled.
// A field that straddles two words contributes its low part to the first and its high part
// to the second.  Codes outside [lo, hi] are stored modulo 2^bits.
__global__ __launch_bounds__(256) void k_pack(const int8_t* __restrict__ codes,
                                              uint32_t* __restrict__ packed, int64_t rows,
                                              int64_t n, int bits, int64_t wpr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * wpr) return;
  const int64_t r = idx / wpr, w = idx - r * wpr;
  const int lo = -(1 << (bits - 1));
  const unsigned mask = (1u << bits) - 1u;
  const int64_t bit0 = 32 * w;
  int64_t c = bit0 / bits;                      // first field overlapping the word
  int64_t c_end = (bit0 + 32 + bits - 1) / bits;  // one past the last one
  if (c_end > n) c_end = n;
  const int8_t* row = codes + r * n;
  uint32_t word = 0;
  for (; c < c_end; ++c) {
    const unsigned u = (unsigned)((int)row[c] - lo) & mask;
    const int64_t off = c * bits - bit0;  // may be negative for the first field
    if (off >= 0)
      word |= u << off;
    else
      word |= u >> (-off);
  }
  packed[idx] = word;
}

__device__ inline unsigned field(const uint32_t* __restrict__ row, int64_t c, int bits,
                                 int64_t wpr) {
  const int64_t pos = c * bits;
  const int64_t w = pos >> 5;
  const int sh = (int)(pos & 31);
  unsigned v = row[w] >> sh;
  if (sh + bits > 32 && w + 1 < wpr) v |= row[w + 1] << (32 - sh);
  return v & ((1u << bits) - 1u);
}

// Q = s * (u + lo): one thread per entry (coalesced stores; adjacent lanes share words).
template <typename T>
__global__ __launch_bounds__(256) void k_unpack(const uint32_t* __restrict__ packed,
                                                const T* __restrict__ scales, T* __restrict__ Q,
                                                int64_t rows, int64_t n, int bits, int64_t wpr) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * n) return;
  const int64_t r = idx / n, c = idx - r * n;
  const int lo = -(1 << (bits - 1));
  const int z = (int)field(packed + r * wpr, c, bits, wpr) + lo;
  Q[idx] = scales[r] * (T)z;
}

constexpr int kMaxBatch = 8;

// Y[b][r] = s[r] * sum_c z[r][c] * X[b][c]: one wave per row.  Lane l takes the four
// consecutive codes c = 4l + 256k .. 4l + 256k + 3 (so the X loads of a wave cover one
// contiguous range); their 4*bits <= 32 bits lie in at most two adjacent words, read as one
// 64-bit window.  Per-lane sums are combined by a butterfly over the wave.
template <typename T>
__global__ __launch_bounds__(256) void k_packed_gemv(const uint32_t* __restrict__ packed,
                                                     const T* __restrict__ scales,
                                                     const T* __restrict__ X, T* __restrict__ Y,
                                                     int64_t rows, int64_t n, int bits,
                                                     int64_t wpr, int batch) {
  const int lane = threadIdx.x & 63;
  const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lo = -(1 << (bits - 1));
  const unsigned mask = (1u << bits) - 1u;
  const uint32_t* row = packed + r * wpr;
  T acc[kMaxBatch];
#pragma unroll
  for (int b = 0; b < kMaxBatch; ++b) acc[b] = T(0);
  for (int64_t c = 4 * (int64_t)lane; c < n; c += 256) {
    const int64_t pos = c * bits, w = pos >> 5;
    const int sh = (int)(pos & 31);
    const uint64_t win = (uint64_t)row[w] | (w + 1 < wpr ? (uint64_t)row[w + 1] << 32 : 0ull);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c + j < n) {
        const T z = (T)((int)((unsigned)(win >> (sh + j * bits)) & mask) + lo);
#pragma unroll
        for (int b = 0; b < kMaxBatch; ++b)
          if (b < batch) acc[b] += z * X[(int64_t)b * n + c + j];
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

}  // namespace

int64_t packed_row_words(int64_t n, int bits) { return (n * bits + 31) / 32; }

hipError_t pack_enqueue(int64_t rows, int64_t n, int bits, const int8_t* codes,
                        uint32_t* packed, hipStream_t s) {
  const int64_t wpr = packed_row_words(n, bits);
  const int64_t blocks = cdiv(rows * wpr, 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  prof_begin(KC_PACK, s);
  k_pack<<<(unsigned)blocks, 256, 0, s>>>(codes, packed, rows, n, bits, wpr);
  prof_end(KC_PACK, s, 0.0, (double)rows * (double)n + 4.0 * (double)rows * (double)wpr);
  return hipGetLastError();
}

hipError_t unpack_enqueue(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                          const void* scales, void* Q, hipStream_t s) {
  const int64_t wpr = packed_row_words(n, bits);
  const int64_t blocks = cdiv(rows * n, 256);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const double es = dtype == 0 ? 4.0 : 8.0;
  prof_begin(KC_PACK, s);
  if (dtype == 0)
    k_unpack<float><<<(unsigned)blocks, 256, 0, s>>>(packed, (const float*)scales, (float*)Q,
                                                      rows, n, bits, wpr);
  else
    k_unpack<double><<<(unsigned)blocks, 256, 0, s>>>(packed, (const double*)scales,
                                                       (double*)Q, rows, n, bits, wpr);
  prof_end(KC_PACK, s, (double)rows * (double)n,
           4.0 * (double)rows * (double)wpr + es * (double)rows * ((double)n + 1.0));
  return hipGetLastError();
}

hipError_t packed_gemv_enqueue(int64_t rows, int64_t n, int bits, int dtype,
                               const uint32_t* packed, const void* scales, int batch,
                               const void* X, void* Y, hipStream_t s) {
  if (batch < 1 || batch > kMaxBatch) return hipErrorInvalidValue;
  const int64_t wpr = packed_row_words(n, bits);
  const int64_t blocks = cdiv(rows, 4);
  if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
  const double es = dtype == 0 ? 4.0 : 8.0;
  prof_begin(KC_PACK, s);
  if (dtype == 0)
    k_packed_gemv<float><<<(unsigned)blocks, 256, 0, s>>>(
        packed, (const float*)scales, (const float*)X, (float*)Y, rows, n, bits, wpr, batch);
  else
    k_packed_gemv<double><<<(unsigned)blocks, 256, 0, s>>>(
        packed, (const double*)scales, (const double*)X, (double*)Y, rows, n, bits, wpr, batch);
  prof_end(KC_PACK, s, 2.0 * (double)batch * (double)rows * (double)n,
           4.0 * (double)rows * (double)wpr +
               es * ((double)rows + (double)batch * ((double)n + (double)rows)));
  return hipGetLastError();
}

}  // namespace g2d
