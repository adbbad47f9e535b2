// Internal host-side interface between the C ABI (api.hip) and the kernel files.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>


namespace g2d {

constexpr size_t kAlign = 256;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Factor stage (factor.hip): U' (dtype) of one SPD matrix A (dtype), fp64 inside.
size_t factor_workspace(int64_t p);
hipError_t factor_enqueue(int64_t p, int dtype, const void* A, void* U, void* ws, int* info,
                          int side_code, hipStream_t s);
// Both factors at once, in one persistent launch on s: A (m x m) and B (n x n); info codes
// code_a for A and code_b for B.
hipError_t factor_pair_enqueue(int64_t m, const void* A, void* Ua, void* ws_a, int64_t n,
                               const void* B, void* Ub, void* ws_b, int dtype, int* info,
                               hipStream_t s, int code_a = 1, int code_b = 2);

// info codes of the three-factor call: a non-SPD A1, A2 or A3.
constexpr int kInfoA1 = 5, kInfoA2 = 6, kInfoA3 = 7;

// Sweep stage (sweep.hip): codes/Q from W, U'_a, U'_b, scales (all dtype).
size_t sweep_workspace(int64_t m, int64_t n, int dtype);
hipError_t sweep_enqueue(int64_t m, int64_t n, int bits, int dtype, const void* W,
                         const void* Ua, const void* Ub, const void* scales, int8_t* codes,
                         void* Q, void* ws, int* info, hipStream_t s);

// Three Kronecker factors (kron3.hip): codes/Q of an m1 x m2 x m3 tensor (all dtype).
size_t kron3_workspace(int64_t m1, int64_t m2, int64_t m3, int dtype);
hipError_t kron3_enqueue(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const void* W,
                         const void* A1, const void* A2, const void* A3, const void* scales,
                         int8_t* codes, void* Q, void* ws, int* info, hipStream_t s);

// Packed codes (pack.hip): ceil(n*bits/32) uint32 words per row.
int64_t packed_row_words(int64_t n, int bits);
hipError_t pack_enqueue(int64_t rows, int64_t n, int bits, const int8_t* codes,
                        uint32_t* packed, hipStream_t s);
hipError_t unpack_enqueue(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                          const void* scales, void* Q, hipStream_t s);
hipError_t packed_gemv_enqueue(int64_t rows, int64_t n, int bits, int dtype,
                               const uint32_t* packed, const void* scales, int batch,
                               const void* X, void* Y, hipStream_t s);

// Kronecker factor accumulation (gram.hip): A (p x p, symmetric) += alpha X^T X, X N x p.
hipError_t gram_enqueue(int64_t p, int64_t N, int dtype, const void* X, double alpha, void* A,
                        hipStream_t s);

}  // namespace g2d
