// C ABI of the GPTQ-2D library (declared in include/gptq2d.h): argument checks on the
// host, workspace carve-up, and the factor -> sweep call sequence on one stream.
#include <hip/hip_runtime.h>

#include "../../include/gptq2d.h"
#include "launch.hpp"

using g2d::align_up;

namespace {

bool bad_dtype(int dtype) { return dtype != GPTQ2D_F32 && dtype != GPTQ2D_F64; }

// Largest problem edge accepted: keeps every 64-bit offset and every grid dimension in
// range (grid.y of the elementwise kernels is p/4 <= 65535 requires p <= 262140).
constexpr int64_t kMaxDim = 262140;

// Stream-ordered scratch: the caller's buffer, or one allocated (and freed) on stream.
struct Scratch {
  void* ptr = nullptr;
  bool owned = false;
  hipStream_t s = nullptr;
  int acquire(void* user, size_t user_bytes, size_t need, hipStream_t stream) {
    s = stream;
    if (user != nullptr) {
      ptr = user;
      return 0;
    }
    if (need == 0) return 0;
    if (hipMallocAsync(&ptr, need, stream) != hipSuccess) {
      (void)hipGetLastError();
      return GPTQ2D_ERR_ALLOC;
    }
    owned = true;
    (void)user_bytes;
    return 0;
  }
  ~Scratch() {
    if (owned) (void)hipFreeAsync(ptr, s);
  }
};

__global__ void k_clear_info(int* info) {
  if (threadIdx.x < 2) info[threadIdx.x] = 0;
}

// A fill kernel rather than a memset node, so the call can be captured into a graph.
int clear_info(int* info, hipStream_t s) {
  if (info == nullptr) return 0;
  k_clear_info<<<1, 64, 0, s>>>(info);
  return hipGetLastError() == hipSuccess ? 0 : GPTQ2D_ERR_HIP;
}

int status(hipError_t e) { return e == hipSuccess ? 0 : GPTQ2D_ERR_HIP; }

}  // namespace

extern "C" {

size_t gptq2d_factor_workspace_bytes(int64_t p, int dtype) {
  if (p <= 0 || p > kMaxDim || bad_dtype(dtype)) return 0;
  return g2d::factor_workspace(p);
}

int gptq2d_factor(int64_t p, int dtype, const void* A, void* U_unit, void* workspace,
                  size_t workspace_bytes, int* info, void* stream) {
  if (p <= 0 || p > kMaxDim) return -1;
  if (bad_dtype(dtype)) return -2;
  if (A == nullptr) return -3;
  if (U_unit == nullptr) return -4;
  const size_t need = g2d::factor_workspace(p);
  if (workspace != nullptr && workspace_bytes < need) return -6;
  if (workspace == nullptr && workspace_bytes != 0) return -6;
  hipStream_t s = (hipStream_t)stream;
  Scratch ws;
  int rc = ws.acquire(workspace, workspace_bytes, need, s);
  if (rc) return rc;
  if ((rc = clear_info(info, s))) return rc;
  return status(g2d::factor_enqueue(p, dtype, A, U_unit, ws.ptr, info, 1, s));
}

size_t gptq2d_sweep_workspace_bytes(int64_t m, int64_t n, int dtype) {
  if (m <= 0 || n <= 0 || m > kMaxDim || n > kMaxDim || bad_dtype(dtype)) return 0;
  return g2d::sweep_workspace(m, n, dtype);
}

int gptq2d_quantize_factored(int64_t m, int64_t n, int bits, int dtype, const void* W,
                             const void* Ua_unit, const void* Ub_unit, const void* scales,
                             int8_t* codes, void* Q, void* workspace, size_t workspace_bytes,
                             int* info, void* stream) {
  if (m <= 0 || m > kMaxDim) return -1;
  if (n <= 0 || n > kMaxDim) return -2;
  if (bits < 2 || bits > 8) return -3;
  if (bad_dtype(dtype)) return -4;
  if (W == nullptr) return -5;
  if (Ua_unit == nullptr) return -6;
  if (Ub_unit == nullptr) return -7;
  if (scales == nullptr) return -8;
  if (codes == nullptr) return -9;
  if (Q == nullptr) return -10;
  const size_t need = g2d::sweep_workspace(m, n, dtype);
  if (workspace != nullptr && workspace_bytes < need) return -12;
  if (workspace == nullptr && workspace_bytes != 0) return -12;
  hipStream_t s = (hipStream_t)stream;
  Scratch ws;
  int rc = ws.acquire(workspace, workspace_bytes, need, s);
  if (rc) return rc;
  if ((rc = clear_info(info, s))) return rc;
  return status(g2d::sweep_enqueue(m, n, bits, dtype, W, Ua_unit, Ub_unit, scales, codes, Q,
                                   ws.ptr, info, s));
}

size_t gptq2d_workspace_bytes(int64_t m, int64_t n, int dtype) {
  if (m <= 0 || n <= 0 || m > kMaxDim || n > kMaxDim || bad_dtype(dtype)) return 0;
  const size_t es = dtype == GPTQ2D_F32 ? sizeof(float) : sizeof(double);
  const size_t fa = g2d::factor_workspace(m), fb = g2d::factor_workspace(n);
  const size_t sw = g2d::sweep_workspace(m, n, dtype);
  size_t scratch = fa > fb ? fa : fb;
  if (sw > scratch) scratch = sw;
  return align_up((size_t)m * m * es) + align_up((size_t)n * n * es) + scratch;
}

int gptq2d_quantize(int64_t m, int64_t n, int bits, int dtype, const void* W, const void* A,
                    const void* B, const void* scales, int8_t* codes, void* Q, void* workspace,
                    size_t workspace_bytes, int* info, void* stream) {
  if (m <= 0 || m > kMaxDim) return -1;
  if (n <= 0 || n > kMaxDim) return -2;
  if (bits < 2 || bits > 8) return -3;
  if (bad_dtype(dtype)) return -4;
  if (W == nullptr) return -5;
  if (A == nullptr) return -6;
  if (B == nullptr) return -7;
  if (scales == nullptr) return -8;
  if (codes == nullptr) return -9;
  if (Q == nullptr) return -10;
  const size_t need = gptq2d_workspace_bytes(m, n, dtype);
  if (workspace != nullptr && workspace_bytes < need) return -12;
  if (workspace == nullptr && workspace_bytes != 0) return -12;
  hipStream_t s = (hipStream_t)stream;
  Scratch ws;
  int rc = ws.acquire(workspace, workspace_bytes, need, s);
  if (rc) return rc;
  if ((rc = clear_info(info, s))) return rc;
  const size_t es = dtype == GPTQ2D_F32 ? sizeof(float) : sizeof(double);
  char* c = (char*)ws.ptr;
  void* Ua = c;
  c += align_up((size_t)m * m * es);
  void* Ub = c;
  c += align_up((size_t)n * n * es);
  void* scratch = c;
  hipError_t e = g2d::factor_enqueue(m, dtype, A, Ua, scratch, info, 1, s);
  if (e == hipSuccess) e = g2d::factor_enqueue(n, dtype, B, Ub, scratch, info, 2, s);
  if (e == hipSuccess)
    e = g2d::sweep_enqueue(m, n, bits, dtype, W, Ua, Ub, scales, codes, Q, scratch, info, s);
  return status(e);
}

const char* gptq2d_strerror(int st) {
  if (st == 0) return "success";
  if (st < 0) return "invalid argument (the negated value is the 1-based argument index)";
  if (st == GPTQ2D_ERR_HIP) return "HIP runtime error while enqueuing work";
  if (st == GPTQ2D_ERR_ALLOC) return "device allocation of the workspace failed";
  return "unknown status";
}

}  // extern "C"
