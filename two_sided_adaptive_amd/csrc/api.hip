// C ABI of the GPTQ-2D library (declared in include/gptq2d.h): argument checks on the
// host, workspace carve-up, and the factor -> sweep call sequence on one stream.
#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "../../include/gptq2d.h"
#include "launch.hpp"
#include "prof.hpp"

using g2d::align_up;

// ---------------------------------------------------------------------------
// measurement hook (see prof.hpp)
// ---------------------------------------------------------------------------
namespace g2d {
namespace {

struct Pending {
  int cls;
  hipEvent_t a, b;
  double flops, bytes;
};

struct ProfState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> pool;
  std::vector<Pending> pending;
  hipEvent_t open[KC_COUNT] = {};
  double ms[KC_COUNT] = {}, flops[KC_COUNT] = {}, bytes[KC_COUNT] = {};
  int64_t launches[KC_COUNT] = {};
  // band-update tasks per task class (near, next, far) in the window of the last read
  double last_task_ms[kTaskClasses] = {}, last_task_flops[kTaskClasses] = {};
  int64_t last_task_n[kTaskClasses] = {};
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    hipEvent_t e = nullptr;
    (void)hipEventCreate(&e);
    return e;
  }
};

ProfState& prof() {
  static ProfState st;
  return st;
}

}  // namespace

bool prof_on() { return prof().on; }

void prof_begin(int cls, hipStream_t s) {
  ProfState& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> g(p.mu);
  hipEvent_t e = p.get();
  (void)hipEventRecord(e, s);
  p.open[cls] = e;
}

void prof_end(int cls, hipStream_t s, double flops, double bytes) {
  ProfState& p = prof();
  if (!p.on) return;
  std::lock_guard<std::mutex> g(p.mu);
  hipEvent_t e = p.get();
  (void)hipEventRecord(e, s);
  p.pending.push_back(Pending{cls, p.open[cls], e, flops, bytes});
  p.open[cls] = nullptr;
}

}  // namespace g2d

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

// Factor A and B (one persistent launch), then the sweep, on stream s, with the workspace
// at ws (at least gptq2d_workspace_bytes(m, n, dtype) bytes, 256-byte aligned).
int quantize_enqueue(int64_t m, int64_t n, int bits, int dtype, const void* W, const void* A,
                     const void* B, const void* scales, int8_t* codes, void* Q, void* ws,
                     int* info, hipStream_t s) {
  const size_t es = dtype == GPTQ2D_F32 ? sizeof(float) : sizeof(double);
  char* c = (char*)ws;
  void* Ua = c;
  c += align_up((size_t)m * m * es);
  void* Ub = c;
  c += align_up((size_t)n * n * es);
  void* scratch_a = c;
  void* scratch_b = c + g2d::factor_workspace(m);
  hipError_t e =
      g2d::factor_pair_enqueue(m, A, Ua, scratch_a, n, B, Ub, scratch_b, dtype, info, s);
  if (e == hipSuccess)
    e = g2d::sweep_enqueue(m, n, bits, dtype, W, Ua, Ub, scales, codes, Q, c, info, s);
  return status(e);
}

// ---------------------------------------------------------------------------
// static scratch of gptq2d_quantize_noalloc
// ---------------------------------------------------------------------------
// One buffer per device, in the code object's device memory: it exists on every device the
// library runs on until the process ends, and the entry point never allocates.  In host
// code `scratch` names a host-side stand-in, not device memory: its device address is
// looked up once per device (scratch_address) and only that address is used.
constexpr size_t kNoAllocBytes = (size_t)GPTQ2D_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

// Device address of this device's scratch buffer (looked up on the first call on a device,
// with that device current).
int scratch_address(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GPTQ2D_ERR_HIP;
  std::lock_guard<std::mutex> g(g_scratch_mu);
  if (g_scratch_dev[dev] == nullptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || ptr == nullptr) {
      (void)hipGetLastError();
      return GPTQ2D_ERR_HIP;
    }
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return 0;
}

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
  size_t scratch = fa + fb;  // the two factorisations run concurrently
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
  // Both factors in one persistent launch, then the sweep, on the caller's stream.
  return quantize_enqueue(m, n, bits, dtype, W, A, B, scales, codes, Q, ws.ptr, info, s);
}

int gptq2d_quantize_noalloc(int64_t m, int64_t n, int bits, int dtype, const void* W,
                            const void* A, const void* B, const void* scales, int8_t* codes,
                            void* Q, int* info, void* stream) {
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
  if (gptq2d_workspace_bytes(m, n, dtype) > kNoAllocBytes) return GPTQ2D_ERR_SCRATCH;
  void* ws = nullptr;
  int rc = scratch_address(&ws);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  if ((rc = clear_info(info, s))) return rc;
  // every counter, flag and accumulator the kernels read before writing is cleared (or
  // stored before it is read) by the launches themselves, so the previous call's contents
  // of the buffer do not matter
  return quantize_enqueue(m, n, bits, dtype, W, A, B, scales, codes, Q, ws, info, s);
}

size_t gptq2d_workspace3_bytes(int64_t m1, int64_t m2, int64_t m3, int dtype) {
  if (m1 <= 0 || m2 <= 0 || m3 <= 0 || m1 > kMaxDim || m2 > kMaxDim || m3 > kMaxDim ||
      bad_dtype(dtype))
    return 0;
  return g2d::kron3_workspace(m1, m2, m3, dtype);
}

int gptq2d_quantize3(int64_t m1, int64_t m2, int64_t m3, int bits, int dtype, const void* W,
                     const void* A1, const void* A2, const void* A3, const void* scales,
                     int8_t* codes, void* Q, void* workspace, size_t workspace_bytes, int* info,
                     void* stream) {
  if (m1 <= 0 || m1 > kMaxDim) return -1;
  if (m2 <= 0 || m2 > kMaxDim) return -2;
  if (m3 <= 0 || m3 > kMaxDim) return -3;
  if (bits < 2 || bits > 8) return -4;
  if (bad_dtype(dtype)) return -5;
  if (W == nullptr) return -6;
  if (A1 == nullptr) return -7;
  if (A2 == nullptr) return -8;
  if (A3 == nullptr) return -9;
  if (scales == nullptr) return -10;
  if (codes == nullptr) return -11;
  if (Q == nullptr) return -12;
  const size_t need = gptq2d_workspace3_bytes(m1, m2, m3, dtype);
  if (workspace != nullptr && workspace_bytes < need) return -14;
  if (workspace == nullptr && workspace_bytes != 0) return -14;
  hipStream_t s = (hipStream_t)stream;
  Scratch ws;
  int rc = ws.acquire(workspace, workspace_bytes, need, s);
  if (rc) return rc;
  if ((rc = clear_info(info, s))) return rc;
  return status(g2d::kron3_enqueue(m1, m2, m3, bits, dtype, W, A1, A2, A3, scales, codes, Q,
                                   ws.ptr, info, s));
}

size_t gptq2d_packed_row_words(int64_t n, int bits) {
  if (n <= 0 || n > ((int64_t)1 << 40) || bits < 2 || bits > 8) return 0;
  return (size_t)g2d::packed_row_words(n, bits);
}

int gptq2d_pack(int64_t rows, int64_t n, int bits, const int8_t* codes, uint32_t* packed,
                void* stream) {
  if (rows <= 0 || rows > ((int64_t)1 << 40)) return -1;
  if (n <= 0 || n > ((int64_t)1 << 40)) return -2;
  if (bits < 2 || bits > 8) return -3;
  if (codes == nullptr) return -4;
  if (packed == nullptr) return -5;
  return status(g2d::pack_enqueue(rows, n, bits, codes, packed, (hipStream_t)stream));
}

int gptq2d_unpack(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                  const void* scales, void* Q, void* stream) {
  if (rows <= 0 || rows > ((int64_t)1 << 40)) return -1;
  if (n <= 0 || n > ((int64_t)1 << 40)) return -2;
  if (bits < 2 || bits > 8) return -3;
  if (bad_dtype(dtype)) return -4;
  if (packed == nullptr) return -5;
  if (scales == nullptr) return -6;
  if (Q == nullptr) return -7;
  return status(g2d::unpack_enqueue(rows, n, bits, dtype, packed, scales, Q, (hipStream_t)stream));
}

int gptq2d_packed_gemv(int64_t rows, int64_t n, int bits, int dtype, const uint32_t* packed,
                       const void* scales, int batch, const void* X, void* Y, void* stream) {
  if (rows <= 0 || rows > ((int64_t)1 << 40)) return -1;
  if (n <= 0 || n > ((int64_t)1 << 40)) return -2;
  if (bits < 2 || bits > 8) return -3;
  if (bad_dtype(dtype)) return -4;
  if (packed == nullptr) return -5;
  if (scales == nullptr) return -6;
  if (batch < 1 || batch > 8) return -7;
  if (X == nullptr) return -8;
  if (Y == nullptr) return -9;
  return status(g2d::packed_gemv_enqueue(rows, n, bits, dtype, packed, scales, batch, X, Y,
                                         (hipStream_t)stream));
}

int gptq2d_gram_accumulate(int64_t p, int64_t N, int dtype, const void* X, double alpha,
                           void* A, void* stream) {
  if (p <= 0 || p > kMaxDim) return -1;
  if (N <= 0) return -2;
  if (bad_dtype(dtype)) return -3;
  if (X == nullptr) return -4;
  if (!(alpha == alpha) || alpha == 1.0 / 0.0 || alpha == -1.0 / 0.0) return -5;
  if (A == nullptr) return -6;
  return status(g2d::gram_enqueue(p, N, dtype, X, alpha, A, (hipStream_t)stream));
}

int gptq2d_gram_accumulate_batched(int count, const int64_t* p, const int64_t* N, int dtype,
                                   const void* const* X, const double* alpha, void* const* A,
                                   void* stream) {
  if (count <= 0) return -1;
  if (p == nullptr) return -2;
  if (N == nullptr) return -3;
  if (bad_dtype(dtype)) return -4;
  if (X == nullptr) return -5;
  if (alpha == nullptr) return -6;
  if (A == nullptr) return -7;
  for (int l = 0; l < count; ++l) {
    if (p[l] <= 0 || p[l] > kMaxDim) return -2;
    if (N[l] <= 0) return -3;
    if (X[l] == nullptr) return -5;
    if (!(alpha[l] == alpha[l]) || alpha[l] == 1.0 / 0.0 || alpha[l] == -1.0 / 0.0) return -6;
    if (A[l] == nullptr) return -7;
  }
  for (int l = 0; l < count; ++l) {
    const hipError_t e = g2d::gram_enqueue(p[l], N[l], dtype, X[l], alpha[l], A[l],
                                           (hipStream_t)stream);
    if (e != hipSuccess) return status(e);
  }
  return 0;
}

int gptq2d_profile_enable(int on) {
  g2d::ProfState& p = g2d::prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return 0;
}

int gptq2d_profile_read(int n_classes, double* ms, int64_t* launches, double* flops,
                        double* bytes) {
  if (n_classes < 0) return -1;
  g2d::ProfState& p = g2d::prof();
  std::lock_guard<std::mutex> g(p.mu);
  int rc = 0;
  for (const g2d::Pending& e : p.pending) {
    float t = 0.f;
    if (hipEventSynchronize(e.b) != hipSuccess || hipEventElapsedTime(&t, e.a, e.b) != hipSuccess)
      rc = GPTQ2D_ERR_HIP;
    p.ms[e.cls] += t;
    p.flops[e.cls] += e.flops;
    p.bytes[e.cls] += e.bytes;
    p.launches[e.cls] += 1;
    p.pool.push_back(e.a);
    p.pool.push_back(e.b);
  }
  p.pending.clear();
  {
    double cu_ms[g2d::kTaskClasses] = {}, fl[g2d::kTaskClasses] = {};
    int64_t tasks[g2d::kTaskClasses] = {};
    if (g2d::band_stats_collect(cu_ms, fl, tasks) != hipSuccess) rc = GPTQ2D_ERR_HIP;
    for (int c = 0; c < g2d::kTaskClasses; ++c) {
      p.ms[g2d::KC_BAND_GEMM] += cu_ms[c];
      p.flops[g2d::KC_BAND_GEMM] += fl[c];
      p.launches[g2d::KC_BAND_GEMM] += tasks[c];
      p.last_task_ms[c] = cu_ms[c];
      p.last_task_flops[c] = fl[c];
      p.last_task_n[c] = tasks[c];
    }
  }
  const int n = n_classes < g2d::KC_COUNT ? n_classes : g2d::KC_COUNT;
  for (int c = 0; c < n; ++c) {
    if (ms) ms[c] = p.ms[c];
    if (launches) launches[c] = p.launches[c];
    if (flops) flops[c] = p.flops[c];
    if (bytes) bytes[c] = p.bytes[c];
  }
  for (int c = 0; c < g2d::KC_COUNT; ++c) {
    p.ms[c] = p.flops[c] = p.bytes[c] = 0.0;
    p.launches[c] = 0;
  }
  return rc;
}

int gptq2d_profile_task_classes(int n_classes, double* cu_ms, int64_t* tasks, double* flops) {
  if (n_classes < 0) return -1;
  g2d::ProfState& p = g2d::prof();
  std::lock_guard<std::mutex> g(p.mu);
  const int n = n_classes < g2d::kTaskClasses ? n_classes : g2d::kTaskClasses;
  for (int c = 0; c < n; ++c) {
    if (cu_ms) cu_ms[c] = p.last_task_ms[c];
    if (tasks) tasks[c] = p.last_task_n[c];
    if (flops) flops[c] = p.last_task_flops[c];
  }
  return 0;
}

const char* gptq2d_profile_class_name(int cls) {
  static const char* names[g2d::KC_COUNT] = {"sweep", "band_gemm", "factor", "other",
                                                  "slab_feedback", "packed", "gram"};
  return (cls >= 0 && cls < g2d::KC_COUNT) ? names[cls] : "unknown";
}

const char* gptq2d_strerror(int st) {
  if (st == 0) return "success";
  if (st < 0) return "invalid argument (the negated value is the 1-based argument index)";
  if (st == GPTQ2D_ERR_HIP) return "HIP runtime error while enqueuing work";
  if (st == GPTQ2D_ERR_ALLOC) return "device allocation of the workspace failed";
  if (st == GPTQ2D_ERR_SCRATCH)
    return "the problem needs more workspace than the static scratch buffer of "
           "gptq2d_quantize_noalloc holds (GPTQ2D_NOALLOC_SCRATCH_BYTES)";
  return "unknown status";
}

}  // extern "C"
