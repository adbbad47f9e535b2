// Sweep stage for gfx950: anti-diagonal two-sided adaptive rounding with
// separable band feedback.
//
// Page reference: arxivlens page "GPTQ-2D: Cubic-Time Two-Sided Adaptive Rounding",
// Results (entries of one anti-diagonal are independent and are rounded together;
// feedback is rank-one and separable, realised by a few band-like matrix products),
// Methodology (anti-diagonal rounds with a buffer of accumulated feedback), Abstract
// (two levels of blocking); mind-verse article, section "Die algorithmische Neuerung
// und ihre Auswirkungen" (anti-diagonal processing, parallel inside each one).
//
// With unit factors U'a, U'b the rounding target of entry (k,l) is
//   t[k,l] = W[k,l] - sum_{i<k} U'a[i,k] R[i,l] - sum_{j<l} Delta[k,j] U'b[j,l]
// where R (vertical residual) = W - G - Q and Delta = t - Q.  (k,l) depends only on
// entries above it in its column and left of it in its row, so every anti-diagonal
// is an antichain.
//
// Blocking (64 x 64 blocks, outer blocks of G x G blocks):
//   * k_round rounds all blocks of one block anti-diagonal; inside a block the four
//     waves own 16-row micro-rows and walk 16x16 micro-tiles along micro anti-
//     diagonals; feedback between micro-tiles is an MFMA product from LDS, feedback
//     inside a micro-tile is applied entry by entry along its 31 anti-diagonal steps.
//   * k_band applies the band feedback of the finished blocks to the blocks below
//     (Wg -= U'a^T R) and to the right (Hc += Delta U'b): within an outer block with
//     the 64-deep panel of one block, across outer blocks with the whole outer block
//     as the inner dimension once its last block is done.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"

namespace g2d {
namespace {

constexpr int BB = 64;   // block edge
constexpr int MU = 16;   // micro-tile edge
constexpr int GOUT = 4;  // blocks per outer block edge (outer block = 256)

template <typename T>
struct RoundSmem {
  T ua[BB][BB + 1];       // diagonal block of U'a
  T ub[BB][BB + 1];       // diagonal block of U'b
  T rr[BB][BB + 1];       // R of this block
  T dd[BB][BB + 1];       // Delta of this block
  T g0[4][MU][MU + 1];    // per wave: W - G(outside micro-tile) of the current micro-tile
  T h0[4][MU][MU + 1];    // per wave: H(outside micro-tile)
  T sc[BB];
};

__device__ inline void wave_lds_fence() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ inline float rint_t(float x) { return rintf(x); }
__device__ inline double rint_t(double x) { return rint(x); }

template <typename T>
__global__ __launch_bounds__(256) void k_round(int64_t m, int64_t n, int D, int Mb, int Nb,
                                               int lo, int hi, const T* __restrict__ Ua,
                                               const T* __restrict__ Ub,
                                               const T* __restrict__ scales,
                                               const T* __restrict__ Wg, const T* __restrict__ Hc,
                                               T* __restrict__ R, T* __restrict__ Dl,
                                               int8_t* __restrict__ codes, T* __restrict__ Q) {
  typedef typename Mfma<T>::acc_t acc_t;
  __shared__ RoundSmem<T> sm;
  const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
  const int K = kmin + blockIdx.x;
  const int L = D - K;
  const int64_t r0 = (int64_t)K * BB, c0 = (int64_t)L * BB;
  const int mr = (m - r0) < BB ? (int)(m - r0) : BB;
  const int nc = (n - c0) < BB ? (int)(n - c0) : BB;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int r = lane & 15, q = lane >> 4;

  for (int idx = tid; idx < BB * BB; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    sm.ua[i][j] = (i < mr && j < mr) ? Ua[(r0 + i) * m + r0 + j] : T(0);
    sm.ub[i][j] = (i < nc && j < nc) ? Ub[(c0 + i) * n + c0 + j] : T(0);
    sm.rr[i][j] = T(0);
    sm.dd[i][j] = T(0);
  }
  if (tid < BB) sm.sc[tid] = tid < mr ? scales[r0 + tid] : T(1);
  __syncthreads();

  const int gr = MU * w + r;  // block row handled by this lane in the micro sweep
  const T s_r = sm.sc[gr];
  const T tlo = T(lo), thi = T(hi);
  T cu[4];  // in-micro-tile vertical coefficients U'a[i][r], rows i above r
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = 4 * q + u;
    cu[u] = (i < r) ? sm.ua[MU * w + i][MU * w + r] : T(0);
  }

  for (int d = 0; d < 2 * (BB / MU) - 1; ++d) {
    const int j = d - w;  // micro-column of this wave's micro-tile (wave-uniform)
    if (j >= 0 && j < BB / MU) {
      const int mc0 = MU * j;
      // outside-micro-tile feedback: V = U'a[rows above]^T R, H = Delta[left] U'b
      T wv[4], hv[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = MU * w + Mfma<T>::row(lane, e), c = mc0 + (lane & 15);
        const bool ok = i < mr && c < nc;
        wv[e] = ok ? Wg[(r0 + i) * n + c0 + c] : T(0);
        hv[e] = ok ? Hc[(r0 + i) * n + c0 + c] : T(0);
      }
      acc_t av = acc_t{0, 0, 0, 0}, ah = acc_t{0, 0, 0, 0};
      for (int k0 = 0; k0 < MU * w; k0 += 4) {
        const T a = sm.ua[k0 + (lane >> 4)][MU * w + (lane & 15)];
        const T b = sm.rr[k0 + (lane >> 4)][mc0 + (lane & 15)];
        av = Mfma<T>::run(a, b, av);
      }
      for (int k0 = 0; k0 < mc0; k0 += 4) {
        const T a = sm.dd[MU * w + (lane & 15)][k0 + (lane >> 4)];
        const T b = sm.ub[k0 + (lane >> 4)][mc0 + (lane & 15)];
        ah = Mfma<T>::run(a, b, ah);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sm.g0[w][Mfma<T>::row(lane, e)][lane & 15] = wv[e] - av[e];
        sm.h0[w][Mfma<T>::row(lane, e)][lane & 15] = hv[e] + ah[e];
      }
      wave_lds_fence();
      // micro sweep: step st handles the micro anti-diagonal r + l = st
      for (int st = 0; st < 2 * MU - 1; ++st) {
        const int l = st - r;
        const bool act = (l >= 0) && (l < MU);
        const int lc = act ? l : 0;
        T pv = T(0), ph = T(0);
#pragma unroll
        for (int u = 0; u < 4; ++u) pv += cu[u] * sm.rr[MU * w + 4 * q + u][mc0 + lc];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int jj = 4 * q + u;
          const T cb = (jj < lc) ? sm.ub[mc0 + jj][mc0 + lc] : T(0);
          ph += sm.dd[gr][mc0 + jj] * cb;
        }
        pv += __shfl_xor(pv, 16);
        pv += __shfl_xor(pv, 32);
        ph += __shfl_xor(ph, 16);
        ph += __shfl_xor(ph, 32);
        const T g = sm.g0[w][r][lc] - pv;
        const T h = sm.h0[w][r][lc] + ph;
        const T t = g - h;
        T z = rint_t(t / s_r);
        z = z < tlo ? tlo : (z > thi ? thi : z);
        const T qv = s_r * z;
        if (act && q == 0) {
          sm.rr[gr][mc0 + l] = g - qv;
          sm.dd[gr][mc0 + l] = t - qv;
          if (gr < mr && mc0 + l < nc) {
            const int64_t o = (r0 + gr) * n + c0 + mc0 + l;
            codes[o] = (int8_t)(int)z;
            Q[o] = qv;
          }
        }
        wave_lds_fence();
      }
    }
    __syncthreads();
  }
  for (int idx = tid; idx < BB * BB; idx += 256) {
    const int i = idx >> 6, j = idx & 63;
    if (i < mr && j < nc) {
      R[(r0 + i) * n + c0 + j] = sm.rr[i][j];
      Dl[(r0 + i) * n + c0 + j] = sm.dd[i][j];
    }
  }
}

// Band feedback of the blocks on anti-diagonal D.  z = 0: vertical, target row block
// t = K+1+x of column L; z = 1: horizontal, target column block t = L+1+x of row K.
template <typename T>
__global__ __launch_bounds__(256) void k_band(int64_t m, int64_t n, int D, int Mb, int Nb,
                                              const T* Ua, const T* Ub, const T* R, const T* Dl,
                                              T* Wg, T* Hc) {
  __shared__ TileSmem<T> sm;
  const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
  const int K = kmin + blockIdx.y;
  const int L = D - K;
  if (blockIdx.z == 0) {
    const int t = K + 1 + blockIdx.x;
    if (t >= Mb) return;
    int64_t src0;
    int ks;
    if (t / GOUT == K / GOUT) {
      src0 = (int64_t)K * BB;
    } else if (K % GOUT == GOUT - 1) {
      src0 = (int64_t)(K - (GOUT - 1)) * BB;
    } else {
      return;
    }
    const int64_t send = (int64_t)(K + 1) * BB < m ? (int64_t)(K + 1) * BB : m;
    ks = (int)(send - src0);
    const int64_t tr0 = (int64_t)t * BB, c0 = (int64_t)L * BB;
    const int M = (m - tr0) < BB ? (int)(m - tr0) : BB;
    const int N = (n - c0) < BB ? (int)(n - c0) : BB;
    tile_gemm<T, true, false>(Ua + src0 * m + tr0, m, R + src0 * n + c0, n, Wg + tr0 * n + c0, n, M,
                              N, 0, ks, T(-1), T(1), sm);
  } else {
    const int t = L + 1 + blockIdx.x;
    if (t >= Nb) return;
    int64_t src0;
    if (t / GOUT == L / GOUT) {
      src0 = (int64_t)L * BB;
    } else if (L % GOUT == GOUT - 1) {
      src0 = (int64_t)(L - (GOUT - 1)) * BB;
    } else {
      return;
    }
    const int64_t send = (int64_t)(L + 1) * BB < n ? (int64_t)(L + 1) * BB : n;
    const int ks = (int)(send - src0);
    const int64_t r0 = (int64_t)K * BB, tc0 = (int64_t)t * BB;
    const int M = (m - r0) < BB ? (int)(m - r0) : BB;
    const int N = (n - tc0) < BB ? (int)(n - tc0) : BB;
    tile_gemm<T, false, false>(Dl + r0 * n + src0, n, Ub + src0 * n + tc0, n, Hc + r0 * n + tc0, n,
                               M, N, 0, ks, T(1), T(1), sm);
  }
}

// Wg = W, Hc = 0.
template <typename T>
__global__ __launch_bounds__(256) void k_init(int64_t count, const T* __restrict__ W,
                                              T* __restrict__ Wg, T* __restrict__ Hc) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < count;
       i += (int64_t)gridDim.x * 256) {
    Wg[i] = W[i];
    Hc[i] = T(0);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_check_scales(int64_t m, const T* __restrict__ s,
                                                      int* info) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= m) return;
  const T v = s[i];
  if (!(v > T(0)) || !isfinite(v)) record_info(info, 3, (int)(i + 1));
}

template <typename T>
hipError_t sweep_typed(int64_t m, int64_t n, int bits, const T* W, const T* Ua, const T* Ub,
                       const T* scales, int8_t* codes, T* Q, void* ws, int* info, hipStream_t s) {
  const size_t mn = (size_t)m * n;
  char* c = (char*)ws;
  T* Wg = (T*)c;
  c += align_up(mn * sizeof(T));
  T* Hc = (T*)c;
  c += align_up(mn * sizeof(T));
  T* R = (T*)c;
  c += align_up(mn * sizeof(T));
  T* Dl = (T*)c;
  const int lo = -(1 << (bits - 1)), hi = (1 << (bits - 1)) - 1;
  const int Mb = (int)cdiv(m, BB), Nb = (int)cdiv(n, BB);
  k_check_scales<T><<<(unsigned)cdiv(m, 256), 256, 0, s>>>(m, scales, info);
  const int64_t ig = cdiv((int64_t)mn, 256) < 8192 ? cdiv((int64_t)mn, 256) : 8192;
  k_init<T><<<(unsigned)ig, 256, 0, s>>>((int64_t)mn, W, Wg, Hc);
  const int maxt = (Mb > Nb ? Mb : Nb) - 1;
  for (int D = 0; D <= Mb + Nb - 2; ++D) {
    const int kmin = D - (Nb - 1) > 0 ? D - (Nb - 1) : 0;
    const int kmax = D < Mb - 1 ? D : Mb - 1;
    const int nblk = kmax - kmin + 1;
    k_round<T><<<nblk, 256, 0, s>>>(m, n, D, Mb, Nb, lo, hi, Ua, Ub, scales, Wg, Hc, R, Dl, codes,
                                    Q);
    if (D < Mb + Nb - 2 && maxt > 0)
      k_band<T><<<dim3(maxt, nblk, 2), 256, 0, s>>>(m, n, D, Mb, Nb, Ua, Ub, R, Dl, Wg, Hc);
  }
  return hipGetLastError();
}

}  // namespace

size_t sweep_workspace(int64_t m, int64_t n, int dtype) {
  const size_t es = dtype == 0 ? sizeof(float) : sizeof(double);
  return 4 * align_up((size_t)m * n * es);
}

hipError_t sweep_enqueue(int64_t m, int64_t n, int bits, int dtype, const void* W,
                         const void* Ua, const void* Ub, const void* scales, int8_t* codes,
                         void* Q, void* ws, int* info, hipStream_t s) {
  if (dtype == 0)
    return sweep_typed<float>(m, n, bits, (const float*)W, (const float*)Ua, (const float*)Ub,
                              (const float*)scales, codes, (float*)Q, ws, info, s);
  return sweep_typed<double>(m, n, bits, (const double*)W, (const double*)Ua, (const double*)Ub,
                             (const double*)scales, codes, (double*)Q, ws, info, s);
}

}  // namespace g2d
