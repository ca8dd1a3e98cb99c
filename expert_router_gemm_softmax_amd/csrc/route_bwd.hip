// Router backward (B1, with the gradient unpermute-sum B2 fused in).  The
// router is a shared parameter with an ordinary gradient ("GPU expert
// parallel", section "Sharded by expert, replicated everywhere else");
// index, top-k and capacity steps are piecewise constant and pass no
// gradient.
//   dp[t, idx[t,j]] = dgate[t,j] for kept j;  dz = p * (dp - sum_e p dp)
//   dX  = sum_{kept j} dXp[row_of[t,j]] + dz Wr^T
//   dWr = x^T dz,  db = sum_t dz
// dWr and db are reduced in fixed order (split over token chunks, then a
// sequential sum over the chunks): bitwise deterministic.
#include "common.h"

namespace moe {

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, hipStream_t s);

namespace {

constexpr int kDxTok = 16;   // tokens per block in the dX kernel
constexpr int kDwE = 64;     // experts per block in the dWr kernel
constexpr int kDwChunk = 64; // tokens staged per LDS chunk in the dWr kernel

__global__ __launch_bounds__(256) void route_bwd_dz_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_of, const float* __restrict__ dgate,
    float* __restrict__ dz, int64_t T_, int E, int k) {
  const int lane = threadIdx.x & 63;
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * 4) {
    float p[4], dp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      p[i] = e < E ? probs[t * E + e] : 0.0f;
      dp[i] = 0.0f;
    }
    for (int j = 0; j < k; ++j) {
      if (row_of[t * k + j] < 0) continue;
      const int e = idx[t * k + j];
      const float g = dgate[t * k + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (e == lane + 64 * i) dp[i] = g;
    }
    float sp = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sp += p[i] * dp[i];
    sp = wave_sum(sp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      if (e < E) dz[t * E + e] = p[i] * (dp[i] - sp);
    }
  }
}

// dX[t][i] = sum_j dXp[row][i] + sum_e dz[t][e] wrT[e][i]
template <typename T>
__global__ __launch_bounds__(256) void route_bwd_dx_kernel(
    const float* __restrict__ dz, const T* __restrict__ wrT, const T* __restrict__ dXp,
    const int32_t* __restrict__ row_of, T* __restrict__ dX, int64_t T_, int d, int E,
    int k) {
  extern __shared__ float sdz[];  // [kDxTok][E]
  int32_t* srow = reinterpret_cast<int32_t*>(sdz + kDxTok * E);  // [kDxTok][k]
  const int64_t t0 = (int64_t)blockIdx.x * kDxTok;
  for (int o = threadIdx.x; o < kDxTok * E; o += 256) {
    const int tt = o / E;
    sdz[o] = t0 + tt < T_ ? dz[t0 * E + o] : 0.0f;
  }
  for (int o = threadIdx.x; o < kDxTok * k; o += 256) {
    const int tt = o / k;
    srow[o] = t0 + tt < T_ ? row_of[t0 * k + o] : -1;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d; i += 256) {
    float acc[kDxTok];
#pragma unroll
    for (int tt = 0; tt < kDxTok; ++tt) acc[tt] = 0.0f;
    for (int e = 0; e < E; ++e) {
      const float w = St<T>::to_f(wrT[(int64_t)e * d + i]);
#pragma unroll
      for (int tt = 0; tt < kDxTok; ++tt) acc[tt] += sdz[tt * E + e] * w;
    }
#pragma unroll
    for (int tt = 0; tt < kDxTok; ++tt) {
      const int64_t t = t0 + tt;
      if (t >= T_) break;
      float sum = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int32_t r = srow[tt * k + j];
        if (r >= 0) sum += St<T>::to_f(dXp[(int64_t)r * d + i]);
      }
      dX[t * d + i] = St<T>::from_f(sum + acc[tt]);
    }
  }
}

// partial[sp][i][e] = sum_{t in split sp} x[t][i] dz[t][e];
// dbp[sp][e] = sum_{t in split sp} dz[t][e]
template <typename T>
__global__ __launch_bounds__(256) void route_bwd_dw_kernel(
    const T* __restrict__ x, const float* __restrict__ dz, float* __restrict__ part,
    float* __restrict__ dbp, int64_t T_, int d, int E) {
  __shared__ float sdz[kDwChunk][kDwE];
  const int sp = blockIdx.x;
  const int i = blockIdx.y * 256 + threadIdx.x;
  const int e0 = blockIdx.z * kDwE;
  const int ne = min(kDwE, E - e0);
  const int64_t tbeg = (int64_t)sp * kDwrRows;
  const int64_t tend = min<int64_t>(tbeg + kDwrRows, T_);
  float acc[kDwE];
#pragma unroll
  for (int q = 0; q < kDwE; ++q) acc[q] = 0.0f;
  float dbacc = 0.0f;
  for (int64_t tc = tbeg; tc < tend; tc += kDwChunk) {
    const int nt = (int)min<int64_t>(kDwChunk, tend - tc);
    for (int o = threadIdx.x; o < kDwChunk * kDwE; o += 256) {
      const int tt = o / kDwE, q = o % kDwE;
      sdz[tt][q] = (tt < nt && q < ne) ? dz[(tc + tt) * E + e0 + q] : 0.0f;
    }
    __syncthreads();
    if (i < d) {
      for (int tt = 0; tt < nt; ++tt) {
        const float xv = St<T>::to_f(x[(tc + tt) * d + i]);
#pragma unroll
        for (int q = 0; q < kDwE; ++q) acc[q] += xv * sdz[tt][q];
      }
    }
    if (blockIdx.y == 0 && threadIdx.x < ne)
      for (int tt = 0; tt < nt; ++tt) dbacc += sdz[tt][threadIdx.x];
    __syncthreads();
  }
  if (i < d) {
    float* o = part + ((int64_t)sp * d + i) * E + e0;
#pragma unroll
    for (int q = 0; q < kDwE; ++q)
      if (q < ne) o[q] = acc[q];
  }
  if (blockIdx.y == 0 && threadIdx.x < ne) dbp[(int64_t)sp * E + e0 + threadIdx.x] = dbacc;
}

template <typename T>
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ dbp, T* __restrict__ dWr,
    float* __restrict__ db, int nsplit, int d, int E) {
  const int64_t n = (int64_t)d * E;
  for (int64_t o = blockIdx.x * 256 + threadIdx.x; o < n; o += (int64_t)gridDim.x * 256) {
    float s = 0.0f;
    for (int sp = 0; sp < nsplit; ++sp) s += part[(int64_t)sp * n + o];
    dWr[o] = St<T>::from_f(s);
  }
  if (blockIdx.x == 0 && db != nullptr)
    for (int e = threadIdx.x; e < E; e += 256) {
      float s = 0.0f;
      for (int sp = 0; sp < nsplit; ++sp) s += dbp[(int64_t)sp * E + e];
      db[e] = s;
    }
}

template <typename T>
int route_bwd_t(const moe_cfg& c, const T* x, const T* Wr, const float* probs,
                const int32_t* idx, const int32_t* row_of, const float* dgate,
                const T* dXp, T* dX, T* dWr, float* db, void* ws, hipStream_t s) {
  const WsLayout L = ws_layout(c);
  float* dz = ws_ptr<float>(ws, L.dz);
  T* wrT = ws_ptr<T>(ws, L.wrT);
  float* part = ws_ptr<float>(ws, L.dwr_part);
  float* dbp = ws_ptr<float>(ws, L.db_part);
  int rc = launch_transpose_wr(c, Wr, wrT, s);
  if (rc != MOE_OK) return rc;
  if (c.T > 0) {
    const int g1 = (int)std::min<int64_t>(ceil_div(c.T, 4), 65536);
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DZ, s,
               route_bwd_dz_kernel<<<g1, 256, 0, s>>>(probs, idx, row_of, dgate, dz, c.T,
                                                      c.E, c.k));
    const int g2 = (int)ceil_div(c.T, kDxTok);
    const size_t sm2 = (size_t)kDxTok * c.E * 4 + (size_t)kDxTok * c.k * 4;
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DX, s,
               route_bwd_dx_kernel<T><<<g2, 256, sm2, s>>>(dz, wrT, dXp, row_of, dX, c.T,
                                                          c.d, c.E, c.k));
  }
  const int nsplit = c.T > 0 ? (int)ceil_div(c.T, kDwrRows) : 0;
  if (nsplit > 0) {
    dim3 g3(nsplit, (unsigned)ceil_div(c.d, 256), (unsigned)ceil_div(c.E, kDwE));
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DW, s,
               route_bwd_dw_kernel<T><<<g3, 256, 0, s>>>(x, dz, part, dbp, c.T, c.d, c.E));
  }
  const int g4 = (int)std::min<int64_t>(ceil_div((int64_t)c.d * c.E, 256), 4096);
  MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DW, s,
             route_bwd_reduce_kernel<T><<<g4, 256, 0, s>>>(part, dbp, dWr, db, nsplit, c.d,
                                                          c.E));
  return MOE_OK;
}

}  // namespace

int launch_route_bwd(const moe_cfg& c, const void* x, const void* Wr,
                     const float* probs, const int32_t* idx, const int32_t* row_of,
                     const float* dgate, const void* dXp, void* dX, void* dWr, float* db,
                     void* ws, hipStream_t s) {
  if (c.dtype == MOE_BF16)
    return route_bwd_t<uint16_t>(c, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(Wr), probs, idx, row_of, dgate,
                                 static_cast<const uint16_t*>(dXp),
                                 static_cast<uint16_t*>(dX), static_cast<uint16_t*>(dWr), db,
                                 ws, s);
  return route_bwd_t<float>(c, static_cast<const float*>(x), static_cast<const float*>(Wr),
                            probs, idx, row_of, dgate, static_cast<const float*>(dXp),
                            static_cast<float*>(dX), static_cast<float*>(dWr), db, ws, s);
}

}  // namespace moe
