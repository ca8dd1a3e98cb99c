// Gate-weighted combine (F5), its backward (B5) and the gradient
// unpermute-sum (B2).  The inverse of the permutation returns expert
// outputs to token order ("GPU expert parallel", section "The step
// timeline"); backward retraces it.  All three are HBM-bound gathers:
// one wave per token, one 16-byte vector per lane per step, fp32 math.
#include "common.h"

namespace moe {
namespace {

constexpr int kCW = 4;  // waves per block

// out[t] = sum over kept j (ascending) of gate[t,j] * Y[row_of[t,j]]
template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(
    const T* __restrict__ Y, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, T* __restrict__ out, int64_t T_, int d, int k) {
  constexpr int V = St<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blockIdx.x * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * kCW) {
    const int32_t* rows = row_of + t * k;
    const float* gt = gate + t * k;
    for (int c = lane; c < nch; c += kWave) {
      float acc[V];
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int32_t r = rows[j];
        if (r < 0) continue;
        const float gj = gt[j];
        float y[V];
        St<T>::unpack(ld16(Y + (int64_t)r * d + c * V), y);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] += gj * y[q];
      }
      st16(out + t * d + c * V, St<T>::pack(acc));
    }
  }
}

// dYp[row] = gate * dOut[t];  dgate[t,j] = <dOut[t], Y[row]> (0 if dropped)
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ dOut, const T* __restrict__ Y, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, T* __restrict__ dYp, float* __restrict__ dgate,
    int64_t T_, int d, int k) {
  constexpr int V = St<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blockIdx.x * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * kCW) {
    for (int j = 0; j < k; ++j) {
      const int32_t r = row_of[t * k + j];
      if (r < 0) {
        if (lane == 0) dgate[t * k + j] = 0.0f;
        continue;
      }
      const float gj = gate[t * k + j];
      float part = 0.0f;
      for (int c = lane; c < nch; c += kWave) {
        float g[V], y[V], o[V];
        St<T>::unpack(ld16(dOut + t * d + c * V), g);
        St<T>::unpack(ld16(Y + (int64_t)r * d + c * V), y);
#pragma unroll
        for (int q = 0; q < V; ++q) {
          part += g[q] * y[q];
          o[q] = gj * g[q];
        }
        st16(dYp + (int64_t)r * d + c * V, St<T>::pack(o));
      }
      part = wave_sum(part);
      if (lane == 0) dgate[t * k + j] = part;
    }
  }
}

// dXe[t] = sum over kept j of dXp[row_of[t,j]]  (float output)
template <typename T>
__global__ __launch_bounds__(256) void unpermute_bwd_kernel(
    const T* __restrict__ dXp, const int32_t* __restrict__ row_of, float* __restrict__ dXe,
    int64_t T_, int d, int k) {
  constexpr int V = St<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blockIdx.x * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * kCW) {
    for (int c = lane; c < nch; c += kWave) {
      float acc[V];
#pragma unroll
      for (int q = 0; q < V; ++q) acc[q] = 0.0f;
      for (int j = 0; j < k; ++j) {
        const int32_t r = row_of[t * k + j];
        if (r < 0) continue;
        float v[V];
        St<T>::unpack(ld16(dXp + (int64_t)r * d + c * V), v);
#pragma unroll
        for (int q = 0; q < V; ++q) acc[q] += v[q];
      }
      float* o = dXe + t * d + c * V;
#pragma unroll
      for (int q = 0; q < V; q += 4)
        st16(o + q, u32x4{__float_as_uint(acc[q]), __float_as_uint(acc[q + 1]),
                          __float_as_uint(acc[q + 2]), __float_as_uint(acc[q + 3])});
    }
  }
}

inline int token_grid(int64_t T_) {
  const int64_t b = ceil_div(T_, kCW);
  return (int)(b < 65536 ? b : 65536);
}

}  // namespace

int launch_combine(const moe_cfg& c, const void* Y, const int32_t* row_of,
                   const float* gate, void* out, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int grid = token_grid(c.T);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_COMBINE, s,
               combine_kernel<uint16_t><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Y), row_of, gate,
                   static_cast<uint16_t*>(out), c.T, c.d, c.k));
  else
    MOE_LAUNCH(MOE_KERNEL_COMBINE, s,
               combine_kernel<float><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(Y), row_of, gate, static_cast<float*>(out),
                   c.T, c.d, c.k));
  return MOE_OK;
}

int launch_combine_bwd(const moe_cfg& c, const void* dOut, const void* Y,
                       const int32_t* row_of, const float* gate, void* dYp,
                       float* dgate, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int grid = token_grid(c.T);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_COMBINE_BWD, s,
               combine_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(dOut), static_cast<const uint16_t*>(Y),
                   row_of, gate, static_cast<uint16_t*>(dYp), dgate, c.T, c.d, c.k));
  else
    MOE_LAUNCH(MOE_KERNEL_COMBINE_BWD, s,
               combine_bwd_kernel<float><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(dOut), static_cast<const float*>(Y), row_of,
                   gate, static_cast<float*>(dYp), dgate, c.T, c.d, c.k));
  return MOE_OK;
}

int launch_unpermute_bwd(const moe_cfg& c, const void* dXp, const int32_t* row_of,
                         float* dXe, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int grid = token_grid(c.T);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_UNPERMUTE_BWD, s,
               unpermute_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(dXp), row_of, dXe, c.T, c.d, c.k));
  else
    MOE_LAUNCH(MOE_KERNEL_UNPERMUTE_BWD, s,
               unpermute_bwd_kernel<float><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(dXp), row_of, dXe, c.T, c.d, c.k));
  return MOE_OK;
}

}  // namespace moe
