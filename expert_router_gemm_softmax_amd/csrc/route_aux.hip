// Routing diagnostics and the auxiliary load-balancing loss.  The
// distributed-training tutorial (section "The Capacity Factor") adds a
// balancing penalty, weighted by a small coefficient, that evens out the
// experts' token loads, and watches the drop rate and the expert load
// distribution.  The loss is the standard balancing loss over the fraction
// of assignments each expert receives and its mean router probability:
//   L = alpha * E * sum_e f_e P_e,  f_e = counts[e] / (T k),
//   P_e = (1/T) sum_t probs[t, e]
// and the drop rate is 1 - R / (T k) with R = offsets[E] the kept rows.
// The expert loads are counts itself.
//
// Two kernels: per-block column sums of probs over kAuxTokens tokens (one
// thread per expert, rows read coalesced across experts, all loads in
// flight), then one block that sums the partials per expert in fp64 (one
// wave per expert, lane-strided), forms the loss with a fixed tree over
// experts and writes aux[0] = L, aux[1] = drop rate.  Every sum has a fixed
// order, so the result is deterministic.
#include "common.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void route_aux_part_kernel(const float* __restrict__ probs,
                                                              float* __restrict__ part,
                                                              int64_t T_, int E) {
  const int e = threadIdx.x;
  if (e >= E) return;
  const int64_t t0 = (int64_t)blockIdx.x * kAuxTokens;
  const int n = (int)(T_ - t0 < kAuxTokens ? T_ - t0 : kAuxTokens);
  const float* p = probs + t0 * E + e;
  // every row's load in flight at once (indices clamped into the block's
  // rows so that no load sits behind a branch), then the sum in token order
  float v[kAuxTokens];
#pragma unroll
  for (int q = 0; q < kAuxTokens; ++q) v[q] = p[(int64_t)min(q, n - 1) * E];
#pragma unroll
  for (int q = 0; q < kAuxTokens; ++q)
    if (q >= n) v[q] = 0.0f;
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < kAuxTokens; ++q) s += v[q];
  part[(int64_t)e * gridDim.x + blockIdx.x] = s;
}

// One block of 1024 threads: wave w sums the partials of experts w, w+16,
// ... (lane-strided in fp64, then the fixed wave tree), then a fixed tree
// over experts forms the loss.
__global__ __launch_bounds__(1024) void route_aux_final_kernel(
    const float* __restrict__ part, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ offsets, float* __restrict__ aux, int nblk, int64_t T_,
    int E, int k, float coeff) {
  __shared__ double red[256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (threadIdx.x < 256) red[threadIdx.x] = 0.0;
  __syncthreads();
  constexpr int U = 16;  // loads in flight per lane
  for (int e = w; e < E; e += 16) {
    const float* pe = part + (int64_t)e * nblk;
    double s = 0.0;
    for (int b0 = 0; b0 < nblk; b0 += kWave * U) {
      float v[U];
#pragma unroll
      for (int q = 0; q < U; ++q) v[q] = pe[min(b0 + q * kWave + lane, nblk - 1)];
#pragma unroll
      for (int q = 0; q < U; ++q)
        if (b0 + q * kWave + lane >= nblk) v[q] = 0.0f;
#pragma unroll
      for (int q = 0; q < U; ++q) s += (double)v[q];
    }
    s = wave_sum_d(s);
    if (lane == 0) red[e] = (double)counts[e] * s;  // counts_e * T P_e
  }
  __syncthreads();
  for (int h = 128; h > 0; h >>= 1) {
    if (threadIdx.x < h) red[threadIdx.x] += red[threadIdx.x + h];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const double tk = (double)T_ * (double)k;
    aux[0] = (float)((double)coeff * (double)E * red[0] / (tk * (double)T_));
    aux[1] = (float)(1.0 - (double)offsets[E] / tk);
  }
}

// aux[0] = aux[1] = 0 for an empty batch
__global__ void route_aux_zero_kernel(float* __restrict__ aux) {
  if (threadIdx.x < 2) aux[threadIdx.x] = 0.0f;
}

}  // namespace

int launch_route_aux(const moe_cfg& c, const float* probs, const int32_t* counts,
                     const int32_t* offsets, float* aux, void* ws, hipStream_t s) {
  if (c.T == 0) {
    MOE_LAUNCH(MOE_KERNEL_ROUTE_AUX, s, route_aux_zero_kernel<<<1, 64, 0, s>>>(aux));
    return MOE_OK;
  }
  const WsLayout L = ws_layout(c);
  float* part = ws_ptr<float>(ws, L.aux_part);
  // both kernels are timed as one launch
  prof_begin(c, MOE_KERNEL_ROUTE_AUX, s);
  MOE_LAUNCH_NP(MOE_KERNEL_ROUTE_AUX,
                route_aux_part_kernel<<<L.nblk_aux, 256, 0, s>>>(probs, part, c.T, c.E));
  MOE_LAUNCH_NP(MOE_KERNEL_ROUTE_AUX,
                route_aux_final_kernel<<<1, 1024, 0, s>>>(part, counts, offsets, aux,
                                                         L.nblk_aux, c.T, c.E, c.k,
                                                         c.aux_coeff));
  prof_end(c, MOE_KERNEL_ROUTE_AUX, s);
  return MOE_OK;
}

}  // namespace moe
