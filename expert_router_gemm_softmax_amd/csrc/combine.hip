// Gate-weighted combine (F5), its backward (B5) and the gradient
// unpermute-sum (B2).  The inverse of the permutation returns expert
// outputs to token order ("GPU expert parallel", section "The step
// timeline"); backward retraces it.  All three are HBM-bound gathers:
// one wave per token, one 16-byte vector per lane per step, fp32 math.
#include "common.h"

namespace moe {
namespace {

constexpr int kCW = 4;   // waves per block
constexpr int kCPL = 8;     // 16-byte chunks per lane in one pass over a row
constexpr int kBwdCPL = 4;  // the same for combine backward (fewer registers)

// Loads the chunks of one pass (chunk c = g0 + s*64 + lane) of row r of src
// into v; chunks past the row end, and every chunk of a dropped row
// (r < 0), are not loaded.  NT: the step's last read of these rows (dOut and
// Y in the combine backward, dXp in the unpermute-sum), marked non-temporal
// so that they do not push the kernel's output (read by the next kernel) out
// of the memory-side cache.
template <typename T, int CPL, bool NT = false>
__device__ __forceinline__ void load_pass(const T* __restrict__ src, int64_t r, int d, int g0,
                                          int nch, int lane, u32x4 (&v)[CPL]) {
  constexpr int V = St<T>::kVec;
  if (r < 0) return;
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    const int c = g0 + s * kWave + lane;
    if (c < nch) {
      if constexpr (NT)
        v[s] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * d + c * V));
      else
        v[s] = ld16(src + r * d + c * V);
    }
  }
}

// The router backward's dz of one token for E = 8 RV experts, dz = hi + lo
// of the bf16 pair in dzb [T][2E]
template <int RV>
__device__ __forceinline__ void load_dz(const uint16_t* __restrict__ dzb, int64_t t,
                                        float (&dzf)[8 * RV]) {
  const uint16_t* dz = dzb + t * (16 * RV);
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    float hi[8], lo[8];
    St<uint16_t>::unpack(ld16(dz + 8 * r), hi);
    St<uint16_t>::unpack(ld16(dz + 8 * RV + 8 * r), lo);
#pragma unroll
    for (int e = 0; e < 8; ++e) dzf[8 * r + e] = hi[e] + lo[e];
  }
}
// sum_e dz[e] Wr[i,e] in fp32, expert order (Wr [d][8 RV] bf16, 16-byte rows)
template <int RV>
__device__ __forceinline__ float router_term(const float (&dzf)[8 * RV],
                                             const uint16_t* __restrict__ Wr, int i) {
  const uint16_t* wr = Wr + (int64_t)i * (8 * RV);
  float u = 0.0f;
#pragma unroll
  for (int r = 0; r < RV; ++r) {
    float w8[8];
    St<uint16_t>::unpack(ld16(wr + 8 * r), w8);
#pragma unroll
    for (int e = 0; e < 8; ++e) u += dzf[8 * r + e] * w8[e];
  }
  return u;
}

// out[t] = sum over kept j (ascending) of g_j * src[row_of[t,j]], with
// g_j = gate[t,j] (combine) or 1 (gradient unpermute-sum, fp32 output).
// With a fallback row source fb (the identity fallback: x for the combine,
// dOut for the unpermute-sum) a dropped j adds gate[t,j] * fb[t] in its
// place.  One wave per token; two assignments' rows are in flight at once.
// RV > 0 (bf16, E = 8 RV experts): the router backward's dX instead,
// RN_bf16(unpermute-sum + sum_e dz[t,e] Wr[i,e]), the unpermute-sum taken
// exactly as the fp32 one above and the router term added last (dz = hi +
// lo of the bf16 pair in dzb [T][2E]; Wr [d][E]) -- the E products per
// output run on the VALU, and no fp32 sum goes through HBM.  The result is
// bitwise router_dx_kernel's on the fp32 unpermute-sum.
// NTL: the rows are read non-temporally -- the unpermute-sum's dXp (its last
// read in the step), and the combine's Y when it cannot stay in the
// memory-side cache until the combine backward reads it again.
template <typename T, typename OutT, bool GATED, int RV = 0, bool NTL = !GATED>
__global__ __launch_bounds__(256) void gather_sum_kernel(
    const T* __restrict__ src, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, const T* __restrict__ fb, OutT* __restrict__ out,
    int64_t T_, int d, int k, const uint16_t* __restrict__ dzb = nullptr,
    const uint16_t* __restrict__ Wr = nullptr) {
  constexpr int V = St<T>::kVec;
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blockIdx.x * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * kCW) {
    const int32_t* rows = row_of + t * k;
    float dzf[RV > 0 ? 8 * RV : 1];
    if constexpr (RV > 0) load_dz<RV>(dzb, t, dzf);
    for (int g0 = 0; g0 < nch; g0 += kWave * kCPL) {
      float acc[kCPL][V];
#pragma unroll
      for (int s = 0; s < kCPL; ++s)
#pragma unroll
        for (int q = 0; q < V; ++q) acc[s][q] = 0.0f;
      for (int j = 0; j < k; j += 2) {
        const int32_t r0 = rows[j];
        const int32_t r1 = j + 1 < k ? rows[j + 1] : -2;  // -2: no assignment
        const bool u0 = r0 >= 0 || (fb && r0 == -1);
        const bool u1 = r1 >= 0 || (fb && r1 == -1);
        u32x4 y0[kCPL], y1[kCPL];
        load_pass<T, kCPL, NTL>(r0 >= 0 ? src : fb, u0 ? (r0 >= 0 ? (int64_t)r0 : t) : -1, d,
                                   g0, nch, lane, y0);
        load_pass<T, kCPL, NTL>(r1 >= 0 ? src : fb, u1 ? (r1 >= 0 ? (int64_t)r1 : t) : -1, d,
                                   g0, nch, lane, y1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int32_t r = h ? r1 : r0;
          if (!(h ? u1 : u0)) continue;
          const float g = (GATED || r < 0) ? gate[t * k + j + h] : 1.0f;
#pragma unroll
          for (int s = 0; s < kCPL; ++s) {
            if (g0 + s * kWave + lane >= nch) continue;
            float y[V];
            St<T>::unpack(h ? y1[s] : y0[s], y);
#pragma unroll
            for (int q = 0; q < V; ++q) acc[s][q] += g * y[q];
          }
        }
      }
      if constexpr (RV > 0) {
        // the router term last: RN(unpermute-sum + sum_e dz[t,e] Wr[i,e])
#pragma unroll
        for (int s = 0; s < kCPL; ++s) {
          const int c = g0 + s * kWave + lane;
          if (c >= nch) continue;
#pragma unroll
          for (int q = 0; q < V; ++q) acc[s][q] += router_term<RV>(dzf, Wr, c * V + q);
        }
      }
#pragma unroll
      for (int s = 0; s < kCPL; ++s) {
        const int c = g0 + s * kWave + lane;
        if (c >= nch) continue;
        if constexpr (sizeof(OutT) == sizeof(T)) {
          // the layer's output (combine) or the router's dX: read by no
          // later kernel of the step, so stored non-temporally, leaving the
          // memory-side cache to the backward's inputs
          __builtin_nontemporal_store(St<T>::pack(acc[s]),
                                      reinterpret_cast<u32x4*>(out + t * d + c * V));
        } else {
          float* o = reinterpret_cast<float*>(out) + t * d + c * V;
#pragma unroll
          for (int q = 0; q < V; q += 4)
            st16(o + q, u32x4{__float_as_uint(acc[s][q]), __float_as_uint(acc[s][q + 1]),
                              __float_as_uint(acc[s][q + 2]), __float_as_uint(acc[s][q + 3])});
        }
      }
    }
  }
}

// The router backward's dX from the fp32 unpermute-sum dXe [T][d] (bf16,
// E = 8 RV experts): dX[t,i] = RN_bf16(dXe[t,i] + sum_e dz[t,e] Wr[i,e]),
// one wave per token, 8 consecutive outputs per lane and pass.
template <int RV>
__global__ __launch_bounds__(256) void router_dx_kernel(const float* __restrict__ dxe,
                                                        const uint16_t* __restrict__ dzb,
                                                        const uint16_t* __restrict__ Wr,
                                                        uint16_t* __restrict__ dX, int64_t T_,
                                                        int d) {
  const int lane = threadIdx.x & 63;
  const int nch = d / 8;
  for (int64_t t = (int64_t)blockIdx.x * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)gridDim.x * kCW) {
    float dzf[8 * RV];
    load_dz<RV>(dzb, t, dzf);
    for (int c = lane; c < nch; c += kWave) {
      const float* src = dxe + t * d + c * 8;
      const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
      const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 4);
      float v[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[q] = a0[q] + router_term<RV>(dzf, Wr, c * 8 + q);
        v[q + 4] = a1[q] + router_term<RV>(dzf, Wr, c * 8 + q + 4);
      }
      st16(dX + t * d + c * 8, St<uint16_t>::pack(v));
    }
  }
}

// dYp[row] = gate * dOut[t];  dgate[t,j] = <dOut[t], Y[row]> (0 if dropped).
// One wave per token: each pass holds dOut's chunks in registers while the
// k rows of Y stream past, two at a time; lane j keeps dgate[t,j].
// With the identity fallback (x given) a dropped j gets <dOut[t], x[t]>.
template <typename T>
__global__ __launch_bounds__(256) void combine_bwd_kernel(
    const T* __restrict__ dOut, const T* __restrict__ Y, const int32_t* __restrict__ row_of,
    const float* __restrict__ gate, const T* __restrict__ x, T* __restrict__ dYp,
    float* __restrict__ dgate, int64_t T_, int d, int k, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ tiles, int E, int BM, int32_t* __restrict__ plan, int te) {
  constexpr int V = St<T>::kVec;
  int blk = blockIdx.x, nblk = gridDim.x;
  if (tiles != nullptr) {
    // the first block writes the grouped GEMMs' M-tile prefix and the
    // weight-gradient split plan and nothing else, so that this work runs
    // beside the token blocks rather than before one of them
    if (blk == 0) {
      __shared__ int s_wave[4];
      const int e = threadIdx.x;
      const int m = e < E ? offsets[e + 1] - offsets[e] : 0;
      block_tile_prefix(m, E, BM, tiles, s_wave);
      if (plan != nullptr) block_krag_plan(m, E, te, plan, s_wave);
      return;
    }
    --blk;
    --nblk;
  }
  const int lane = threadIdx.x & 63;
  const int nch = d / V;
  for (int64_t t = (int64_t)blk * kCW + (threadIdx.x >> 6); t < T_;
       t += (int64_t)nblk * kCW) {
    const int32_t* rows = row_of + t * k;
    float mine = 0.0f;  // lane j < k: dgate[t, j]
    for (int g0 = 0; g0 < nch; g0 += kWave * kBwdCPL) {
      u32x4 gv[kBwdCPL];
      load_pass<T, kBwdCPL, true>(dOut, t, d, g0, nch, lane, gv);
      for (int j = 0; j < k; j += 2) {
        const int32_t r0 = rows[j];
        const int32_t r1 = j + 1 < k ? rows[j + 1] : -2;  // -2: no assignment
        const bool u0 = r0 >= 0 || (x && r0 == -1);
        const bool u1 = r1 >= 0 || (x && r1 == -1);
        u32x4 y0[kBwdCPL], y1[kBwdCPL];
        load_pass<T, kBwdCPL, true>(r0 >= 0 ? Y : x, u0 ? (r0 >= 0 ? (int64_t)r0 : t) : -1, d, g0,
                                    nch, lane, y0);
        load_pass<T, kBwdCPL, true>(r1 >= 0 ? Y : x, u1 ? (r1 >= 0 ? (int64_t)r1 : t) : -1, d, g0,
                                    nch, lane, y1);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int32_t r = h ? r1 : r0;
          if (!(h ? u1 : u0)) continue;  // uniform over the wave
          const float gj = gate[t * k + j + h];
          float pp = 0.0f;
#pragma unroll
          for (int s = 0; s < kBwdCPL; ++s) {
            const int c = g0 + s * kWave + lane;
            if (c >= nch) continue;
            float g[V], y[V], o[V];
            St<T>::unpack(gv[s], g);
            St<T>::unpack(h ? y1[s] : y0[s], y);
#pragma unroll
            for (int q = 0; q < V; ++q) {
              pp += g[q] * y[q];
              o[q] = gj * g[q];
            }
            if (r >= 0) st16(dYp + (int64_t)r * d + c * V, St<T>::pack(o));
          }
          pp = wave_sum_xor(pp);
          if (lane == j + h) mine += pp;
        }
      }
    }
    if (lane < k) dgate[t * k + lane] = (rows[lane] >= 0 || x) ? mine : 0.0f;
  }
}

inline int token_grid(int64_t T_) {
  const int64_t b = ceil_div(T_, kCW);
  return (int)(b < 65536 ? b : 65536);
}

}  // namespace

// The memory-side cache (MALL) of MI355X, 256 MB: Y larger than it is read
// non-temporally by the combine (c4_large: combine 242 -> 222 us, the
// combine backward unchanged; with Y inside it, as at c2_zipf, the combine
// backward would lose its cache hits: 31 -> 37 us).
constexpr size_t kMallBytes = (size_t)256 << 20;

int launch_combine(const moe_cfg& c, const void* Y, const int32_t* row_of,
                   const float* gate, const void* x, void* out, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int grid = token_grid(c.T);
  const void* fb = (c.flags & MOE_FLAG_DROP_IDENTITY) ? x : nullptr;
  const bool nt = (size_t)rows_max(c) * (size_t)c.d * elem_bytes(c) > kMallBytes;
  if (c.dtype == MOE_BF16 && nt)
    MOE_LAUNCH(MOE_KERNEL_COMBINE, s,
               gather_sum_kernel<uint16_t, uint16_t, true, 0, true><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Y), row_of, gate,
                   static_cast<const uint16_t*>(fb), static_cast<uint16_t*>(out), c.T, c.d,
                   c.k));
  else if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_COMBINE, s,
               gather_sum_kernel<uint16_t, uint16_t, true><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Y), row_of, gate,
                   static_cast<const uint16_t*>(fb), static_cast<uint16_t*>(out), c.T, c.d,
                   c.k));
  else
    MOE_LAUNCH(MOE_KERNEL_COMBINE, s,
               gather_sum_kernel<float, float, true><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(Y), row_of, gate, static_cast<const float*>(fb),
                   static_cast<float*>(out), c.T, c.d, c.k));
  return MOE_OK;
}

int launch_combine_bwd(const moe_cfg& c, const void* dOut, const void* Y,
                       const int32_t* row_of, const float* gate, const void* x, void* dYp,
                       float* dgate, hipStream_t s, const int32_t* offsets, int32_t* tiles,
                       int32_t* plan) {
  if (c.T == 0) return MOE_OK;
  const int BM = ffn_row_tile(c);
  // one more block for the schedule when the tiles are asked for
  const int grid = token_grid(c.T) + (tiles != nullptr ? 1 : 0);
  const void* fb = (c.flags & MOE_FLAG_DROP_IDENTITY) ? x : nullptr;
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_COMBINE_BWD, s,
               combine_bwd_kernel<uint16_t><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(dOut), static_cast<const uint16_t*>(Y),
                   row_of, gate, static_cast<const uint16_t*>(fb),
                   static_cast<uint16_t*>(dYp), dgate, c.T, c.d, c.k, offsets, tiles, c.E, BM,
                   plan, (int)krag_te(c)));
  else
    MOE_LAUNCH(MOE_KERNEL_COMBINE_BWD, s,
               combine_bwd_kernel<float><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(dOut), static_cast<const float*>(Y), row_of,
                   gate, static_cast<const float*>(fb), static_cast<float*>(dYp), dgate,
                   c.T, c.d, c.k, offsets, tiles, c.E, BM, nullptr, 0));
  return MOE_OK;
}

int launch_unpermute_bwd(const moe_cfg& c, const void* dXp, const int32_t* row_of,
                         const float* gate, const void* dOut, float* dXe, hipStream_t s,
                         int kernel_id) {
  if (c.T == 0) return MOE_OK;
  const int grid = token_grid(c.T);
  const void* fb = (c.flags & MOE_FLAG_DROP_IDENTITY) ? dOut : nullptr;
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(kernel_id, s,
               gather_sum_kernel<uint16_t, float, false><<<grid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(dXp), row_of, gate,
                   static_cast<const uint16_t*>(fb), dXe, c.T, c.d, c.k));
  else
    MOE_LAUNCH(kernel_id, s,
               gather_sum_kernel<float, float, false><<<grid, 256, 0, s>>>(
                   static_cast<const float*>(dXp), row_of, gate, static_cast<const float*>(fb),
                   dXe, c.T, c.d, c.k));
  return MOE_OK;
}

int launch_router_dx(const moe_cfg& c, const float* dXe, const uint16_t* dzb, const void* Wr,
                     void* dX, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  if (c.dtype != MOE_BF16 || (c.E != 8 && c.E != 16)) return MOE_ERR_UNIMPLEMENTED;
  const int grid = token_grid(c.T);
  const uint16_t* w = static_cast<const uint16_t*>(Wr);
  uint16_t* o = static_cast<uint16_t*>(dX);
  if (c.E == 8)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DX, s,
               router_dx_kernel<1><<<grid, 256, 0, s>>>(dXe, dzb, w, o, c.T, c.d));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DX, s,
               router_dx_kernel<2><<<grid, 256, 0, s>>>(dXe, dzb, w, o, c.T, c.d));
  return MOE_OK;
}

int launch_unpermute_router_dx(const moe_cfg& c, const void* dXp, const int32_t* row_of,
                               const float* gate, const void* dOut, const uint16_t* dzb,
                               const void* Wr, void* dX, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  if (c.dtype != MOE_BF16 || (c.E != 8 && c.E != 16)) return MOE_ERR_UNIMPLEMENTED;
  const int grid = token_grid(c.T);
  const uint16_t* fb =
      (c.flags & MOE_FLAG_DROP_IDENTITY) ? static_cast<const uint16_t*>(dOut) : nullptr;
  const uint16_t* src = static_cast<const uint16_t*>(dXp);
  const uint16_t* w = static_cast<const uint16_t*>(Wr);
  uint16_t* o = static_cast<uint16_t*>(dX);
  if (c.E == 8)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DX, s,
               gather_sum_kernel<uint16_t, uint16_t, false, 1><<<grid, 256, 0, s>>>(
                   src, row_of, gate, fb, o, c.T, c.d, c.k, dzb, w));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DX, s,
               gather_sum_kernel<uint16_t, uint16_t, false, 2><<<grid, 256, 0, s>>>(
                   src, row_of, gate, fb, o, c.T, c.d, c.k, dzb, w));
  return MOE_OK;
}

}  // namespace moe
