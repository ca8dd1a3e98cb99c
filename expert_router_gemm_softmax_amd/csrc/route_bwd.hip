// Router backward (B1).  The router is a shared parameter with an ordinary
// gradient ("GPU expert parallel", section "Sharded by expert, replicated
// everywhere else"); index, top-k and capacity steps are piecewise constant
// and pass no gradient.
//   dp[t, e] = a_e + dgate[t,j] if e = idx[t,j] for a kept j, else a_e
//   (with renormalised gates g_j = p_j / S the gate term of a selected j is
//   (dgate_j - sum_i g_i dgate_i) / S instead, dropped j included)
//   dz = p * (dp - sum_e p dp)
// where a_e = alpha E counts[e] / (T k T) is the gradient of the
// load-balancing loss (zero when its coefficient alpha is zero); under the
// identity fallback of dropped assignments their dgate counts as well.
//   dX  = dXe + dz Wr^T,  dWr = x^T dz,  db = sum_t dz
// dXe is the gradient unpermute-sum (B2): either the caller's fp32 buffer
// (the per-step entry point) or, in the layer backward, gathered here from
// dXp (B2 fused in).  Both products run on the grouped GEMM kernels.  For
// bf16 storage dz is split into bf16 high and low parts (dz = hi + lo to
// ~2^-16 relative), and the products use [hi | lo] against Wr stacked
// twice, so the router gradient keeps ~fp32 accuracy on bf16 MFMA.  dX is
// one row-GEMM whose epilogue adds dXe; dWr is a k-ragged GEMM over uniform
// token chunks writing fp32 partials, summed in fixed order with db.  With
// 8 or 16 experts (bf16) dz Wr^T runs on the VALU instead (combine.hip),
// fused with the gather in the layer backward.  The two forms give bitwise
// the same dX.
#include "gemm.h"

namespace moe {

// combine.hip: the router backward's dX for bf16 storage and E = 8 or 16,
// the unpermute-sum of dXp plus dz Wr^T in one pass (dzb: the [T][2E] bf16
// hi/lo pair of dz); MOE_ERR_UNIMPLEMENTED for other shapes
int launch_unpermute_router_dx(const moe_cfg& c, const void* dXp, const int32_t* row_of,
                               const float* gate, const void* dOut, const uint16_t* dzb,
                               const void* Wr, void* dX, hipStream_t s);
// the same from a finished fp32 unpermute-sum dXe [T][d]
int launch_router_dx(const moe_cfg& c, const float* dXe, const uint16_t* dzb, const void* Wr,
                     void* dX, hipStream_t s);
namespace {

// wrp[i][e] = wrp[i][Ep + e] = Wr[i][e] (zero for E <= e < Ep): the router
// weights stacked twice for the [hi | lo] products, a grid-stride share of
// the copy per block of the dz kernel
__device__ __forceinline__ void stack_wr(const uint16_t* __restrict__ Wr,
                                         uint16_t* __restrict__ wrp, int d, int E, int Ep) {
  const int64_t n = (int64_t)d * 2 * Ep;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int i = (int)(o / (2 * Ep));
    int e = (int)(o - (int64_t)i * 2 * Ep);
    if (e >= Ep) e -= Ep;
    wrp[o] = e < E ? Wr[(int64_t)i * E + e] : (uint16_t)0;
  }
}

// dz for kDzTokens tokens per block (one wave per token); writes dz (fp32
// storage) or its bf16 hi/lo split (bf16 storage), and the block's partial
// sums of dz for db; for bf16 storage also the stacked router weights.
// counts may be NULL when aux_scale is zero.
template <bool BF>
__global__ __launch_bounds__(256) void route_bwd_dz_kernel(
    const float* __restrict__ probs, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ row_of, const int32_t* __restrict__ counts,
    const float* __restrict__ dgate, float* __restrict__ dz, uint16_t* __restrict__ dzb,
    float* __restrict__ db_part, const uint16_t* __restrict__ Wr, uint16_t* __restrict__ wrp,
    int d, int64_t T_, int E, int Ep, int k, float aux_scale, bool renorm, bool fallback) {
  if constexpr (BF) stack_wr(Wr, wrp, d, E, Ep);
  __shared__ float sdb[4][256];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  float dbacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  // balancing-loss gradient, the same for every token
  float a[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = lane + 64 * i;
    a[i] = aux_scale != 0.0f && e < E ? aux_scale * (float)counts[e] : 0.0f;
  }
  const int64_t t0 = (int64_t)blockIdx.x * kDzTokens;
  for (int tt = w; tt < kDzTokens; tt += 4) {
    const int64_t t = t0 + tt;
    if (t >= T_) break;
    float p[4], dp[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      p[i] = e < E ? probs[t * E + e] : 0.0f;
      dp[i] = a[i];
    }
    if (renorm) {
      // gates g_j = p_j / S (S summed in selection order, as the forward);
      // dL/dp_j = (dgate_j - sum_i g_i dgate_i) / S for every selected j
      auto psel = [&](int j) {  // an index outside [0, E) counts as probability 0
        const int e = idx[t * k + j];
        return (unsigned)e < (unsigned)E ? probs[t * E + e] : 0.0f;
      };
      float S = 0.0f;
      for (int j = 0; j < k; ++j) S += psel(j);
      float G = 0.0f;
      for (int j = 0; j < k; ++j) {
        const float dg = row_of[t * k + j] < 0 && !fallback ? 0.0f : dgate[t * k + j];
        G += psel(j) / S * dg;
      }
      for (int j = 0; j < k; ++j) {
        const int e = idx[t * k + j];
        const float dg = row_of[t * k + j] < 0 && !fallback ? 0.0f : dgate[t * k + j];
        const float g = (dg - G) / S;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e == lane + 64 * i) dp[i] += g;
      }
    } else {
      for (int j = 0; j < k; ++j) {
        if (row_of[t * k + j] < 0 && !fallback) continue;
        const int e = idx[t * k + j];
        const float g = dgate[t * k + j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (e == lane + 64 * i) dp[i] += g;
      }
    }
    float sp = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) sp += p[i] * dp[i];
    sp = wave_sum(sp);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i;
      const float v = p[i] * (dp[i] - sp);  // 0 for padded experts
      if (e < E) dbacc[i] += v;
      if constexpr (BF) {
        if (e < Ep) {
          const uint16_t hi = f2bf(v);
          dzb[t * 2 * Ep + e] = hi;
          dzb[t * 2 * Ep + Ep + e] = f2bf(v - bf2f(hi));
        }
      } else {
        if (e < E) dz[t * E + e] = v;
      }
    }
  }
  // fixed-order block reduction of the per-wave partial sums
#pragma unroll
  for (int i = 0; i < 4; ++i) sdb[w][lane + 64 * i] = dbacc[i];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += 256)
    db_part[(int64_t)e * gridDim.x + blockIdx.x] =
        (sdb[0][e] + sdb[1][e]) + (sdb[2][e] + sdb[3][e]);
}


// dWr[i][e] = sum over chunks (fixed order) of part[c][i][e] (+ the low half)
// and db[e] = sum over blocks of db_part[e][b]
template <typename T>
__global__ __launch_bounds__(256) void route_bwd_reduce_kernel(
    const float* __restrict__ part, const float* __restrict__ db_part, T* __restrict__ dWr,
    float* __restrict__ db, int nchunks, int nblk_dz, int d, int E, int Nw, int Ep) {
  const int64_t n = (int64_t)d * E;
  for (int64_t o = blockIdx.x * 256 + threadIdx.x; o < n; o += (int64_t)gridDim.x * 256) {
    const int64_t i = o / E;
    const int e = (int)(o - i * E);
    // chunks in ascending order; 8 chunks' loads in flight per step
    const float* p0 = part + i * Nw + e;
    const int64_t cs = (int64_t)d * Nw;
    const bool two = Nw != E;
    float s = 0.0f;
    for (int c0 = 0; c0 < nchunks; c0 += 8) {
      float hi8[8], lo8[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const bool ok = c0 + q < nchunks;
        hi8[q] = ok ? p0[(c0 + q) * cs] : 0.0f;
        lo8[q] = ok && two ? p0[(c0 + q) * cs + Ep] : 0.0f;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) s += hi8[q] + lo8[q];
    }
    dWr[o] = St<T>::from_f(s);
  }
  // db[e]: one wave per expert over its row of block partials (lane-strided
  // fixed-order sums, then the fixed wave tree)
  if (db != nullptr) {
    const int lane = threadIdx.x & 63;
    for (int e = blockIdx.x * 4 + (threadIdx.x >> 6); e < E; e += gridDim.x * 4) {
      const float* row = db_part + (int64_t)e * nblk_dz;
      float s = 0.0f;
      for (int b = lane; b < nblk_dz; b += kWave) s += row[b];
      s = wave_sum(s);
      if (lane == 0) db[e] = s;
    }
  }
}

template <typename T>
int route_bwd_t(const moe_cfg& c, const T* x, const T* Wr, const float* probs,
                const int32_t* idx, const int32_t* row_of, const int32_t* counts,
                const float* gate, const void* dOut, const float* dgate, const T* dXp,
                const float* dXe, T* dX, T* dWr, float* db, void* ws, hipStream_t s) {
  constexpr bool BF = sizeof(T) == 2;
  const WsLayout L = ws_layout(c);
  const int Ep = bwd_ep(c.E);
  float* dz = ws_ptr<float>(ws, L.dz);
  uint16_t* dzb = ws_ptr<uint16_t>(ws, L.dzb);
  uint16_t* wrp = ws_ptr<uint16_t>(ws, L.wrp);
  float* part = ws_ptr<float>(ws, L.dwr_part);
  float* dbp = ws_ptr<float>(ws, L.db_part);
  const int nblk = c.T > 0 ? (int)ceil_div(c.T, kDzTokens) : 0;
  // a_e = aux_scale counts[e]
  const float aux_scale =
      c.aux_coeff > 0.0f && c.T > 0
          ? (float)((double)c.aux_coeff * c.E / ((double)c.T * c.k * (double)c.T))
          : 0.0f;
  if (nblk > 0)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DZ, s,
               route_bwd_dz_kernel<BF><<<nblk, 256, 0, s>>>(
                   probs, idx, row_of, counts, dgate, dz, dzb, dbp,
                   BF ? reinterpret_cast<const uint16_t*>(Wr) : nullptr, wrp, c.d, c.T, c.E, Ep,
                   c.k, aux_scale, (c.flags & MOE_FLAG_RENORM) != 0,
                   (c.flags & MOE_FLAG_DROP_IDENTITY) != 0));
  int rc;
  if (c.T > 0 && BF && (c.E == 8 || c.E == 16) &&
      (reinterpret_cast<uintptr_t>(Wr) & 15) == 0) {
    // few experts: dz Wr^T is E FMAs per output, done on the VALU (inside the
    // unpermute-sum's pass when dXp is given: no fp32 sum through HBM, no GEMM
    // launch); Wr's rows are read as 16-byte vectors
    rc = dXe ? launch_router_dx(c, dXe, dzb, Wr, dX, s)
             : launch_unpermute_router_dx(c, dXp, row_of, gate, dOut, dzb, Wr, dX, s);
    if (rc != MOE_OK) return rc;
  } else if (c.T > 0) {
    // dX = [dz_hi | dz_lo] [Wr | Wr]^T + dXe (fp32), dXe gathered from dXp
    // into the workspace unless the caller gives it
    float* dxe = const_cast<float*>(dXe);
    if (dxe == nullptr) {
      dxe = ws_ptr<float>(ws, L.dxe);
      rc = launch_unpermute_bwd(c, dXp, row_of, gate, dOut, dxe, s, MOE_KERNEL_ROUTE_BWD_DX);
      if (rc != MOE_OK) return rc;
    }
    GemmArgs g{};
    g.E = 1;
    g.M = (int)c.T;
    g.N = c.d;
    g.K = BF ? 2 * Ep : c.E;
    g.A = BF ? static_cast<const void*>(dzb) : static_cast<const void*>(dz);
    g.lda = g.K;
    g.B = BF ? static_cast<const void*>(wrp) : static_cast<const void*>(Wr);
    g.ldb = g.K;
    g.C = dX;
    g.ldc = c.d;
    g.Aux = dxe;
    g.part = ws_ptr<float>(ws, L.gpart);
    // short K (2 Ep): the epilogue's fp32 reads dominate, so use tiles that
    // fit three blocks per CU and overlap it with other blocks' MFMAs
    g.bm = g.bn = 128;
    rc = launch_gemm(MOE_KERNEL_ROUTE_BWD_DX, MODE_ROW, true, EPI_ADDF32, c, g, s);
    if (rc != MOE_OK) return rc;
  }
  if (c.T > 0) {
    // dWr partials = x^T [dz_hi | dz_lo] over uniform token chunks
    GemmArgs h{};
    h.E = L.dwr_chunks;
    h.chunk = L.dwr_chunk;
    h.K = (int)c.T;
    h.M = c.d;
    h.N = L.dwr_n;
    h.A = x;
    h.lda = c.d;
    h.B = BF ? static_cast<const void*>(dzb) : static_cast<const void*>(dz);
    h.ldb = L.dwr_n;
    h.C = part;
    h.ldc = L.dwr_n;
    h.c_estride = (int64_t)c.d * L.dwr_n;
    rc = launch_gemm(MOE_KERNEL_ROUTE_BWD_DW, MODE_KRAG, false, EPI_F32, c, h, s);
    if (rc != MOE_OK) return rc;
  }
  const int nch = c.T > 0 ? L.dwr_chunks : 0;
  const int g4 = (int)std::min<int64_t>(ceil_div((int64_t)c.d * c.E, 256), 4096);
  MOE_LAUNCH(MOE_KERNEL_ROUTE_BWD_DW, s,
             route_bwd_reduce_kernel<T><<<g4, 256, 0, s>>>(part, dbp, dWr, db, nch, nblk,
                                                          c.d, c.E, L.dwr_n, Ep));
  return MOE_OK;
}

}  // namespace

int launch_route_bwd(const moe_cfg& c, const void* x, const void* Wr,
                     const float* probs, const int32_t* idx, const int32_t* row_of,
                     const int32_t* counts, const float* gate, const void* dOut,
                     const float* dgate, const void* dXp, const float* dXe, void* dX,
                     void* dWr, float* db, void* ws, hipStream_t s) {
  if (c.dtype == MOE_BF16)
    return route_bwd_t<uint16_t>(c, static_cast<const uint16_t*>(x),
                                 static_cast<const uint16_t*>(Wr), probs, idx, row_of, counts,
                                 gate, dOut, dgate, static_cast<const uint16_t*>(dXp), dXe,
                                 static_cast<uint16_t*>(dX), static_cast<uint16_t*>(dWr), db,
                                 ws, s);
  return route_bwd_t<float>(c, static_cast<const float*>(x), static_cast<const float*>(Wr),
                            probs, idx, row_of, counts, gate, dOut, dgate,
                            static_cast<const float*>(dXp), dXe, static_cast<float*>(dX),
                            static_cast<float*>(dWr), db, ws, s);
}

}  // namespace moe
