// Router forward (F1): logits z = x Wr + b, softmax over all experts,
// top-k in the order (z descending, expert ascending), gates = chosen
// probabilities.  Expert-parallel MoE layer, "GPU expert parallel"
// (aicassindra.com), sections "The step timeline" and "Sharded by expert,
// replicated everywhere else" (router decisions must agree on every rank).
//
// Decision rule.  The decision is defined on the canonical logit
// z = RN_fp32(sum_i x_i Wr_ie + b_e) with the sum in fp64.  The fast path
// computes zf with fp32 accumulation (bf16 MFMA, or fp32 VALU for float
// storage).  If every gap between neighbours in the top-(k+1) of zf is at
// least tau, the order of zf is the canonical order (|zf - z| < tau/2).
// Otherwise every expert whose zf lies within tau of the (k+1)-th value or
// above it is rescored in fp64 and the top-k is taken among those: any
// expert below that band has k+1 experts canonically above it.
//
// Layout: one block = 4 waves x 32 tokens.  The bf16 logits use
// v_mfma_f32_32x32x16_bf16 with tokens on M and experts on N (padded to a
// multiple of 32); each lane streams its token row straight from HBM
// (64 contiguous bytes per 64-wide K chunk: the K order inside a chunk is
// permuted identically for both operands), the transposed router weights
// are staged through LDS once per block and shared by its 4 waves.
#include "common.h"

#include <float.h>

namespace moe {

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, hipStream_t s);

namespace {

constexpr int kRW = 4;     // waves per block
constexpr int kRT = 32;    // tokens per wave
constexpr int kRBK = 64;   // K chunk
constexpr int kRBKP = 72;  // LDS row of the staged weight chunk (elements)

struct RouteSmem {
  int zs_stride;  // floats per token row of logits
  size_t zs_off, stats_off, idx_off, uz_off, ue_off, total;
};

__host__ __device__ inline RouteSmem route_smem(int Epad, int k, int elem) {
  RouteSmem m{};
  m.zs_stride = Epad + 1;
  size_t zs = (size_t)kRW * kRT * m.zs_stride * 4;
  size_t sb = elem == 2 ? (size_t)2 * Epad * kRBKP * 2 : 0;
  size_t u = zs > sb ? zs : sb;
  m.zs_off = 0;
  m.stats_off = (u + 15) / 16 * 16;
  m.idx_off = m.stats_off + (size_t)3 * kRW * kRT * 4;
  m.uz_off = m.idx_off + (size_t)kRW * kRT * k * 4;
  m.ue_off = m.uz_off + (size_t)kRW * Epad * 4;
  m.total = m.ue_off + (size_t)kRW * Epad * 4;
  return m;
}

// wrT[e][i] = Wr[i][e] for e < E, zero rows for E <= e < Epad.
template <typename T>
__global__ void transpose_wr_kernel(const T* __restrict__ Wr, T* __restrict__ wrT,
                                    int d, int E, int Epad) {
  const int64_t n = (int64_t)Epad * d;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(o / d), i = (int)(o - (int64_t)e * d);
    wrT[o] = e < E ? Wr[(int64_t)i * E + e] : T(0);
  }
}

// bf16 logits of the wave's 32 tokens into zs (fp32 accumulate, + bias).
template <int NT>
__device__ __forceinline__ void logits_mfma(const uint16_t* __restrict__ x,
                                            const uint16_t* __restrict__ wrT,
                                            const float* __restrict__ bias,
                                            int64_t T_, int d, int E, int64_t t_w,
                                            uint16_t* sB, float* zs, int zs_stride) {
  constexpr int Epad = 32 * NT;
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int64_t tr = t_w + r;
  const bool row_ok = tr < T_;
  const uint16_t* xrow = x + (row_ok ? tr : 0) * (int64_t)d;
  const int nkc = (d + kRBK - 1) / kRBK;

  f32x16 acc[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc[n] = f32x16{};

  u32x4 a_cur[4], a_nxt[4], b_nxt[NT];
  auto load_a = [&](int kc, u32x4 (&a)[4]) {
    const int k0 = kc * kRBK + h * 32;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int kq = k0 + q * 8;
      a[q] = (row_ok && kq < d) ? ld16(xrow + kq) : u32x4{0, 0, 0, 0};
    }
  };
  // Epad rows x 8 chunks of 16 bytes per K chunk; NT chunks per thread
  auto load_b = [&](int kc, u32x4 (&bq)[NT]) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * 256;
      const int e = c >> 3, q = c & 7;
      const int kq = kc * kRBK + q * 8;
      bq[i] = kq < d ? ld16(wrT + (int64_t)e * d + kq) : u32x4{0, 0, 0, 0};
    }
  };
  auto store_b = [&](int buf, const u32x4 (&bq)[NT]) {
#pragma unroll
    for (int i = 0; i < NT; ++i) {
      const int c = threadIdx.x + i * 256;
      const int e = c >> 3, q = c & 7;
      *reinterpret_cast<u32x4*>(sB + ((size_t)buf * Epad + e) * kRBKP + q * 8) = bq[i];
    }
  };

  // Token rows stream two K chunks ahead of the MFMAs: three register sets
  // with fixed roles (a rotating copy would wait on the loads in flight);
  // the router weights go through the LDS double buffer one chunk ahead.
  u32x4 a_2[4];
  auto step = [&](int kc, u32x4 (&acur)[4], u32x4 (&afar)[4]) {
    if (kc >= nkc) return;
    const int buf = kc & 1;
    const bool more = kc + 1 < nkc;
    if (kc + 2 < nkc) load_a(kc + 2, afar);
    if (more) load_b(kc + 1, b_nxt);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const bf16x8 a = __builtin_bit_cast(bf16x8, acur[kk]);
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const u32x4 bv = *reinterpret_cast<const u32x4*>(
            sB + ((size_t)buf * Epad + n * 32 + r) * kRBKP + (h * 4 + kk) * 8);
        acc[n] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            a, __builtin_bit_cast(bf16x8, bv), acc[n], 0, 0, 0);
      }
    }
    if (more) store_b(buf ^ 1, b_nxt);
    __syncthreads();
  };
  load_a(0, a_cur);
  if (nkc > 1) load_a(1, a_nxt);
  load_b(0, b_nxt);
  store_b(0, b_nxt);
  __syncthreads();
  for (int kc = 0; kc < nkc; kc += 3) {
    step(kc, a_cur, a_2);
    step(kc + 1, a_nxt, a_cur);
    step(kc + 2, a_2, a_nxt);
  }
  // D[i][j]: token i = 8*(v/4) + 4*h + v%4, expert j = n*32 + r
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int j = n * 32 + r;
    if (j < E) {
      const float bj = bias ? bias[j] : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int i = 8 * (v >> 2) + 4 * h + (v & 3);
        zs[i * zs_stride + j] = acc[n][v] + bj;
      }
    }
  }
}

// fp32 logits (VALU): lane (token r, parity h) sums experts e = h, h+2, ...
__device__ __forceinline__ void logits_valu(const float* __restrict__ x,
                                            const float* __restrict__ wrT,
                                            const float* __restrict__ bias,
                                            int64_t T_, int d, int E, int64_t t_w,
                                            float* zs, int zs_stride) {
  const int lane = threadIdx.x & 63, h = lane >> 5, r = lane & 31;
  const int64_t tr = t_w + r;
  if (tr < T_) {
    const float* xrow = x + tr * (int64_t)d;
    for (int e = h; e < E; e += 2) {
      const float* wr = wrT + (int64_t)e * d;
      float acc = 0.0f;
      for (int i = 0; i < d; ++i) acc += xrow[i] * wr[i];
      zs[r * zs_stride + e] = acc + (bias ? bias[e] : 0.0f);
    }
  }
  __syncthreads();
}

template <typename T, int NT, int KL>
__global__ __launch_bounds__(256) void route_kernel(
    const T* __restrict__ x, const T* __restrict__ wrT, const float* __restrict__ bias,
    float* __restrict__ probs, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int64_t T_, int d, int E, int Epad, int k,
    float tau) {
  extern __shared__ __align__(16) unsigned char smem[];
  const RouteSmem L = route_smem(Epad, k, (int)sizeof(T));
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t_w = (int64_t)blockIdx.x * (kRW * kRT) + (int64_t)w * kRT;
  float* zs = reinterpret_cast<float*>(smem + L.zs_off) + (size_t)w * kRT * L.zs_stride;
  float* s_max = reinterpret_cast<float*>(smem + L.stats_off) + w * kRT;
  float* s_sum = s_max + kRW * kRT;
  float* s_thr = s_sum + kRW * kRT;
  int32_t* s_idx = reinterpret_cast<int32_t*>(smem + L.idx_off) + (size_t)w * kRT * k;
  float* s_uz = reinterpret_cast<float*>(smem + L.uz_off) + (size_t)w * Epad;
  int32_t* s_ue = reinterpret_cast<int32_t*>(smem + L.ue_off) + (size_t)w * Epad;

  // ---- phase 1: fast logits
  if constexpr (sizeof(T) == 2) {
    logits_mfma<NT>(reinterpret_cast<const uint16_t*>(x),
                    reinterpret_cast<const uint16_t*>(wrT), bias, T_, d, E, t_w,
                    reinterpret_cast<uint16_t*>(smem + L.zs_off), zs, L.zs_stride);
    __syncthreads();
  } else {
    logits_valu(reinterpret_cast<const float*>(x), reinterpret_cast<const float*>(wrT),
                bias, T_, d, E, t_w, zs, L.zs_stride);
  }

  // ---- phase 2: softmax statistics and top-(k+1) of the fast logits
  bool flag = false;
  if (lane < kRT && t_w + lane < T_) {
    const float* zr = zs + lane * L.zs_stride;
    float m = -FLT_MAX;
    for (int e = 0; e < E; ++e) m = fmaxf(m, zr[e]);
    float ssum = 0.0f;
    for (int e = 0; e < E; ++e) ssum += expf(zr[e] - m);
    float val[KL];
    int id[KL];
#pragma unroll
    for (int q = 0; q < KL; ++q) { val[q] = -INFINITY; id[q] = 0x7fffffff; }
    for (int e = 0; e < E; ++e) {
      float v = zr[e];
      int ie = e;
#pragma unroll
      for (int q = 0; q < KL; ++q) {
        const bool before = v > val[q] || (v == val[q] && ie < id[q]);
        if (before) {
          const float tv = val[q]; val[q] = v; v = tv;
          const int ti = id[q]; id[q] = ie; ie = ti;
        }
      }
    }
    const int ngap = E > k ? k : k - 1;
    float vk = -INFINITY;
#pragma unroll
    for (int q = 0; q < KL; ++q) {
      if (q < ngap && q + 1 < KL && val[q] - val[q + 1] < tau) flag = true;
      if (q == k) vk = val[q];
      if (q < k) s_idx[lane * k + q] = id[q];
    }
    s_max[lane] = m;
    s_sum[lane] = ssum;
    s_thr[lane] = E > k ? vk - tau : -INFINITY;
  }
  __syncthreads();

  // ---- phase 3: canonical fp64 rescoring where the fast order is uncertain
  uint64_t fm = __ballot(flag);
  while (fm) {
    const int tl = __builtin_ctzll(fm);
    fm &= fm - 1;
    const int64_t t = t_w + tl;
    const float thr = s_thr[tl];
    int nU = 0;
    for (int base = 0; base < E; base += 64) {
      const int e = base + lane;
      const bool in = e < E && zs[tl * L.zs_stride + e] >= thr;
      uint64_t um = __ballot(in);
      while (um) {
        const int ee = base + __builtin_ctzll(um);
        um &= um - 1;
        // fp64 dot product of the token row with the expert's weights:
        // 16-byte vectors, every lane's loads issued before their use
        constexpr int V = St<T>::kVec;
        const T* xr = x + t * (int64_t)d;
        const T* wr = wrT + (int64_t)ee * d;
        const int nch = d / V;
        double acc = 0.0;
        for (int c0 = lane; c0 < nch; c0 += 4 * 64) {
          u32x4 xv[4], wv[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int c = c0 + q * 64;
            if (c < nch) {
              xv[q] = ld16(xr + c * V);
              wv[q] = ld16(wr + c * V);
            }
          }
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (c0 + q * 64 >= nch) continue;
            float xf[V], wf[V];
            St<T>::unpack(xv[q], xf);
            St<T>::unpack(wv[q], wf);
#pragma unroll
            for (int i = 0; i < V; ++i) acc += (double)xf[i] * (double)wf[i];
          }
        }
        acc = wave_sum_d(acc);
        if (lane == 0) {
          s_uz[nU] = (float)(acc + (double)(bias ? bias[ee] : 0.0f));
          s_ue[nU] = ee;
        }
        ++nU;
      }
    }
    if (lane == 0) {
      for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int u = 0; u < nU; ++u) {
          if (s_ue[u] < 0) continue;
          if (best < 0 || s_uz[u] > s_uz[best] ||
              (s_uz[u] == s_uz[best] && s_ue[u] < s_ue[best]))
            best = u;
        }
        s_idx[tl * k + j] = s_ue[best];
        s_ue[best] = -1;
      }
    }
  }
  __syncthreads();

  // ---- phase 4: probabilities, chosen experts and gates (coalesced writes)
  const int64_t rem = T_ - t_w;
  const int nvalid = rem <= 0 ? 0 : (rem < kRT ? (int)rem : kRT);
  for (int o = lane; o < nvalid * E; o += 64) {
    const int tt = o / E, e = o - tt * E;
    probs[(t_w + tt) * E + e] = expf(zs[tt * L.zs_stride + e] - s_max[tt]) / s_sum[tt];
  }
  for (int o = lane; o < nvalid * k; o += 64) {
    const int tt = o / k, j = o - tt * k;
    const int e = s_idx[tt * k + j];
    idx_out[(t_w + tt) * k + j] = e;
    gate_out[(t_w + tt) * k + j] = expf(zs[tt * L.zs_stride + e] - s_max[tt]) / s_sum[tt];
  }
}

template <typename T, int NT, int KL>
int launch_route_t(const moe_cfg& c, const T* x, const T* Wr, const float* b,
                   float* probs, int32_t* idx, float* gate, T* wrT, hipStream_t s) {
  const int Epad = 32 * NT;
  int rc = launch_transpose_wr(c, Wr, wrT, s);
  if (rc != MOE_OK) return rc;
  const float tau = c.route_margin > 0.0f ? c.route_margin : 1e-3f;
  const RouteSmem L = route_smem(Epad, c.k, (int)sizeof(T));
  const int grid = (int)ceil_div(c.T, kRW * kRT);
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
             route_kernel<T, NT, KL><<<grid, 256, L.total, s>>>(
                 x, wrT, b, probs, idx, gate, c.T, c.d, c.E, Epad, c.k, tau));
  return MOE_OK;
}

template <typename T, int NT>
int route_kl(const moe_cfg& c, const T* x, const T* Wr, const float* b, float* probs,
             int32_t* idx, float* gate, T* wrT, hipStream_t s) {
  if (c.k <= 1) return launch_route_t<T, NT, 2>(c, x, Wr, b, probs, idx, gate, wrT, s);
  if (c.k <= 2) return launch_route_t<T, NT, 3>(c, x, Wr, b, probs, idx, gate, wrT, s);
  if (c.k <= 4) return launch_route_t<T, NT, 5>(c, x, Wr, b, probs, idx, gate, wrT, s);
  if (c.k <= 8) return launch_route_t<T, NT, 9>(c, x, Wr, b, probs, idx, gate, wrT, s);
  if (c.k <= 16) return launch_route_t<T, NT, 17>(c, x, Wr, b, probs, idx, gate, wrT, s);
  return launch_route_t<T, NT, 33>(c, x, Wr, b, probs, idx, gate, wrT, s);
}

}  // namespace

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, hipStream_t s) {
  const int Epad = route_epad(c.E);
  const int64_t n = (int64_t)Epad * c.d;
  const int tgrid = (int)std::min<int64_t>(ceil_div(n, 256), 4096);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<uint16_t><<<tgrid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Wr), static_cast<uint16_t*>(wrT), c.d, c.E,
                   Epad));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<float><<<tgrid, 256, 0, s>>>(
                   static_cast<const float*>(Wr), static_cast<float*>(wrT), c.d, c.E, Epad));
  return MOE_OK;
}

int route_smem_bytes(int E, int k, int elem) {
  return (int)route_smem(route_epad(E), k, elem).total;
}

int launch_route(const moe_cfg& c, const void* x, const void* Wr, const float* b,
                 float* probs, int32_t* idx, float* gate, void* wrT, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const int nt = (c.E + 31) / 32;
  if (c.dtype == MOE_FP32) {
    // VALU logits: only the LDS row stride depends on the padding
    auto xf = static_cast<const float*>(x);
    auto wf = static_cast<const float*>(Wr);
    auto tf = static_cast<float*>(wrT);
    if (nt <= 1) return route_kl<float, 1>(c, xf, wf, b, probs, idx, gate, tf, s);
    if (nt <= 2) return route_kl<float, 2>(c, xf, wf, b, probs, idx, gate, tf, s);
    if (nt <= 4) return route_kl<float, 4>(c, xf, wf, b, probs, idx, gate, tf, s);
    return route_kl<float, 8>(c, xf, wf, b, probs, idx, gate, tf, s);
  }
  auto xb = static_cast<const uint16_t*>(x);
  auto wb = static_cast<const uint16_t*>(Wr);
  auto tb = static_cast<uint16_t*>(wrT);
  if (nt <= 1) return route_kl<uint16_t, 1>(c, xb, wb, b, probs, idx, gate, tb, s);
  if (nt <= 2) return route_kl<uint16_t, 2>(c, xb, wb, b, probs, idx, gate, tb, s);
  if (nt <= 4) return route_kl<uint16_t, 4>(c, xb, wb, b, probs, idx, gate, tb, s);
  return route_kl<uint16_t, 8>(c, xb, wb, b, probs, idx, gate, tb, s);
}

}  // namespace moe
