// Router forward (F1): logits z = x Wr + b, softmax over all experts,
// top-k in the order (z descending, expert ascending), gates = chosen
// probabilities.  Expert-parallel MoE layer, "GPU expert parallel"
// (aicassindra.com), sections "The step timeline" and "Sharded by expert,
// replicated everywhere else" (router decisions must agree on every rank).
//
// Decision rule.  The decision is defined on the canonical logit
// z = RN_fp32(sum_i x_i Wr_ie + b_e) with the sum in fp64.  The fast path
// computes zf with fp32 accumulation.  If every gap between neighbours in
// the top-(k+1) of zf is at least tau, the order of zf is the canonical
// order (|zf - z| < tau/2).  Otherwise every expert whose zf lies within
// tau of the (k+1)-th value or above it is rescored in fp64 and the top-k
// is taken among those: any expert below that band has k+1 experts
// canonically above it.
//
// Two kernels.  The fast logits x Wr come from the grouped GEMM (one group
// of T rows, the transposed router weights as a K-contiguous operand, fp32
// epilogue into a [T, Epad] workspace matrix): the router is a skinny GEMM
// whose cost is reading x once.  The select kernel then takes 32 tokens per
// wave: softmax statistics and top-(k+1) per token (one lane per token),
// fp64 rescoring of uncertain tokens (one wave per token), and coalesced
// writes of probabilities, experts and gates.
#include "gemm.h"

#include <float.h>

namespace moe {

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, int* wl_count,
                        hipStream_t s);

namespace {

struct RouteWorklist {
  int* count;  // number of uncertain tokens
  int* tok;    // [T] their token indices
  int* n;      // [T] their candidate counts
  int* e;      // [T, Epad] their candidate experts, ascending
};

constexpr int kRW = 4;     // waves per block
constexpr int kRT = 32;    // tokens per wave

struct RouteSmem {
  int zs_stride;  // floats per token row of logits
  size_t zs_off, stats_off, idx_off, total;
};

__host__ __device__ inline RouteSmem route_smem(int Epad, int k) {
  RouteSmem m{};
  m.zs_stride = Epad + 1;
  const size_t u = (size_t)kRW * kRT * m.zs_stride * 4;
  m.zs_off = 0;
  m.stats_off = (u + 15) / 16 * 16;
  m.idx_off = m.stats_off + (size_t)3 * kRW * kRT * 4;
  m.total = m.idx_off + (size_t)kRW * kRT * k * 4;
  return m;
}

// wrT[e][i] = Wr[i][e] for e < E, zero rows for E <= e < Epad.
template <typename T>
__global__ void transpose_wr_kernel(const T* __restrict__ Wr, T* __restrict__ wrT,
                                    int d, int E, int Epad, int* __restrict__ wl_count) {
  if (wl_count && blockIdx.x == 0 && threadIdx.x == 0) *wl_count = 0;
  const int64_t n = (int64_t)Epad * d;
  for (int64_t o = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int e = (int)(o / d), i = (int)(o - (int64_t)e * d);
    wrT[o] = e < E ? Wr[(int64_t)i * E + e] : T(0);
  }
}

template <typename T, int KL>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ zf, const T* __restrict__ x, const T* __restrict__ wrT,
    const float* __restrict__ bias, float* __restrict__ probs, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int* __restrict__ wl_count, int* __restrict__ wl_tok,
    int* __restrict__ wl_n, int* __restrict__ wl_e, int64_t T_, int d, int E, int Epad, int k,
    float tau) {
  extern __shared__ __align__(16) unsigned char smem[];
  const RouteSmem L = route_smem(Epad, k);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t t_w = (int64_t)blockIdx.x * (kRW * kRT) + (int64_t)w * kRT;
  float* zs = reinterpret_cast<float*>(smem + L.zs_off) + (size_t)w * kRT * L.zs_stride;
  float* s_max = reinterpret_cast<float*>(smem + L.stats_off) + w * kRT;
  float* s_sum = s_max + kRW * kRT;
  float* s_thr = s_sum + kRW * kRT;
  int32_t* s_idx = reinterpret_cast<int32_t*>(smem + L.idx_off) + (size_t)w * kRT * k;

  // ---- phase 1: fast logits of the wave's tokens (+ bias) into LDS
  {
    const int64_t rem = T_ - t_w;
    const int nv = rem <= 0 ? 0 : (rem < kRT ? (int)rem : kRT);
    for (int o = lane; o < nv * E; o += kWave) {
      const int tt = o / E, e = o - tt * E;
      zs[tt * L.zs_stride + e] = zf[(t_w + tt) * Epad + e] + (bias ? bias[e] : 0.0f);
    }
  }
  __syncthreads();

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

  // ---- phase 3: tokens whose fast order is uncertain go to the rescoring
  // worklist with their candidate experts (ascending); their idx and gate
  // written below are provisional and replaced by route_rescore_kernel
  uint64_t fm = __ballot(flag);
  while (fm) {
    const int tl = __builtin_ctzll(fm);
    fm &= fm - 1;
    const float thr = s_thr[tl];
    int slot = 0;
    if (lane == 0) slot = atomicAdd(wl_count, 1);
    slot = __shfl(slot, 0, kWave);
    int n = 0;
    for (int base = 0; base < E; base += kWave) {
      const int e = base + lane;
      const bool in = e < E && zs[tl * L.zs_stride + e] >= thr;
      const uint64_t um = __ballot(in);
      if (in) wl_e[(int64_t)slot * Epad + n + __popcll(um & ((1ull << lane) - 1ull))] = e;
      n += __popcll(um);
    }
    if (lane == 0) {
      wl_tok[slot] = (int)(t_w + tl);
      wl_n[slot] = n;
    }
  }

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

// Canonical rescoring of the worklist: one wave per uncertain token.  Each
// candidate's logit is RN_fp32(fp64 sum of x_i Wr_ie + b_e), two candidates
// at a time with all their 16-byte loads in flight; then the top-k among
// the candidates (z descending, expert ascending) replaces the token's
// provisional experts and gates.  wl_z (the fast-logit workspace, no longer
// needed) holds the canonical logits.
template <typename T>
__global__ __launch_bounds__(256) void route_rescore_kernel(
    const int* __restrict__ wl_count, const int* __restrict__ wl_tok,
    const int* __restrict__ wl_n, const int* __restrict__ wl_e, float* __restrict__ wl_z,
    const T* __restrict__ x, const T* __restrict__ wrT, const float* __restrict__ bias,
    const float* __restrict__ probs, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int d, int E, int Epad, int k) {
  constexpr int V = St<T>::kVec;
  constexpr int CPL = 4;  // 16-byte chunks per lane per pass
  const int lane = threadIdx.x & 63;
  const int count = *wl_count;
  const int nch = d / V;
  for (int slot = blockIdx.x * 4 + (threadIdx.x >> 6); slot < count; slot += gridDim.x * 4) {
    const int64_t t = wl_tok[slot];
    const int n = wl_n[slot];
    const int* cand = wl_e + (int64_t)slot * Epad;
    float* cz = wl_z + (int64_t)slot * Epad;
    const T* xr = x + t * d;
    for (int c0 = 0; c0 < n; c0 += 2) {
      const int e0 = cand[c0];
      const int e1 = c0 + 1 < n ? cand[c0 + 1] : e0;
      const T* w0 = wrT + (int64_t)e0 * d;
      const T* w1 = wrT + (int64_t)e1 * d;
      double a0 = 0.0, a1 = 0.0;
      for (int g = lane; g < nch; g += CPL * kWave) {
        u32x4 xv[CPL], v0[CPL], v1[CPL];
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          const int c = g + q * kWave;
          if (c < nch) {
            xv[q] = ld16(xr + c * V);
            v0[q] = ld16(w0 + c * V);
            v1[q] = ld16(w1 + c * V);
          }
        }
#pragma unroll
        for (int q = 0; q < CPL; ++q) {
          if (g + q * kWave >= nch) continue;
          float xf[V], f0[V], f1[V];
          St<T>::unpack(xv[q], xf);
          St<T>::unpack(v0[q], f0);
          St<T>::unpack(v1[q], f1);
#pragma unroll
          for (int i = 0; i < V; ++i) {
            a0 += (double)xf[i] * (double)f0[i];
            a1 += (double)xf[i] * (double)f1[i];
          }
        }
      }
      a0 = wave_sum_d(a0);
      a1 = wave_sum_d(a1);
      if (lane == 0) {
        cz[c0] = (float)(a0 + (double)(bias ? bias[e0] : 0.0f));
        if (c0 + 1 < n) cz[c0 + 1] = (float)(a1 + (double)(bias ? bias[e1] : 0.0f));
      }
    }
    if (lane == 0) {
      uint64_t used[4] = {0, 0, 0, 0};  // n <= Epad <= 256
      for (int j = 0; j < k; ++j) {
        int best = -1;
        float bz = 0.0f;
        int be = 0;
        for (int u = 0; u < n; ++u) {
          if ((used[u >> 6] >> (u & 63)) & 1ull) continue;
          const float zu = cz[u];
          const int eu = cand[u];
          if (best < 0 || zu > bz || (zu == bz && eu < be)) {
            best = u;
            bz = zu;
            be = eu;
          }
        }
        used[best >> 6] |= 1ull << (best & 63);
        idx_out[t * k + j] = be;
        gate_out[t * k + j] = probs[t * E + be];
      }
    }
  }
}

template <typename T, int KL>
int launch_route_t(const moe_cfg& c, const T* x, const T* Wr, const float* b, float* probs,
                   int32_t* idx, float* gate, T* wrT, float* zf, const RouteWorklist& wl,
                   hipStream_t s) {
  const int Epad = route_epad(c.E);
  int rc = launch_transpose_wr(c, Wr, wrT, wl.count, s);
  if (rc != MOE_OK) return rc;
  // zf = x wrT^T: one group of T rows, N = Epad, K = d
  GemmArgs g{};
  g.E = 1;
  g.M = (int)c.T;
  g.N = Epad;
  g.K = c.d;
  g.A = x;
  g.lda = c.d;
  g.B = wrT;
  g.ldb = c.d;
  g.C = zf;
  g.ldc = Epad;
  g.bn = Epad <= 64 ? 64 : 128;
  g.bm = ceil_div(c.T, 128) * ceil_div(Epad, g.bn) >= 256 ? 128 : 64;
  rc = launch_gemm(MOE_KERNEL_ROUTE_LOGITS, MODE_ROW, true, EPI_F32, c, g, s);
  if (rc != MOE_OK) return rc;
  const float tau = c.route_margin > 0.0f ? c.route_margin : 1e-3f;
  const RouteSmem L = route_smem(Epad, c.k);
  const int grid = (int)ceil_div(c.T, kRW * kRT);
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
             route_kernel<T, KL><<<grid, 256, L.total, s>>>(
                 zf, x, wrT, b, probs, idx, gate, wl.count, wl.tok, wl.n, wl.e, c.T, c.d,
                 c.E, Epad, c.k, tau));
  const int rgrid = (int)std::min<int64_t>(ceil_div(c.T, 4), 2048);
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
             route_rescore_kernel<T><<<rgrid, 256, 0, s>>>(
                 wl.count, wl.tok, wl.n, wl.e, zf, x, wrT, b, probs, idx, gate, c.d, c.E,
                 Epad, c.k));
  return MOE_OK;
}

template <typename T>
int route_kl(const moe_cfg& c, const T* x, const T* Wr, const float* b, float* probs,
             int32_t* idx, float* gate, T* wrT, float* zf, const RouteWorklist& wl,
             hipStream_t s) {
  if (c.k <= 1) return launch_route_t<T, 2>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
  if (c.k <= 2) return launch_route_t<T, 3>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
  if (c.k <= 4) return launch_route_t<T, 5>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
  if (c.k <= 8) return launch_route_t<T, 9>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
  if (c.k <= 16) return launch_route_t<T, 17>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
  return launch_route_t<T, 33>(c, x, Wr, b, probs, idx, gate, wrT, zf, wl, s);
}

}  // namespace

int launch_transpose_wr(const moe_cfg& c, const void* Wr, void* wrT, int* wl_count,
                        hipStream_t s) {
  const int Epad = route_epad(c.E);
  const int64_t n = (int64_t)Epad * c.d;
  const int tgrid = (int)std::min<int64_t>(ceil_div(n, 256), 4096);
  if (c.dtype == MOE_BF16)
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<uint16_t><<<tgrid, 256, 0, s>>>(
                   static_cast<const uint16_t*>(Wr), static_cast<uint16_t*>(wrT), c.d, c.E,
                   Epad, wl_count));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE_PREP, s,
               transpose_wr_kernel<float><<<tgrid, 256, 0, s>>>(
                   static_cast<const float*>(Wr), static_cast<float*>(wrT), c.d, c.E, Epad,
                   wl_count));
  return MOE_OK;
}

int route_smem_bytes(int E, int k) {
  return (int)route_smem(route_epad(E), k).total;
}

int launch_route(const moe_cfg& c, const void* x, const void* Wr, const float* b,
                 float* probs, int32_t* idx, float* gate, void* ws, hipStream_t s) {
  if (c.T == 0) return MOE_OK;
  const WsLayout L = ws_layout(c);
  RouteWorklist wl;
  wl.count = ws_ptr<int>(ws, L.wl_count);
  wl.tok = ws_ptr<int>(ws, L.wl_tok);
  wl.n = ws_ptr<int>(ws, L.wl_n);
  wl.e = ws_ptr<int>(ws, L.wl_e);
  float* zf = ws_ptr<float>(ws, L.zf);
  if (c.dtype == MOE_FP32)
    return route_kl<float>(c, static_cast<const float*>(x), static_cast<const float*>(Wr), b,
                           probs, idx, gate, ws_ptr<float>(ws, L.wrT), zf, wl, s);
  return route_kl<uint16_t>(c, static_cast<const uint16_t*>(x),
                            static_cast<const uint16_t*>(Wr), b, probs, idx, gate,
                            ws_ptr<uint16_t>(ws, L.wrT), zf, wl, s);
}

}  // namespace moe
