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
// whose cost is reading x once.  The select kernel takes one token per wave
// (lanes across experts): softmax statistics, top-(k+1), coalesced writes of
// probabilities, experts and gates, and the worklist of uncertain tokens;
// the rescoring kernel then certifies those tokens in fp64, one per wave.
// Gates are the chosen probabilities, or (MOE_FLAG_RENORM) those divided by
// their sum taken in selection order; both kernels form them the same way.
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

// Wave argmax over (value, expert) pairs: larger value first, lower
// expert on equal values (-0 == +0).
__device__ __forceinline__ bool route_better(float v, int e, float w, int f) {
  return v > w || (v == w && e < f);
}
// The wave's best (v, e) under route_better, in every lane: DPP exchanges
// within each row of 16, then the four row winners compared in row order
// (route_better is a strict total order, so the pairing does not matter).
template <int CTRL>
__device__ __forceinline__ void argmax_step(float& v, int& e) {
  const float w = dpp_f<CTRL>(v);
  const int f = dpp_i<CTRL>(e);
  if (route_better(w, f, v, e)) {
    v = w;
    e = f;
  }
}
__device__ __forceinline__ void wave_argmax(float& v, int& e) {
  argmax_step<kDppXor1>(v, e);
  argmax_step<kDppXor2>(v, e);
  argmax_step<kDppHalfMirror>(v, e);
  argmax_step<kDppMirror>(v, e);
  float bv = readlane_f(v, 0);
  int be = __builtin_amdgcn_readlane(e, 0);
#pragma unroll
  for (int r = 1; r < 4; ++r) {
    const float w = readlane_f(v, 16 * r);
    const int f = __builtin_amdgcn_readlane(e, 16 * r);
    if (route_better(w, f, bv, be)) {
      bv = w;
      be = f;
    }
  }
  v = bv;
  e = be;
}

// Select: one wave per token, lane l holding experts l, l+64, ... (NS
// slots).  Softmax statistics by wave reductions; the top-(k+1) by k+1
// rounds of a wave argmax; tokens whose adjacent top-(k+1) gaps fall below
// tau go to the rescoring worklist with their candidate experts (fast logit
// >= the (k+1)-th - tau), and their experts and gates written here are
// provisional.
template <int NS>
__global__ __launch_bounds__(256) void route_kernel(
    const float* __restrict__ zf, const float* __restrict__ bias, float* __restrict__ probs,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out, int* __restrict__ wl_count,
    int* __restrict__ wl_tok, int* __restrict__ wl_n, int* __restrict__ wl_e, int64_t T_,
    int E, int Epad, int k, float tau, bool renorm) {
  const int lane = threadIdx.x & 63;
  const int64_t nw = (int64_t)gridDim.x * 4;
  float bz[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const int e = lane + kWave * i;
    bz[i] = (e < E && bias) ? bias[e] : 0.0f;
  }
  for (int64_t t = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); t < T_; t += nw) {
    float z[NS];
    float m = -INFINITY;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = lane + kWave * i;
      z[i] = e < E ? zf[t * Epad + e] + bz[i] : -INFINITY;
      m = fmaxf(m, z[i]);
    }
    m = wave_max(m);
    float ps[NS], sum = 0.0f;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      ps[i] = lane + kWave * i < E ? expf(z[i] - m) : 0.0f;
      sum += ps[i];
    }
    sum = wave_sum(sum);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int e = lane + kWave * i;
      ps[i] = ps[i] / sum;
      if (e < E) probs[t * E + e] = ps[i];
    }
    // top-(k+1): taken experts are marked per slot
    const int nsel = E > k ? k + 1 : k;
    uint32_t taken = 0;
    float vsel_prev = 0.0f, vk = -INFINITY;
    bool flag = false;
    float psel = 0.0f, S = 0.0f;  // lane j: probability of the j-th choice
    for (int j = 0; j < nsel; ++j) {
      float v = -INFINITY;
      int e = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int ei = lane + kWave * i;
        if (ei < E && !((taken >> i) & 1u) && route_better(z[i], ei, v, e)) {
          v = z[i];
          e = ei;
        }
      }
      wave_argmax(v, e);
      if ((e & 63) == lane) taken |= 1u << (e >> 6);
      if (j > 0 && vsel_prev - v < tau) flag = true;
      vsel_prev = v;
      if (j < k) {
        // the owner lane writes the expert; its probability goes to lane j
        float pe = 0.0f;
#pragma unroll
        for (int i = 0; i < NS; ++i)
          if (i == (e >> 6)) pe = ps[i];
        pe = readlane_f(pe, e & 63);  // e is wave-uniform
        S += pe;
        if (lane == j) psel = pe;
        if ((e & 63) == lane) idx_out[t * k + j] = e;
      } else {
        vk = v;
      }
    }
    if (lane < k) gate_out[t * k + lane] = renorm ? psel / S : psel;
    if (flag) {  // uniform over the wave
      const float thr = E > k ? vk - tau : -INFINITY;
      int slot = 0;
      if (lane == 0) slot = atomicAdd(wl_count, 1);
      slot = __builtin_amdgcn_readlane(slot, 0);
      int n = 0;
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int e = lane + kWave * i;
        const bool in = e < E && z[i] >= thr;
        const uint64_t um = __ballot(in);
        if (in) wl_e[(int64_t)slot * Epad + n + __popcll(um & ((1ull << lane) - 1ull))] = e;
        n += __popcll(um);
      }
      if (lane == 0) {
        wl_tok[slot] = (int)t;
        wl_n[slot] = n;
      }
    }
  }
}

constexpr int kRescoreGroup = 4;  // candidates rescored together

// Canonical rescoring of the worklist: one wave per uncertain token.  Each
// candidate's logit is RN_fp32(fp64 sum of x_i Wr_ie + b_e), four
// candidates at a time with all their 16-byte loads in flight; lane u % 64
// keeps candidate u.  Then the top-k among the candidates (z descending,
// expert ascending, by wave argmax) replaces the token's provisional
// experts and gates.
template <typename T>
__global__ __launch_bounds__(256) void route_rescore_kernel(
    const int* __restrict__ wl_count, const int* __restrict__ wl_tok,
    const int* __restrict__ wl_n, const int* __restrict__ wl_e, const T* __restrict__ x, const T* __restrict__ wrT, const float* __restrict__ bias,
    const float* __restrict__ probs, int32_t* __restrict__ idx_out,
    float* __restrict__ gate_out, int d, int E, int Epad, int k, bool renorm) {
  constexpr int V = St<T>::kVec;
  constexpr int CPL = 4;  // 16-byte chunks per lane per pass
  const int lane = threadIdx.x & 63;
  const int count = *wl_count;
  const int nch = d / V;
  for (int slot = blockIdx.x * 4 + (threadIdx.x >> 6); slot < count; slot += gridDim.x * 4) {
    const int64_t t = wl_tok[slot];
    const int n = wl_n[slot];
    const int* cand = wl_e + (int64_t)slot * Epad;
    float cz[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // candidate lane + 64 i, canonical z
    const T* xr = x + t * d;
    for (int c0 = 0; c0 < n; c0 += kRescoreGroup) {
      const T* wr[kRescoreGroup];
      int ec[kRescoreGroup];
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) {
        ec[q] = cand[c0 + q < n ? c0 + q : c0];
        wr[q] = wrT + (int64_t)ec[q] * d;
      }
      double acc[kRescoreGroup];
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) acc[q] = 0.0;
      for (int g = lane; g < nch; g += CPL * kWave) {
        u32x4 xv[CPL], wv[kRescoreGroup][CPL];
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          const int c = g + u * kWave;
          if (c < nch) {
            xv[u] = ld16(xr + c * V);
#pragma unroll
            for (int q = 0; q < kRescoreGroup; ++q) wv[q][u] = ld16(wr[q] + c * V);
          }
        }
#pragma unroll
        for (int u = 0; u < CPL; ++u) {
          if (g + u * kWave >= nch) continue;
          float xf[V];
          St<T>::unpack(xv[u], xf);
#pragma unroll
          for (int q = 0; q < kRescoreGroup; ++q) {
            float wf[V];
            St<T>::unpack(wv[q][u], wf);
#pragma unroll
            for (int i = 0; i < V; ++i) acc[q] += (double)xf[i] * (double)wf[i];
          }
        }
      }
#pragma unroll
      for (int q = 0; q < kRescoreGroup; ++q) {
        const double sum = wave_sum_d(acc[q]);
        const int u = c0 + q;  // lane u % 64 keeps candidate u in slot u / 64
        if (u < n && (u & 63) == lane) {
          const float zc = (float)(sum + (double)(bias ? bias[ec[q]] : 0.0f));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i == (u >> 6)) cz[i] = zc;
        }
      }
    }
    // top-k among the candidates by k rounds of a wave argmax
    int ce[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int u = lane + kWave * i;
      ce[i] = u < n ? cand[u] : 0x7fffffff;
    }
    uint32_t taken = 0;
    float psel = 0.0f, S = 0.0f;  // lane j: probability of the j-th choice
    for (int j = 0; j < k; ++j) {
      float v = -INFINITY;
      int e = 0x7fffffff;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < n && !((taken >> i) & 1u) && route_better(cz[i], ce[i], v, e)) {
          v = cz[i];
          e = ce[i];
        }
      wave_argmax(v, e);
      // the lane holding the winner marks it and writes the expert
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (lane + kWave * i < n && ce[i] == e && !((taken >> i) & 1u)) {
          taken |= 1u << i;
          idx_out[t * k + j] = e;
        }
      const float pe = e < E ? probs[t * E + e] : 0.0f;  // e < E: n >= k candidates
      S += pe;
      if (lane == j) psel = pe;
    }
    if (lane < k) gate_out[t * k + lane] = renorm ? psel / S : psel;
  }
}

template <typename T>
int launch_route_t(const moe_cfg& c, const T* x, const T* Wr, const float* b, float* probs,
                   int32_t* idx, float* gate, T* wrT, float* zf, const RouteWorklist& wl,
                   hipStream_t s) {
  const int Epad = route_epad(c.E);
  const bool renorm = (c.flags & MOE_FLAG_RENORM) != 0;
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
  const int grid = (int)std::min<int64_t>(ceil_div(c.T, 4), 16384);
  if (Epad <= 64)
    MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
               route_kernel<1><<<grid, 256, 0, s>>>(zf, b, probs, idx, gate, wl.count, wl.tok,
                                                    wl.n, wl.e, c.T, c.E, Epad, c.k, tau,
                                                    renorm));
  else if (Epad <= 128)
    MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
               route_kernel<2><<<grid, 256, 0, s>>>(zf, b, probs, idx, gate, wl.count, wl.tok,
                                                    wl.n, wl.e, c.T, c.E, Epad, c.k, tau,
                                                    renorm));
  else
    MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
               route_kernel<4><<<grid, 256, 0, s>>>(zf, b, probs, idx, gate, wl.count, wl.tok,
                                                    wl.n, wl.e, c.T, c.E, Epad, c.k, tau,
                                                    renorm));
  const int rgrid = (int)std::min<int64_t>(ceil_div(c.T, 4), 2048);
  MOE_LAUNCH(MOE_KERNEL_ROUTE, s,
             route_rescore_kernel<T><<<rgrid, 256, 0, s>>>(
                 wl.count, wl.tok, wl.n, wl.e, x, wrT, b, probs, idx, gate, c.d, c.E,
                 Epad, c.k, renorm));
  return MOE_OK;
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
    return launch_route_t<float>(c, static_cast<const float*>(x), static_cast<const float*>(Wr), b,
                           probs, idx, gate, ws_ptr<float>(ws, L.wrT), zf, wl, s);
  return launch_route_t<uint16_t>(c, static_cast<const uint16_t*>(x),
                            static_cast<const uint16_t*>(Wr), b, probs, idx, gate,
                            ws_ptr<uint16_t>(ws, L.wrT), zf, wl, s);
}

}  // namespace moe
