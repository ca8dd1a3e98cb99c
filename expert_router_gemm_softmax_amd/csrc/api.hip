// C-ABI of the MoE layer library: argument validation, workspace layout and
// the step sequence of the layer forward and backward.  Every entry point validates everything before it enqueues
// anything; on an error nothing is enqueued and nothing is written.
#include <float.h>
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "common.h"

namespace moe {

namespace {
thread_local char g_last_error[160] = "";
}  // namespace

void note_launch_error(int kid, hipError_t e) {
  snprintf(g_last_error, sizeof g_last_error, "kernel %d: %s (%s)", kid, hipGetErrorName(e),
           hipGetErrorString(e));
}

// ------------------------------------------------------------------ validation
namespace {

// Drop error state left by earlier HIP calls that are not this library's,
// so that the checks after our launches see only our launches.
inline void clear_stale_error() {
  (void)hipGetLastError();
  g_last_error[0] = '\0';
}

int check_cfg(const moe_cfg* c) {
  if (!c) return MOE_ERR_ARG;
  if (c->dtype != MOE_FP32 && c->dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (c->T < 0 || c->T > 0x7fffffffLL) return MOE_ERR_ARG;
  if (c->k < 1 || c->k > 32 || c->E < c->k || c->E > 256) return MOE_ERR_ARG;
  if (c->d < 1 || c->f < 1) return MOE_ERR_ARG;
  if (c->capacity < MOE_NO_CAPACITY) return MOE_ERR_ARG;
  if ((c->flags & ~(MOE_FLAG_RECOMPUTE | MOE_FLAG_RENORM | MOE_FLAG_SLOT_PRIORITY |
                    MOE_FLAG_DROP_IDENTITY)) != 0)
    return MOE_ERR_ARG;
  if (c->T * c->k > 0x7fffffffLL) return MOE_ERR_SHAPE;
  if (!(c->route_margin == c->route_margin)) return MOE_ERR_ARG;  // NaN
  if (!(c->aux_coeff >= 0.0f && c->aux_coeff <= FLT_MAX)) return MOE_ERR_ARG;  // NaN, <0, inf
  if (c->probe) {
    const moe_probe* p = c->probe;
    if (p->kernel_id < 0 || p->kernel_id >= MOE_KERNEL_COUNT_ || p->capacity < 0 ||
        p->count < 0 || (p->capacity > 0 && (!p->begin || !p->end)))
      return MOE_ERR_ARG;
  }
  const size_t s = elem_bytes(*c);
  if ((c->d * s) % 16 != 0 || (c->f * s) % 16 != 0) return MOE_ERR_ALIGN;
  return MOE_OK;
}

// a tensor of `bytes` bytes: NULL only if empty; `align`-byte aligned
int need(const void* p, size_t bytes, size_t align) {
  if (bytes == 0) return MOE_OK;
  if (!p) return MOE_ERR_ARG;
  if (reinterpret_cast<uintptr_t>(p) % align != 0) return MOE_ERR_ALIGN;
  return MOE_OK;
}

int need_ws(const moe_cfg& c, const void* ws, size_t ws_bytes) {
  const size_t want = ws_layout(c).total;
  if (ws_bytes < want) return MOE_ERR_WORKSPACE;
  return need(ws, want, 256);
}

#define MOE_TRY(expr)            \
  do {                           \
    const int rc_ = (expr);      \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

struct Sizes {
  size_t s, Td, TE, Tk, E1, Rd, Rf, Edf, dE, Rmax;
};
Sizes sizes(const moe_cfg& c) {
  Sizes z;
  z.s = elem_bytes(c);
  z.Rmax = (size_t)rows_max(c);
  z.Td = (size_t)c.T * c.d * z.s;
  z.TE = (size_t)c.T * c.E * 4;
  z.Tk = (size_t)c.T * c.k * 4;
  z.E1 = (size_t)(c.E + 1) * 4;
  z.Rd = z.Rmax * c.d * z.s;
  z.Rf = z.Rmax * c.f * z.s;
  z.Edf = (size_t)c.E * c.d * c.f * z.s;
  z.dE = (size_t)c.d * c.E * z.s;
  return z;
}

inline hipStream_t S(moe_stream_t s) { return reinterpret_cast<hipStream_t>(s); }

// A and H are caller buffers unless the recomputation mode keeps them in
// the workspace
inline bool saves_ah(const moe_cfg& c) { return (c.flags & MOE_FLAG_RECOMPUTE) == 0; }
// the identity fallback of dropped assignments reads x, gate and dOut
inline bool fallback(const moe_cfg& c) { return (c.flags & MOE_FLAG_DROP_IDENTITY) != 0; }

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_capacity(int64_t T, int32_t k, int32_t E, double cf) {
  if (!(cf >= 0.0) || isinf(cf) || E <= 0 || T < 0 || k < 0) return MOE_NO_CAPACITY;
  if (k > 0 && T > INT64_MAX / k) return MOE_NO_CAPACITY;  // T*k not representable
  const int64_t tk = T * (int64_t)k;
  if (tk == 0 || cf == 0.0) return 0;
  // C >= T*k keeps every assignment: saturate there (cf >= E suffices)
  if (cf >= (double)E) return tk;
  // The factor is read as its shortest decimal that converts back to the
  // same double (what a user typed, e.g. 1.1 rather than the binary value
  // just above it): digits M and exponent q with cf = M * 10^q.
  char buf[40];
  int p = 1;
  for (; p <= 17; ++p) {
    snprintf(buf, sizeof buf, "%.*e", p - 1, cf);
    if (strtod(buf, nullptr) == cf) break;
  }
  if (p > 17) p = 17;
  snprintf(buf, sizeof buf, "%.*e", p - 1, cf);
  // buf = "D.DDDDe[+-]X": mantissa digits, then the decimal exponent
  unsigned __int128 M = 0;
  int nd = 0;
  const char* c = buf;
  for (; *c && *c != 'e'; ++c)
    if (*c >= '0' && *c <= '9') {
      M = M * 10 + (unsigned)(*c - '0');
      ++nd;
    }
  const int q = atoi(c + 1) - (nd - 1);
  // C = ceil(M * 10^q * T * k / E) in exact integer arithmetic: M < 2^57
  // and T k < 2^63, so M T k < 2^120; for q > 0, M 10^q = cf < E < 2^31.
  unsigned __int128 num = M * (unsigned __int128)tk;
  unsigned __int128 den = (unsigned __int128)E;
  if (q >= 0) {
    for (int i = 0; i < q; ++i) num *= 10;
  } else {
    for (int i = 0; i < -q; ++i) {
      // den past 2^120 exceeds num: 0 < value < 1, so C = 1
      if (den > ((unsigned __int128)1 << 120)) return 1;
      den *= 10;
    }
  }
  const unsigned __int128 C = (num + den - 1) / den;
  return C >= (unsigned __int128)tk ? tk : (int64_t)C;
}

int64_t moe_rows_max(const moe_cfg* cfg) {
  if (check_cfg(cfg) != MOE_OK) return -1;
  return rows_max(*cfg);
}

size_t moe_workspace_bytes(const moe_cfg* cfg) {
  if (check_cfg(cfg) != MOE_OK) return 0;
  return ws_layout(*cfg).total;
}

int moe_check_cfg(const moe_cfg* cfg) { return check_cfg(cfg); }

const char* moe_status_str(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (null pointer or out-of-range value)";
    case MOE_ERR_DTYPE: return "unknown dtype";
    case MOE_ERR_SHAPE: return "inconsistent or too large shape";
    case MOE_ERR_ALIGN: return "row or pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_bytes(cfg)";
    case MOE_ERR_LAUNCH: return "kernel launch failed";
    case MOE_ERR_UNIMPLEMENTED: return "not implemented";
    default: return "unknown status";
  }
}

int moe_route(const moe_cfg* cfg, const void* x, const void* Wr, const float* b,
              float* probs, int32_t* idx, float* gate, void* ws, size_t ws_bytes,
              moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(Wr, z.dE, 4));
  if (b) MOE_TRY(need(b, (size_t)c.E * 4, 4));
  MOE_TRY(need(probs, z.TE, 4));
  MOE_TRY(need(idx, z.Tk, 4));
  MOE_TRY(need(gate, z.Tk, 4));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_route(c, x, Wr, b, probs, idx, gate, ws, S(stream));
}

int moe_permute(const moe_cfg* cfg, const void* x, const int32_t* idx, int32_t* counts,
                int32_t* offsets, int32_t* row_of, int32_t* src_of, void* x_perm, void* ws,
                size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(idx, z.Tk, 4));
  MOE_TRY(need(counts, (size_t)c.E * 4, 4));
  MOE_TRY(need(offsets, z.E1, 4));
  MOE_TRY(need(row_of, z.Tk, 4));
  MOE_TRY(need(src_of, z.Rmax * 4, 4));
  MOE_TRY(need(x_perm, z.Rd, 16));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_permute(c, x, idx, counts, offsets, row_of, src_of, x_perm, ws, S(stream));
}

int moe_permute_noalloc(const moe_cfg* cfg, const void* x, const int32_t* idx,
                        int32_t* counts, int32_t* offsets, int32_t* row_of, int32_t* src_of,
                        void* x_perm, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(idx, z.Tk, 4));
  MOE_TRY(need(counts, (size_t)c.E * 4, 4));
  MOE_TRY(need(offsets, z.E1, 4));
  MOE_TRY(need(row_of, z.Tk, 4));
  MOE_TRY(need(src_of, z.Rmax * 4, 4));
  MOE_TRY(need(x_perm, z.Rd, 16));
  clear_stale_error();
  if (permute_noalloc_scratch_bytes(c) > permute_noalloc_scratch_max()) {
    snprintf(g_last_error, sizeof g_last_error,
             "moe_permute_noalloc: %zu bytes of scratch needed, %zu available",
             permute_noalloc_scratch_bytes(c), permute_noalloc_scratch_max());
    return MOE_ERR_WORKSPACE;
  }
  return launch_permute_noalloc(c, x, idx, counts, offsets, row_of, src_of, x_perm,
                                S(stream));
}

int moe_grouped_ffn(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                    const void* W1, const void* W2, void* A, void* H, void* Y, void* ws,
                    size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x_perm, z.Rd, 16));
  MOE_TRY(need(offsets, z.E1, 4));
  MOE_TRY(need(W1, z.Edf, 16));
  MOE_TRY(need(W2, z.Edf, 16));
  if (saves_ah(c)) {
    MOE_TRY(need(A, z.Rf, 16));
    MOE_TRY(need(H, z.Rf, 16));
  }
  MOE_TRY(need(Y, z.Rd, 16));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_ffn_fwd(c, x_perm, offsets, W1, W2, A, H, Y, ws, S(stream));
}

int moe_combine(const moe_cfg* cfg, const void* Y, const int32_t* row_of, const float* gate,
                const void* x, void* out, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(Y, z.Rd, 16));
  MOE_TRY(need(row_of, z.Tk, 4));
  MOE_TRY(need(gate, z.Tk, 4));
  if (fallback(c)) MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(out, z.Td, 16));
  clear_stale_error();
  return launch_combine(c, Y, row_of, gate, x, out, S(stream));
}

int moe_combine_bwd(const moe_cfg* cfg, const void* dOut, const void* Y,
                    const int32_t* row_of, const float* gate, const void* x, void* dYp,
                    float* dgate, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(dOut, z.Td, 16));
  MOE_TRY(need(Y, z.Rd, 16));
  MOE_TRY(need(row_of, z.Tk, 4));
  MOE_TRY(need(gate, z.Tk, 4));
  if (fallback(c)) MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(dYp, z.Rd, 16));
  MOE_TRY(need(dgate, z.Tk, 4));
  clear_stale_error();
  return launch_combine_bwd(c, dOut, Y, row_of, gate, x, dYp, dgate, S(stream));
}

int moe_grouped_ffn_bwd(const moe_cfg* cfg, const void* x_perm, const int32_t* offsets,
                        const void* W1, const void* W2, const void* A, const void* H,
                        const void* dYp, void* dXp, void* dW1, void* dW2, void* ws,
                        size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x_perm, z.Rd, 16));
  MOE_TRY(need(offsets, z.E1, 4));
  MOE_TRY(need(W1, z.Edf, 16));
  MOE_TRY(need(W2, z.Edf, 16));
  if (saves_ah(c)) {
    MOE_TRY(need(A, z.Rf, 16));
    MOE_TRY(need(H, z.Rf, 16));
  }
  MOE_TRY(need(dYp, z.Rd, 16));
  MOE_TRY(need(dXp, z.Rd, 16));
  MOE_TRY(need(dW1, z.Edf, 16));
  MOE_TRY(need(dW2, z.Edf, 16));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_ffn_bwd(c, x_perm, offsets, W1, W2, A, H, dYp, dXp, dW1, dW2, ws,
                        S(stream));
}

int moe_unpermute_bwd(const moe_cfg* cfg, const void* dXp, const int32_t* row_of,
                      const float* gate, const void* dOut, float* dXe, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(dXp, z.Rd, 16));
  MOE_TRY(need(row_of, z.Tk, 4));
  if (fallback(c)) {
    MOE_TRY(need(gate, z.Tk, 4));
    MOE_TRY(need(dOut, z.Td, 16));
  }
  MOE_TRY(need(dXe, (size_t)c.T * c.d * 4, 16));
  clear_stale_error();
  return launch_unpermute_bwd(c, dXp, row_of, gate, dOut, dXe, S(stream));
}

int moe_router_aux(const moe_cfg* cfg, const float* probs, const int32_t* counts,
                   const int32_t* offsets, float* aux, void* ws, size_t ws_bytes,
                   moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(probs, z.TE, 4));
  MOE_TRY(need(counts, (size_t)c.E * 4, 4));
  MOE_TRY(need(offsets, z.E1, 4));
  MOE_TRY(need(aux, 2 * sizeof(float), 4));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_route_aux(c, probs, counts, offsets, aux, ws, S(stream));
}

int moe_route_bwd(const moe_cfg* cfg, const void* x, const void* Wr, const float* probs,
                  const int32_t* idx, const int32_t* row_of, const int32_t* counts,
                  const float* dgate, const float* dXe, void* dX, void* dWr, float* db,
                  void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(Wr, z.dE, 4));
  MOE_TRY(need(probs, z.TE, 4));
  MOE_TRY(need(idx, z.Tk, 4));
  MOE_TRY(need(row_of, z.Tk, 4));
  if (c.aux_coeff > 0.0f) MOE_TRY(need(counts, (size_t)c.E * 4, 4));
  MOE_TRY(need(dgate, z.Tk, 4));
  MOE_TRY(need(dXe, (size_t)c.T * c.d * 4, 16));
  MOE_TRY(need(dX, z.Td, 16));
  MOE_TRY(need(dWr, z.dE, 4));
  if (db) MOE_TRY(need(db, (size_t)c.E * 4, 4));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  clear_stale_error();
  return launch_route_bwd(c, x, Wr, probs, idx, row_of, counts, nullptr, nullptr, dgate,
                          nullptr, dXe, dX, dWr, db, ws, S(stream));
}

static int check_ctx(const moe_cfg& c, const moe_ctx* x) {
  if (!x) return MOE_ERR_ARG;
  const Sizes z = sizes(c);
  MOE_TRY(need(x->probs, z.TE, 4));
  MOE_TRY(need(x->idx, z.Tk, 4));
  MOE_TRY(need(x->gate, z.Tk, 4));
  MOE_TRY(need(x->counts, (size_t)c.E * 4, 4));
  MOE_TRY(need(x->offsets, z.E1, 4));
  MOE_TRY(need(x->row_of, z.Tk, 4));
  MOE_TRY(need(x->src_of, z.Rmax * 4, 4));
  MOE_TRY(need(x->x_perm, z.Rd, 16));
  if (saves_ah(c)) {
    MOE_TRY(need(x->A, z.Rf, 16));
    MOE_TRY(need(x->H, z.Rf, 16));
  }
  MOE_TRY(need(x->Y, z.Rd, 16));
  if (x->aux) MOE_TRY(need(x->aux, 2 * sizeof(float), 4));
  return MOE_OK;
}

static int check_weights(const moe_cfg& c, const moe_weights* w) {
  if (!w) return MOE_ERR_ARG;
  const Sizes z = sizes(c);
  MOE_TRY(need(w->Wr, z.dE, 4));
  if (w->b) MOE_TRY(need(w->b, (size_t)c.E * 4, 4));
  MOE_TRY(need(w->W1, z.Edf, 16));
  MOE_TRY(need(w->W2, z.Edf, 16));
  return MOE_OK;
}

int moe_layer_fwd(const moe_cfg* cfg, const moe_weights* w, const void* x, void* out,
                  const moe_ctx* ctx, void* ws, size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(check_weights(c, w));
  MOE_TRY(check_ctx(c, ctx));
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(out, z.Td, 16));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  const hipStream_t s = S(stream);
  const WsLayout L = ws_layout(c);
  clear_stale_error();
  MOE_TRY(launch_route(c, x, w->Wr, w->b, ctx->probs, ctx->idx, ctx->gate, ws, s));
  // the permute also writes the grouped GEMMs' tile schedule
  int32_t* tiles = ws_ptr<int32_t>(ws, L.tiles);
  MOE_TRY(launch_permute(c, x, ctx->idx, ctx->counts, ctx->offsets, ctx->row_of,
                         ctx->src_of, ctx->x_perm, ws, s, tiles));
  if (ctx->aux)
    MOE_TRY(launch_route_aux(c, ctx->probs, ctx->counts, ctx->offsets, ctx->aux, ws, s));
  MOE_TRY(launch_ffn_fwd(c, ctx->x_perm, ctx->offsets, w->W1, w->W2, ctx->A, ctx->H, ctx->Y,
                         ws, s, /*have_tiles=*/true));
  return launch_combine(c, ctx->Y, ctx->row_of, ctx->gate, x, out, s);
}

int moe_layer_bwd(const moe_cfg* cfg, const moe_weights* w, const void* x, const void* dOut,
                  const moe_ctx* ctx, void* dX, const moe_grads* g, void* ws,
                  size_t ws_bytes, moe_stream_t stream) {
  MOE_TRY(check_cfg(cfg));
  const moe_cfg& c = *cfg;
  const Sizes z = sizes(c);
  MOE_TRY(check_weights(c, w));
  MOE_TRY(check_ctx(c, ctx));
  if (!g) return MOE_ERR_ARG;
  MOE_TRY(need(g->dWr, z.dE, 4));
  if (g->db) MOE_TRY(need(g->db, (size_t)c.E * 4, 4));
  MOE_TRY(need(g->dW1, z.Edf, 16));
  MOE_TRY(need(g->dW2, z.Edf, 16));
  MOE_TRY(need(x, z.Td, 16));
  MOE_TRY(need(dOut, z.Td, 16));
  MOE_TRY(need(dX, z.Td, 16));
  MOE_TRY(need_ws(c, ws, ws_bytes));
  const hipStream_t s = S(stream);
  const WsLayout L = ws_layout(c);
  float* dgate = ws_ptr<float>(ws, L.dgate);
  void* dYp = ws_ptr<void>(ws, L.dYp);
  void* dXp = ws_ptr<void>(ws, L.dXp);
  clear_stale_error();
  // the combine backward also writes the grouped GEMMs' tile schedule and
  // the weight-gradient split plan
  int32_t* tiles = ws_ptr<int32_t>(ws, L.tiles);
  int32_t* plan = c.dtype == MOE_BF16 ? ws_ptr<int32_t>(ws, L.kplan) : nullptr;
  MOE_TRY(launch_combine_bwd(c, dOut, ctx->Y, ctx->row_of, ctx->gate, x, dYp, dgate, s,
                             ctx->offsets, tiles, plan));
  MOE_TRY(launch_ffn_bwd(c, ctx->x_perm, ctx->offsets, w->W1, w->W2, ctx->A, ctx->H, dYp,
                         dXp, g->dW1, g->dW2, ws, s, /*have_tiles=*/true));
  // the unpermute-sum of dXp is fused into the router's dX
  return launch_route_bwd(c, x, w->Wr, ctx->probs, ctx->idx, ctx->row_of, ctx->counts,
                          ctx->gate, dOut, dgate, dXp, nullptr, dX, g->dWr, g->db, ws, s);
}

const char* moe_last_error(void) { return g_last_error; }

}  // extern "C"
