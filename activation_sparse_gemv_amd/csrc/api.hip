// C ABI of libsfnn.so: argument validation, workspace layout and the launch
// sequence of each entry point.  No allocation, no host<->device copies, no
// synchronisation: everything is enqueued on the caller's stream.
#include <algorithm>
#include <mutex>
#include <numeric>
#include <vector>

#include "../../include/sfnn.h"
#include "common.hpp"
#include "launch.hpp"

using namespace sfnn;

namespace {

constexpr size_t kAlign = 256;
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool al16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }
bool al4(const void* p) { return p == nullptr || ((uintptr_t)p & 3u) == 0; }

struct Layout {
  size_t z = 0, hrow = 0, partial = 0, mask = 0, uni = 0, ids = 0, count = 0, rbuf = 0, xbuf = 0, rtmp = 0,
         hbuf = 0, hmax = 0, sid = 0, total = 0;
  int G = 0;
};

// Workspace: predictor stage-1 output z; the per-row FFN's activations h
// (up -> down); the matrix-core FFN's partial rows; masks, union mask, ids,
// count; the residual chain's two fp32 rows and layer input; the matrix-core
// FFN's h (one 32-token pass), its per-step token maxima and slot ids.
Layout layout(const sfnn_pred* p, const sfnn_ffn* f, int batch) {
  Layout L;
  size_t off = 0;
  const int ff = f ? f->d_ff : (p ? p->d_ff : 0);
  const int dm = f ? f->d_model : (p ? p->d_model : 0);
  if (p) {
    // z [B][r], and for fp16 predictors the matrix-core stage 1's partial z
    // of up to kPred1MaxSplits d_model slices right behind it
    L.z = off;
    off += up((size_t)batch * p->rank * 4);
    if (p->wtype == SFNN_F16) off += up((size_t)kPred1MaxSplits * batch * p->rank * 4);
  }
  if (f) {
    L.G = ffn_groups(f->d_model, f->d_ff);
    L.hrow = off;
    off += up((size_t)batch * f->d_ff * 4);
    // matrix-core partial rows, or the per-row down projection's row groups
    L.partial = off;
    off += up((size_t)kMfmaPartRows * batch * f->d_model * 4);
  }
  L.mask = off;
  off += up((size_t)batch * (ff / 64) * 8);
  L.uni = off;
  off += up((size_t)(ff / 64) * 8);
  L.ids = off;
  off += up((size_t)ff * 4);
  L.count = off;
  off += up(4);
  L.rbuf = off;
  off += up((size_t)2 * batch * dm * 4);
  L.xbuf = off;
  off += up((size_t)batch * dm * 4);
  L.rtmp = off;
  off += up((size_t)batch * dm * 4);
  if (f) {
    // matrix-core FFN: h of one 32-token pass (fp32), the largest |h| per
    // 32-slot step and token, and the slot ids
    L.hbuf = off;
    off += up((size_t)32 * f->d_ff * 4);
    L.hmax = off;
    off += up((size_t)(f->d_ff / 32) * 32 * 4);
    L.sid = off;
    off += up((size_t)f->d_ff * 4);
  }
  L.total = off;
  return L;
}

bool batch_ok(int b) { return b >= 1 && b <= 64; }
bool dff_ok(int f) { return f >= 64 && f <= 65536 && f % 64 == 0; }
bool dmodel_ok(int d) { return d >= 128 && d <= 16384 && d % 128 == 0; }

sfnn_status check_pred(const sfnn_pred* p) {
  if (!p || !p->w1_t || !p->w2_t || !p->tau) return SFNN_E_NULL;
  if (p->wtype != SFNN_F32 && p->wtype != SFNN_F16) return SFNN_E_DTYPE;
  if (!dmodel_ok(p->d_model) || !dff_ok(p->d_ff) || p->rank < 8 || p->rank > 2048 || p->rank % 8)
    return SFNN_E_SHAPE;
  if (p->hot_prefix < 0 || p->hot_prefix > p->d_ff || p->hot_prefix % 64) return SFNN_E_SHAPE;
  if (!al16(p->w1_t) || !al16(p->w2_t) || !al16(p->tau)) return SFNN_E_ALIGN;
  return SFNN_OK;
}

sfnn_status check_ffn(const sfnn_ffn* f) {
  if (!f || !f->w_up || !f->w_down_t) return SFNN_E_NULL;
  if (f->wtype != SFNN_F32 && f->wtype != SFNN_F16 && f->wtype != SFNN_I4G128) return SFNN_E_DTYPE;
  if (f->act != SFNN_RELU && f->act != SFNN_REGLU) return SFNN_E_DTYPE;
  if (f->act == SFNN_REGLU && !f->w_gate) return SFNN_E_NULL;
  if (f->wtype == SFNN_I4G128 && (!f->s_up || !f->s_down_t || (f->act == SFNN_REGLU && !f->s_gate)))
    return SFNN_E_NULL;
  if (!dmodel_ok(f->d_model) || !dff_ok(f->d_ff)) return SFNN_E_SHAPE;
  const void* ps[] = {f->w_up, f->w_gate, f->w_down_t, f->s_up, f->s_gate, f->s_down_t,
                      f->b_up, f->b_gate, f->b_down};
  for (const void* q : ps)
    if (!al16(q)) return SFNN_E_ALIGN;
  return SFNN_OK;
}

// The dense switch: from this batch on a layer skips the predictor (a
// positive threshold; zero and negative values never switch).
bool runs_dense(const sfnn_pred* p, int batch) { return p->dense_min_batch > 0 && batch >= p->dense_min_batch; }

int x_type_of_ffn(const sfnn_ffn* f) { return f->wtype == SFNN_F32 ? SFNN_F32 : SFNN_F16; }

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

sfnn_status hip_status(hipError_t e) { return e == hipSuccess ? SFNN_OK : SFNN_E_HIP; }

PredLaunch pred_launch(const sfnn_pred* p, const void* x, int batch, uint64_t* mask, uint64_t* uni,
                       float* logits, float* z) {
  PredLaunch L;
  L.wt = p->wtype == SFNN_F32 ? WT_F32 : WT_F16;
  L.d = p->d_model;
  L.f = p->d_ff;
  L.r = p->rank;
  L.w1_t = p->w1_t;
  L.w2_t = p->w2_t;
  L.tau = p->tau;
  L.x = x;
  L.batch = batch;
  L.z = z;
  if (p->wtype == SFNN_F16) L.zpart = z + up((size_t)batch * p->rank * 4) / 4;  // see layout()
  L.mask = mask;
  L.union_mask = uni;
  L.logits = logits;
  L.hot = p->hot_prefix / 64;
  return L;
}

sfnn_status do_predict(const sfnn_pred* p, const void* x, int batch, uint64_t* mask, uint64_t* uni,
                       float* logits, float* z, hipStream_t s) {
  return hip_status(launch_predict(pred_launch(p, x, batch, mask, uni, logits, z), s));
}

FfnLaunch ffn_launch(const sfnn_ffn* f, const void* x, int batch, const uint64_t* mask, float* y, char* ws,
                     const Layout& Lw) {
  FfnLaunch L;
  L.wt = f->wtype == SFNN_F32 ? WT_F32 : (f->wtype == SFNN_F16 ? WT_F16 : WT_I4);
  L.act = f->act == SFNN_RELU ? ACT_RELU : ACT_REGLU;
  L.d = f->d_model;
  L.f = f->d_ff;
  L.w_up = f->w_up;
  L.w_gate = f->w_gate;
  L.w_down_t = f->w_down_t;
  L.s_up = f->s_up;
  L.s_gate = f->s_gate;
  L.s_down_t = f->s_down_t;
  L.b_up = f->b_up;
  L.b_gate = f->b_gate;
  L.b_down = f->b_down;
  L.x = x;
  L.batch = batch;
  L.src = SRC_DENSE;
  L.ids = nullptr;
  L.count = nullptr;
  L.union_mask = nullptr;
  L.ids_out = nullptr;
  L.count_out = nullptr;
  L.mask = mask;
  L.y = y;
  L.r_in = nullptr;
  L.r_out = nullptr;
  L.hrow = reinterpret_cast<float*>(ws + Lw.hrow);
  L.partial = reinterpret_cast<float*>(ws + Lw.partial);
  L.groups = Lw.G;
  L.hbuf = ws + Lw.hbuf;
  L.hmax = reinterpret_cast<float*>(ws + Lw.hmax);
  L.sidbuf = reinterpret_cast<int32_t*>(ws + Lw.sid);
  L.mfma_min_batch = f->mfma_min_batch;
  return L;
}

}  // namespace

extern "C" {

size_t sfnn_workspace_bytes(const sfnn_pred* pred, const sfnn_ffn* ffn, int32_t batch) {
  if (!batch_ok(batch) || (!pred && !ffn)) return 0;
  if (pred && check_pred(pred) == SFNN_E_SHAPE) return 0;
  if (ffn && check_ffn(ffn) == SFNN_E_SHAPE) return 0;
  return layout(pred, ffn, batch).total;
}

sfnn_status sfnn_predict(const sfnn_pred* pred, const void* x, int32_t batch, uint64_t* mask, float* logits,
                         void* ws, size_t ws_bytes, void* stream) {
  sfnn_status st = check_pred(pred);
  if (st != SFNN_OK) return st;
  if (!x || !mask || !ws) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(mask) || !al16(logits) || !al16(ws)) return SFNN_E_ALIGN;
  const Layout Lw = layout(pred, nullptr, batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  char* w = (char*)ws;
  return do_predict(pred, x, batch, mask, reinterpret_cast<uint64_t*>(w + Lw.uni), logits,
                    reinterpret_cast<float*>(w + Lw.z), as_stream(stream));
}

sfnn_status sfnn_compact(const uint64_t* mask, int32_t batch, int32_t d_ff, int32_t* ids, int32_t* count,
                         uint64_t* union_mask, void* stream) {
  if (!mask || !ids || !count) return SFNN_E_NULL;
  if (!batch_ok(batch) || !dff_ok(d_ff)) return SFNN_E_SHAPE;
  if (!al16(mask) || !al16(ids) || !al4(count) || !al16(union_mask)) return SFNN_E_ALIGN;
  return hip_status(launch_compact(mask, batch, d_ff, ids, count, union_mask, as_stream(stream)));
}

sfnn_status sfnn_sparse_ffn(const sfnn_ffn* ffn, const void* x, int32_t batch, const int32_t* ids,
                            const int32_t* count, const uint64_t* mask, float* y, void* ws, size_t ws_bytes,
                            void* stream) {
  sfnn_status st = check_ffn(ffn);
  if (st != SFNN_OK) return st;
  if (!x || !ids || !count || !y || !ws) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(ids) || !al4(count) || !al16(mask) || !al16(y) || !al16(ws)) return SFNN_E_ALIGN;
  const Layout Lw = layout(nullptr, ffn, batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  FfnLaunch L = ffn_launch(ffn, x, batch, mask, y, (char*)ws, Lw);
  L.src = SRC_IDS;
  L.ids = ids;
  L.count = count;
  return hip_status(launch_ffn(L, as_stream(stream)));
}

sfnn_status sfnn_dense_ffn(const sfnn_ffn* ffn, const void* x, int32_t batch, float* y, void* ws,
                           size_t ws_bytes, void* stream) {
  sfnn_status st = check_ffn(ffn);
  if (st != SFNN_OK) return st;
  if (!x || !y || !ws) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(y) || !al16(ws)) return SFNN_E_ALIGN;
  const Layout Lw = layout(nullptr, ffn, batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  return hip_status(launch_ffn(ffn_launch(ffn, x, batch, nullptr, y, (char*)ws, Lw), as_stream(stream)));
}

static sfnn_status check_pair(const sfnn_pred* pred, const sfnn_ffn* ffn) {
  sfnn_status st = check_pred(pred);
  if (st != SFNN_OK) return st;
  st = check_ffn(ffn);
  if (st != SFNN_OK) return st;
  if (pred->d_model != ffn->d_model || pred->d_ff != ffn->d_ff) return SFNN_E_SHAPE;
  if (pred->wtype != x_type_of_ffn(ffn)) return SFNN_E_DTYPE;
  return SFNN_OK;
}

}  // extern "C"

namespace {

// predict -> compact -> sparse FFN of one layer on a checked workspace w.
sfnn_status run_layer(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x, int32_t batch, float* y,
                      uint64_t* mask, int32_t* ids, int32_t* count, char* w, const Layout& Lw, hipStream_t s) {
  if (!mask) mask = reinterpret_cast<uint64_t*>(w + Lw.mask);
  if (!ids) ids = reinterpret_cast<int32_t*>(w + Lw.ids);
  if (!count) count = reinterpret_cast<int32_t*>(w + Lw.count);
  if (runs_dense(pred, batch)) {
    // past the crossover: every neuron for every token, reported as an all-ones mask
    if (launch_fill_dense(mask, (size_t)batch * (pred->d_ff / 64), ids, 1, pred->d_ff, count, 1, s) != hipSuccess)
      return SFNN_E_HIP;
    return hip_status(launch_ffn(ffn_launch(ffn, x, batch, nullptr, y, w, Lw), s));
  }
  uint64_t* uni = reinterpret_cast<uint64_t*>(w + Lw.uni);
  // predictor (writes the batch's union mask), then the FFN compacts the
  // union in its first kernel and writes ids/count on the way
  sfnn_status st = do_predict(pred, x, batch, mask, uni, nullptr, reinterpret_cast<float*>(w + Lw.z), s);
  if (st != SFNN_OK) return st;
  FfnLaunch L = ffn_launch(ffn, x, batch, batch > 1 ? mask : nullptr, y, w, Lw);
  L.src = SRC_UNION;
  L.union_mask = uni;
  L.ids_out = ids;
  L.count_out = count;
  return hip_status(launch_ffn(L, s));
}

sfnn_status check_layer_args(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x, int32_t batch, float* y,
                             uint64_t* mask, int32_t* ids, int32_t* count) {
  sfnn_status st = check_pair(pred, ffn);
  if (st != SFNN_OK) return st;
  if (!x || !y) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(y) || !al16(mask) || !al16(ids) || !al4(count)) return SFNN_E_ALIGN;
  return SFNN_OK;
}

}  // namespace

// The no-allocation variant's workspace: one array per GPU, held until the
// process ends.  Host code never uses this name as an address (on the host it
// is only a stand-in for the symbol); scratch_ptr() gives each device's own
// address, looked up once per device with that device current.
static __device__ __align__(256) unsigned char scratch[SFNN_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

sfnn_status scratch_ptr(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SFNN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SFNN_E_HIP;
    g_scratch_dev[dev] = ptr;
  }
  *out = static_cast<char*>(g_scratch_dev[dev]);
  return SFNN_OK;
}

}  // namespace

extern "C" {

sfnn_status sfnn_layer(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x, int32_t batch, float* y,
                       uint64_t* mask, int32_t* ids, int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  sfnn_status st = check_layer_args(pred, ffn, x, batch, y, mask, ids, count);
  if (st != SFNN_OK) return st;
  if (!ws) return SFNN_E_NULL;
  if (!al16(ws)) return SFNN_E_ALIGN;
  const Layout Lw = layout(pred, ffn, batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  return run_layer(pred, ffn, x, batch, y, mask, ids, count, (char*)ws, Lw, as_stream(stream));
}

sfnn_status sfnn_layer_noalloc(const sfnn_pred* pred, const sfnn_ffn* ffn, const void* x, int32_t batch, float* y,
                               uint64_t* mask, int32_t* ids, int32_t* count, void* stream) {
  sfnn_status st = check_layer_args(pred, ffn, x, batch, y, mask, ids, count);
  if (st != SFNN_OK) return st;
  const Layout Lw = layout(pred, ffn, batch);
  if (Lw.total > SFNN_NOALLOC_SCRATCH_BYTES) return SFNN_E_WORKSPACE;  // checked before any HIP call
  char* w = nullptr;
  st = scratch_ptr(&w);
  if (st != SFNN_OK) return st;
  return run_layer(pred, ffn, x, batch, y, mask, ids, count, w, Lw, as_stream(stream));
}

sfnn_status sfnn_stack_decode(int32_t n_layers, const sfnn_pred* preds, const sfnn_ffn* ffns, int32_t batch,
                              const float* r_in, float* r_out, float eps, int32_t flags, void* x_cap, float* y_cap,
                              uint64_t* mask_cap, int32_t* ids_cap, int32_t* count_cap, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!preds || !ffns || !r_in || !r_out || !ws) return SFNN_E_NULL;
  if (n_layers < 1 || !batch_ok(batch)) return SFNN_E_SHAPE;
  if (flags & ~SFNN_STACK_LOOKAHEAD) return SFNN_E_SHAPE;
  for (int l = 0; l < n_layers; ++l) {
    const sfnn_status st = check_pair(&preds[l], &ffns[l]);
    if (st != SFNN_OK) return st;
    if (preds[l].d_model != preds[0].d_model || preds[l].d_ff != preds[0].d_ff || preds[l].rank != preds[0].rank ||
        preds[l].wtype != preds[0].wtype || ffns[l].wtype != ffns[0].wtype || ffns[l].act != ffns[0].act)
      return SFNN_E_SHAPE;
  }
  if (!(eps > 0.0f)) return SFNN_E_SHAPE;
  if (!al16(r_in) || !al16(r_out) || !al16(x_cap) || !al16(y_cap) || !al16(mask_cap) || !al16(ids_cap) ||
      !al4(count_cap) || !al16(ws))
    return SFNN_E_ALIGN;
  const Layout Lw = layout(&preds[0], &ffns[0], batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  char* w = (char*)ws;
  hipStream_t s = as_stream(stream);
  const int d = preds[0].d_model, f = preds[0].d_ff, W = f / 64;
  const int xb = preds[0].wtype == SFNN_F32 ? 4 : 2;
  float* rbuf[2] = {reinterpret_cast<float*>(w + Lw.rbuf),
                    reinterpret_cast<float*>(w + Lw.rbuf) + (size_t)batch * d};
  uint64_t* uni = reinterpret_cast<uint64_t*>(w + Lw.uni);
  float* z = reinterpret_cast<float*>(w + Lw.z);
  // per-layer buffers: captures when given, else shared workspace
  auto x_of = [&](int l) -> void* { return x_cap ? (char*)x_cap + (size_t)l * batch * d * xb : (void*)(w + Lw.xbuf); };
  auto m_of = [&](int l) { return mask_cap ? mask_cap + (size_t)l * batch * W : reinterpret_cast<uint64_t*>(w + Lw.mask); };
  auto i_of = [&](int l) { return ids_cap ? ids_cap + (size_t)l * f : reinterpret_cast<int32_t*>(w + Lw.ids); };
  auto c_of = [&](int l) { return count_cap ? count_cap + l : reinterpret_cast<int32_t*>(w + Lw.count); };
  auto y_of = [&](int l) { return y_cap ? y_cap + (size_t)l * batch * d : nullptr; };
  // r_l, the residual entering layer l: r_0 = r_in, r_L = r_out, ping-pong between
  auto r_of = [&](int l) -> float* {
    if (l == 0) return const_cast<float*>(r_in);
    if (l == n_layers) return r_out;
    return rbuf[(l - 1) & 1];
  };
  auto ffn_of = [&](int l) {
    FfnLaunch F = ffn_launch(&ffns[l], x_of(l), batch, batch > 1 ? m_of(l) : nullptr, y_of(l), w, Lw);
    F.src = SRC_UNION;
    F.union_mask = uni;
    F.ids_out = i_of(l);
    F.count_out = c_of(l);
    return F;
  };

  // the dense switch, per layer: such a layer has no predictor and runs the
  // dense FFN; its reports (when captured) are the all-ones mask, 0..f-1, f
  std::vector<char> dense((size_t)n_layers);
  int n_dense = 0;
  for (int l = 0; l < n_layers; ++l) n_dense += dense[l] = runs_dense(&preds[l], batch);
  auto dense_ffn_of = [&](int l) {
    FfnLaunch F = ffn_launch(&ffns[l], x_of(l), batch, nullptr, y_of(l), w, Lw);
    F.r_in = r_of(l);
    F.r_out = r_of(l + 1);
    return F;
  };
  if (n_dense && (mask_cap || ids_cap || count_cap)) {
    if (n_dense == n_layers) {
      if (launch_fill_dense(mask_cap, (size_t)n_layers * batch * W, ids_cap, n_layers, f, count_cap, n_layers, s) !=
          hipSuccess)
        return SFNN_E_HIP;
    } else {
      for (int l = 0; l < n_layers; ++l)
        if (dense[l] && launch_fill_dense(mask_cap ? m_of(l) : nullptr, (size_t)batch * W,
                                          ids_cap ? i_of(l) : nullptr, 1, f, count_cap ? c_of(l) : nullptr, 1,
                                          s) != hipSuccess)
          return SFNN_E_HIP;
    }
  }

  if (n_dense == n_layers) {
    // every layer past its switch: RMSNorm then the dense FFN
    for (int l = 0; l < n_layers; ++l) {
      if (launch_residual_rmsnorm(r_of(l), nullptr, nullptr, batch, d, eps, x_of(l), xb == 4 ? WT_F32 : WT_F16, s) !=
          hipSuccess)
        return SFNN_E_HIP;
      if (launch_ffn(dense_ffn_of(l), s) != hipSuccess) return SFNN_E_HIP;
    }
    return SFNN_OK;
  }

  if (flags & SFNN_STACK_LOOKAHEAD) {
    std::vector<PredLaunch> P((size_t)n_layers);
    std::vector<FfnLaunch> F((size_t)n_layers);
    std::vector<const float*> R((size_t)n_layers + 1);
    for (int l = 0; l < n_layers; ++l) {
      P[l] = pred_launch(&preds[l], nullptr, batch, m_of(l), uni, nullptr, z);
      F[l] = dense[l] ? dense_ffn_of(l) : ffn_of(l);
    }
    for (int l = 0; l <= n_layers; ++l) R[l] = r_of(l);
    return hip_status(launch_stack_lookahead(P.data(), F.data(), R.data(), n_layers, eps,
                                             reinterpret_cast<float*>(w + Lw.rtmp), n_dense ? dense.data() : nullptr,
                                             s));
  }

  for (int l = 0; l < n_layers; ++l) {
    if (dense[l]) {
      if (launch_residual_rmsnorm(r_of(l), nullptr, nullptr, batch, d, eps, x_of(l), xb == 4 ? WT_F32 : WT_F16, s) !=
              hipSuccess ||
          launch_ffn(dense_ffn_of(l), s) != hipSuccess)
        return SFNN_E_HIP;
      continue;
    }
    // x_l = RMSNorm(r_l), built inside the predictor's first kernel
    PredLaunch P = pred_launch(&preds[l], nullptr, batch, m_of(l), uni, nullptr, z);
    P.norm.r_in = r_of(l);
    P.norm.x_out = x_of(l);
    P.norm.eps = eps;
    if (launch_predict(P, s) != hipSuccess) return SFNN_E_HIP;
    // y_l and r_{l+1} = r_l + y_l (the last layer writes the caller's r_out)
    FfnLaunch F = ffn_of(l);
    F.r_in = r_of(l);
    F.r_out = r_of(l + 1);
    if (launch_ffn(F, s) != hipSuccess) return SFNN_E_HIP;
  }
  return SFNN_OK;
}

sfnn_status sfnn_residual_rmsnorm(const float* r_in, const float* y, float* r_out, int32_t batch,
                                  int32_t d_model, float eps, void* x_out, int32_t xtype, void* stream) {
  if (!r_in || !r_out || !x_out) return SFNN_E_NULL;
  if (!batch_ok(batch) || !dmodel_ok(d_model)) return SFNN_E_SHAPE;
  if (xtype != SFNN_F32 && xtype != SFNN_F16) return SFNN_E_DTYPE;
  if (!al16(r_in) || !al16(y) || !al16(r_out) || !al16(x_out)) return SFNN_E_ALIGN;
  return hip_status(launch_residual_rmsnorm(r_in, y, r_out, batch, d_model, eps, x_out,
                                            xtype == SFNN_F32 ? WT_F32 : WT_F16, as_stream(stream)));
}

sfnn_status sfnn_fire_counts(const uint64_t* masks, int32_t n_masks, int32_t d_ff, uint32_t* counts,
                             void* stream) {
  if (!masks || !counts) return SFNN_E_NULL;
  if (n_masks < 1 || !dff_ok(d_ff)) return SFNN_E_SHAPE;
  if (!al16(masks) || !al16(counts)) return SFNN_E_ALIGN;
  return hip_status(launch_fire_counts(masks, n_masks, d_ff, counts, as_stream(stream)));
}

sfnn_status sfnn_hot_first_perm(const uint32_t* counts, int32_t d_ff, int32_t* perm) {
  if (!counts || !perm) return SFNN_E_NULL;
  if (d_ff < 1) return SFNN_E_SHAPE;
  std::vector<int32_t> idx((size_t)d_ff);
  std::iota(idx.begin(), idx.end(), 0);
  std::stable_sort(idx.begin(), idx.end(), [&](int32_t a, int32_t b) { return counts[a] > counts[b]; });
  std::copy(idx.begin(), idx.end(), perm);
  return SFNN_OK;
}

sfnn_status sfnn_dense_min_batch(const uint32_t* counts, int32_t n_profiled, int32_t d_ff, float crossover,
                                 int32_t max_batch, int32_t* out) {
  if (!counts || !out) return SFNN_E_NULL;
  if (n_profiled < 1 || d_ff < 1 || max_batch < 1 || !(crossover > 0.0f && crossover <= 1.0f)) return SFNN_E_SHAPE;
  // q_i = 1 - p_i, the chance a token leaves neuron i off; u(b) = 1 - mean_i q_i^b
  std::vector<double> q((size_t)d_ff), qb((size_t)d_ff, 1.0);
  for (int i = 0; i < d_ff; ++i) {
    if (counts[i] > (uint32_t)n_profiled) return SFNN_E_SHAPE;
    q[i] = 1.0 - (double)counts[i] / (double)n_profiled;
  }
  for (int b = 1; b <= max_batch; ++b) {
    double off = 0.0;  // sum_i q_i^b
    for (int i = 0; i < d_ff; ++i) off += (qb[i] *= q[i]);
    if (1.0 - off / d_ff >= (double)crossover) {
      *out = b;
      return SFNN_OK;
    }
  }
  *out = -1;
  return SFNN_OK;
}

sfnn_status sfnn_gather_rows(const void* src, const int32_t* perm, int32_t n_rows, int64_t row_bytes, void* dst,
                             void* stream) {
  if (!src || !perm || !dst) return SFNN_E_NULL;
  if (n_rows < 1 || row_bytes < 2 || (row_bytes & 1)) return SFNN_E_SHAPE;
  if (!al16(src) || !al16(perm) || !al16(dst)) return SFNN_E_ALIGN;
  // other workgroups write dst rows while row perm[k] of src is read: the two
  // ranges must not overlap (an in-place relayout would race)
  const uintptr_t n = (uintptr_t)n_rows * (uintptr_t)row_bytes;
  const uintptr_t s0 = (uintptr_t)src, d0 = (uintptr_t)dst;
  if (s0 < d0 + n && d0 < s0 + n) return SFNN_E_SHAPE;
  return hip_status(launch_gather_rows(src, perm, n_rows, row_bytes, dst, as_stream(stream)));
}

sfnn_status sfnn_probe_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (!buf || !sink) return SFNN_E_NULL;
  if (bytes < 16 || bytes % 16) return SFNN_E_SHAPE;
  if (!al16(buf) || !al16(sink)) return SFNN_E_ALIGN;
  return hip_status(launch_probe_read(buf, bytes, sink, as_stream(stream)));
}

sfnn_status sfnn_probe_copy(const void* src, void* dst, size_t bytes, void* stream) {
  if (!src || !dst) return SFNN_E_NULL;
  if (bytes < 16 || bytes % 16) return SFNN_E_SHAPE;
  if (!al16(src) || !al16(dst)) return SFNN_E_ALIGN;
  return hip_status(launch_probe_copy(src, dst, bytes, as_stream(stream)));
}

namespace {

constexpr int kIsgMaxGroups = 512;

struct IsgLayout {
  size_t mask = 0, ids = 0, count = 0, partial = 0, hbuf = 0, sid = 0, total = 0;
  int G = 0;
};

IsgLayout isg_layout(const sfnn_isg* op, int batch) {
  IsgLayout L;
  size_t off = 0;
  L.G = isg_groups(op->n_out, kIsgMaxGroups);
  L.mask = off;
  off += up((size_t)(op->n_in / 64) * 8);
  L.ids = off;
  off += up((size_t)op->n_in * 4);
  L.count = off;
  off += up(4);
  L.partial = off;
  off += up((size_t)L.G * batch * op->n_out * 4);
  if (op->wtype == SFNN_F16) {  // matrix-core path: one 32-token pass of h and the slot map
    L.hbuf = off;
    off += up((size_t)32 * op->n_in * 4);
    L.sid = off;
    off += up((size_t)op->n_in * 4);
  }
  L.total = off;
  return L;
}

sfnn_status check_isg(const sfnn_isg* op) {
  if (!op || !op->w_t) return SFNN_E_NULL;
  if (op->wtype != SFNN_F32 && op->wtype != SFNN_F16) return SFNN_E_DTYPE;
  if (op->n_in < 64 || op->n_in > 65536 || op->n_in % 64 || op->n_out < 128 || op->n_out > 65536 ||
      op->n_out % 128)
    return SFNN_E_SHAPE;
  if (!al16(op->w_t) || !al16(op->bias)) return SFNN_E_ALIGN;
  return SFNN_OK;
}

}  // namespace

size_t sfnn_isg_workspace_bytes(const sfnn_isg* op, int32_t batch) {
  if (check_isg(op) == SFNN_E_SHAPE || !op || !batch_ok(batch)) return 0;
  return isg_layout(op, batch).total;
}

namespace {

// The input-sparse GEMV once the arguments are checked; w: its workspace.
IsgLaunch isg_launch_of(const sfnn_isg* op, const void* x, int32_t batch, float* y, int32_t* cols, int32_t* count,
                        char* w, const IsgLayout& Lw, bool listed) {
  IsgLaunch L;
  L.listed = listed;
  L.wt = op->wtype == SFNN_F32 ? WT_F32 : WT_F16;
  L.n_in = op->n_in;
  L.n_out = op->n_out;
  L.w_t = op->w_t;
  L.bias = op->bias;
  L.x = x;
  L.batch = batch;
  L.mask = reinterpret_cast<uint64_t*>(w + Lw.mask);
  L.ids = cols ? cols : reinterpret_cast<int32_t*>(w + Lw.ids);
  L.count = count ? count : reinterpret_cast<int32_t*>(w + Lw.count);
  L.partial = reinterpret_cast<float*>(w + Lw.partial);
  L.groups = Lw.G;
  L.y = y;
  if (op->wtype == SFNN_F16) {
    L.hbuf = w + Lw.hbuf;
    L.sidbuf = reinterpret_cast<int32_t*>(w + Lw.sid);
  }
  return L;
}

sfnn_status run_isg(const sfnn_isg* op, const void* x, int32_t batch, float* y, int32_t* cols, int32_t* count,
                    char* w, const IsgLayout& Lw, hipStream_t s, bool listed = false) {
  return hip_status(launch_isg(isg_launch_of(op, x, batch, y, cols, count, w, Lw, listed), s));
}

// Head-gated projections: shapes the kernels and the input-sparse GEMV accept.
sfnn_status check_heads(const sfnn_heads* op) {
  if (!op || !op->w_qkv || !op->w_o_t) return SFNN_E_NULL;
  if (op->wtype != SFNN_F32 && op->wtype != SFNN_F16) return SFNN_E_DTYPE;
  const long n = (long)op->n_heads * op->head_dim;
  if (!dmodel_ok(op->d_model) || op->n_heads < 1 || op->head_dim < 8 || op->head_dim > 512 ||
      op->head_dim % 8 || n % 64 || n > 65536)
    return SFNN_E_SHAPE;
  if (!al16(op->w_qkv) || !al16(op->b_qkv) || !al16(op->w_o_t) || !al16(op->b_o)) return SFNN_E_ALIGN;
  return SFNN_OK;
}

sfnn_isg isg_of(const sfnn_heads* op) {
  sfnn_isg g;
  g.n_in = op->n_heads * op->head_dim;
  g.n_out = op->d_model;
  g.wtype = op->wtype;
  g.w_t = op->w_o_t;
  g.bias = op->b_o;
  return g;
}

}  // namespace

sfnn_status sfnn_input_sparse_gemv(const sfnn_isg* op, const void* x, int32_t batch, float* y, int32_t* cols,
                                   int32_t* count, void* ws, size_t ws_bytes, void* stream) {
  sfnn_status st = check_isg(op);
  if (st != SFNN_OK) return st;
  if (!x || !y || !ws) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(y) || !al16(cols) || !al4(count) || !al16(ws)) return SFNN_E_ALIGN;
  const IsgLayout Lw = isg_layout(op, batch);
  if (ws_bytes < Lw.total) return SFNN_E_WORKSPACE;
  return run_isg(op, x, batch, y, cols, count, (char*)ws, Lw, as_stream(stream));
}

size_t sfnn_heads_workspace_bytes(const sfnn_heads* op, int32_t batch) {
  if (check_heads(op) == SFNN_E_SHAPE || !op || !batch_ok(batch)) return 0;
  const sfnn_isg g = isg_of(op);
  const size_t gated = up((size_t)batch * g.n_in * (op->wtype == SFNN_F32 ? 4 : 2));
  return gated + isg_layout(&g, batch).total;
}

sfnn_status sfnn_head_qkv(const sfnn_heads* op, const void* x, int32_t batch, const uint64_t* head_mask, float* qkv,
                          void* stream) {
  sfnn_status st = check_heads(op);
  if (st != SFNN_OK) return st;
  if (!x || !head_mask || !qkv) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(x) || !al16(head_mask) || !al16(qkv)) return SFNN_E_ALIGN;
  HeadQkvLaunch L;
  L.wt = op->wtype == SFNN_F32 ? WT_F32 : WT_F16;
  L.d = op->d_model;
  L.H = op->n_heads;
  L.hd = op->head_dim;
  L.w_qkv = op->w_qkv;
  L.b_qkv = op->b_qkv;
  L.x = x;
  L.batch = batch;
  L.head_mask = head_mask;
  L.out = qkv;
  return hip_status(launch_head_qkv(L, as_stream(stream)));
}

sfnn_status sfnn_head_out(const sfnn_heads* op, const void* attn, int32_t batch, const uint64_t* head_mask, float* y,
                          void* ws, size_t ws_bytes, void* stream) {
  sfnn_status st = check_heads(op);
  if (st != SFNN_OK) return st;
  if (!attn || !head_mask || !y || !ws) return SFNN_E_NULL;
  if (!batch_ok(batch)) return SFNN_E_SHAPE;
  if (!al16(attn) || !al16(head_mask) || !al16(y) || !al16(ws)) return SFNN_E_ALIGN;
  if (ws_bytes < sfnn_heads_workspace_bytes(op, batch)) return SFNN_E_WORKSPACE;
  const sfnn_isg g = isg_of(op);
  const int wt = op->wtype == SFNN_F32 ? WT_F32 : WT_F16;
  const size_t gated = up((size_t)batch * g.n_in * (wt == WT_F32 ? 4 : 2));
  char* w = (char*)ws;
  const hipStream_t s = as_stream(stream);
  const IsgLayout Lw = isg_layout(&g, batch);
  int32_t* ids = reinterpret_cast<int32_t*>(w + gated + Lw.ids);
  int32_t* cnt = reinterpret_cast<int32_t*>(w + gated + Lw.count);
  if (launch_head_gate(wt, attn, batch, op->n_heads, op->head_dim, head_mask, w, ids, cnt, s) != hipSuccess)
    return SFNN_E_HIP;
  return run_isg(&g, w, batch, y, ids, cnt, w + gated, Lw, s, true);
}

const char* sfnn_status_str(sfnn_status s) {
  switch (s) {
    case SFNN_OK: return "ok";
    case SFNN_E_NULL: return "required pointer is NULL";
    case SFNN_E_SHAPE: return "size outside the supported limits";
    case SFNN_E_ALIGN: return "pointer not 16-byte aligned";
    case SFNN_E_DTYPE: return "unknown or inconsistent data type";
    case SFNN_E_WORKSPACE: return "workspace too small";
    case SFNN_E_HIP: return "HIP launch error";
  }
  return "unknown status";
}

int32_t sfnn_version(void) { return 350; }  // 300: sfnn_ffn.mfma_min_batch; 310: sfnn_input_sparse_gemv; 320: sfnn_pred.hot_prefix; 330: head-gated projections; 340: sfnn_pred.dense_min_batch; 350: sfnn_dense_min_batch, per-layer stack switch, no default threshold

}  // extern "C"
