// C ABI of the routed-MoE layer: host-side validation, workspace layout and
// kernel dispatch.  No call allocates device memory or synchronises.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <atomic>

#include "../../include/moe.h"
#include "kernels.h"
#include "layer.h"

using namespace moe;

namespace {

constexpr int kMaxE = 1024;
constexpr int kMaxK = 32;
constexpr int kMaxH = 8192;
constexpr int kMaxI = 4096;
constexpr int kMaxSlots = 16384;
constexpr int kMaxVerifyT = 64;        // rows of one verify pass
constexpr int kMaxVocab = 1 << 26;
constexpr int64_t kMaxT = int64_t(1) << 22;
constexpr size_t kAlign = 256;
constexpr int kRouterGemmMinT = 256;       // tokens from which the router runs on MFMA
constexpr int64_t kFfnGemmMinPairs = 2048; // pairs from which the FFN runs as grouped GEMMs

// Budget of the fused launch's waits (ns; 0 = the default) and the test hold.
constexpr uint64_t kDefaultWaitNs = 100000000ull;
std::atomic<uint64_t> g_wait_ns{0};
std::atomic<int32_t> g_hold{0};
std::atomic<uint64_t*> g_trace{nullptr};   // phase stamps of the fused launch (diagnostics)
std::atomic<int32_t> g_det{0};             // fused launch: y summed in a fixed order

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool valid_pool(const moe_mat& m, int fmt) {
  if (m.fmt != fmt || !m.data) return false;
  if (fmt == MOE_W_F32) return aligned(m.data, 16);
  return m.scale && m.min && aligned(m.data, 16) && aligned(m.scale, 4) && aligned(m.min, 4);
}

bool has_shared(const moe_layer_desc* d) { return d->sh_gate.data != nullptr; }

// Checks the layer description.  Returns MOE_OK, MOE_ERR_INVALID or
// MOE_ERR_UNSUPPORTED.
moe_status check_desc(const moe_layer_desc* d) {
  if (!d) return MOE_ERR_INVALID;
  if (d->E < 1 || d->k < 1 || d->k > d->E || d->H < 32 || d->I < 32 || d->H % 32 || d->I % 32 ||
      d->num_slots < 1)
    return MOE_ERR_INVALID;
  if (d->E > kMaxE || d->k > kMaxK || d->H > kMaxH || d->I > kMaxI || d->num_slots > kMaxSlots)
    return MOE_ERR_UNSUPPORTED;
  if (!d->slot_of_expert && d->num_slots != d->E) return MOE_ERR_INVALID;
  if (d->router_fmt != MOE_W_F32 && d->router_fmt != MOE_W_BF16) return MOE_ERR_UNSUPPORTED;
  if (!d->router_w || !aligned(d->router_w, 16)) return MOE_ERR_INVALID;
  const int fmt = d->gate.fmt;
  if (fmt != MOE_W_F32 && fmt != MOE_W_Q2B32 && fmt != MOE_W_Q4B32) return MOE_ERR_UNSUPPORTED;
  if (fmt == MOE_W_Q2B32 && (d->H % 64 || d->I % 64)) return MOE_ERR_INVALID;
  if (!valid_pool(d->gate, fmt) || !valid_pool(d->up, fmt) || !valid_pool(d->down, fmt))
    return MOE_ERR_INVALID;
  if (has_shared(d) &&
      (!valid_pool(d->sh_gate, fmt) || !valid_pool(d->sh_up, fmt) || !valid_pool(d->sh_down, fmt)))
    return MOE_ERR_INVALID;
  return MOE_OK;
}

// Checks a slot pool for moe_slot_refresh.
moe_status check_pool(const moe_slot_pool* p) {
  if (!p) return MOE_ERR_INVALID;
  if (p->L < 1 || p->E < 1 || p->num_slots < 1 || p->H < 32 || p->I < 32 || p->H % 32 ||
      p->I % 32)
    return MOE_ERR_INVALID;
  if (int64_t(p->L) * p->E > 65536 || p->num_slots > kMaxSlots || p->H > kMaxH || p->I > kMaxI)
    return MOE_ERR_UNSUPPORTED;
  const int fmt = p->gate.fmt;
  if (fmt != MOE_W_F32 && fmt != MOE_W_Q2B32 && fmt != MOE_W_Q4B32) return MOE_ERR_UNSUPPORTED;
  if (fmt == MOE_W_Q2B32 && (p->H % 64 || p->I % 64)) return MOE_ERR_INVALID;
  const moe_mat* m[6] = {&p->gate, &p->up, &p->down, &p->store_gate, &p->store_up, &p->store_down};
  for (int i = 0; i < 6; ++i)
    if (!valid_pool(*m[i], fmt)) return MOE_ERR_INVALID;
  if (!p->usage || !p->slot_of || !p->expert_of) return MOE_ERR_INVALID;
  return MOE_OK;
}

// Workspace regions (each 256-byte aligned), in this order:
//   layer   hand-off region of the fused moe_layer (layer_region_bytes;
//           sized from the layer shape alone, so it sits at the same place
//           for every T)
//   logits  [T][E] fp32
//   active  slot[cap], start[cap+1], count[1]
//   slotbuf [T*k] int32 (moe_layer's slot_idx when the caller passes none)
//   pairbuf [T*k][H] fp32 + sharedbuf [T][H] fp32 (moe_layer only, T <= 16)
//   bucket  off[S+1] + pair[T*k] (moe_layer only)
//   h       [T*k + T][I] fp32 (GEMV path), or the grouped-GEMM tile list and
//           fp16 h (GEMM path): the larger of the two
//   resolve large-path counters
struct WsLayout {
  size_t layer, logits, active, slotbuf, pairbuf, sharedbuf, bucket, h, resolve, total;
  int cap;
};

WsLayout layout(const moe_layer_desc* d, int64_t T) {
  WsLayout w;
  const int64_t P = T * d->k;
  w.cap = int(P < d->num_slots ? P : d->num_slots);
  size_t o = 0;
  w.layer = o;
  o += up(layer_region_bytes(d->E, d->k, d->H, d->I));
  w.logits = o;
  o += up(size_t(T) * d->E * 4);
  w.active = o;
  o += up(size_t(2 * w.cap + 2) * 4);
  w.slotbuf = o;
  o += up(size_t(P) * 4);
  const bool layer_sized = T <= MOE_LAYER_MAX_T;
  w.pairbuf = o;
  o += layer_sized ? up(size_t(P) * d->H * 4) : 0;
  w.sharedbuf = o;
  o += layer_sized ? up(size_t(T) * d->H * 4) : 0;
  w.bucket = o;
  o += layer_sized ? up(size_t(d->num_slots + 1 + P) * 4) : 0;
  w.h = o;
  const size_t h_gemv = size_t(P + T) * d->I * 4;
  const size_t h_gemm = ffn_gemm_ws(int(T), d->k, d->H, d->I, d->num_slots);
  o += up(h_gemv > h_gemm ? h_gemv : h_gemm);
  w.resolve = o;
  o += up(resolve_large_ws(int(T), d->k, d->num_slots));
  w.total = o;
  return w;
}

template <typename Tp>
Tp* at(void* ws, size_t off) {
  return reinterpret_cast<Tp*>(static_cast<uint8_t*>(ws) + off);
}

ActiveList active_at(void* ws, const WsLayout& w) {
  ActiveList a;
  a.slot = at<int32_t>(ws, w.active);
  a.start = a.slot + w.cap;
  a.count = a.start + w.cap + 1;
  return a;
}

moe_status check_ws(const moe_layer_desc* d, int64_t T, void* ws, size_t ws_bytes) {
  const WsLayout w = layout(d, T);
  if (!ws || !aligned(ws, kAlign)) return MOE_ERR_INVALID;
  if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

moe_status device_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_DEVICE; }

// The grouped GEMM reads eight scales (or mins) at a time: every scale and
// min plane 16-byte aligned (the ABI only promises 4).
bool planes_16b_aligned(const moe_layer_desc* d) {
  const moe_mat* m[6] = {&d->gate, &d->up, &d->down, &d->sh_gate, &d->sh_up, &d->sh_down};
  for (int i = 0; i < 6; ++i) {
    if (i >= 3 && !has_shared(d)) break;
    if (!aligned(m[i]->scale, 16) || !aligned(m[i]->min, 16)) return false;
  }
  return true;
}

FfnArgs ffn_args(const moe_layer_desc* d, const uint16_t* x, int T) {
  FfnArgs a;
  memset(&a, 0, sizeof(a));
  a.x = x;
  a.T = T;
  a.k = d->k;
  a.H = d->H;
  a.I = d->I;
  a.fmt = d->gate.fmt;
  a.g = make_view(d->gate, d->I, d->H);
  a.u = make_view(d->up, d->I, d->H);
  a.d = make_view(d->down, d->H, d->I);
  if (has_shared(d)) {
    a.sg = make_view(d->sh_gate, d->I, d->H);
    a.su = make_view(d->sh_up, d->I, d->H);
    a.sd = make_view(d->sh_down, d->H, d->I);
  }
  return a;
}

moe_status run_route(const moe_layer_desc* d, const uint16_t* x, int T, int32_t* idx, float* gate,
                     void* ws, const WsLayout& w, hipStream_t st) {
  float* logits = at<float>(ws, w.logits);
  hipError_t e;
  if (T >= kRouterGemmMinT && d->router_fmt == MOE_W_BF16 && d->H % 64 == 0)
    e = launch_router_mfma(x, T, d->H, d->E, static_cast<const uint16_t*>(d->router_w),
                           d->router_bias, logits, st);
  else
    e = launch_router(x, T, d->H, d->E, d->router_fmt, d->router_w, d->router_bias, logits, st);
  if (e == hipSuccess) e = launch_topk(logits, T, d->E, d->k, idx, gate, st);
  return device_status(e);
}

moe_status run_resolve(const moe_layer_desc* d, const int32_t* idx, const float* gate, int T,
                       int32_t* slot_idx, int32_t* bucket_off, int32_t* bucket_pair,
                       moe_miss* miss, int32_t* miss_off, void* ws, const WsLayout& w,
                       hipStream_t st) {
  const ActiveList act = active_at(ws, w);
  hipError_t e;
  if (int64_t(T) * d->k <= kResolveSmallMax)
    e = launch_resolve_small(T, d->k, d->E, d->num_slots, idx, gate, d->slot_of_expert, slot_idx,
                             bucket_off, bucket_pair, miss, miss_off, act, st);
  else
    e = launch_resolve_large(T, d->k, d->E, d->num_slots, idx, gate, d->slot_of_expert, slot_idx,
                             bucket_off, bucket_pair, miss, miss_off, act,
                             at<void>(ws, w.resolve), st);
  if (e == hipSuccess && d->usage_counts)
    e = launch_count_usage(T * d->k, d->E, idx, d->usage_counts, st);
  return device_status(e);
}

// The expert FFN of one bucketed batch (the body of moe_expert_ffn; with
// y_acc set, of moe_expert_ffn_accum).
moe_status run_ffn(const moe_layer_desc* d, const uint16_t* x, int T, const int32_t* bucket_off,
                   const int32_t* bucket_pair, float* pair_out, float* shared_out, void* ws,
                   const WsLayout& w, hipStream_t st, float* y_acc = nullptr,
                   const float* gate = nullptr) {
  FfnArgs a = ffn_args(d, x, T);
  a.act = active_at(ws, w);
  a.active_cap = w.cap;
  a.bucket_pair = bucket_pair;
  a.h = at<float>(ws, w.h);
  a.h_sh = a.h + size_t(T) * d->k * d->I;
  a.pair_out = pair_out;
  a.shared_out = shared_out;
  a.y_acc = y_acc;
  a.gate = gate;
  hipError_t e = launch_active_from_offsets(d->num_slots, bucket_off, a.act, st);
  if (e == hipSuccess) {
    if (int64_t(T) * d->k >= kFfnGemmMinPairs && ffn_gemm_ok(a.fmt, d->H, d->I) &&
        ffn_gemm_fits(T, d->k, d->H, d->I) && planes_16b_aligned(d))
      e = launch_ffn_gemm(a, d->num_slots, bucket_off, at<void>(ws, w.h), st);
    else
      e = launch_ffn_gemv(a, st);
  }
  return device_status(e);
}

// Workspace of the chunked prefill: one or two halves, each a full
// workspace for `chunk` tokens followed by the chunk's buckets, pair outputs
// and shared-expert outputs.
struct PrefillHalf {
  WsLayout w;
  size_t boff, bpair, pair_out, shared_out, total;
};

PrefillHalf prefill_half(const moe_layer_desc* d, int chunk) {
  PrefillHalf h;
  h.w = layout(d, chunk);
  size_t o = h.w.total;
  h.boff = o;
  o += up(size_t(d->num_slots + 1) * 4);
  h.bpair = o;
  o += up(size_t(chunk) * d->k * 4);
  h.pair_out = o;
  o += up(size_t(chunk) * d->k * d->H * 4);
  h.shared_out = o;
  o += up(size_t(chunk) * d->H * 4);
  h.total = o;
  return h;
}

// Events of the prefill pipeline, made once per device and host thread.
struct PrefillEvents {
  hipEvent_t fork = nullptr, routed[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr};
  bool ok = false;
};

PrefillEvents* prefill_events() {
  static thread_local PrefillEvents ev[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  PrefillEvents& e = ev[dev];
  if (!e.ok) {
    if (hipEventCreateWithFlags(&e.fork, hipEventDisableTiming) != hipSuccess) return nullptr;
    for (int i = 0; i < 2; ++i) {
      if (hipEventCreateWithFlags(&e.routed[i], hipEventDisableTiming) != hipSuccess ||
          hipEventCreateWithFlags(&e.done[i], hipEventDisableTiming) != hipSuccess)
        return nullptr;
    }
    e.ok = true;
  }
  return &e;
}

// Whether moe_layer takes the fused launch for this layer and T.
bool fused_shape(const moe_layer_desc* d, int T) {
  const int fmt = d->gate.fmt;
  return layer_fused_ok(fmt, T, d->k, d->E, d->H, d->I) &&
         (fmt == MOE_W_F32 || d->router_fmt == MOE_W_BF16);
}

// Arguments of the fused launch (region: its hand-off region).
LayerArgs layer_args(const moe_layer_desc* desc, const uint16_t* x, int T, float* y,
                     int32_t* topk_idx, float* topk_gate, int32_t* slot_idx, moe_miss* miss,
                     int32_t* miss_off, uint8_t* region) {
  LayerArgs L;
  memset(&L, 0, sizeof(L));
  L.x = x;
  L.T = T;
  L.E = desc->E;
  L.k = desc->k;
  L.H = desc->H;
  L.I = desc->I;
  L.S = desc->num_slots;
  L.rfmt = desc->router_fmt;
  L.has_sh = has_shared(desc) ? 1 : 0;
  L.W = desc->router_w;
  L.bias = desc->router_bias;
  L.slot_of = desc->slot_of_expert;
  const FfnArgs f = ffn_args(desc, x, T);
  auto planes = [](const MatView& v) { return Planes{v.codes, v.scale, v.mn}; };
  L.g = planes(f.g);
  L.u = planes(f.u);
  L.d = planes(f.d);
  L.sg = planes(f.sg);
  L.su = planes(f.su);
  L.sd = planes(f.sd);
  L.mat_bytes = f.g.mat_bytes;     // the same for all six: I x H weights each
  L.mat_blocks = f.g.mat_blocks;
  L.y = y;
  L.idx = topk_idx;
  L.gate = topk_gate;
  L.slot_idx = slot_idx;
  L.miss = miss;
  L.miss_off = miss_off;
  L.usage = desc->usage_counts;
  L.region = region;
  const uint64_t ns = g_wait_ns.load(std::memory_order_relaxed);
  L.wait_ticks = (ns ? ns : kDefaultWaitNs) / 10;   // the real-time counter runs at 100 MHz
  if (L.wait_ticks == 0) L.wait_ticks = 1;
  L.debug_hold = g_hold.load(std::memory_order_relaxed);
  L.trace = g_trace.load(std::memory_order_relaxed);
  L.det = g_det.load(std::memory_order_relaxed) ? 1 : 0;
  return L;
}

}  // namespace

extern "C" {

const char* moe_status_string(int32_t s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or format";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_DEVICE: return "device launch failed";
    default: return "unknown status";
  }
}

int32_t moe_version(void) { return 101; }

moe_status moe_workspace_size(const moe_layer_desc* desc, int32_t T, size_t* bytes) {
  const moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (!bytes || T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  *bytes = layout(desc, T).total;
  return MOE_OK;
}

moe_status moe_route(const moe_layer_desc* desc, const uint16_t* x, int32_t T, int32_t* topk_idx,
                     float* topk_gate, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !topk_idx || !topk_gate) return MOE_ERR_INVALID;
  if ((s = check_ws(desc, T, ws, ws_bytes)) != MOE_OK) return s;
  return run_route(desc, x, T, topk_idx, topk_gate, ws, layout(desc, T),
                   static_cast<hipStream_t>(stream));
}

moe_status moe_resolve_slots(const moe_layer_desc* desc, const int32_t* topk_idx,
                             const float* topk_gate, int32_t T, int32_t* slot_idx,
                             int32_t* bucket_off, int32_t* bucket_pair, moe_miss* miss,
                             int32_t* miss_off, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!topk_idx || !topk_gate || !slot_idx || !bucket_off || !bucket_pair || !miss || !miss_off)
    return MOE_ERR_INVALID;
  if ((s = check_ws(desc, T, ws, ws_bytes)) != MOE_OK) return s;
  return run_resolve(desc, topk_idx, topk_gate, T, slot_idx, bucket_off, bucket_pair, miss,
                     miss_off, ws, layout(desc, T), static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                          const int32_t* bucket_off, const int32_t* bucket_pair, float* pair_out,
                          float* shared_out, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !bucket_off || !bucket_pair || !pair_out ||
      (has_shared(desc) && !shared_out))
    return MOE_ERR_INVALID;
  if (!aligned(pair_out, 16) || (shared_out && !aligned(shared_out, 16))) return MOE_ERR_INVALID;
  if ((s = check_ws(desc, T, ws, ws_bytes)) != MOE_OK) return s;
  return run_ffn(desc, x, T, bucket_off, bucket_pair, pair_out, shared_out, ws, layout(desc, T),
                 static_cast<hipStream_t>(stream));
}

moe_status moe_expert_ffn_accum(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                                const int32_t* bucket_off, const int32_t* bucket_pair,
                                const float* topk_gate, float* y, void* ws, size_t ws_bytes,
                                void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !bucket_off || !bucket_pair || !topk_gate || !y || !aligned(y, 16))
    return MOE_ERR_INVALID;
  if ((s = check_ws(desc, T, ws, ws_bytes)) != MOE_OK) return s;
  return run_ffn(desc, x, T, bucket_off, bucket_pair, nullptr, nullptr, ws, layout(desc, T),
                 static_cast<hipStream_t>(stream), y, topk_gate);
}

moe_status moe_combine(const moe_layer_desc* desc, int32_t T, const int32_t* slot_idx,
                       const float* topk_gate, const float* pair_out, const float* shared_out,
                       float* y, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!slot_idx || !topk_gate || !pair_out || !y || !aligned(pair_out, 16) || !aligned(y, 16) ||
      (shared_out && !aligned(shared_out, 16)))
    return MOE_ERR_INVALID;
  return device_status(launch_combine(T, desc->k, desc->H, slot_idx, topk_gate, pair_out,
                                      shared_out, y, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer(const moe_layer_desc* desc, const uint16_t* x, int32_t T, float* y,
                     int32_t* topk_idx, float* topk_gate, int32_t* slot_idx, moe_miss* miss,
                     int32_t* miss_off, void* ws, size_t ws_bytes, void* stream) {
  moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > MOE_LAYER_MAX_T) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16) || !topk_idx || !topk_gate || !miss ||
      !miss_off)
    return MOE_ERR_INVALID;
  if ((s = check_ws(desc, T, ws, ws_bytes)) != MOE_OK) return s;
  const WsLayout w = layout(desc, T);
  hipStream_t st = static_cast<hipStream_t>(stream);
  int32_t* boff = at<int32_t>(ws, w.bucket);
  int32_t* bpair = boff + desc->num_slots + 1;
  float* pairbuf = at<float>(ws, w.pairbuf);
  float* shbuf = has_shared(desc) ? at<float>(ws, w.sharedbuf) : nullptr;
  const int fmt = desc->gate.fmt;
  if (fused_shape(desc, T)) {
    const LayerArgs L = layer_args(desc, x, T, y, topk_idx, topk_gate, slot_idx, miss, miss_off,
                                   at<uint8_t>(ws, w.layer));
    return device_status(launch_layer_fused(L, fmt, st, nullptr));
  }
  int32_t* sl = slot_idx ? slot_idx : at<int32_t>(ws, w.slotbuf);
  s = run_route(desc, x, T, topk_idx, topk_gate, ws, w, st);
  if (s == MOE_OK)
    s = run_resolve(desc, topk_idx, topk_gate, T, sl, boff, bpair, miss, miss_off, ws, w, st);
  if (s != MOE_OK) return s;
  FfnArgs a = ffn_args(desc, x, T);
  a.act = active_at(ws, w);
  a.active_cap = w.cap;
  a.bucket_pair = bpair;
  a.h = at<float>(ws, w.h);
  a.h_sh = a.h + size_t(T) * desc->k * desc->I;
  a.pair_out = pairbuf;
  a.shared_out = shbuf;
  hipError_t e = launch_ffn_gemv(a, st);
  if (e == hipSuccess)
    e = launch_combine(T, desc->k, desc->H, sl, topk_gate, pairbuf, shbuf, y, st);
  return device_status(e);
}

moe_status moe_layer_noalloc(const moe_layer_desc* desc, const uint16_t* x, int32_t T, float* y,
                             int32_t* topk_idx, float* topk_gate, int32_t* slot_idx,
                             moe_miss* miss, int32_t* miss_off, void* stream) {
  const moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (T < 0) return MOE_ERR_INVALID;
  if (T > MOE_LAYER_MAX_T) return MOE_ERR_UNSUPPORTED;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16) || !topk_idx || !topk_gate || !miss ||
      !miss_off)
    return MOE_ERR_INVALID;
  if (!fused_shape(desc, T) ||
      layer_region_bytes(desc->E, desc->k, desc->H, desc->I) > size_t(MOE_LAYER_SCRATCH_BYTES))
    return MOE_ERR_UNSUPPORTED;
  const LayerArgs L =
      layer_args(desc, x, T, y, topk_idx, topk_gate, slot_idx, miss, miss_off, nullptr);
  return device_status(launch_layer_noalloc(L, desc->gate.fmt, static_cast<hipStream_t>(stream)));
}

moe_status moe_layer_check(const void* ws, size_t ws_bytes, void* stream) {
  hipStream_t st = static_cast<hipStream_t>(stream);
  const uint8_t* region = static_cast<const uint8_t*>(ws);   // the hand-off region: offset 0
  if (!ws) {
    uint8_t* p = nullptr;
    if (layer_scratch_address(&p) != hipSuccess) return MOE_ERR_DEVICE;
    if (!p) return MOE_OK;   // no moe_layer_noalloc call on this GPU yet
    region = p;
  } else if (!aligned(ws, kAlign) || ws_bytes < 256) {
    return MOE_ERR_INVALID;
  }
  if (hipStreamSynchronize(st) != hipSuccess) return MOE_ERR_DEVICE;
  uint32_t err = 0;   // the error word of the region's header
  if (hipMemcpy(&err, region + kRegionErr, 4, hipMemcpyDeviceToHost) != hipSuccess)
    return MOE_ERR_DEVICE;
  if (err && !ws && (layer_scratch_clear(st) != hipSuccess || hipStreamSynchronize(st) != hipSuccess))
    return MOE_ERR_DEVICE;
  return err ? MOE_ERR_DEVICE : MOE_OK;
}

void moe_set_wait_budget(uint64_t ns, int32_t hold) {
  g_wait_ns.store(ns, std::memory_order_relaxed);
  g_hold.store(hold, std::memory_order_relaxed);
}

void moe_set_trace(uint64_t* trace) { g_trace.store(trace, std::memory_order_relaxed); }

void moe_set_deterministic(int32_t on) { g_det.store(on ? 1 : 0, std::memory_order_relaxed); }

moe_status moe_slot_refresh_workspace_size(const moe_slot_pool* pool, size_t* bytes) {
  const moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  if (!bytes) return MOE_ERR_INVALID;
  *bytes = 0;   // the refresh keeps its working set in LDS
  return MOE_OK;
}

moe_status moe_slot_refresh(const moe_slot_pool* pool, int32_t max_swaps, int32_t* swaps,
                            int32_t* n_swaps, void* ws, size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  const moe_status s = check_pool(pool);
  if (s != MOE_OK) return s;
  if (max_swaps < 0 || !n_swaps || (max_swaps > 0 && !swaps)) return MOE_ERR_INVALID;
  if (max_swaps > MOE_REFRESH_MAX_SWAPS) return MOE_ERR_UNSUPPORTED;
  RefreshArgs a;
  memset(&a, 0, sizeof(a));
  a.N = pool->L * pool->E;
  a.S = pool->num_slots;
  a.max_swaps = max_swaps;
  a.usage = pool->usage;
  a.slot_of = pool->slot_of;
  a.expert_of = pool->expert_of;
  a.swaps = swaps;
  a.n_swaps = n_swaps;
  const moe_mat* pm[3] = {&pool->gate, &pool->up, &pool->down};
  const moe_mat* sm[3] = {&pool->store_gate, &pool->store_up, &pool->store_down};
  for (int m = 0; m < 3; ++m) {
    // gate/up [I][H] and down [H][I]: the same size
    const MatView v = make_view(*pm[m], pool->I, pool->H);
    RefreshMat& r = a.mats[m];
    const bool f32 = pm[m]->fmt == MOE_W_F32;
    r.pool_codes = static_cast<uint8_t*>(const_cast<void*>(pm[m]->data));
    r.pool_scale = f32 ? nullptr : const_cast<uint16_t*>(pm[m]->scale);
    r.pool_min = f32 ? nullptr : const_cast<uint16_t*>(pm[m]->min);
    r.store_codes = static_cast<const uint8_t*>(sm[m]->data);
    r.store_scale = f32 ? nullptr : sm[m]->scale;
    r.store_min = f32 ? nullptr : sm[m]->min;
    r.mat_bytes = v.mat_bytes;
    r.mat_blocks = f32 ? 0 : v.mat_blocks;
  }
  return device_status(launch_slot_refresh(a, static_cast<hipStream_t>(stream)));
}

moe_status moe_prefill_workspace_size(const moe_layer_desc* desc, int32_t T, int32_t chunk,
                                      size_t* bytes) {
  const moe_status s = check_desc(desc);
  if (s != MOE_OK) return s;
  if (!bytes || T < 0 || chunk < 1) return MOE_ERR_INVALID;
  if (T > kMaxT) return MOE_ERR_UNSUPPORTED;
  const int c = T < chunk ? (T > 0 ? T : 1) : chunk;
  *bytes = prefill_half(desc, c).total * (T > c ? 2 : 1);
  return MOE_OK;
}

moe_status moe_prefill_layer(const moe_layer_desc* desc, const uint16_t* x, int32_t T,
                             int32_t chunk, float* y, int32_t* topk_idx, float* topk_gate,
                             int32_t* slot_idx, void* ws, size_t ws_bytes, void* stream,
                             void* aux_stream) {
  size_t need = 0;
  moe_status s = moe_prefill_workspace_size(desc, T, chunk, &need);
  if (s != MOE_OK) return s;
  if (T == 0) return MOE_OK;
  if (!x || !aligned(x, 16) || !y || !aligned(y, 16) || !topk_idx || !topk_gate || !slot_idx)
    return MOE_ERR_INVALID;
  if (!ws || !aligned(ws, kAlign)) return MOE_ERR_INVALID;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  const int C = T < chunk ? T : chunk;
  const int n_chunks = (T + C - 1) / C;
  const PrefillHalf ph = prefill_half(desc, C);
  hipStream_t main = static_cast<hipStream_t>(stream);
  hipStream_t aux = aux_stream ? static_cast<hipStream_t>(aux_stream) : main;
  PrefillEvents* ev = n_chunks > 1 || aux != main ? prefill_events() : nullptr;
  if ((n_chunks > 1 || aux != main) && !ev) return MOE_ERR_DEVICE;
  // the aux stream starts after the work already queued on the main stream
  if (aux != main && (hipEventRecord(ev->fork, main) != hipSuccess ||
                      hipStreamWaitEvent(aux, ev->fork, 0) != hipSuccess))
    return MOE_ERR_DEVICE;
  const int k = desc->k, H = desc->H;
  for (int c = 0; c < n_chunks; ++c) {
    const int t0 = c * C, Tc = T - t0 < C ? T - t0 : C, h = c & 1;
    void* half = static_cast<char*>(ws) + size_t(h) * ph.total;
    int32_t* boff = at<int32_t>(half, ph.boff);
    int32_t* bpair = at<int32_t>(half, ph.bpair);
    float* pair_out = at<float>(half, ph.pair_out);
    float* sh_out = has_shared(desc) ? at<float>(half, ph.shared_out) : nullptr;
    const uint16_t* xc = x + size_t(t0) * H;
    int32_t* idx = topk_idx + size_t(t0) * k;
    float* gate = topk_gate + size_t(t0) * k;
    int32_t* sl = slot_idx + size_t(t0) * k;
    // routing of chunk c (after chunk c - 2, the last user of this half, is done)
    if (c >= 2 && hipStreamWaitEvent(aux, ev->done[h], 0) != hipSuccess) return MOE_ERR_DEVICE;
    if ((s = run_route(desc, xc, Tc, idx, gate, half, ph.w, aux)) != MOE_OK) return s;
    if ((s = run_resolve(desc, idx, gate, Tc, sl, boff, bpair, nullptr, nullptr, half, ph.w,
                         aux)) != MOE_OK)
      return s;
    if (ev && (hipEventRecord(ev->routed[h], aux) != hipSuccess ||
               hipStreamWaitEvent(main, ev->routed[h], 0) != hipSuccess))
      return MOE_ERR_DEVICE;
    // experts and combine of chunk c, while chunk c + 1 is routed
    if ((s = run_ffn(desc, xc, Tc, boff, bpair, pair_out, sh_out, half, ph.w, main)) != MOE_OK)
      return s;
    if ((s = device_status(launch_combine(Tc, k, H, sl, gate, pair_out, sh_out,
                                          y + size_t(t0) * H, main))) != MOE_OK)
      return s;
    if (ev && hipEventRecord(ev->done[h], main) != hipSuccess) return MOE_ERR_DEVICE;
  }
  return MOE_OK;
}

moe_status moe_verify_workspace_size(int32_t T, int32_t V, size_t* bytes) {
  if (!bytes || T < 1 || V < 1) return MOE_ERR_INVALID;
  if (T > kMaxVerifyT || V > kMaxVocab) return MOE_ERR_UNSUPPORTED;
  *bytes = up(size_t(T) * verify_parts(T, V) * 8);
  return MOE_OK;
}

moe_status moe_verify_accept(const float* logits, int32_t T, int32_t V, const int32_t* draft,
                             int32_t* out_tokens, int32_t* n_out, void* ws, size_t ws_bytes,
                             void* stream) {
  size_t need = 0;
  const moe_status s = moe_verify_workspace_size(T, V, &need);
  if (s != MOE_OK) return s;
  if (!logits || !out_tokens || !n_out || (T > 1 && !draft)) return MOE_ERR_INVALID;
  if (!ws || !aligned(ws, kAlign)) return MOE_ERR_INVALID;
  if (ws_bytes < need) return MOE_ERR_WORKSPACE;
  return device_status(launch_verify_accept(logits, T, V, T > 1 ? draft : out_tokens, out_tokens,
                                            n_out, ws, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
