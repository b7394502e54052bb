// Reference oracle for the routed mixture-of-experts layer -- TEST
// INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
// leg of the benchmark may call it; the product path never does.
//
// Plain, slow, single-threaded C++ in fp64.  It shares no code, header or
// table with the HIP path.  Every input is widened exactly (bf16, fp16 and
// fp32 to double) and every step is the plain definition, written in the
// order the pages describe one decode step:
//
//   [MD] ModelDock, "Strata はなぜ少ない VRAM でも速いのか" (why Strata is fast
//        with little VRAM):
//        - section "問題" (the problem): 48 layers x 512 experts, the router of
//          every layer picks 10 experts per token; a shared expert belongs to
//          the weights every token uses;
//        - section "1 トークン、三者の分担" (one token, three workers): the GPU
//          runs the router, the 10 chosen expert ids are dispatched -- experts
//          already in VRAM to the GPU, the rest elsewhere -- and the GPU sums
//          the expert results before the next layer;
//        - section "粗から細へ" (coarse to fine) and its placement figure: a
//          per-card slot table of individual resident experts.
//
// Where the pages are silent the plain readings are used: SwiGLU with silu
// on the gate projection;
// gate weights = softmax over the k selected logits (router bias included);
// shared expert added with weight 1; top-k order = descending logit, lower
// expert id first on ties; quantised blocks of 32 weights along a row with
// one fp16 scale d and one fp16 min m, weight = d*q + m.
//
// Parity pins: every function here is checked by tests/test_oracle_pins.py
// against closed forms, hand-packed blocks, brute force and invariants.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <cmath>
#include <numeric>
#include <vector>

namespace {

enum { FMT_F32 = 0, FMT_BF16 = 1, FMT_Q2 = 2, FMT_Q4 = 3 };

double bf16_value(uint16_t b) {
  uint32_t u = uint32_t(b) << 16;
  float f;
  memcpy(&f, &u, 4);
  return double(f);
}

// IEEE half -> double, written out from the format: sign, 5-bit exponent
// (bias 15), 10-bit fraction; exponent 0 is subnormal (no implicit one).
double f16_value(uint16_t b) {
  const int sign = (b >> 15) & 1;
  const int expo = (b >> 10) & 31;
  const int frac = b & 1023;
  double v;
  if (expo == 0)
    v = std::ldexp(double(frac), -24);
  else if (expo == 31)
    v = frac ? NAN : INFINITY;
  else
    v = std::ldexp(double(1024 + frac), expo - 25);
  return sign ? -v : v;
}

// One weight of a [rows][cols] matrix, row-major with K = cols contiguous.
// Quantised: 32 consecutive weights of a row form a block with scale d and
// min m; the code of column c is bits*(c mod (8/bits)) up in byte
// (r*cols + c)*bits/8.
double weight(int fmt, const void* data, const uint16_t* scale, const uint16_t* mn,
              int cols, int64_t r, int64_t c) {
  const int64_t i = r * cols + c;
  if (fmt == FMT_F32) return double(static_cast<const float*>(data)[i]);
  if (fmt == FMT_BF16) return bf16_value(static_cast<const uint16_t*>(data)[i]);
  const uint8_t* bytes = static_cast<const uint8_t*>(data);
  int q;
  if (fmt == FMT_Q2)
    q = (bytes[i / 4] >> (2 * (c % 4))) & 3;
  else
    q = (bytes[i / 2] >> (4 * (c % 2))) & 15;
  const int64_t blk = r * (cols / 32) + c / 32;
  return f16_value(scale[blk]) * double(q) + f16_value(mn[blk]);
}

double silu(double a) { return a / (1.0 + std::exp(-a)); }

bool valid_fmt(int f) { return f == FMT_F32 || f == FMT_BF16 || f == FMT_Q2 || f == FMT_Q4; }

}  // namespace

extern "C" {

double oracle_bf16(uint16_t b) { return bf16_value(b); }
double oracle_f16(uint16_t b) { return f16_value(b); }

// Dequantise a whole [rows][cols] matrix to fp64 (row-major).
int oracle_dequant(int fmt, int rows, int cols, const void* data, const uint16_t* scale,
                   const uint16_t* mn, double* out) {
  if (!valid_fmt(fmt) || rows < 0 || cols < 0 || (fmt >= FMT_Q2 && cols % 32)) return 1;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t c = 0; c < cols; ++c) out[r * cols + c] = weight(fmt, data, scale, mn, cols, r, c);
  return 0;
}

// Router ([MD] "問題", "1 トークン、三者の分担"): logit[t][e] =
// sum_h x[t][h] * W[e][h] + bias[e].  x bf16 [T][H]; W f32 or bf16 [E][H];
// bias fp32 [E] or NULL.
int oracle_router(int T, int E, int H, const uint16_t* x, int wfmt, const void* W,
                  const float* bias, double* logits) {
  if (T < 0 || E <= 0 || H <= 0 || (wfmt != FMT_F32 && wfmt != FMT_BF16)) return 1;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double s = 0.0;
      for (int h = 0; h < H; ++h)
        s += bf16_value(x[int64_t(t) * H + h]) * weight(wfmt, W, nullptr, nullptr, H, e, h);
      if (bias) s += double(bias[e]);
      logits[int64_t(t) * E + e] = s;
    }
  return 0;
}

// Top-k and gates ([MD] "問題": the router picks 10 of 512 per token).
// Order: descending logit, lower expert id first on equal logits (a stable
// sort of ids 0..E-1 by descending logit).  Gates: softmax over the k
// selected logits.
int oracle_topk(int T, int E, int k, const double* logits, int32_t* idx, double* gate) {
  if (T < 0 || k < 1 || k > E) return 1;
  std::vector<int> ids(E);
  for (int t = 0; t < T; ++t) {
    const double* l = logits + int64_t(t) * E;
    std::iota(ids.begin(), ids.end(), 0);
    std::stable_sort(ids.begin(), ids.end(), [l](int a, int b) { return l[a] > l[b]; });
    const double lmax = l[ids[0]];
    double z = 0.0;
    for (int j = 0; j < k; ++j) z += std::exp(l[ids[j]] - lmax);
    for (int j = 0; j < k; ++j) {
      idx[int64_t(t) * k + j] = ids[j];
      gate[int64_t(t) * k + j] = std::exp(l[ids[j]] - lmax) / z;
    }
  }
  return 0;
}

// Slot resolution ([MD] "1 トークン、三者の分担" and the placement figure of
// "粗から細へ"): slot = slot_of[expert] (identity when slot_of is NULL); a
// pair is a hit when its slot is >= 0.  Misses are listed as (expert, token,
// gate) in (token, j) order, miss_off[t] .. miss_off[t+1] holding token t's.
int oracle_resolve(int T, int k, int E, const int32_t* idx, const double* gate,
                   const int32_t* slot_of, int32_t* slot_idx, int32_t* miss_expert,
                   int32_t* miss_token, double* miss_gate, int32_t* miss_off) {
  if (T < 0 || k < 1 || k > E) return 1;
  int n = 0;
  for (int t = 0; t < T; ++t) {
    miss_off[t] = n;
    for (int j = 0; j < k; ++j) {
      const int64_t p = int64_t(t) * k + j;
      const int e = idx[p];
      const int s = slot_of ? slot_of[e] : e;
      slot_idx[p] = s;
      if (s < 0) {
        miss_expert[n] = e;
        miss_token[n] = t;
        miss_gate[n] = gate[p];
        ++n;
      }
    }
  }
  miss_off[T] = n;
  return 0;
}

// Usage counts (the adaptive tier of [MD] "粗から細へ" follows the experts
// the conversation actually uses): every choice of expert e adds one to
// usage[e], hits and misses alike.
int oracle_count_usage(int T, int k, int E, const int32_t* idx, uint32_t* usage) {
  if (T < 0 || k < 1 || E < 1) return 1;
  for (int64_t p = 0; p < int64_t(T) * k; ++p) {
    const int e = idx[p];
    if (e < 0 || e >= E) return 1;
    usage[e] += 1u;
  }
  return 0;
}

// One refresh of a global slot table ([MD] "粗から細へ": slots are filled
// by a usage ranking; the adaptive tier swaps a bounded number of experts
// toward the ones in use).  Written from the definition, step by step:
//   u(j) = min(usage[j], 65535);
//   candidates: experts j with slot_of[j] < 0 and u(j) > 0, ranked by u
//     descending, then j ascending;
//   victims: free slots (expert_of[s] < 0) by s ascending, then occupied
//     slots by u(expert_of[s]) ascending, then s ascending;
//   swap i takes candidate i into victim i's slot while i < max_swaps, both
//     lists last and the victim is free or u(candidate) > u(victim's expert);
//   tables: slot_of[old] = -1, slot_of[new] = s, expert_of[s] = new;
//   every count is then halved.
// swaps[3*i .. 3*i+2] = (s, new, old or -1); *n_swaps = the number of swaps.
int oracle_slot_refresh(int N, int S, uint32_t* usage, int32_t* slot_of, int32_t* expert_of,
                        int max_swaps, int32_t* swaps, int32_t* n_swaps) {
  if (N < 1 || S < 1 || max_swaps < 0) return 1;
  auto u = [&](int j) -> int64_t { return usage[j] < 65535u ? int64_t(usage[j]) : 65535; };
  std::vector<int> cand;
  for (int j = 0; j < N; ++j)
    if (slot_of[j] < 0 && u(j) > 0) cand.push_back(j);
  std::sort(cand.begin(), cand.end(), [&](int a, int b) {
    if (u(a) != u(b)) return u(a) > u(b);
    return a < b;
  });
  std::vector<int> vict;
  for (int s = 0; s < S; ++s)
    if (expert_of[s] < 0) vict.push_back(s);
  std::vector<int> occ;
  for (int s = 0; s < S; ++s)
    if (expert_of[s] >= 0) occ.push_back(s);
  std::sort(occ.begin(), occ.end(), [&](int a, int b) {
    const int64_t ua = u(expert_of[a]), ub = u(expert_of[b]);
    if (ua != ub) return ua < ub;
    return a < b;
  });
  vict.insert(vict.end(), occ.begin(), occ.end());
  int n = 0;
  while (n < max_swaps && n < int(cand.size()) && n < int(vict.size())) {
    const int s = vict[n], j = cand[n], old = expert_of[s];
    if (old >= 0 && !(u(j) > u(old))) break;
    swaps[3 * n] = s;
    swaps[3 * n + 1] = j;
    swaps[3 * n + 2] = old;
    ++n;
  }
  for (int i = 0; i < n; ++i) {
    const int s = swaps[3 * i], j = swaps[3 * i + 1], old = swaps[3 * i + 2];
    if (old >= 0) slot_of[old] = -1;
    slot_of[j] = s;
    expert_of[s] = j;
  }
  for (int j = 0; j < N; ++j) usage[j] >>= 1;
  *n_swaps = n;
  return 0;
}

// Bucket the hit pairs by slot, stably: a counting sort over slots 0..S-1
// in pair order p = t*k + j.  bucket_off[S+1]; bucket_pair[bucket_off[S]].
// Each distinct resident expert then appears once with all of its tokens
// ([MD] "予測してから検証する": verifying several tokens costs only the
// extra experts they route to).
int oracle_bucket(int T, int k, int S, const int32_t* slot_idx, int32_t* bucket_off,
                  int32_t* bucket_pair) {
  if (T < 0 || k < 1 || S < 0) return 1;
  const int64_t P = int64_t(T) * k;
  std::vector<int64_t> count(S, 0);
  for (int64_t p = 0; p < P; ++p) {
    const int s = slot_idx[p];
    if (s >= S) return 1;
    if (s >= 0) count[s]++;
  }
  int64_t run = 0;
  for (int s = 0; s < S; ++s) {
    bucket_off[s] = int32_t(run);
    run += count[s];
  }
  bucket_off[S] = int32_t(run);
  std::vector<int64_t> fill(S, 0);
  for (int64_t p = 0; p < P; ++p) {
    const int s = slot_idx[p];
    if (s >= 0) bucket_pair[bucket_off[s] + fill[s]++] = int32_t(p);
  }
  return 0;
}

// Expert FFN (SwiGLU) for n tokens of one expert:
//   a = G x, u = U x, h_i = silu(a_i) * u_i, o = D h
// G, U are [I][H], D is [H][I]; each given as (data, scale, min) in format
// fmt.  x bf16 [n][H]; o fp64 [n][H].  Each weight row is dequantised once
// and applied to every token; the sums run over the input index in order.
int oracle_ffn(int fmt, int H, int I, const void* g, const uint16_t* gs, const uint16_t* gm,
               const void* u, const uint16_t* us, const uint16_t* um, const void* d,
               const uint16_t* ds, const uint16_t* dm, int n, const uint16_t* x, double* o) {
  if (!valid_fmt(fmt) || H <= 0 || I <= 0 || n < 0) return 1;
  if (fmt >= FMT_Q2 && (H % 32 || I % 32)) return 1;
  std::vector<double> xv(int64_t(n) * H), hv(int64_t(n) * I), row(std::max(H, I));
  for (int64_t i = 0; i < int64_t(n) * H; ++i) xv[i] = bf16_value(x[i]);
  std::vector<double> a(n);
  for (int i = 0; i < I; ++i) {
    for (int h = 0; h < H; ++h) row[h] = weight(fmt, g, gs, gm, H, i, h);
    for (int t = 0; t < n; ++t) {
      double s = 0.0;
      for (int h = 0; h < H; ++h) s += row[h] * xv[int64_t(t) * H + h];
      a[t] = s;
    }
    for (int h = 0; h < H; ++h) row[h] = weight(fmt, u, us, um, H, i, h);
    for (int t = 0; t < n; ++t) {
      double s = 0.0;
      for (int h = 0; h < H; ++h) s += row[h] * xv[int64_t(t) * H + h];
      hv[int64_t(t) * I + i] = silu(a[t]) * s;
    }
  }
  for (int r = 0; r < H; ++r) {
    for (int i = 0; i < I; ++i) row[i] = weight(fmt, d, ds, dm, I, r, i);
    for (int t = 0; t < n; ++t) {
      double s = 0.0;
      for (int i = 0; i < I; ++i) s += row[i] * hv[int64_t(t) * I + i];
      o[int64_t(t) * H + r] = s;
    }
  }
  return 0;
}

// Combine ([MD] "1 トークン、三者の分担": the GPU sums the expert results):
//   y[t] = shared[t] + sum_{j = 0..k-1, slot_idx[t][j] >= 0} gate[t][j] * o[t*k+j]
// shared may be NULL (no shared expert).  pair_out is [T*k][H].
int oracle_combine(int T, int k, int H, const int32_t* slot_idx, const double* gate,
                   const double* pair_out, const double* shared, double* y) {
  if (T < 0 || k < 1 || H <= 0) return 1;
  for (int t = 0; t < T; ++t)
    for (int r = 0; r < H; ++r) {
      double s = shared ? shared[int64_t(t) * H + r] : 0.0;
      for (int j = 0; j < k; ++j) {
        const int64_t p = int64_t(t) * k + j;
        if (slot_idx[p] >= 0) s += gate[p] * pair_out[p * H + r];
      }
      y[int64_t(t) * H + r] = s;
    }
  return 0;
}

// Whole layer with every pool in host memory: router -> top-k -> gates ->
// resolve -> bucket -> FFN of every hit pair -> shared expert -> combine.
// Pools are stacked by slot: gate/up [S][I][H], down [S][H][I] in format fmt
// (codes, scale, min planes; scale/min NULL for f32).  sh_* may be NULL (no
// shared expert).  Outputs: y [T][H]; idx, gate, slot_idx [T][k]; miss_*
// [T*k]; miss_off [T+1]; bucket_off [S+1]; bucket_pair [T*k].
int oracle_layer(int T, int E, int k, int H, int I, int S, const uint16_t* x, int router_fmt,
                 const void* router_w, const float* router_bias, const int32_t* slot_of,
                 int fmt, const void* g, const uint16_t* gs, const uint16_t* gm,
                 const void* u, const uint16_t* us, const uint16_t* um, const void* d,
                 const uint16_t* ds, const uint16_t* dm, const void* shg,
                 const uint16_t* shgs, const uint16_t* shgm, const void* shu,
                 const uint16_t* shus, const uint16_t* shum, const void* shd,
                 const uint16_t* shds, const uint16_t* shdm, double* y, int32_t* idx,
                 double* gate, int32_t* slot_idx, int32_t* miss_expert, int32_t* miss_token,
                 double* miss_gate, int32_t* miss_off, int32_t* bucket_off,
                 int32_t* bucket_pair) {
  if (T < 0 || k < 1 || k > E || S < 0 || !valid_fmt(fmt)) return 1;
  const int64_t P = int64_t(T) * k;
  std::vector<double> logits(int64_t(T) * E);
  int rc = oracle_router(T, E, H, x, router_fmt, router_w, router_bias, logits.data());
  if (!rc) rc = oracle_topk(T, E, k, logits.data(), idx, gate);
  if (!rc)
    rc = oracle_resolve(T, k, E, idx, gate, slot_of, slot_idx, miss_expert, miss_token,
                        miss_gate, miss_off);
  if (!rc) rc = oracle_bucket(T, k, S, slot_idx, bucket_off, bucket_pair);
  if (rc) return rc;
  // per-slot plane sizes
  const int bits = fmt == FMT_Q2 ? 2 : fmt == FMT_Q4 ? 4 : fmt == FMT_BF16 ? 16 : 32;
  const int64_t m_bytes = int64_t(I) * H * bits / 8;      // gate/up/down: same count
  const int64_t m_blocks = int64_t(I) * H / 32;
  auto off = [&](const void* base, int64_t s) {
    return static_cast<const void*>(static_cast<const uint8_t*>(base) + s * m_bytes);
  };
  auto boff = [&](const uint16_t* base, int64_t s) -> const uint16_t* {
    return base ? base + s * m_blocks : nullptr;
  };
  std::vector<double> pair_out(P * H, 0.0), o(H);
  for (int64_t p = 0; p < P; ++p) {
    const int s = slot_idx[p];
    if (s < 0) continue;
    const int t = int(p / k);
    rc = oracle_ffn(fmt, H, I, off(g, s), boff(gs, s), boff(gm, s), off(u, s), boff(us, s),
                    boff(um, s), off(d, s), boff(ds, s), boff(dm, s), 1,
                    x + int64_t(t) * H, o.data());
    if (rc) return rc;
    std::copy(o.begin(), o.end(), pair_out.begin() + p * H);
  }
  std::vector<double> shared;
  if (shg) {
    shared.resize(int64_t(T) * H);
    rc = oracle_ffn(fmt, H, I, shg, shgs, shgm, shu, shus, shum, shd, shds, shdm, T, x,
                    shared.data());
    if (rc) return rc;
  }
  return oracle_combine(T, k, H, slot_idx, gate, pair_out.data(),
                        shg ? shared.data() : nullptr, y);
}

// Acceptance of a verify pass ([MD] "予測してから検証する": a draft layer
// proposes up to 3 next tokens, one pass of the model checks them all, keeps
// the ones the model agrees with and adds one token of its own, so the
// output equals plain greedy decoding).  Row i of logits [T][V] is the
// model's prediction after input i of the verify batch (input 0 = the last
// accepted token, input i = draft token i); draft [T-1].  The model's greedy
// token after input i is g_i = the index of the largest logit of row i, the
// lowest index on equal values.  Draft i+1 is kept while it equals g_i; with
// a drafts kept, the output is g_0 .. g_a (the kept drafts, then the model's
// own token), n_out = a + 1.
int oracle_verify_accept(int T, int V, const double* logits, const int32_t* draft, int32_t* out,
                         int32_t* n_out) {
  if (T < 1 || V < 1) return 1;
  std::vector<int32_t> g(T);
  for (int i = 0; i < T; ++i) {
    const double* l = logits + int64_t(i) * V;
    int best = 0;
    for (int v = 1; v < V; ++v)
      if (l[v] > l[best]) best = v;
    g[i] = best;
  }
  int a = 0;
  while (a < T - 1 && draft[a] == g[a]) ++a;
  for (int i = 0; i <= a; ++i) out[i] = g[i];
  *n_out = a + 1;
  return 0;
}

}  // extern "C"
