// Host tier of the routed-expert layer: the experts the GPU does not hold,
// computed on the CPU from host-memory weights, for the misses the GPU path
// lists.
//
// [MD] ModelDock, "Strata はなぜ少ない VRAM でも速いのか", section
// "1 トークン、三者の分担": the card runs the experts it holds, the experts
// that are not on the card are computed by the CPU next to the RAM that
// holds them (that share of the step is bound by DRAM bandwidth), and the
// results are summed.  Here the card's part is moe_layer / moe_expert_ffn
// with a partial slot table (hits, plus the shared expert) and this file
// computes the listed misses, so that y_partial + misses = y_full.
//
// Work of one call: the misses are grouped by expert (ascending id), each
// group holding its tokens in ascending order; every expert's weights are
// streamed once for all of its tokens.
//  1. gate/up: rows of every group are split among threads; for each token
//     of the group a = G_e x_t, u = U_e x_t, h = silu(a) * u (fp32);
//  2. down: output rows are split among threads; each thread, for the rows
//     it owns, goes through the groups in order and adds g * (D_e h) into
//     y[t] -- so every element of y receives its additions in one fixed
//     order and the result does not depend on the thread count.
// Dequant is fused: a 32-weight block contributes d * sum(q x) + m * sum(x),
// sum(x) taken once per token and block.  AVX-512 when the CPU has it, else
// plain C++; both sum in the same block order.

#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <condition_variable>
#include <functional>
#include <mutex>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <thread>
#include <vector>

#include "moe.h"

namespace {

float bf16_to_f32(uint16_t b) {
  const uint32_t u = uint32_t(b) << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

// IEEE binary16 to binary32 (exact): normal numbers move their exponent
// and mantissa fields; zeros, subnormals, infinities and NaNs are handled
// apart.
float f16_to_f32(uint16_t h) {
  const uint32_t sign = uint32_t(h & 0x8000u) << 16, e = (h >> 10) & 31, m = h & 1023;
  uint32_t u;
  if (e != 0 && e != 31) {
    u = sign | ((e + 112) << 23) | (m << 13);
  } else if (e == 31) {
    u = sign | 0x7F800000u | (m << 13);
  } else {
    const float v = std::ldexp(float(m), -24);
    std::memcpy(&u, &v, 4);
    u |= sign;
  }
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

float silu(float a) { return a / (1.f + std::exp(-a)); }

// One matrix pool on the host: n matrices of [rows][cols].
struct View {
  int fmt, rows, cols;
  const uint8_t* codes;   // Q2/Q4
  const float* w;         // F32
  const uint16_t* sc;
  const uint16_t* mn;
  int64_t row_bytes() const { return int64_t(cols) * (fmt == MOE_W_Q2B32 ? 2 : 4) / 8; }
  int nb() const { return cols / 32; }
};

constexpr int kTok = 4;   // tokens per pass over a row

// Block code sums  s[v] = sum_j q_j x_v[32b + j]  of one row for up to kTok
// vectors, then acc[v] += d * s[v] + m * xs_v[b]: plain C++.
void row_dot_ref(const View& M, int64_t e, int r, const float* const* x,
                 const float* const* xs, int n, float* out) {
  float acc[kTok] = {0.f, 0.f, 0.f, 0.f};
  if (M.fmt == MOE_W_F32) {
    const float* w = M.w + (e * M.rows + r) * int64_t(M.cols);
    for (int c = 0; c < M.cols; ++c)
      for (int v = 0; v < n; ++v) acc[v] += w[c] * x[v][c];
  } else {
    const uint8_t* row = M.codes + (e * M.rows + r) * M.row_bytes();
    const int64_t mb = (e * M.rows + r) * int64_t(M.nb());
    const int bits = M.fmt == MOE_W_Q2B32 ? 2 : 4, per_byte = 8 / bits, mask = (1 << bits) - 1;
    for (int b = 0; b < M.nb(); ++b) {
      const float d = f16_to_f32(M.sc[mb + b]), m = f16_to_f32(M.mn[mb + b]);
      float s[kTok] = {0.f, 0.f, 0.f, 0.f};
      for (int j = 0; j < 32; ++j) {
        const int c = 32 * b + j;
        const float q = float((row[c / per_byte] >> (bits * (c % per_byte))) & mask);
        for (int v = 0; v < n; ++v) s[v] += q * x[v][c];
      }
      for (int v = 0; v < n; ++v) acc[v] += d * s[v] + m * xs[v][b];
    }
  }
  for (int v = 0; v < n; ++v) out[v] = acc[v];
}

// The same with AVX-512: 16 columns per vector, codes widened by variable
// shifts.  N (the number of vectors) is a compile-time constant so that the
// accumulators stay in registers; even and odd blocks accumulate apart.
template <int N>
__attribute__((target("avx512f,avx512bw,avx512vl"))) void row_dot_avx512_n(
    const View& M, int64_t e, int r, const float* const* x, const float* const* xs, float* out) {
  __m512 acc[2][N];
  float accm[N];
  for (int v = 0; v < N; ++v) {
    acc[0][v] = acc[1][v] = _mm512_setzero_ps();
    accm[v] = 0.f;
  }
  if (M.fmt == MOE_W_F32) {
    const float* w = M.w + (e * M.rows + r) * int64_t(M.cols);
    for (int c = 0; c < M.cols; c += 16) {
      const __m512 wv = _mm512_loadu_ps(w + c);
      for (int v = 0; v < N; ++v)
        acc[0][v] = _mm512_fmadd_ps(wv, _mm512_loadu_ps(x[v] + c), acc[0][v]);
    }
  } else {
    const uint8_t* row = M.codes + (e * M.rows + r) * M.row_bytes();
    const int64_t mb = (e * M.rows + r) * int64_t(M.nb());
    const bool q2 = M.fmt == MOE_W_Q2B32;
    // Q2: lane j takes column j of a 16-column half, bits 2j of its dword;
    // Q4: lane j takes dword j / 8 of the half, bits 4 (j % 8).
    const __m512i sh2 = _mm512_setr_epi32(0, 2, 4, 6, 8, 10, 12, 14, 16, 18, 20, 22, 24, 26, 28, 30);
    const __m512i sh4 = _mm512_setr_epi32(0, 4, 8, 12, 16, 20, 24, 28, 0, 4, 8, 12, 16, 20, 24, 28);
    const __m512i sel4 = _mm512_setr_epi32(0, 0, 0, 0, 0, 0, 0, 0, 1, 1, 1, 1, 1, 1, 1, 1);
    const __m512i m2 = _mm512_set1_epi32(3), m4 = _mm512_set1_epi32(15);
    alignas(64) float dd[16], mm[16];
    for (int b = 0; b < M.nb(); ++b) {
      if (b % 16 == 0) {   // the next 16 blocks' scales and minima (fp16 -> fp32)
        const int nbk = std::min(16, M.nb() - b);
        const __mmask16 k = __mmask16((1u << nbk) - 1u);
        _mm512_store_ps(dd, _mm512_cvtph_ps(_mm256_maskz_loadu_epi16(k, M.sc + mb + b)));
        _mm512_store_ps(mm, _mm512_cvtph_ps(_mm256_maskz_loadu_epi16(k, M.mn + mb + b)));
      }
      __m512 q[2];
      if (q2) {
        uint32_t wd[2];
        std::memcpy(wd, row + 8 * b, 8);
        for (int hh = 0; hh < 2; ++hh)
          q[hh] = _mm512_cvtepi32_ps(
              _mm512_and_si512(_mm512_srlv_epi32(_mm512_set1_epi32(int(wd[hh])), sh2), m2));
      } else {
        const __m512i w4 = _mm512_castsi128_si512(_mm_loadu_si128(reinterpret_cast<const __m128i*>(row + 16 * b)));
        for (int hh = 0; hh < 2; ++hh) {
          const __m512i pair = _mm512_permutexvar_epi32(
              _mm512_add_epi32(sel4, _mm512_set1_epi32(2 * hh)), w4);
          q[hh] = _mm512_cvtepi32_ps(_mm512_and_si512(_mm512_srlv_epi32(pair, sh4), m4));
        }
      }
      const __m512 d = _mm512_set1_ps(dd[b % 16]);
      const float m = mm[b % 16];
      for (int v = 0; v < N; ++v) {
        const float* xb = x[v] + 32 * b;
        const __m512 sv = _mm512_fmadd_ps(q[1], _mm512_loadu_ps(xb + 16),
                                          _mm512_mul_ps(q[0], _mm512_loadu_ps(xb)));
        acc[b & 1][v] = _mm512_fmadd_ps(d, sv, acc[b & 1][v]);
        accm[v] += m * xs[v][b];
      }
    }
  }
  for (int v = 0; v < N; ++v)
    out[v] = _mm512_reduce_add_ps(_mm512_add_ps(acc[0][v], acc[1][v])) + accm[v];
}

void row_dot_avx512(const View& M, int64_t e, int r, const float* const* x,
                    const float* const* xs, int n, float* out) {
  switch (n) {
    case 1: row_dot_avx512_n<1>(M, e, r, x, xs, out); break;
    case 2: row_dot_avx512_n<2>(M, e, r, x, xs, out); break;
    case 3: row_dot_avx512_n<3>(M, e, r, x, xs, out); break;
    default: row_dot_avx512_n<4>(M, e, r, x, xs, out); break;
  }
}

using RowDot = void (*)(const View&, int64_t, int, const float* const*, const float* const*, int,
                        float*);

// AVX-512 when the CPU has it, unless MOE_HOST_ISA=generic asks for the
// plain code (for CPUs where wide vectors lower the clock).
bool use_avx512() {
  const char* isa = std::getenv("MOE_HOST_ISA");
  if (isa && std::strcmp(isa, "generic") == 0) return false;
  __builtin_cpu_init();
  return __builtin_cpu_supports("avx512f") && __builtin_cpu_supports("avx512bw") &&
         __builtin_cpu_supports("avx512vl");
}

RowDot pick_row_dot() { return use_avx512() ? row_dot_avx512 : row_dot_ref; }

View view_of(const moe_mat& m, int rows, int cols) {
  View v{};
  v.fmt = m.fmt;
  v.rows = rows;
  v.cols = cols;
  v.codes = static_cast<const uint8_t*>(m.data);
  v.w = static_cast<const float*>(m.data);
  v.sc = m.scale;
  v.mn = m.min;
  return v;
}

// Worker threads kept for the life of the process.  run(n, threads, f)
// calls f(i) for every i in [0, n) on the caller and up to threads - 1
// workers, items taken from a shared counter (each item writes its own
// outputs, so which thread takes it does not matter), and returns when all
// are done.  One run at a time (a mutex serialises callers).
class Pool {
 public:
  template <typename F>
  void run(int n, int threads, F&& f) {
    threads = std::max(1, std::min(threads, n));
    if (threads == 1) {
      for (int i = 0; i < n; ++i) f(i);
      return;
    }
    std::lock_guard<std::mutex> one_run(run_mu_);
    {
      std::lock_guard<std::mutex> lk(mu_);
      while (int(workers_.size()) < threads - 1)
        workers_.emplace_back([this, id = int(workers_.size())] { loop(id); });
      job_ = [&f](int i) { f(i); };
      n_ = n;
      next_.store(0);
      want_ = threads - 1;
      busy_ = threads - 1;
      ++gen_;
    }
    cv_.notify_all();
    work();
    std::unique_lock<std::mutex> lk(mu_);
    done_cv_.wait(lk, [this] { return busy_ == 0; });
    job_ = nullptr;
  }

  ~Pool() {
    {
      std::lock_guard<std::mutex> lk(mu_);
      stop_ = true;
    }
    cv_.notify_all();
    for (auto& t : workers_) t.join();
  }

 private:
  void work() {
    for (int i = next_.fetch_add(1); i < n_; i = next_.fetch_add(1)) job_(i);
  }
  void loop(int id) {
    uint64_t seen = 0;
    for (;;) {
      std::unique_lock<std::mutex> lk(mu_);
      cv_.wait(lk, [&] { return stop_ || gen_ != seen; });
      if (stop_) return;
      seen = gen_;
      if (id >= want_) continue;   // not needed for this run
      lk.unlock();
      work();
      lk.lock();
      if (--busy_ == 0) done_cv_.notify_one();
    }
  }

  std::mutex run_mu_, mu_;
  std::condition_variable cv_, done_cv_;
  std::vector<std::thread> workers_;
  std::function<void(int)> job_;
  std::atomic<int> next_{0};
  int n_ = 0, want_ = 0, busy_ = 0;
  uint64_t gen_ = 0;
  bool stop_ = false;
};

Pool& pool() {
  static Pool p;
  return p;
}

template <typename F>
void parallel_for(int n, int threads, F f) {
  pool().run(n, threads, f);
}

bool mat_ok(const moe_mat& m, int fmt) {
  if (m.fmt != fmt || !m.data) return false;
  if (fmt == MOE_W_F32) return true;
  return (fmt == MOE_W_Q2B32 || fmt == MOE_W_Q4B32) && m.scale && m.min;
}

}  // namespace

extern "C" int32_t moe_host_isa(void) { return use_avx512() ? 1 : 0; }

extern "C" moe_status moe_host_miss_ffn(int32_t E, int32_t H, int32_t I, moe_mat gate, moe_mat up,
                                        moe_mat down, const uint16_t* x, int32_t T,
                                        const moe_miss* miss, const int32_t* miss_off, float* y,
                                        int32_t n_threads) {
  if (T < 0 || E < 1 || H < 32 || I < 32 || H % 32 || I % 32 || H > 65536 || I > 65536)
    return MOE_ERR_INVALID;
  if (T == 0) return MOE_OK;
  if (!x || !miss_off || !y) return MOE_ERR_INVALID;
  const int fmt = gate.fmt;
  if (fmt != MOE_W_F32 && fmt != MOE_W_Q2B32 && fmt != MOE_W_Q4B32) return MOE_ERR_UNSUPPORTED;
  if (!mat_ok(gate, fmt) || !mat_ok(up, fmt) || !mat_ok(down, fmt)) return MOE_ERR_INVALID;
  // the list: offsets non-decreasing from 0, every entry's token and expert
  // in range, a token naming an expert at most once
  if (miss_off[0] != 0) return MOE_ERR_INVALID;
  for (int t = 0; t < T; ++t)
    if (miss_off[t + 1] < miss_off[t]) return MOE_ERR_INVALID;
  const int n_miss = miss_off[T];
  if (n_miss > 0 && !miss) return MOE_ERR_INVALID;
  for (int t = 0; t < T; ++t)
    for (int i = miss_off[t]; i < miss_off[t + 1]; ++i) {
      if (miss[i].token != t || miss[i].expert < 0 || miss[i].expert >= E) return MOE_ERR_INVALID;
      for (int j = miss_off[t]; j < i; ++j)
        if (miss[j].expert == miss[i].expert) return MOE_ERR_INVALID;
    }
  if (n_miss == 0) return MOE_OK;

  int threads = n_threads > 0 ? n_threads : int(std::thread::hardware_concurrency());
  threads = std::max(1, std::min(threads, 256));
  static const RowDot row_dot = pick_row_dot();
  const View G = view_of(gate, I, H), U = view_of(up, I, H), D = view_of(down, H, I);

  // groups: misses by expert (ascending id), tokens ascending within a group
  std::vector<int> order(n_miss);
  for (int i = 0; i < n_miss; ++i) order[i] = i;
  std::stable_sort(order.begin(), order.end(),
                   [&](int a, int b) { return miss[a].expert < miss[b].expert; });
  std::vector<int> gstart;   // group g holds order[gstart[g] .. gstart[g+1])
  for (int i = 0; i < n_miss; ++i)
    if (i == 0 || miss[order[i]].expert != miss[order[i - 1]].expert) gstart.push_back(i);
  const int n_groups = int(gstart.size());
  gstart.push_back(n_miss);

  // tokens as fp32 with per-block sums (only tokens that have misses)
  std::vector<float> xf(size_t(T) * H), xs(size_t(T) * (H / 32));
  for (int t = 0; t < T; ++t) {
    if (miss_off[t + 1] == miss_off[t]) continue;
    for (int c = 0; c < H; ++c) xf[size_t(t) * H + c] = bf16_to_f32(x[size_t(t) * H + c]);
    for (int b = 0; b < H / 32; ++b) {
      float s = 0.f;
      for (int j = 0; j < 32; ++j) s += xf[size_t(t) * H + 32 * b + j];
      xs[size_t(t) * (H / 32) + b] = s;
    }
  }

  // 1. gate/up: h[i of order][I], rows of each group in blocks of 16
  std::vector<float> h(size_t(n_miss) * I), hs(size_t(n_miss) * (I / 32));
  constexpr int kRows = 16;
  const int rb_per = (I + kRows - 1) / kRows;
  parallel_for(n_groups * rb_per, threads, [&](int wi) {
    const int g = wi / rb_per, r0 = (wi % rb_per) * kRows, r1 = std::min(I, r0 + kRows);
    const int64_t e = miss[order[gstart[g]]].expert;
    for (int p0 = gstart[g]; p0 < gstart[g + 1]; p0 += kTok) {
      const int n = std::min(kTok, gstart[g + 1] - p0);
      const float* xv[kTok];
      const float* xsv[kTok];
      for (int v = 0; v < n; ++v) {
        const int t = miss[order[p0 + v]].token;
        xv[v] = xf.data() + size_t(t) * H;
        xsv[v] = xs.data() + size_t(t) * (H / 32);
      }
      for (int r = r0; r < r1; ++r) {
        float a[kTok], u[kTok];
        row_dot(G, e, r, xv, xsv, n, a);
        row_dot(U, e, r, xv, xsv, n, u);
        for (int v = 0; v < n; ++v) h[size_t(p0 + v) * I + r] = silu(a[v]) * u[v];
      }
    }
  });
  for (int p = 0; p < n_miss; ++p)
    for (int b = 0; b < I / 32; ++b) {
      float s = 0.f;
      for (int j = 0; j < 32; ++j) s += h[size_t(p) * I + 32 * b + j];
      hs[size_t(p) * (I / 32) + b] = s;
    }

  // 2. down: each thread owns output rows, groups in order
  const int ob_per = (H + kRows - 1) / kRows;
  parallel_for(ob_per, threads, [&](int wi) {
    const int r0 = wi * kRows, r1 = std::min(H, r0 + kRows);
    for (int g = 0; g < n_groups; ++g) {
      const int64_t e = miss[order[gstart[g]]].expert;
      for (int p0 = gstart[g]; p0 < gstart[g + 1]; p0 += kTok) {
        const int n = std::min(kTok, gstart[g + 1] - p0);
        const float* hv[kTok];
        const float* hsv[kTok];
        for (int v = 0; v < n; ++v) {
          hv[v] = h.data() + size_t(p0 + v) * I;
          hsv[v] = hs.data() + size_t(p0 + v) * (I / 32);
        }
        for (int r = r0; r < r1; ++r) {
          float o[kTok];
          row_dot(D, e, r, hv, hsv, n, o);
          for (int v = 0; v < n; ++v) {
            const moe_miss& mm = miss[order[p0 + v]];
            y[size_t(mm.token) * H + r] += mm.gate * o[v];
          }
        }
      }
    }
  });
  return MOE_OK;
}
