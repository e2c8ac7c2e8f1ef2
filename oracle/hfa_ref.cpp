// CPU oracle for exact attention forward -- TEST INFRASTRUCTURE ONLY.
//
// This file is the slow, obviously-correct reference that the GPU kernels are
// checked against.  Only the test suite, the smoke check and the CPU-baseline
// leg of the benchmark may load it; the product library never links or calls
// it, and it shares no code, header or constant with the GPU path.
//
// Arithmetic is IEEE fp64 throughout.  Inputs (fp32, or bf16 given as raw
// 16-bit patterns) are widened exactly to fp64 before any arithmetic.  exp and
// log are the host libm functions, called, not reimplemented.
//
// Two entry points:
//
//  hfa_ref_attn_fwd         the definition, "Attention(Q,K,V) = softmax(QK^T /
//                           sqrt(d_k)) V" (neuralmasteryai "Hardware
//                           Acceleration & Custom Kernels", section 2), with the
//                           numerically stable row softmax of the book chapter
//                           "Triton and kernel fusion" (section "Fusion": pad,
//                           subtract the row max, exponentiate, sum, divide).
//                           Every score row S[i, 0:N] is materialised in fp64
//                           before the softmax is taken.
//
//  hfa_ref_attn_fwd_online  the same quantity computed by the online
//                           normalisation identity of the same section 2, step 2
//                           (running max m and running denominator, there called
//                           d, here l), applied tile by tile over the keys with
//                           the running output sums rescaled by the same factor.
//                           tile == 1 is the scalar recurrence exactly as the
//                           page states it.  Used only to pin the identity
//                           against the definition.
//
// Two more for the standalone row softmax (book chapter "Triton and kernel
// fusion", section "Fusion", and its stretch exercise on rows wider than one
// block):
//
//  hfa_ref_softmax_rows         y_ij = exp(x_ij - m_i) / sum_j exp(x_ij - m_i),
//                               m_i = max_j x_ij, over fp32 rows widened to fp64.
//
//  hfa_ref_softmax_rows_online  the same, with (m_i, l_i) taken in one sweep by
//                               the running-max / running-sum identity (the
//                               neuralmasteryai section 2, step 2 recurrence)
//                               over chunks of `chunk` columns; chunk == 1 is
//                               the scalar recurrence.  Used only to pin the
//                               identity against the definition.
//
// One more for the RMS normalisation of the same pages (TritonForge "Fused
// RMSNorm" card: RMSNorm(x) = x / sqrt(sum_i x_i^2 / d + eps) * gamma; book
// chapter "Triton and kernel fusion", section "Fused residual add + RMSNorm":
// the residual is added first, the sum is normalised, and the sum itself is
// returned as a second output):
//
//  hfa_ref_rmsnorm  s_ij = x_ij + r_ij, formed in fp32 as the chapter's kernel
//                   forms it (both operands upcast to fp32, one fp32 add; s = x
//                   when there is no residual), then in fp64
//                   y_ij = s_ij / sqrt(sum_j s_ij^2 / C + eps) * w_j.
//                   Returns y and s, both fp64.
//
// Both attention entry points also return the row log-sum-exp
// LSE_i = ln(sum_j exp(s_ij)) of the scaled scores (natural log).  The pages do not define it; it is the plain
// reading: the running max plus the log of the running denominator.
//
// Layout: q, k, v are contiguous [B, H, N, d].  `rows` (may be NULL) selects
// which query rows of every (b, h) head are computed; outputs are
// o[B*H, R, d] and lse[B*H, R] in fp64, R = n_rows (or N when rows is NULL).
//
// Return value: 0 on success, -1 on an invalid argument.

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>

namespace {

// dtype codes of the oracle's own ABI: 0 = fp32, 1 = bf16 bit patterns.
double widen(const void* base, int dtype, int64_t idx) {
  if (dtype == 0) return static_cast<double>(static_cast<const float*>(base)[idx]);
  // bf16 is the upper half of an fp32 bit pattern: shifting it back is exact.
  uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return static_cast<double>(f);
}

struct Problem {
  const void* q;
  const void* k;
  const void* v;
  int dtype;
  int64_t BH, N, d;
  double scale;
  const int64_t* rows;
  int64_t R;
  double* o;
  double* lse;
  int64_t tile;  // 0 = direct definition, >= 1 = online recurrence with this key tile
};

// Widened copy of one head's K or V: [N, d] fp64.
void widen_head(const void* src, int dtype, int64_t head, int64_t N, int64_t d,
                std::vector<double>& dst) {
  dst.resize(static_cast<size_t>(N * d));
  const int64_t base = head * N * d;
  for (int64_t t = 0; t < N * d; ++t) dst[t] = widen(src, dtype, base + t);
}

// Score s_j = scale * sum_c q_c * k_jc for one query row against every key.
void score_row(const std::vector<double>& qrow, const std::vector<double>& K, int64_t N,
               int64_t d, double scale, std::vector<double>& S) {
  for (int64_t j = 0; j < N; ++j) {
    double dot = 0.0;
    for (int64_t c = 0; c < d; ++c) dot += qrow[c] * K[j * d + c];
    S[j] = scale * dot;
  }
}

// Definition: materialise the score row, subtract its max, exponentiate,
// normalise, weight V.
void row_direct(const std::vector<double>& qrow, const std::vector<double>& K,
                const std::vector<double>& V, int64_t N, int64_t d, double scale,
                std::vector<double>& S, double* out, double* lse_out) {
  score_row(qrow, K, N, d, scale, S);
  double m = S[0];
  for (int64_t j = 1; j < N; ++j) m = std::max(m, S[j]);
  double l = 0.0;
  for (int64_t j = 0; j < N; ++j) {
    S[j] = std::exp(S[j] - m);  // S now holds the unnormalised probabilities p_j
    l += S[j];
  }
  for (int64_t c = 0; c < d; ++c) {
    double num = 0.0;
    for (int64_t j = 0; j < N; ++j) num += S[j] * V[j * d + c];
    out[c] = num / l;
  }
  *lse_out = m + std::log(l);
}

// Online normalisation: keys arrive in tiles of `tile`; the state is the
// running max m, the running denominator l and the running weighted sums acc.
// On each tile: m_new = max(m_old, max of the tile's scores);
//   l   <- l   * e^(m_old - m_new) + sum_j e^(x_j - m_new)
//   acc <- acc * e^(m_old - m_new) + sum_j e^(x_j - m_new) v_j
// and finally O = acc / l, LSE = m + ln l.
void row_online(const std::vector<double>& qrow, const std::vector<double>& K,
                const std::vector<double>& V, int64_t N, int64_t d, double scale, int64_t tile,
                std::vector<double>& S, std::vector<double>& acc, double* out, double* lse_out) {
  score_row(qrow, K, N, d, scale, S);
  double m_old = -INFINITY;
  double l = 0.0;
  std::fill(acc.begin(), acc.end(), 0.0);
  for (int64_t j0 = 0; j0 < N; j0 += tile) {
    const int64_t j1 = std::min(N, j0 + tile);
    double m_new = m_old;
    for (int64_t j = j0; j < j1; ++j) m_new = std::max(m_new, S[j]);
    const double alpha = std::exp(m_old - m_new);  // exp(-inf) = 0 on the first tile
    double tile_sum = 0.0;
    for (int64_t c = 0; c < d; ++c) acc[c] *= alpha;
    for (int64_t j = j0; j < j1; ++j) {
      const double p = std::exp(S[j] - m_new);
      tile_sum += p;
      for (int64_t c = 0; c < d; ++c) acc[c] += p * V[j * d + c];
    }
    l = l * alpha + tile_sum;
    m_old = m_new;
  }
  for (int64_t c = 0; c < d; ++c) out[c] = acc[c] / l;
  *lse_out = m_old + std::log(l);
}

void run(const Problem& P, int threads) {
  std::vector<double> K, V;
  for (int64_t h = 0; h < P.BH; ++h) {
    widen_head(P.k, P.dtype, h, P.N, P.d, K);
    widen_head(P.v, P.dtype, h, P.N, P.d, V);
    auto worker = [&](int64_t r_begin, int64_t r_end) {
      std::vector<double> S(static_cast<size_t>(P.N));
      std::vector<double> acc(static_cast<size_t>(P.d));
      std::vector<double> qrow(static_cast<size_t>(P.d));
      for (int64_t r = r_begin; r < r_end; ++r) {
        const int64_t i = P.rows ? P.rows[r] : r;
        for (int64_t c = 0; c < P.d; ++c) qrow[c] = widen(P.q, P.dtype, (h * P.N + i) * P.d + c);
        double* out = P.o + (h * P.R + r) * P.d;
        double* lse = P.lse + h * P.R + r;
        if (P.tile == 0)
          row_direct(qrow, K, V, P.N, P.d, P.scale, S, out, lse);
        else
          row_online(qrow, K, V, P.N, P.d, P.scale, P.tile, S, acc, out, lse);
      }
    };
    const int64_t nt = std::max<int64_t>(1, std::min<int64_t>(threads, P.R));
    std::vector<std::thread> pool;
    const int64_t chunk = (P.R + nt - 1) / nt;
    for (int64_t t = 0; t < nt; ++t) {
      const int64_t b = t * chunk, e = std::min(P.R, b + chunk);
      if (b < e) pool.emplace_back(worker, b, e);
    }
    for (auto& th : pool) th.join();
  }
}

int check_and_run(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                  int64_t N, int64_t d, double scale, const int64_t* rows, int64_t n_rows,
                  double* o, double* lse, int threads, int64_t tile) {
  if (!q || !k || !v || !o || !lse) return -1;
  if (dtype != 0 && dtype != 1) return -1;
  if (B < 1 || H < 1 || N < 1 || d < 1 || tile < 0) return -1;
  if (!std::isfinite(scale)) return -1;
  const int64_t R = rows ? n_rows : N;
  if (R < 0) return -1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= N) return -1;
  if (threads < 1) threads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  Problem P{q, k, v, dtype, B * H, N, d, scale, rows, R, o, lse, tile};
  run(P, threads);
  return 0;
}

// ---- standalone row softmax -------------------------------------------------

// Definition form of one row: max, exponentials, sum, divide (fp64).
void softmax_row_direct(const float* x, int64_t C, double* y) {
  double m = -INFINITY;
  for (int64_t j = 0; j < C; ++j) m = std::max(m, static_cast<double>(x[j]));
  double l = 0.0;
  for (int64_t j = 0; j < C; ++j) {
    y[j] = std::exp(static_cast<double>(x[j]) - m);
    l += y[j];
  }
  for (int64_t j = 0; j < C; ++j) y[j] /= l;
}

// One sweep for (m, l) by the running identity over chunks, then the outputs:
// for each chunk, m_new = max(m, chunk max), l = l * exp(m - m_new) +
// sum over the chunk of exp(x - m_new).
void softmax_row_online(const float* x, int64_t C, int64_t chunk, double* y) {
  double m = -INFINITY, l = 0.0;
  for (int64_t b = 0; b < C; b += chunk) {
    const int64_t e = std::min(C, b + chunk);
    double cm = -INFINITY;
    for (int64_t j = b; j < e; ++j) cm = std::max(cm, static_cast<double>(x[j]));
    const double m_new = std::max(m, cm);
    double cs = 0.0;
    for (int64_t j = b; j < e; ++j) cs += std::exp(static_cast<double>(x[j]) - m_new);
    l = (l == 0.0 ? 0.0 : l * std::exp(m - m_new)) + cs;
    m = m_new;
  }
  for (int64_t j = 0; j < C; ++j) y[j] = std::exp(static_cast<double>(x[j]) - m) / l;
}

int softmax_check_and_run(const float* x, int64_t R, int64_t C, int64_t chunk, const int64_t* rows,
                          int64_t n_rows, double* y, int threads) {
  if (!x || !y || R < 1 || C < 1 || chunk < 0) return -1;
  const int64_t n = rows ? n_rows : R;
  if (n < 0) return -1;
  if (rows)
    for (int64_t r = 0; r < n_rows; ++r)
      if (rows[r] < 0 || rows[r] >= R) return -1;
  for (int64_t i = 0; i < (rows ? n_rows : R); ++i) {
    const float* row = x + (rows ? rows[i] : i) * C;
    for (int64_t j = 0; j < C; ++j)
      if (!std::isfinite(row[j])) return -1;
  }
  if (threads < 1) threads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  auto worker = [&](int64_t b, int64_t e) {
    for (int64_t i = b; i < e; ++i) {
      const float* row = x + (rows ? rows[i] : i) * C;
      if (chunk == 0)
        softmax_row_direct(row, C, y + i * C);
      else
        softmax_row_online(row, C, chunk, y + i * C);
    }
  };
  const int64_t per = (n + threads - 1) / threads;
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    const int64_t b = t * per, e = std::min(n, b + per);
    if (b < e) pool.emplace_back(worker, b, e);
  }
  for (auto& th : pool) th.join();
  return 0;
}

// ---- RMS normalisation ---------------------------------------------------------

// The fp32 sum of the chapter's kernel: both operands upcast to fp32, one
// IEEE fp32 add (round to nearest even; the build disables contraction).
double residual_sum(const void* x, const void* r, int dtype, int64_t idx) {
  const float a = static_cast<float>(widen(x, dtype, idx));
  if (!r) return static_cast<double>(a);
  const float b = static_cast<float>(widen(r, dtype, idx));
  const float sum = a + b;
  return static_cast<double>(sum);
}

// One row: the sum, its mean square, the normalised and weighted output.
// Returns false when the mean square plus eps is not positive.
bool rmsnorm_row(const void* x, const void* r, const void* w, int dtype, int64_t row, int64_t C,
                 double eps, double* y, double* s) {
  double sq = 0.0;
  for (int64_t j = 0; j < C; ++j) {
    s[j] = residual_sum(x, r, dtype, row * C + j);
    sq += s[j] * s[j];
  }
  const double denom = std::sqrt(sq / static_cast<double>(C) + eps);
  if (!(denom > 0.0)) return false;
  for (int64_t j = 0; j < C; ++j) y[j] = s[j] / denom * widen(w, dtype, j);
  return true;
}

int rmsnorm_check_and_run(const void* x, const void* r, const void* w, int dtype, int64_t R, int64_t C,
                          double eps, const int64_t* rows, int64_t n_rows, double* y, double* s_out,
                          int threads) {
  if (!x || !w || !y || R < 1 || C < 1 || (dtype != 0 && dtype != 1)) return -1;
  if (!std::isfinite(eps) || eps < 0.0) return -1;
  const int64_t n = rows ? n_rows : R;
  if (n < 0) return -1;
  if (rows)
    for (int64_t i = 0; i < n_rows; ++i)
      if (rows[i] < 0 || rows[i] >= R) return -1;
  for (int64_t j = 0; j < C; ++j)
    if (!std::isfinite(widen(w, dtype, j))) return -1;
  for (int64_t i = 0; i < n; ++i) {
    const int64_t row = rows ? rows[i] : i;
    for (int64_t j = 0; j < C; ++j) {
      if (!std::isfinite(widen(x, dtype, row * C + j))) return -1;
      if (r && !std::isfinite(widen(r, dtype, row * C + j))) return -1;
    }
  }
  if (threads < 1) threads = static_cast<int>(std::max(1u, std::thread::hardware_concurrency()));
  std::vector<int> ok(static_cast<size_t>(threads), 1);
  auto worker = [&](int t, int64_t b, int64_t e) {
    std::vector<double> scratch(static_cast<size_t>(C));
    for (int64_t i = b; i < e; ++i) {
      double* s = s_out ? s_out + i * C : scratch.data();
      if (!rmsnorm_row(x, r, w, dtype, rows ? rows[i] : i, C, eps, y + i * C, s)) ok[t] = 0;
    }
  };
  const int64_t per = (n + threads - 1) / threads;
  std::vector<std::thread> pool;
  for (int t = 0; t < threads; ++t) {
    const int64_t b = t * per, e = std::min(n, b + per);
    if (b < e) pool.emplace_back(worker, t, b, e);
  }
  for (auto& th : pool) th.join();
  for (int v : ok)
    if (!v) return -1;
  return 0;
}

}  // namespace

extern "C" {

// x, r (may be NULL: no residual), w: contiguous, dtype 0 = fp32, 1 = bf16 bit
// patterns; x and r are [R, C], w is [C].  rows (may be NULL) selects the rows
// computed.  y and s_out (may be NULL) are fp64 [n_rows or R, C].  0 on
// success, -1 on an invalid argument (non-finite inputs, eps < 0, or a row
// whose mean square plus eps is 0).
int hfa_ref_rmsnorm(const void* x, const void* r, const void* w, int dtype, int64_t R, int64_t C, double eps,
                    const int64_t* rows, int64_t n_rows, double* y, double* s_out, int threads) {
  return rmsnorm_check_and_run(x, r, w, dtype, R, C, eps, rows, n_rows, y, s_out, threads);
}

// x: fp32 [R, C] contiguous; rows (may be NULL) selects the rows computed;
// y: fp64 [n_rows or R, C].  0 on success, -1 on an invalid argument
// (non-finite inputs included).
int hfa_ref_softmax_rows(const float* x, int64_t R, int64_t C, const int64_t* rows, int64_t n_rows, double* y,
                         int threads) {
  return softmax_check_and_run(x, R, C, 0, rows, n_rows, y, threads);
}

int hfa_ref_softmax_rows_online(const float* x, int64_t R, int64_t C, int64_t chunk, const int64_t* rows,
                                int64_t n_rows, double* y, int threads) {
  if (chunk < 1) return -1;
  return softmax_check_and_run(x, R, C, chunk, rows, n_rows, y, threads);
}

int hfa_ref_attn_fwd(const void* q, const void* k, const void* v, int dtype, int64_t B, int64_t H,
                     int64_t N, int64_t d, double scale, const int64_t* rows, int64_t n_rows,
                     double* o, double* lse, int threads) {
  return check_and_run(q, k, v, dtype, B, H, N, d, scale, rows, n_rows, o, lse, threads, 0);
}

int hfa_ref_attn_fwd_online(const void* q, const void* k, const void* v, int dtype, int64_t B,
                            int64_t H, int64_t N, int64_t d, double scale, int64_t tile,
                            const int64_t* rows, int64_t n_rows, double* o, double* lse,
                            int threads) {
  if (tile < 1) return -1;
  return check_and_run(q, k, v, dtype, B, H, N, d, scale, rows, n_rows, o, lse, threads, tile);
}

}  // extern "C"
