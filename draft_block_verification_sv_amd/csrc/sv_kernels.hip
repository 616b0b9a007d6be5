// HIP kernels for batched draft-block verification on gfx950 (MI355X).
//
// One call of the verification path runs five kernels on the caller's stream:
//
//   sv_plan      one workgroup: packed-layout offsets from k (AdaFlash paper,
//                Section 3.3: one batch of total length sum k_b), per-row
//                descriptors, input validation.
//   sv_rows      the streaming pass (sv_rows.hip).  One wavefront per (row, slice):
//                every target and draft logit is read from HBM exactly once, with
//                16-byte loads, and reduced to per-slice statistics: max, the
//                softmax sums at temperature 1 and T_b, the first argmax, and for
//                draft rows the two quantities the clipped reverse-KL needs,
//                W = sum E_y (l_q - l_p) and G = max E_y (l_q - l_p), E_y the
//                slice-relative exponential of the draft logit.
//   sv_finalize  one wavefront per target row: combines the slice statistics in a
//                fixed order into log-normalisers; the clipped reverse-KL (AdaFlash
//                paper, Section 3.1 equation) from W and the sums, re-reading only
//                slices where an entry could reach delta; the acceptance test
//                u < min(1, p_T(x)/q_T(x)) (paper, Section 2.1) or, for T = 0, the
//                argmax match (DFlash notes, Section 5.2, worked example #4).
//   sv_sample_chunks  grid (request, 2048-column chunk): the first-rejection scan,
//                then the mass of each chunk of the residual max(0, p_T - q_T) at
//                the rejected position (reading notes, basic recipe step 4) or of
//                p_T of the bonus row (DFlash notes, Section 3.1 step 6).
//   sv_sample_finish  one workgroup per request: locates u * Z among the chunk
//                masses, scans that one chunk for the token, and emits a_b drafts
//                + 1 token.
//
// Why W and G make one HBM pass enough for the clipped sum:
//   t_y = q_y (ln q_y - ln p_y) = ln2 * 2^(k_y - LZq) * (L2E d_y + c2), with
//   d_y = l_q - l_p, k_y = l_q * L2E, c2 = LZp - LZq (log2 normalisers).  Inside a
//   slice with offset K_s, 2^(k_y - LZq) = E_y 2^(K_s - LZq), so
//     sum_{y in s} t_y      = ln2 2^(K_s - LZq) (L2E W_s + c2 S_s)      (exact), and
//     max_{y in s} t_y     <= ln2 2^(K_s - LZq) (L2E G_s + max(c2, 0)).
//   When that bound is below delta no entry of the slice is clipped and the exact
//   unclipped sum is the clipped sum; otherwise the slice (8 KiB) is re-read and
//   summed entry by entry with min(delta, .).
#include <float.h>
#include <math.h>

#include "sv_device.h"
#include "sv_layout.h"
#include "sv_launch.h"

namespace sv {

constexpr int kReqInvalid = 4 | 8 | 16;  // SV_DEV_BAD_TOKEN | BAD_TEMPERATURE | BAD_UNIFORM

// =========================================================================== plan
__device__ __forceinline__ int block_excl_scan_1024(int v, int* lds_waves, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int o = __shfl_up(x, d, 64);
    if (lane >= d) x += o;
  }
  if (lane == 63) lds_waves[wave] = x;
  __syncthreads();
  int base = 0, tot = 0;
  for (int w = 0; w < 16; ++w) {
    if (w < wave) base += lds_waves[w];
    tot += lds_waves[w];
  }
  __syncthreads();
  *total = tot;
  return base + x - v;
}

__global__ __launch_bounds__(1024) void sv_plan_kernel(PlanArgs a) {
  __shared__ int s_waves[16];
  __shared__ int s_bad_len, s_status;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_bad_len = 0;
    s_status = 0;
  }
  __syncthreads();
  Workspace& ws = a.ws;
  // 1. offsets: exclusive scan of k_b + 1 over the requests, 1024 at a time
  int carry = 0;
  for (int64_t base = 0; base < a.B; base += 1024) {
    const int64_t b = base + tid;
    int kb = 0;
    if (b < a.B) {
      kb = a.k[b];
      if (kb < 1 || kb > a.k_max) {
        atomicOr(&s_bad_len, 1);
        kb = 0;
      }
    }
    int total = 0;
    const int excl = block_excl_scan_1024(b < a.B ? kb + 1 : 0, s_waves, &total);
    if (b < a.B) ws.off_t[b] = carry + excl;
    carry += total;
  }
  __syncthreads();
  const bool bad_len = s_bad_len != 0;
  const bool mismatch = !bad_len && (static_cast<int64_t>(carry) != a.n_d + a.B);
  if (tid == 0) {
    ws.off_t[a.B] = carry;
    ws.glob[0] = (bad_len || mismatch) ? 1 : 0;
  }
  if (!bad_len && !mismatch) {
    // 2. per request: temperature mode, and the descriptor of each of its rows (stores only)
    for (int64_t b = tid; b < a.B; b += 1024) {
      const int off = ws.off_t[b];
      const int kb = a.k[b];
      const float T = a.temperature ? a.temperature[b] : 1.0f;
      int flags = 0, mode = 0;
      float beta = kL2E;
      if (!(T >= 0.0f) || isinf(T) || (T > 0.0f && T < FLT_MIN)) {
        flags = 8;
      } else if (T == 0.0f) {
        mode = 1;
      } else if (T != 1.0f) {
        mode = 2;
        beta = kL2E / T;
      }
      for (int i = 0; i <= kb; ++i) {
        RowDesc rd;
        rd.d = (i < kb) ? static_cast<int32_t>(off - b + i) : -1;
        rd.b = static_cast<int32_t>(b);
        rd.mode = mode;
        rd.beta = beta;
        ws.desc[off + i] = rd;
      }
      ws.req_flags[b] = flags;
      if (flags) atomicOr(&s_status, flags);
    }
    __syncthreads();  // descriptors and flags written above are visible to the whole block
    // 3. per target row: the row's uniform, and the draft token it scores
    const int64_t n_t = a.n_d + a.B;
    for (int64_t t = tid; t < n_t; t += 1024) {
      const RowDesc rd = ws.desc[t];
      const float u = a.uniforms[t];
      int f = (u >= 0.0f && u < 1.0f) ? 0 : 16;
      if (rd.d >= 0) {
        const int32_t x = a.tokens[rd.d];
        if (x < 0 || static_cast<int64_t>(x) >= a.V) f |= 4;
      }
      if (f) {
        atomicOr(&ws.req_flags[rd.b], f);
        atomicOr(&s_status, f);
      }
    }
  }
  __syncthreads();
  if (tid == 0) *a.device_status = s_status | (bad_len ? 1 : 0) | (mismatch ? 2 : 0);
}

// =========================================================================== finalize
template <int DT>
__device__ __forceinline__ float load_logit(const void* base, int64_t idx) {
  if constexpr (DT == 0) return bf16_at(static_cast<const uint16_t*>(base) + idx);
  else return static_cast<const float*>(base)[idx];
}

// Combines the slice records [rec0, rec0 + n_slices) of one row into the log2
// normaliser LZ = K + log2(sum_s S_s 2^(K_s - K)), K_s = fp32(m_s * scale) exactly as the
// streaming kernel formed its offset, K = fp32(M * scale).
__device__ __forceinline__ double combine_lz(const float* m, const float* S, int64_t rec0,
                                             int64_t n_slices, float M, float scale, int lane) {
  const float K = M * scale;
  double acc = 0.0;
  for (int64_t s = lane; s < n_slices; s += 64) {
    const float Ks = m[rec0 + s] * scale;
    acc += static_cast<double>(S[rec0 + s]) * exp2(static_cast<double>(Ks) - static_cast<double>(K));
  }
  return static_cast<double>(K) + log2(wave_sum_d(acc));
}

__device__ __forceinline__ float combine_max(const float* m, int64_t rec0, int64_t n_slices,
                                             int lane) {
  float v = -INFINITY;
  for (int64_t s = lane; s < n_slices; s += 64) v = fmaxf(v, m[rec0 + s]);
  return wave_max_f(v);
}

// Clipped reverse-KL of one row pair from its slice records; re-reads the slices whose
// bound may reach delta.
template <int DT>
__device__ double clipped_rkl_row(const FinArgs& a, int64_t t, int64_t d, int64_t rec0, double LZp,
                                  double LZq, int lane) {
  const double c2 = LZp - LZq;
  const double c2pos = c2 > 0.0 ? c2 : 0.0;
  const double delta = static_cast<double>(a.delta);
  double acc = 0.0;
  const int64_t S = a.n_slices;
  for (int64_t base = 0; base < S; base += 64) {
    const int64_t s = base + lane;
    double contrib = 0.0;
    bool fail = false;
    if (s < S) {
      const double Ks = static_cast<double>(a.part.mq[rec0 + s] * kL2E);
      const double scale = kLn2 * exp2(Ks - LZq);
      const double bound = scale * (static_cast<double>(kL2E) * a.part.g[rec0 + s] + c2pos * 1.0001);
      fail = !(bound * 1.0001 < delta);
      contrib = scale * (static_cast<double>(kL2E) * a.part.w[rec0 + s] + c2 * a.part.sq[rec0 + s]);
    }
    uint64_t mask = __ballot(fail);
    while (mask) {
      const int owner = __builtin_ctzll(mask);
      mask &= mask - 1;
      const int64_t ss = base + owner;
      // direct sum over the slice's columns: min(delta, q_y ln(q_y / p_y))
      const float c2f = static_cast<float>(c2);
      const float deltaf = a.delta;
      float part = 0.0f;
      for (int c = 0; c < kGroups; ++c) {
        for (int e = 0; e < 8; ++e) {
          const int64_t col = ss * kSlice + c * 512 + lane * 8 + e;
          if (col < a.V) {
            const float lq = load_logit<DT>(a.draft, d * a.ld_d + col);
            const float lp = load_logit<DT>(a.target, t * a.ld_t + col);
            const float kq = static_cast<float>(static_cast<double>(lq) * kL2E - LZq);
            const float q = fast_exp2(kq);
            const float term = q * static_cast<float>(kLn2) * __builtin_fmaf(lq - lp, kL2E, c2f);
            part += fminf(term, deltaf);
          }
        }
      }
      const double direct = wave_sum_d(static_cast<double>(part));
      if (lane == owner) contrib = direct;
    }
    acc += contrib;
  }
  return wave_sum_d(acc);
}

template <int DT>
__global__ __launch_bounds__(256) void sv_finalize_kernel(FinArgs a) {
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int64_t unit = static_cast<int64_t>(blockIdx.x) * kFinWavesPerBlock + wave;
  if (unit >= a.n_units) return;
  const int64_t S = a.n_slices;
  const int64_t rec0 = unit * S;

  if (!a.desc) {  // clipped reverse-KL only: unit = draft row
    const int64_t d = unit;
    const int64_t t = a.p_row_index ? a.p_row_index[d] : d;
    if (t < 0 || t >= a.n_target_rows) {
      if (lane == 0) {
        a.rkl_out[d] = NAN;
        atomicOr(a.device_status, 2);
      }
      return;
    }
    const float Mp = combine_max(a.part.mp, rec0, S, lane);
    const float Mq = combine_max(a.part.mq, rec0, S, lane);
    const double LZp = combine_lz(a.part.mp, a.part.sp, rec0, S, Mp, kL2E, lane);
    const double LZq = combine_lz(a.part.mq, a.part.sq, rec0, S, Mq, kL2E, lane);
    const double R = clipped_rkl_row<DT>(a, t, d, rec0, LZp, LZq, lane);
    if (lane == 0) a.rkl_out[d] = static_cast<float>(R);
    return;
  }

  // verification: unit = target row
  const int64_t t = unit;
  if (a.glob[0]) {  // void call: every per-draft output is NaN
    if (lane == 0 && t < a.n_d) {
      if (a.rkl_out) a.rkl_out[t] = NAN;
      if (a.p_at) a.p_at[t] = NAN;
      if (a.q_at) a.q_at[t] = NAN;
    }
    return;
  }
  const RowDesc rd = a.desc[t];
  const int64_t d = rd.d;
  const int mode = rd.mode;
  const float beta = rd.beta;

  const float Mp = combine_max(a.part.mp, rec0, S, lane);
  const double LZ1p = combine_lz(a.part.mp, a.part.sp, rec0, S, Mp, kL2E, lane);
  const double LZTp = (mode == 2) ? combine_lz(a.part.mp, a.part.stp, rec0, S, Mp, beta, lane) : LZ1p;
  int argp = 0;
  if (mode == 1) {
    int best = 0x7fffffff;
    for (int64_t s = lane; s < S; s += 64)
      if (a.part.mp[rec0 + s] == Mp) best = min(best, a.part.ap[rec0 + s]);
    argp = wave_min_int(best);
  }
  if (lane == 0) {
    const float KT = Mp * beta;
    a.t_off[t] = -KT;
    a.t_lz[t] = static_cast<float>(LZTp - static_cast<double>(KT));
    a.t_arg[t] = argp;
  }
  if (d < 0) return;  // bonus row

  const float Mq = combine_max(a.part.mq, rec0, S, lane);
  const double LZ1q = combine_lz(a.part.mq, a.part.sq, rec0, S, Mq, kL2E, lane);
  const double LZTq = (mode == 2) ? combine_lz(a.part.mq, a.part.stq, rec0, S, Mq, beta, lane) : LZ1q;
  if (lane == 0) {
    const float KT = Mq * beta;
    a.d_off[d] = -KT;
    a.d_lz[d] = static_cast<float>(LZTq - static_cast<double>(KT));
  }
  if (a.rkl_out) {
    const double R = clipped_rkl_row<DT>(a, t, d, rec0, LZ1p, LZ1q, lane);
    if (lane == 0) a.rkl_out[d] = static_cast<float>(R);
  }
  if (lane == 0) {
    const int flags = a.req_flags[rd.b];
    int accept = 0;
    float pa = NAN, qa = NAN;
    if (!(flags & kReqInvalid)) {
      const int32_t x = a.tokens[d];
      const double lpx = load_logit<DT>(a.target, t * a.ld_t + x);
      const double lqx = load_logit<DT>(a.draft, d * a.ld_d + x);
      const double sc = (mode == 2) ? static_cast<double>(beta) : static_cast<double>(kL2E);
      const double Lp = lpx * sc - LZTp;  // log2 p_T(x)
      const double Lq = lqx * sc - LZTq;  // log2 q_T(x)
      if (mode == 1) {
        accept = (x == argp) ? 1 : 0;
      } else {
        const double ratio = fmin(1.0, exp2(Lp - Lq));
        accept = (static_cast<double>(a.uniforms[t]) < ratio) ? 1 : 0;
      }
      pa = static_cast<float>(exp2(Lp));
      qa = static_cast<float>(exp2(Lq));
    }
    a.acc[d] = accept;
    if (a.p_at) a.p_at[d] = pa;
    if (a.q_at) a.q_at[d] = qa;
  }
}

// =========================================================================== sample
// Masses of the thread's 8 columns of chunk c: r (residual or p_T) and p_T.
template <int DT, bool VEC>
__device__ __forceinline__ void chunk_masses(const SampleArgs& a, int64_t t, int64_t d, bool pair,
                                             float beta, float offp, float lzp, float offq,
                                             float lzq, int64_t c, int tid, float (&r)[8],
                                             float (&pm)[8]) {
  const int64_t col = c * kChunk + tid * 8;
  float lp[8], lq[8];
  if constexpr (DT == 0) {
    const uint16_t* P = static_cast<const uint16_t*>(a.target) + t * a.ld_t;
    const uint16_t* Q = static_cast<const uint16_t*>(a.draft) + d * a.ld_d;
    if (VEC && col + 8 <= a.V) {
      const uint4 w = *reinterpret_cast<const uint4*>(P + col);
      lp[0] = bf16_lo(w.x); lp[1] = bf16_hi(w.x); lp[2] = bf16_lo(w.y); lp[3] = bf16_hi(w.y);
      lp[4] = bf16_lo(w.z); lp[5] = bf16_hi(w.z); lp[6] = bf16_lo(w.w); lp[7] = bf16_hi(w.w);
      if (pair) {
        const uint4 v = *reinterpret_cast<const uint4*>(Q + col);
        lq[0] = bf16_lo(v.x); lq[1] = bf16_hi(v.x); lq[2] = bf16_lo(v.y); lq[3] = bf16_hi(v.y);
        lq[4] = bf16_lo(v.z); lq[5] = bf16_hi(v.z); lq[6] = bf16_lo(v.w); lq[7] = bf16_hi(v.w);
      }
    } else {
      for (int e = 0; e < 8; ++e) {
        const bool ok = col + e < a.V;
        lp[e] = ok ? bf16_at(P + col + e) : -INFINITY;
        lq[e] = (ok && pair) ? bf16_at(Q + col + e) : -INFINITY;
      }
    }
  } else {
    const float* P = static_cast<const float*>(a.target) + t * a.ld_t;
    const float* Q = static_cast<const float*>(a.draft) + d * a.ld_d;
    for (int e = 0; e < 8; ++e) {
      const bool ok = col + e < a.V;
      lp[e] = ok ? P[col + e] : -INFINITY;
      lq[e] = (ok && pair) ? Q[col + e] : -INFINITY;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const float p = fast_exp2(__builtin_fmaf(lp[e], beta, offp) - lzp);
    pm[e] = p;
    if (pair) {
      const float q = fast_exp2(__builtin_fmaf(lq[e], beta, offq) - lzq);
      r[e] = fmaxf(p - q, 0.0f);
    } else {
      r[e] = p;
    }
  }
}

// The first rejected position of request b (k_b if none); read by thread 0.
__device__ __forceinline__ int accept_length(const SampleArgs& a, int64_t b, int kb, int64_t off) {
  int al = kb;
  for (int i = 0; i < kb; ++i)
    if (!a.acc[off - b + i]) {
      al = i;
      break;
    }
  return al;
}

// Chunk masses of the row the request draws its final token from.  Grid (request,
// chunk); greedy, invalid and void requests have nothing to draw.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void sv_sample_chunks_kernel(SampleArgs a) {
  const int64_t b = blockIdx.x;
  const int64_t c = blockIdx.y;
  const int tid = threadIdx.x;
  __shared__ double s_scan[4];
  __shared__ int s_alen;
  if (a.glob[0]) return;
  const int kb = a.k[b];
  const int64_t off = a.off_t[b];
  if (a.req_flags[b] & kReqInvalid) return;
  const RowDesc rd = a.desc[off];
  if (rd.mode == 1) return;
  if (tid == 0) s_alen = accept_length(a, b, kb, off);
  __syncthreads();
  const int alen = s_alen;
  const int64_t t = off + alen;
  const bool pair = alen < kb;
  const int64_t d = off - b + alen;
  const float offq = pair ? a.d_off[d] : 0.0f, lzq = pair ? a.d_lz[d] : 0.0f;
  float r[8], pm[8];
  chunk_masses<DT, VEC>(a, t, d, pair, rd.beta, a.t_off[t], a.t_lz[t], offq, lzq, c, tid, r, pm);
  double rs = 0.0, ps = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    rs += static_cast<double>(r[e]);
    ps += static_cast<double>(pm[e]);
  }
  const double r_incl = block_inclusive_scan_256(rs, s_scan);
  const double p_incl = block_inclusive_scan_256(ps, s_scan);
  if (tid == kSampleThreads - 1) {
    a.chunk_r[b * a.n_chunks + c] = r_incl;
    a.chunk_p[b * a.n_chunks + c] = p_incl;
  }
}

// One workgroup per request: first-rejection scan, inverse CDF over the chunk masses,
// then over the 2048 columns of the chosen chunk; writes accept_len and out_tokens.
template <int DT, bool VEC>
__global__ __launch_bounds__(256) void sv_sample_finish_kernel(SampleArgs a) {
  const int64_t b = blockIdx.x;
  const int tid = threadIdx.x;
  __shared__ double s_scan[4];
  __shared__ double s_incl[kSampleThreads];
  __shared__ int s_alen, s_cstar, s_usep, s_tok, s_fallback, s_lastpos;
  __shared__ double s_thr;

  if (a.glob[0]) {  // void call
    if (tid == 0) a.accept_len[b] = -1;
    for (int64_t t = b + static_cast<int64_t>(tid) * a.B; t < a.n_t;
         t += static_cast<int64_t>(kSampleThreads) * a.B)
      a.out_tokens[t] = -1;
    return;
  }
  const int kb = a.k[b];
  const int64_t off = a.off_t[b];
  if (a.req_flags[b] & kReqInvalid) {
    if (tid == 0) a.accept_len[b] = -1;
    for (int j = tid; j <= kb; j += kSampleThreads) a.out_tokens[off + j] = -1;
    return;
  }
  if (tid == 0) s_alen = accept_length(a, b, kb, off);
  __syncthreads();
  const int alen = s_alen;
  const RowDesc rd = a.desc[off];
  const int64_t t = off + alen;
  const bool pair = alen < kb;
  const int64_t d = off - b + alen;

  auto emit = [&](int tok) {
    if (tid == 0) a.accept_len[b] = alen;
    for (int j = tid; j <= kb; j += kSampleThreads)
      a.out_tokens[off + j] = (j < alen) ? a.tokens[off - b + j] : (j == alen ? tok : -1);
  };

  if (rd.mode == 1) {  // greedy: the target argmax at the first mismatch (or the bonus row)
    emit(a.t_arg[t]);
    return;
  }

  if (tid == 0) {
    const double* cr = a.chunk_r + b * a.n_chunks;
    const double* cp = a.chunk_p + b * a.n_chunks;
    double Z = 0.0;
    for (int64_t cc = 0; cc < a.n_chunks; ++cc) Z += cr[cc];
    int usep = 0;
    if (!(Z > 0.0)) {  // zero residual mass (rounding only): draw from p_T of the same row
      usep = 1;
      Z = 0.0;
      for (int64_t cc = 0; cc < a.n_chunks; ++cc) Z += cp[cc];
    }
    const double* cm = usep ? cp : cr;
    const double thr = static_cast<double>(a.uniforms[off + kb]) * Z;
    double cum = 0.0, before = 0.0;
    int cstar = -1, fallback = 0;
    for (int64_t cc = 0; cc < a.n_chunks; ++cc) {
      const double nxt = cum + cm[cc];
      if (nxt > thr) {
        cstar = static_cast<int>(cc);
        before = cum;
        break;
      }
      cum = nxt;
    }
    if (cstar < 0) {  // rounding left u * Z at or past the end: last chunk with mass
      fallback = 1;
      for (int64_t cc = a.n_chunks - 1; cc >= 0; --cc)
        if (cm[cc] > 0.0) {
          cstar = static_cast<int>(cc);
          break;
        }
      if (cstar < 0) cstar = 0;
    }
    s_cstar = cstar;
    s_usep = usep;
    s_thr = thr - before;
    s_fallback = fallback;
    s_tok = 0x7fffffff;
    s_lastpos = -1;
  }
  __syncthreads();
  const int cstar = s_cstar;
  const bool usep = s_usep != 0;
  const float offq = pair ? a.d_off[d] : 0.0f, lzq = pair ? a.d_lz[d] : 0.0f;
  float r[8], pm[8];
  chunk_masses<DT, VEC>(a, t, d, pair, rd.beta, a.t_off[t], a.t_lz[t], offq, lzq, cstar, tid, r,
                        pm);
  double mine[8];
  double tsum = 0.0;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    mine[e] = static_cast<double>(usep ? pm[e] : r[e]);
    tsum += mine[e];
  }
  const double incl = block_inclusive_scan_256(tsum, s_scan);
  s_incl[tid] = incl;
  __syncthreads();
  const double excl = tid ? s_incl[tid - 1] : 0.0;
  const double thr = s_thr;
  const int64_t col0 = static_cast<int64_t>(cstar) * kChunk + tid * 8;
  if (!s_fallback && excl <= thr && incl > thr) {
    double cum = excl;
    int found = -1;
    for (int e = 0; e < 8; ++e) {
      cum += mine[e];
      if (cum > thr && mine[e] > 0.0) {
        found = e;
        break;
      }
    }
    if (found < 0)  // rounding inside the thread: its last id with mass
      for (int e = 7; e >= 0; --e)
        if (mine[e] > 0.0) {
          found = e;
          break;
        }
    if (found >= 0) atomicMin(&s_tok, static_cast<int>(col0 + found));
  }
  int last = -1;
  for (int e = 7; e >= 0; --e)
    if (mine[e] > 0.0) {
      last = static_cast<int>(col0 + e);
      break;
    }
  if (last >= 0) atomicMax(&s_lastpos, last);
  __syncthreads();
  // no thread claimed u * Z (rounding): the chunk's last id with positive mass
  const int tok = (s_tok != 0x7fffffff) ? s_tok : (s_lastpos < 0 ? 0 : s_lastpos);
  emit(tok);
}

// =========================================================================== launchers
hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(sv_plan_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_finalize(int dtype, const FinArgs& a, hipStream_t st) {
  const int64_t blocks = (a.n_units + kFinWavesPerBlock - 1) / kFinWavesPerBlock;
  if (blocks == 0) return hipSuccess;
  if (dtype == 0)
    hipLaunchKernelGGL(sv_finalize_kernel<0>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(sv_finalize_kernel<1>, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_sample_chunks(int dtype, bool vec, const SampleArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B), static_cast<unsigned>(a.n_chunks));
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_sample_chunks_kernel<0, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((sv_sample_chunks_kernel<0, false>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((sv_sample_chunks_kernel<1, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_sample_finish(int dtype, bool vec, const SampleArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B));
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_sample_finish_kernel<0, true>), grid, dim3(256), 0, st, a);
    else hipLaunchKernelGGL((sv_sample_finish_kernel<0, false>), grid, dim3(256), 0, st, a);
  } else {
    hipLaunchKernelGGL((sv_sample_finish_kernel<1, false>), grid, dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
