// HIP kernels around the streaming pass (gfx950 / MI355X).
//
// A verification call runs, on the caller's stream:
//   sv_plan            (batches above kInlinePlanMaxB requests only) one workgroup:
//                      packed-layout offsets from k (AdaFlash paper, Section 3.3: one
//                      batch of total length sum k_b) and the request of every row.
//   sv_rowpair         the streaming pass fused with each row's finalize (sv_rowpair.hip).
//   sv_draw            the draw masses, per kChunk-column chunk, of each request's draw
//                      row: the residual max(0, p_T - q_T) at the first rejected position
//                      (reading notes, basic recipe step 4) or p_T of the bonus row (DFlash
//                      notes, Section 3.1 step 6); a request's row is spread over several
//                      workgroups so the whole chip takes part, and the last of them to
//                      finish scans the masses, takes the inverse CDF at u * Z and emits
//                      the tokens; it folds the request's input checks into device_status.
// sv_clipped_rkl runs sv_rowpair alone and then sv_status.
#include <float.h>
#include <math.h>
#include <stddef.h>

#include "sv_device.h"
#include "sv_lanes.h"
#include "sv_layout.h"
#include "sv_launch.h"

namespace sv {

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
  __shared__ int s_bad_len;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad_len = 0;
  __syncthreads();
  Workspace& ws = a.ws;
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
    if (b < a.B) {
      ws.off_t[b] = carry + excl;
      ws.arrive[b] = 0;  // the draw kernel counts its workgroups from zero
    }
    carry += total;
  }
  __syncthreads();
  const bool bad_len = s_bad_len != 0;
  const bool mismatch = !bad_len && (static_cast<int64_t>(carry) != a.n_d + a.B);
  if (tid == 0) {
    ws.off_t[a.B] = carry;
    ws.glob[0] = (bad_len || mismatch) ? 1 : 0;
    *a.device_status = (bad_len ? 1 : 0) | (mismatch ? 2 : 0);
  }
  if (bad_len || mismatch) return;
  for (int64_t b = tid; b < a.B; b += 1024) {  // draft-row units first, bonus units last
    const int off = ws.off_t[b];
    const int kb = a.k[b];
    for (int i = 0; i < kb; ++i) ws.desc[off - b + i] = RowDesc{off + i, static_cast<int32_t>(b)};
    ws.desc[a.n_d + b] = RowDesc{off + kb, static_cast<int32_t>(b)};
  }
}

// =========================================================================== OPD loss
// Per request: l_OPD = alpha mean_i(-ln q(x*_i)) + (1 - alpha) mean_i R_i over its k_b
// packed draft rows (AdaFlash paper, Section 3.1).  One workgroup: fixed-order exclusive
// scan of k for the row offsets, then each thread sums its requests' rows in row order in
// fp64.  Bad lengths or sum k_b != n_rows give NaN and SV_DEV_* bits; *device_status is
// written once, with the rows' own flags (row_flags) folded in.
// With coef, also each row's gradient coefficients (alpha / k_b, (1 - alpha) / k_b) (NaN
// for a void call).
__global__ __launch_bounds__(1024) void sv_opd_reduce_kernel(const int32_t* k, int64_t B,
                                                             int64_t n_rows, const float* rkl,
                                                             const float* hard, float alpha,
                                                             const int32_t* row_flags,
                                                             float* opd_out, float* coef,
                                                             int32_t* device_status) {
  __shared__ int s_waves[16];
  __shared__ int s_bad, s_rows;
  const int tid = threadIdx.x;
  if (tid == 0) s_bad = s_rows = 0;
  __syncthreads();
  int rf = 0;
  for (int64_t i = tid; i < n_rows; i += 1024) rf |= row_flags[i];
  if (rf) atomicOr(&s_rows, rf);
  int carry = 0;
  for (int64_t base = 0; base < B; base += 1024) {  // validate and total first
    const int64_t b = base + tid;
    int kb = 0;
    if (b < B) {
      kb = k[b];
      if (kb < 1 || kb > 64) {
        atomicOr(&s_bad, 1);
        kb = 0;
      }
    }
    int total = 0;
    block_excl_scan_1024(kb, s_waves, &total);
    carry += total;
  }
  __syncthreads();
  const int bad = s_bad ? 1 : (static_cast<int64_t>(carry) != n_rows ? 2 : 0);
  if (tid == 0) *device_status = bad | s_rows;
  carry = 0;
  for (int64_t base = 0; base < B; base += 1024) {
    const int64_t b = base + tid;
    const int kb = (b < B && !bad) ? k[b] : 0;
    int total = 0;
    const int off = carry + block_excl_scan_1024(kb, s_waves, &total);
    carry += total;
    if (b < B) {
      if (bad) {
        if (opd_out) opd_out[b] = NAN;
      } else {
        const double a = static_cast<double>(alpha);
        if (opd_out) {
          double sh = 0.0, sr = 0.0;
          for (int i = 0; i < kb; ++i) {
            sh += static_cast<double>(hard[off + i]);
            sr += static_cast<double>(rkl[off + i]);
          }
          opd_out[b] = static_cast<float>((a * sh + (1.0 - a) * sr) / static_cast<double>(kb));
        }
        if (coef) {
          const float ch = static_cast<float>(a / kb), cr = static_cast<float>((1.0 - a) / kb);
          for (int i = 0; i < kb; ++i) {
            coef[2 * (off + i)] = ch;
            coef[2 * (off + i) + 1] = cr;
          }
        }
      }
    }
  }
  if (bad && coef)
    for (int64_t i = tid; i < 2 * n_rows; i += 1024) coef[i] = NAN;
}

// =========================================================================== OPD gradient
// d l_OPD,b / d a_z for every draft row r of request b, a its drafter logits (temperature 1):
//   c_h (q_z - 1[z = x*]) + c_r q_z (g_z - S_g),   g_z = 1[t_z < delta] (L_z + 1),
// with L_z = ln q_z - ln p_z, t_z = q_z L_z, c_h = alpha / k_b, c_r = (1 - alpha) / k_b, and
// S_g = sum_y q_y g_y from the forward pass (the clip passes no gradient where it is active;
// on t = delta exactly the clipped side is taken).  One 256-thread workgroup per row, each
// thread 8 consecutive columns per step; the row is read once more and the gradient row
// written once.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);  // NaN
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte loads that bypass cache retention (every logit is read once); the gradient goes out
// with plain stores (measured faster than nontemporal ones).
__device__ __forceinline__ uint4 nt_load(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  uint4 r;
  __builtin_memcpy(&r, &v, 16);
  return r;
}
__device__ __forceinline__ void nt_store(void* p, const uint4& w) { *reinterpret_cast<uint4*>(p) = w; }

template <int DT>
__device__ __forceinline__ void load8(const void* row, int64_t col, int V, bool vec, float (&x)[8]) {
  if constexpr (DT == 0) {
    const uint16_t* p = static_cast<const uint16_t*>(row) + col;
    if (vec && col + 8 <= V) {
      unpack8(nt_load(p), x);
    } else {
      for (int e = 0; e < 8; ++e) x[e] = (col + e < V) ? bf16_at(p + e) : 0.0f;
    }
  } else {
    const float* p = static_cast<const float*>(row) + col;
    if (vec && col + 8 <= V) {
      const uint4 a = nt_load(p), b = nt_load(p + 4);
      x[0] = __uint_as_float(a.x); x[1] = __uint_as_float(a.y);
      x[2] = __uint_as_float(a.z); x[3] = __uint_as_float(a.w);
      x[4] = __uint_as_float(b.x); x[5] = __uint_as_float(b.y);
      x[6] = __uint_as_float(b.z); x[7] = __uint_as_float(b.w);
    } else {
      for (int e = 0; e < 8; ++e) x[e] = (col + e < V) ? p[e] : 0.0f;
    }
  }
}

template <int DT, int GT, bool VEC>
__global__ __launch_bounds__(256) void sv_opd_grad_kernel(GradArgs a) {
  const int64_t r = blockIdx.x;
  const int tid = threadIdx.x;
  const int64_t t = a.p_row_index ? a.p_row_index[r] : r;
  const int V = a.V;
  const bool ok = t >= 0 && t < a.n_target_rows;  // a void call has NaN coefficients
  const RowStats st = a.stats[r];
  const float ch = a.coef[2 * r], cr = a.coef[2 * r + 1];
  const double Kq = rint(st.lzq);
  const float kq = static_cast<float>(-Kq), fq = static_cast<float>(st.lzq - Kq);
  const float c2 = static_cast<float>(st.lzp - st.lzq);
  const float sg = static_cast<float>(st.sg);
  const int x = st.top1;
  const float ln2 = static_cast<float>(kLn2);
  const size_t es = DT == 0 ? 2 : 4;
  const void* prow = static_cast<const char*>(a.target) + (ok ? t : 0) * a.ld_t * es;
  const void* qrow = static_cast<const char*>(a.draft) + r * a.ld_d * es;
  char* grow = static_cast<char*>(a.grad) + r * a.ld_g * (GT == 0 ? 2 : 4);
  auto grad8 = [&](int64_t col, const float (&lp)[8], const float (&lq)[8]) {
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float q = fast_exp2(__builtin_fmaf(lq[e], kL2E, kq) - fq);
      const float L = ln2 * __builtin_fmaf(lq[e] - lp[e], kL2E, c2);
      const float gz = (q * L < a.delta) ? L + 1.0f : 0.0f;
      const float onehot = (col + e == x) ? 1.0f : 0.0f;
      g[e] = ok ? __builtin_fmaf(cr * q, gz - sg, ch * (q - onehot)) : NAN;
    }
    if constexpr (GT == 0) {
      uint16_t* o = reinterpret_cast<uint16_t*>(grow) + col;
      if (VEC && col + 8 <= V) {
        uint4 w;
        w.x = bf16_rne(g[0]) | (static_cast<uint32_t>(bf16_rne(g[1])) << 16);
        w.y = bf16_rne(g[2]) | (static_cast<uint32_t>(bf16_rne(g[3])) << 16);
        w.z = bf16_rne(g[4]) | (static_cast<uint32_t>(bf16_rne(g[5])) << 16);
        w.w = bf16_rne(g[6]) | (static_cast<uint32_t>(bf16_rne(g[7])) << 16);
        nt_store(o, w);
      } else {
        for (int e = 0; e < 8; ++e)
          if (col + e < V) o[e] = bf16_rne(g[e]);
      }
    } else {
      float* o = reinterpret_cast<float*>(grow) + col;
      if (VEC && col + 8 <= V) {
        nt_store(o, make_uint4(__float_as_uint(g[0]), __float_as_uint(g[1]),
                               __float_as_uint(g[2]), __float_as_uint(g[3])));
        nt_store(o + 4, make_uint4(__float_as_uint(g[4]), __float_as_uint(g[5]),
                                   __float_as_uint(g[6]), __float_as_uint(g[7])));
      } else {
        for (int e = 0; e < 8; ++e)
          if (col + e < V) o[e] = g[e];
      }
    }
  };
  constexpr int64_t kStep = 256 * 8;
  int64_t col = static_cast<int64_t>(tid) * 8;
  for (; col < V; col += kStep) {
    float lp0[8], lq0[8];
    load8<DT>(prow, col, V, VEC, lp0);
    load8<DT>(qrow, col, V, VEC, lq0);
    grad8(col, lp0, lq0);
  }
}

// =========================================================================== status
// OR of the per-row flags of a clipped-reverse-KL call into *device_status.
__global__ __launch_bounds__(256) void sv_status_kernel(const int32_t* row_flags, int64_t n,
                                                        int32_t* device_status) {
  __shared__ int s;
  if (threadIdx.x == 0) s = 0;
  __syncthreads();
  int f = 0;
  for (int64_t i = threadIdx.x; i < n; i += 256) f |= row_flags[i];
  if (f) atomicOr(&s, f);
  __syncthreads();
  if (threadIdx.x == 0) *device_status = s;
}

// =========================================================================== sample
constexpr int kReqInvalid = 4 | 8 | 16;  // SV_DEV_BAD_TOKEN | BAD_TEMPERATURE | BAD_UNIFORM
// s_waitcnt operand that waits for every outstanding vector memory operation of the wave
// (vmcnt = 0) and leaves the export and LDS/scalar counters at their maxima (gfx9 encoding).
constexpr int kWaitVmcnt0 = 0x0F70;

// Draw masses of the lane's 8 columns starting at col: the residual max(0, p_T - q_T) of
// a row pair (need_q), else p_T.  p_T(y) = 2^(fma(l_p(y), beta, offp) - lzp): the
// fma is exact before its one rounding and lzp is small, so p_T keeps fp32 accuracy.
struct RowScale {
  float beta, offp, lzp, offq, lzq;
};

__device__ __forceinline__ float draw_mass(float lp, float lq, bool need_q, const RowScale& k) {
  const float p = fast_exp2(__builtin_fmaf(lp, k.beta, k.offp) - k.lzp);
  return need_q ? fmaxf(p - fast_exp2(__builtin_fmaf(lq, k.beta, k.offq) - k.lzq), 0.0f) : p;
}


template <int DT, bool VEC>
__device__ __forceinline__ void column_masses(const SampleArgs& a, int64_t t, int64_t d,
                                              bool need_q, const RowScale& k, int64_t col,
                                              float (&r)[8]) {
  float lp[8], lq[8];
  if constexpr (DT == 0) {
    const uint16_t* P = static_cast<const uint16_t*>(a.target) + t * a.ld_t;
    const uint16_t* Q = static_cast<const uint16_t*>(a.draft) + d * a.ld_d;
    if (VEC && col + 8 <= a.V) {
      const uint4 w = *reinterpret_cast<const uint4*>(P + col);
      lp[0] = bf16_lo(w.x); lp[1] = bf16_hi(w.x); lp[2] = bf16_lo(w.y); lp[3] = bf16_hi(w.y);
      lp[4] = bf16_lo(w.z); lp[5] = bf16_hi(w.z); lp[6] = bf16_lo(w.w); lp[7] = bf16_hi(w.w);
      if (need_q) {
        const uint4 v = *reinterpret_cast<const uint4*>(Q + col);
        lq[0] = bf16_lo(v.x); lq[1] = bf16_hi(v.x); lq[2] = bf16_lo(v.y); lq[3] = bf16_hi(v.y);
        lq[4] = bf16_lo(v.z); lq[5] = bf16_hi(v.z); lq[6] = bf16_lo(v.w); lq[7] = bf16_hi(v.w);
      }
    } else {
      for (int e = 0; e < 8; ++e) {
        const bool ok = col + e < a.V;
        lp[e] = ok ? bf16_at(P + col + e) : -INFINITY;
        lq[e] = (ok && need_q) ? bf16_at(Q + col + e) : -INFINITY;
      }
    }
  } else {
    const float* P = static_cast<const float*>(a.target) + t * a.ld_t;
    const float* Q = static_cast<const float*>(a.draft) + d * a.ld_d;
    for (int e = 0; e < 8; ++e) {
      const bool ok = col + e < a.V;
      lp[e] = ok ? P[col + e] : -INFINITY;
      lq[e] = (ok && need_q) ? Q[col + e] : -INFINITY;
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = draw_mass(lp[e], lq[e], need_q, k);
}

// A request's state: whether the call is void, T_b, length, first target row, input
// flags (OR over its k_b + 1 rows), the first rejected position a_b, and what the draw needs
// of row a_b (its exp2 offsets, its argmax).  Gathered by one wave in one round of loads: the
// call flag, T_b, k_b, the first target row, and lane i's slot of position i (the slots sit
// at a fixed stride per request, so they need nothing from the other loads); the values of
// row a_b are taken from lane a_b by a shuffle.  Lane i's draft token (into *tok) and uniform
// (into *u) are fetched after that round and used only by the pick and the emit.
struct ReqState {
  int void_call, kb, flags, alen, targ;
  float T;
  int64_t off;
  RowScale k;
};

__device__ __forceinline__ ReqState wave_request_state(const SampleArgs& a, int64_t b, int* tok,
                                                       float* u) {
  const int lane = threadIdx.x & 63;
  ReqState r;
  r.k.beta = r.k.offp = r.k.lzp = r.k.offq = r.k.lzq = 0.f;
  r.targ = 0;
  r.void_call = a.glob[0];
  r.T = a.force_greedy ? 0.0f : (a.temperature ? a.temperature[b] : 1.0f);
  r.kb = a.k[b];
  r.off = a.off_t[b];
  RowOut ro{};
  if (lane < a.kmax1) ro = a.rowout[b * a.kmax1 + lane];
  int f = 0, targ = 0;
  bool rej = false;
  float beta = 0.f, offp = 0.f, lzp = 0.f, offq = 0.f, lzq = 0.f;
  *tok = -1;
  *u = 0.f;
  if (!r.void_call) {
    if (lane <= r.kb) {
      f = ro.flags;
      beta = ro.beta;
      offp = ro.offp;
      lzp = ro.lzp;
      targ = ro.targ;
      if (a.uniforms) *u = a.uniforms[r.off + lane];
    }
    if (lane < r.kb) {
      rej = !ro.acc;
      offq = ro.offq;
      lzq = ro.lzq;
      *tok = a.tokens[r.off - b + lane];
    }
    if (r.kb >= 64 && lane == 0) f |= a.rowout[b * a.kmax1 + 64].flags;  // k_b = 64: row 64
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) f |= __shfl_xor(f, m, 64);
  r.flags = f;
  const uint64_t mask = __ballot(rej);
  r.alen = mask ? __builtin_ctzll(mask) : r.kb;
  if (r.alen < 64) {
    r.k.beta = __shfl(beta, r.alen, 64);
    r.k.offp = __shfl(offp, r.alen, 64);
    r.k.lzp = __shfl(lzp, r.alen, 64);
    r.k.offq = __shfl(offq, r.alen, 64);
    r.k.lzq = __shfl(lzq, r.alen, 64);
    r.targ = __shfl(targ, r.alen, 64);
  } else if (!r.void_call) {  // k_b = 64 and every draft accepted: the bonus row is row 64
    const RowOut rb = a.rowout[b * a.kmax1 + 64];
    r.k.beta = rb.beta;
    r.k.offp = rb.offp;
    r.k.lzp = rb.lzp;
    r.k.offq = r.k.lzq = 0.f;
    r.targ = rb.targ;
  }
  return r;
}

// The request's final uniform (slot k_b), from the lanes' uniforms.
__device__ __forceinline__ float final_uniform(const SampleArgs& a, const ReqState& r, float u) {
  if (r.kb < 64) return __shfl(u, r.kb < 0 ? 0 : r.kb, 64);
  return a.uniforms ? a.uniforms[r.off + 64] : 0.f;
}


// Draw masses of chunks [c_begin, c_end) of one row into out[c]; wave w of WAVES takes
// chunks c_begin + w, + WAVES, ...  Each lane sums its kChunkGroups groups of 8 columns
// (groups 512 columns apart) in fp32; the lane sums are combined in fp64.  For aligned
// bf16 rows the loads of BATCH chunks are issued before any arithmetic.
// DEVICE_OUT: out is global memory read by another workgroup of the same launch; each mass
// is then written with a device-scope store (written through to the device's coherence
// point, past this XCD's L2), see sv_draw.
template <bool DEVICE_OUT>
__device__ __forceinline__ void put_mass(double* out, int c, double v) {
  if constexpr (DEVICE_OUT) __hip_atomic_store(out + c, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else out[c] = v;
}

template <int DT, bool VEC, int WAVES, int BATCH, bool NEED_Q, bool DEVICE_OUT>
__device__ __forceinline__ void chunk_masses_t(const SampleArgs& a, int64_t t, int64_t d,
                                               const RowScale& k, int c_begin, int c_end,
                                               int wave, int lane, double* out) {
  const int n_full = a.V / kChunk;  // chunks that lie wholly inside [0, V)
  int c0 = c_begin + wave;
  if constexpr (DT == 0 && VEC) {
    const uint16_t* P = static_cast<const uint16_t*>(a.target) + t * a.ld_t + lane * 8;
    const uint16_t* Q = static_cast<const uint16_t*>(a.draft) + d * a.ld_d + lane * 8;
    constexpr int NL = BATCH * kChunkGroups;  // 16-byte loads per row per lane per batch
    // full batches: every chunk of the batch inside the range and inside [0, V)
    for (; c0 + (BATCH - 1) * WAVES < min(c_end, n_full); c0 += BATCH * WAVES) {
      uint4 wp[NL], wq[NL];
#pragma unroll
      for (int j = 0; j < NL; ++j) {
        const int64_t col =
            static_cast<int64_t>(c0 + (j / kChunkGroups) * WAVES) * kChunk + (j % kChunkGroups) * 512;
        wp[j] = *reinterpret_cast<const uint4*>(P + col);
        if constexpr (NEED_Q) wq[j] = *reinterpret_cast<const uint4*>(Q + col);
      }
#pragma unroll
      for (int h = 0; h < BATCH; ++h) {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < kChunkGroups; ++g) {
          float lp[8], lq[8];
          unpack8(wp[h * kChunkGroups + g], lp);
          if constexpr (NEED_Q) unpack8(wq[h * kChunkGroups + g], lq);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc += draw_mass(lp[e], NEED_Q ? lq[e] : 0.0f, NEED_Q, k);
        }
        const double cs = wave_sum_d(static_cast<double>(acc));
        if (lane == 0) put_mass<DEVICE_OUT>(out, c0 + h * WAVES, cs);
      }
    }
  }
  for (int c = c0; c < c_end; c += WAVES) {  // the rest, one chunk at a time, bounds-checked
    float acc = 0.0f;
    for (int g = 0; g < kChunkGroups; ++g) {
      float r[8];
      column_masses<DT, VEC>(a, t, d, NEED_Q, k,
                             static_cast<int64_t>(c) * kChunk + g * 512 + lane * 8, r);
      for (int e = 0; e < 8; ++e) acc += r[e];
    }
    const double cs = wave_sum_d(static_cast<double>(acc));
    if (lane == 0) put_mass<DEVICE_OUT>(out, c, cs);
  }
}

template <int DT, bool VEC, int WAVES, int BATCH, bool DEVICE_OUT>
__device__ __forceinline__ void chunk_masses(const SampleArgs& a, int64_t t, int64_t d, bool need_q,
                                             const RowScale& k, int c_begin, int c_end, int wave,
                                             int lane, double* out) {
  if (need_q)
    chunk_masses_t<DT, VEC, WAVES, BATCH, true, DEVICE_OUT>(a, t, d, k, c_begin, c_end, wave, lane, out);
  else
    chunk_masses_t<DT, VEC, WAVES, BATCH, false, DEVICE_OUT>(a, t, d, k, c_begin, c_end, wave, lane, out);
}

// The clipped reverse-KL of draft row d (target row t), which the streaming pass left
// provisional with a record of its heavy lanes (RklFix), finished by the draw launch: each heavy lane
// is summed again from the logits in fp64 (exp2 in fp64, against the lane's own offsets), the
// normalisers are formed with the new sums, and R moves to them.  With LZp, LZq the streaming
// pass's normalisers and LZp', LZq' the new ones, c2 = LZp - LZq, c2' = LZp' - LZq' and
// s = 2^-(LZq' - LZq), every term the pass kept, t_y = ln2 q_y (L2E (l_q - l_p)_y + c2) with
// q_y = 2^(l_q L2E - LZq), becomes s t_y + s ln2 (c2' - c2) q_y unless it was clipped at delta
// (the clip set is taken as the pass found it, its bound being 1e-4 away from delta).  Over
// the lanes other than the heavy closed-form ones that is
//   r_rest + (s - 1) u1 + s ln2 (c2' - c2) u0,
// u1 the sum of their unclipped terms and u0 their q-mass; each heavy closed-form lane adds
// ln2 2^(k_q - LZq') (L2E W + c2' S_q) with its new W and S_q.
// A row's record as one 32-bit word per lane (lanes past the record hold 0); a wave reads it
// with one vector load, early, and takes the fields out with readlane.  The load goes through a
// bounds-checked buffer over the records (empty without them) and is issued with no branch
// around it, so nothing waits for it before its first use; want = false reads 0.
__device__ __forceinline__ uint32_t load_fix_words(const SampleArgs& a, int64_t d, bool want,
                                                   int lane) {
  const int bytes = (a.rkl_out && a.fix)
                        ? static_cast<int>(a.B * (a.kmax1 - 1) * static_cast<int64_t>(sizeof(RklFix)))
                        : 0;
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<RklFix*>(a.fix), 0, bytes, kBufWord3);
  const int off = (want && lane < kFixDwords)
                      ? static_cast<int>(d * static_cast<int64_t>(sizeof(RklFix))) + lane * 4
                      : bytes;
  return __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0);
}
__device__ __forceinline__ int fix_word(uint32_t w, int i) { return __builtin_amdgcn_readlane(w, i); }
__device__ __forceinline__ double fix_double(uint32_t w, int i) {
  return __hiloint2double(fix_word(w, i + 1), fix_word(w, i));
}

// R of draft row d from its record (n heavy lanes) and the heavy lanes' new sums, sums(j) for
// heavy lane j; lane 0 of the wave stores it.
template <class Sums>
__device__ __forceinline__ void finish_rkl_from(const SampleArgs& a, int64_t d, uint32_t rec, int n,
                                                int lane, Sums&& sums) {
  const float Kp = __int_as_float(fix_word(rec, offsetof(RklFix, kp_ref) / 4));
  const float Kq = __int_as_float(fix_word(rec, offsetof(RklFix, kq_ref) / 4));
  double Sp = fix_double(rec, offsetof(RklFix, sp_rest) / 4);
  double Sq = fix_double(rec, offsetof(RklFix, sq_rest) / 4);
  double HW = 0.0, HS = 0.0;
  for (int j = 0; j < n; ++j) {
    const int h0 = offsetof(RklFix, h) / 4 + j * 4;
    const bool direct = fix_word(rec, h0 + 1) != 0;
    const float hkp = __int_as_float(fix_word(rec, h0 + 2));
    const float hkq = __int_as_float(fix_word(rec, h0 + 3));
    const LaneSums e = sums(j);
    const double sp = e.sp, sq = e.sq, w = e.w;
    if (sp > 0.0) Sp += ldexp(sp, static_cast<int>(hkp - Kp));
    if (sq > 0.0) {
      const int e = static_cast<int>(hkq - Kq);
      Sq += ldexp(sq, e);
      if (!direct) {
        HW += ldexp(w, e);
        HS += ldexp(sq, e);
      }
    }
  }
  const double LZp = static_cast<double>(Kp) + log2_d(Sp);
  const double LZq = static_cast<double>(Kq) + log2_d(Sq);
  const double dp = LZp - fix_double(rec, offsetof(RklFix, lzp) / 4);
  const double dq = LZq - fix_double(rec, offsetof(RklFix, lzq) / 4);
  const double s = exp2_d(-dq);
  const double R = fix_double(rec, offsetof(RklFix, r_rest) / 4) +
                   (s - 1.0) * fix_double(rec, offsetof(RklFix, u1) / 4) +
                   s * kLn2 * (dp - dq) * fix_double(rec, offsetof(RklFix, u0) / 4) +
                   kLn2 * exp2_d(static_cast<double>(Kq) - LZq) *
                       (static_cast<double>(kL2E) * HW + (LZp - LZq) * HS);
  if (lane == 0) a.rkl_out[d] = static_cast<float>(R);
}

template <int DT>
__device__ __forceinline__ const void* logits_row(const void* base, int64_t r, int64_t ld) {
  return static_cast<const char*>(base) + r * ld * (DT == 0 ? 2 : 4);
}

// Each draft row has a workgroup of its own, after the drawing ones, so that the rows start
// with the launch and the draw waits for none of them.  The heavy lanes' blocks (lane_blocks:
// four for the folded lanes of a split row whose parts were folded, four times as long, else
// one) are spread over the waves, item i = (lane i / blocks,
// block i % blocks) to wave i % 4; the blocks' sums meet in s_part, and wave 0 adds them up in
// block order, as one wave would.  The record (n = 0 for a row the stream finished, and for
// every row of a void call) names the row's target row.
template <int DT, bool VEC>
__device__ __forceinline__ void finish_rkl_row_own(const SampleArgs& a, int64_t d, int wave,
                                                   int lane, double* s_part) {
  static_assert(kMassWaves == kRowWaves && kFixLanes * kMassWaves * 3 <= kMaxChunks, "block sums fit s_part");
  const uint32_t rec = load_fix_words(a, d, true, lane);
  const int n = min(fix_word(rec, offsetof(RklFix, n) / 4), kFixLanes);
  if (n <= 0) return;
  const int64_t t = fix_word(rec, offsetof(RklFix, t_row) / 4);
  const void* prow = logits_row<DT>(a.target, t, a.ld_t);
  const void* qrow = logits_row<DT>(a.draft, d, a.ld_d);
  const int blocks = lane_blocks(fix_word(rec, offsetof(RklFix, h) / 4));  // the same for every lane of the row
  for (int it = wave; it < n * blocks; it += kMassWaves) {
    const int j = it / blocks, q = it - j * blocks;
    const int h0 = offsetof(RklFix, h) / 4 + j * 4;
    const LaneSums e = exact_lane_sums<DT, VEC>(
        prow, qrow, a.V, static_cast<int>(a.n_slices), fix_word(rec, h0), q, lane,
        static_cast<double>(__int_as_float(fix_word(rec, h0 + 2))),
        static_cast<double>(__int_as_float(fix_word(rec, h0 + 3))));
    if (lane == 0) {
      double* o = s_part + (j * kMassWaves + q) * 3;
      o[0] = e.sp;
      o[1] = e.sq;
      o[2] = e.w;
    }
  }
  __syncthreads();
  if (wave == 0) {
    finish_rkl_from(a, d, rec, n, lane, [&](int j) {
      LaneSums r{0.0, 0.0, 0.0};
      for (int q = 0; q < blocks; ++q) {
        const double* o = s_part + (j * kMassWaves + q) * 3;
        r.sp += o[0];
        r.sq += o[1];
        r.w += o[2];
      }
      return r;
    });
  }
}

// One request's part of sv_draw for workgroup g (see the kernel below); returns once the
// calling wave has nothing more to do for the draw.
template <int DT, bool VEC>
__device__ __forceinline__ void draw_request(const SampleArgs& a, int64_t b, int g, int tid, int lane,
                                             int wave, int my_tok, float my_u, const ReqState& rq,
                                             double* s_pm, int* s_ticket) {
  const int kb = rq.kb;
  const int64_t off = rq.off;
  if (rq.flags & kReqInvalid) {
    if (g == 0) {
      if (tid == 0) {
        a.accept_len[b] = -1;
        atomicOr(a.device_status, rq.flags & kReqInvalid);
      }
      for (int j = tid; j <= kb; j += kMassThreads) a.out_tokens[off + j] = -1;
      for (int j = tid; j < kb; j += kMassThreads) {
        if (a.p_at) a.p_at[off - b + j] = NAN;
        if (a.q_at) a.q_at[off - b + j] = NAN;
      }
    }
    return;
  }
  const int alen = rq.alen;
  // wave 0 writes the outputs: a_b drafts (held in its lanes), the final token, then -1
  auto emit = [&](int tok) {
    if (lane == 0) a.accept_len[b] = alen;
    for (int j = lane; j <= kb; j += 64)
      a.out_tokens[off + j] = (j < alen) ? my_tok : (j == alen ? tok : -1);
  };
  if (rq.T == 0.0f) {  // greedy: the target argmax at the first mismatch (or the bonus row)
    if (g == 0 && wave == 0) emit(rq.targ);
    return;
  }

  const int64_t t = off + alen;
  const bool pair = alen < kb;
  const int64_t d = off - b + alen;
  const int nc = static_cast<int>(a.n_chunks);
  double* cm = a.chunk_mass + b * a.n_chunks;
  {
    const int c_begin = g * kMassChunksPerBlock;
    const int c_end = min(nc, c_begin + kMassChunksPerBlock);
    chunk_masses<DT, VEC, kMassWaves, 2, true>(a, t, d, pair, rq.k, c_begin, c_end, wave, lane, cm);
  }
  // Hand-off to the picking workgroup without cache-wide maintenance: the masses went out
  // as device-scope stores (written through to the coherence point shared by every XCD);
  // each wave waits until its stores are complete, the barrier joins the waves, and only
  // then does thread 0 take a ticket with a device-scope atomic.  The workgroup holding the
  // last ticket reads the masses back with device-scope loads, which bypass its L2.
  // (An agent-scope fence here would write back and invalidate the XCD's whole L2 per wave.)
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  __syncthreads();
  if (tid == 0) *s_ticket = __hip_atomic_fetch_add(a.arrive + b, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*s_ticket != a.mass_blocks - 1) return;

  // ---- 1. chunk level (every wave computes the same total, so they agree on the fallback).
  // The masses are read back once; wave 0, which draws, keeps its lanes' masses in s_pm.
  const int cpl = (nc + 63) / 64;  // chunks per lane
  const int c_lo = min(nc, lane * cpl), c_hi = min(nc, c_lo + cpl);
  bool usep = false;
  double lsum = 0.0;
  for (int c = c_lo; c < c_hi; ++c) {
    const double m = __hip_atomic_load(cm + c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (wave == 0) s_pm[c] = m;
    lsum += m;
  }
  double Z = wave_sum_d(lsum);
  if (!(Z > 0.0)) {  // zero residual mass (rounding only): draw from p_T of the same row
    usep = true;
    __syncthreads();  // wave 0's copies are written before s_pm is refilled
    chunk_masses<DT, VEC, kMassWaves, 2, false>(a, t, d, false, rq.k, 0, nc, wave, lane, s_pm);
    __syncthreads();
    lsum = 0.0;
    for (int c = c_lo; c < c_hi; ++c) lsum += s_pm[c];
    Z = wave_sum_d(lsum);
  }
  if (wave != 0) return;  // one wave draws
  double incl = lsum;  // fixed-order inclusive scan of the lane sums
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const double o = __shfl_up(incl, dd, 64);
    if (lane >= dd) incl += o;
  }
  double excl = __shfl_up(incl, 1, 64);
  if (lane == 0) excl = 0.0;
  const double thr = static_cast<double>(final_uniform(a, rq, my_u)) * Z;
  // chunk c of the lane spans [s_c, s_{c+1}), s_{c_lo} = excl, s_{c+1} = s_c + m_c, and the
  // lane's last chunk ends at incl: the intervals tile [0, Z) exactly
  int sel = -1, last = -1;
  double sel_start = 0.0;
  double s_c = excl;
  for (int c = c_lo; c < c_hi; ++c) {
    const double m_c = s_pm[c];  // the residual's masses, or p_T's after the fallback
    const double e_c = (c == c_hi - 1) ? incl : s_c + m_c;
    if (m_c > 0.0) {
      last = c;
      if (sel < 0 && s_c <= thr && thr < e_c) {
        sel = c;
        sel_start = s_c;
      }
    }
    s_c = e_c;
  }
  const uint64_t hit_c = __ballot(sel >= 0);
  bool fallback = false;
  int cstar;
  double thr_c;
  if (hit_c) {
    const int src = __builtin_ctzll(hit_c);
    cstar = __shfl(sel, src, 64);
    thr_c = thr - __shfl(sel_start, src, 64);
  } else {  // rounding: the last chunk with mass
    fallback = true;
    const uint64_t has = __ballot(last >= 0);
    cstar = has ? __shfl(last, 63 - __builtin_clzll(has), 64) : 0;
    thr_c = 0.0;
  }

  // ---- 2. column level: lane l owns columns cstar * kChunk + 32 l .. + 32
  const int64_t colL = static_cast<int64_t>(cstar) * kChunk + lane * kChunkGroups * 8;
  const RowScale k = rq.k;
  float m[kChunkGroups * 8];
  double csum = 0.0;
#pragma unroll
  for (int gg = 0; gg < kChunkGroups; ++gg) {
    float r[8];
    column_masses<DT, VEC>(a, t, d, pair && !usep, k, colL + gg * 8, r);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      m[gg * 8 + e] = r[e];
      csum += static_cast<double>(r[e]);
    }
  }
  double cincl = csum;
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const double o = __shfl_up(cincl, dd, 64);
    if (lane >= dd) cincl += o;
  }
  double cexcl = __shfl_up(cincl, 1, 64);
  if (lane == 0) cexcl = 0.0;
  int found = -1;
  if (!fallback && cexcl <= thr_c && cincl > thr_c) {
    double cum = cexcl;
#pragma unroll
    for (int e = 0; e < kChunkGroups * 8; ++e) {
      cum += static_cast<double>(m[e]);
      if (found < 0 && cum > thr_c && m[e] > 0.0f) found = e;
    }
    if (found < 0)  // rounding inside the lane: its last id with mass
#pragma unroll
      for (int e = 0; e < kChunkGroups * 8; ++e)
        if (m[e] > 0.0f) found = e;
  }
  int lastc = -1;
#pragma unroll
  for (int e = 0; e < kChunkGroups * 8; ++e)
    if (m[e] > 0.0f) lastc = e;
  const uint64_t hit = __ballot(found >= 0);
  int tok;
  if (hit) {
    const int src = __builtin_ctzll(hit);
    tok = __shfl(static_cast<int>(colL) + found, src, 64);
  } else {  // no lane claimed u * Z (rounding): the chunk's last id with positive mass
    const uint64_t has = __ballot(lastc >= 0);
    const int src = has ? 63 - __builtin_clzll(has) : 0;
    tok = __shfl(static_cast<int>(colL) + (lastc < 0 ? 0 : lastc), src, 64);
  }
  emit(tok);
}

// sv_draw: workgroup g of request b computes the draw masses of chunks
// [g * kMassChunksPerBlock, (g + 1) * kMassChunksPerBlock) of the request's draw row into
// chunk_mass[b * n_chunks + c]; the last of the request's workgroups to finish (a ticket
// from its arrival counter, after a device-wide fence) then draws the token from them:
//   1. the chunk where the prefix of the masses first exceeds u * Z (u the request's last
//      uniform, Z the total): one wave, lane l owning a run of consecutive chunks, fp64
//      sums in chunk order and a fixed-order scan across the lanes;
//   2. the column inside that chunk: one wave, 32 consecutive columns per lane, the fp64
//      prefix again in column order; the row is read once more only there;
//   3. emit: a_b accepted drafts, the final token, -1 after.
// A residual whose masses sum to zero (rounding only) is redrawn from p_T of the same row,
// whose chunk masses the picking workgroup then computes itself.  Greedy requests (and
// every request of sv_verify_block_greedy) emit the target's argmax from workgroup 0; void
// calls and invalid requests are written by workgroup 0, with their input-check bits.
// Each wave derives the request state itself (a few cached loads), so only the pick needs
// the workgroup's barrier.  With the reverse-KL, the workgroups after the drawing ones take
// one draft row each and finish it if the streaming pass left it to this launch
// (finish_rkl_row_own).  Register use is capped so that all the drawing workgroups of a
// B = 128 call are resident at once.
template <int DT, bool VEC>
__global__ __launch_bounds__(kMassThreads) __attribute__((amdgpu_waves_per_eu(5)))
void sv_draw_kernel(SampleArgs a) {
  __shared__ double s_pm[kMaxChunks];  // the picking wave's chunk masses (p_T's after a fallback)
  __shared__ int s_ticket;  // the workgroup's draw ticket
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t drawing = a.B * a.mass_blocks;
  if (static_cast<int64_t>(blockIdx.x) >= drawing) {  // a draft row's heavy lanes
    finish_rkl_row_own<DT, VEC>(a, blockIdx.x - drawing, wave, lane, s_pm);
    return;
  }
  const int64_t b = blockIdx.x / a.mass_blocks;
  const int g = static_cast<int>(blockIdx.x - b * a.mass_blocks);
  int my_tok;    // lane i holds draft token i of the request
  float my_u;    // and the uniform of target row i
  const ReqState rq = wave_request_state(a, b, &my_tok, &my_u);

  if (rq.void_call) {  // void call: the layout is unknown, so -1 everywhere, strided by B
    if (g == 0) {
      if (tid == 0) a.accept_len[b] = -1;
      for (int64_t t = b + static_cast<int64_t>(tid) * a.B; t < a.n_t;
           t += static_cast<int64_t>(kMassThreads) * a.B)
        a.out_tokens[t] = -1;
    }
    return;
  }
  draw_request<DT, VEC>(a, b, g, tid, lane, wave, my_tok, my_u, rq, s_pm, &s_ticket);
}

// =========================================================================== branch lookup
// After verification: which prepared successor block a request can reuse (D3D review page,
// Methodology, inference paragraph: a verified prefix that matches a prepared branch is a
// cache hit).  A branch is keyed by (accept length, token emitted after the accepted drafts),
// token -1 matching any; the hit is the first matching branch in the request's list, -1 for
// none.  A workgroup takes 16 requests, one wave each: the rows before its first request
// (sum of k_c + 1 over valid lengths) by a reduction over k, then each wave reads its a_b,
// the token at row off_t[b] + a_b, and compares 64 keys per step (ballot, lowest index).
// A request with k_b or a_b out of range, or a row past n_tokens, gets -1.
constexpr int kBranchWaves = 16;
__global__ __launch_bounds__(64 * kBranchWaves) void sv_branch_kernel(BranchArgs a) {
  __shared__ long long s_red[kBranchWaves];
  __shared__ long long s_off[kBranchWaves];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kBranchWaves;
  auto rows_of = [&](int64_t c) -> long long {
    const int kc = a.k[c];
    return (kc >= 1 && kc <= a.k_max) ? kc + 1 : 0;
  };
  long long part = 0;
  for (int64_t c = tid; c < b0; c += 64 * kBranchWaves) part += rows_of(c);
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) part += __shfl_xor(part, m, 64);
  if (lane == 0) s_red[wave] = part;
  __syncthreads();
  if (tid == 0) {
    long long base = 0;
    for (int w = 0; w < kBranchWaves; ++w) base += s_red[w];
    for (int i = 0; i < kBranchWaves; ++i) {
      s_off[i] = base;
      if (b0 + i < a.B) base += rows_of(b0 + i);
    }
  }
  __syncthreads();
  const int64_t b = b0 + wave;
  if (b >= a.B) return;
  const int kb = a.k[b], al = a.accept_len[b];
  const long long row = s_off[wave] + al;
  int hit = -1;
  if (kb >= 1 && kb <= a.k_max && al >= 0 && al <= kb && row < a.n_tokens) {
    const int y = a.out_tokens[row];
    const int32_t* pos = a.branch_pos + b * a.n_branch;
    const int32_t* tok = a.branch_tok + b * a.n_branch;
    for (int j0 = 0; j0 < a.n_branch; j0 += 64) {
      const int j = j0 + lane;
      const bool match = j < a.n_branch && pos[j] == al && (tok[j] == y || tok[j] == -1);
      const uint64_t m = __ballot(match);
      if (m) {
        hit = j0 + __builtin_ctzll(m);
        break;
      }
    }
  }
  if (lane == 0) a.hit[b] = hit;
}

// =========================================================================== tree walk
// Greedy verification of a draft tree per request (DFlash notes, Sections 5.1-5.2; AdaFlash
// paper, Appendix B.1), after sv_row_argmax has written the argmax of every target row (the
// root's row and one per node).  A workgroup takes 16 requests, one wave each.  Every workgroup
// checks the whole call (each n_b in [1, max_nodes], sum n_b = n_nodes_total) and sums n_c over
// the requests before its own for their first node and row.  A wave keeps its request's
// parents and tokens in registers (16 per lane), checks them (a parent must be -1 or an earlier
// node; a token must lie in [0, V)), then walks: from the root, the lowest-index child whose
// token is the current row's argmax (a wave minimum), until no child matches; that node's
// argmax is the final token.  device_status was zeroed by the argmax kernel; bits are OR-ed in.
constexpr int kTreeWaves = 16;
constexpr int kTreeMaxNodes = 1024;  // SV_MAX_TREE_NODES
constexpr int kTreePerLane = kTreeMaxNodes / 64;
__global__ __launch_bounds__(64 * kTreeWaves) void sv_tree_walk_kernel(TreeArgs a) {
  __shared__ int s_args[kTreeWaves * (kTreeMaxNodes + 1)];
  __shared__ long long s_before[kTreeWaves], s_total[kTreeWaves];
  __shared__ int s_bad[kTreeWaves];
  __shared__ long long s_off[kTreeWaves];
  __shared__ int s_void;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t b0 = static_cast<int64_t>(blockIdx.x) * kTreeWaves;
  long long before = 0, total = 0;
  int bad = 0;
  for (int64_t c = tid; c < a.B; c += 64 * kTreeWaves) {
    const int nc = a.n_nodes[c];
    if (nc < 1 || nc > a.max_nodes) {
      bad = 1;
    } else {
      total += nc;
      if (c < b0) before += nc;
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    before += __shfl_xor(before, m, 64);
    total += __shfl_xor(total, m, 64);
    bad |= __shfl_xor(bad, m, 64);
  }
  if (lane == 0) {
    s_before[wave] = before;
    s_total[wave] = total;
    s_bad[wave] = bad;
  }
  __syncthreads();
  if (tid == 0) {
    long long bsum = 0, tsum = 0;
    int anybad = 0;
    for (int w = 0; w < kTreeWaves; ++w) {
      bsum += s_before[w];
      tsum += s_total[w];
      anybad |= s_bad[w];
    }
    s_void = anybad ? 1 : (tsum != a.n_nodes_total ? 2 : 0);
    if (!s_void)
      for (int i = 0; i < kTreeWaves; ++i) {
        s_off[i] = bsum;
        if (b0 + i < a.B) bsum += a.n_nodes[b0 + i];
      }
    if (s_void && blockIdx.x == 0) atomicOr(a.device_status, s_void);
  }
  __syncthreads();
  if (s_void) {  // the layout is unknown: -1 everywhere, strided over the grid
    const int64_t stride = static_cast<int64_t>(gridDim.x) * 64 * kTreeWaves;
    for (int64_t t = static_cast<int64_t>(blockIdx.x) * 64 * kTreeWaves + tid; t < a.n_nodes_total + a.B;
         t += stride) {
      a.out_tokens[t] = -1;
      if (a.out_nodes && t < a.n_nodes_total) a.out_nodes[t] = -1;
    }
    for (int64_t b = b0 + tid; b < min<int64_t>(a.B, b0 + kTreeWaves); b += 64 * kTreeWaves)
      a.accept_len[b] = -1;
    return;
  }
  const int64_t b = b0 + wave;
  if (b >= a.B) return;
  const int n = a.n_nodes[b];
  const int64_t on = s_off[wave], ot = on + b;  // first node, first target row
  int pr[kTreePerLane], tk[kTreePerLane];
  int flags = 0;
#pragma unroll
  for (int m = 0; m < kTreePerLane; ++m) {
    const int j = lane + 64 * m;
    pr[m] = -2;
    tk[m] = -1;
    if (j < n) {
      pr[m] = a.parent[on + j];
      tk[m] = a.tokens[on + j];
      if (pr[m] < -1 || pr[m] >= j) flags |= 32;  // SV_DEV_BAD_PARENT
      if (tk[m] < 0 || tk[m] >= a.V) flags |= 4;  // SV_DEV_BAD_TOKEN
    }
  }
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) flags |= __shfl_xor(flags, m, 64);
  if (flags) {
    if (lane == 0) {
      a.accept_len[b] = -1;
      atomicOr(a.device_status, flags);
    }
    for (int j = lane; j <= n; j += 64) a.out_tokens[ot + j] = -1;
    if (a.out_nodes)
      for (int j = lane; j < n; j += 64) a.out_nodes[on + j] = -1;
    return;
  }
  // the request's row argmaxes (root, then nodes) staged in this wave's LDS slice, so each step
  // of the walk reads LDS instead of waiting on a global load
  int* s_arg = s_args + wave * (kTreeMaxNodes + 1);
  for (int j = lane; j <= n; j += 64) s_arg[j] = a.arg[ot + j];
  int cur = -1, len = 0, g;
  while (true) {
    g = s_arg[cur + 1];
    int best = 0x7fffffff;
#pragma unroll
    for (int m = kTreePerLane - 1; m >= 0; --m)
      if (pr[m] == cur && tk[m] == g) best = lane + 64 * m;
    const int nxt = wave_min_int(best);
    if (nxt == 0x7fffffff) break;
    if (lane == 0) {
      a.out_tokens[ot + len] = g;
      if (a.out_nodes) a.out_nodes[on + len] = nxt;
    }
    ++len;
    cur = nxt;
  }
  if (lane == 0) {
    a.out_tokens[ot + len] = g;
    a.accept_len[b] = len;
  }
  for (int j = len + 1 + lane; j <= n; j += 64) a.out_tokens[ot + j] = -1;
  if (a.out_nodes)
    for (int j = len + lane; j < n; j += 64) a.out_nodes[on + j] = -1;
}

// =========================================================================== launchers
hipError_t launch_plan(const PlanArgs& a, hipStream_t st) {
  hipLaunchKernelGGL(sv_plan_kernel, dim3(1), dim3(1024), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_opd_reduce(const int32_t* k, int64_t B, int64_t n_rows, const float* rkl,
                             const float* hard, float alpha, const int32_t* row_flags,
                             float* opd_out, float* coef, int32_t* device_status, hipStream_t st) {
  hipLaunchKernelGGL(sv_opd_reduce_kernel, dim3(1), dim3(1024), 0, st, k, B, n_rows, rkl, hard,
                     alpha, row_flags, opd_out, coef, device_status);
  return hipGetLastError();
}

hipError_t launch_opd_grad(int dtype, int grad_dtype, bool vec, const GradArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.n_rows)), blk(256);
  if (dtype == 0 && grad_dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_opd_grad_kernel<0, 0, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((sv_opd_grad_kernel<0, 0, false>), grid, blk, 0, st, a);
  } else if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_opd_grad_kernel<0, 1, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((sv_opd_grad_kernel<0, 1, false>), grid, blk, 0, st, a);
  } else if (grad_dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_opd_grad_kernel<1, 0, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((sv_opd_grad_kernel<1, 0, false>), grid, blk, 0, st, a);
  } else {
    if (vec) hipLaunchKernelGGL((sv_opd_grad_kernel<1, 1, true>), grid, blk, 0, st, a);
    else hipLaunchKernelGGL((sv_opd_grad_kernel<1, 1, false>), grid, blk, 0, st, a);
  }
  return hipGetLastError();
}

hipError_t launch_status(const int32_t* row_flags, int64_t n, int32_t* device_status,
                         hipStream_t st) {
  hipLaunchKernelGGL(sv_status_kernel, dim3(1), dim3(256), 0, st, row_flags, n, device_status);
  return hipGetLastError();
}

hipError_t launch_tree_walk(const TreeArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.B + kTreeWaves - 1) / kTreeWaves));
  hipLaunchKernelGGL(sv_tree_walk_kernel, grid, dim3(64 * kTreeWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_branch(const BranchArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>((a.B + kBranchWaves - 1) / kBranchWaves));
  hipLaunchKernelGGL(sv_branch_kernel, grid, dim3(64 * kBranchWaves), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_draw(int dtype, bool vec, const SampleArgs& a, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(a.B * a.mass_blocks + a.fix_rows));
  if (dtype == 0) {
    if (vec) hipLaunchKernelGGL((sv_draw_kernel<0, true>), grid, dim3(kMassThreads), 0, st, a);
    else hipLaunchKernelGGL((sv_draw_kernel<0, false>), grid, dim3(kMassThreads), 0, st, a);
  } else {
    hipLaunchKernelGGL((sv_draw_kernel<1, false>), grid, dim3(kMassThreads), 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace sv
